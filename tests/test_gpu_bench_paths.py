"""Full-size parity of exactly the launches bench.py times, on MI355X.

Each workload is set up as the benchmark sets it up: both tensors fitted by the
library's own host fit (kvtc_fit_host), the stored rows appended, then the
paired calls (kvtc_append_kv, kvtc_fetch_kv) through the prepared bindings.
The oracle then evaluates its own arithmetic on the frozen state of those same
blobs (rebuilt from their sections) and both tensors are checked on sampled
units: codes (exemption band), packing, and reconstruction.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import kvtc_oracle as O
from kv_cache_compression_kvtc_amd import synth
from kv_cache_compression_kvtc_amd import kvtc as K

from gpu_helpers import (DeviceStore, check_codes_dp, check_codes_mixed, check_recon_unit, lib_cfg, oracle_cfg,
                         state_from_blob)

pytestmark = pytest.mark.gpu


def print_case(*a):
    print("CASE", *a, flush=True)


class BenchLayer:
    """Key and value tensors of a workload fitted by kvtc_fit_host, with the
    prepared paired calls the benchmark uses."""

    def __init__(self, w, s_fit, S):
        self.X = [synth.generate(w, t, 0, S) for t in (synth.KEY, synth.VALUE)]
        cfg = lib_cfg(oracle_cfg(w))
        self.blobs = [K.kvtc_fit_host(cfg, np.ascontiguousarray(x[:, :, :s_fit])) for x in self.X]
        self.sts = [state_from_blob(b) for b in self.blobs]
        self.stores = [DeviceStore(b, S) for b in self.blobs]
        self.xs = [torch.from_numpy(x).cuda() for x in self.X]
        self.outs = [torch.empty((w.B, w.H, S, w.D), dtype=torch.float16, device="cuda:0") for _ in range(2)]
        st = self.stores
        self.append = K.PreparedAppendKV(*[(self.blobs[i], st[i].blob_dev, self.xs[i], st[i].codes, st[i].params)
                                           for i in range(2)], S)
        self.fetch = K.PreparedFetchKV(*[(self.blobs[i], st[i].blob_dev, st[i].codes, st[i].params, self.outs[i])
                                         for i in range(2)], S)
        self.S = S

    def check(self, units_per_tensor, seed):
        torch.cuda.synchronize()
        rng = np.random.default_rng(seed)
        for i in range(2):
            st, rows = self.sts[i], self.stores[i].rows(self.S)
            units = rng.choice(st.U, size=min(units_per_tensor, st.U), replace=False)
            if st.cfg.mode == "dp":
                check_codes_dp(st, self.X[i], rows, units=units)
                prm = [None] * st.U
            else:
                prm = self.stores[i].params_np(self.S)
                check_codes_mixed(st, self.X[i], rows, prm, units=units)
            for u in units:
                check_recon_unit(st, rows[u], u, self.outs[i], prm[u], what=f"tensor {i} unit {u}")


def test_bench_path_batched_decode_full_size():
    """Batched decode (B=64, H=8, D=128): 8192 stored rows, then decode steps of
    one paired append (one launch for K and V) and one paired fetch of every row
    (one launch of 1024 blocks); 32 sampled units of K and of V."""
    print_case("bench path: batched decode")
    w = synth.WORKLOADS[4]
    S0, steps = w.s_prefill, 3
    layer = BenchLayer(w, S0, S0 + steps)
    layer.append(0, S0)
    for s in range(S0, S0 + steps):
        layer.append(s, s + 1)
        layer.fetch(0, s + 1)
    layer.check(32, seed=8)


def test_bench_path_long_context_full_size():
    """Long context (B=1, H=8, S=131072, rank by energy on the first 8192 rows):
    paired append of the prefix, paired one-shot append of the remaining 122880
    rows, paired fetch of the whole sequence; every unit of K and of V."""
    print_case("bench path: long context")
    w = synth.WORKLOADS[5]
    layer = BenchLayer(w, w.s_prefill, w.s_total)
    layer.append(0, w.s_prefill)
    layer.append(w.s_prefill, w.s_total)
    layer.fetch(0, w.s_total)
    layer.check(8, seed=9)


def test_bench_path_group_head_full_size():
    """Group-head workload (B=1, H=32 in 4 groups of 8, S=16384, rank 256):
    paired one-shot append and paired fetch; every unit of K and of V."""
    print_case("bench path: group head")
    w = synth.WORKLOADS[3]
    layer = BenchLayer(w, w.s_prefill, w.s_total)
    layer.append(0, w.s_total)
    layer.fetch(0, w.s_total)
    layer.check(4, seed=10)
