"""kvtc_attend_noalloc (the allocation-free attention entry point) against
kvtc_attend, through the C ABI, on MI355X: two calls in a row, the second on
fewer rows and another query, each equal to kvtc_attend's output on the same
inputs (the same kernels run on the library's fixed scratch instead of a
caller workspace, so the outputs are bit-identical)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import kvtc_oracle as O
from kv_cache_compression_kvtc_amd import synth
from kv_cache_compression_kvtc_amd import kvtc as K

from gpu_helpers import DeviceStore, blob_from_oracle, oracle_cfg

pytestmark = pytest.mark.gpu


def test_attend_noalloc_matches_attend_on_two_calls():
    print("CASE attend noalloc", flush=True)
    w = synth.WORKLOADS[4]
    f = dict(w.__dict__)
    f.update(B=4, s_prefill=2048, s_total=2048 + 700)
    w = synth.Workload(**f)
    Xk, Xv = synth.generate(w, 0), synth.generate(w, 1)
    S = Xk.shape[2]
    stores = []
    for X in (Xk, Xv):
        ds = DeviceStore(blob_from_oracle(O.fit(oracle_cfg(w), X[:, :, :w.s_prefill])), S)
        ds.append(X, 0)
        stores.append(ds)
    att = K.Attend(*[(d.blob, d.blob_dev, d.codes, d.params) for d in stores], S)
    assert K.kvtc_attend_workspace(stores[0].blob, stores[1].blob, S) <= 16 << 20
    g = torch.Generator(device="cuda:0").manual_seed(5)
    for s_end, dtype in ((S, torch.float16), (S - 611, torch.float32)):
        q = torch.randn((w.B, w.H, w.D), device="cuda:0", generator=g).to(dtype)
        want = att(q, s_end)
        got = torch.full_like(want, float("nan"))
        att.noalloc(q, s_end, got)
        torch.cuda.synchronize()
        assert torch.equal(got, want), s_end
