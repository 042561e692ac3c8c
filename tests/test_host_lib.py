"""Host half of libkvtc against the oracle, symbol exports and error paths (no GPU).

The fit, DP allocation, blob builder and byte accounting run on the CPU, so
they are compared with the oracle here.  Device entry points are only called
with arguments that fail validation, which returns before any HIP call.
"""
import ctypes as C
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

from oracle import kvtc_oracle as O
from kv_cache_compression_kvtc_amd import synth
from kv_cache_compression_kvtc_amd import kvtc as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvtc.h")


def oracle_cfg(w, **kw):
    c = O.Config(mode=w.mode, head_dim=w.D, heads_per_unit=w.heads_per_unit, rank=w.rank,
                 energy=w.energy, budget=w.budget, choices=w.choices, beta=w.beta,
                 hi_bits=w.hi_bits, lo_bits=w.lo_bits, hi_fraction=w.hi_fraction,
                 group_size=w.group_size)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def lib_cfg(oc: O.Config):
    return K.make_config(oc.mode, oc.head_dim, oc.heads_per_unit, oc.rank, oc.energy,
                         oc.resolved_budget(), oc.choices, oc.beta, oc.hi_bits, oc.lo_bits,
                         oc.group_size, oc.hi_fraction)


def blob_from_oracle(st: O.TensorState) -> np.ndarray:
    """The device state blob built from the oracle's frozen state (oracle -> library only)."""
    return K.kvtc_state_build(lib_cfg(st.cfg), st.B, st.H, st.r, st.mu32,
                              np.ascontiguousarray(st.V32.transpose(0, 2, 1)), st.lam,
                              st.bits.astype(np.uint8), st.qmin32, st.qscale32)


# ---------------------------------------------------------------- exports
def test_loaded_library_was_built_from_the_current_sources():
    from kv_cache_compression_kvtc_amd.build import source_hash, library_build_id
    assert K.build_id() == source_hash() == library_build_id()


def test_library_exports_every_declared_symbol():
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(kvtc_\w+)\s*\(", text, flags=re.M))
    assert {"kvtc_fit_host", "kvtc_append", "kvtc_fetch", "kvtc_bytes"} <= declared
    lib = C.CDLL(K.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert declared == set(K.EXPORTED)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_ctypes_structs_match_the_c_header(tmp_path):
    src = tmp_path / "s.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "kvtc.h"\n'
                   'int main(){printf("%zu %zu %zu %zu %zu %zu\\n", sizeof(kvtc_config),'
                   ' sizeof(kvtc_state_header), sizeof(kvtc_bytes_report), sizeof(kvtc_unit_info),'
                   ' offsetof(kvtc_state_header, s_prefill), offsetof(kvtc_state_header, off_bias));'
                   'printf("%zu %zu %zu\\n", sizeof(kvtc_tensor_ref), offsetof(kvtc_tensor_ref, dtype),'
                   ' offsetof(kvtc_tensor_ref, strides));}\n')
    exe = tmp_path / "s"
    subprocess.run(["gcc", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()]
    want = [C.sizeof(K.Config), C.sizeof(K.StateHeader), C.sizeof(K.BytesReport), C.sizeof(K.UnitInfo),
            K.StateHeader.s_prefill.offset, K.StateHeader.off_bias.offset,
            C.sizeof(K.TensorRef), K.TensorRef.dtype.offset, K.TensorRef.strides.offset]
    assert got == want


# ---------------------------------------------------------------- DP allocation
def test_allocation_identical_to_oracle_on_identical_lambdas(rng):
    for trial in range(40):
        r = int(rng.integers(1, 130))
        lam = np.sort(rng.gamma(0.3, 1.0, size=r))[::-1] * float(rng.choice([1.0, 1e-3, 7.5]))
        choices = tuple(sorted(set([0] + rng.choice([1, 2, 3, 4, 8], size=int(rng.integers(1, 5))).tolist())))
        budget = int(rng.integers(0, 4 * r + 1))
        beta = float(rng.choice([1.0, 0.7, 3.0]))
        want = O.allocate_dp(lam, budget, choices, beta)
        got = K.kvtc_allocate_bits(lam, budget, choices, beta)
        assert got.tolist() == want.tolist(), (trial, r, budget, choices, beta)


def test_allocation_errors():
    with pytest.raises(K.KVTCError) as e:
        K.kvtc_allocate_bits(np.ones(3), -1, (0, 1))
    assert e.value.status == K.E_CONFIG
    with pytest.raises(K.KVTCError) as e:
        K.kvtc_allocate_bits(np.ones(3), 2, (1, 2))             # 3 components need >= 3 bits
    assert e.value.status == K.E_CONFIG
    with pytest.raises(K.KVTCError) as e:
        K.kvtc_allocate_bits(np.ones(3), 8, (0, 5))
    assert e.value.status == K.E_CONFIG


# ---------------------------------------------------------------- fit
def _compare_fit(w, tensor, oc=None):
    X = synth.generate(w, tensor, 0, w.s_prefill)
    oc = oc or oracle_cfg(w)
    st = O.fit(oc, X)
    v = K.state_view(K.kvtc_fit_host(lib_cfg(oc), X))
    h = v["header"]
    assert (h.units, h.dg, h.rmax) == (st.U, st.Dg, st.bits.shape[1])
    assert h.s_prefill == X.shape[2]
    assert v["rank"].tolist() == st.r.tolist()
    assert np.array_equal(v["mu"], st.mu32)
    assert np.abs(v["lambda"] - st.lam).max() <= 1e-12 * st.lam.max()
    assert np.array_equal(v["bits"], st.bits.astype(np.uint8))
    for u in range(st.U):
        ns = int(v["n_slots"][u])
        comps = v["slot_comp"][u, :ns]
        assert comps.tolist() == np.flatnonzero(st.bits[u]).tolist()
        # basis vectors: equal up to the last fp32 rounding of a float64 eigenvector
        Vo = st.V32[u][:, comps].T.astype(np.float64)
        assert np.abs(v["basis"][u, :ns] - Vo).max() <= 2 ** -23
    if oc.mode == "dp":
        sc = np.where(st.qscale32 > 0, st.qscale32, 1.0).astype(np.float64)
        assert (np.abs(v["qmin"].astype(np.float64) - st.qmin32) <= 1e-6 * sc).all()
        assert (np.abs(v["qscale"].astype(np.float64) - st.qscale32) <= 1e-6 * sc).all()
    return st, v


@pytest.mark.parametrize("tensor", [0, 1])
def test_fit_matches_oracle_tiny(tensor):
    _compare_fit(synth.WORKLOADS[1], tensor)


def test_fit_matches_oracle_llama_layer_keys_with_outliers():
    _compare_fit(synth.WORKLOADS[2], 0)


def test_fit_energy_rank_long_context_values():
    st, v = _compare_fit(synth.WORKLOADS[5], 1)
    assert 1 < int(v["rank"][0]) < 128


def test_fit_group_head_small():
    # PALU page: contiguous head groups share one projection (2 groups of 2 heads, D=64)
    w = synth.Workload(90, "gh-small", B=1, H=4, D=64, dtype="f16", s_prefill=300, s_total=300,
                       alpha_k=1.2, alpha_v=0.8, n_outliers_k=2, mode="mixed", heads_per_unit=2,
                       rank=48, hi_bits=4, lo_bits=2, hi_fraction=0.25, group_size=16)
    st, v = _compare_fit(w, 0)
    assert v["header"].n_hi == 16 and v["header"].n_qgroups == 3


# ---------------------------------------------------------------- blob builder
def test_state_build_derived_sections_follow_their_definitions():
    w = synth.WORKLOADS[1]
    X = synth.generate(w, 1, 0, 256)
    st = O.fit(oracle_cfg(w, budget=80), X)
    blob = blob_from_oracle(st)
    v = K.state_view(blob)
    h = v["header"]
    assert h.row_stride == max(O.row_stride_bytes(st.row_bits(u)) for u in range(st.U))
    for u in range(st.U):
        comps = np.flatnonzero(st.bits[u])
        ns = len(comps)
        offs, rb = O.field_offsets(st.bits[u][comps])
        assert v["row_bits"][u] == rb
        sb = v["slot_bits"][u, :ns]
        assert ((sb & 0xFFFFFF) == offs).all() and ((sb >> 24) == st.bits[u][comps]).all()
        assert (v["slot_bits"][u, ns:] == 0).all() and (v["slot_comp"][u, ns:] == -1).all()
        sc = st.qscale32[u][comps].astype(np.float64)
        Vc = st.V32[u][:, comps].astype(np.float64)                        # [dg, ns]
        w16 = (Vc * sc[None, :]).astype(np.float16)                        # rounded once from float64
        # fetch order: each run of equal widths is padded to whole 16-slot
        # k-steps; inside each 8-slot half of a 4-bit k-step the slots sit in
        # the nibble order 0,2,4,6,1,3,5,7 and a 2-bit k-step in the byte-lane
        # order below (the orders the kernel unpacks them in)
        widths = st.bits[u][comps]
        nib = [0, 2, 4, 6, 1, 3, 5, 7]
        # 2-bit k-steps: column c holds slot two[c] (codes one per byte after
        # masking the k-step's 32-bit window with 0x03030303 at shifts 0,2,4,6)
        two = [0, 4, 8, 12, 1, 5, 9, 13, 2, 6, 10, 14, 3, 7, 11, 15]
        place, descs, k, in_step = [], [], 0, 0
        for j in range(ns):
            if j == 0 or widths[j] != widths[j - 1] or in_step == 16:
                k = (k + 15) // 16 * 16
                descs.append((int(offs[j]), int(widths[j])))
                in_step = 0
            e = in_step % 8
            if widths[j] == 4:
                kk = k - e + nib.index(e)
            elif widths[j] == 2:
                kk = k - in_step + two[in_step]
            else:
                kk = k
            place.append((kk, j))
            k += 1
            in_step += 1
        kf = h.kfetch
        assert kf == 16 * len(descs)
        want = np.zeros((st.Dg, kf), np.float16)
        for kk, j in place:
            want[:, kk] = w16[:, j]
        assert np.array_equal(v["w16"][u], want)
        fs = np.full(kf, -1, np.int32)
        for kk, j in place:
            fs[kk] = j
        assert np.array_equal(v["fslot"][u], fs)
        kd = v["kdesc"][u]
        assert [(int(d & 0xFFFF), int((d >> 16) & 0xF)) for d in kd] == descs
        bias = st.mu32[u].astype(np.float64) + Vc @ st.qmin32[u][comps].astype(np.float64)
        assert np.abs(v["bias"][u] - bias).max() <= 2 ** -23 * np.abs(bias).max() * 2
        assert np.array_equal(v["qlo"][u, :ns], st.qmin32[u][comps].astype(np.float64))
        inv = np.where(sc > 0, 1.0 / np.where(sc > 0, sc, 1), 0.0)
        assert np.array_equal(v["qinv"][u, :ns], inv)
        # int8 append operands: the five balanced base-256 digits of each slot's
        # rint(basis * 2^38) (exact integers: int64 arithmetic), and mean . basis
        dig = v["vdig"][u].astype(np.int64)                                 # [5, kslots, dg]
        assert dig.min() >= -128 and dig.max() <= 127 and np.abs(dig[4]).max() <= 64
        vq = np.rint(np.ldexp(st.V32[u][:, comps].astype(np.float64).T, 38)).astype(np.int64)   # [ns, dg]
        got = sum(dig[k, :ns] * (256 ** k) for k in range(5))
        assert np.array_equal(got, vq)
        assert (dig[:, ns:] == 0).all()
        # offset: mean . basis minus 2^-62 * 0x808080 * sum_d vq (the constant of the
        # row digits, which are the bytes of x * 2^24 ^ 0x808080)
        mv = Vc.T @ st.mu32[u].astype(np.float64) - np.ldexp(vq.sum(axis=1).astype(np.float64) * 0x808080, -62)
        assert np.abs(v["mv"][u, :ns] - mv).max() <= 1e-12 * (np.abs(st.mu32[u]).sum() + st.Dg)


def test_state_without_unit_basis_has_no_int8_operands():
    """A basis entry above 1 in magnitude (not an orthonormal basis) leaves the
    digit sections out: the blob says so with zero offsets."""
    w = synth.WORKLOADS[1]
    X = synth.generate(w, 1, 0, 256)
    st = O.fit(oracle_cfg(w, budget=80), X)
    st.V32 = st.V32.copy()
    st.V32[0, 0, 0] = 1.5
    v = K.state_view(blob_from_oracle(st))
    assert v["header"].off_vdig == 0 and v["header"].off_mv == 0 and v["vdig"] is None


# ---------------------------------------------------------------- bytes
def test_bytes_report_matches_oracle_dp():
    w = synth.WORKLOADS[1]
    for budget in (128, 40):
        X = synth.generate(w, 0)
        st = O.fit(oracle_cfg(w, budget=budget), X[:, :, :256])
        rows, _ = O.append(st, X)
        S = X.shape[2]
        want = O.bytes_report(st, rows, None, S)
        got = K.kvtc_bytes(blob_from_oracle(st), rows, None, S, S)
        for k in ("fixed_payload", "entropy_payload", "entropy_table", "stored_payload", "basis",
                  "quant_params", "total", "pre_entropy", "fp16_equiv", "n_survived",
                  "units_entropy_coded"):
            assert got[k] == getattr(want, k), k
        assert got["device_store"] == st.U * S * st.row_stride


def test_bytes_report_matches_oracle_mixed():
    w = synth.Workload(91, "gh-bytes", B=1, H=4, D=64, dtype="f16", s_prefill=200, s_total=200,
                       alpha_k=1.0, alpha_v=1.0, mode="mixed", heads_per_unit=4, rank=64,
                       hi_bits=4, lo_bits=2, group_size=32)
    X = synth.generate(w, 1)
    st = O.fit(oracle_cfg(w), X)
    rows, params = O.append(st, X)
    want = O.bytes_report(st, rows, params, 200)
    got = K.kvtc_bytes(blob_from_oracle(st), rows, params.view(np.uint32), 200, 200)
    for k in ("fixed_payload", "stored_payload", "basis", "quant_params", "total", "pre_entropy",
              "fp16_equiv", "n_survived"):
        assert got[k] == getattr(want, k), k
    # the hi count rounds to whole quantisation groups: 0.25 * 64 -> one group of 32
    assert O.effective_bits(st) == pytest.approx((32 * 4 + 32 * 2) / 256)


# ---------------------------------------------------------------- error paths
def test_fit_config_errors():
    X = np.zeros((1, 2, 8, 64), np.float32)
    base = dict(mode="dp", head_dim=64, rank=64, budget=128, choices=(0, 1, 2))
    bad = [dict(budget=-1), dict(choices=(0, 5)), dict(rank=65), dict(head_dim=48)]
    for b in bad:
        kw = dict(base)
        kw.update(b)
        cfg = K.make_config(**kw)
        with pytest.raises(K.KVTCError) as e:
            K.kvtc_fit_host(cfg, X if kw["head_dim"] == 64 else np.zeros((1, 2, 8, 48), np.float32))
        assert e.value.status == K.E_CONFIG, b
    with pytest.raises(K.KVTCError) as e:                       # a prefill needs S > 1
        K.kvtc_fit_host(K.make_config(**base), X[:, :, :1])
    assert e.value.status == K.E_CONFIG
    with pytest.raises(K.KVTCError) as e:                       # no bit choice fits the budget
        K.kvtc_fit_host(K.make_config(**dict(base, budget=10, choices=(1, 2))), X)
    assert e.value.status == K.E_CONFIG
    with pytest.raises(K.KVTCError) as e:
        K.kvtc_fit_host(K.make_config(**base), X.astype(np.float64))
    assert e.value.status == K.E_DTYPE
    with pytest.raises(K.KVTCError) as e:                       # heads must split into groups
        K.kvtc_fit_host(K.make_config(mode="mixed", head_dim=64, heads_per_unit=3), X)
    assert e.value.status == K.E_SHAPE


def _raw(name):
    return getattr(C.CDLL(K.LIB_PATH), name)


def _device_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0     # counts devices without initialising one
    except Exception:
        return False


# The tests below pass a fake device address that only validation failures keep
# from being used; they run only where no GPU is visible, so a regression in the
# validation can never launch a kernel on that address.
no_device_only = pytest.mark.skipif(_device_visible(), reason="passes fake device addresses; CPU container only")


@no_device_only
def test_device_entry_points_validate_before_launch():
    w = synth.WORKLOADS[1]
    X = synth.generate(w, 0, 0, 256)
    st = O.fit(oracle_cfg(w), X)
    blob = blob_from_oracle(st)
    fake = C.c_void_p(0x1000)        # never dereferenced: every call below fails validation first
    strides = (C.c_int64 * 4)(2 * 64 * 10, 64 * 10, 64, 1)
    app = _raw("kvtc_append")
    app.restype = C.c_int32
    app.argtypes = K._sig["kvtc_append"][1]
    # capacity overflow
    assert app(blob.ctypes.data, fake, fake, K.F32, strides, 1, 2, 10, 95, fake, None, 100, None) == K.E_CAPACITY
    # shape mismatch with the state
    assert app(blob.ctypes.data, fake, fake, K.F32, strides, 1, 3, 10, 0, fake, None, 100, None) == K.E_SHAPE
    # non-unit innermost stride
    bad = (C.c_int64 * 4)(1280, 640, 64, 2)
    assert app(blob.ctypes.data, fake, fake, K.F32, bad, 1, 2, 10, 0, fake, None, 100, None) == K.E_SHAPE
    # dtype
    assert app(blob.ctypes.data, fake, fake, 7, strides, 1, 2, 10, 0, fake, None, 100, None) == K.E_DTYPE
    # corrupt state
    broken = blob.copy()
    broken[0] ^= 0xFF
    assert app(broken.ctypes.data, fake, fake, K.F32, strides, 1, 2, 10, 0, fake, None, 100, None) == K.E_STATE
    # missing code store
    assert app(blob.ctypes.data, fake, fake, K.F32, strides, 1, 2, 10, 0, None, None, 100, None) == K.E_ARG
    fet = _raw("kvtc_fetch")
    fet.restype = C.c_int32
    fet.argtypes = K._sig["kvtc_fetch"][1]
    ostr = (C.c_int64 * 4)(2 * 100 * 64, 100 * 64, 64, 1)
    assert fet(blob.ctypes.data, fake, fake, None, 100, 0, 101, fake, ostr, None) == K.E_CAPACITY
    assert fet(blob.ctypes.data, fake, fake, None, 100, 5, 4, fake, ostr, None) == K.E_ARG
    odd = (C.c_int64 * 4)(2 * 100 * 64, 100 * 64, 65, 1)        # rows not 16-byte aligned
    assert fet(blob.ctypes.data, fake, fake, None, 100, 0, 10, fake, odd, None) == K.E_SHAPE
    assert fet(blob.ctypes.data, fake, fake, None, 100, 0, 10, C.c_void_p(0x1002), ostr, None) == K.E_ARG
    assert fet(broken.ctypes.data, fake, fake, None, 100, 0, 10, fake, ostr, None) == K.E_STATE
    # empty ranges are valid no-ops and touch nothing
    assert fet(blob.ctypes.data, fake, fake, None, 100, 7, 7, fake, ostr, None) == K.OK
    assert app(blob.ctypes.data, fake, fake, K.F32, strides, 1, 2, 0, 3, fake, None, 100, None) == K.OK


def test_store_sizes():
    w = synth.WORKLOADS[1]
    st = O.fit(oracle_cfg(w), synth.generate(w, 0, 0, 256))
    cb, pb = K.kvtc_store_bytes(blob_from_oracle(st), 300)
    assert cb == st.U * 300 * st.row_stride and pb == 0


@no_device_only
def test_paired_entry_points_validate_both_tensors_before_launch():
    """kvtc_append_kv / kvtc_fetch_kv check the key and the value tensor before
    anything is launched: a bad value tensor fails the call even when the key
    tensor is valid (fake device pointers are never dereferenced)."""
    w = synth.WORKLOADS[1]
    st = O.fit(oracle_cfg(w), synth.generate(w, 0, 0, 256))
    blob = blob_from_oracle(st)
    broken = blob.copy()
    broken[0] ^= 0xFF
    fake = 0x1000

    def ref(b, dtype=K.F32, capacity=100, strides=(2 * 64 * 10, 64 * 10, 64, 1)):
        r = K.TensorRef()
        r.state_host, r.state_dev, r.codes_dev, r.rows_dev = b.ctypes.data, fake, fake, fake
        r.capacity, r.dtype = capacity, dtype
        for i, v in enumerate(strides):
            r.strides[i] = v
        return r

    app = _raw("kvtc_append_kv")
    app.restype = C.c_int32
    app.argtypes = K._sig["kvtc_append_kv"][1]
    good = ref(blob)
    assert app(C.byref(good), C.byref(ref(broken)), 1, 2, 10, 0, None) == K.E_STATE
    assert app(C.byref(good), C.byref(ref(blob, dtype=9)), 1, 2, 10, 0, None) == K.E_DTYPE
    assert app(C.byref(good), C.byref(ref(blob, capacity=50)), 1, 2, 10, 45, None) == K.E_CAPACITY
    assert app(C.byref(good), C.byref(ref(blob)), 1, 3, 10, 0, None) == K.E_SHAPE
    assert app(C.byref(good), None, 1, 2, 10, 0, None) == K.E_ARG
    assert app(C.byref(good), C.byref(ref(blob)), 1, 2, 0, 0, None) == K.OK       # empty: nothing to do
    fet = _raw("kvtc_fetch_kv")
    fet.restype = C.c_int32
    fet.argtypes = K._sig["kvtc_fetch_kv"][1]
    out_strides = (2 * 100 * 64, 100 * 64, 64, 1)
    assert fet(C.byref(ref(blob, strides=out_strides)), C.byref(ref(broken, strides=out_strides)), 0, 10,
               None) == K.E_STATE
    odd = (2 * 100 * 64, 100 * 64, 65, 1)                    # value rows not 16-byte aligned
    assert fet(C.byref(ref(blob, strides=out_strides)), C.byref(ref(blob, strides=odd)), 0, 10, None) == K.E_SHAPE
    assert fet(C.byref(ref(blob, strides=out_strides)), C.byref(ref(blob, strides=out_strides)), 0, 101,
               None) == K.E_CAPACITY
    assert fet(C.byref(ref(blob, strides=out_strides)), C.byref(ref(blob, strides=out_strides)), 4, 4,
               None) == K.OK


@no_device_only
def test_attend_validates_before_launch():
    """kvtc_attend rejects key and value tensors of different shapes, short
    workspaces, rows past the capacity and bad query types before anything is
    launched; kvtc_attend_gqa also query-head counts that are not a multiple of
    the stored heads, or more than 32 queries per unit."""
    w = synth.WORKLOADS[1]
    st = O.fit(oracle_cfg(w), synth.generate(w, 0, 0, 256))
    blob = blob_from_oracle(st)
    wm = synth.WORKLOADS[3]
    Xm = synth.generate(wm, 0, 0, 64)[:, :8]
    mixed = K.kvtc_fit_host(K.make_config("mixed", 128, 8, 64, group_size=32), np.ascontiguousarray(Xm))
    U, ks = st.U, K.header(blob).kslots
    # one segment (100 rows) is finished in its blocks: no workspace; 4096 rows
    # over 2 units take 16 segments of 256 rows (enough blocks, segments of at
    # least 256 rows), whose partial sums [U][16][ks + 2] f32 are the workspace
    assert K.kvtc_attend_workspace(blob, blob, 100) == 0
    S = 4096
    need = K.kvtc_attend_workspace(blob, blob, S)
    assert need == U * 16 * (ks + 2) * 4
    fake = 0x1000

    def ref(b, capacity=S):
        r = K.TensorRef()
        r.state_host, r.state_dev, r.codes_dev, r.capacity = b.ctypes.data, fake, fake, capacity
        return r

    att = _raw("kvtc_attend")
    att.restype = C.c_int32
    att.argtypes = K._sig["kvtc_attend"][1]
    s3 = (C.c_int64 * 3)(2 * 64, 64, 1)
    good = ref(blob)
    work = 0x10000

    def call(kr, vr, qdt=K.F32, s_end=S, wbytes=need, work_ptr=work, qs=s3):
        return att(C.byref(kr), C.byref(vr), fake, qdt, qs, s_end, fake, s3, work_ptr, wbytes, None)

    assert call(good, ref(mixed)) == K.E_SHAPE              # 2 heads of 64 vs 8 heads of 128
    assert call(good, good, wbytes=need - 4) == K.E_BUFSIZE
    assert call(good, good, work_ptr=0) == K.E_BUFSIZE
    assert call(good, good, s_end=S + 1) == K.E_CAPACITY
    assert call(good, good, qdt=5) == K.E_DTYPE
    assert call(good, good, qs=(C.c_int64 * 3)(128, 64, 2)) == K.E_SHAPE
    gqa = _raw("kvtc_attend_gqa")
    gqa.restype = C.c_int32
    gqa.argtypes = K._sig["kvtc_attend_gqa"][1]
    need4 = K.kvtc_attend_gqa_workspace(blob, blob, 8, 100)
    assert need4 > 0

    def call_g(hq, wbytes=need4):
        return gqa(C.byref(good), C.byref(good), hq, fake, K.F32, s3, 100, fake, s3, work, wbytes, None)

    assert call_g(3) == K.E_SHAPE                   # not a multiple of the 2 stored heads
    assert call_g(2 * 33) == K.E_SHAPE              # 33 queries per head
    assert call_g(0) == K.E_ARG
    assert call_g(8, wbytes=need4 - 4) == K.E_BUFSIZE
    with pytest.raises(K.KVTCError):
        K.kvtc_attend_gqa_workspace(blob, blob, 3, 100)


def _state_status(blob):
    fn = _raw("kvtc_store_bytes")
    fn.restype = C.c_int32
    fn.argtypes = K._sig["kvtc_store_bytes"][1]
    a, b = C.c_size_t(0), C.c_size_t(0)
    return fn(blob.ctypes.data, 10, C.byref(a), C.byref(b))


def _set_header(blob, field, value):
    off = getattr(K.StateHeader, field).offset
    size = getattr(K.StateHeader, field).size
    blob[off:off + size] = np.frombuffer(int(value).to_bytes(size, "little", signed=True), np.uint8)


def test_corrupt_or_truncated_state_is_rejected():
    """A header whose sections would end past total_bytes, or whose per-unit
    counts exceed its capacities, is a corrupt state; a blob shorter than its
    total_bytes is refused by the binding before its pointer is passed."""
    w = synth.WORKLOADS[1]
    st = O.fit(oracle_cfg(w), synth.generate(w, 0, 0, 256))
    blob = blob_from_oracle(st)
    h = K.header(blob)
    assert _state_status(blob) == K.OK
    for field, value in (("units", h.units + 1), ("batch", h.batch), ("kfetch", h.kfetch + 4096),
                         ("kslots", h.kslots + 4096), ("rmax", h.rmax), ("total_bytes", h.total_bytes - 256),
                         ("off_basis", h.total_bytes - 256), ("dg", h.dg)):
        bad = blob.copy()
        _set_header(bad, field, value)
        if field == "units":                  # units must also match batch * heads
            _set_header(bad, "batch", h.batch + 1)
            _set_header(bad, "units", (h.batch + 1) * h.heads)
        want = K.OK if (field, value) in (("batch", h.batch), ("rmax", h.rmax), ("dg", h.dg)) else K.E_STATE
        assert _state_status(bad) == want, field
    # a unit claiming more stored slots than the header's capacity
    bad = blob.copy()
    ui = np.frombuffer(bad, np.int32, count=4 * h.units, offset=h.off_unit).copy().reshape(h.units, 4)
    ui[1, 1] = h.kslots + 1
    bad[h.off_unit:h.off_unit + ui.nbytes] = ui.view(np.uint8).ravel()
    assert _state_status(bad) == K.E_STATE
    # truncated host blob: refused by the binding
    with pytest.raises(K.KVTCError) as e:
        K.kvtc_store_bytes(blob[: h.total_bytes - 1].copy(), 10)
    assert e.value.status == K.E_STATE
    with pytest.raises(K.KVTCError) as e:
        K.kvtc_store_bytes(blob[:64].copy(), 10)
    assert e.value.status == K.E_STATE


def test_huge_budget_allocates_quickly_and_like_the_widest_budget(rng):
    """The DP never spends more than r * max(choices) bits, so any larger budget
    gives the allocation of that budget, in the same time."""
    import time
    lam = np.sort(rng.gamma(1.0, size=96))[::-1]
    ch = (0, 2, 4, 8)
    ref = K.kvtc_allocate_bits(lam, 96 * 8, ch)
    t = time.perf_counter()
    for budget in (10 ** 7, 2 ** 31 - 1):
        assert np.array_equal(K.kvtc_allocate_bits(lam, budget, ch), ref)
    assert time.perf_counter() - t < 2.0
    assert (ref == 8).all()


def test_bytes_report_hand_worked_values():
    """kvtc_bytes against values derived by hand from the KVTC page's "Byte
    accounting" (payload, order-0 Huffman with fixed-width fallback, fp16 basis,
    mean and (min, scale)) and the PALU page's (fp32 projection and mean, params
    per token and quantisation group).  The oracle's byte pins use the same cases
    at D = 4; here D = 64, the smallest head size the library accepts:
      widths (2, 0, 1), S = 8: payload 3 (Huffman 10 + 8 bits = 3 bytes + table 6
        is not below 3); basis 2 * (64 * 2 + 64) = 384; params 8; total 395;
      width 8 (+ a dropped one), S = 1000, 990 zeros and 10 x 255: Huffman 1000
        bits = 125 bytes + table 256 < 1000 -> coded; basis 2 * (64 + 64) = 256;
        params 4; total 125 + 256 + 256 + 4 = 641; pre-entropy 1000 + 260 = 1260;
      width 2, every code 2: S = 32 -> 4 + 4 = 8 is not below 8: 8 + 256 + 4 = 268;
        S = 40 -> 5 + 4 < 10: 5 + 4 + 256 + 4 = 269;
      group head, 2 heads (Dg = 128), rank 32, 16 components at 4 bits and 16 at
        2 (96 bits), groups of 16, S = 5: payload ceil(5 * 96 / 8) = 60;
        projection 4 * (128 * 32 + 128) = 16896; params 4 * 5 * 2 = 40; total 16996."""
    def run(mode, hpu, H, bits, codes, group_size=32, hi_fraction=0.25):
        bits = np.asarray(bits)
        D = 64
        U, r, Dg = H // hpu, len(bits), D * hpu
        cfg = K.make_config(mode, D, hpu, r, budget=int(bits.sum()), choices=(0, 1, 2, 4, 8),
                            group_size=group_size, hi_fraction=hi_fraction)
        basis = np.zeros((U, r, Dg), np.float32)
        basis[:, np.arange(r), np.arange(r)] = 1.0
        blob = K.kvtc_state_build(cfg, 1, H, np.full(U, r), np.zeros((U, Dg)), basis, None,
                                  np.tile(bits, (U, 1)), np.zeros((U, r)), np.ones((U, r)))
        h = K.header(blob)
        S = codes.shape[0]
        rows = O.pack_rows(codes, bits, h.row_stride)
        store = np.ascontiguousarray(np.tile(rows[None], (U, 1, 1)))
        rep = K.kvtc_bytes(blob, store, None, S, S)
        rep.pop("device_store")
        return rep

    codes = np.zeros((8, 3), np.int64)
    codes[:, 0] = [0, 0, 0, 0, 0, 0, 1, 3]
    codes[:, 2] = 1
    assert run("dp", 1, 1, [2, 0, 1], codes) == dict(
        fixed_payload=3, entropy_payload=0, entropy_table=0, stored_payload=3, basis=384, quant_params=8,
        total=395, pre_entropy=395, fp16_equiv=1024, n_survived=2, units_entropy_coded=0)
    codes = np.zeros((1000, 2), np.int64)
    codes[:10, 0] = 255
    assert run("dp", 1, 1, [8, 0], codes) == dict(
        fixed_payload=1000, entropy_payload=125, entropy_table=256, stored_payload=125, basis=256,
        quant_params=4, total=641, pre_entropy=1260, fp16_equiv=128000, n_survived=1, units_entropy_coded=1)
    for S, coded, total in ((32, 0, 268), (40, 1, 269)):
        rep = run("dp", 1, 1, [2], np.full((S, 1), 2, np.int64))
        assert (rep["units_entropy_coded"], rep["total"]) == (coded, total)
    assert run("mixed", 2, 2, [4] * 16 + [2] * 16, np.ones((5, 32), np.int64), group_size=16,
               hi_fraction=0.5) == dict(
        fixed_payload=60, entropy_payload=0, entropy_table=0, stored_payload=60, basis=16896, quant_params=40,
        total=16996, pre_entropy=16996, fp16_equiv=1280, n_survived=32, units_entropy_coded=0)


@no_device_only
def test_attend_noalloc_rejects_a_call_beyond_its_scratch():
    """kvtc_attend_noalloc refuses, before touching the device, a call whose
    workspace would exceed KVTC_ATTEND_SCRATCH_BYTES (16 MiB)."""
    w = synth.WORKLOADS[1]
    st = O.fit(oracle_cfg(w), synth.generate(w, 0, 0, 256))
    blob = blob_from_oracle(st)
    fake = C.c_void_p(0x1000)        # never dereferenced: the size check fails first
    big = 1 << 29                    # rows: partial sums of 58255 segments (9216 rows) per unit
    assert K.kvtc_attend_workspace(blob, blob, big) > 16 << 20
    refs = []
    for _ in range(2):
        r = K.TensorRef()
        r.state_host, r.state_dev, r.codes_dev, r.capacity = blob.ctypes.data, 0x1000, 0x1000, big
        refs.append(r)
    fn = _raw("kvtc_attend_noalloc")
    fn.restype = C.c_int32
    fn.argtypes = K._sig["kvtc_attend_noalloc"][1]
    qs = (C.c_int64 * 3)(2 * 64, 64, 1)
    assert fn(C.byref(refs[0]), C.byref(refs[1]), fake, K.F16, qs, big, fake, qs, None) == K.E_BUFSIZE
