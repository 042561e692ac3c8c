"""The int8 append path on MI355X against the fp64 path, byte for byte.

Bulk appends of fp16 rows run on int8 MFMA: an exact integer product of the
rows' and the basis's digits, each decision (code, group-head fp16 range)
certified against an error bound, and the fp64 tile of the bulk kernel for any
block with a decision it cannot certify.  The same rows given as fp32 take the
fp64 kernels with the same values (every fp16 value is exact in fp32), so both
calls must store identical codes and params.  The oracle comparison of these
stores is in test_gpu_parity.py; here the two device paths are held to
identity, including blocks that must fall back: rows outside the int8 range and
decisions too close to a rounding boundary to certify.  The int8 path serves
wide units (group-head caches); narrower ones take the fp64 kernels.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import kvtc_oracle as O
from kv_cache_compression_kvtc_amd import synth
from kv_cache_compression_kvtc_amd import kvtc as K

from gpu_helpers import DeviceStore, blob_from_oracle, oracle_cfg

pytestmark = pytest.mark.gpu


def small(wid, **kw):
    w = synth.WORKLOADS[wid]
    fields = dict(w.__dict__)
    fields.update(kw)
    return synth.Workload(**fields)


def print_case(*a):
    print("CASE", *a, flush=True)


def both_paths(blob, X, cuts):
    """Stores of X appended in the pieces [cuts[i], cuts[i+1]) as fp16 and as fp32 rows."""
    S = X.shape[2]
    out = []
    for dt in (np.float16, np.float32):
        ds = DeviceStore(blob, capacity=S + 5)
        xd = torch.from_numpy(np.ascontiguousarray(X.astype(dt))).cuda()
        for a, b in zip(cuts[:-1], cuts[1:]):
            ds.append(xd[:, :, a:b], a)
        rows = ds.rows(S).copy()
        prm = ds.params_np(S).copy() if ds.params is not None else None
        out.append((rows, prm))
    return out


def assert_same(paths, what):
    (r16, p16), (r32, p32) = paths
    bad = np.argwhere(r16 != r32)
    assert bad.size == 0, f"{what}: {len(bad)} code bytes differ, first at {bad[:3].tolist()}"
    if p16 is not None:
        assert np.array_equal(p16.view(np.uint16), p32.view(np.uint16)), f"{what}: params differ"


I8_CASES = [
    # name, workload, tensor: group-head units (1024 features, 256 or 160 slots
    # in groups of 64 per block)
    ("palu-k", small(3, H=16, s_prefill=2048, s_total=2048 + 45), 0),
    ("palu-v", small(3, H=16, s_prefill=2048, s_total=2048 + 45), 1),
    ("palu-v-rank160", small(3, H=16, s_prefill=2048, s_total=2048 + 45, rank=160), 1),
]


def uncertain_groups(st, X):
    """(token, group) pairs of unit rows X whose fp16 range or codes the int8
    path cannot certify even with half its error bound around the oracle's
    float64 latents: their blocks must take the fp64 tile.  The bound is the
    kernel's, E = 2^-39 (1.5 sum|x| + 1.1 dg + 0.5 sum|mu|)."""
    xu = O.gather_units(X, st.hpu)
    out = 0
    for u in range(st.U):
        r = int(st.r[u])
        L = O.project(xu[u], st.mu32[u], st.V32[u][:, :r])
        E = 0.5 * 2.0 ** -39 * (1.5 * np.abs(xu[u].astype(np.float64)).sum(1) + 1.1 * st.Dg +
                                0.5 * np.abs(st.mu32[u].astype(np.float64)).sum())
        for g0 in range(0, r, 32):
            Lg = L[:, g0:g0 + 32]
            cm = 2.0 ** int(st.bits[u, g0]) - 1
            mn, mx = Lg.min(1), Lg.max(1)
            h = lambda v: v.astype(np.float16)
            bad = (h(mn - E) != h(mn + E)) | (h((mx - E - (mn + E)) / cm) != h((mx + E - (mn - E)) / cm))
            lo = h(mn).astype(np.float64)
            sc = h((mx - mn) / cm).astype(np.float64)
            inv = np.where(sc > 0, 1.0 / np.where(sc > 0, sc, 1.0), 0.0)
            q = lambda l: np.clip(np.rint((l - lo[:, None]) * inv[:, None]), 0, cm)
            bad |= (q(Lg - E[:, None]) != q(Lg + E[:, None])).any(1)
            out += int(bad.sum())
    return out


@pytest.mark.parametrize("name,w,tensor", I8_CASES, ids=[c[0] for c in I8_CASES])
def test_int8_append_stores_the_bytes_of_the_fp64_path(name, w, tensor):
    print_case("i8 paths", name)
    X = synth.generate(w, tensor)
    st = O.fit(oracle_cfg(w), X[:, :, : w.s_prefill])
    blob = blob_from_oracle(st)
    assert K.header(blob).off_vdig != 0
    S = X.shape[2]
    if name == "palu-k":
        # the case holds decisions the int8 path must leave to the fp64 tile
        assert uncertain_groups(st, X) > 0
    # a bulk prefill, a ragged 17-row append and the rest
    cuts = [0, w.s_prefill, w.s_prefill + 17, S]
    assert_same(both_paths(blob, X, cuts), name)


@pytest.mark.parametrize("name,w,tensor", [I8_CASES[0]], ids=["palu-k"])
def test_rows_outside_the_int8_range_fall_back(name, w, tensor):
    print_case("i8 range fallback", name)
    X = synth.generate(w, tensor)
    st = O.fit(oracle_cfg(w), X[:, :, : w.s_prefill])
    blob = blob_from_oracle(st)
    X = X.copy()
    rng = np.random.default_rng(5)
    S = X.shape[2]
    for t in rng.choice(S, size=6, replace=False):
        X[:, :, t, :] = (X[:, :, t, :].astype(np.float32) * 300.0).astype(X.dtype)   # |x| well above 127
    assert_same(both_paths(blob, X, [0, S]), name)
