"""Decode attention from the codes on the general path, on MI355X, against the
oracle: grouped query heads over per-head caches (kvtc_attend_gqa) and
group-head caches (kvtc_attend and kvtc_attend_gqa; PALU cache API page,
"Design": latents are reconstructed only for attention).  The bar is the one of
the per-head tests: within 2e-3 of each value channel's range over the stored
rows, half an fp16 ulp, and 1e-5 of the largest value magnitude."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import kvtc_oracle as O
from kv_cache_compression_kvtc_amd import synth
from kv_cache_compression_kvtc_amd import kvtc as K

from gpu_helpers import DeviceStore, blob_from_oracle, oracle_cfg

pytestmark = pytest.mark.gpu


def print_case(*a):
    print("CASE", *a, flush=True)


def small(wid, **kw):
    w = synth.WORKLOADS[wid]
    fields = dict(w.__dict__)
    fields.update(kw)
    return synth.Workload(**fields)


def check(ref, got, Vh, G, what):
    """ref [B, Hq, D]; Vh [B, H, S, D], query head hq against KV head hq // G."""
    got = got.cpu().numpy().astype(np.float64)
    Vq = np.repeat(Vh, G, axis=1)
    rng_d = Vq.max(axis=2) - Vq.min(axis=2)
    bound = (2e-3 * rng_d + 0.5 * np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
             + 1e-5 * np.abs(Vq).max(axis=(2, 3))[:, :, None])
    err = np.abs(got - ref)
    i = np.unravel_index(np.argmax(err - bound), err.shape)
    assert (err <= bound).all(), (what, int((err > bound).sum()), i, float(err[i]), float(bound[i]))


GQA_CASES = [
    # name, workload, query heads per KV head
    ("llama-gqa4", small(2, s_total=4096 + 77), 4),
    ("batched-gqa2", small(4, B=3, s_prefill=2048, s_total=2048 + 45), 2),
    ("tiny-gqa3", small(1), 3),
    ("palu", small(3, H=16, s_prefill=2048, s_total=2048 + 33), 1),
    ("palu-gqa4", small(3, H=16, s_prefill=2048, s_total=2048 + 33), 4),
]


@pytest.mark.parametrize("name,w,G", GQA_CASES, ids=[c[0] for c in GQA_CASES])
def test_attend_general_path_matches_oracle(name, w, G):
    print_case("attend general", name)
    Xk, Xv = synth.generate(w, 0), synth.generate(w, 1)
    S = Xk.shape[2]
    sts = [O.fit(oracle_cfg(w), X[:, :, : w.s_prefill]) for X in (Xk, Xv)]
    stores = [DeviceStore(blob_from_oracle(st), S + 3) for st in sts]
    for ds, X in zip(stores, (Xk, Xv)):
        ds.append(X, 0)
    rows = [ds.rows(S) for ds in stores]
    prm = [ds.params_np(S) if ds.params is not None else None for ds in stores]
    refs = [(ds.blob, ds.blob_dev, ds.codes, ds.params) for ds in stores]
    Hq = w.H * G
    att = K.Attend(*refs, S + 3, q_heads=Hq)
    rng = np.random.default_rng(7)
    q = rng.normal(size=(w.B, Hq, w.D)) * 1.5
    qd = torch.from_numpy(q.astype(np.float32)).cuda()
    for s_end in (S, S - 300 if S > 600 else S // 2 + 1, 1):
        pk = None if prm[0] is None else prm[0][:, :s_end]
        pv = None if prm[1] is None else prm[1][:, :s_end]
        ref = O.attend(sts[0], rows[0][:, :s_end], sts[1], rows[1][:, :s_end], q, pk, pv)
        Vh = O.fetch(sts[1], rows[1][:, :s_end], pv)
        check(ref, att(qd, s_end), Vh, G, f"{name} s_end={s_end}")
    assert not att(qd, 0).float().abs().sum().item()            # empty cache: zeros
    if G == 1:
        # kvtc_attend (no query-head count) takes the same path for these caches
        plain = K.Attend(*refs, S + 3)
        assert torch.equal(plain(qd, S), att(qd, S))
        # and the allocation-free form agrees bit for bit
        out = torch.empty_like(plain(qd, S))
        plain.noalloc(qd, S, out)
        torch.cuda.synchronize()
        assert torch.equal(out, plain(qd, S))


def test_attend_group_head_full_size():
    """The group-head workload at full size (B=1, H=32 in 4 groups of 8,
    S=16384, rank 256), one query per head and 4 query heads per KV head."""
    print_case("attend group head full size")
    w = synth.WORKLOADS[3]
    S = w.s_total
    Xk, Xv = synth.generate(w, 0), synth.generate(w, 1)
    sts = [O.fit(oracle_cfg(w), X) for X in (Xk, Xv)]
    stores = [DeviceStore(blob_from_oracle(st), S) for st in sts]
    for ds, X in zip(stores, (Xk, Xv)):
        ds.append(torch.from_numpy(X).cuda(), 0)
    rows = [ds.rows(S) for ds in stores]
    prm = [ds.params_np(S) for ds in stores]
    Kh, Vh = O.fetch(sts[0], rows[0], prm[0]), O.fetch(sts[1], rows[1], prm[1])
    rng = np.random.default_rng(8)
    for G in (1, 4):
        att = K.Attend(*[(ds.blob, ds.blob_dev, ds.codes, ds.params) for ds in stores], S, q_heads=w.H * G)
        q = rng.normal(size=(1, w.H * G, w.D))
        got = att(torch.from_numpy(q.astype(np.float32)).cuda(), S)
        ref = np.zeros_like(q)
        for hq in range(w.H * G):
            ref[0, hq] = O.attend_rows(Kh[0, hq // G], Vh[0, hq // G], q[0, hq])
        check(ref, got, Vh, G, f"group head G={G}")
