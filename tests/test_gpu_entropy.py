"""Entropy-coded storage on MI355X (kvtc_entropy_encode / kvtc_entropy_decode)
against the oracle.

KVTC cache module page, "Byte accounting": order-0 Huffman per kept component
with a fixed-width fallback.  On the same device store:
* the archive's size is the accounting's stored payload plus tables (the
  oracle's bytes_report and the library's kvtc_bytes);
* its bytes equal the oracle's archive of the same rows, byte for byte (both
  build code lengths with the documented tie-breaking rule, canonical codes,
  the same layout); the code lengths are those of an optimal code;
* decoding restores the packed rows bit for bit, and a fetch of the decoded
  store equals a fetch of the original.
"""
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


ENTROPY_CASES = [
    ("tiny-k", small(1), 0, 288),
    ("tiny-v-fixed-width", small(1), 1, 40),
    ("llama-k", small(2, s_total=4096 + 40), 0, 4096 + 40),
    ("batched-b3-v", small(4, B=3, s_prefill=700, s_total=700), 1, 700),
    ("long-k-r4", small(5, s_prefill=4096, s_total=4096 + 300), 0, 4096 + 300),
    # 256 slots of 8 bits: 256-byte rows and 64 K symbol positions per unit, the
    # decoder's variant with the symbol lists in global memory (too large for
    # LDS next to the rows and tables)
    ("wide-rows-8bit", small(2, D=256, H=1, rank=256, budget=2048, choices=(0, 8), n_outliers_k=0,
                             s_prefill=600, s_total=600), 0, 600),
]


@pytest.mark.parametrize("name,w,tensor,S", ENTROPY_CASES, ids=[c[0] for c in ENTROPY_CASES])
def test_entropy_archive_matches_oracle_and_round_trips(name, w, tensor, S):
    print_case("entropy", name)
    X = synth.generate(w, tensor, 0, max(S, w.s_prefill))
    st = O.fit(oracle_cfg(w), X[:, :, : w.s_prefill])
    cap = X.shape[2] + 5
    ds = DeviceStore(blob_from_oracle(st), cap)
    ds.append(X, 0)
    rows = ds.rows(S)
    arc = K.EntropyArchive(ds.blob, ds.blob_dev, ds.codes, cap, S)
    h = arc.header
    rep = O.bytes_report(st, rows, None, S)
    lib = K.kvtc_bytes(ds.blob, ds.codes.cpu().numpy(), None, cap, S)
    assert h.archive_bytes == rep.stored_payload + rep.entropy_table
    assert (h.payload_bytes, h.table_bytes, h.units_coded) == (rep.stored_payload, rep.entropy_table,
                                                               rep.units_entropy_coded)
    assert (lib["stored_payload"], lib["entropy_table"]) == (rep.stored_payload, rep.entropy_table)
    want, info = O.entropy_archive(st, rows, S)
    got = arc.bytes()
    assert [bool(u.coded) for u in arc.units()] == [c for c, _, _ in info]
    assert [(u.offset, u.bytes) for u in arc.units()] == [(o, n) for _, o, n in info]
    assert got.tobytes() == want, name
    # restore into a fresh store: the rows and the fetch come back exactly
    back = DeviceStore(ds.blob, cap)
    back.codes.fill_(0xA5)
    arc.decode(back.codes, cap)
    assert np.array_equal(back.rows(S), rows)
    if st.row_stride <= 192:                           # rows the fetch kernels take
        assert torch.equal(back.fetch(0, S), ds.fetch(0, S))


def test_entropy_full_size_batched_decode():
    """The batched-decode store at full size (512 units x 8193 rows, K and V):
    archive size equal to the library's accounting and an exact round trip;
    two sampled units' parts decoded by the oracle from the device's tables."""
    print_case("entropy full size")
    w = synth.WORKLOADS[4]
    S = w.s_prefill + 1
    for tensor in (0, 1):
        X = synth.generate(w, tensor, 0, S)
        x = torch.from_numpy(X).cuda()
        blob = K.kvtc_fit_device(K.make_config(w.mode, w.D, 1, w.rank, budget=w.budget, choices=w.choices),
                                 x[:, :, : w.s_prefill])
        ds = DeviceStore(blob, S)
        ds.append(x, 0)
        arc = K.EntropyArchive(ds.blob, ds.blob_dev, ds.codes, S, S)
        lib = K.kvtc_bytes(ds.blob, ds.codes.cpu().numpy(), None, S, S)
        assert arc.header.archive_bytes == lib["stored_payload"] + lib["entropy_table"]
        back = DeviceStore(ds.blob, S)
        arc.decode(back.codes, S)
        torch.cuda.synchronize()
        assert torch.equal(back.codes, ds.codes)
        print(f"tensor {tensor}: fixed {lib['fixed_payload']} B -> archive {arc.header.archive_bytes} B "
              f"({arc.header.units_coded} of 512 units coded)", flush=True)
        # two units decoded by the oracle from the archive's own tables
        v = K.state_view(blob)
        data = arc.bytes().tobytes()
        rows = ds.rows(S)
        for un_i in (3, 300):
            un = arc.units()[un_i]
            assert un.coded
            r = int(v["rank"][un_i])
            bits = [int(b) for b in v["bits"][un_i, :r]]
            part = data[un.offset: un.offset + un.bytes]
            lens, p = [None] * r, 0
            for i, b in enumerate(bits):
                if b:
                    lens[i] = np.frombuffer(part[p: p + 2 ** b], np.uint8).astype(np.int64)
                    p += 2 ** b
            # the first slot's stream opens the unit's stream: its first 600 codes
            first = next(i for i, b in enumerate(bits) if b)
            codes = O.entropy_decode_unit(part[p:], 600, [bits[first]], [lens[first]])
            assert np.array_equal(codes[:, 0], O.unpack_rows(rows[un_i], bits)[:600, first])
