"""CPU oracle for transform-coded KV-cache append/fetch -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path (the C-ABI library and
its Python binding) never imports, calls or links anything under ``oracle/``,
and this module imports nothing from the product.

Everything here is plain NumPy in float64, written step by step from three
documentation pages:

* the KVTC cache module page (``veloxquant_mlx.cache.kvtc_cache`` source):
  module docstring sections "NOT PATH-DEPENDENT", "Design" and "Byte
  accounting"; ``_TensorKVTC.fit_prefill_from_pca``, ``append`` and
  ``_requantize``; ``KVTCKVCache.__init__`` (config fields), ``update_and_fetch``
  and the byte properties;
* the TurboQuant cache module page (``veloxquant_mlx.cache.turboquant_cache``
  source): ``__init__`` (packed row length), ``_unpack_indices_block`` (the
  little-endian field order of its bit packer) and ``attend`` (one query per
  head: scores against the stored keys divided by sqrt(d), softmax over the
  stored rows, weighted sum of the decoded values);
* the PALU cache API page (``veloxquant_mlx.cache.palu_cache``): "Design",
  "Byte accounting" and the ``PALUKVCache`` parameter list.

Readings taken where the pages are silent (each is also listed with its
reason in the design notes of the repository):

* min/scale of each DP component are frozen at prefill; later latents outside
  the prefill range clamp to the end codes (``clamp_fraction`` measures how
  often); ``refit`` / ``append_refit`` give the page's own alternative, the
  ranges refitted over every accumulated row on each call;
* the DP's "analytic distortion proxy" is ``D_i(0) = lam_i`` (dropped) and
  ``D_i(b) = beta * lam_i * 4**-b`` (Gaussian distortion-rate), ties broken
  towards fewer bits;
* the quantiser is min/max affine with ``2**b`` levels, round-half-even, clamp;
* codes are packed token-major, least-significant bit first, in component
  order; a row is padded with zero bits to a whole number of 32-bit words;
* the group-head "group size" is a per-token group of consecutive latent
  components with an fp16 (min, scale) pair;
* Huffman tables cost one byte per symbol of a component's alphabet.

Parity unpinned (no value on the pages to check against, only the reading
above): the DP proxy and ``beta``; frozen versus refit ranges; the Huffman
table format; the meaning of the group-head quantisation group; the sign
convention of eigenvectors.
"""
from __future__ import annotations

from dataclasses import dataclass
import heapq
import math

import numpy as np

ALLOWED_BITS = (0, 1, 2, 3, 4, 8)


# --------------------------------------------------------------------------
# configuration (mirrors the cache's config fields; KVTC cache module page,
# ``KVTCKVCache.__init__``; PALU cache API page, ``PALUKVCache`` parameters)
# --------------------------------------------------------------------------
@dataclass
class Config:
    mode: str = "dp"            # "dp": per-unit DP bits; "mixed": hi/lo group-head bits
    head_dim: int = 128
    heads_per_unit: int = 1
    rank: int = 0               # > 0 fixed rank; 0 -> energy threshold
    energy: float = 0.90
    budget: int = -1            # DP: bits per token; < 0 -> 4 * head_dim (page default)
    choices: tuple = (0, 1, 2, 3, 4, 8)
    beta: float = 1.0
    hi_bits: int = 4
    lo_bits: int = 2
    hi_fraction: float = 0.25
    group_size: int = 32

    def resolved_budget(self) -> int:
        return 4 * self.head_dim if self.budget < 0 else self.budget


class OracleConfigError(ValueError):
    pass


# --------------------------------------------------------------------------
# fit: local PCA (KVTC page, "Design" step 1 and ``update_and_fetch``: one
# local PCA per (batch, head) on the prefill rows; PALU page, "Design" step 2:
# one shared projection per contiguous head group)
# --------------------------------------------------------------------------
def pca_fit(X: np.ndarray):
    """Mean, eigenvalues (descending, clamped at 0) and eigenvectors (columns).

    Covariance with 1/S normalisation.  Each eigenvector is signed so that its
    entry of largest magnitude is positive (first such entry on ties).
    """
    X = np.asarray(X, dtype=np.float64)
    S = X.shape[0]
    mean = X.sum(axis=0) / S
    Y = X - mean[None, :]
    C = (Y.T @ Y) / S
    lam, V = np.linalg.eigh(C)
    order = np.argsort(-lam, kind="stable")
    lam = np.maximum(lam[order], 0.0)
    V = V[:, order]
    for j in range(V.shape[1]):
        k = int(np.argmax(np.abs(V[:, j])))
        if V[k, j] < 0:
            V[:, j] = -V[:, j]
    return mean, lam, V


def energy_rank(lam: np.ndarray, tau: float) -> int:
    """Smallest k >= 1 whose leading eigenvalues hold at least tau of the total.

    PALU page, ``palu_rank=None`` -> ``palu_energy_threshold`` (default 0.90).
    """
    total = 0.0
    for v in lam:
        total += float(v)
    if total <= 0.0:
        return 1
    acc = 0.0
    for k, v in enumerate(lam, start=1):
        acc += float(v)
        if acc >= tau * total:
            return k
    return len(lam)


# --------------------------------------------------------------------------
# bit allocation (KVTC page, opening docstring: DP-optimal, discrete,
# per-component, a component may get 0 bits; ``KVTCKVCache.__init__``:
# ``kvtc_bit_budget`` = total bits per token over all components)
# --------------------------------------------------------------------------
def distortion(lam_i: float, b: int, beta: float) -> float:
    """Proxy distortion of one component at b bits (0 bits drops it)."""
    if b == 0:
        return lam_i
    return beta * lam_i * (4.0 ** (-b))


def allocate_dp(lam: np.ndarray, budget: int, choices, beta: float) -> np.ndarray:
    """Exact DP over (component, bits used); minimise total proxy distortion.

    ``best[c]`` after component i is the least distortion of components
    0..i using exactly c bits.  Candidate widths are tried in ascending order
    and replace the incumbent only when strictly smaller, so the narrower width
    wins ties; the final total is chosen the same way, so fewer bits win ties.
    """
    choices = sorted(set(int(b) for b in choices))
    r = len(lam)
    if budget < 0:
        raise OracleConfigError("budget must be >= 0")
    inf = math.inf
    best = np.full(budget + 1, inf)
    best[0] = 0.0
    pick = np.zeros((r, budget + 1), dtype=np.int64)
    for i in range(r):
        nxt = np.full(budget + 1, inf)
        arg = np.full(budget + 1, -1, dtype=np.int64)
        for b in choices:
            if b > budget:
                continue
            cand = np.full(budget + 1, inf)
            cand[b:] = best[: budget + 1 - b] + distortion(float(lam[i]), b, beta)
            better = cand < nxt
            nxt[better] = cand[better]
            arg[better] = b
        best = nxt
        pick[i] = arg
    c_end, v_end = -1, inf
    for c in range(budget + 1):
        if best[c] < v_end:
            v_end, c_end = best[c], c
    if c_end < 0:
        raise OracleConfigError("budget infeasible for the bit choices")
    bits = np.zeros(r, dtype=np.int64)
    c = c_end
    for i in range(r - 1, -1, -1):
        bits[i] = pick[i, c]
        c -= bits[i]
    assert c == 0
    return bits


def dp_objective(lam: np.ndarray, bits: np.ndarray, beta: float) -> float:
    return float(sum(distortion(float(l), int(b), beta) for l, b in zip(lam, bits)))


def allocate_mixed(r: int, hi: int, lo: int, hi_fraction: float, group_size: int) -> np.ndarray:
    """Leading components at ``hi`` bits, the rest at ``lo`` (PALU page, mixed-bit).

    The hi count is rounded to a whole number of quantisation groups.
    """
    n_hi = group_size * int(math.floor(hi_fraction * r / group_size + 0.5))
    n_hi = min(max(n_hi, 0), r)
    bits = np.full(r, lo, dtype=np.int64)
    bits[:n_hi] = hi
    return bits


# --------------------------------------------------------------------------
# projection, quantisation (KVTC page, ``_TensorKVTC._requantize``: centre,
# multiply by the frozen basis, quantise each surviving component)
# --------------------------------------------------------------------------
def project(X: np.ndarray, mu32: np.ndarray, V32: np.ndarray) -> np.ndarray:
    """Latents ``(x - mean) @ V`` in float64 from the stored fp32 mean and basis."""
    Y = np.asarray(X, dtype=np.float64) - mu32.astype(np.float64)[None, :]
    return Y @ V32.astype(np.float64)


def frozen_ranges(Xp: np.ndarray, mu32, V32, bits):
    """Per-component (min, scale) over the prefill latents, stored as fp32.

    ``scale = (max - min) / (2**b - 1)``; a constant component gets scale 0.
    Dropped components keep (0, 0).
    """
    L = project(Xp, mu32, V32)
    r = V32.shape[1]
    qmin = np.zeros(r, dtype=np.float32)
    qscale = np.zeros(r, dtype=np.float32)
    for i in range(r):
        b = int(bits[i])
        if b == 0:
            continue
        lo = float(L[:, i].min())
        hi = float(L[:, i].max())
        qmin[i] = np.float32(lo)
        qscale[i] = np.float32((hi - lo) / (2 ** b - 1)) if hi > lo else np.float32(0.0)
    return qmin, qscale


def quantize_affine(l, lo, scale, b: int) -> np.ndarray:
    """``clamp(round_half_even((l - lo) / scale), 0, 2**b - 1)``; scale 0 gives code 0.

    ``lo`` and ``scale`` broadcast against ``l`` (scalars for a DP component,
    per-token columns for a group-head quantisation group).
    """
    l = np.asarray(l, dtype=np.float64)
    lo = np.asarray(lo, dtype=np.float64)
    scale = np.asarray(scale, dtype=np.float64)
    safe = np.where(scale == 0.0, 1.0, scale)
    t = (l - lo) / safe
    c = np.rint(t)
    c = np.where(np.isnan(c) | (scale == 0.0), 0.0, c)
    return np.clip(c, 0, 2 ** b - 1).astype(np.int64)


def quantize_dp(L: np.ndarray, bits, qmin32, qscale32) -> np.ndarray:
    codes = np.zeros(L.shape, dtype=np.int64)
    for i, b in enumerate(bits):
        if b:
            codes[:, i] = quantize_affine(L[:, i], float(qmin32[i]), float(qscale32[i]), int(b))
    return codes


def quantize_mixed(L: np.ndarray, bits, group_size: int):
    """Per token and per group of consecutive components: fp16 (min, scale), then codes.

    ``min16 = fp16(min)``, ``scale16 = fp16((max - min) / (2**b - 1))``, both
    rounded to nearest-even from float64; codes are taken against the fp16
    pair, which is what the fetch sees.
    """
    n, r = L.shape
    ng = (r + group_size - 1) // group_size
    codes = np.zeros((n, r), dtype=np.int64)
    params = np.zeros((n, ng, 2), dtype=np.float16)
    for g in range(ng):
        a, e = g * group_size, min(r, (g + 1) * group_size)
        b = int(bits[a])
        seg = L[:, a:e]
        mn = seg.min(axis=1)
        mx = seg.max(axis=1)
        min16 = mn.astype(np.float16)
        scale16 = ((mx - mn) / (2 ** b - 1)).astype(np.float16)
        params[:, g, 0] = min16
        params[:, g, 1] = scale16
        codes[:, a:e] = quantize_affine(seg, min16.astype(np.float64)[:, None],
                                        scale16.astype(np.float64)[:, None], b)
    return codes, params


# --------------------------------------------------------------------------
# bit packing (TurboQuant page: a b-bit field of coordinate j sits at bit
# offset j*b of the row, least significant bit first -- its vectorised unpack
# reads field k of a byte as (byte >> k*b) & (2**b - 1) and uses numpy's
# little bit order for b = 1)
# --------------------------------------------------------------------------
def field_offsets(bits) -> tuple[np.ndarray, int]:
    """Bit offset of each component's field in a row, and the row's bit count."""
    offs = np.zeros(len(bits), dtype=np.int64)
    o = 0
    for i, b in enumerate(bits):
        offs[i] = o
        o += int(b)
    return offs, o


def row_stride_bytes(row_bits: int) -> int:
    """Bytes per stored row: whole 32-bit words."""
    return 4 * ((row_bits + 31) // 32)


def pack_rows(codes: np.ndarray, bits, row_stride: int) -> np.ndarray:
    n = codes.shape[0]
    offs, row_bits = field_offsets(bits)
    assert row_bits <= 8 * row_stride
    plane = np.zeros((n, 8 * row_stride), dtype=np.uint8)
    for i, b in enumerate(bits):
        for j in range(int(b)):
            plane[:, offs[i] + j] = (codes[:, i] >> j) & 1
    return np.packbits(plane, axis=1, bitorder="little")


def unpack_rows(rows: np.ndarray, bits) -> np.ndarray:
    plane = np.unpackbits(np.asarray(rows, dtype=np.uint8), axis=1, bitorder="little").astype(np.int64)
    offs, _ = field_offsets(bits)
    codes = np.zeros((rows.shape[0], len(bits)), dtype=np.int64)
    for i, b in enumerate(bits):
        for j in range(int(b)):
            codes[:, i] |= plane[:, offs[i] + j] << j
    return codes


# --------------------------------------------------------------------------
# dequantisation and reconstruction (KVTC page, ``kvtc_decompress`` result:
# fp16 [S_total, D] per (batch, head); PALU page: latent -> dequant ->
# reconstruct on every fetch)
# --------------------------------------------------------------------------
def dequant_dp(codes: np.ndarray, bits, qmin32, qscale32) -> np.ndarray:
    Lh = np.zeros(codes.shape, dtype=np.float64)
    for i, b in enumerate(bits):
        if b:
            Lh[:, i] = float(qmin32[i]) + codes[:, i].astype(np.float64) * float(qscale32[i])
    return Lh


def dequant_mixed(codes: np.ndarray, params: np.ndarray, group_size: int) -> np.ndarray:
    n, r = codes.shape
    Lh = np.zeros((n, r), dtype=np.float64)
    for g in range(params.shape[1]):
        a, e = g * group_size, min(r, (g + 1) * group_size)
        mn = params[:, g, 0].astype(np.float64)[:, None]
        sc = params[:, g, 1].astype(np.float64)[:, None]
        Lh[:, a:e] = mn + codes[:, a:e].astype(np.float64) * sc
    return Lh


def reconstruct(Lh: np.ndarray, mu32: np.ndarray, V32: np.ndarray) -> np.ndarray:
    """``latent @ V^T + mean`` in float64."""
    return Lh @ V32.astype(np.float64).T + mu32.astype(np.float64)[None, :]


# --------------------------------------------------------------------------
# order-0 Huffman cost (KVTC page, "Byte accounting": entropy-coded payload +
# table, never above fixed width because fixed width is kept when Huffman
# does not pay for itself)
# --------------------------------------------------------------------------
def huffman_bits(counts) -> int:
    """Total coded bits of an optimal prefix code for these symbol counts.

    Equals the sum of the weights of all internal nodes of a Huffman tree.
    A single distinct symbol still costs one bit per occurrence.
    """
    w = [int(c) for c in counts if c > 0]
    if not w:
        return 0
    if len(w) == 1:
        return w[0]
    heapq.heapify(w)
    total = 0
    while len(w) > 1:
        a = heapq.heappop(w)
        b = heapq.heappop(w)
        total += a + b
        heapq.heappush(w, a + b)
    return total


def huffman_lengths(counts) -> np.ndarray:
    """Code length of every symbol in an optimal prefix code for these counts
    (0 for absent symbols): the depths of the leaves of a Huffman tree.  A lone
    symbol gets length 1.  Which of several optimal length sets comes out depends
    on tie-breaking; the total ``sum(counts * lengths)`` does not and equals
    ``huffman_bits(counts)``."""
    counts = [int(c) for c in counts]
    lengths = np.zeros(len(counts), dtype=np.int64)
    live = [i for i, c in enumerate(counts) if c > 0]
    if len(live) == 1:
        lengths[live[0]] = 1
    if len(live) <= 1:
        return lengths
    # heap of (weight, tiebreak, symbols under the node); every merge deepens its symbols by one
    heap = [(counts[i], i, [i]) for i in live]
    heapq.heapify(heap)
    nxt = len(counts)
    while len(heap) > 1:
        wa, _, sa = heapq.heappop(heap)
        wb, _, sb = heapq.heappop(heap)
        for i in sa + sb:
            lengths[i] += 1
        heapq.heappush(heap, (wa + wb, nxt, sa + sb))
        nxt += 1
    return lengths


def canonical_codes(lengths) -> np.ndarray:
    """Canonical prefix code of the given lengths: symbols ordered by (length,
    symbol value) take consecutive code values, the value doubling (shifted
    left) whenever the length grows; codes are read most significant bit first."""
    lengths = np.asarray(lengths, dtype=np.int64)
    codes = np.zeros(len(lengths), dtype=np.int64)
    order = sorted((int(l), i) for i, l in enumerate(lengths) if l > 0)
    code, prev = 0, 0
    for k, (l, i) in enumerate(order):
        if k:
            code += 1
        code <<= (l - prev)
        prev = l
        codes[i] = code
    return codes


def entropy_encode_unit(codes: np.ndarray, bits, lengths) -> bytes:
    """One unit's entropy-coded payload: for each stored component in order, its
    codes of every row in row order, each written as its canonical prefix code,
    most significant code bit first; the stream's bit p is bit p % 8 of byte
    p // 8 (the little-endian bit order of the code rows); zero-padded to whole
    bytes.  ``codes [S, r]`` per component, ``lengths[i]`` the symbol lengths of
    component i (ignored for dropped components)."""
    out = []
    for i, b in enumerate(bits):
        if not b:
            continue
        can = canonical_codes(lengths[i])
        for c in codes[:, i]:
            l, v = int(lengths[i][c]), int(can[c])
            out.extend((v >> (l - 1 - k)) & 1 for k in range(l))
    out.extend([0] * (-len(out) % 8))
    return np.packbits(np.array(out, dtype=np.uint8), bitorder="little").tobytes()


def entropy_decode_unit(payload: bytes, S: int, bits, lengths) -> np.ndarray:
    """Inverse of entropy_encode_unit: codes ``[S, r]`` (zero for dropped
    components), decoded bit by bit against the canonical code of each
    component's lengths."""
    stream = np.unpackbits(np.frombuffer(payload, dtype=np.uint8), bitorder="little")
    codes = np.zeros((S, len(bits)), dtype=np.int64)
    p = 0
    for i, b in enumerate(bits):
        if not b:
            continue
        can = canonical_codes(lengths[i])
        table = {(int(lengths[i][c]), int(can[c])): c for c in range(len(can)) if lengths[i][c] > 0}
        for s in range(S):
            v, l = 0, 0
            while (l, v) not in table:
                v = (v << 1) | int(stream[p])
                p += 1
                l += 1
                assert l <= 64, "not a prefix code of these lengths"
            codes[s, i] = table[(l, v)]
    return codes


# --------------------------------------------------------------------------
# whole-tensor state, append, fetch
# --------------------------------------------------------------------------
@dataclass
class TensorState:
    """Frozen per-tensor state (K or V), one entry per unit."""
    cfg: Config
    B: int
    H: int
    D: int
    hpu: int
    r: np.ndarray          # [U] kept rank per unit
    mu32: np.ndarray       # [U, Dg] float32
    lam: np.ndarray        # [U, Dg] float64 eigenvalues, descending
    V32: np.ndarray        # [U, Dg, rmax] float32 basis (columns are components)
    bits: np.ndarray       # [U, rmax] bits per component (0 = dropped)
    qmin32: np.ndarray     # [U, rmax] float32 (DP)
    qscale32: np.ndarray   # [U, rmax] float32 (DP)
    row_stride: int

    @property
    def U(self) -> int:
        return self.mu32.shape[0]

    @property
    def Dg(self) -> int:
        return self.mu32.shape[1]

    def row_bits(self, u: int) -> int:
        return int(self.bits[u].sum())

    def n_groups(self) -> int:
        rmax = self.bits.shape[1]
        gs = self.cfg.group_size
        return (rmax + gs - 1) // gs


def gather_units(x: np.ndarray, hpu: int) -> np.ndarray:
    """[B, H, n, D] -> [U, n, hpu*D]: unit (b, g) concatenates heads g*hpu .. g*hpu+hpu-1."""
    B, H, n, D = x.shape
    G = H // hpu
    y = x.reshape(B, G, hpu, n, D).transpose(0, 1, 3, 2, 4)
    return y.reshape(B * G, n, hpu * D)


def scatter_units(y: np.ndarray, B: int, H: int, hpu: int) -> np.ndarray:
    U, n, Dg = y.shape
    D = Dg // hpu
    G = H // hpu
    return y.reshape(B, G, n, hpu, D).transpose(0, 1, 3, 2, 4).reshape(B, H, n, D)


def validate(cfg: Config, H: int, S: int):
    if cfg.mode not in ("dp", "mixed"):
        raise OracleConfigError("mode")
    if cfg.heads_per_unit < 1 or H % cfg.heads_per_unit:
        raise OracleConfigError("heads_per_unit must divide H")
    if S < 2:
        raise OracleConfigError("a prefill needs at least 2 rows")
    if cfg.mode == "dp":
        if cfg.resolved_budget() < 0:
            raise OracleConfigError("budget must be >= 0")
        if not cfg.choices or any(int(b) not in ALLOWED_BITS for b in cfg.choices):
            raise OracleConfigError("bit choices")
    else:
        if cfg.hi_bits not in ALLOWED_BITS[1:] or cfg.lo_bits not in ALLOWED_BITS[1:]:
            raise OracleConfigError("mixed widths")
        if cfg.group_size < 1:
            raise OracleConfigError("group size")
    if cfg.rank < 0 or cfg.rank > cfg.head_dim * cfg.heads_per_unit:
        raise OracleConfigError("rank")


def fit(cfg: Config, X: np.ndarray) -> TensorState:
    """Fit one tensor's frozen state on its prefill rows ``X [B, H, S, D]``."""
    B, H, S, D = X.shape
    assert D == cfg.head_dim
    validate(cfg, H, S)
    hpu = cfg.heads_per_unit
    Xu = gather_units(np.asarray(X, dtype=np.float64), hpu)
    U, _, Dg = Xu.shape
    fits = [pca_fit(Xu[u]) for u in range(U)]
    if cfg.rank > 0:
        ranks = [cfg.rank] * U
    else:
        ranks = [energy_rank(lam, cfg.energy) for _, lam, _ in fits]
        if cfg.mode == "mixed":           # one stored rank for every head group
            ranks = [max(ranks)] * U
    rmax = max(ranks)
    mu32 = np.zeros((U, Dg), np.float32)
    lam_all = np.zeros((U, Dg), np.float64)
    V32 = np.zeros((U, Dg, rmax), np.float32)
    bits = np.zeros((U, rmax), np.int64)
    qmin = np.zeros((U, rmax), np.float32)
    qscale = np.zeros((U, rmax), np.float32)
    for u, (mean, lam, V) in enumerate(fits):
        r = ranks[u]
        mu32[u] = mean.astype(np.float32)
        lam_all[u] = lam
        V32[u, :, :r] = V[:, :r].astype(np.float32)
        if cfg.mode == "dp":
            bits[u, :r] = allocate_dp(lam[:r], cfg.resolved_budget(), cfg.choices, cfg.beta)
            qmin[u, :r], qscale[u, :r] = frozen_ranges(Xu[u], mu32[u], V32[u, :, :r], bits[u, :r])
        else:
            bits[u, :r] = allocate_mixed(r, cfg.hi_bits, cfg.lo_bits, cfg.hi_fraction, cfg.group_size)
    stride = max(row_stride_bytes(int(bits[u].sum())) for u in range(U))
    return TensorState(cfg, B, H, D, hpu, np.array(ranks), mu32, lam_all, V32, bits, qmin, qscale,
                       stride)


def append(st: TensorState, x: np.ndarray):
    """Encode new rows ``x [B, H, n, D]``: returns packed rows ``[U, n, stride]``
    (uint8) and, for the group-head mode, params ``[U, n, n_groups, 2]`` (fp16)."""
    xu = gather_units(np.asarray(x), st.hpu)
    U, n, _ = xu.shape
    rows = np.zeros((U, n, st.row_stride), np.uint8)
    params = np.zeros((U, n, st.n_groups(), 2), np.float16) if st.cfg.mode == "mixed" else None
    for u in range(U):
        r = int(st.r[u])
        L = project(xu[u], st.mu32[u], st.V32[u, :, :r])
        bits = st.bits[u, :r]
        if st.cfg.mode == "dp":
            codes = quantize_dp(L, bits, st.qmin32[u, :r], st.qscale32[u, :r])
        else:
            codes, p = quantize_mixed(L, bits, st.cfg.group_size)
            params[u, :, : p.shape[1]] = p
        rows[u] = pack_rows(codes, bits, st.row_stride)
    return rows, params


def refit(st: TensorState, X_all: np.ndarray) -> TensorState:
    """Refit mode: the KVTC page's own decode semantics (``_TensorKVTC.append``
    concatenates the new rows to every row accumulated so far and
    ``_requantize`` re-projects them all through the frozen basis and mean,
    then quantises each kept component with a min/max fitted over all of
    them).  Basis, mean and widths stay frozen; only the per-component
    (min, scale) are recomputed over the accumulated rows ``X_all [B, H, S, D]``,
    in the same form as the prefill ranges (float32 min and scale of the
    float64 latents).  DP mode only: group-head rows carry their own per-token
    ranges.  Returns a new state; ``st`` is unchanged."""
    assert st.cfg.mode == "dp"
    xu = gather_units(np.asarray(X_all), st.hpu)
    qmin = np.zeros_like(st.qmin32)
    qscale = np.zeros_like(st.qscale32)
    for u in range(st.U):
        r = int(st.r[u])
        qmin[u, :r], qscale[u, :r] = frozen_ranges(xu[u], st.mu32[u], st.V32[u, :, :r], st.bits[u, :r])
    return TensorState(st.cfg, st.B, st.H, st.D, st.hpu, st.r, st.mu32, st.lam, st.V32, st.bits, qmin, qscale,
                       st.row_stride)


def append_refit(st: TensorState, X_all: np.ndarray):
    """Refit-mode store of the accumulated rows ``X_all [B, H, S, D]``: the
    refitted state and every row's packed codes under it ``[U, S, stride]``
    (earlier rows' codes change whenever a range grows)."""
    st2 = refit(st, X_all)
    rows, _ = append(st2, X_all)
    return st2, rows


def clamp_fraction(st: TensorState, x: np.ndarray) -> float:
    """Frozen mode: the fraction of kept latents of rows ``x [B, H, n, D]`` whose
    code is decided by the clamp, i.e. whose unclamped rounded code
    ``rint((l - min) / scale)`` lies outside [0, 2**b - 1] (a latent beyond the
    prefill range; the cost of freezing the ranges)."""
    xu = gather_units(np.asarray(x), st.hpu)
    out = total = 0
    for u in range(st.U):
        r = int(st.r[u])
        L = project(xu[u], st.mu32[u], st.V32[u, :, :r])
        for i in np.flatnonzero(st.bits[u, :r]):
            sc = float(st.qscale32[u, i])
            if sc == 0.0:
                continue
            q = np.rint((L[:, i] - float(st.qmin32[u, i])) / sc)
            out += int(((q < 0) | (q > 2 ** int(st.bits[u, i]) - 1)).sum())
            total += L.shape[0]
    return out / max(total, 1)


def fetch(st: TensorState, rows: np.ndarray, params=None) -> np.ndarray:
    """Reconstruct every stored row: float64 ``[B, H, S, D]``."""
    U, S, _ = rows.shape
    out = np.zeros((U, S, st.Dg), np.float64)
    for u in range(U):
        r = int(st.r[u])
        bits = st.bits[u, :r]
        codes = unpack_rows(rows[u], bits)
        if st.cfg.mode == "dp":
            Lh = dequant_dp(codes, bits, st.qmin32[u, :r], st.qscale32[u, :r])
        else:
            Lh = dequant_mixed(codes, params[u], st.cfg.group_size)
        out[u] = reconstruct(Lh, st.mu32[u], st.V32[u, :, :r])
    return scatter_units(out, st.B, st.H, st.hpu)


# --------------------------------------------------------------------------
# decode attention over the stored cache (TurboQuant cache module page,
# ``attend``: one query per head, scores against every stored key divided by
# sqrt(d), softmax over the stored rows, weighted sum of the decoded values;
# PALU cache API page, "Design": the latents are reconstructed only for
# attention)
# --------------------------------------------------------------------------
def attend_rows(Kh: np.ndarray, Vh: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Attention of one query ``q [D]`` over keys ``Kh [S, D]`` and values
    ``Vh [S, D]``: ``softmax(Kh @ q / sqrt(D)) @ Vh`` in float64; zeros when
    nothing is stored (the page returns zeros for an empty cache)."""
    S, D = Kh.shape
    if S == 0:
        return np.zeros(D, np.float64)
    scores = Kh.astype(np.float64) @ np.asarray(q, np.float64) / math.sqrt(D)
    w = np.exp(scores - scores.max())          # softmax, shifted by its maximum
    w /= w.sum()
    return w @ Vh.astype(np.float64)


def attend(st_k: TensorState, rows_k: np.ndarray, st_v: TensorState, rows_v: np.ndarray,
           q: np.ndarray, params_k=None, params_v=None) -> np.ndarray:
    """Decode attention of queries ``q [B, Hq, D]`` over the reconstructed keys
    and values of the stored rows: float64 ``[B, Hq, D]``.  Hq is a multiple G
    of the stored heads H; query head hq attends KV head hq // G (grouped-query
    attention with consecutive query heads sharing a KV head; G = 1 is one
    query per head).  Group-head tensors are reconstructed as fetch does."""
    Kh, Vh = fetch(st_k, rows_k, params_k), fetch(st_v, rows_v, params_v)
    B, H = Kh.shape[:2]
    Hq = q.shape[1]
    assert Hq % H == 0, "query heads must be a multiple of the stored heads"
    G = Hq // H
    out = np.zeros((B, Hq, Kh.shape[3]), np.float64)
    for b in range(B):
        for hq in range(Hq):
            out[b, hq] = attend_rows(Kh[b, hq // G], Vh[b, hq // G], q[b, hq])
    return out


def to_f16(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp16 (the fetch output dtype)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16)


# --------------------------------------------------------------------------
# byte accounting (KVTC page: ``kvtc_bytes``, ``pre_entropy_bytes``,
# ``entropy_coding_gain``, ``full_seq_bytes``, ``compression_ratio``;
# PALU page, "Byte accounting": latents at the mixed-bit rate + fp32 projection)
# --------------------------------------------------------------------------
@dataclass
class BytesReport:
    fixed_payload: int = 0        # ceil(S * row_bits / 8) summed over units
    entropy_payload: int = 0      # Huffman payload of the units that take it
    entropy_table: int = 0
    stored_payload: int = 0       # payload actually counted (coded or fixed width)
    basis: int = 0
    quant_params: int = 0
    total: int = 0                # stored payload + table + basis + quant params
    pre_entropy: int = 0          # fixed payload + basis + quant params
    fp16_equiv: int = 0           # B * H * S * D * 2 (one tensor)
    n_survived: int = 0
    units_entropy_coded: int = 0


def bytes_report(st: TensorState, rows: np.ndarray, params, S: int) -> BytesReport:
    rep = BytesReport()
    rep.fp16_equiv = st.B * st.H * S * st.D * 2
    for u in range(st.U):
        r = int(st.r[u])
        bits = st.bits[u, :r]
        row_bits = int(bits.sum())
        fixed = (S * row_bits + 7) // 8
        rep.fixed_payload += fixed
        if st.cfg.mode == "dp":
            n_surv = int(np.count_nonzero(bits))
            rep.n_survived += n_surv
            side = 2 * (st.Dg * n_surv + st.Dg) + 2 * 2 * n_surv      # fp16 basis, mean, (min, scale)
            rep.basis += 2 * (st.Dg * n_surv + st.Dg)
            rep.quant_params += 2 * 2 * n_surv
            codes = unpack_rows(rows[u, :S], bits)
            hbits = 0
            table = 0
            for i, b in enumerate(bits):
                if b:
                    counts = np.bincount(codes[:, i], minlength=2 ** int(b))
                    hbits += huffman_bits(counts)
                    table += 2 ** int(b)
            payload = (hbits + 7) // 8
            if payload + table < fixed:
                rep.entropy_payload += payload
                rep.entropy_table += table
                rep.stored_payload += payload
                rep.units_entropy_coded += 1
                rep.total += payload + table + side
            else:
                rep.stored_payload += fixed
                rep.total += fixed + side
            rep.pre_entropy += fixed + side
        else:
            rep.n_survived += r
            proj = 4 * (st.Dg * r + st.Dg)                        # fp32 V_g and mu_g
            qp = 4 * S * st.n_groups()                            # fp16 (min, scale) per token-group
            rep.basis += proj
            rep.quant_params += qp
            rep.stored_payload += fixed
            rep.total += fixed + proj + qp
            rep.pre_entropy += fixed + proj + qp
    return rep


def entropy_archive(st: TensorState, rows: np.ndarray, S: int, lengths=None):
    """The entropy-coded storage of a DP tensor's first S rows (KVTC page, "Byte
    accounting": order-0 Huffman per kept component with a fixed-width fallback).
    Per unit, in unit order, byte aligned:
      coded (when payload + table < fixed width): the table -- for each kept
        component, 2**b bytes, byte k the code length of symbol k (0 if absent)
        -- then entropy_encode_unit's payload;
      fixed width: the rows' bits back to back (row s at bits [s*rb, (s+1)*rb) of
        the unit's part), ceil(S * rb / 8) bytes.
    ``lengths[u][i]`` gives the code lengths to use (any optimal set; default:
    huffman_lengths).  Returns (archive bytes, [(coded, offset, size)] per unit)."""
    assert st.cfg.mode == "dp"
    parts, info, off = [], [], 0
    for u in range(st.U):
        r = int(st.r[u])
        bits = [int(b) for b in st.bits[u, :r]]
        rb = sum(bits)
        codes = unpack_rows(rows[u, :S], bits)
        lens = [None] * r
        for i, b in enumerate(bits):
            if b:
                lens[i] = (np.asarray(lengths[u][i]) if lengths is not None else
                           huffman_lengths(np.bincount(codes[:, i], minlength=2 ** b)))
        table = b"".join(bytes(lens[i].astype(np.uint8)) for i, b in enumerate(bits) if b)
        fixed = (S * rb + 7) // 8
        payload = entropy_encode_unit(codes, bits, lens)
        if len(payload) + len(table) < fixed:
            part, coded = table + payload, True
        else:
            plane = np.unpackbits(np.asarray(rows[u, :S], np.uint8), axis=1, bitorder="little")[:, :rb]
            part, coded = np.packbits(plane.reshape(-1), bitorder="little").tobytes(), False
        parts.append(part)
        info.append((coded, off, len(part)))
        off += len(part)
    return b"".join(parts), info


def entropy_restore(st: TensorState, archive: bytes, info, S: int) -> np.ndarray:
    """Inverse of entropy_archive: the packed rows ``[U, S, row_stride]``."""
    rows = np.zeros((st.U, S, st.row_stride), np.uint8)
    for u, (coded, off, size) in enumerate(info):
        r = int(st.r[u])
        bits = [int(b) for b in st.bits[u, :r]]
        part = archive[off: off + size]
        if coded:
            lens, p = [None] * r, 0
            for i, b in enumerate(bits):
                if b:
                    lens[i] = np.frombuffer(part[p: p + 2 ** b], np.uint8).astype(np.int64)
                    p += 2 ** b
            rows[u] = pack_rows(entropy_decode_unit(part[p:], S, bits, lens), bits, st.row_stride)
        else:
            rb = sum(bits)
            plane = np.unpackbits(np.frombuffer(part, np.uint8), bitorder="little")[: S * rb].reshape(S, rb)
            full = np.zeros((S, 8 * st.row_stride), np.uint8)
            full[:, :rb] = plane
            rows[u] = np.packbits(full, axis=1, bitorder="little")
    return rows


def full_seq_bytes(B: int, H: int, S: int, D: int) -> int:
    """fp16 K + V size of the uncompressed cache."""
    return B * H * S * D * 2 * 2


def effective_bits(st: TensorState) -> float:
    """Stored code bits per original coordinate: (r / Dg) * weighted average width."""
    return float(np.mean([st.row_bits(u) for u in range(st.U)])) / st.Dg
