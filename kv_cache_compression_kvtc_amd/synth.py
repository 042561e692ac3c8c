"""Seeded synthetic K/V rows for the five workloads, shared by tests, bench and smoke.

This module draws inputs only. It holds none of the compression arithmetic
(no fit, no projection, no quantisation): it builds rows with a prescribed
covariance spectrum so that a local PCA has something to find, as the KVTC
cache module page assumes (its docstring, "Design": local PCA on the prefill
batch, then a frozen basis for every later token).

Per unit (one (batch, head) pair, or one (batch, head-group) for the
group-head workload), with ``rng = default_rng([workload, tensor, b, u])``:

* eigen-spectrum ``lam_k = k ** -alpha`` for ``k = 1..Dg``;
* ``Q`` from the QR factorisation of a standard-normal ``Dg x Dg`` matrix,
  columns sign-fixed so that ``diag(R) > 0`` (a Haar-random rotation);
* per-channel offset ``mu = 0.5 * N(0, 1)``;
* rows ``X = mu + (Z * sqrt(lam)) @ Q.T`` with ``Z ~ N(0, 1)`` ``[S, Dg]``;
* key outliers: the same channel indices in every head, drawn once per
  workload with ``default_rng([workload, 99])``; the whole channel is scaled;
* optional iid noise from its own stream ``default_rng([workload, tensor, b, u, 1])``;
* the result is rounded to fp16 (round-to-nearest-even) unless the workload is fp32.

Rows are prefix-consistent: the first ``S`` rows do not depend on how many
rows are drawn in total, so a prefill and its continuation can be generated
separately or together.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
import os

import numpy as np

KEY, VALUE = 0, 1


@dataclass(frozen=True)
class Workload:
    """Shapes, spectra and method settings of one seeded workload."""

    wid: int
    name: str
    B: int
    H: int
    D: int
    dtype: str                      # "f32" or "f16"
    s_prefill: int                  # rows the frozen state is fitted on
    s_total: int                    # rows stored after the timed/parity appends
    alpha_k: float
    alpha_v: float
    n_outliers_k: int = 0
    outlier_scale: float = 20.0
    noise: float = 0.0
    # method settings
    mode: str = "dp"                # "dp" (per-(b,h) DP bits) or "mixed" (group-head)
    heads_per_unit: int = 1
    rank: int = 0                   # 0 -> energy threshold
    energy: float = 0.90
    budget: int = 0
    choices: tuple = (0, 1, 2, 3, 4, 8)
    beta: float = 1.0
    hi_bits: int = 4
    lo_bits: int = 2
    hi_fraction: float = 0.25
    group_size: int = 32
    decode_steps: int = 0           # single-token appends after s_prefill (decode workloads)
    notes: str = ""

    @property
    def Dg(self) -> int:
        return self.D * self.heads_per_unit

    @property
    def units(self) -> int:
        return self.B * self.H // self.heads_per_unit


WORKLOADS = {
    1: Workload(1, "tiny", B=1, H=2, D=64, dtype="f32", s_prefill=256, s_total=288,
                alpha_k=1.5, alpha_v=1.5, noise=0.01, rank=64, budget=128,
                choices=(0, 1, 2, 4, 8), decode_steps=32,
                notes="prefill 256 then 32 single-token appends"),
    2: Workload(2, "llama3-8b-layer", B=1, H=8, D=128, dtype="f16", s_prefill=4096,
                s_total=4096 + 256, alpha_k=1.2, alpha_v=0.8, n_outliers_k=4, rank=128,
                budget=256, choices=(0, 1, 2, 3, 4, 8), decode_steps=256,
                notes="prefill 4096 then 256 decode steps of (append 1, fetch all)"),
    3: Workload(3, "palu-group-head", B=1, H=32, D=128, dtype="f16", s_prefill=16384,
                s_total=16384, alpha_k=1.2, alpha_v=0.8, n_outliers_k=4, mode="mixed",
                heads_per_unit=8, rank=256, hi_bits=4, lo_bits=2, hi_fraction=0.25,
                group_size=32, notes="4 groups of 8 heads, shared projection, r=256"),
    4: Workload(4, "batched-decode", B=64, H=8, D=128, dtype="f16", s_prefill=8192,
                s_total=8192 + 1, alpha_k=1.2, alpha_v=0.8, n_outliers_k=4, rank=96,
                budget=320, choices=(0, 2, 4, 8), decode_steps=1,
                notes="8192 stored per sequence; each step appends 1 and fetches all"),
    5: Workload(5, "long-context", B=1, H=8, D=128, dtype="f16", s_prefill=8192,
                s_total=131072, alpha_k=1.2, alpha_v=0.8, n_outliers_k=4, rank=0,
                energy=0.90, budget=192, choices=(0, 1, 2, 3, 4, 8),
                notes="fit on first 8192, one-shot append of 122880, full fetch"),
}


def outlier_channels(w: Workload) -> np.ndarray:
    """Key outlier channel indices within one head (same for every head)."""
    if w.n_outliers_k == 0:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.default_rng([w.wid, 99])
    return np.sort(rng.choice(w.D, size=w.n_outliers_k, replace=False))


def unit_rows(w: Workload, tensor: int, b: int, u: int, s_begin: int, s_end: int) -> np.ndarray:
    """Rows ``[s_begin, s_end)`` of one unit, float64 ``[n, Dg]`` before the dtype cast."""
    Dg = w.Dg
    alpha = w.alpha_k if tensor == KEY else w.alpha_v
    rng = np.random.default_rng([w.wid, tensor, b, u])
    lam = np.arange(1, Dg + 1, dtype=np.float64) ** (-alpha)
    A = rng.standard_normal((Dg, Dg))
    Q, R = np.linalg.qr(A)
    Q = Q * np.where(np.diag(R) < 0, -1.0, 1.0)[None, :]
    mu = 0.5 * rng.standard_normal(Dg)
    Z = rng.standard_normal((s_end, Dg))[s_begin:]
    X = mu[None, :] + (Z * np.sqrt(lam)[None, :]) @ Q.T
    if w.noise:
        nrng = np.random.default_rng([w.wid, tensor, b, u, 1])
        X = X + w.noise * nrng.standard_normal((s_end, Dg))[s_begin:]
    if tensor == KEY and w.n_outliers_k:
        idx = outlier_channels(w)
        cols = (np.arange(w.heads_per_unit)[:, None] * w.D + idx[None, :]).ravel()
        X[:, cols] *= w.outlier_scale
    return X


def np_dtype(w: Workload):
    return np.float32 if w.dtype == "f32" else np.float16


def generate(w: Workload, tensor: int, s_begin: int = 0, s_end: int | None = None,
             threads: int | None = None) -> np.ndarray:
    """Rows ``[s_begin, s_end)`` of one tensor as ``[B, H, n, D]`` in the workload dtype."""
    if s_end is None:
        s_end = w.s_total
    n = s_end - s_begin
    out = np.empty((w.B, w.H, n, w.D), dtype=np_dtype(w))
    G = w.H // w.heads_per_unit

    def one(unit):
        b, g = divmod(unit, G)
        X = unit_rows(w, tensor, b, g, s_begin, s_end).astype(np_dtype(w))
        for j in range(w.heads_per_unit):
            out[b, g * w.heads_per_unit + j] = X[:, j * w.D:(j + 1) * w.D]

    units = range(w.B * G)
    nthreads = threads or min(16, os.cpu_count() or 1)
    if len(units) == 1 or nthreads == 1:
        for unit in units:
            one(unit)
    else:
        with ThreadPoolExecutor(max_workers=nthreads) as ex:
            list(ex.map(one, units))
    return out
