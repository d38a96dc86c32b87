"""Shared test helpers: the oracle applied per (sequence, KV head), and the tolerances.

Tolerances (stated for the decode step):
  * summaries: bit-exact (bf16 min/max);
  * scores: |gpu - ref| <= 1e-5 * max(|ref|, floor), floor = the largest
    sum_d |q_d| * max(|kmin_d|, |kmax_d|) over the rows (guards values near 0);
  * selection: identical sets, except swaps among blocks whose oracle scores lie
    within 1e-5 relative of the K-th oracle score;
  * plan, resident, table: bit-exact given the selected set;
  * attention output: max abs error 2e-3 (fp32 output from bf16 K/V); the
    log-sum-exp is held to the same absolute bound.
"""
from __future__ import annotations

import math
from typing import Dict

import numpy as np
import torch

from oracle import ref

SCORE_RTOL = 1e-5
OUT_ATOL = 2e-3


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def i64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.int64).numpy()


def score_floor(q: np.ndarray, summ: np.ndarray) -> np.ndarray:
    """[B, H, NB] floor for the relative score tolerance."""
    qa = np.abs(q).reshape(q.shape[0], q.shape[1], -1, q.shape[-1])          # [B, H, R, d]
    ka = np.maximum(np.abs(summ[:, :, :, 0, :]), np.abs(summ[:, :, :, 1, :]))  # [B, H, NB, d]
    return np.einsum("bhrd,bhnd->bhrn", qa, ka).max(axis=2)


def check_scores(gpu: np.ndarray, expect: np.ndarray, floor: np.ndarray, where: str = "") -> float:
    fin = np.isfinite(expect)
    assert np.array_equal(np.isneginf(gpu), np.isneginf(expect)), f"{where}: -inf pattern differs"
    if not fin.any():
        return 0.0
    err = np.abs(gpu[fin] - expect[fin]) / np.maximum(np.abs(expect[fin]), floor[fin])
    worst = float(err.max())
    assert worst <= SCORE_RTOL, f"{where}: score rel err {worst:.3g} > {SCORE_RTOL}"
    return worst


def selection_equivalent(gpu_sel: np.ndarray, ref_sel: np.ndarray, ref_scores: np.ndarray) -> bool:
    """True if the two selections (one head) differ only by swaps among near-ties of the K-th score."""
    g = set(int(x) for x in gpu_sel if x >= 0)
    r = set(int(x) for x in ref_sel if x >= 0)
    if len(g) != len(r) or len([x for x in gpu_sel if x >= 0]) != len(g):
        return False
    if g == r:
        return True
    valid = [int(x) for x in ref_sel if x >= 0]
    kth = ref_scores[valid[-1]]
    tol = SCORE_RTOL * max(abs(kth), 1e-30)
    return all(abs(ref_scores[x] - kth) <= tol for x in g ^ r)


def plan_robust(scores: np.ndarray, sel: np.ndarray, resident: np.ndarray, cap: int, n_cand: int) -> bool:
    """True if every score comparison that decides the oracle's plan for one head has a gap
    larger than the score tolerance (so fp32 rounding on the GPU cannot flip it)."""
    s = scores
    tol = lambda a, b: SCORE_RTOL * max(abs(a), abs(b), 1e-30)
    valid = [int(x) for x in sel if x >= 0]
    K = sel.shape[0]
    if len(valid) == K and n_cand > K:
        order = sorted(range(n_cand), key=lambda j: (-s[j], j))
        a, b = s[order[K - 1]], s[order[K]]
        if abs(a - b) <= tol(a, b):
            return False
    R = set(int(x) for x in resident if x >= 0)
    new = [x for x in valid if x not in R]
    n = min(cap, len(new))
    if 0 < n < len(new) and abs(s[new[n - 1]] - s[new[n]]) <= tol(s[new[n - 1]], s[new[n]]):
        return False
    n_empty = int(np.sum(resident < 0))
    m = n - n_empty
    stale = sorted([int(x) for x in resident if x >= 0 and int(x) not in set(valid)],
                   key=lambda x: (s[x], -x))
    if 0 < m < len(stale) and abs(s[stale[m - 1]] - s[stale[m]]) <= tol(s[stale[m - 1]], s[stale[m]]):
        return False
    return True


def oracle_head(q, k, v, lens, resident_row, top_k, window, cap, scale, b, h,
                block: int = 16) -> Dict[str, np.ndarray]:
    """The whole oracle step for one (sequence b, KV head h); inputs are CPU tensors
    of the full batch (only that head's slices are converted)."""
    qh = f64(q[b:b + 1, h:h + 1])
    kh = f64(k[b:b + 1, h:h + 1])
    vh = f64(v[b:b + 1, h:h + 1])
    L = np.array([int(lens[b])])
    summ = ref.build_summaries(kh, L, block)
    res = ref.decode_step(qh, summ, kh, vh, L, np.asarray(resident_row)[None, None], top_k, window,
                          cap, scale, block)
    res["summ"] = summ
    out = {key: val[0, 0] if isinstance(val, np.ndarray) and val.ndim >= 2 else val
           for key, val in res.items()}
    out["head_inputs"] = (qh, kh, vh, L, block)   # for attention over another table
    return out


def oracle_selection_head(q, k, lens, top_k, window, b, h, block: int = 16) -> np.ndarray:
    """The oracle's top-K for one head (used to build resident sets)."""
    qh = f64(q[b:b + 1, h:h + 1])
    kh = f64(k[b:b + 1, h:h + 1])
    L = np.array([int(lens[b])])
    s = ref.score_blocks(qh, ref.build_summaries(kh, L, block), L, window, block)
    return ref.topk_blocks(s, L, top_k, window, block)[0, 0]


def default_scale() -> float:
    return 1.0 / math.sqrt(128)
