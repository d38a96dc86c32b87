"""Seeded synthetic inputs for one decode step of one attention layer.

This module draws the inputs only: queries (a target plus drafts per query
head), keys and values, per-sequence lengths, planted "hot" blocks, and the
perturbation that turns a given block selection into a resident set.  It holds
none of the method's arithmetic -- no block scoring, no selection, no transfer
plan, no attention -- so that the CPU oracle and the HIP path can both take
their inputs from here without sharing any computation.

Shapes follow the decode-step problem statement of the OasisKV pages (batch B,
context L, N_kv KV heads, GQA group G, head dim d_h = 128, blocks of bs tokens
(16 by default; 8, 32 and 64 as a variant),
top-K blocks per KV head, fetch ratio); see the xllm-io paper review,
section six (default parameters: block size 16, K = 128 blocks per KV head).

Layouts (all contiguous, head-major):
  q, q_prev : bf16 [B, N_kv, G, Q, 128]   Q = 1 + drafts; index 0 is the target
  k, v      : bf16 [B, N_kv, NB, bs, 128] NB = ceil(L / bs) blocks per sequence
  seq_lens  : int32 [B]
  planted   : bool [B, N_kv, NB]          blocks that received a key boost
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Dict, Optional

import numpy as np
import torch

HEAD_DIM = 128
BLOCK = 16


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic decode-step workload (one layer unless ``layers`` > 1)."""

    name: str
    batch: int
    num_kv_heads: int
    group: int
    ctx: int                      # maximum context length L in tokens
    num_drafts: int               # D; each query head carries 1 target + D drafts
    top_k: int                    # K blocks per KV head
    window: int                   # W local-window tokens, always resident
    fetch_ratio: float            # cap C = floor(ratio * K) new blocks per head per step
    planted: int                  # planted hot blocks per (b, kv head); ignored if heavy_tail
    min_len: Optional[int] = None  # lengths ~ U[min_len, ctx] (inclusive) if set, else all = ctx
    boost: float = 2.0            # planted key shift: boost * unit(q_target)
    heavy_tail: bool = False      # every candidate block gets Exp(1) * unit(q_target)
    resident: str = "prev"        # "prev": previous step's selection; "swap": current with swaps
    resident_swaps: int = 0       # members replaced for the "swap" recipe
    layers: int = 1
    seed: int = 0
    draft_sigma: float = 0.3      # draft = target + N(0, sigma^2)
    head_dim: int = HEAD_DIM
    block: int = BLOCK

    # ---- derived sizes -------------------------------------------------
    @property
    def queries(self) -> int:
        return 1 + self.num_drafts

    @property
    def max_blocks(self) -> int:
        return -(-self.ctx // self.block)

    @property
    def num_q_heads(self) -> int:
        return self.num_kv_heads * self.group

    @property
    def cap(self) -> int:
        # floor(ratio * K) taken in double with a small guard so that ratios
        # such as 0.29 at K = 100 do not floor one short.
        return int(math.floor(self.fetch_ratio * self.top_k + 1e-9))

    @property
    def window_blocks_max(self) -> int:
        return -(-self.window // self.block) + 1

    @property
    def table_stride(self) -> int:
        return self.top_k + self.window_blocks_max

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    # Small parity case: 1 sequence, 2 KV heads x group 4, L = 4096, K = 16.
    "tiny_4k": Workload(name="tiny_4k", batch=1, num_kv_heads=2, group=4, ctx=4096,
                        num_drafts=3, top_k=16, window=64, fetch_ratio=0.05, planted=8,
                        resident="swap", resident_swaps=4),
    # Qwen3-8B attention-layer shape at 32K context.
    "qwen3_8b_32k": Workload(name="qwen3_8b_32k", batch=8, num_kv_heads=8, group=4, ctx=32768,
                             num_drafts=4, top_k=128, window=128, fetch_ratio=0.05, planted=64,
                             resident="prev"),
    # Long-context single layer at 128K, resident set drifted by 10 %.
    "long_128k": Workload(name="long_128k", batch=4, num_kv_heads=8, group=4, ctx=131072,
                          num_drafts=4, top_k=128, window=128, fetch_ratio=0.05, planted=128,
                          resident="swap", resident_swaps=12),
    # High-batch reasoning decode, 36 layers back to back, lengths U[8192, 16384].
    "reasoning_36l": Workload(name="reasoning_36l", batch=64, num_kv_heads=8, group=4, ctx=16384,
                              min_len=8192, num_drafts=4, top_k=128, window=64, fetch_ratio=0.05,
                              planted=32, resident="prev", layers=36),
    # Qwen3-235B-A22B attention shape (4 KV heads x group 16), heavy-tailed hot blocks,
    # resident set churned by 25 %.
    "qwen3_235b_32k": Workload(name="qwen3_235b_32k", batch=32, num_kv_heads=4, group=16, ctx=32768,
                               num_drafts=4, top_k=128, window=128, fetch_ratio=0.05, planted=0,
                               heavy_tail=True, resident="swap", resident_swaps=32),
}


# ---- geometry helpers (pure index arithmetic on lengths) ----------------------

def num_blocks(seq_len: int, block: int = BLOCK) -> int:
    return -(-int(seq_len) // block)


def first_window_block(seq_len: int, window: int, block: int = BLOCK) -> int:
    """First block that overlaps the last ``window`` tokens; blocks before it are candidates."""
    return max(0, (int(seq_len) - int(window)) // block)


# ---- seeded substreams ----------------------------------------------------------

def _seed(w: Workload, *parts) -> int:
    key = repr((w.name, w.seed) + tuple(parts)).encode()
    return int.from_bytes(hashlib.sha256(key).digest()[:8], "little") & ((1 << 63) - 1)


def _gen(w: Workload, device, *parts) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(_seed(w, *parts))
    return g


def seq_lens(w: Workload) -> torch.Tensor:
    """int32 [B]; shared by every layer of the workload."""
    if w.min_len is None:
        return torch.full((w.batch,), w.ctx, dtype=torch.int32)
    g = _gen(w, "cpu", "lens")
    return torch.randint(w.min_len, w.ctx + 1, (w.batch,), generator=g, dtype=torch.int64).to(torch.int32)


def generate(w: Workload, device="cpu", layer: int = 0, with_kv: bool = True) -> Dict[str, torch.Tensor]:
    """Draw one layer's inputs on ``device`` (a CPU or GPU torch device).

    The values depend on the device's random number generator, so inputs are
    drawn once on one device and copied wherever else they are needed.
    """
    dev = torch.device(device)
    B, H, G, Q, D, d = w.batch, w.num_kv_heads, w.group, w.queries, w.num_drafts, w.head_dim
    NB, bs = w.max_blocks, w.block
    lens = seq_lens(w)

    # Target query per query head ~ N(0, 1), rounded to bf16 (round to nearest even).
    g = _gen(w, dev, "q_target", layer)
    q_target = torch.randn((B, H, G, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    # Drafts: bf16(fp32(target) + N(0, sigma^2)).
    g = _gen(w, dev, "q_drafts", layer)
    noise = torch.randn((B, H, G, D, d), generator=g, device=dev, dtype=torch.float32) * w.draft_sigma
    drafts = (q_target.float()[:, :, :, None, :] + noise).to(torch.bfloat16)
    q = torch.cat([q_target[:, :, :, None, :], drafts], dim=3).contiguous()
    out = {"q": q, "seq_lens": lens.to(dev)}
    if w.resident == "prev":
        # The previous step's queries: an independent perturbation of every row.
        g = _gen(w, dev, "q_prev", layer)
        noise = torch.randn((B, H, G, Q, d), generator=g, device=dev, dtype=torch.float32) * w.draft_sigma
        out["q_prev"] = (q_target.float()[:, :, :, None, :] + noise).to(torch.bfloat16).contiguous()

    # Candidate mask per (b, block): blocks before the first window block.
    w0 = torch.tensor([first_window_block(int(x), w.window, bs) for x in lens], dtype=torch.int64, device=dev)
    j = torch.arange(NB, device=dev, dtype=torch.int64)
    cand = (j[None, :] < w0[:, None])[:, None, :].expand(B, H, NB)          # [B, H, NB]

    # Planted hot blocks: which query head of the group each block answers to,
    # and how strongly it is shifted along that head's target direction.
    g = _gen(w, dev, "plant", layer)
    head_of_block = torch.randint(0, G, (B, H, NB), generator=g, device=dev)
    if w.heavy_tail:
        coef = torch.empty((B, H, NB), device=dev, dtype=torch.float32).exponential_(1.0, generator=g)
        planted = cand.clone()
    else:
        r = torch.rand((B, H, NB), generator=g, device=dev, dtype=torch.float32)
        r = torch.where(cand, r, torch.full_like(r, 2.0))
        n_plant = min(w.planted, NB)
        planted = torch.zeros((B, H, NB), dtype=torch.bool, device=dev)
        if n_plant > 0:
            idx = torch.topk(r, n_plant, dim=-1, largest=False).indices
            planted.scatter_(-1, idx, True)
        planted &= cand  # fewer candidates than planted blocks: plant them all
        coef = torch.full((B, H, NB), float(w.boost), device=dev, dtype=torch.float32)
    coef = coef * planted.float()
    unit = q_target.float()
    unit = unit / unit.norm(dim=-1, keepdim=True)                              # [B, H, G, d]
    shift = torch.gather(unit, 2, head_of_block[..., None].expand(B, H, NB, d)) * coef[..., None]
    out["planted"] = planted

    if with_kv:
        k = torch.empty((B, H, NB, bs, d), dtype=torch.bfloat16, device=dev)
        v = torch.empty_like(k)
        gk = _gen(w, dev, "k", layer)
        gv = _gen(w, dev, "v", layer)
        for b in range(B):  # per sequence, to bound the fp32 temporaries
            kb = torch.randn((H, NB, bs, d), generator=gk, device=dev, dtype=torch.float32)
            kb += shift[b][:, :, None, :]
            k[b] = kb.to(torch.bfloat16)
            v[b] = torch.randn((H, NB, bs, d), generator=gv, device=dev, dtype=torch.float32).to(torch.bfloat16)
            del kb
        out["k"], out["v"] = k, v
    return out


def resident_for_head(w: Workload, selection_row, n_cand: int, b: int, h: int, layer: int = 0):
    """Resident slot row for one (sequence, KV head) from its block selection.

    The slots hold the selected blocks in ascending block order, empty slots
    (-1) last.  For the "swap" recipe ``resident_swaps`` random members are then
    replaced, slot for slot, by random candidate blocks outside the selection.
    The random draws depend only on (b, h, layer), not on other heads.
    """
    sel = np.asarray(selection_row, dtype=np.int64)
    K = sel.shape[0]
    res = np.full(K, -1, dtype=np.int64)
    s = np.sort(sel[sel >= 0])
    res[: s.size] = s
    n = min(w.resident_swaps, s.size) if w.resident == "swap" else 0
    if n > 0:
        outside = np.setdiff1d(np.arange(n_cand), s)
        n = min(n, outside.size)
        if n > 0:
            rng = np.random.default_rng(_seed(w, "resident", layer, b, h))
            slots = rng.choice(s.size, size=n, replace=False)
            res[slots] = rng.choice(outside, size=n, replace=False)
    return res


def resident_from_selection(w: Workload, selection: torch.Tensor, lens: torch.Tensor,
                            layer: int = 0) -> torch.Tensor:
    """Resident slot tables [B, N_kv, K] (int32, CPU) from per-head selections."""
    sel = selection.detach().to("cpu", torch.int64).numpy()
    B, H, K = sel.shape
    res = np.full((B, H, K), -1, dtype=np.int64)
    for b in range(B):
        n_cand = first_window_block(int(lens[b]), w.window, w.block)
        for h in range(H):
            res[b, h] = resident_for_head(w, sel[b, h], n_cand, b, h, layer)
    return torch.from_numpy(res.astype(np.int32))


def random_scores(shape, seed: int, distinct: bool = True, levels: int = 7) -> torch.Tensor:
    """fp32 test scores for exercising selection and planning on their own.

    With ``distinct`` the values are a random permutation of a spaced grid, so
    every comparison has one answer; otherwise values are drawn uniformly from
    ``levels`` equally spaced values, so that exact ties are common (few levels:
    large groups of equal scores; many levels: small groups spread over the range).
    """
    g = torch.Generator().manual_seed(seed)
    n = int(np.prod(shape))
    if distinct:
        perm = torch.randperm(n, generator=g)
        vals = (perm.to(torch.float64) * 0.37 - 0.11 * n).to(torch.float32)
    else:
        lo = -(levels // 2)
        vals = torch.randint(lo, lo + levels, (n,), generator=g).to(torch.float32) * 0.5
    return vals.reshape(shape)


def random_resident(K: int, n_cand: int, n_empty: int, seed: int) -> torch.Tensor:
    """A resident slot table of K distinct candidate blocks with ``n_empty`` empty (-1) slots,
    in random slot order."""
    rng = np.random.default_rng(seed)
    n_fill = max(0, min(K - n_empty, n_cand))
    r = np.full(K, -1, dtype=np.int64)
    r[:n_fill] = rng.choice(n_cand, size=n_fill, replace=False)
    rng.shuffle(r)
    return torch.from_numpy(r.astype(np.int32))
