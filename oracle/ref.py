"""Plain fp64 CPU oracle for one OasisKV look-ahead sparse-attention decode step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import or run this module.  The product path
(the HIP library and its binding) never calls it and shares no code with it.

Every function is the plain definition of its step, written for reading, not
for speed: numpy in float64, loops over (sequence, KV head) where that is
clearer.  Inputs arrive as float64 arrays holding bf16 values exactly (the
caller widens them), int arrays for lengths, selections and slot tables.

Sources (the pages on OasisKV, arXiv 2608.08097):
  [xllm]    xllm-io.github.io paper review
  [lode]    lode.cx article
  [legible] legiblepapers.com summary
Where the pages leave a step open, the docstring names the reading taken.

Parity status: every function here is pinned by CPU tests against brute force,
closed forms, textbook routines or exhaustive enumeration of the rule on tiny
instances.  End-to-end values are not printed on the pages, so no test can
pin them to the pages directly; that is stated where it matters.
"""
from __future__ import annotations

import math
from typing import Dict, Tuple

import numpy as np

NEG_INF = -np.inf


def num_blocks(seq_len: int, block: int = 16) -> int:
    """Blocks that hold at least one of the ``seq_len`` tokens."""
    return (int(seq_len) + block - 1) // block


def first_window_block(seq_len: int, window: int, block: int = 16) -> int:
    """First block overlapping the last ``window`` tokens.

    [xllm] section three, training flow step 2: the GPU keeps the selected
    historical blocks plus the local window.  Reading: residency is block
    granular, so every block that holds one of the last W tokens is pinned and
    the blocks before it are the scoring candidates.
    """
    return max(0, (int(seq_len) - int(window)) // block)


def fetch_cap(fetch_ratio: float, top_k: int) -> int:
    """C = floor(fetch_ratio * K) new blocks per head per step.

    [xllm] section three, component table (Capped Eviction Policy: fetch
    ratio 0.05 by default, limits blocks newly brought in per head per step);
    [legible] FAQ Q7.  Taken in double with a 1e-9 guard so that a ratio
    such as 0.29 at K = 100 does not floor to 28.
    """
    return int(math.floor(float(fetch_ratio) * int(top_k) + 1e-9))


# ---------------------------------------------------------------------------
# O0  per-block min/max key summaries
# ---------------------------------------------------------------------------

def build_summaries(k: np.ndarray, seq_lens: np.ndarray, block: int = 16) -> np.ndarray:
    """Per-block, per-dimension min and max of the keys ("compressed keys").

    [xllm] section three, component table (Compressed Key Cache: a
    per-dimension min/max summary for each logical block, 1/16 of the full KV
    size) and section two, algorithm layer (Quest-style min/max pooling).

    k: [B, H, NB, block, d].  Returns [B, H, NB, 2, d] with slot 0 = min and
    slot 1 = max over the valid tokens (global token index < seq_len) of each
    block.  A block with no valid token gets zeros.
    """
    B, H, NB, bs, d = k.shape
    out = np.zeros((B, H, NB, 2, d), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        for j in range(NB):
            n_valid = min(bs, L - j * bs)
            if n_valid <= 0:
                continue
            toks = k[b, :, j, :n_valid, :]            # [H, n_valid, d]
            out[b, :, j, 0, :] = toks.min(axis=1)
            out[b, :, j, 1, :] = toks.max(axis=1)
    return out


# ---------------------------------------------------------------------------
# O1  look-ahead block scores
# ---------------------------------------------------------------------------

def score_blocks(q: np.ndarray, summ: np.ndarray, seq_lens: np.ndarray, window: int,
                 block: int = 16) -> np.ndarray:
    """Upper-bound score of every candidate block for every KV head.

    [xllm] section two, algorithm layer: the draft tokens' query vectors scan
    the compressed key summary to predict next step's most important blocks;
    [lode] "The Insight", point 2.  The bound per query row is the Quest
    criterion sum_d max(q_d * kmin_d, q_d * kmax_d), which is >= q . k for
    every key k inside the block.  One score per (KV head, block) is the max
    over the G query heads of the group and over the target and draft queries
    (the aggregation convention this implementation adopts).

    q: [B, H, G, Q, d]; summ: [B, H, NB, 2, d].  Returns [B, H, NB] with
    -inf for non-candidates (the local-window blocks and beyond).
    """
    B, H, G, Q, d = q.shape
    NB = summ.shape[2]
    s = np.full((B, H, NB), NEG_INF, dtype=np.float64)
    for b in range(B):
        n_cand = first_window_block(int(seq_lens[b]), window, block)
        if n_cand == 0:
            continue
        for h in range(H):
            kmin = summ[b, h, :n_cand, 0, :]               # [n, d]
            kmax = summ[b, h, :n_cand, 1, :]
            rows = q[b, h].reshape(G * Q, d)               # [R, d]
            lo = rows[:, None, :] * kmin[None, :, :]       # [R, n, d]
            hi = rows[:, None, :] * kmax[None, :, :]
            bound = np.maximum(lo, hi).sum(axis=-1)        # [R, n]
            s[b, h, :n_cand] = bound.max(axis=0)
    return s


# ---------------------------------------------------------------------------
# O2  head-wise top-K block selection
# ---------------------------------------------------------------------------

def topk_blocks(scores: np.ndarray, seq_lens: np.ndarray, top_k: int, window: int,
                block: int = 16) -> np.ndarray:
    """The K best candidate blocks per KV head, best first.

    [xllm] section three, component table (Look-ahead Attention: top-K = 128
    blocks per head) and section six (block size 16, K = 128 blocks per KV
    head).  Order: higher score first; on equal scores the lower block index
    first.  Candidates are the blocks before the local window; with fewer than
    K candidates the tail is padded with -1.

    scores: [B, H, NB] (any float dtype; comparisons happen in that dtype).
    Returns int64 [B, H, K].
    """
    B, H, NB = scores.shape
    out = np.full((B, H, top_k), -1, dtype=np.int64)
    for b in range(B):
        n_cand = first_window_block(int(seq_lens[b]), window, block)
        if n_cand == 0:
            continue
        idx = np.arange(n_cand)
        for h in range(H):
            s = scores[b, h, :n_cand]
            order = np.lexsort((idx, -s))                  # primary: -score; secondary: index
            m = min(top_k, n_cand)
            out[b, h, :m] = order[:m]
    return out


# ---------------------------------------------------------------------------
# O3  capped-eviction transfer plan against the resident set
# ---------------------------------------------------------------------------

def _plan_one(s: np.ndarray, sel: np.ndarray, res: np.ndarray, cap: int):
    """Plan for one (sequence, KV head).  See ``build_plan``."""
    K = res.shape[0]
    chosen = [int(x) for x in sel if x >= 0]
    chosen_set = set(chosen)
    res_set = set(int(x) for x in res if x >= 0)

    # New blocks: selected but not resident, best first (selection order).
    admit = [x for x in chosen if x not in res_set]
    n = min(cap, len(admit))
    admit = admit[:n]

    # Victim slots: empty slots first (ascending slot), then slots whose block
    # left the selection, worst first (lowest score; equal scores: higher block
    # index first).
    empty = [i for i in range(K) if res[i] < 0]
    stale = [i for i in range(K) if res[i] >= 0 and int(res[i]) not in chosen_set]
    stale.sort(key=lambda i: (s[int(res[i])], -int(res[i])))
    victims = (empty + stale)[:n]

    plan = np.full((cap, 3), -1, dtype=np.int64)
    new_res = res.astype(np.int64).copy()
    for row, (slot, blk) in enumerate(zip(sorted(victims), sorted(admit))):
        plan[row] = (slot, blk, int(res[slot]))
        new_res[slot] = blk
    return plan, n, new_res


def build_plan(scores: np.ndarray, topk: np.ndarray, resident: np.ndarray, seq_lens: np.ndarray,
               cap: int, window: int, block: int = 16) -> Dict[str, np.ndarray]:
    """Capped-eviction transfer plan, the updated resident set, and the attention table.

    [xllm] section three, training flow step 3 (background: compare the
    predicted top-K with the resident set and build the transfer plan) and
    component table (Capped Eviction Policy: at most C newly admitted blocks
    per head per step); [legible] FAQ Q7 (the cap bounds newly admitted
    blocks at the KV-selection stage).  Head-wise mapping entries are the only
    thing that changes ([xllm] section four, Head-wise Mapping row).

    Readings where the pages are silent:
      * which blocks to admit when more than C are new: the C best in the
        selection order;
      * which slots to free: empty slots first (ascending slot), then slots
        whose block left the selection, lowest score first (equal scores:
        higher block index first);
      * pairing: freed slots in ascending slot order take the admitted blocks
        in ascending block order; the plan lists (slot, new, old) by slot,
        old = -1 for an empty slot, unused rows -1;
      * the attention table is the updated resident entries in slot order
        (empty slots skipped) followed by the local-window blocks
        [first_window_block, num_blocks) ([xllm] section three, training
        flow step 2: selected historical blocks plus the local window); a
        resident block that the window has reached (the window moves as the
        sequence grows) is listed once, as a window block, as in
        resident_table.

    scores: [B, H, NB]; topk: [B, H, K]; resident: [B, H, K] (-1 = empty).
    Returns dict with plan [B, H, C, 3], plan_count [B, H], resident [B, H, K],
    table [B, H, K + ceil(W/16) + 1] (-1 padded), table_count [B, H].
    """
    B, H, K = resident.shape
    T = K + -(-window // block) + 1
    plan = np.full((B, H, cap, 3), -1, dtype=np.int64)
    plan_count = np.zeros((B, H), dtype=np.int64)
    new_res = np.full((B, H, K), -1, dtype=np.int64)
    table = np.full((B, H, T), -1, dtype=np.int64)
    table_count = np.zeros((B, H), dtype=np.int64)
    for b in range(B):
        L = int(seq_lens[b])
        w0, nb = first_window_block(L, window, block), num_blocks(L, block)
        for h in range(H):
            p, n, r = _plan_one(scores[b, h], topk[b, h], resident[b, h], cap)
            plan[b, h], plan_count[b, h], new_res[b, h] = p, n, r
            entries = [int(x) for x in r if 0 <= x < w0] + list(range(w0, nb))
            table[b, h, : len(entries)] = entries
            table_count[b, h] = len(entries)
    return {"plan": plan, "plan_count": plan_count, "resident": new_res,
            "table": table, "table_count": table_count}


def resident_table(resident: np.ndarray, seq_lens: np.ndarray, window: int,
                   block: int = 16) -> Tuple[np.ndarray, np.ndarray]:
    """The working set held as a resident slot table, written out as a table.

    [legible] summary (the foreground attends over the entries resident in
    HBM now); [xllm] section three, training flow step 2 (selected historical
    blocks plus the local window).  The entries are the resident blocks in
    slot order, empty slots skipped, then the window blocks
    [first_window_block, num_blocks).  Reading: a resident block at or past
    the first window block is listed once, as a window block (the window can
    move past a block that was selected when the sequence was shorter).

    resident: [B, H, K] (-1 = empty).  Returns table [B, H, K + ceil(W/16) + 1]
    (-1 padded) and table_count [B, H].
    """
    B, H, K = resident.shape
    T = K + -(-window // block) + 1
    table = np.full((B, H, T), -1, dtype=np.int64)
    table_count = np.zeros((B, H), dtype=np.int64)
    for b in range(B):
        L = int(seq_lens[b])
        w0, nb = first_window_block(L, window, block), num_blocks(L, block)
        for h in range(H):
            entries = [int(x) for x in resident[b, h] if 0 <= x < w0] + list(range(w0, nb))
            table[b, h, : len(entries)] = entries
            table_count[b, h] = len(entries)
    return table, table_count


# ---------------------------------------------------------------------------
# O4  sparse decode attention over the head-wise block table
# ---------------------------------------------------------------------------

def sparse_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, table: np.ndarray,
                     table_count: np.ndarray, seq_lens: np.ndarray, scale: float,
                     block: int = 16) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of each target query over the tokens of its KV head's table.

    [xllm] section three, training flow step 3 (foreground: a normal
    attention forward pass) over the sparse working set of section three's
    architecture figure; [legible] summary (standard attention on the sparse
    KV set resident in HBM).  Readings: only the target query (row 0)
    attends; every token index < seq_len of a listed block is visible (no
    mask inside the context); tokens >= seq_len in a partial block are
    dropped; scale is the caller's (1/sqrt(d_h) in practice).  With no token
    at all the output is 0 and the log-sum-exp is -inf.

    q: [B, H, G, Q, d]; k, v: [B, H, NB, block, d]; table: [B, H, T].
    Returns out [B, H, G, d] and lse [B, H, G] (natural log of sum exp(z)).
    """
    B, H, G, Q, d = q.shape
    out = np.zeros((B, H, G, d), dtype=np.float64)
    lse = np.full((B, H, G), NEG_INF, dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        for h in range(H):
            blocks = [int(x) for x in table[b, h, : int(table_count[b, h])]]
            toks = [(j, t) for j in blocks for t in range(block) if j * block + t < L]
            if not toks:
                continue
            jj = np.array([x[0] for x in toks])
            tt = np.array([x[1] for x in toks])
            kt = k[b, h, jj, tt, :]                         # [n, d]
            vt = v[b, h, jj, tt, :]
            for g in range(G):
                z = (kt @ q[b, h, g, 0, :]) * scale         # [n]
                m = z.max()
                e = np.exp(z - m)
                den = e.sum()
                out[b, h, g] = (e[:, None] * vt).sum(axis=0) / den
                lse[b, h, g] = m + math.log(den)
    return out, lse


# ---------------------------------------------------------------------------
# Prediction quality: which blocks the true next query attends to
# ---------------------------------------------------------------------------

def block_attention_mass(q_true: np.ndarray, k: np.ndarray, seq_lens: np.ndarray, window: int,
                         scale: float, block: int = 16) -> np.ndarray:
    """Share of each candidate block in the true query's attention, per KV head.

    For query head g of (b, h), the softmax of scale * q_true[b,h,g] . k_t over
    every valid token t (candidates and window), summed over the tokens of block
    j; the head-wise figure is the largest share over the group, as the
    selection aggregates over the group.  Candidate blocks only (the window is
    always resident); -inf elsewhere.  This is the set the look-ahead predicts:
    [xllm] section four, Figure 4 (top-20 block prediction accuracy of the draft
    query against a previous-token proxy) and Figure 6 (agreement of the draft
    query's top-K set with the true next-token query's).  Reading: "the blocks
    the true next query needs" is the top of this share.

    q_true: [B, H, G, d]; k: [B, H, NB, block, d].  Returns [B, H, NB].
    """
    B, H, NB, bs, d = k.shape
    G = q_true.shape[2]
    out = np.full((B, H, NB), NEG_INF)
    for b in range(B):
        L = int(seq_lens[b])
        n_cand = first_window_block(L, window, block)
        if L <= 0:
            continue
        flat = k[b].reshape(H, NB * bs, d)[:, :L]            # [H, L, d]
        for h in range(H):
            best = np.full(n_cand, NEG_INF)
            for g in range(G):
                z = flat[h] @ q_true[b, h, g] * scale        # [L]
                p = np.exp(z - z.max())
                p /= p.sum()
                per_block = np.add.reduceat(p, np.arange(0, L, bs))[:n_cand]
                best = np.maximum(best, per_block)
            out[b, h, :n_cand] = best
    return out


def captured_attention(q_true: np.ndarray, k: np.ndarray, seq_lens: np.ndarray, window: int,
                       scale: float, selection: np.ndarray, block: int = 16) -> np.ndarray:
    """Share of the true query's attention over the candidate blocks that a
    selection holds, per KV head, averaged over the query heads of the group.

    For query head g of (b, h): the softmax of scale * q_true[b,h,g] . k_t over
    every valid token t, summed over the tokens of the selected candidate blocks,
    divided by the same sum over all candidate blocks (the window is attended in
    any case).  Unlike a block overlap it counts tokens, so selections of equal
    token budget made at different block sizes compare on one scale.  [xllm]
    section four, Figures 4 and 6 measure how well the look-ahead finds the
    blocks the next token needs; this is the attention those blocks carry.
    Reading: a head with no candidate block counts as fully captured (1.0).

    q_true: [B, H, G, d]; k: [B, H, NB, block, d]; selection: [B, H, K] block
    ids (-1 and ids outside the candidates are ignored).  Returns [B, H].
    """
    B, H, NB, bs, d = k.shape
    G = q_true.shape[2]
    out = np.ones((B, H))
    for b in range(B):
        L = int(seq_lens[b])
        n_cand = first_window_block(L, window, block)
        if L <= 0 or n_cand == 0:
            continue
        flat = k[b].reshape(H, NB * bs, d)[:, :L]
        for h in range(H):
            sel = np.unique([int(j) for j in selection[b, h] if 0 <= j < n_cand]).astype(np.int64)
            fractions = []
            for g in range(G):
                z = flat[h] @ q_true[b, h, g] * scale
                p = np.exp(z - z.max())
                p /= p.sum()
                per_block = np.add.reduceat(p, np.arange(0, L, bs))[:n_cand]
                fractions.append(per_block[sel].sum() / per_block.sum())
            out[b, h] = float(np.mean(fractions))
    return out


def top_overlap(pred: np.ndarray, true: np.ndarray, n: int) -> float:
    """|first n of pred & first n of true| / n for two rankings (block ids, best
    first, -1 padded); 1.0 when both are empty."""
    a = {int(x) for x in pred[:n] if x >= 0}
    b = {int(x) for x in true[:n] if x >= 0}
    m = max(len(a), len(b))
    return 1.0 if m == 0 else len(a & b) / m


# ---------------------------------------------------------------------------
# Executing the plan: the working set in HBM
# ---------------------------------------------------------------------------
#
# The full K/V of every sequence stays in its tier (host memory, or HBM when it
# fits), addressed as before by (sequence, KV head, logical block): that page
# table never changes.  HBM holds each KV head's working set: a pool of K block
# slots that the head's resident slot table maps to logical blocks (the
# head-wise logical-to-logical map), and a ring of window blocks.  Sources:
# [xllm] section three, component table (head-wise mapping: a logical-to-logical
# layer above the paged cache, a different sparse block set per KV head) and
# training flow step 2 (after the sparsification conversion the full cache sits
# in CPU memory and the GPU keeps only the selected historical blocks and the
# local window); [xllm] section four, innovations table (the page table stays,
# only head-wise mapping entries change); [legible] FAQ Q4; [lode] points 1 and 3
# (hot entries in HBM, needed blocks pulled in from the larger tier).
# Readings: a pool slot holds one whole block (16 tokens of K and of V) and slot s
# of the pool is slot s of the slot table; logical block j of the window lives in
# ring slot j mod (ceil(W/16) + 1), the most window blocks a length can have.

def window_ring_slots(window: int, block: int = 16) -> int:
    """Ring slots per KV head: the most blocks the last ``window`` tokens can touch."""
    return -(-int(window) // block) + 1


def fill_working_set(k: np.ndarray, v: np.ndarray, resident: np.ndarray, seq_lens: np.ndarray,
                     window: int, block: int = 16):
    """The working set of a slot table, gathered from the full cache.

    Pool slot s of (b, h) holds logical block resident[b, h, s] (zeros for an
    empty slot); ring slot j mod WB holds window block j for every j in
    [first_window_block, num_blocks) (zeros elsewhere).
    k, v: [B, H, NB, block, d]; resident: [B, H, K].  Returns pool_k, pool_v
    [B, H, K, block, d] and ring_k, ring_v [B, H, WB, block, d].
    """
    B, H, NB, bs, d = k.shape
    K = resident.shape[2]
    WB = window_ring_slots(window, block)
    pool_k = np.zeros((B, H, K, bs, d))
    pool_v = np.zeros((B, H, K, bs, d))
    ring_k = np.zeros((B, H, WB, bs, d))
    ring_v = np.zeros((B, H, WB, bs, d))
    for b in range(B):
        L = int(seq_lens[b])
        w0, nb = first_window_block(L, window, block), num_blocks(L, block)
        for h in range(H):
            for s in range(K):
                j = int(resident[b, h, s])
                if 0 <= j < NB:
                    pool_k[b, h, s] = k[b, h, j]
                    pool_v[b, h, s] = v[b, h, j]
            for j in range(w0, nb):
                ring_k[b, h, j % WB] = k[b, h, j]
                ring_v[b, h, j % WB] = v[b, h, j]
    return pool_k, pool_v, ring_k, ring_v


def execute_plan(pool_k: np.ndarray, pool_v: np.ndarray, plan: np.ndarray, plan_count: np.ndarray,
                 k: np.ndarray, v: np.ndarray):
    """Moves the admitted blocks into their slots: every plan row (slot, new,
    old) of (b, h), rows below plan_count, copies logical block ``new`` of the
    full cache into pool slot ``slot``; the evicted block ``old`` needs no
    transfer (the full tier keeps every block).  [xllm] section three, training
    flow step 3 (the transfer plan goes out as an asynchronous host-link
    transfer) and section five (KV transfer).  Returns new pool arrays.
    """
    pk, pv = pool_k.copy(), pool_v.copy()
    B, H = plan_count.shape
    for b in range(B):
        for h in range(H):
            for i in range(int(plan_count[b, h])):
                slot, new = int(plan[b, h, i, 0]), int(plan[b, h, i, 1])
                pk[b, h, slot] = k[b, h, new]
                pv[b, h, slot] = v[b, h, new]
    return pk, pv


def append_token(k: np.ndarray, v: np.ndarray, summ: np.ndarray, ring_k: np.ndarray,
                 ring_v: np.ndarray, k_new: np.ndarray, v_new: np.ndarray, seq_lens: np.ndarray,
                 window: int, block: int = 16):
    """Appends one decoded token per sequence: its key and value go to position
    L = seq_lens[b] of the full cache and of the window ring, and the summary of
    its block L // 16 is updated in place of a rebuild: the token's key itself
    when it opens the block, else the elementwise min and max with the summary so
    far.  [xllm] section three, component table (per-block per-dimension min/max
    summaries) and section five (compressed-key update).  The caller then counts
    the token into seq_lens.  Requires L < NB * block.

    k_new, v_new: [B, H, d].  Returns updated copies of k, v, summ, ring_k, ring_v.
    """
    k, v, summ = k.copy(), v.copy(), summ.copy()
    ring_k, ring_v = ring_k.copy(), ring_v.copy()
    B, H = k.shape[:2]
    WB = ring_k.shape[2]
    for b in range(B):
        L = int(seq_lens[b])
        j, t = divmod(L, block)
        for h in range(H):
            k[b, h, j, t] = k_new[b, h]
            v[b, h, j, t] = v_new[b, h]
            ring_k[b, h, j % WB, t] = k_new[b, h]
            ring_v[b, h, j % WB, t] = v_new[b, h]
            if t == 0:
                summ[b, h, j, 0] = k_new[b, h]
                summ[b, h, j, 1] = k_new[b, h]
            else:
                summ[b, h, j, 0] = np.minimum(summ[b, h, j, 0], k_new[b, h])
                summ[b, h, j, 1] = np.maximum(summ[b, h, j, 1], k_new[b, h])
    return k, v, summ, ring_k, ring_v


def pool_attention(q: np.ndarray, pool_k: np.ndarray, pool_v: np.ndarray, ring_k: np.ndarray,
                   ring_v: np.ndarray, resident: np.ndarray, seq_lens: np.ndarray, window: int,
                   scale: float, block: int = 16) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of each target query over its head's working set as stored in
    HBM: the pool slots whose block is historical (0 <= resident < first window
    block; every token of such a block is inside the length) and the window
    blocks, read from their ring slots with tokens past the length dropped.
    Same softmax as ``sparse_attention``.  Returns out [B, H, G, d], lse [B, H, G].
    """
    B, H, G, Q, d = q.shape
    WB = ring_k.shape[2]
    out = np.zeros((B, H, G, d))
    lse = np.full((B, H, G), NEG_INF)
    for b in range(B):
        L = int(seq_lens[b])
        w0, nb = first_window_block(L, window, block), num_blocks(L, block)
        for h in range(H):
            ks, vs = [], []
            for s in range(resident.shape[2]):
                if 0 <= int(resident[b, h, s]) < w0:
                    ks.append(pool_k[b, h, s])
                    vs.append(pool_v[b, h, s])
            for j in range(w0, nb):
                n = min(block, L - j * block)
                ks.append(ring_k[b, h, j % WB, :n])
                vs.append(ring_v[b, h, j % WB, :n])
            if not ks:
                continue
            kt, vt = np.concatenate(ks), np.concatenate(vs)
            for g in range(G):
                z = (kt @ q[b, h, g, 0]) * scale
                m = z.max()
                e = np.exp(z - m)
                out[b, h, g] = (e[:, None] * vt).sum(axis=0) / e.sum()
                lse[b, h, g] = m + math.log(e.sum())
    return out, lse


# ---------------------------------------------------------------------------
# The whole step
# ---------------------------------------------------------------------------

def decode_step(q, summ, k, v, seq_lens, resident, top_k: int, window: int, cap: int,
                scale: float, block: int = 16) -> Dict[str, np.ndarray]:
    """score -> top-K -> capped plan -> sparse attention over the updated table.

    [xllm] section three, training flow step 3 (draft queries scan the
    summaries, predict top-K, compare with the resident set, build the
    transfer plan) followed by attention over the head-wise table.  Reading:
    attention uses the table after the plan is applied.
    """
    s = score_blocks(q, summ, seq_lens, window, block)
    sel = topk_blocks(s, seq_lens, top_k, window, block)
    p = build_plan(s, sel, resident, seq_lens, cap, window, block)
    out, lse = sparse_attention(q, k, v, p["table"], p["table_count"], seq_lens, scale, block)
    return {"scores": s, "topk": sel, **p, "out": out, "lse": lse}


def decode_step_overlapped(q, summ, k, v, seq_lens, resident, top_k: int, window: int, cap: int,
                           scale: float, block: int = 16) -> Dict[str, np.ndarray]:
    """Foreground attention over the blocks resident now, and the background
    look-ahead that produces the resident set of the next step.

    [lode] point 3 (while the current token's attention runs over the hot KV
    entries, a background pipeline finds and stages the blocks needed next);
    [legible] summary (foreground attention over the resident entries,
    background look-ahead attention predicting future blocks); [xllm] section
    three, training flow step 3.  The two parts share only their inputs: the
    attention uses ``resident_table(resident)``; the plan is ``build_plan`` on
    the look-ahead scores and selection.  The returned ``resident`` is the
    next step's slot table.
    """
    table, tcount = resident_table(resident, seq_lens, window, block)
    out, lse = sparse_attention(q, k, v, table, tcount, seq_lens, scale, block)
    s = score_blocks(q, summ, seq_lens, window, block)
    sel = topk_blocks(s, seq_lens, top_k, window, block)
    p = build_plan(s, sel, resident, seq_lens, cap, window, block)
    return {"scores": s, "topk": sel, **p, "out": out, "lse": lse,
            "attn_table": table, "attn_table_count": tcount}
