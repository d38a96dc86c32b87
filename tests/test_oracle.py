"""Pins for the fp64 oracle: brute force, closed forms, textbook routines, invariants.

None of these tests re-types the oracle's own formula; each checks it against
something the pages or the mathematics fix independently, chosen so that a
dropped term, a wrong sign, a wrong index or a transposed operand fails.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _bf16(x):
    """Round float64 values to bf16 and widen back (inputs hold bf16 values exactly)."""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def _tiny_inputs(seed=0, B=2, H=2, G=2, Q=3, NB=9, d=8, lens=(137, 100)):
    r = _rng(seed)
    q = _bf16(r.standard_normal((B, H, G, Q, d)))
    k = _bf16(r.standard_normal((B, H, NB, 16, d)))
    v = _bf16(r.standard_normal((B, H, NB, 16, d)))
    return q, k, v, np.array(lens[:B])


# ---------------------------------------------------------------------------
# O0 summaries
# ---------------------------------------------------------------------------

def test_summaries_aligned_equal_library_reduction():
    r = _rng(1)
    k = _bf16(r.standard_normal((2, 3, 5, 16, 8)))
    lens = np.array([80, 80])
    s = ref.build_summaries(k, lens)
    np.testing.assert_array_equal(s[:, :, :, 0, :], np.amin(k, axis=3))
    np.testing.assert_array_equal(s[:, :, :, 1, :], np.amax(k, axis=3))


def test_summaries_ignore_tokens_past_length():
    r = _rng(2)
    k = _bf16(r.standard_normal((1, 1, 3, 16, 4)))
    k[0, 0, 2, 5:, :] = 1e6            # tokens 37.. are past the length
    k[0, 0, 2, 5:, 1] = -1e6
    lens = np.array([37])
    s = ref.build_summaries(k, lens)
    # brute force over the valid tokens only
    for d in range(4):
        vals = [k[0, 0, 2, t, d] for t in range(16) if 32 + t < 37]
        assert s[0, 0, 2, 0, d] == min(vals)
        assert s[0, 0, 2, 1, d] == max(vals)
    assert np.all(np.abs(s) < 1e5)


def test_summaries_bracket_and_attain():
    q, k, v, lens = _tiny_inputs(3)
    s = ref.build_summaries(k, lens)
    B, H, NB = k.shape[:3]
    for b in range(B):
        for j in range(NB):
            n = min(16, int(lens[b]) - 16 * j)
            if n <= 0:
                assert np.all(s[b, :, j] == 0)
                continue
            toks = k[b, :, j, :n, :]
            assert np.all(s[b, :, j, 0][:, None, :] <= toks)
            assert np.all(s[b, :, j, 1][:, None, :] >= toks)
            assert np.all(np.any(toks == s[b, :, j, 0][:, None, :], axis=1))
            assert np.all(np.any(toks == s[b, :, j, 1][:, None, :], axis=1))


def test_summary_is_one_sixteenth_of_kv():
    # [xllm] section three component table: the compressed key cache is 1/16 of the full KV.
    d, block = 128, 16
    summary_elems = 2 * d            # min and max per block
    kv_elems = 2 * block * d         # keys and values per block
    assert summary_elems * 16 == kv_elems


# ---------------------------------------------------------------------------
# O1 scores
# ---------------------------------------------------------------------------

def test_score_bounds_every_true_dot_product():
    q, k, v, lens = _tiny_inputs(4)
    W = 16
    summ = ref.build_summaries(k, lens)
    s = ref.score_blocks(q, summ, lens, W)
    B, H, G, Q, d = q.shape
    for b in range(B):
        n_cand = ref.first_window_block(lens[b], W)
        for h in range(H):
            for j in range(n_cand):
                n = min(16, int(lens[b]) - 16 * j)
                dots = q[b, h].reshape(-1, d) @ k[b, h, j, :n].T   # every row x every valid token
                assert s[b, h, j] >= dots.max() - 1e-12


def test_score_closed_forms():
    r = _rng(5)
    d = 8
    # 16 identical keys: the bound is tight, score = max over rows of q . k.
    key = _bf16(r.standard_normal(d))
    k = np.broadcast_to(key, (1, 1, 2, 16, d)).copy()
    q = _bf16(r.standard_normal((1, 1, 2, 2, d)))
    lens = np.array([32])
    s = ref.score_blocks(q, ref.build_summaries(k, lens), lens, window=0)
    assert s[0, 0, 0] == pytest.approx(max(float(row @ key) for row in q[0, 0].reshape(-1, d)), abs=1e-12)
    # non-negative queries read the max summary; non-positive queries the min summary
    k = _bf16(r.standard_normal((1, 1, 2, 16, d)))
    summ = ref.build_summaries(k, lens)
    qp = np.abs(q)
    s = ref.score_blocks(qp, summ, lens, window=0)
    assert s[0, 0, 1] == pytest.approx(max(float(row @ summ[0, 0, 1, 1]) for row in qp[0, 0].reshape(-1, d)), abs=1e-12)
    qn = -np.abs(q)
    s = ref.score_blocks(qn, summ, lens, window=0)
    assert s[0, 0, 1] == pytest.approx(max(float(row @ summ[0, 0, 1, 0]) for row in qn[0, 0].reshape(-1, d)), abs=1e-12)


def test_score_sign_split_identity_matmul():
    # max(q*a, q*b) = q+ * b + q- * a for a <= b, evaluated as one library matmul.
    q, k, v, lens = _tiny_inputs(6)
    W = 16
    summ = ref.build_summaries(k, lens)
    s = ref.score_blocks(q, summ, lens, W)
    B, H, G, Q, d = q.shape
    for b in range(B):
        n_cand = ref.first_window_block(lens[b], W)
        for h in range(H):
            rows = q[b, h].reshape(-1, d)
            A = np.concatenate([np.maximum(rows, 0), np.minimum(rows, 0)], axis=1)      # [R, 2d]
            Bm = np.concatenate([summ[b, h, :n_cand, 1], summ[b, h, :n_cand, 0]], axis=1)  # [n, 2d]
            alt = np.matmul(A, Bm.T).max(axis=0)
            np.testing.assert_allclose(s[b, h, :n_cand], alt, rtol=0, atol=1e-12)
            assert np.all(np.isneginf(s[b, h, n_cand:]))


def test_score_max_aggregation_pure_python():
    q, k, v, lens = _tiny_inputs(7, B=1, H=1, G=2, Q=2, NB=4, d=4, lens=(64,))
    summ = ref.build_summaries(k, lens)
    s = ref.score_blocks(q, summ, lens, window=16)
    for j in range(3):
        best = -math.inf
        for g in range(2):
            for i in range(2):
                tot = 0.0
                for dd in range(4):
                    a = q[0, 0, g, i, dd] * summ[0, 0, j, 0, dd]
                    c = q[0, 0, g, i, dd] * summ[0, 0, j, 1, dd]
                    tot += a if a > c else c
                best = max(best, tot)
        assert s[0, 0, j] == pytest.approx(best, abs=1e-12)
    assert s[0, 0, 3] == -math.inf


# ---------------------------------------------------------------------------
# O2 top-K
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("distinct", [True, False])
def test_topk_equals_full_sort(distinct):
    r = _rng(8)
    B, H, NB = 2, 3, 40
    scores = r.standard_normal((B, H, NB)) if distinct else r.integers(-2, 3, (B, H, NB)).astype(float)
    lens = np.array([16 * 40, 16 * 10 + 3])
    W, K = 16, 12
    sel = ref.topk_blocks(scores, lens, K, W)
    for b in range(B):
        n_cand = ref.first_window_block(lens[b], W)
        for h in range(H):
            full = sorted(range(n_cand), key=lambda j: (-scores[b, h, j], j))
            expect = (full + [-1] * K)[:K]
            assert list(sel[b, h]) == expect


def test_topk_fewer_candidates_than_k_pads():
    scores = np.array([[[3.0, 1.0, 2.0, 9.0, 9.0]]])
    lens = np.array([16 * 3 + 64])        # W = 64 -> candidates 0..2
    sel = ref.topk_blocks(scores, lens, 5, 64)
    assert list(sel[0, 0]) == [0, 2, 1, -1, -1]


def test_topk_brute_force_subsets():
    # The selected set maximises the score sum among all K-subsets (distinct scores).
    r = _rng(9)
    s = r.standard_normal(9)
    lens = np.array([16 * 9])
    sel = ref.topk_blocks(s[None, None], lens, 3, 0)[0, 0]
    best = max(itertools.combinations(range(9), 3), key=lambda c: sum(s[list(c)]))
    assert set(sel) == set(best)


# ---------------------------------------------------------------------------
# O3 plan
# ---------------------------------------------------------------------------

def test_plan_worked_example():
    with open(os.path.join(GOLDEN, "plan_worked_example.json")) as f:
        ex = json.load(f)
    NB = ex["num_blocks"]
    scores = np.full((1, 1, NB), -np.inf)
    sc = np.array(ex["scores_candidates"], dtype=float)
    scores[0, 0, : sc.size] = sc
    lens = np.array([ex["seq_len"]])
    K, W = ex["top_k"], ex["window"]
    sel = ref.topk_blocks(scores, lens, K, W)
    assert list(sel[0, 0]) == ex["expected_topk"]
    res = np.array([[ex["resident"]]])
    for case in ex["cases"]:
        p = ref.build_plan(scores, sel, res, lens, case["cap"], W)
        n = case["plan_count"]
        assert p["plan_count"][0, 0] == n
        assert p["plan"][0, 0, :n].tolist() == case["plan"]
        assert np.all(p["plan"][0, 0, n:] == -1)
        assert p["resident"][0, 0].tolist() == case["resident_after"]
        tc = int(p["table_count"][0, 0])
        assert p["table"][0, 0, :tc].tolist() == case["table"]
        assert np.all(p["table"][0, 0, tc:] == -1)


def _check_plan_invariants(s, S, R, cap, p, n_cand):
    S_set = set(int(x) for x in S if x >= 0)
    R_list = [int(x) for x in R]
    R_set = set(x for x in R_list if x >= 0)
    Rn = [int(x) for x in p["resident"]]
    n = int(p["plan_count"])
    A = [x for x in S if x >= 0 and int(x) not in R_set]
    assert n == min(cap, len(A))
    changed = [i for i in range(len(R_list)) if R_list[i] != Rn[i]]
    assert len(changed) == n
    assert set(x for x in Rn if x >= 0) <= R_set | S_set
    assert len(set(Rn) & S_set) == len(R_set & S_set) + n
    assert len([x for x in Rn if x >= 0]) == len(set(x for x in Rn if x >= 0))      # distinct
    assert all(x < n_cand for x in Rn if x >= 0)                                      # no window block
    # admitted blocks beat every new block left out; evicted stale blocks score no higher
    admitted = set(int(r[1]) for r in p["plan"][:n])
    left = [x for x in A if int(x) not in admitted]
    for a in admitted:
        for o in left:
            assert (s[a], -a) > (s[o], -o)
    evicted = [int(r[2]) for r in p["plan"][:n] if r[2] >= 0]
    kept_stale = [x for x in Rn if x >= 0 and x in R_set and x not in S_set]
    if evicted:
        for e in evicted:
            for kst in kept_stale:
                assert (s[e], -e) <= (s[kst], -kst)
    # empty slots are filled before any stale slot is evicted
    n_empty = sum(1 for x in R_list if x < 0)
    assert len(evicted) == max(0, n - n_empty)
    # the plan lists slots in ascending order and pairs them with ascending new blocks
    slots = [int(r[0]) for r in p["plan"][:n]]
    news = [int(r[1]) for r in p["plan"][:n]]
    assert slots == sorted(slots) and news == sorted(news)


def test_plan_invariants_random():
    r = _rng(10)
    for trial in range(300):
        K = int(r.integers(1, 9))
        n_cand = int(r.integers(1, 20))
        W = 32
        L = 16 * n_cand + W
        NB = n_cand + 3
        s = np.full(NB, -np.inf)
        s[:n_cand] = r.integers(-4, 5, n_cand) if trial % 2 else r.standard_normal(n_cand)
        S = ref.topk_blocks(s[None, None], np.array([L]), K, W)[0, 0]
        n_fill = min(K, n_cand, int(r.integers(0, K + 1)))
        R = np.full(K, -1)
        R[:n_fill] = r.choice(n_cand, n_fill, replace=False)
        r.shuffle(R)
        cap = int(r.integers(0, K + 2))
        p = ref.build_plan(s[None, None], S[None, None], R[None, None], np.array([L]), cap, W)
        one = {k: v[0, 0] for k, v in p.items()}
        _check_plan_invariants(s, S, R, cap, one, n_cand)
        # table = updated residents in slot order, then the window blocks
        tc = int(one["table_count"])
        entries = [int(x) for x in one["resident"] if x >= 0] + list(range(n_cand, ref.num_blocks(L)))
        assert one["table"][:tc].tolist() == entries


def test_plan_special_cases():
    r = _rng(11)
    K, n_cand, W = 8, 30, 64
    L = 16 * n_cand + W
    s = np.full(n_cand + 5, -np.inf)
    s[:n_cand] = r.standard_normal(n_cand)
    S = ref.topk_blocks(s[None, None], np.array([L]), K, W)
    R_full = np.array(r.choice(n_cand, K, replace=False))[None, None]
    # cap >= K with a full resident set: the resident set becomes the selection
    p = ref.build_plan(s[None, None], S, R_full, np.array([L]), K, W)
    assert set(p["resident"][0, 0].tolist()) == set(S[0, 0].tolist())
    # cap = 0: nothing changes
    p = ref.build_plan(s[None, None], S, R_full, np.array([L]), 0, W)
    assert p["plan_count"][0, 0] == 0 and np.array_equal(p["resident"], R_full)
    # resident == selection: empty plan whatever the cap
    p = ref.build_plan(s[None, None], S, S[:, :, ::-1].copy(), np.array([L]), K, W)
    assert p["plan_count"][0, 0] == 0


def test_plan_exhaustive_tiny():
    # Every resident set of K = 3 slots over 6 candidates (with empties), every cap:
    # the result equals the rule stated in words, evaluated by enumeration of
    # all slot assignments and picking the unique one the rule allows.
    s = np.array([0.5, 2.0, -1.0, 3.0, 1.0, 0.0, -np.inf, -np.inf])
    L, W, K = 16 * 6 + 32, 32, 3
    S = ref.topk_blocks(s[None, None], np.array([L]), K, W)[0, 0]       # [3, 1, 4]
    assert S.tolist() == [3, 1, 4]
    vals = [-1] + list(range(6))
    for R in itertools.product(vals, repeat=K):
        filled = [x for x in R if x >= 0]
        if len(filled) != len(set(filled)):
            continue
        for cap in range(0, 4):
            p = ref.build_plan(s[None, None], S[None, None], np.array(R)[None, None], np.array([L]), cap, W)
            newR = p["resident"][0, 0].tolist()
            # enumerate all outcomes: choose which slots change and to what
            new_blocks = [x for x in S if x not in R]
            n = min(cap, len(new_blocks))
            want_new = set(new_blocks[:n])                       # best n by selection order
            empties = [i for i in range(K) if R[i] < 0]
            stale = sorted([i for i in range(K) if R[i] >= 0 and R[i] not in S],
                           key=lambda i: (s[R[i]], -R[i]))
            want_slots = sorted((empties + stale)[:n])
            candidates = []
            for slots in itertools.combinations(range(K), n):
                for perm in itertools.permutations(sorted(want_new)):
                    out = list(R)
                    for sl, bl in zip(slots, perm):
                        out[sl] = bl
                    ok = (list(slots) == want_slots and list(perm) == sorted(want_new))
                    if ok:
                        candidates.append(out)
            assert len(candidates) == 1
            assert newR == candidates[0]


def test_plan_exhaustive_k4_over_12_candidates():
    """Every slot table of K = 4 slots over 12 candidates (empties included) and every
    cap 0..4, on scores with ties: the plan equals the rule in words (the best n new
    blocks of the selection, n = min(cap, new); empties first by slot, then stale slots
    lowest score first, equal scores higher block first; slots ascending take blocks
    ascending; everything else unchanged)."""
    s = np.array([1.0, 3.0, 2.0, 3.0, 0.5, 2.0, 1.0, 4.0, 0.5, 2.0, 1.5, 1.0])
    W, K = 48, 4
    L = 16 * 12 + W
    S = ref.topk_blocks(s[None, None], np.array([L]), K, W)[0, 0].tolist()
    assert S == [7, 1, 3, 2]                     # 3.0 tie: block 1 before 3; 2.0 tie: 2 first
    Sset = set(S)
    n_cfg = 0
    for R in itertools.product([-1] + list(range(12)), repeat=K):
        filled = [x for x in R if x >= 0]
        if len(filled) != len(set(filled)):
            continue
        n_cfg += 1
        new_blocks = [x for x in S if x not in R]
        empties = [i for i in range(K) if R[i] < 0]
        stale = sorted([i for i in range(K) if R[i] >= 0 and R[i] not in Sset],
                       key=lambda i: (s[R[i]], -R[i]))
        for cap in range(0, 5):
            p = ref.build_plan(s[None, None], np.array(S)[None, None], np.array(R)[None, None],
                               np.array([L]), cap, W)
            n = min(cap, len(new_blocks))
            slots = sorted((empties + stale)[:n])
            blocks = sorted(new_blocks[:n])
            want = list(R)
            for sl, bl in zip(slots, blocks):
                want[sl] = bl
            assert p["resident"][0, 0].tolist() == want, (R, cap)
            assert int(p["plan_count"][0, 0]) == n
            rows = [tuple(int(x) for x in p["plan"][0, 0, i]) for i in range(n)]
            assert rows == [(sl, bl, R[sl]) for sl, bl in zip(slots, blocks)], (R, cap)
    assert n_cfg == 1 + 4 * 12 + 6 * 132 + 4 * 1320 + 11880


# ---------------------------------------------------------------------------
# O4 attention
# ---------------------------------------------------------------------------

def test_attention_all_blocks_equals_dense_sdpa():
    q, k, v, lens = _tiny_inputs(12, B=2, H=2, G=3, Q=2, NB=6, d=16, lens=(96, 77))
    B, H, G, Q, d = q.shape
    NB = k.shape[2]
    table = np.tile(np.arange(NB), (B, H, 1))
    tc = np.full((B, H), NB)
    scale = 1 / math.sqrt(d)
    out, lse = ref.sparse_attention(q, k, v, table, tc, lens, scale)
    for b in range(B):
        L = int(lens[b])
        kk = torch.from_numpy(k[b].reshape(H, NB * 16, d)[:, :L])
        vv = torch.from_numpy(v[b].reshape(H, NB * 16, d)[:, :L])
        qq = torch.from_numpy(q[b, :, :, 0, :])                              # [H, G, d]
        dense = torch.nn.functional.scaled_dot_product_attention(
            qq[:, :, None, :], kk[:, None].expand(H, G, L, d), vv[:, None].expand(H, G, L, d), scale=scale)
        np.testing.assert_allclose(out[b], dense[:, :, 0, :].numpy(), rtol=0, atol=1e-12)
        z = torch.einsum("hgd,htd->hgt", qq, kk) * scale
        np.testing.assert_allclose(lse[b], torch.logsumexp(z, dim=-1).numpy(), rtol=0, atol=1e-12)


def test_attention_special_cases():
    q, k, v, lens = _tiny_inputs(13, B=1, H=1, G=2, Q=2, NB=5, d=8, lens=(70,))
    scale = 0.3
    # constant values: output equals that value
    vc = np.broadcast_to(np.arange(8.0), v.shape).copy()
    table = np.array([[[4, 0, 2, -1, -1]]])
    tc = np.array([[3]])
    out, _ = ref.sparse_attention(q, k, vc, table, tc, lens, scale)
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(np.arange(8.0), (2, 8)), atol=1e-12)
    # permutation invariance
    o1, l1 = ref.sparse_attention(q, k, v, table, tc, lens, scale)
    o2, l2 = ref.sparse_attention(q, k, v, np.array([[[2, 4, 0, -1, -1]]]), tc, lens, scale)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l1, l2, atol=1e-12)
    # one partial block (block 4 holds tokens 64..69): closed-form softmax over 6 tokens
    o, l = ref.sparse_attention(q, k, v, np.array([[[4, -1, -1, -1, -1]]]), np.array([[1]]), lens, scale)
    for g in range(2):
        z = [float(q[0, 0, g, 0] @ k[0, 0, 4, t]) * scale for t in range(6)]
        m = max(z)
        w = [math.exp(x - m) for x in z]
        expect = sum(wi * v[0, 0, 4, t] for t, wi in enumerate(w)) / sum(w)
        np.testing.assert_allclose(o[0, 0, g], expect, atol=1e-12)
        assert l[0, 0, g] == pytest.approx(m + math.log(sum(w)), abs=1e-12)
    # no token at all: zeros and -inf
    o, l = ref.sparse_attention(q, k, v, np.full((1, 1, 5), -1), np.array([[0]]), lens, scale)
    assert np.all(o == 0) and np.all(np.isneginf(l))


def test_attention_uses_target_query_only():
    q, k, v, lens = _tiny_inputs(14, B=1, H=1, G=1, Q=3, NB=3, d=8, lens=(48,))
    table, tc = np.array([[[0, 1, 2]]]), np.array([[3]])
    o1, _ = ref.sparse_attention(q, k, v, table, tc, lens, 0.35)
    q2 = q.copy()
    q2[:, :, :, 1:, :] = 0.0
    o2, _ = ref.sparse_attention(q2, k, v, table, tc, lens, 0.35)
    np.testing.assert_array_equal(o1, o2)


# ---------------------------------------------------------------------------
# geometry, cap, budget
# ---------------------------------------------------------------------------

def test_window_geometry():
    # the window blocks overlap the last W tokens; count <= ceil(W/16) + 1
    for L in range(1, 400):
        for W in (0, 1, 15, 16, 17, 64, 128):
            w0, nb = ref.first_window_block(L, W), ref.num_blocks(L)
            toks = set(range(max(0, L - W), L))
            covered = set(t for j in range(w0, nb) for t in range(16 * j, min(16 * j + 16, L)))
            assert toks <= covered
            if w0 > 0:
                assert 16 * w0 <= L - W          # block w0 - 1 lies wholly before the window
            assert nb - w0 <= -(-W // 16) + 1


def test_fetch_cap_values():
    assert ref.fetch_cap(0.05, 128) == 6          # default ratio at K = 128
    assert ref.fetch_cap(0.05, 16) == 0
    assert ref.fetch_cap(0.29, 100) == 29
    assert [ref.fetch_cap(x, 128) for x in (0.01, 0.02, 0.05, 0.10, 0.20)] == [1, 2, 6, 12, 25]
    assert ref.fetch_cap(1.0, 128) == 128


def test_token_budget():
    # [lode] and [xllm] section six: K = 128 blocks of 16 tokens is the 2,048-token budget.
    assert 128 * 16 == 2048


# ---------------------------------------------------------------------------
# the whole step on the small synthetic workload
# ---------------------------------------------------------------------------

def test_decode_step_tiny_workload():
    import synth
    w = synth.WORKLOADS["tiny_4k"]
    inp = synth.generate(w, "cpu")
    f64 = lambda t: t.to(torch.float64).numpy()
    q, k, v = f64(inp["q"]), f64(inp["k"]), f64(inp["v"])
    lens = inp["seq_lens"].numpy()
    summ = ref.build_summaries(k, lens)
    s = ref.score_blocks(q, summ, lens, w.window)
    sel = ref.topk_blocks(s, lens, w.top_k, w.window)
    R = synth.resident_from_selection(w, torch.from_numpy(sel), inp["seq_lens"]).numpy()
    res = ref.decode_step(q, summ, k, v, lens, R, w.top_k, w.window, w.cap, 1 / math.sqrt(128))
    assert w.cap == 0
    assert np.all(res["plan_count"] == 0) and np.array_equal(res["resident"], R)
    # planted blocks carry a +2|q| shift along one target direction, several standard
    # deviations of the bound's spread: most of them make the top-K
    planted = inp["planted"].numpy()
    for h in range(w.num_kv_heads):
        hot = set(np.nonzero(planted[0, h])[0].tolist())
        assert len(hot) == w.planted
        assert len(hot & set(sel[0, h].tolist())) >= w.planted // 2
    assert np.all(res["table_count"] == w.top_k + 4)
    assert np.all(np.isfinite(res["out"]))


# ---------------------------------------------------------------------------
# The working set as resident slots (foreground attention of the overlapped step)
# ---------------------------------------------------------------------------

def test_resident_table_hand_example():
    # len 700, W 64: first window block floor(636 / 16) = 39, blocks ceil(700 / 16) = 44.
    # Slot 1 is empty; block 40 lies in the window and is listed once, as a window block.
    R = np.array([[[5, -1, 40, 2]]])
    table, count = ref.resident_table(R, np.array([700]), 64)
    assert count.tolist() == [[7]]
    assert table[0, 0, :7].tolist() == [5, 2, 39, 40, 41, 42, 43]
    assert np.all(table[0, 0, 7:] == -1) and table.shape[-1] == 4 + 4 + 1


def test_plan_table_lists_a_window_reached_block_once():
    """Hand example: len 700, W 64, so the first window block is floor(636 / 16) = 39
    and the blocks run to ceil(700 / 16) = 44.  Slots hold [5, -1, 40, 2]: slot 1 is
    empty and block 40 lies in the window.  The selection is [5, 2, 10, 11]."""
    NB, K, W = 48, 4, 64
    lens = np.array([700])
    scores = np.full((1, 1, NB), -np.inf)
    scores[0, 0, :39] = np.linspace(1.0, 0.5, 39)   # candidates only; 40 is not one
    scores[0, 0, [5, 2, 10, 11]] = [9.0, 8.0, 7.0, 6.0]
    sel = ref.topk_blocks(scores, lens, K, W)
    assert sel[0, 0].tolist() == [5, 2, 10, 11]
    R = np.array([[[5, -1, 40, 2]]])
    # cap 0: nothing moves; block 40 is attended once, as a window block
    p = ref.build_plan(scores, sel, R, lens, 0, W)
    assert p["resident"][0, 0].tolist() == [5, -1, 40, 2]
    assert p["table_count"].tolist() == [[7]]
    assert p["table"][0, 0, :7].tolist() == [5, 2, 39, 40, 41, 42, 43]
    # cap 1: the best new block (10) fills the empty slot; 40 stays resident, listed once
    p = ref.build_plan(scores, sel, R, lens, 1, W)
    assert p["resident"][0, 0].tolist() == [5, 10, 40, 2]
    assert p["table"][0, 0, :8].tolist() == [5, 10, 2, 39, 40, 41, 42, 43]
    # cap 4: both new blocks; the empty slot, then the window-reached block (score -inf,
    # the worst stale one) are freed, and slots 1, 2 take blocks 10, 11 in order
    p = ref.build_plan(scores, sel, R, lens, 4, W)
    assert p["plan_count"].tolist() == [[2]]
    assert p["plan"][0, 0, :2].tolist() == [[1, 10, -1], [2, 11, 40]]
    assert p["resident"][0, 0].tolist() == [5, 10, 11, 2]
    assert p["table"][0, 0, :9].tolist() == [5, 10, 11, 2, 39, 40, 41, 42, 43]
    # either way the table is the resident-slot table of the updated set
    for cap in (0, 1, 4):
        p = ref.build_plan(scores, sel, R, lens, cap, W)
        table, count = ref.resident_table(p["resident"], lens, W)
        np.testing.assert_array_equal(table, p["table"])
        np.testing.assert_array_equal(count, p["table_count"])


def test_resident_table_of_planned_set_is_the_plan_table():
    r = _rng(11)
    B, H, NB, K, W = 2, 3, 64, 12, 40
    lens = np.array([1000, 611])
    for trial in range(5):
        scores = r.standard_normal((B, H, NB))
        sel = ref.topk_blocks(scores, lens, K, W)
        res = np.full((B, H, K), -1)
        for b in range(B):
            n_cand = ref.first_window_block(int(lens[b]), W)
            for h in range(H):
                m = min(K - trial, n_cand)
                nb = ref.num_blocks(int(lens[b]))
                res[b, h, :m] = r.choice(nb, size=m, replace=False)   # window blocks too
                r.shuffle(res[b, h])
        p = ref.build_plan(scores, sel, res, lens, 3, W)
        table, count = ref.resident_table(p["resident"], lens, W)
        np.testing.assert_array_equal(table, p["table"])
        np.testing.assert_array_equal(count, p["table_count"])


@pytest.mark.parametrize("cap", [0, 4])
def test_overlapped_step_agrees_with_serial_when_the_plan_changes_nothing(cap):
    """The two step orders attend over the same blocks exactly when the plan leaves
    the slot table unchanged: cap 0, or a resident set equal to the selection."""
    q, k, v, lens = _tiny_inputs(seed=3, NB=12, lens=(190, 150))
    summ = ref.build_summaries(k, lens)
    K, W = 5, 32
    s = ref.score_blocks(q, summ, lens, W)
    sel = ref.topk_blocks(s, lens, K, W)
    R = sel.copy() if cap else sel[:, :, ::-1].copy()     # the selected set, in some slot order
    a = ref.decode_step(q, summ, k, v, lens, R, K, W, cap, 0.125)
    o = ref.decode_step_overlapped(q, summ, k, v, lens, R, K, W, cap, 0.125)
    assert np.all(a["plan_count"] == 0) and np.all(o["plan_count"] == 0)
    np.testing.assert_array_equal(o["resident"], R)
    np.testing.assert_allclose(o["out"], a["out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(o["lse"], a["lse"], rtol=0, atol=1e-12)
    # and the attention differs once the plan does change the set
    R2 = np.where(np.arange(K) < 2, -1, sel)              # two empty slots to fill
    a2 = ref.decode_step(q, summ, k, v, lens, R2, K, W, 4, 0.125)
    o2 = ref.decode_step_overlapped(q, summ, k, v, lens, R2, K, W, 4, 0.125)
    assert np.all(a2["plan_count"] == 2)
    assert np.abs(o2["out"] - a2["out"]).max() > 1e-6


# ---------------------------------------------------------------------------
# The working set in HBM: pool, window ring, plan execution, appended tokens
# ---------------------------------------------------------------------------

def _marked_cache(B, H, NB, d=4):
    """K and V whose every token row holds (b, h, block, token) codes: a copy's origin
    can be read off the values."""
    k = np.zeros((B, H, NB, 16, d))
    for b, h, j, t in itertools.product(range(B), range(H), range(NB), range(16)):
        k[b, h, j, t] = [b, h, j, t][:d] + [0] * max(0, d - 4)
    return k, -k


def test_ring_slot_hand_example():
    """W = 32: ring of ceil(32/16) + 1 = 3 slots.  Length 100: blocks 0..6, first
    window block (100 - 32) // 16 = 4, so blocks 4, 5, 6 sit in ring slots 1, 2, 0."""
    assert ref.window_ring_slots(32) == 3 and ref.window_ring_slots(0) == 1
    assert ref.window_ring_slots(128) == 9 and ref.window_ring_slots(64) == 5
    k, v = _marked_cache(1, 1, 8)
    R = np.array([[[2, -1, 0]]])
    pk, pv, rk, rv = ref.fill_working_set(k, v, R, np.array([100]), 32)
    assert rk.shape == (1, 1, 3, 16, 4)
    assert [int(rk[0, 0, s, 0, 2]) for s in range(3)] == [6, 4, 5]
    assert np.array_equal(rv[0, 0, 1], -k[0, 0, 4])
    assert np.array_equal(pk[0, 0, 0], k[0, 0, 2]) and np.array_equal(pk[0, 0, 2], k[0, 0, 0])
    assert not pk[0, 0, 1].any() and not pv[0, 0, 1].any()      # the empty slot stays empty


def test_ring_of_zero_window_holds_the_partial_last_block():
    k, v = _marked_cache(1, 1, 4)
    _, _, rk, _ = ref.fill_working_set(k, v, np.full((1, 1, 2), -1), np.array([37]), 0)
    assert rk.shape[2] == 1 and int(rk[0, 0, 0, 0, 2]) == 2      # block 2 holds tokens 32..36
    _, _, rk, _ = ref.fill_working_set(k, v, np.full((1, 1, 2), -1), np.array([48]), 0)
    assert not rk.any()                                           # aligned: no window block


@pytest.mark.parametrize("window", [0, 40, 64])
def test_pool_attention_equals_table_attention(window):
    """Attention over the working set as stored (pool slots + ring) equals attention
    over the slot table written out as a table, read from the full cache."""
    q, k, v, lens = _tiny_inputs(seed=21, NB=12, lens=(187, 100))
    r = _rng(22)
    B, H, K = 2, 2, 5
    R = np.full((B, H, K), -1)
    for b, h in itertools.product(range(B), range(H)):
        nb = ref.num_blocks(int(lens[b]))
        picks = r.choice(nb, size=K - 1, replace=False)           # may reach into the window
        R[b, h, : K - 1] = picks
        r.shuffle(R[b, h])
    scale = 1 / math.sqrt(8)
    pk, pv, rk, rv = ref.fill_working_set(k, v, R, lens, window)
    out, lse = ref.pool_attention(q, pk, pv, rk, rv, R, lens, window, scale)
    table, tc = ref.resident_table(R, lens, window)
    eo, el = ref.sparse_attention(q, k, v, table, tc, lens, scale)
    np.testing.assert_allclose(out, eo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, el, rtol=0, atol=1e-12)


def test_execute_plan_gives_the_gather_of_the_next_slot_table():
    """After the plan's copies the pool is exactly what gathering the updated slot
    table from the full cache gives: admitted blocks in their slots, the rest
    untouched."""
    q, k, v, lens = _tiny_inputs(seed=23, NB=14, lens=(220, 150))
    summ = ref.build_summaries(k, lens)
    W, K, cap = 32, 6, 3
    s = ref.score_blocks(q, summ, lens, W)
    sel = ref.topk_blocks(s, lens, K, W)
    r = _rng(24)
    R = np.full((2, 2, K), -1)
    for b, h in itertools.product(range(2), range(2)):
        nc = ref.first_window_block(int(lens[b]), W)
        R[b, h, :4] = r.choice(nc, size=4, replace=False)
    p = ref.build_plan(s, sel, R, lens, cap, W)
    assert p["plan_count"].sum() > 0
    pk, pv, _, _ = ref.fill_working_set(k, v, R, lens, W)
    nk, nv = ref.execute_plan(pk, pv, p["plan"], p["plan_count"], k, v)
    ek, ev, _, _ = ref.fill_working_set(k, v, p["resident"], lens, W)
    np.testing.assert_array_equal(nk, ek)
    np.testing.assert_array_equal(nv, ev)
    np.testing.assert_array_equal(pk, ref.fill_working_set(k, v, R, lens, W)[0])   # inputs untouched


def test_append_token_matches_a_rebuild():
    """Tokens appended one at a time (across block boundaries, from a partial block):
    after each, the summaries equal a rebuild from the full cache, the ring equals
    a fresh gather of the window, and the full cache holds the token."""
    r = _rng(25)
    B, H, NB, d, W = 2, 2, 6, 8, 24
    k = _bf16(r.standard_normal((B, H, NB, 16, d)))
    v = _bf16(r.standard_normal((B, H, NB, 16, d)))
    lens = np.array([13, 30])
    summ = ref.build_summaries(k, lens)
    R = np.full((B, H, 2), -1)
    _, _, rk, rv = ref.fill_working_set(k, v, R, lens, W)
    for step in range(40):
        kn = _bf16(r.standard_normal((B, H, d)) * (1 + step % 3))
        vn = _bf16(r.standard_normal((B, H, d)))
        k, v, summ, rk, rv = ref.append_token(k, v, summ, rk, rv, kn, vn, lens, W)
        for b in range(B):
            j, t = divmod(int(lens[b]), 16)
            assert np.array_equal(k[b, :, j, t], kn[b]) and np.array_equal(v[b, :, j, t], vn[b])
        lens = lens + 1
        rebuilt = ref.build_summaries(k, lens)
        for b in range(B):
            nb = ref.num_blocks(int(lens[b]))
            np.testing.assert_array_equal(summ[b, :, :nb], rebuilt[b, :, :nb])
        _, _, ek, ev = ref.fill_working_set(k, v, R, lens, W)
        for b in range(B):
            L = int(lens[b])
            for j in range(ref.first_window_block(L, W), ref.num_blocks(L)):
                n = min(16, L - 16 * j)
                np.testing.assert_array_equal(rk[b, :, j % 3, :n], ek[b, :, j % 3, :n])
                np.testing.assert_array_equal(rv[b, :, j % 3, :n], ev[b, :, j % 3, :n])


# ---------------------------------------------------------------------------
# Prediction quality: attention share per block, ranking overlap
# ---------------------------------------------------------------------------

def test_block_mass_through_per_block_log_sum_exp():
    """A block's share is exp(lse over the block alone - lse over every token), the
    log-sum-exps coming from the (separately pinned) attention oracle; the group
    takes the largest share."""
    q, k, v, lens = _tiny_inputs(seed=51, NB=10, lens=(150, 77))
    W, scale = 32, 1 / math.sqrt(8)
    qt = q[:, :, :, 0, :]
    mass = ref.block_attention_mass(qt, k, lens, W, scale)
    B, H, G = qt.shape[:3]
    for b, h in itertools.product(range(B), range(H)):
        L = int(lens[b])
        nb, nc = ref.num_blocks(L), ref.first_window_block(L, W)
        sub = (q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1])
        all_t = np.arange(nb)[None, None]
        _, lse_all = ref.sparse_attention(*sub, all_t, np.array([[nb]]), lens[b:b + 1], scale)
        for j in range(10):
            if j >= nc:
                assert mass[b, h, j] == -np.inf
                continue
            _, lse_j = ref.sparse_attention(*sub, np.array([[[j]]]), np.array([[1]]), lens[b:b + 1], scale)
            expect = np.exp(lse_j[0, 0] - lse_all[0, 0]).max()
            np.testing.assert_allclose(mass[b, h, j], expect, rtol=1e-12)


def test_block_mass_closed_forms():
    """Identical keys: every token weighs 1/L, so a full block holds 16/L; shares of
    the candidates plus the window's add up to 1 for a single query head."""
    B, H, NB, d = 1, 1, 8, 4
    k = np.ones((B, H, NB, 16, d))
    q = np.array([[[[0.3, -1.0, 2.0, 0.5]]]])
    m = ref.block_attention_mass(q, k, np.array([100]), 20, 0.5)
    nc = ref.first_window_block(100, 20)                      # 5 candidate blocks
    np.testing.assert_allclose(m[0, 0, :nc], 16 / 100, rtol=1e-13)
    assert np.all(m[0, 0, nc:] == -np.inf)
    q2, k2, _, lens = _tiny_inputs(seed=52, B=1, H=1, G=1, NB=9, lens=(137,))
    m2 = ref.block_attention_mass(q2[:, :, :, 0, :], k2, lens, 0, 0.7)
    z = k2[0, 0].reshape(-1, 8)[:137] @ q2[0, 0, 0, 0] * 0.7
    p = np.exp(z - z.max()) / np.exp(z - z.max()).sum()
    window_share = p[ref.first_window_block(137, 0) * 16:].sum()
    np.testing.assert_allclose(m2[0, 0, :8].sum() + window_share, 1.0, rtol=1e-12)


def test_top_overlap_by_hand():
    assert ref.top_overlap(np.array([3, 1, 2, 9]), np.array([1, 3, 5, 9]), 2) == 1.0
    assert ref.top_overlap(np.array([3, 1, 2, 9]), np.array([1, 5, 3, 9]), 2) == 0.5
    assert ref.top_overlap(np.array([3, 1, 2, 9]), np.array([7, 5, 3, 9]), 4) == 0.5
    assert ref.top_overlap(np.array([4, -1, -1]), np.array([4, -1, -1]), 3) == 1.0
    assert ref.top_overlap(np.array([-1, -1]), np.array([-1, -1]), 2) == 1.0


# ---------------------------------------------------------------------------
# Block sizes other than 16 (the pages fix 16; 8, 32 and 64 are a sweep variant)
# ---------------------------------------------------------------------------

def test_summaries_of_merged_blocks():
    """A block of 2b tokens is two blocks of b tokens: its summary is the elementwise
    min / max of the halves' summaries over the halves that hold a valid token."""
    r = _rng(40)
    B, H, NB16, d = 3, 2, 8, 8
    k16 = _bf16(r.standard_normal((B, H, NB16, 16, d)))
    lens = np.array([128, 71, 9])                      # aligned, partial, inside the first half
    s16 = ref.build_summaries(k16, lens, 16)
    for small, big in ((8, 16), (16, 32), (32, 64)):
        ks = k16.reshape(B, H, -1, small, d)
        kb = k16.reshape(B, H, -1, big, d)
        ss, sb = ref.build_summaries(ks, lens, small), ref.build_summaries(kb, lens, big)
        if small == 16:
            np.testing.assert_array_equal(ss, s16)
        for b, j in itertools.product(range(B), range(kb.shape[2])):
            L = int(lens[b])
            halves = [2 * j + i for i in range(2) if (2 * j + i) * small < L]
            if not halves:
                assert not sb[b, :, j].any()
                continue
            np.testing.assert_array_equal(sb[b, :, j, 0], np.min([ss[b, :, i, 0] for i in halves], axis=0))
            np.testing.assert_array_equal(sb[b, :, j, 1], np.max([ss[b, :, i, 1] for i in halves], axis=0))


@pytest.mark.parametrize("block", [8, 32, 64])
def test_score_bounds_every_true_dot_product_other_block_sizes(block):
    r = _rng(41 + block)
    B, H, G, Q, d, NB = 2, 2, 2, 3, 8, 5
    q = _bf16(r.standard_normal((B, H, G, Q, d)))
    k = _bf16(r.standard_normal((B, H, NB, block, d)))
    lens = np.array([NB * block, NB * block - block - 3])
    W = block // 2 + 1
    s = ref.score_blocks(q, ref.build_summaries(k, lens, block), lens, W, block)
    for b in range(B):
        n_cand = (int(lens[b]) - W) // block                 # blocks wholly before the window
        assert np.all(np.isneginf(s[b, :, n_cand:]))
        for h, j in itertools.product(range(H), range(n_cand)):
            dots = q[b, h].reshape(-1, d) @ k[b, h, j].T
            assert s[b, h, j] >= dots.max() - 1e-12
            # attained when every row's sign pattern is met by one token: a lone token
            one = k.copy()
            one[b, h, j] = k[b, h, j, :1]
            s1 = ref.score_blocks(q, ref.build_summaries(one, lens, block), lens, W, block)
            assert s1[b, h, j] == pytest.approx((q[b, h].reshape(-1, d) @ k[b, h, j, 0]).max(), abs=1e-12)


@pytest.mark.parametrize("block", [8, 32, 64])
def test_attention_all_blocks_equals_dense_other_block_sizes(block):
    r = _rng(50 + block)
    B, H, G, Q, d = 2, 2, 3, 2, 16
    NB = 256 // block
    q = _bf16(r.standard_normal((B, H, G, Q, d)))
    k = _bf16(r.standard_normal((B, H, NB, block, d)))
    v = _bf16(r.standard_normal((B, H, NB, block, d)))
    lens = np.array([256, 211])
    table = np.tile(np.arange(NB), (B, H, 1))
    tc = np.full((B, H), NB)
    scale = 1 / math.sqrt(d)
    out, lse = ref.sparse_attention(q, k, v, table, tc, lens, scale, block)
    for b in range(B):
        L = int(lens[b])
        kk = torch.from_numpy(k[b].reshape(H, NB * block, d)[:, :L])
        vv = torch.from_numpy(v[b].reshape(H, NB * block, d)[:, :L])
        qq = torch.from_numpy(q[b, :, :, 0, :])
        dense = torch.nn.functional.scaled_dot_product_attention(
            qq[:, :, None, :], kk[:, None].expand(H, G, L, d), vv[:, None].expand(H, G, L, d), scale=scale)
        np.testing.assert_allclose(out[b], dense[:, :, 0, :].numpy(), rtol=0, atol=1e-12)
        z = torch.einsum("hgd,htd->hgt", qq, kk) * scale
        np.testing.assert_allclose(lse[b], torch.logsumexp(z, dim=-1).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("block", [8, 32, 64])
def test_window_geometry_other_block_sizes(block):
    assert ref.num_blocks(100, 32) == 4 and ref.first_window_block(100, 40, 32) == 1
    assert ref.num_blocks(100, 8) == 13 and ref.first_window_block(100, 40, 8) == 7
    for L in range(1, 300):
        for W in (0, 1, block - 1, block, block + 1, 64, 128):
            w0, nb = ref.first_window_block(L, W, block), ref.num_blocks(L, block)
            toks = set(range(max(0, L - W), L))
            covered = set(t for j in range(w0, nb) for t in range(block * j, min(block * j + block, L)))
            assert toks <= covered
            assert block * nb >= L > block * (nb - 1)
            if w0 > 0:
                assert block * w0 <= L - W
            assert nb - w0 <= ref.window_ring_slots(W, block) == -(-W // block) + 1


@pytest.mark.parametrize("block", [8, 32])
def test_pool_attention_equals_table_attention_other_block_sizes(block):
    r = _rng(60 + block)
    B, H, G, Q, d, K = 2, 2, 2, 2, 8, 5
    NB = 192 // block
    q = _bf16(r.standard_normal((B, H, G, Q, d)))
    k = _bf16(r.standard_normal((B, H, NB, block, d)))
    v = _bf16(r.standard_normal((B, H, NB, block, d)))
    lens = np.array([187, 100])
    R = np.full((B, H, K), -1)
    for b, h in itertools.product(range(B), range(H)):
        nb = ref.num_blocks(int(lens[b]), block)
        R[b, h, : K - 1] = r.choice(nb, size=K - 1, replace=False)
        r.shuffle(R[b, h])
    scale = 1 / math.sqrt(d)
    for window in (0, 40):
        pk, pv, rk, rv = ref.fill_working_set(k, v, R, lens, window, block)
        out, lse = ref.pool_attention(q, pk, pv, rk, rv, R, lens, window, scale, block)
        table, tc = ref.resident_table(R, lens, window, block)
        eo, el = ref.sparse_attention(q, k, v, table, tc, lens, scale, block)
        np.testing.assert_allclose(out, eo, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, el, rtol=0, atol=1e-12)


@pytest.mark.parametrize("block", [8, 32])
def test_append_token_matches_a_rebuild_other_block_sizes(block):
    r = _rng(70 + block)
    B, H, d, W = 2, 2, 8, 24
    NB = 96 // block
    k = _bf16(r.standard_normal((B, H, NB, block, d)))
    v = _bf16(r.standard_normal((B, H, NB, block, d)))
    lens = np.array([13, 30])
    summ = ref.build_summaries(k, lens, block)
    R = np.full((B, H, 2), -1)
    WB = ref.window_ring_slots(W, block)
    _, _, rk, rv = ref.fill_working_set(k, v, R, lens, W, block)
    for step in range(40):
        kn = _bf16(r.standard_normal((B, H, d)) * (1 + step % 3))
        vn = _bf16(r.standard_normal((B, H, d)))
        k, v, summ, rk, rv = ref.append_token(k, v, summ, rk, rv, kn, vn, lens, W, block)
        for b in range(B):
            assert np.array_equal(k.reshape(B, H, -1, d)[b, :, int(lens[b])], kn[b])
        lens = lens + 1
        rebuilt = ref.build_summaries(k, lens, block)
        np.testing.assert_array_equal(summ, rebuilt)
        _, _, ek, ev = ref.fill_working_set(k, v, R, lens, W, block)
        for b in range(B):
            L = int(lens[b])
            for j in range(ref.first_window_block(L, W, block), ref.num_blocks(L, block)):
                n = min(block, L - block * j)
                np.testing.assert_array_equal(rk[b, :, j % WB, :n], ek[b, :, j % WB, :n])


# ---------------------------------------------------------------------------
# Captured attention (the quality figure compared across block sizes)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("block", [8, 16, 32, 64])
def test_captured_attention_pins(block):
    """All candidates capture everything, none capture nothing, disjoint selections
    add, and identical keys spread the attention evenly over the tokens; with one
    query head it is the block shares of block_attention_mass, normalised."""
    r = _rng(80 + block)
    B, H, G, d = 2, 2, 3, 16
    NB = 512 // block
    q = _bf16(r.standard_normal((B, H, G, d)))
    k = _bf16(r.standard_normal((B, H, NB, block, d)))
    lens = np.array([512, 300])
    W, scale = 40, 1 / math.sqrt(d)
    n_cand = [ref.first_window_block(int(x), W, block) for x in lens]
    everything = np.full((B, H, NB), -1)
    for b in range(B):
        everything[b, :, :n_cand[b]] = np.arange(n_cand[b])
    np.testing.assert_allclose(ref.captured_attention(q, k, lens, W, scale, everything, block), 1.0,
                               rtol=0, atol=1e-12)
    nothing = np.full((B, H, 4), -1)
    assert np.all(ref.captured_attention(q, k, lens, W, scale, nothing, block) == 0.0)
    # ids outside the candidates (window, past the sequence) are ignored
    beyond = np.full((B, H, 2), NB + 3)
    beyond[:, :, 0] = [[n_cand[0]] * H, [n_cand[1]] * H]
    assert np.all(ref.captured_attention(q, k, lens, W, scale, beyond, block) == 0.0)
    for b in range(B):
        perm = r.permutation(n_cand[b])
        a, c = perm[: len(perm) // 3], perm[len(perm) // 3:]
        sa = np.full((B, H, len(perm)), -1)
        sc = np.full((B, H, len(perm)), -1)
        sa[b, :, :len(a)] = a
        sc[b, :, :len(c)] = c
        fa = ref.captured_attention(q, k, lens, W, scale, sa, block)[b]
        fc = ref.captured_attention(q, k, lens, W, scale, sc, block)[b]
        np.testing.assert_allclose(fa + fc, 1.0, rtol=0, atol=1e-12)
    same = np.broadcast_to(k[:, :, :1, :1], k.shape).copy()         # one key everywhere
    sel = np.full((B, H, 3), -1)
    sel[:, :, :3] = [0, 2, 3]
    got = ref.captured_attention(q, same, lens, W, scale, sel, block)
    for b in range(B):
        np.testing.assert_allclose(got[b], 3 * block / (n_cand[b] * block), rtol=0, atol=1e-12)
    q1 = q[:, :, :1]
    mass = ref.block_attention_mass(q1, k, lens, W, scale, block)
    got1 = ref.captured_attention(q1, k, lens, W, scale, sel, block)
    for b in range(B):
        for h in range(H):
            m = mass[b, h, :n_cand[b]]
            np.testing.assert_allclose(got1[b, h], m[[0, 2, 3]].sum() / m.sum(), rtol=1e-12)


def test_captured_attention_by_hand():
    """Two blocks of two tokens, one query head: the shares come from the softmax
    written out by hand."""
    q = np.array([[[[1.0, 0.0]]]])                        # [1, 1, 1, 2]
    k = np.array([[[[[0.0, 0.0], [1.0, 0.0]], [[2.0, 0.0], [0.0, 5.0]], [[9.0, 9.0], [9.0, 9.0]]]]])
    lens = np.array([5])                                  # window 1 token: block 2 is the window
    e = np.exp([0.0, 1.0, 2.0, 0.0, 9.0])
    p = e / e.sum()
    cand = p[0] + p[1] + p[2] + p[3]
    got = ref.captured_attention(q, k, lens, 1, 1.0, np.array([[[1, -1]]]), 2)
    np.testing.assert_allclose(got[0, 0], (p[2] + p[3]) / cand, rtol=1e-14)
