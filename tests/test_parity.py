"""GPU parity: every liboasis entry point against the fp64 oracle (tolerances in _helpers).

All calls go through the C ABI (ctypes binding).  Inputs are seeded synthetic
tensors; no expected value comes from the GPU.
"""
import math
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import ref
from tests._helpers import (OUT_ATOL, check_scores, default_scale, f64, i64, oracle_head,
                            oracle_selection_head, plan_robust, score_floor, selection_equivalent)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(msg):
    print(f"[parity] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    import oasis_score_summaries_amd as oa
    oa.load()
    return oa


def _dims(oa, B, H, G, NB, Q, K, W, ratio):
    return oa.make_dims(B, H, G, NB, Q, K, W, ratio)


def _small_inputs(seed, B, H, G, Q, NB, lens, integer=False):
    g = torch.Generator().manual_seed(seed)
    if integer:
        q = torch.randint(-3, 4, (B, H, G, Q, 128), generator=g).to(torch.bfloat16)
        k = torch.randint(-4, 5, (B, H, NB, 16, 128), generator=g).to(torch.bfloat16)
    else:
        q = torch.randn((B, H, G, Q, 128), generator=g).to(torch.bfloat16)
        k = torch.randn((B, H, NB, 16, 128), generator=g).to(torch.bfloat16)
    v = torch.randn((B, H, NB, 16, 128), generator=g).to(torch.bfloat16)
    return q, k, v, torch.tensor(lens, dtype=torch.int32)


# ---------------------------------------------------------------------------
# S0 summaries and S1 scores
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("B,H,G,Q,NB,lens", [
    (1, 2, 4, 4, 256, [4096]),
    (3, 2, 1, 1, 37, [592, 1, 300]),            # ragged tail, single-token sequence
    (2, 1, 16, 8, 70, [1100, 17]),              # 128 query rows
    (2, 3, 16, 5, 129, [2064, 2049]),           # 80 query rows, partial last tile
])
def test_summaries_and_scores(lib, B, H, G, Q, NB, lens):
    _say(f"summaries+scores B={B} H={H} G={G} Q={Q} NB={NB} lens={lens}")
    q, k, v, L = _small_inputs(11 + NB, B, H, G, Q, NB, lens)
    W = 64
    d = _dims(lib, B, H, G, NB, Q, min(8, NB), W, 0.05)
    summ = lib.build_summaries(d, k.to(DEV), L.to(DEV))
    scores = lib.score_summaries(d, q.to(DEV), summ, L.to(DEV))
    torch.cuda.synchronize()
    ref_summ = ref.build_summaries(f64(k), L.numpy())
    np.testing.assert_array_equal(f64(summ), ref_summ)
    ref_s = ref.score_blocks(f64(q), ref_summ, L.numpy(), W)
    check_scores(f64(scores), ref_s, score_floor(f64(q), ref_summ), "scores")


# ---------------------------------------------------------------------------
# S2 top-K and S3 plan on given fp32 scores: decisions in the same precision, bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("NB,K,lens,distinct,levels", [
    (2048, 128, [32768, 32768 - 77, 900, 100], True, 0),
    (2048, 128, [32768, 5000], False, 7),        # large groups of exact ties
    (2048, 128, [32768, 20000], False, 512),     # small tie groups in every digit
    (4096, 256, [65536, 4000], False, 1500),
    (8192, 128, [131072], True, 0),
    (8192, 128, [131072, 70000], False, 3000),
    (32768, 1024, [524288, 300000], True, 0),    # largest supported NB and K
    (300, 1, [4800, 16], True, 0),               # K = 1; a sequence with no candidate
    (40, 40, [640, 200], False, 7),              # K = NB
])
def test_topk_on_given_scores(lib, NB, K, lens, distinct, levels):
    _say(f"topk NB={NB} K={K} lens={lens} distinct={distinct} levels={levels}")
    B, H, W = len(lens), 3, 128
    scores = synth.random_scores((B, H, NB), seed=NB + K, distinct=distinct, levels=levels)
    L = torch.tensor(lens, dtype=torch.int32)
    d = _dims(lib, B, H, 4, NB, 5, K, W, 0.05)
    got = lib.topk_blocks(d, scores.to(DEV), L.to(DEV))
    torch.cuda.synchronize()
    expect = ref.topk_blocks(scores.numpy(), L.numpy(), K, W)
    np.testing.assert_array_equal(i64(got), expect)


@pytest.mark.parametrize("cap_ratio", [0.0, 1 / 128, 4 / 128, 0.05, 1.0])
@pytest.mark.parametrize("distinct", [True, False])
def test_plan_on_given_scores(lib, cap_ratio, distinct):
    B, H, NB, K, W = 3, 4, 2048, 128, 128
    lens = [32768, 20000 + 5, 3000]
    _say(f"plan ratio={cap_ratio} distinct={distinct}")
    scores = synth.random_scores((B, H, NB), seed=7, distinct=distinct)
    L = torch.tensor(lens, dtype=torch.int32)
    sel = ref.topk_blocks(scores.numpy(), L.numpy(), K, W)
    res = torch.empty((B, H, K), dtype=torch.int32)
    for b in range(B):
        n_cand = ref.first_window_block(lens[b], W)
        for h in range(H):
            n_empty = [0, 5, K // 2, K][h]
            r = synth.random_resident(K, n_cand, n_empty, seed=100 * b + h).numpy()
            if h == 1:  # mostly the selection, a few strangers, five empty slots
                rng = np.random.default_rng(b)
                s = sel[b, h][sel[b, h] >= 0]
                keep = s[: K - n_empty - 10]
                others = rng.choice(np.setdiff1d(np.arange(n_cand), s), K - n_empty - keep.size,
                                    replace=False)
                r = np.concatenate([keep, others, -np.ones(n_empty, dtype=np.int64)])
                rng.shuffle(r)
            res[b, h] = torch.from_numpy(r.astype(np.int32))
    d = _dims(lib, B, H, 4, NB, 5, K, W, cap_ratio)
    cap = lib.fetch_cap(d)
    assert cap == ref.fetch_cap(cap_ratio, K)
    res_dev = res.to(DEV)
    out = lib.build_plan(d, scores.to(DEV), torch.from_numpy(sel.astype(np.int32)).to(DEV), L.to(DEV), res_dev)
    torch.cuda.synchronize()
    expect = ref.build_plan(scores.numpy(), sel, res.numpy(), L.numpy(), cap, W)
    for key in ("plan", "plan_count", "resident", "table", "table_count"):
        np.testing.assert_array_equal(i64(out[key]), expect[key], err_msg=key)


# ---------------------------------------------------------------------------
# S4 attention on given tables
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("G,lens,NB", [(4, [4096, 1000], 256), (1, [77], 5), (16, [2048, 33], 128),
                                       (8, [513, 16], 40)])
def test_attention_on_given_tables(lib, G, lens, NB):
    _say(f"attention G={G} lens={lens} NB={NB}")
    B, H, Q, K, W = len(lens), 2, 2, min(16, NB), 64
    q, k, v, L = _small_inputs(5 + G, B, H, G, Q, NB, lens)
    d = _dims(lib, B, H, G, NB, Q, K, W, 0.05)
    T = lib.table_stride(d)
    rng = np.random.default_rng(G)
    table = np.full((B, H, T), -1, dtype=np.int64)
    tc = np.zeros((B, H), dtype=np.int64)
    for b in range(B):
        nb = ref.num_blocks(lens[b])
        for h in range(H):
            n = [min(T, nb), min(3, nb), 0][(b + h) % 3] if (b, h) != (0, 0) else min(T, nb)
            ids = rng.choice(nb, size=n, replace=False) if n else np.array([], dtype=np.int64)
            if n and (b, h) == (0, 0) and nb - 1 not in ids:
                ids[0] = nb - 1        # the partial last block
            table[b, h, :n] = ids
            tc[b, h] = n
    scale = default_scale()
    out, lse = lib.sparse_decode_attn(d, q.to(DEV), k.to(DEV), v.to(DEV),
                                      torch.from_numpy(table.astype(np.int32)).to(DEV),
                                      torch.from_numpy(tc.astype(np.int32)).to(DEV), L.to(DEV), scale)
    torch.cuda.synchronize()
    eo, el = ref.sparse_attention(f64(q), f64(k), f64(v), table, tc, L.numpy(), scale)
    np.testing.assert_allclose(f64(out), eo, rtol=0, atol=OUT_ATOL)
    fin = np.isfinite(el)
    assert np.array_equal(np.isneginf(f64(lse)), ~fin)
    np.testing.assert_allclose(f64(lse)[fin], el[fin], rtol=0, atol=OUT_ATOL)


@pytest.mark.parametrize("B,H,G,K,nsplit", [(2, 3, 1, 56, 16), (2, 3, 3, 52, 15), (2, 3, 2, 60, 17),
                                             (2, 4, 4, 56, 16), (1, 8, 8, 56, 16), (2, 4, 16, 56, 16),
                                             (2, 4, 16, 60, 17)])
def test_attention_merge_forms(lib, B, H, G, K, nsplit):
    """The merge's two forms on either side of 16 splits per head: one wave per query head
    (query-head counts that do not fill the last workgroup, KV heads placed by XCD or in
    order) and one workgroup per query head; full, short and empty tables."""
    _say(f"attention merge B={B} H={H} G={G} K={K}")
    NB, W, Q = 128, 64, 2
    lens = [2048, 1500][:B]
    q, k, v, L = _small_inputs(40 + G + K, B, H, G, Q, NB, lens)
    d = _dims(lib, B, H, G, NB, Q, K, W, 0.05)
    T = lib.table_stride(d)
    assert (T + 3) // 4 == nsplit           # one 16-token unit per wave, four waves per split
    rng = np.random.default_rng(K * 100 + G)
    table = np.full((B, H, T), -1, dtype=np.int64)
    tc = np.zeros((B, H), dtype=np.int64)
    for b in range(B):
        nb = ref.num_blocks(lens[b])
        for h in range(H):
            n = [min(T, nb), min(T, nb), min(5, nb), 0][(b * H + h) % 4]
            table[b, h, :n] = rng.choice(nb, size=n, replace=False)
            tc[b, h] = n
    scale = default_scale()
    out, lse = lib.sparse_decode_attn(d, q.to(DEV), k.to(DEV), v.to(DEV),
                                      torch.from_numpy(table.astype(np.int32)).to(DEV),
                                      torch.from_numpy(tc.astype(np.int32)).to(DEV), L.to(DEV), scale)
    torch.cuda.synchronize()
    eo, el = ref.sparse_attention(f64(q), f64(k), f64(v), table, tc, L.numpy(), scale)
    np.testing.assert_allclose(f64(out), eo, rtol=0, atol=OUT_ATOL)
    fin = np.isfinite(el)
    assert np.array_equal(np.isneginf(f64(lse)), ~fin)
    np.testing.assert_allclose(f64(lse)[fin], el[fin], rtol=0, atol=OUT_ATOL)
    # The merge adds fp32 partials: a dropped, doubled or misweighted split, or a query
    # head's record taken for another's, moves the output far more than this.
    assert np.abs(f64(out) - eo).max() <= 1e-4
    assert np.abs(f64(lse)[fin] - el[fin]).max() <= 1e-4


def test_attention_all_blocks_matches_dense(lib):
    """Table = every block: the sparse path reduces to dense decode attention."""
    B, H, G, Q, NB = 2, 2, 4, 1, 64
    lens = [1024, 1000]
    q, k, v, L = _small_inputs(3, B, H, G, Q, NB, lens)
    d = _dims(lib, B, H, G, NB, Q, 8, 0, 0.05)
    T = NB
    table = torch.arange(NB, dtype=torch.int32).repeat(B, H, 1)
    tc = torch.tensor([[ref.num_blocks(x)] * H for x in lens], dtype=torch.int32)
    out, _ = lib.sparse_decode_attn(d, q.to(DEV), k.to(DEV), v.to(DEV), table.to(DEV), tc.to(DEV),
                                    L.to(DEV), default_scale())
    torch.cuda.synchronize()
    for b in range(B):
        kk = k[b].float().reshape(H, NB * 16, 128)[:, : lens[b]].double()
        vv = v[b].float().reshape(H, NB * 16, 128)[:, : lens[b]].double()
        qq = q[b, :, :, 0].double()
        dense = torch.nn.functional.scaled_dot_product_attention(
            qq[:, :, None], kk[:, None].expand(H, G, -1, -1), vv[:, None].expand(H, G, -1, -1),
            scale=default_scale())[:, :, 0]
        np.testing.assert_allclose(f64(out[b]), dense.numpy(), rtol=0, atol=OUT_ATOL)
    assert T == NB


# ---------------------------------------------------------------------------
# The fused step
# ---------------------------------------------------------------------------

def _run_step(lib, w, inp_dev, resident_cpu, into_next=False):
    d = lib.dims_for(w)
    summ = lib.build_summaries(d, inp_dev["k"], inp_dev["seq_lens"])
    res_dev = resident_cpu.to(DEV)
    out = lib.decode_step(d, inp_dev["q"], summ, inp_dev["k"], inp_dev["v"], inp_dev["seq_lens"],
                          res_dev, default_scale(),
                          resident_next=torch.empty_like(res_dev) if into_next else None)
    torch.cuda.synchronize()
    return {key: val.detach().cpu() for key, val in out.items()}, summ


PLAN_KEYS = ("topk", "plan", "plan_count", "resident", "table", "table_count")


def _plan_valid(got, exp, b, h, resident_row, cap, tol):
    """The GPU's plan for one head obeys the capped-eviction rule up to near-ties
    (score differences within ``tol``) in the oracle's scores."""
    s = exp["scores"]
    S = [int(x) for x in i64(got["topk"][b, h]) if x >= 0]
    R = [int(x) for x in resident_row]
    Rset = set(x for x in R if x >= 0)
    new = [x for x in S if x not in Rset]
    n = int(got["plan_count"][b, h])
    assert n == min(cap, len(new))
    plan = i64(got["plan"][b, h])[:n]
    admitted = [int(r[1]) for r in plan]
    assert set(admitted) <= set(new)
    for a in admitted:
        for o in set(new) - set(admitted):
            assert s[a] >= s[o] - tol
    slots = [int(r[0]) for r in plan]
    assert slots == sorted(slots) and admitted == sorted(admitted)
    n_empty = sum(1 for x in R if x < 0)
    evicted = [R[i] for i in slots if R[i] >= 0]
    assert len(evicted) == max(0, n - n_empty)
    kept_stale = [x for i, x in enumerate(R) if x >= 0 and x not in set(S) and i not in slots]
    for e in evicted:
        assert e not in set(S)
        for k in kept_stale:
            assert s[e] <= s[k] + tol
    Rn = list(R)
    for r in plan:
        assert int(r[2]) == R[int(r[0])]
        Rn[int(r[0])] = int(r[1])
    assert Rn == [int(x) for x in i64(got["resident"][b, h])]


def _compare_head(w, got, exp, b, h, resident_row, robust: bool) -> bool:
    """Scores within tolerance and the selection equal up to near-ties, always.  If the
    GPU's selection, plan and table equal the oracle's, the attention output is
    compared too (returns True); otherwise the head must have a near-tie in a
    deciding comparison, its plan must still obey the rule, and its attention must
    equal the oracle's over the GPU's own table (returns False)."""
    floor = score_floor(exp["q64"][None, None], exp["summ"][None, None])[0, 0]
    check_scores(f64(got["scores"][b, h]), exp["scores"], floor, f"scores b={b} h={h}")
    gsel, esel = i64(got["topk"][b, h]), exp["topk"]
    assert selection_equivalent(gsel, esel, exp["scores"]), f"selection b={b} h={h}"
    same = all(np.array_equal(i64(got[key][b, h]), exp[key]) for key in PLAN_KEYS)
    if not same:
        assert not robust, f"b={b} h={h}: the plan differs although no decision is a near-tie"
        fin = exp["scores"][np.isfinite(exp["scores"])]
        _plan_valid(got, exp, b, h, resident_row, w.cap, 1e-5 * float(np.abs(fin).max()))
        qh, kh, vh, L, block = exp["head_inputs"]
        eo, el = ref.sparse_attention(qh, kh, vh, i64(got["table"][b, h])[None, None],
                                      i64(got["table_count"][b, h]).reshape(1, 1), L,
                                      default_scale(), block)
        np.testing.assert_allclose(f64(got["out"][b, h]), eo[0, 0], rtol=0, atol=OUT_ATOL)
        np.testing.assert_allclose(f64(got["lse"][b, h]), el[0, 0], rtol=0, atol=OUT_ATOL)
        return False
    np.testing.assert_allclose(f64(got["out"][b, h]), exp["out"], rtol=0, atol=OUT_ATOL)
    fin = np.isfinite(exp["lse"])
    np.testing.assert_allclose(f64(got["lse"][b, h])[fin], exp["lse"][fin], rtol=0, atol=OUT_ATOL)
    return True


def test_decode_step_tiny_workload(lib):
    w = synth.WORKLOADS["tiny_4k"]
    _say(f"decode_step {w.name}")
    inp = synth.generate(w, "cpu")
    lens = inp["seq_lens"]
    sel = np.stack([np.stack([oracle_selection_head(inp["q"], inp["k"], lens, w.top_k, w.window, b, h)
                              for h in range(w.num_kv_heads)]) for b in range(w.batch)])
    resident = synth.resident_from_selection(w, torch.from_numpy(sel), lens)
    got, _ = _run_step(lib, w, {k: v.to(DEV) for k, v in inp.items()}, resident)
    for b in range(w.batch):
        for h in range(w.num_kv_heads):
            exp = oracle_head(inp["q"], inp["k"], inp["v"], lens, resident[b, h].numpy(), w.top_k,
                              w.window, w.cap, default_scale(), b, h)
            exp["q64"] = f64(inp["q"][b, h])
            assert _compare_head(w, got, exp, b, h, resident[b, h].numpy(), robust=True)


@pytest.mark.parametrize("into_next", [False, True])
@pytest.mark.parametrize("ratio,W,lens", [(0.05, 64, [4096, 1000, 70]), (0.25, 0, [4096, 1024, 16]),
                                          (1.0, 128, [4000, 2222, 130])])
def test_decode_step_integer_inputs(lib, ratio, W, lens, into_next):
    """Small-integer q and k make every score exact in fp32 and fp64, so every
    selection and plan decision (exact ties included) must agree bit for bit.  In
    place and into resident_next (at cap 1 the form that redoes the touched splits)."""
    _say(f"decode_step integer ratio={ratio} W={W} lens={lens} into_next={into_next}")
    B, H, G, Q, NB, K = len(lens), 3, 4, 5, 256, 24
    q, k, v, L = _small_inputs(21, B, H, G, Q, NB, lens, integer=True)
    w = synth.Workload(name="int", batch=B, num_kv_heads=H, group=G, ctx=NB * 16, num_drafts=Q - 1,
                       top_k=K, window=W, fetch_ratio=ratio, planted=0)
    resident = torch.empty((B, H, K), dtype=torch.int32)
    for b in range(B):
        for h in range(H):
            resident[b, h] = synth.random_resident(K, ref.first_window_block(lens[b], W), [0, 3, K][h], 50 * b + h)
    inp_dev = {"q": q.to(DEV), "k": k.to(DEV), "v": v.to(DEV), "seq_lens": L.to(DEV)}
    got, _ = _run_step(lib, w, inp_dev, resident, into_next)
    for b in range(B):
        for h in range(H):
            exp = oracle_head(q, k, v, L, resident[b, h].numpy(), K, W, w.cap, default_scale(), b, h)
            exp["q64"] = f64(q[b, h])
            np.testing.assert_array_equal(f64(got["scores"][b, h]), exp["scores"])
            assert _compare_head(w, got, exp, b, h, resident[b, h].numpy(), robust=True)


@pytest.mark.parametrize("NB,ratio", [(100, 0.25), (300, 0.05), (1000, 1.0)])
def test_decode_step_many_heads(lib, NB, ratio):
    """128 (sequence, KV head) pairs: the selection runs in 256-thread workgroups
    (1, 2 and 4 scores per thread); integer inputs, so every decision must agree
    with the oracle bit for bit."""
    B, H, G, Q, K, W = 32, 4, 2, 3, 24, 32
    lens = [int(x) for x in np.random.default_rng(NB).integers(1, NB * 16 + 1, size=B)]
    _say(f"decode_step many heads NB={NB} ratio={ratio}")
    q, k, v, L = _small_inputs(23, B, H, G, Q, NB, lens, integer=True)
    w = synth.Workload(name="many", batch=B, num_kv_heads=H, group=G, ctx=NB * 16, num_drafts=Q - 1,
                       top_k=K, window=W, fetch_ratio=ratio, planted=0)
    resident = torch.empty((B, H, K), dtype=torch.int32)
    for b in range(B):
        for h in range(H):
            resident[b, h] = synth.random_resident(K, ref.first_window_block(lens[b], W), h, 7 * b + h)
    inp_dev = {"q": q.to(DEV), "k": k.to(DEV), "v": v.to(DEV), "seq_lens": L.to(DEV)}
    got, _ = _run_step(lib, w, inp_dev, resident)
    for b in range(B):
        for h in range(H):
            exp = oracle_head(q, k, v, L, resident[b, h].numpy(), K, W, w.cap, default_scale(), b, h)
            exp["q64"] = f64(q[b, h])
            np.testing.assert_array_equal(f64(got["scores"][b, h]), exp["scores"])
            assert _compare_head(w, got, exp, b, h, resident[b, h].numpy(), robust=True)


def test_decode_step_deterministic(lib):
    w = synth.WORKLOADS["tiny_4k"].with_(batch=2, fetch_ratio=0.25)
    inp = {k: v.to(DEV) for k, v in synth.generate(w, "cpu").items()}
    resident = synth.random_resident(w.top_k, 200, 2, 9).repeat(w.batch, w.num_kv_heads, 1)
    a, _ = _run_step(lib, w, inp, resident)
    b, _ = _run_step(lib, w, inp, resident)
    for key in a:
        assert torch.equal(a[key], b[key]), key


# ---------------------------------------------------------------------------
# Full-size workloads, sampled heads, in the benchmark's launch configuration
# ---------------------------------------------------------------------------

def _sample_heads(w, n=6):
    rng = np.random.default_rng(1234)
    heads = list(dict.fromkeys([(0, 0), (w.batch - 1, w.num_kv_heads - 1)]))
    n = min(n, w.batch * w.num_kv_heads)
    while len(heads) < n:
        heads.append((int(rng.integers(w.batch)), int(rng.integers(w.num_kv_heads))))
        heads = list(dict.fromkeys(heads))
    return heads


def _full_size_case(lib, w, layer=0):
    _say(f"full-size {w.name} layer={layer}: generating")
    inp = synth.generate(w, DEV, layer=layer)
    d = lib.dims_for(w)
    summ = lib.build_summaries(d, inp["k"], inp["seq_lens"])
    lens = inp["seq_lens"].cpu()
    # Resident sets: the GPU's own selection for every head (as the benchmark builds
    # them), then the oracle's for the sampled heads, which are the ones compared.
    q_sel = inp["q_prev"] if w.resident == "prev" else inp["q"]
    sc = lib.score_summaries(d, q_sel, summ, inp["seq_lens"])
    sel = lib.topk_blocks(d, sc, inp["seq_lens"])
    resident = synth.resident_from_selection(w, sel, lens, layer=layer)
    heads = _sample_heads(w)
    cpu = {}
    for (b, h) in heads:
        for key in ("q", "k", "v"):
            cpu.setdefault(key, {})[(b, h)] = inp[key][b:b + 1, h:h + 1].cpu()
        if w.resident == "prev":
            cpu.setdefault("q_prev", {})[(b, h)] = inp["q_prev"][b:b + 1, h:h + 1].cpu()
        qs = cpu["q_prev" if w.resident == "prev" else "q"][(b, h)]
        osel = oracle_selection_head(qs, cpu["k"][(b, h)], lens[b:b + 1], w.top_k, w.window, 0, 0,
                                     w.block)
        n_cand = ref.first_window_block(int(lens[b]), w.window, w.block)
        resident[b, h] = torch.from_numpy(synth.resident_for_head(w, osel, n_cand, b, h, layer).astype(np.int32))
    _say(f"full-size {w.name} layer={layer}: decode_step")
    res_dev = resident.to(DEV)
    out = lib.decode_step(d, inp["q"], summ, inp["k"], inp["v"], inp["seq_lens"], res_dev, default_scale())
    torch.cuda.synchronize()
    got = {key: val.detach().cpu() for key, val in out.items()}
    # summaries of the sampled heads are checked bit-exactly too
    n_exact = 0
    for (b, h) in heads:
        _say(f"full-size {w.name} layer={layer}: oracle b={b} h={h}")
        exp = oracle_head(cpu["q"][(b, h)], cpu["k"][(b, h)], cpu["v"][(b, h)], lens[b:b + 1],
                          resident[b, h].numpy(), w.top_k, w.window, w.cap, default_scale(), 0, 0,
                          w.block)
        np.testing.assert_array_equal(f64(summ[b, h]), exp["summ"])
        exp["q64"] = f64(cpu["q"][(b, h)][0, 0])
        robust = plan_robust(exp["scores"], exp["topk"], resident[b, h].numpy(), w.cap,
                             ref.first_window_block(int(lens[b]), w.window, w.block))
        n_exact += _compare_head(w, got, exp, b, h, resident[b, h].numpy(), robust)
        # whatever the robustness, the GPU's own outputs must be self-consistent
        tc = int(got["table_count"][b, h])
        assert int(got["plan_count"][b, h]) <= w.cap
        w0 = ref.first_window_block(int(lens[b]), w.window, w.block)
        rb = got["resident"][b, h]
        assert tc == int(((rb >= 0) & (rb < w0)).sum()) + ref.num_blocks(int(lens[b]), w.block) - w0
        assert torch.isfinite(got["out"][b, h]).all()
    # fp32 scoring error (~1e-7 relative) is far below the 1e-5 tolerance, so nearly
    # every sampled head must reproduce the oracle's plan and table exactly
    assert n_exact >= len(heads) - 1, f"only {n_exact} of {len(heads)} sampled heads matched exactly"
    # The overlapped step on the same inputs (the benchmark's configuration): the same
    # plan outputs, and attention over the slot table as it was before the plan.
    _say(f"full-size {w.name} layer={layer}: overlapped step")
    res0 = resident.to(DEV)
    rn = torch.empty_like(res0)
    ov = lib.decode_step_overlapped(d, inp["q"], summ, inp["k"], inp["v"], inp["seq_lens"], res0, rn,
                                    default_scale())
    torch.cuda.synchronize()
    for key in ("scores", "topk", "plan", "plan_count", "table", "table_count"):
        assert torch.equal(ov[key].cpu(), got[key]), key
    assert torch.equal(rn.cpu(), got["resident"])
    for (b, h) in heads:
        lb = lens[b:b + 1].numpy()
        table, tc = ref.resident_table(i64(resident[b:b + 1, h:h + 1]), lb, w.window, w.block)
        eo, el = ref.sparse_attention(f64(cpu["q"][(b, h)]), f64(cpu["k"][(b, h)]),
                                      f64(cpu["v"][(b, h)]), table, tc, lb, default_scale(), w.block)
        np.testing.assert_allclose(f64(ov["out"][b, h].cpu()), eo[0, 0], rtol=0, atol=OUT_ATOL)
        np.testing.assert_allclose(f64(ov["lse"][b, h].cpu()), el[0, 0], rtol=0, atol=OUT_ATOL)
    # The serial step with its own resident_next (where it applies, the overlapped launch
    # 1 plus the touched splits redone): the same plan outputs, and on every head the
    # attention of the in-place step up to the order of the fp32 additions (its splits
    # cut the same tokens differently); a split redone over the wrong slots would move
    # the output by about a block's share of the softmax mass, far above 1e-4.
    _say(f"full-size {w.name} layer={layer}: serial step into resident_next "
         f"(touched splits redone: {lib.decode_step_redoes_touched_splits(d)})")
    rn2 = torch.empty_like(res0)
    s2 = lib.decode_step(d, inp["q"], summ, inp["k"], inp["v"], inp["seq_lens"], resident.to(DEV),
                         default_scale(), resident_next=rn2)
    torch.cuda.synchronize()
    for key in ("scores", "topk", "plan", "plan_count", "table", "table_count"):
        assert torch.equal(s2[key].cpu(), got[key]), key
    assert torch.equal(rn2.cpu(), got["resident"])
    np.testing.assert_allclose(f64(s2["out"].cpu()), f64(got["out"]), rtol=0, atol=1e-4)
    np.testing.assert_allclose(f64(s2["lse"].cpu()), f64(got["lse"]), rtol=0, atol=1e-4)
    del inp, summ, out, ov, s2
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["qwen3_8b_32k", "long_128k", "qwen3_235b_32k"])
def test_full_size_workload(lib, name):
    _full_size_case(lib, synth.WORKLOADS[name])


def _zero_scale_check(w, v, lens, table, table_count, out, lse, where):
    """With scale 0 every attended token weighs the same: exp(lse) is the number of
    tokens of the head's table below the length, and out is the mean of their V rows
    (fp64 on the device).  Every head is checked."""
    bs = w.block
    for b in range(w.batch):
        L = int(lens[b])
        for h in range(w.num_kv_heads):
            blocks = [int(x) for x in table[b, h, : int(table_count[b, h])]]
            count = sum(min(bs, L - bs * j) for j in blocks if 0 <= j and bs * j < L)
            got_n = np.exp(f64(lse[b, h]))
            assert np.all(np.abs(got_n - count) <= 1e-6 * count), f"{where} b={b} h={h}: exp(lse) {got_n} vs {count}"
            idx = torch.tensor(blocks, dtype=torch.int64, device=v.device)
            vb = v[b, h].index_select(0, idx).to(torch.float64)               # [n, bs, 128]
            tok = torch.arange(bs, device=v.device)[None, :] + bs * idx[:, None]
            mean = (vb * (tok < L)[:, :, None]).sum(dim=(0, 1)) / count
            err = (out[b, h].to(v.device).to(torch.float64) - mean[None, :]).abs().max().item()
            assert err <= 1e-5, f"{where} b={b} h={h}: out differs from the mean of V by {err:.3g}"


@pytest.mark.parametrize("name,layer", [("qwen3_235b_32k", 0), ("reasoning_36l", 17), ("qwen3_8b_32k", 0)])
def test_full_size_zero_scale_every_head(lib, name, layer):
    """At full size, in the benchmark's launch configuration (Qwen3-235B: eight-round
    attention splits; 36 layers: four rounds), both step orders with scale 0 (the serial
    one in place and into resident_next, at Qwen3-8B the form that redoes the touched
    splits), on every head: the merged log-sum-exp counts the attended tokens exactly and the output is
    the mean of their V rows.  A dropped or doubled token moves exp(lse) by one count
    (above 1e-6 relative up to a million tokens) and the output by about 1/count."""
    w = synth.WORKLOADS[name]
    _say(f"zero-scale full size {name} layer={layer}: generating")
    inp = synth.generate(w, DEV, layer=layer)
    d = lib.dims_for(w)
    summ = lib.build_summaries(d, inp["k"], inp["seq_lens"])
    sel = lib.topk_blocks(d, lib.score_summaries(d, inp["q"], summ, inp["seq_lens"]), inp["seq_lens"])
    lens = inp["seq_lens"].cpu().numpy()
    resident = synth.resident_from_selection(w, sel, torch.from_numpy(lens), layer=layer).to(DEV)
    res_cpu = i64(resident)
    _say(f"zero-scale full size {name}: serial step")
    ser = lib.decode_step(d, inp["q"], summ, inp["k"], inp["v"], inp["seq_lens"], resident.clone(), 0.0)
    ser = {key: val.detach().cpu() for key, val in ser.items()}
    _zero_scale_check(w, inp["v"], lens, i64(ser["table"]), i64(ser["table_count"]), ser["out"], ser["lse"],
                      f"{name} serial")
    _say(f"zero-scale full size {name}: serial step into resident_next")
    rn_s = torch.empty_like(resident)
    ser2 = lib.decode_step(d, inp["q"], summ, inp["k"], inp["v"], inp["seq_lens"], resident, 0.0,
                           resident_next=rn_s)
    ser2 = {key: val.detach().cpu() for key, val in ser2.items()}
    assert torch.equal(ser2["table"], ser["table"]) and torch.equal(ser2["table_count"], ser["table_count"])
    _zero_scale_check(w, inp["v"], lens, i64(ser2["table"]), i64(ser2["table_count"]), ser2["out"],
                      ser2["lse"], f"{name} serial into resident_next")
    _say(f"zero-scale full size {name}: overlapped step")
    rn = torch.empty_like(resident)
    ov = lib.decode_step_overlapped(d, inp["q"], summ, inp["k"], inp["v"], inp["seq_lens"], resident, rn, 0.0)
    ov = {key: val.detach().cpu() for key, val in ov.items()}
    table, tc = ref.resident_table(res_cpu, lens, w.window, w.block)
    _zero_scale_check(w, inp["v"], lens, table, tc, ov["out"], ov["lse"], f"{name} overlapped")
    del inp, summ
    torch.cuda.empty_cache()


@pytest.mark.parametrize("top_k,ratio", [(64, 0.05), (192, 0.05), (128, 0.01), (128, 0.02),
                                         (128, 0.10), (128, 0.20), (128, 1.0)])
def test_variant_sweep_shapes(lib, top_k, ratio):
    """The shapes of the K and fetch-ratio sweep (the pages' ablations) at the
    Qwen3-8B 32K shape, two sequences and two KV heads."""
    w = synth.WORKLOADS["qwen3_8b_32k"].with_(batch=2, num_kv_heads=2, top_k=top_k, fetch_ratio=ratio)
    _full_size_case(lib, w)


@pytest.mark.parametrize("layer", [0, 17, 35])
def test_full_size_reasoning_layer(lib, layer):
    _full_size_case(lib, synth.WORKLOADS["reasoning_36l"], layer=layer)


def test_largest_supported_sizes(lib):
    """max_blocks = 32768 (a 512K-token context), K = 1024, a 4096-token window, 16
    query heads and a cap of 512, a ragged last block: both step orders.  Scores are
    checked on sampled blocks (the oracle's product over every block would not fit
    the host), selection, plan and attention on the GPU's own scores and tables."""
    B, H, G, Q, NB, K, W, ratio = 1, 1, 16, 2, 32768, 1024, 4096, 0.5
    L = NB * 16 - 5
    _say("largest sizes: generating")
    g = torch.Generator().manual_seed(77)
    q = torch.randn((B, H, G, Q, 128), generator=g).to(torch.bfloat16)
    k = torch.randn((B, H, NB, 16, 128), generator=g).to(torch.bfloat16)
    v = torch.randn((B, H, NB, 16, 128), generator=g).to(torch.bfloat16)
    lens = torch.tensor([L], dtype=torch.int32)
    d = _dims(lib, B, H, G, NB, Q, K, W, ratio)
    C = lib.fetch_cap(d)
    assert C == 512
    n_cand = ref.first_window_block(L, W)
    res = synth.random_resident(K, n_cand, 100, 5).reshape(1, 1, K)
    qd, kd, vd, ld = q.to(DEV), k.to(DEV), v.to(DEV), lens.to(DEV)
    summ = lib.build_summaries(d, kd, ld)
    _say("largest sizes: serial and overlapped steps")
    ser = lib.decode_step(d, qd, summ, kd, vd, ld, res.to(DEV).clone(), default_scale())
    ser = {key: val.cpu() for key, val in ser.items()}
    rn = torch.empty_like(res).to(DEV)
    ov = lib.decode_step_overlapped(d, qd, summ, kd, vd, ld, res.to(DEV), rn, default_scale())
    ov = {key: val.cpu() for key, val in ov.items()}
    torch.cuda.synchronize()
    # scores of sampled blocks against the oracle on those blocks alone
    rng = np.random.default_rng(3)
    blocks = np.sort(rng.choice(n_cand, size=256, replace=False))
    summ_s = f64(summ[:, :, blocks].cpu())
    exp_s = ref.score_blocks(f64(q), summ_s, np.array([len(blocks) * 16]), 0)
    floor = score_floor(f64(q), summ_s)
    check_scores(f64(ser["scores"][:, :, blocks]), exp_s, floor, "sampled scores")
    np.testing.assert_array_equal(f64(summ[:, :, blocks[:8]].cpu()),
                                  ref.build_summaries(f64(k[:, :, blocks[:8]]),
                                                      np.array([8 * 16]))[:, :, :8])
    # selection and plan on the GPU's own scores (both orders share them)
    sc = f64(ser["scores"])
    np.testing.assert_array_equal(f64(ov["scores"]), sc)
    sel = ref.topk_blocks(sc, lens.numpy(), K, W)
    np.testing.assert_array_equal(i64(ser["topk"]), sel)
    plan = ref.build_plan(sc, sel, i64(res), lens.numpy(), C, W)
    for key in ("plan", "plan_count", "resident", "table", "table_count"):
        np.testing.assert_array_equal(i64(ser[key]), plan[key], err_msg=key)
        np.testing.assert_array_equal(i64(ov[key]), plan[key], err_msg=key)
    assert int(ser["plan_count"][0, 0]) == C
    # attention: serial over the updated table, overlapped over the slot table as it was
    _say("largest sizes: oracle attention")
    qf, kf, vf = f64(q), f64(k), f64(v)
    eo, _ = ref.sparse_attention(qf, kf, vf, plan["table"], plan["table_count"], lens.numpy(),
                                 default_scale())
    np.testing.assert_allclose(f64(ser["out"]), eo, rtol=0, atol=OUT_ATOL)
    table, tc = ref.resident_table(i64(res), lens.numpy(), W)
    eo2, _ = ref.sparse_attention(qf, kf, vf, table, tc, lens.numpy(), default_scale())
    np.testing.assert_allclose(f64(ov["out"]), eo2, rtol=0, atol=OUT_ATOL)


# ---------------------------------------------------------------------------
# Degenerate cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("ratio,into_next", [(1.0, False), (0.25, True)])
def test_no_candidates_and_short_sequences(lib, ratio, into_next):
    """len < W: nothing to score or select; the table is the window alone.  In place,
    and into resident_next at cap 1 (the form that redoes the touched splits, with
    nothing to redo)."""
    B, H, G, Q, NB, K, W = 3, 2, 4, 2, 16, 4, 128
    lens = [100, 1, 128]
    q, k, v, L = _small_inputs(2, B, H, G, Q, NB, lens)
    w = synth.Workload(name="short", batch=B, num_kv_heads=H, group=G, ctx=NB * 16, num_drafts=Q - 1,
                       top_k=K, window=W, fetch_ratio=ratio, planted=0)
    if into_next:
        assert lib.decode_step_redoes_touched_splits(lib.dims_for(w))
    resident = torch.full((B, H, K), -1, dtype=torch.int32)
    got, _ = _run_step(lib, w, {"q": q.to(DEV), "k": k.to(DEV), "v": v.to(DEV), "seq_lens": L.to(DEV)},
                       resident, into_next)
    assert torch.all(got["topk"] == -1) and torch.all(got["plan_count"] == 0)
    for b in range(B):
        for h in range(H):
            exp = oracle_head(q, k, v, L, resident[b, h].numpy(), K, W, w.cap, default_scale(), b, h)
            np.testing.assert_array_equal(i64(got["table"][b, h]), exp["table"])
            np.testing.assert_allclose(f64(got["out"][b, h]), exp["out"], rtol=0, atol=OUT_ATOL)


# ---------------------------------------------------------------------------
# Overlapped (foreground / background) step, resident-slot attention, HIP graphs
# ---------------------------------------------------------------------------

def _prepared_inputs(lib, w, seed_layer=0):
    inp = {k: v.to(DEV) for k, v in synth.generate(w, "cpu", layer=seed_layer).items()}
    d = lib.dims_for(w)
    summ = lib.build_summaries(d, inp["k"], inp["seq_lens"])
    n_cand = [ref.first_window_block(int(x), w.window) for x in inp["seq_lens"].cpu()]
    res = torch.stack([torch.stack([synth.random_resident(w.top_k, n_cand[b], 3, 10 * b + h)
                                    for h in range(w.num_kv_heads)]) for b in range(w.batch)]).to(DEV)
    return d, inp, summ, res


def _step_outputs(bufs, rn):
    return {**{k: v.clone() for k, v in bufs.as_dict().items()}, "resident": rn.clone()}


@pytest.mark.parametrize("shape", [
    {},                                                # 259 blocks, K = 16
    {"group": 8, "num_drafts": 1},                     # 8 query heads per KV head
    {"top_k": 300, "ctx": 8192 + 40},                  # K above 256 (1024-thread selection)
    {"ctx": 2048 * 16 + 40, "min_len": 30000, "top_k": 64},   # 2051 blocks
    {"group": 8, "num_drafts": 4},                     # 40 query rows, 8 query heads
    {"group": 16, "num_drafts": 1},                    # 32 query rows, 16 query heads
    {"group": 4, "num_drafts": 11},                    # 48 query rows, 4 query heads
    {"group": 16, "num_drafts": 4},                    # 80 query rows (Qwen3-235B's 16 x 5)
    {"group": 16, "num_drafts": 5},                    # 96 query rows: the fused launch's widest
    {"group": 16, "num_drafts": 6},                    # 112 query rows: scoring in its own kernel
])
def test_overlapped_step_matches_its_parts(lib, shape):
    """The overlapped step is the serial step's background half plus the attention
    over the current slot table: its plan outputs equal the serial step's bit for
    bit, its attention equals oasis_sparse_decode_attn_resident's up to the order of
    the merge's additions, and the attention matches the oracle's over the
    resident table.  Shapes on both sides of the fused kernels' limits."""
    base = dict(batch=5, num_kv_heads=3, fetch_ratio=0.25, ctx=4096 + 40, min_len=1000)
    w = synth.WORKLOADS["tiny_4k"].with_(**{**base, **shape})
    _say(f"overlapped step vs its parts {shape}")
    d, inp, summ, res = _prepared_inputs(lib, w)
    scale = default_scale()
    serial_bufs, over_bufs = lib.StepBuffers(d, DEV), lib.StepBuffers(d, DEV)
    rn_serial, rn_over = torch.empty_like(res), torch.empty_like(res)
    lib.decode_step(d, inp["q"], summ, inp["k"], inp["v"], inp["seq_lens"], res, scale,
                    buffers=serial_bufs, resident_next=rn_serial)
    lib.decode_step_overlapped(d, inp["q"], summ, inp["k"], inp["v"], inp["seq_lens"], res, rn_over,
                               scale, buffers=over_bufs)
    alone, alone_lse = lib.sparse_decode_attn_resident(d, inp["q"], inp["k"], inp["v"], res,
                                                       inp["seq_lens"], scale)
    torch.cuda.synchronize()
    a, o = _step_outputs(serial_bufs, rn_serial), _step_outputs(over_bufs, rn_over)
    for key in ("scores", "topk", "plan", "plan_count", "table", "table_count", "resident"):
        assert torch.equal(a[key], o[key]), key
    # Same split records; the fused merge spreads the splits over more waves, so only
    # the order of the final fp32 additions differs.
    np.testing.assert_allclose(f64(o["out"].cpu()), f64(alone.cpu()), rtol=0, atol=1e-6)
    np.testing.assert_allclose(f64(o["lse"].cpu()), f64(alone_lse.cpu()), rtol=0, atol=1e-6)
    assert not torch.equal(o["out"], a["out"])   # the plan changed the set: a different attention
    lens = inp["seq_lens"].cpu().numpy()
    table, tc = ref.resident_table(i64(res.cpu()), lens, w.window)
    eo, el = ref.sparse_attention(f64(inp["q"].cpu()), f64(inp["k"].cpu()), f64(inp["v"].cpu()),
                                  table, tc, lens, scale)
    np.testing.assert_allclose(f64(o["out"].cpu()), eo, rtol=0, atol=OUT_ATOL)
    np.testing.assert_allclose(f64(o["lse"].cpu()), el, rtol=0, atol=OUT_ATOL)


@pytest.mark.parametrize("shape", [
    {},                                                   # K = 64, cap 4, 18 splits
    {"group": 8, "num_drafts": 1},                        # 8 query heads per KV head
    {"group": 16, "num_drafts": 4},                       # 16 query heads, 80 query rows
    {"fetch_ratio": 0.0},                                 # cap 0: nothing to redo, the merge alone
    {"ctx": 2048, "min_len": 60},                         # rows the window covers, empty slot tables
    {"block": 8}, {"block": 32}, {"block": 64, "top_k": 32},   # a slot in half a unit .. four units
    {"top_k": 128, "fetch_ratio": 0.03, "ctx": 8192 + 40, "batch": 32, "num_kv_heads": 8},  # 256 heads: 4 rounds
    {"workload": "qwen3_8b_32k", "batch": 2, "num_kv_heads": 2},   # 35 splits
])
def test_serial_step_redoes_the_touched_splits(lib, shape):
    """oasis_decode_step with its own resident_next: launch 1 of the overlapped step,
    then only the splits holding a slot that the plan changed, redone over the updated
    slot table, and the merge.  Three steps in a row on one workspace, each: the plan
    outputs equal the oracle's on the step's own scores; the attention equals
    oasis_sparse_decode_attn_resident over the updated slot table bit for bit (the
    same split records, merged by the same kernel: a split left out or redone over
    the wrong slots would differ) and the oracle's attention over the updated table;
    the hand-off region is zero again afterwards."""
    shape = dict(shape)
    base = dict(batch=5, num_kv_heads=3, top_k=64, fetch_ratio=0.0625, ctx=4096 + 40, min_len=1000)
    w = synth.WORKLOADS[shape.pop("workload", "tiny_4k")]
    w = w.with_(**({**base, **shape} if w.name == "tiny_4k" else shape))
    _say(f"serial step redoing the touched splits {shape}")
    inp = {kk: t.to(DEV) for kk, t in synth.generate(w, "cpu").items()}
    d = lib.dims_for(w)
    assert lib.decode_step_redoes_touched_splits(d)
    summ = lib.build_summaries(d, inp["k"], inp["seq_lens"])
    lens = inp["seq_lens"].cpu().numpy()
    n_cand = [ref.first_window_block(int(x), w.window, w.block) for x in lens]
    res = torch.stack([torch.stack([synth.random_resident(w.top_k, n_cand[b], 3, 10 * b + h)
                                    for h in range(w.num_kv_heads)]) for b in range(w.batch)]).to(DEV)
    bufs = lib.StepBuffers(d, DEV)
    attn_need = lib.workspace_bytes(d, lib.table_stride(d))
    scale = default_scale()
    qf, kf, vf = f64(inp["q"]), f64(inp["k"]), f64(inp["v"])
    for step in range(3):
        rn = torch.empty_like(res)
        got = lib.decode_step(d, inp["q"], summ, inp["k"], inp["v"], inp["seq_lens"], res, scale,
                              buffers=bufs, resident_next=rn)
        out, lse = got["out"].clone(), got["lse"].clone()
        alone, alone_lse = lib.sparse_decode_attn_resident(d, inp["q"], inp["k"], inp["v"], rn,
                                                           inp["seq_lens"], scale)
        torch.cuda.synchronize()
        assert lib.workspace_status(d, bufs.ws) == 0
        assert int(torch.count_nonzero(bufs.ws[attn_need:])) == 0, f"step {step}: hand-off region"
        gs = f64(got["scores"])
        sel = ref.topk_blocks(gs, lens, w.top_k, w.window, w.block)
        np.testing.assert_array_equal(i64(got["topk"]), sel)
        pl = ref.build_plan(gs, sel, i64(res), lens, w.cap, w.window, w.block)
        for key in ("plan", "plan_count", "table", "table_count"):
            np.testing.assert_array_equal(i64(got[key]), pl[key], err_msg=key)
        np.testing.assert_array_equal(i64(rn), pl["resident"])
        if w.cap > 0 and step == 0:
            assert int(got["plan_count"].sum()) > 0
        assert torch.equal(out, alone) and torch.equal(lse, alone_lse), f"step {step}"
        eo, el = ref.sparse_attention(qf, kf, vf, pl["table"], pl["table_count"], lens, scale, w.block)
        np.testing.assert_allclose(f64(out), eo, rtol=0, atol=OUT_ATOL)
        np.testing.assert_allclose(f64(lse), el, rtol=0, atol=OUT_ATOL)
        res = rn


def test_overlapped_step_repeated_over_rotating_inputs(lib):
    """Steps queued back to back over rotating input sets, sharing one workspace:
    every step must give its own set's results (the scores handed from the scoring
    workgroups to the selection inside one launch must never be another step's)."""
    w = synth.WORKLOADS["qwen3_8b_32k"].with_(batch=2, num_kv_heads=4)
    _say("overlapped step repeated over rotating inputs")
    n_sets, n_steps = 3, 24
    sets = []
    for i in range(n_sets):
        d, inp, summ, res = _prepared_inputs(lib, w, seed_layer=i)
        bufs = lib.StepBuffers(d, DEV)
        rn = torch.empty_like(res)
        lib.decode_step(d, inp["q"], summ, inp["k"], inp["v"], inp["seq_lens"], res, default_scale(),
                        buffers=bufs, resident_next=rn)
        alone, _ = lib.sparse_decode_attn_resident(d, inp["q"], inp["k"], inp["v"], res,
                                                   inp["seq_lens"], default_scale())
        torch.cuda.synchronize()
        sets.append((d, inp, summ, res, _step_outputs(bufs, rn), alone.clone()))
    shared_ws = lib.StepBuffers(sets[0][0], DEV).ws
    runs = []
    for i in range(n_steps):
        d, inp, summ, res, _, _ = sets[i % n_sets]
        bufs = lib.StepBuffers(d, DEV)
        bufs.ws = shared_ws
        rn = torch.empty_like(res)
        lib.decode_step_overlapped(d, inp["q"], summ, inp["k"], inp["v"], inp["seq_lens"], res, rn,
                                   default_scale(), buffers=bufs)
        runs.append((bufs, rn))
    torch.cuda.synchronize()
    assert lib.workspace_status(sets[0][0], shared_ws) == 0, "a hand-off wait timed out"
    for i, (bufs, rn) in enumerate(runs):
        _, _, _, _, ref_out, alone = sets[i % n_sets]
        got = _step_outputs(bufs, rn)
        for key in ("scores", "topk", "plan", "plan_count", "table", "table_count", "resident"):
            assert torch.equal(got[key], ref_out[key]), f"step {i}: {key}"
        assert (got["out"] - alone).abs().max().item() <= 1e-6, f"step {i}: out"


@pytest.mark.parametrize("G,lens,NB,K", [(4, [4096, 1000, 300], 256, 16), (1, [77, 700], 48, 5),
                                         (16, [2048, 33], 128, 8), (8, [513, 16, 4000], 250, 40)])
def test_attention_over_resident_slots(lib, G, lens, NB, K):
    """Slot tables with empty slots and with blocks that the window has reached."""
    _say(f"attention resident G={G} lens={lens} NB={NB} K={K}")
    B, H, Q, W = len(lens), 3, 2, 64
    q, k, v, L = _small_inputs(40 + G, B, H, G, Q, NB, lens)
    d = _dims(lib, B, H, G, NB, Q, K, W, 0.05)
    rng = np.random.default_rng(G + K)
    R = np.full((B, H, K), -1, dtype=np.int64)
    for b in range(B):
        nb = ref.num_blocks(lens[b])
        for h in range(H):
            n = min(K - h, nb)                         # h empty slots (at least)
            R[b, h, :n] = rng.choice(nb, size=n, replace=False)   # window blocks included
            rng.shuffle(R[b, h])
    scale = default_scale()
    out, lse = lib.sparse_decode_attn_resident(d, q.to(DEV), k.to(DEV), v.to(DEV),
                                               torch.from_numpy(R.astype(np.int32)).to(DEV),
                                               L.to(DEV), scale)
    torch.cuda.synchronize()
    table, tc = ref.resident_table(R, L.numpy(), W)
    eo, el = ref.sparse_attention(f64(q), f64(k), f64(v), table, tc, L.numpy(), scale)
    np.testing.assert_allclose(f64(out), eo, rtol=0, atol=OUT_ATOL)
    fin = np.isfinite(el)
    assert np.array_equal(np.isneginf(f64(lse)), ~fin)
    np.testing.assert_allclose(f64(lse)[fin], el[fin], rtol=0, atol=OUT_ATOL)


@pytest.mark.parametrize("into_next", [False, True])
@pytest.mark.parametrize("ratio", [0.0, 0.125, 0.25, 1.0])
def test_serial_step_with_window_reached_slots(lib, ratio, into_next):
    """oasis_decode_step over slot tables that hold blocks the window has reached, empty
    slots and historical blocks: the plan, the updated slots and the table equal the
    oracle's given the GPU's own scores and selection (a window-reached block is listed
    once, as a window block), and the attention equals the oracle's over the GPU's table.
    In place and into resident_next (at caps 0 and 1 the form that redoes the touched
    splits: a plan row may replace a slot whose block the window has reached)."""
    _say(f"serial step, window-reached slots, ratio={ratio}, into_next={into_next}")
    B, H, G, Q, NB, K, W = 3, 2, 4, 5, 64, 12, 64
    lens = [1000, 700, 300]
    q, k, v, L = _small_inputs(77, B, H, G, Q, NB, lens)
    d = _dims(lib, B, H, G, NB, Q, K, W, ratio)
    cap = ref.fetch_cap(ratio, K)
    rng = np.random.default_rng(17)
    R = np.full((B, H, K), -1, dtype=np.int64)
    for b in range(B):
        nb, w0 = ref.num_blocks(lens[b]), ref.first_window_block(lens[b], W)
        for h in range(H):
            win = list(range(w0, nb))[: 2 + h]                     # blocks the window has reached
            hist = rng.choice(w0, size=K - len(win) - 2, replace=False).tolist()
            row = np.array(win + hist + [-1, -1])
            rng.shuffle(row)
            R[b, h] = row
    R_dev = torch.from_numpy(R.astype(np.int32)).to(DEV)
    rn = torch.empty_like(R_dev) if into_next else None
    if into_next:
        assert lib.decode_step_redoes_touched_splits(d) == (cap <= 1)
    got = lib.decode_step(d, q.to(DEV), lib.build_summaries(d, k.to(DEV), L.to(DEV)), k.to(DEV),
                          v.to(DEV), L.to(DEV), R_dev, default_scale(), resident_next=rn)
    torch.cuda.synchronize()
    got = {key: val.detach().cpu() for key, val in got.items()}
    summ = ref.build_summaries(f64(k), L.numpy())
    check_scores(f64(got["scores"]), ref.score_blocks(f64(q), summ, L.numpy(), W),
                 score_floor(f64(q), summ), "scores")
    gs = f64(got["scores"])
    np.testing.assert_array_equal(i64(got["topk"]), ref.topk_blocks(gs, L.numpy(), K, W))
    exp = ref.build_plan(gs, i64(got["topk"]), R, L.numpy(), cap, W)
    for key in ("plan", "plan_count", "table", "table_count"):
        if key == "plan" and cap == 0:
            continue
        np.testing.assert_array_equal(i64(got[key]), exp[key], err_msg=key)
    np.testing.assert_array_equal(i64(got["resident"]), exp["resident"])
    assert (i64(got["table_count"]) > 0).all()
    eo, el = ref.sparse_attention(f64(q), f64(k), f64(v), i64(got["table"]), i64(got["table_count"]),
                                  L.numpy(), default_scale())
    np.testing.assert_allclose(f64(got["out"]), eo, rtol=0, atol=OUT_ATOL)
    np.testing.assert_allclose(f64(got["lse"]), el, rtol=0, atol=OUT_ATOL)


def test_append_then_step_loop_both_step_orders_agree(lib):
    """A decode loop at cap 0 (the plan never moves a block) over slot tables that hold
    blocks of the local window: each step appends one token, so the window moves on
    and those blocks turn into historical ones.  The serial step (attention over its
    table) and the overlapped step (attention over the slot table) attend the same
    tokens at every step (a block is listed once, as a window block while the window
    covers it), and both equal the oracle."""
    B, H, G, Q, NB, K, W = 2, 2, 4, 3, 40, 8, 32
    lens = [500, 263]
    _say("append-then-step loop, both step orders")
    q, k, v, L = _small_inputs(91, B, H, G, Q, NB, lens)
    d = _dims(lib, B, H, G, NB, Q, K, W, 0.0)
    kd, vd, Ld = k.to(DEV), v.to(DEV), L.to(DEV)
    summ = lib.build_summaries(d, kd, Ld)
    # slot tables holding the first three window blocks and some historical ones
    R = np.full((B, H, K), -1, dtype=np.int64)
    w0_start = [ref.first_window_block(x, W) for x in lens]
    for b in range(B):
        for h in range(H):
            R[b, h, :K - 1] = list(range(w0_start[b], w0_start[b] + 3)) + list(range(h, h + K - 4))
    R_serial = torch.from_numpy(R.astype(np.int32)).to(DEV)
    R_over = R_serial.clone()
    wset = lib.WorkingSet(d, DEV)
    g = torch.Generator().manual_seed(3)
    qd = q.to(DEV)
    reached = 0
    for step in range(40):
        a = lib.decode_step(d, qd, summ, kd, vd, Ld, R_serial, default_scale())
        a = {key: val.clone() for key, val in a.items()}
        rn = torch.empty_like(R_over)
        o = lib.decode_step_overlapped(d, qd, summ, kd, vd, Ld, R_over, rn, default_scale())
        torch.cuda.synchronize()
        assert torch.equal(rn, R_over) and torch.equal(a["resident"], R_serial)   # cap 0: nothing moves
        Lh = Ld.cpu().numpy()
        table, tc = ref.resident_table(i64(R_serial), Lh, W)
        np.testing.assert_array_equal(i64(a["table"]), table, err_msg=f"step {step}: table")
        np.testing.assert_array_equal(i64(a["table_count"]), tc, err_msg=f"step {step}: table_count")
        assert (o["out"] - a["out"]).abs().max().item() <= 1e-5, f"step {step}: out"
        assert (o["lse"] - a["lse"]).abs().max().item() <= 1e-5, f"step {step}: lse"
        if step % 13 == 0 or step == 39:
            eo, el = ref.sparse_attention(f64(qd), f64(kd), f64(vd), table, tc, Lh, default_scale())
            np.testing.assert_allclose(f64(a["out"]), eo, rtol=0, atol=OUT_ATOL)
            np.testing.assert_allclose(f64(a["lse"]), el, rtol=0, atol=OUT_ATOL)
        reached += int(sum(int((i64(R_serial)[b] >= ref.first_window_block(int(Lh[b]), W)).sum())
                           for b in range(B)))
        kn = torch.randn((B, H, 128), generator=g).to(torch.bfloat16).to(DEV)
        vn = torch.randn((B, H, 128), generator=g).to(torch.bfloat16).to(DEV)
        lib.append_token(d, kn, vn, Ld, summ, wset, kd, vd)
        torch.cuda.synchronize()
        Ld += 1
    assert reached > 0, "no resident block lay in the window"
    # the window moved past some of them: they are historical blocks now
    assert any(ref.first_window_block(int(Ld[b]), W) > w0_start[b] for b in range(B))


@pytest.mark.parametrize("shape", ["tiny", "qwen3_8b_2x2", "short", "g16x5"])
def test_overlapped_step_leaves_the_handoff_region_zero(lib, shape):
    """The overlapped step at sizes whose selection runs in launch 1: after every
    step the hand-off region of the workspace (flags, status word, score mailbox) is
    zero again and the status word never records a timed-out wait;
    the step's outputs equal the oracle's, and consecutive steps with different sizes
    share the workspace."""
    if shape == "tiny":
        w = synth.WORKLOADS["tiny_4k"].with_(batch=2, fetch_ratio=0.25)
    elif shape == "qwen3_8b_2x2":
        w = synth.WORKLOADS["qwen3_8b_32k"].with_(batch=2, num_kv_heads=2)
    elif shape == "g16x5":       # 16 query heads x 5 queries: 80 rows, scoring placed by XCD
        w = synth.WORKLOADS["qwen3_235b_32k"].with_(batch=2, num_kv_heads=4, ctx=8192 + 40)
    else:
        w = synth.WORKLOADS["tiny_4k"].with_(batch=3, ctx=1024, min_len=60, fetch_ratio=1.0)
    _say(f"hand-off region, {shape}")
    d = lib.dims_for(w)
    inp = {kk: t.to(DEV) for kk, t in synth.generate(w, "cpu").items()}
    summ = lib.build_summaries(d, inp["k"], inp["seq_lens"])
    sel = lib.topk_blocks(d, lib.score_summaries(d, inp["q"], summ, inp["seq_lens"]), inp["seq_lens"])
    lens = inp["seq_lens"].cpu()
    resident = synth.resident_from_selection(w, sel, lens).to(DEV)
    bufs = lib.StepBuffers(d, DEV)
    attn_need = lib.workspace_bytes(d, lib.table_stride(d))
    for step in range(3):
        rn = torch.empty_like(resident)
        got = lib.decode_step_overlapped(d, inp["q"], summ, inp["k"], inp["v"], inp["seq_lens"], resident, rn,
                                         buffers=bufs)
        torch.cuda.synchronize()
        assert lib.workspace_status(d, bufs.ws) == 0
        tail = bufs.ws[attn_need:]
        assert int(torch.count_nonzero(tail)) == 0, f"step {step}: hand-off region not left zero"
        if step == 0:
            exp = ref.decode_step_overlapped(f64(inp["q"]), f64(summ), f64(inp["k"]), f64(inp["v"]),
                                             lens.numpy(), i64(resident), w.top_k, w.window, w.cap,
                                             default_scale(), w.block)
            gs = f64(got["scores"])
            check_scores(gs, exp["scores"], score_floor(f64(inp["q"]), f64(summ)), "scores")
            np.testing.assert_array_equal(i64(got["topk"]), ref.topk_blocks(gs, lens.numpy(), w.top_k,
                                                                             w.window, w.block))
            pl = ref.build_plan(gs, i64(got["topk"]), i64(resident), lens.numpy(), w.cap, w.window, w.block)
            for key in ("plan_count", "table", "table_count"):
                np.testing.assert_array_equal(i64(got[key]), pl[key], err_msg=key)
            np.testing.assert_array_equal(i64(rn), pl["resident"])
            np.testing.assert_allclose(f64(got["out"]), exp["out"], rtol=0, atol=OUT_ATOL)
            np.testing.assert_allclose(f64(got["lse"]), exp["lse"], rtol=0, atol=OUT_ATOL)
        resident = rn
    # the same workspace then serves steps of other sizes (fewer heads, other cap), once
    # cleared for them
    w2 = w.with_(num_kv_heads=1, fetch_ratio=0.5)
    d2 = lib.dims_for(w2)
    if lib.workspace_bytes(d2) <= bufs.ws.numel():
        inp2 = {kk: t.to(DEV) for kk, t in synth.generate(w2, "cpu").items()}
        summ2 = lib.build_summaries(d2, inp2["k"], inp2["seq_lens"])
        b2 = lib.StepBuffers(d2, DEV)
        b2.ws = bufs.ws
        lib.workspace_clear(d2, bufs.ws)
        r2 = resident[:, :1].contiguous()
        rn2 = torch.empty_like(r2)
        got2 = lib.decode_step_overlapped(d2, inp2["q"], summ2, inp2["k"], inp2["v"], inp2["seq_lens"], r2,
                                          rn2, buffers=b2)
        torch.cuda.synchronize()
        assert lib.workspace_status(d2, bufs.ws) == 0
        lo2, hi2 = lib.workspace_bytes(d2, lib.table_stride(d2)), lib.workspace_bytes(d2)
        assert int(torch.count_nonzero(bufs.ws[lo2:hi2])) == 0
        table, tc = ref.resident_table(i64(r2), inp2["seq_lens"].cpu().numpy(), w2.window, w2.block)
        eo, el = ref.sparse_attention(f64(inp2["q"]), f64(inp2["k"]), f64(inp2["v"]), table, tc,
                                      inp2["seq_lens"].cpu().numpy(), default_scale(), w2.block)
        np.testing.assert_allclose(f64(got2["out"]), eo, rtol=0, atol=OUT_ATOL)


@pytest.mark.parametrize("overlapped,redo", [(False, False), (False, True), (True, False)])
def test_graph_replay_matches_eager(lib, overlapped, redo):
    """Every replay of a captured step, with eager work and syncs between replays,
    gives the eager result bit for bit: the serial step as four kernels and in the form
    that redoes the touched splits, and the overlapped step."""
    w = synth.WORKLOADS["tiny_4k"].with_(batch=4, fetch_ratio=0.25)
    if redo:   # K = 64, cap 4: a plan touches at most 4 of 18 splits
        w = w.with_(top_k=64, fetch_ratio=0.0625)
    _say(f"graph replay overlapped={overlapped} redo={redo}")
    d, inp, summ, res = _prepared_inputs(lib, w, seed_layer=3)
    if not overlapped:
        assert lib.decode_step_redoes_touched_splits(d) == redo
    bufs = lib.StepBuffers(d, DEV)
    rn = torch.empty_like(res)
    st = lib.PreparedStep(d, inp["q"], summ, inp["k"], inp["v"], inp["seq_lens"], res, bufs,
                          resident_next=rn, overlapped=overlapped)
    st()
    torch.cuda.synchronize()
    eager = {**{k: v.clone() for k, v in bufs.as_dict().items()}, "resident": rn.clone()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st()
    for rep in range(4):
        for t in list(bufs.as_dict().values()) + [rn]:
            t.fill_(-7 if t.dtype == torch.int32 else float("nan"))   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {**bufs.as_dict(), "resident": rn}
        for key in eager:
            assert torch.equal(eager[key], got[key]), f"replay {rep}: {key}"


@pytest.mark.parametrize("group,queries,ctx,batch,heads", [
    (4, 5, 4096 + 40, 2, 3),            # each layer selects in its own first launch
    (8, 2, 4096 + 40, 2, 3),            # the same at 8 query heads
    (4, 5, 2048 * 16 + 40, 2, 3),       # 2051 blocks: in the next layer's second launch
    (4, 5, 4096 + 40, 33, 8),           # 264 pairs: in the next layer's first launch
])
def test_layer_pipelined_sweep_matches_the_overlapped_step(lib, group, queries, ctx, batch, heads):
    """Three layers, two decode steps of the layer-pipelined sweep, whose selections run
    in the layer's own first launch, the next layer's first launch, or the next layer's
    second launch with its merge, by size: every layer's plan outputs equal the
    overlapped step's bit for bit, its attention equals it up to the merge's summation
    order and matches the oracle."""
    w = synth.WORKLOADS["tiny_4k"].with_(batch=batch, num_kv_heads=heads, group=group, num_drafts=queries - 1,
                                         fetch_ratio=0.25, ctx=ctx, min_len=1000)
    _say(f"layer-pipelined sweep group={group} ctx={ctx}")
    d = lib.dims_for(w)
    layers, expected = [], []
    for layer in range(3):
        d_, inp, summ, res = _prepared_inputs(lib, w, seed_layer=layer)
        rn = torch.empty_like(res)
        ov = lib.decode_step_overlapped(d, inp["q"], summ, inp["k"], inp["v"], inp["seq_lens"], res, rn,
                                        default_scale())
        torch.cuda.synchronize()
        expected.append(({k: v.clone() for k, v in ov.items()}, rn.clone(), inp, res))
        layers.append((inp["q"], summ, inp["k"], inp["v"], inp["seq_lens"], res))
    sweep = lib.PipelinedLayers(d, layers, default_scale())
    for step in range(2):
        sweep()
        sweep.drain()
        torch.cuda.synchronize()
        for li, (exp, rn, inp, res) in enumerate(expected):
            b = sweep.buffers[li]
            for key in ("scores", "topk", "plan", "plan_count", "table", "table_count"):
                assert torch.equal(getattr(b, key), exp[key]), f"step {step} layer {li}: {key}"
            assert torch.equal(sweep.resident_next[li], rn)
            assert (b.out - exp["out"]).abs().max().item() <= 1e-6
            lens = inp["seq_lens"].cpu().numpy()
            table, tc = ref.resident_table(i64(res.cpu()), lens, w.window)
            eo, _ = ref.sparse_attention(f64(inp["q"].cpu()), f64(inp["k"].cpu()), f64(inp["v"].cpu()),
                                         table, tc, lens, default_scale())
            np.testing.assert_allclose(f64(b.out.cpu()), eo, rtol=0, atol=OUT_ATOL)


def test_pipelined_sweep_graph_replay_matches_eager(lib):
    """A captured layer-pipelined sweep, replayed several times with eager work and
    syncs between the replays, gives the eager sweep's outputs bit for bit."""
    w = synth.WORKLOADS["tiny_4k"].with_(batch=2, num_kv_heads=2, fetch_ratio=0.25)
    _say("pipelined sweep graph replay")
    layers = []
    for layer in range(3):
        d, inp, summ, res = _prepared_inputs(lib, w, seed_layer=layer)
        layers.append((inp["q"], summ, inp["k"], inp["v"], inp["seq_lens"], res))
    sweep = lib.PipelinedLayers(d, layers, default_scale())
    sweep()
    sweep()                          # steady state: the first layer's launch selects the last layer
    torch.cuda.synchronize()
    eager = [_step_outputs(b, rn) for b, rn in zip(sweep.buffers, sweep.resident_next)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sweep()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sweep()
    last = len(layers) - 1
    for rep in range(3):
        for li, (b, rn) in enumerate(zip(sweep.buffers, sweep.resident_next)):
            for key, t in list(b.as_dict().items()) + [("resident", rn)]:
                if li == last and key == "scores":
                    continue         # read by the first layer's launch before being rewritten
                t.fill_(-7 if t.dtype == torch.int32 else float("nan"))   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for li, (b, rn) in enumerate(zip(sweep.buffers, sweep.resident_next)):
            got = {**b.as_dict(), "resident": rn}
            for key, val in eager[li].items():
                assert torch.equal(got[key], val), f"replay {rep} layer {li}: {key}"


def test_layer_pipelined_sweep_at_the_qwen3_8b_shape(lib):
    """Three layers of the Qwen3-8B 32K shape (four sequences, all eight KV heads: each
    layer selects in its own first launch at K = 128 and 2048 blocks), two sweeps:
    every layer's plan outputs and next slot table equal its overlapped step's bit for
    bit and its attention equals it up to the merge's summation order."""
    w = synth.WORKLOADS["qwen3_8b_32k"].with_(batch=4)
    _say("layer-pipelined sweep at the Qwen3-8B shape")
    d = lib.dims_for(w)
    layers, expected = [], []
    for layer in range(3):
        inp = synth.generate(w, DEV, layer=layer)
        summ = lib.build_summaries(d, inp["k"], inp["seq_lens"])
        sel = lib.topk_blocks(d, lib.score_summaries(d, inp["q_prev"], summ, inp["seq_lens"]), inp["seq_lens"])
        res = synth.resident_from_selection(w, sel, inp["seq_lens"].cpu(), layer=layer).to(DEV)
        rn = torch.empty_like(res)
        ov = lib.decode_step_overlapped(d, inp["q"], summ, inp["k"], inp["v"], inp["seq_lens"], res, rn,
                                        default_scale())
        torch.cuda.synchronize()
        expected.append(({k: v.clone() for k, v in ov.items()}, rn.clone()))
        layers.append((inp["q"], summ, inp["k"], inp["v"], inp["seq_lens"], res))
    sweep = lib.PipelinedLayers(d, layers, default_scale())
    for step in range(2):
        sweep()
        sweep.drain()
        torch.cuda.synchronize()
        for li, (exp, rn) in enumerate(expected):
            b = sweep.buffers[li]
            for key in ("scores", "topk", "plan", "plan_count", "table", "table_count"):
                assert torch.equal(getattr(b, key), exp[key]), f"step {step} layer {li}: {key}"
            assert torch.equal(sweep.resident_next[li], rn)
            assert (b.out - exp["out"]).abs().max().item() <= 1e-6
    del layers, expected, sweep
    torch.cuda.empty_cache()
