"""GPU parity at block sizes other than 16 tokens (8, 32 and 64): every entry point
against the fp64 oracle, which takes the block size as a parameter.

The pages fix 16-token blocks (xllm-io review, section six, default parameters);
the other sizes are a sweep variant.  The summaries stay one min and one max row per
block whatever its size, so the scoring and selection change only through the
block geometry (candidates, window blocks); the attention, the working set and
the appended token read and write blocks of 8 to 64 tokens.

All calls go through the C ABI (ctypes binding).  Inputs are seeded synthetic
tensors; no expected value comes from the GPU.
"""
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import ref
from tests._helpers import (OUT_ATOL, check_scores, default_scale, f64, i64, oracle_head,
                            score_floor)

pytestmark = pytest.mark.gpu

DEV = "cuda"
BLOCKS = [8, 32, 64]
PLAN_KEYS = ("topk", "plan", "plan_count", "resident", "table", "table_count")


def _say(msg):
    print(f"[block sizes] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    import oasis_score_summaries_amd as oa
    oa.load()
    return oa


def _inputs(seed, B, H, G, Q, NB, bs, lens, integer=False):
    g = torch.Generator().manual_seed(seed)
    if integer:
        q = torch.randint(-3, 4, (B, H, G, Q, 128), generator=g).to(torch.bfloat16)
        k = torch.randint(-4, 5, (B, H, NB, bs, 128), generator=g).to(torch.bfloat16)
    else:
        q = torch.randn((B, H, G, Q, 128), generator=g).to(torch.bfloat16)
        k = torch.randn((B, H, NB, bs, 128), generator=g).to(torch.bfloat16)
    v = torch.randn((B, H, NB, bs, 128), generator=g).to(torch.bfloat16)
    return q, k, v, torch.tensor(lens, dtype=torch.int32)


def _slot_tables(seed, B, H, K, lens, bs, n_empty_of_h=lambda h: h % 3):
    """Slot tables with empty slots and with blocks anywhere in the sequence
    (window blocks included)."""
    r = np.random.default_rng(seed)
    R = np.full((B, H, K), -1, dtype=np.int64)
    for b in range(B):
        nb = ref.num_blocks(lens[b], bs)
        for h in range(H):
            n = min(K - n_empty_of_h(h), nb)
            R[b, h, :n] = r.choice(nb, size=n, replace=False)
            r.shuffle(R[b, h])
    return R


@pytest.mark.parametrize("bs", BLOCKS)
@pytest.mark.parametrize("W", [64, 40])
def test_decode_step_integer_inputs(lib, bs, W):
    """Small-integer q and k make every score exact in fp32 and fp64, so the
    selection, plan and table (ties included) agree bit for bit; lengths ragged at
    every block size, one shorter than a block."""
    lens = [4096 + 5, 1000, 3, 777]
    B, H, G, Q, K = len(lens), 3, 4, 5, 24
    NB = ref.num_blocks(max(lens), bs) + 2
    _say(f"integer decode step bs={bs} W={W}")
    q, k, v, L = _inputs(100 + bs + W, B, H, G, Q, NB, bs, lens, integer=True)
    d = lib.make_dims(B, H, G, NB, Q, K, W, 0.25, block_size=bs)
    resident = torch.empty((B, H, K), dtype=torch.int32)
    for b in range(B):
        for h in range(H):
            resident[b, h] = synth.random_resident(K, ref.first_window_block(lens[b], W, bs), [0, 3, K][h],
                                                   50 * b + h)
    kd, Ld = k.to(DEV), L.to(DEV)
    summ = lib.build_summaries(d, kd, Ld)
    got = lib.decode_step(d, q.to(DEV), summ, kd, v.to(DEV), Ld, resident.to(DEV), default_scale())
    torch.cuda.synchronize()
    got = {key: val.cpu() for key, val in got.items()}
    for b in range(B):
        for h in range(H):
            exp = oracle_head(q, k, v, L, resident[b, h].numpy(), K, W, d_cap(d), default_scale(), b, h, bs)
            assert np.array_equal(f64(summ[b, h]), exp["summ"]), f"summaries b={b} h={h}"
            np.testing.assert_array_equal(f64(got["scores"][b, h]), exp["scores"])
            for key in PLAN_KEYS:
                np.testing.assert_array_equal(i64(got[key][b, h]), exp[key], err_msg=f"{key} b={b} h={h}")
            np.testing.assert_allclose(f64(got["out"][b, h]), exp["out"], rtol=0, atol=OUT_ATOL)
            fin = np.isfinite(exp["lse"])
            np.testing.assert_allclose(f64(got["lse"][b, h])[fin], exp["lse"][fin], rtol=0, atol=OUT_ATOL)


def d_cap(d):
    return ref.fetch_cap(d.fetch_ratio, d.top_k)


@pytest.mark.parametrize("bs", BLOCKS)
def test_overlapped_step(lib, bs):
    """The overlapped step on N(0,1) data with planted blocks: scores within the
    tolerance of the oracle's, the selection equal to a full sort of the GPU's own
    scores, the plan equal to the oracle's plan on the GPU's own scores and
    selection, and the attention over the slot table as it was within the tolerance."""
    w = synth.WORKLOADS["tiny_4k"].with_(block=bs, batch=3, num_kv_heads=2, fetch_ratio=0.25,
                                         ctx=4096 + 40, min_len=1000, top_k=max(8, 256 // bs))
    _say(f"overlapped step bs={bs} K={w.top_k}")
    inp = synth.generate(w, "cpu")
    d = lib.dims_for(w)
    lens = inp["seq_lens"].numpy()
    n_cand = [ref.first_window_block(int(x), w.window, bs) for x in lens]
    R = torch.stack([torch.stack([synth.random_resident(w.top_k, n_cand[b], 2, 7 * b + h)
                                  for h in range(w.num_kv_heads)]) for b in range(w.batch)])
    dev = {key: t.to(DEV) for key, t in inp.items()}
    summ = lib.build_summaries(d, dev["k"], dev["seq_lens"])
    rn = torch.empty_like(R).to(DEV)
    ov = lib.decode_step_overlapped(d, dev["q"], summ, dev["k"], dev["v"], dev["seq_lens"], R.to(DEV), rn,
                                    default_scale())
    torch.cuda.synchronize()
    ov = {key: val.cpu() for key, val in ov.items()}
    q64, k64, v64 = f64(inp["q"]), f64(inp["k"]), f64(inp["v"])
    summ64 = ref.build_summaries(k64, lens, bs)
    assert np.array_equal(f64(summ), summ64)
    escore = ref.score_blocks(q64, summ64, lens, w.window, bs)
    check_scores(f64(ov["scores"]), escore, score_floor(q64, summ64), f"bs={bs}")
    gs = ov["scores"].numpy()
    esel = ref.topk_blocks(gs, lens, w.top_k, w.window, bs)
    np.testing.assert_array_equal(i64(ov["topk"]), esel)
    plan = ref.build_plan(gs.astype(np.float64), esel, i64(R), lens, w.cap, w.window, bs)
    for key in ("plan", "plan_count", "table", "table_count"):
        np.testing.assert_array_equal(i64(ov[key]), plan[key], err_msg=key)
    np.testing.assert_array_equal(i64(rn), plan["resident"])
    assert int(ov["plan_count"].sum()) > 0
    table, tc = ref.resident_table(i64(R), lens, w.window, bs)
    eo, el = ref.sparse_attention(q64, k64, v64, table, tc, lens, default_scale(), bs)
    np.testing.assert_allclose(f64(ov["out"]), eo, rtol=0, atol=OUT_ATOL)
    np.testing.assert_allclose(f64(ov["lse"]), el, rtol=0, atol=OUT_ATOL)


@pytest.mark.parametrize("bs", BLOCKS)
@pytest.mark.parametrize("G", [1, 4, 16])
def test_attention_tables(lib, bs, G):
    """Attention over compacted tables (random subsets in random order, the
    partial last block included, padded rows past the count) and over slot tables
    (empty slots, blocks the window has reached)."""
    lens = [3000 + 7, 70, 1024]
    B, H, Q, K, W = len(lens), 2, 2, 20, 48
    NB = ref.num_blocks(max(lens), bs) + 1
    _say(f"attention tables bs={bs} G={G}")
    q, k, v, L = _inputs(200 + bs + G, B, H, G, Q, NB, bs, lens)
    d = lib.make_dims(B, H, G, NB, Q, K, W, 0.05, block_size=bs)
    T = 40
    r = np.random.default_rng(bs * G)
    table = np.full((B, H, T), -1, dtype=np.int64)
    tc = np.zeros((B, H), dtype=np.int64)
    for b in range(B):
        nb = ref.num_blocks(lens[b], bs)
        for h in range(H):
            n = min(T - 3, nb) if h == 0 else min(nb, 5)
            blocks = r.choice(nb, size=n, replace=False)
            if nb - 1 not in blocks:
                blocks[0] = nb - 1                      # the partial last block
            table[b, h, :n] = blocks
            tc[b, h] = n
    scale = default_scale()
    qd, kd, vd, Ld = q.to(DEV), k.to(DEV), v.to(DEV), L.to(DEV)
    out, lse = lib.sparse_decode_attn(d, qd, kd, vd, torch.from_numpy(table.astype(np.int32)).to(DEV),
                                      torch.from_numpy(tc.astype(np.int32)).to(DEV), Ld, scale)
    R = _slot_tables(300 + bs, B, H, K, lens, bs)
    rout, rlse = lib.sparse_decode_attn_resident(d, qd, kd, vd, torch.from_numpy(R.astype(np.int32)).to(DEV),
                                                 Ld, scale)
    torch.cuda.synchronize()
    q64, k64, v64 = f64(q), f64(k), f64(v)
    eo, el = ref.sparse_attention(q64, k64, v64, table, tc, L.numpy(), scale, bs)
    np.testing.assert_allclose(f64(out), eo, rtol=0, atol=OUT_ATOL)
    np.testing.assert_allclose(f64(lse), el, rtol=0, atol=OUT_ATOL)
    rt, rtc = ref.resident_table(R, L.numpy(), W, bs)
    eo, el = ref.sparse_attention(q64, k64, v64, rt, rtc, L.numpy(), scale, bs)
    np.testing.assert_allclose(f64(rout), eo, rtol=0, atol=OUT_ATOL)
    np.testing.assert_allclose(f64(rlse), el, rtol=0, atol=OUT_ATOL)


@pytest.mark.parametrize("bs", BLOCKS)
def test_attention_all_blocks_matches_dense(lib, bs):
    """A table of every block is dense attention over the sequence (the oracle's pin
    at any block size): the GPU against dense softmax attention in fp64."""
    lens = [2000 + 3, 129]
    B, H, G, Q = len(lens), 2, 4, 1
    NB = ref.num_blocks(max(lens), bs)
    _say(f"all blocks vs dense bs={bs}")
    q, k, v, L = _inputs(400 + bs, B, H, G, Q, NB, bs, lens)
    d = lib.make_dims(B, H, G, NB, Q, 1, 0, 0.0, block_size=bs)
    table = torch.arange(NB, dtype=torch.int32).repeat(B, H, 1)
    tc = torch.tensor([[ref.num_blocks(x, bs)] * H for x in lens], dtype=torch.int32)
    out, _ = lib.sparse_decode_attn(d, q.to(DEV), k.to(DEV), v.to(DEV), table.to(DEV), tc.to(DEV),
                                    L.to(DEV), default_scale())
    torch.cuda.synchronize()
    for b in range(B):
        kk = k[b].double().reshape(H, NB * bs, 128)[:, : lens[b]]
        vv = v[b].double().reshape(H, NB * bs, 128)[:, : lens[b]]
        qq = q[b, :, :, 0].double()
        dense = torch.nn.functional.scaled_dot_product_attention(
            qq[:, :, None], kk[:, None].expand(H, G, -1, -1), vv[:, None].expand(H, G, -1, -1),
            scale=default_scale())[:, :, 0]
        np.testing.assert_allclose(f64(out[b]), dense.numpy(), rtol=0, atol=OUT_ATOL)


@pytest.mark.parametrize("bs", BLOCKS)
def test_working_set(lib, bs):
    """The working set gathered from the full cache equals the oracle's bit for bit;
    attention over it equals the full-cache slot-table attention bit for bit; the
    plan's copies leave the pool equal to the gather of the next slot table; tokens
    appended across block boundaries keep cache, ring and summaries equal to the
    oracle's."""
    lens = [1500 + 3, 700]
    B, H, G, Q, W = len(lens), 2, 4, 3, 40
    K = max(6, 128 // bs)
    NB = ref.num_blocks(max(lens), bs) + 2
    _say(f"working set bs={bs} K={K}")
    q, k, v, L = _inputs(500 + bs, B, H, G, Q, NB, bs, lens)
    d = lib.make_dims(B, H, G, NB, Q, K, W, 0.5, block_size=bs)
    R = _slot_tables(600 + bs, B, H, K, lens, bs, lambda h: 1 + h)
    Rd = torch.from_numpy(R.astype(np.int32)).to(DEV)
    kd, vd, Ld = k.to(DEV), v.to(DEV), L.to(DEV)
    wset = lib.fill_working_set(d, Rd, Ld, kd, vd)
    out, lse = lib.sparse_decode_attn_pool(d, q.to(DEV), wset, Rd, Ld)
    alone, alone_lse = lib.sparse_decode_attn_resident(d, q.to(DEV), kd, vd, Rd, Ld)
    torch.cuda.synchronize()
    pk, pv, rk, rv = ref.fill_working_set(f64(k), f64(v), R, L.numpy(), W, bs)
    for name, got, exp in (("pool_k", wset.pool_k, pk), ("pool_v", wset.pool_v, pv),
                           ("ring_k", wset.ring_k, rk), ("ring_v", wset.ring_v, rv)):
        assert np.array_equal(f64(got), exp), name
    assert torch.equal(out, alone) and torch.equal(lse, alone_lse)
    eo, el = ref.pool_attention(f64(q), pk, pv, rk, rv, R, L.numpy(), W, default_scale(), bs)
    np.testing.assert_allclose(f64(out), eo, rtol=0, atol=OUT_ATOL)

    # A step's plan, executed: the pool becomes the gather of the next slot table.
    Rc = R.copy()
    Rc[Rc >= np.array([ref.first_window_block(x, W, bs) for x in lens])[:, None, None]] = -1
    Rcd = torch.from_numpy(Rc.astype(np.int32)).to(DEV)
    summ = lib.build_summaries(d, kd, Ld)
    bufs = lib.StepBuffers(d, DEV)
    rn = torch.empty_like(Rcd)
    lib.decode_step(d, q.to(DEV), summ, kd, vd, Ld, Rcd, default_scale(), buffers=bufs, resident_next=rn)
    wset2 = lib.fill_working_set(d, Rcd, Ld, kd, vd)
    lib.execute_plan(d, bufs.plan, bufs.plan_count, kd, vd, wset2)
    expect = lib.fill_working_set(d, rn, Ld, kd, vd)
    torch.cuda.synchronize()
    assert int(bufs.plan_count.sum()) > 0
    assert torch.equal(wset2.pool_k, expect.pool_k) and torch.equal(wset2.pool_v, expect.pool_v)
    pk2, pv2, _, _ = ref.fill_working_set(f64(k), f64(v), Rc, L.numpy(), W, bs)
    ek, ev = ref.execute_plan(pk2, pv2, i64(bufs.plan), i64(bufs.plan_count), f64(k), f64(v))
    assert np.array_equal(f64(wset2.pool_k), ek) and np.array_equal(f64(wset2.pool_v), ev)

    # Appended tokens: more than a block's worth, so that blocks open and close.
    ok, ov, os_ = f64(kd), f64(vd), f64(summ)
    _, _, ork, orv = ref.fill_working_set(ok, ov, Rc, L.numpy(), W, bs)
    wset3 = lib.fill_working_set(d, Rcd, Ld, kd, vd)
    g = torch.Generator().manual_seed(bs)
    for step in range(bs + 5):
        kn = (torch.randn((B, H, 128), generator=g) * (1 + step % 3)).to(torch.bfloat16)
        vn = torch.randn((B, H, 128), generator=g).to(torch.bfloat16)
        lib.append_token(d, kn.to(DEV), vn.to(DEV), Ld, summ, wset3, kd, vd)
        ok, ov, os_, ork, orv = ref.append_token(ok, ov, os_, ork, orv, f64(kn), f64(vn), i64(Ld), W, bs)
        Ld += 1
    torch.cuda.synchronize()
    assert np.array_equal(f64(summ), os_)
    assert np.array_equal(f64(wset3.ring_k), ork) and np.array_equal(f64(wset3.ring_v), orv)
    assert np.array_equal(f64(kd), ok) and np.array_equal(f64(vd), ov)
    rebuilt = lib.build_summaries(d, kd, Ld)
    torch.cuda.synchronize()
    for b in range(B):
        nb = ref.num_blocks(int(Ld[b]), bs)
        assert torch.equal(summ[b, :, :nb], rebuilt[b, :, :nb])


@pytest.mark.parametrize("bs", BLOCKS)
def test_full_size_fixed_token_budget(lib, bs):
    """The Qwen3-8B 32K shape (two sequences, two KV heads) at each block size with
    the pages' 2048-token budget kept: K = 2048 / bs blocks per KV head."""
    from tests.test_parity import _full_size_case
    w = synth.WORKLOADS["qwen3_8b_32k"].with_(batch=2, num_kv_heads=2, block=bs, top_k=2048 // bs)
    _full_size_case(lib, w)


def test_layer_pipelined_sweep_32_token_blocks(lib):
    """The layer-pipelined sweep at 32-token blocks: every layer's outputs equal its
    overlapped step's (plan outputs bit for bit, attention up to the merge order)."""
    w = synth.WORKLOADS["tiny_4k"].with_(block=32, batch=2, num_kv_heads=3, fetch_ratio=0.25,
                                         ctx=4096 + 40, min_len=1000, top_k=12)
    _say("layer-pipelined sweep bs=32")
    d = lib.dims_for(w)
    layers, expected = [], []
    for layer in range(3):
        inp = {key: t.to(DEV) for key, t in synth.generate(w, "cpu", layer=layer).items()}
        summ = lib.build_summaries(d, inp["k"], inp["seq_lens"])
        n_cand = [ref.first_window_block(int(x), w.window, 32) for x in inp["seq_lens"].cpu()]
        res = torch.stack([torch.stack([synth.random_resident(w.top_k, n_cand[b], 2, 10 * b + h + layer)
                                        for h in range(w.num_kv_heads)]) for b in range(w.batch)]).to(DEV)
        rn = torch.empty_like(res)
        ov = lib.decode_step_overlapped(d, inp["q"], summ, inp["k"], inp["v"], inp["seq_lens"], res, rn,
                                        default_scale())
        torch.cuda.synchronize()
        expected.append(({key: val.clone() for key, val in ov.items()}, rn.clone()))
        layers.append((inp["q"], summ, inp["k"], inp["v"], inp["seq_lens"], res))
    sweep = lib.PipelinedLayers(d, layers, default_scale())
    sweep()
    sweep.drain()
    torch.cuda.synchronize()
    for li, (exp, rn) in enumerate(expected):
        b = sweep.buffers[li]
        for key in ("scores", "topk", "plan", "plan_count", "table", "table_count"):
            assert torch.equal(getattr(b, key), exp[key]), f"layer {li}: {key}"
        assert torch.equal(sweep.resident_next[li], rn)
        assert (b.out - exp["out"]).abs().max().item() <= 1e-6


def test_largest_supported_sizes_64_token_blocks(lib):
    """max_blocks = 32768 at 64-token blocks (a 2M-token context, 512 MiB of K per
    head: the largest byte offsets the gather forms), K = 1024, a 4096-token window,
    16 query heads, a cap of 512 and a ragged last block, both step orders.  Scores
    are checked on sampled blocks, selection, plan and attention on the GPU's own
    scores and tables."""
    bs = 64
    B, H, G, Q, NB, K, W, ratio = 1, 1, 16, 2, 32768, 1024, 4096, 0.5
    L = NB * bs - 5
    _say("largest sizes bs=64: generating")
    g = torch.Generator().manual_seed(78)
    q = torch.randn((B, H, G, Q, 128), generator=g).to(torch.bfloat16)
    k = torch.randn((B, H, NB, bs, 128), generator=g).to(torch.bfloat16)
    v = torch.randn((B, H, NB, bs, 128), generator=g).to(torch.bfloat16)
    lens = torch.tensor([L], dtype=torch.int32)
    d = lib.make_dims(B, H, G, NB, Q, K, W, ratio, block_size=bs)
    C = lib.fetch_cap(d)
    assert C == 512
    n_cand = ref.first_window_block(L, W, bs)
    res = synth.random_resident(K, n_cand, 100, 6).reshape(1, 1, K)
    qd, kd, vd, ld = q.to(DEV), k.to(DEV), v.to(DEV), lens.to(DEV)
    summ = lib.build_summaries(d, kd, ld)
    _say("largest sizes bs=64: serial and overlapped steps")
    ser = lib.decode_step(d, qd, summ, kd, vd, ld, res.to(DEV).clone(), default_scale())
    ser = {key: val.cpu() for key, val in ser.items()}
    rn = torch.empty_like(res).to(DEV)
    ov = lib.decode_step_overlapped(d, qd, summ, kd, vd, ld, res.to(DEV), rn, default_scale())
    ov = {key: val.cpu() for key, val in ov.items()}
    torch.cuda.synchronize()
    del qd, kd, vd
    rng = np.random.default_rng(4)
    blocks = np.sort(rng.choice(n_cand, size=256, replace=False))
    summ_s = f64(summ[:, :, blocks].cpu())
    exp_s = ref.score_blocks(f64(q), summ_s, np.array([len(blocks) * bs]), 0, bs)
    check_scores(f64(ser["scores"][:, :, blocks]), exp_s, score_floor(f64(q), summ_s), "sampled scores")
    np.testing.assert_array_equal(f64(summ[:, :, blocks[:8]].cpu()),
                                  ref.build_summaries(f64(k[:, :, blocks[:8]]), np.array([8 * bs]), bs)[:, :, :8])
    sc = f64(ser["scores"])
    np.testing.assert_array_equal(f64(ov["scores"]), sc)
    sel = ref.topk_blocks(sc, lens.numpy(), K, W, bs)
    np.testing.assert_array_equal(i64(ser["topk"]), sel)
    plan = ref.build_plan(sc, sel, i64(res), lens.numpy(), C, W, bs)
    for key in ("plan", "plan_count", "resident", "table", "table_count"):
        np.testing.assert_array_equal(i64(ser[key]), plan[key], err_msg=key)
        np.testing.assert_array_equal(i64(ov[key]), plan[key], err_msg=key)
    assert int(ser["plan_count"][0, 0]) == C
    _say("largest sizes bs=64: oracle attention")
    # Only the blocks some table names are widened to fp64; the others stay zero (never read).
    used = np.union1d(plan["table"][plan["table"] >= 0], ref.resident_table(i64(res), lens.numpy(), W, bs)[0])
    used = used[used >= 0]
    kf = np.zeros((B, H, NB, bs, 128))
    vf = np.zeros((B, H, NB, bs, 128))
    kf[:, :, used] = f64(k[:, :, used])
    vf[:, :, used] = f64(v[:, :, used])
    eo, _ = ref.sparse_attention(f64(q), kf, vf, plan["table"], plan["table_count"], lens.numpy(),
                                 default_scale(), bs)
    np.testing.assert_allclose(f64(ser["out"]), eo, rtol=0, atol=OUT_ATOL)
    table, tc = ref.resident_table(i64(res), lens.numpy(), W, bs)
    eo2, _ = ref.sparse_attention(f64(q), kf, vf, table, tc, lens.numpy(), default_scale(), bs)
    np.testing.assert_allclose(f64(ov["out"]), eo2, rtol=0, atol=OUT_ATOL)


@pytest.mark.parametrize("bs,tier", [(8, "device"), (32, "host"), (64, "device")])
def test_decode_loop_over_the_working_set(lib, bs, tier):
    """Four decode steps over the working set, each followed by an appended token:
    every output equals the full-cache overlapped step's bit for bit and the pool
    holds the next slot table's blocks afterwards; then a captured step over the
    working set replays bit-exactly."""
    w = synth.WORKLOADS["tiny_4k"].with_(block=bs, batch=3, num_kv_heads=2, fetch_ratio=0.25,
                                         ctx=4096 + 40, min_len=1000, top_k=max(8, 256 // bs))
    _say(f"decode loop over the working set bs={bs} {tier}")
    inp = {key: t.to(DEV) for key, t in synth.generate(w, "cpu").items()}
    d = lib.dims_for(w)
    kd, vd, Ld = inp["k"].clone(), inp["v"].clone(), inp["seq_lens"].clone()
    summ = lib.build_summaries(d, kd, Ld)
    n_cand = [ref.first_window_block(int(x), w.window, bs) for x in Ld.cpu()]
    R = torch.stack([torch.stack([synth.random_resident(w.top_k, n_cand[b], 2, 9 * b + h)
                                  for h in range(w.num_kv_heads)]) for b in range(w.batch)]).to(DEV)
    if tier == "host":
        hk, hv = kd.cpu().pin_memory(), vd.cpu().pin_memory()
        src_k, src_v = hk, hv
    else:
        src_k, src_v = kd, vd
    wset = lib.fill_working_set(d, R, Ld, src_k, src_v)
    g = torch.Generator().manual_seed(bs)
    for step in range(4):
        rn_pool, rn_full = torch.empty_like(R), torch.empty_like(R)
        pool_out = {key: t.clone() for key, t in
                    lib.decode_step_pool(d, inp["q"], summ, src_k, src_v, wset, Ld, R, rn_pool).items()}
        full_out = lib.decode_step_overlapped(d, inp["q"], summ, kd, vd, Ld, R, rn_full)
        torch.cuda.synchronize()
        for key in ("scores", "topk", "plan", "plan_count", "table", "table_count", "out", "lse"):
            assert torch.equal(pool_out[key], full_out[key]), f"step {step}: {key}"
        assert torch.equal(rn_pool, rn_full)
        expect = lib.fill_working_set(d, rn_full, Ld, kd, vd)
        torch.cuda.synchronize()
        assert torch.equal(wset.pool_k, expect.pool_k) and torch.equal(wset.pool_v, expect.pool_v)
        kn = torch.randn((w.batch, w.num_kv_heads, 128), generator=g).to(torch.bfloat16).to(DEV)
        vn = torch.randn((w.batch, w.num_kv_heads, 128), generator=g).to(torch.bfloat16).to(DEV)
        lib.append_token(d, kn, vn, Ld, summ, wset, kd, vd)
        if tier == "host":
            lib.append_token(d, kn, vn, Ld, summ.clone(), lib.WorkingSet(d, DEV), hk, hv)
        torch.cuda.synchronize()
        Ld += 1
        R = rn_full
    # A captured step over the working set: before the eager step and before every
    # replay the working set is gathered again for R (the step's copies move the
    # admitted blocks into it), so every replay must equal the eager step, pool included.
    bufs = lib.StepBuffers(d, DEV)
    rn = torch.empty_like(R)
    st = lib.PreparedPoolStep(d, inp["q"], summ, src_k, src_v, wset, Ld, R, bufs, rn)
    lib.fill_working_set(d, R, Ld, src_k, src_v, wset)
    st()
    torch.cuda.synchronize()
    eager = {**{key: t.clone() for key, t in bufs.as_dict().items()}, "resident": rn.clone(),
             "pool_k": wset.pool_k.clone(), "pool_v": wset.pool_v.clone()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st()
    for rep in range(3):
        for t in list(bufs.as_dict().values()) + [rn]:
            t.fill_(-7 if t.dtype == torch.int32 else float("nan"))
        lib.fill_working_set(d, R, Ld, src_k, src_v, wset)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {**bufs.as_dict(), "resident": rn, "pool_k": wset.pool_k, "pool_v": wset.pool_v}
        for key in eager:
            assert torch.equal(eager[key], got[key]), f"replay {rep}: {key}"


@pytest.mark.parametrize("bs", BLOCKS)
def test_no_candidates_and_short_sequences(lib, bs):
    """Lengths at or below the window, a single token, a length one past a block
    boundary and zero window tokens: nothing (or one block) to score; the table is
    the window alone (or the partial last block), both step orders."""
    for W, lens in ((128, [100, 1, 128]), (0, [1, bs + 1, 3 * bs])):
        B, H, G, Q, K = len(lens), 2, 4, 2, 4
        NB = max(ref.num_blocks(max(lens), bs) + 1, K)
        _say(f"short sequences bs={bs} W={W} lens={lens}")
        q, k, v, L = _inputs(90 + bs + W, B, H, G, Q, NB, bs, lens)
        d = lib.make_dims(B, H, G, NB, Q, K, W, 1.0, block_size=bs)
        resident = torch.full((B, H, K), -1, dtype=torch.int32)
        kd, Ld = k.to(DEV), L.to(DEV)
        summ = lib.build_summaries(d, kd, Ld)
        got = lib.decode_step(d, q.to(DEV), summ, kd, v.to(DEV), Ld, resident.to(DEV), default_scale())
        rn = torch.empty_like(resident).to(DEV)
        ov = lib.decode_step_overlapped(d, q.to(DEV), summ, kd, v.to(DEV), Ld, resident.to(DEV), rn,
                                        default_scale())
        torch.cuda.synchronize()
        got = {key: val.cpu() for key, val in got.items()}
        ov = {key: val.cpu() for key, val in ov.items()}
        for b in range(B):
            for h in range(H):
                exp = oracle_head(q, k, v, L, resident[b, h].numpy(), K, W, d_cap(d), default_scale(),
                                  b, h, bs)
                for key in PLAN_KEYS:
                    np.testing.assert_array_equal(i64(got[key][b, h]), exp[key], err_msg=f"{key} b={b}")
                    if key != "resident":
                        np.testing.assert_array_equal(i64(ov[key][b, h]), exp[key], err_msg=f"{key} b={b}")
                np.testing.assert_allclose(f64(got["out"][b, h]), exp["out"], rtol=0, atol=OUT_ATOL)
                # with an empty slot table the overlapped step attends over the window alone
                table, tc = ref.resident_table(resident[b:b + 1, h:h + 1].numpy(), L[b:b + 1].numpy(), W, bs)
                eo, _ = ref.sparse_attention(f64(q[b:b + 1, h:h + 1]), f64(k[b:b + 1, h:h + 1]),
                                             f64(v[b:b + 1, h:h + 1]), table, tc, L[b:b + 1].numpy(),
                                             default_scale(), bs)
                np.testing.assert_allclose(f64(ov["out"][b, h]), eo[0, 0], rtol=0, atol=OUT_ATOL)


@pytest.mark.parametrize("bs", [8, 64])
def test_copy_and_append_edge_cases(lib, bs):
    """Plan rows out of range are skipped and the rest copied (whole blocks of bs
    tokens); with a cap of 0 the copy is a no-op; a sequence at capacity takes no
    appended token while the other takes it at its position."""
    B, H, G, Q, NB, K, W = 2, 2, 4, 1, 8, 4, 2 * bs
    q, k, v, L = _inputs(61 + bs, B, H, G, Q, NB, bs, [NB * bs, 3 * bs + 2])
    kd, vd, Ld = k.to(DEV), v.to(DEV), L.to(DEV)
    d = lib.make_dims(B, H, G, NB, Q, K, W, 0.5, block_size=bs)                    # cap 2
    R = torch.tensor([[[0, 1, 2, -1]] * H] * B, dtype=torch.int32, device=DEV)
    wset = lib.fill_working_set(d, R, Ld, kd, vd)
    before_k, before_v = wset.pool_k.clone(), wset.pool_v.clone()
    plan = torch.tensor([[[[3, 5, -1], [9, 6, 0]], [[0, 99, 0], [1, -4, 1]]],
                         [[[2, 7, 2], [-1, 4, 1]], [[3, 2, -1], [3, 3, -1]]]], dtype=torch.int32, device=DEV)
    count = torch.tensor([[2, 2], [1, 2]], dtype=torch.int32, device=DEV)
    lib.execute_plan(d, plan, count, kd, vd, wset)
    torch.cuda.synchronize()
    exp_k, exp_v = before_k.clone(), before_v.clone()
    for (b, h, slot, blk) in [(0, 0, 3, 5), (1, 0, 2, 7), (1, 1, 3, 2), (1, 1, 3, 3)]:
        exp_k[b, h, slot], exp_v[b, h, slot] = kd[b, h, blk], vd[b, h, blk]
    assert torch.equal(wset.pool_k, exp_k) and torch.equal(wset.pool_v, exp_v)
    d0 = lib.make_dims(B, H, G, NB, Q, K, W, 0.1, block_size=bs)                   # cap 0
    lib.execute_plan(d0, torch.empty((B, H, 0, 3), dtype=torch.int32, device=DEV), count, kd, vd, wset)
    summ = lib.build_summaries(d, kd, Ld)
    s0, r0, k0 = summ.clone(), wset.ring_k.clone(), kd.clone()
    kn = torch.randn((B, H, 128)).to(torch.bfloat16).to(DEV)
    lib.append_token(d, kn, kn, Ld, summ, wset, kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(wset.pool_k, exp_k)
    assert torch.equal(summ[0], s0[0]) and torch.equal(kd[0], k0[0]) and torch.equal(wset.ring_k[0], r0[0])
    pos = 3 * bs + 2
    assert torch.equal(kd[1, :, pos // bs, pos % bs], kn[1])             # the other sequence took it
    WB = lib.window_ring_slots(d)
    assert torch.equal(wset.ring_k[1, :, (pos // bs) % WB, pos % bs], kn[1])
