"""GPU parity of plan execution: the working set in HBM (pool slots, window ring),
the plan's block copies, the appended-token update and attention over the working
set, against the fp64 oracle and against the full-cache forms.

All calls go through the C ABI (ctypes binding).  Inputs are seeded synthetic
tensors; no expected value comes from the GPU.
"""
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import ref
from tests._helpers import OUT_ATOL, default_scale, f64, i64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(msg):
    print(f"[working set] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    import oasis_score_summaries_amd as oa
    oa.load()
    return oa


def _inputs(seed, B, H, G, Q, NB, lens):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, H, G, Q, 128), generator=g).to(torch.bfloat16)
    k = torch.randn((B, H, NB, 16, 128), generator=g).to(torch.bfloat16)
    v = torch.randn((B, H, NB, 16, 128), generator=g).to(torch.bfloat16)
    return q, k, v, torch.tensor(lens, dtype=torch.int32)


def _resident(seed, B, H, K, lens, NB, window):
    """Slot tables with empty slots, historical blocks and blocks the window has reached."""
    r = np.random.default_rng(seed)
    R = np.full((B, H, K), -1, dtype=np.int64)
    for b in range(B):
        nb = ref.num_blocks(lens[b])
        for h in range(H):
            n = min(K - 1 - h % 2, nb)
            R[b, h, :n] = r.choice(nb, size=n, replace=False)
            r.shuffle(R[b, h])
    return R


CASES = [  # B, H, G, Q, NB, K, W, lens
    (2, 3, 4, 2, 40, 8, 64, [600, 33]),
    (1, 2, 8, 1, 300, 32, 0, [4771]),          # no window tokens: the partial last block only
    (3, 2, 16, 2, 70, 12, 40, [1111, 16, 700]),
]


@pytest.mark.parametrize("B,H,G,Q,NB,K,W,lens", CASES)
def test_fill_and_pool_attention(lib, B, H, G, Q, NB, K, W, lens):
    """The gathered working set equals the oracle's bit for bit; attention over it
    equals the full-cache slot-table attention bit for bit (same arithmetic, other
    addresses) and the oracle within the attention tolerance."""
    _say(f"fill + pool attention B={B} H={H} G={G} NB={NB} K={K} W={W}")
    q, k, v, L = _inputs(7 + G, B, H, G, Q, NB, lens)
    d = lib.make_dims(B, H, G, NB, Q, K, W, 0.25)
    R = _resident(11 + K, B, H, K, lens, NB, W)
    Rd = torch.from_numpy(R.astype(np.int32)).to(DEV)
    kd, vd, Ld = k.to(DEV), v.to(DEV), L.to(DEV)
    wset = lib.fill_working_set(d, Rd, Ld, kd, vd)
    out, lse = lib.sparse_decode_attn_pool(d, q.to(DEV), wset, Rd, Ld)
    alone, alone_lse = lib.sparse_decode_attn_resident(d, q.to(DEV), kd, vd, Rd, Ld)
    torch.cuda.synchronize()
    pk, pv, rk, rv = ref.fill_working_set(f64(k), f64(v), R, L.numpy(), W)
    for name, got, exp in (("pool_k", wset.pool_k, pk), ("pool_v", wset.pool_v, pv),
                           ("ring_k", wset.ring_k, rk), ("ring_v", wset.ring_v, rv)):
        assert np.array_equal(f64(got), exp), name
    assert torch.equal(out, alone) and torch.equal(lse, alone_lse)
    eo, el = ref.pool_attention(f64(q), pk, pv, rk, rv, R, L.numpy(), W, default_scale())
    np.testing.assert_allclose(f64(out), eo, rtol=0, atol=OUT_ATOL)
    fin = np.isfinite(el)
    np.testing.assert_allclose(f64(lse)[fin], el[fin], rtol=0, atol=OUT_ATOL)


@pytest.mark.parametrize("tier", ["device", "host"])
def test_execute_plan_fills_the_next_slot_table(lib, tier):
    """After the plan's copies (from HBM or from pinned host memory) the pool is
    exactly the gather of the updated slot table, on the GPU and in the oracle."""
    B, H, G, Q, NB, K, W, lens = 2, 3, 4, 3, 80, 16, 32, [1270, 900]
    _say(f"execute plan from the {tier} tier")
    q, k, v, L = _inputs(31, B, H, G, Q, NB, lens)
    d = lib.make_dims(B, H, G, NB, Q, K, W, 0.25)
    R = _resident(32, B, H, K, lens, NB, W)
    R[R >= np.array([ref.first_window_block(x, W) for x in lens])[:, None, None]] = -1
    Rd = torch.from_numpy(R.astype(np.int32)).to(DEV)
    kd, vd, Ld = k.to(DEV), v.to(DEV), L.to(DEV)
    summ = lib.build_summaries(d, kd, Ld)
    bufs = lib.StepBuffers(d, DEV)
    rn = torch.empty_like(Rd)
    lib.decode_step(d, q.to(DEV), summ, kd, vd, Ld, Rd, default_scale(), buffers=bufs, resident_next=rn)
    src_k, src_v = (kd, vd) if tier == "device" else (k.pin_memory(), v.pin_memory())
    wset = lib.fill_working_set(d, Rd, Ld, src_k, src_v)
    lib.execute_plan(d, bufs.plan, bufs.plan_count, src_k, src_v, wset)
    expect = lib.fill_working_set(d, rn, Ld, kd, vd)
    torch.cuda.synchronize()
    assert int(bufs.plan_count.sum()) > 0
    assert torch.equal(wset.pool_k, expect.pool_k) and torch.equal(wset.pool_v, expect.pool_v)
    pk, pv, _, _ = ref.fill_working_set(f64(k), f64(v), R, L.numpy(), W)
    ek, ev = ref.execute_plan(pk, pv, i64(bufs.plan), i64(bufs.plan_count), f64(k), f64(v))
    assert np.array_equal(f64(wset.pool_k), ek) and np.array_equal(f64(wset.pool_v), ev)


def test_append_token_matches_oracle_and_rebuild(lib):
    """Thirty-five appended tokens, from partial blocks across block boundaries:
    full cache, ring and summaries bit-equal to the oracle after every token, and
    the summaries equal to a rebuild from the full cache."""
    B, H, NB, W = 3, 2, 12, 40
    _, k, v, L = _inputs(41, B, H, 1, 1, NB, [13, 48, 100])
    d = lib.make_dims(B, H, 1, NB, 1, 4, W, 0.25)
    kd, vd, Ld = k.to(DEV), v.to(DEV), L.to(DEV)
    summ = lib.build_summaries(d, kd, Ld)
    R = torch.full((B, H, 4), -1, dtype=torch.int32, device=DEV)
    wset = lib.fill_working_set(d, R, Ld, kd, vd)
    torch.cuda.synchronize()
    ok, ov, os_ = f64(k), f64(v), f64(summ)
    _, _, ork, orv = ref.fill_working_set(ok, ov, i64(R), L.numpy(), W)
    g = torch.Generator().manual_seed(42)
    _say("append 35 tokens")
    for step in range(35):
        kn = (torch.randn((B, H, 128), generator=g) * (1 + step % 4)).to(torch.bfloat16)
        vn = torch.randn((B, H, 128), generator=g).to(torch.bfloat16)
        lib.append_token(d, kn.to(DEV), vn.to(DEV), Ld, summ, wset, kd, vd)
        ok, ov, os_, ork, orv = ref.append_token(ok, ov, os_, ork, orv, f64(kn), f64(vn),
                                                 i64(Ld), W)
        Ld += 1
        torch.cuda.synchronize()
        assert np.array_equal(f64(summ), os_), f"summaries after token {step}"
        assert np.array_equal(f64(wset.ring_k), ork) and np.array_equal(f64(wset.ring_v), orv)
    assert np.array_equal(f64(kd), ok) and np.array_equal(f64(vd), ov)
    rebuilt = lib.build_summaries(d, kd, Ld)
    torch.cuda.synchronize()
    lens = i64(Ld)
    for b in range(B):
        nb = ref.num_blocks(int(lens[b]))
        assert torch.equal(summ[b, :, :nb], rebuilt[b, :, :nb])


@pytest.mark.parametrize("tier", ["device", "host"])
def test_decode_loop_over_the_working_set(lib, tier):
    """Six decode steps, each followed by an appended token: the step over the
    working set (attention from pool and ring, then the plan's copies) gives the
    full-cache overlapped step's outputs bit for bit, and after every step the pool
    holds the next slot table's blocks."""
    w = synth.WORKLOADS["tiny_4k"].with_(batch=3, num_kv_heads=2, fetch_ratio=0.25, ctx=4096 + 40,
                                         min_len=1000)
    _say(f"decode loop over the working set, {tier} tier")
    inp = {kk: t.to(DEV) for kk, t in synth.generate(w, "cpu").items()}
    d = lib.dims_for(w)
    kd, vd, Ld = inp["k"].clone(), inp["v"].clone(), inp["seq_lens"].clone()
    summ = lib.build_summaries(d, kd, Ld)
    n_cand = [ref.first_window_block(int(x), w.window) for x in Ld.cpu()]
    R = torch.stack([torch.stack([synth.random_resident(w.top_k, n_cand[b], 3, 5 * b + h)
                                  for h in range(w.num_kv_heads)]) for b in range(w.batch)]).to(DEV)
    if tier == "host":
        hk, hv = kd.cpu().pin_memory(), vd.cpu().pin_memory()
        src_k, src_v = hk, hv
    else:
        src_k, src_v = kd, vd
    wset = lib.fill_working_set(d, R, Ld, src_k, src_v)
    g = torch.Generator().manual_seed(5)
    for step in range(6):
        rn_pool, rn_full = torch.empty_like(R), torch.empty_like(R)
        pool_out = lib.decode_step_pool(d, inp["q"], summ, src_k, src_v, wset, Ld, R, rn_pool)
        pool_out = {kk: t.clone() for kk, t in pool_out.items()}
        full_out = lib.decode_step_overlapped(d, inp["q"], summ, kd, vd, Ld, R, rn_full)
        torch.cuda.synchronize()
        for key in ("scores", "topk", "plan", "plan_count", "table", "table_count", "out", "lse"):
            assert torch.equal(pool_out[key], full_out[key]), f"step {step}: {key}"
        assert torch.equal(rn_pool, rn_full)
        expect = lib.fill_working_set(d, rn_full, Ld, kd, vd)
        torch.cuda.synchronize()
        assert torch.equal(wset.pool_k, expect.pool_k) and torch.equal(wset.pool_v, expect.pool_v)
        # the next token: into the full cache (both tiers), the ring and the summaries
        kn = torch.randn((w.batch, w.num_kv_heads, 128), generator=g).to(torch.bfloat16).to(DEV)
        vn = torch.randn((w.batch, w.num_kv_heads, 128), generator=g).to(torch.bfloat16).to(DEV)
        lib.append_token(d, kn, vn, Ld, summ, wset, kd, vd)
        if tier == "host":
            lib.append_token(d, kn, vn, Ld, summ.clone(), lib.WorkingSet(d, DEV), hk, hv)
        torch.cuda.synchronize()
        Ld += 1
        R = rn_full
        inp["q"] = torch.randn(inp["q"].shape, generator=g).to(torch.bfloat16).to(DEV)
    if tier == "host":
        assert torch.equal(hk, kd.cpu()) and torch.equal(hv, vd.cpu())


def test_layer_pipelined_copies_match_the_serial_steps(lib):
    """Three layers, three decode steps, the full cache in pinned host memory: with
    the plan's copies on a transfer stream (each layer's next step ordered after its
    copies) every output and every pool equals the one-stream schedule's."""
    w = synth.WORKLOADS["tiny_4k"].with_(batch=2, num_kv_heads=2, fetch_ratio=0.25, ctx=4096 + 40,
                                         min_len=1000)
    _say("layer-pipelined copies vs one stream")
    d = lib.dims_for(w)
    layers = []
    for layer in range(3):
        inp = {kk: t.to(DEV) for kk, t in synth.generate(w, "cpu", layer=layer).items()}
        summ = lib.build_summaries(d, inp["k"], inp["seq_lens"])
        n_cand = [ref.first_window_block(int(x), w.window) for x in inp["seq_lens"].cpu()]
        R = torch.stack([torch.stack([synth.random_resident(w.top_k, n_cand[b], 2, 3 * b + h + layer)
                                      for h in range(w.num_kv_heads)])
                         for b in range(w.batch)]).to(DEV)
        layers.append((inp, summ, R, inp["k"].cpu().pin_memory(), inp["v"].cpu().pin_memory()))

    def run(pipelined):
        fg = torch.cuda.Stream()
        tr = torch.cuda.Stream() if pipelined else None
        steps, done, outs = [], [], []
        with torch.cuda.stream(fg):
            for (inp, summ, R, hk, hv) in layers:
                ws = lib.fill_working_set(d, R, inp["seq_lens"], hk, hv)
                bufs = lib.StepBuffers(d, DEV)
                rn = torch.empty_like(R)
                steps.append((lib.PreparedPoolStep(d, inp["q"], summ, hk, hv, ws, inp["seq_lens"], R,
                                                   bufs, rn), ws, bufs, rn))
                done.append(torch.cuda.Event())
        for t in range(3):
            for li, (st, ws, bufs, rn) in enumerate(steps):
                if pipelined:
                    if t > 0:
                        fg.wait_event(done[li])
                    st(stream=fg, transfer_stream=tr)
                    done[li].record(tr)
                else:
                    st(stream=fg)
                with torch.cuda.stream(fg):
                    outs.append({k: v.clone() for k, v in bufs.as_dict().items()})
        fg.wait_stream(tr) if pipelined else None
        torch.cuda.synchronize()
        pools = [(ws.pool_k.clone(), ws.pool_v.clone()) for (_, ws, _, _) in steps]
        return outs, pools

    serial_outs, serial_pools = run(False)
    pipe_outs, pipe_pools = run(True)
    for i, (a, b) in enumerate(zip(serial_outs, pipe_outs)):
        for key in a:
            assert torch.equal(a[key], b[key]), f"step {i // 3} layer {i % 3}: {key}"
    for (ak, av), (bk, bv) in zip(serial_pools, pipe_pools):
        assert torch.equal(ak, bk) and torch.equal(av, bv)


def test_copy_and_append_edge_cases(lib):
    """Plan rows out of range are skipped and the rest copied; with a cap of 0 the
    copy is a no-op; a sequence at capacity takes no appended token."""
    B, H, G, Q, NB, K, W = 2, 2, 4, 1, 8, 4, 16
    q, k, v, L = _inputs(61, B, H, G, Q, NB, [NB * 16, 50])
    kd, vd, Ld = k.to(DEV), v.to(DEV), L.to(DEV)
    d = lib.make_dims(B, H, G, NB, Q, K, W, 0.5)                    # cap 2
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
    d0 = lib.make_dims(B, H, G, NB, Q, K, W, 0.1)                   # cap 0
    lib.execute_plan(d0, torch.empty((B, H, 0, 3), dtype=torch.int32, device=DEV), count, kd, vd, wset)
    summ = lib.build_summaries(d, kd, Ld)
    s0, r0, k0 = summ.clone(), wset.ring_k.clone(), kd.clone()
    kn = torch.randn((B, H, 128)).to(torch.bfloat16).to(DEV)
    lib.append_token(d, kn, kn, Ld, summ, wset, kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(wset.pool_k, exp_k)
    assert torch.equal(summ[0], s0[0]) and torch.equal(kd[0], k0[0]) and torch.equal(wset.ring_k[0], r0[0])
    assert torch.equal(kd[1, :, 50 // 16, 50 % 16], kn[1])             # the other sequence took it


@pytest.mark.parametrize("tier", ["device", "host"])
def test_step_over_the_working_set_at_the_qwen3_8b_shape(lib, tier):
    """The Qwen3-8B 32K shape (two sequences, all eight KV heads, K = 128, cap 6): the
    step over the working set gives the full-cache overlapped step's outputs bit for
    bit, and its copies leave the pool equal to the gather of the next slot table."""
    w = synth.WORKLOADS["qwen3_8b_32k"].with_(batch=2)
    _say(f"step over the working set at the Qwen3-8B shape, {tier} tier")
    inp = synth.generate(w, DEV)
    d = lib.dims_for(w)
    summ = lib.build_summaries(d, inp["k"], inp["seq_lens"])
    sel = lib.topk_blocks(d, lib.score_summaries(d, inp["q_prev"], summ, inp["seq_lens"]), inp["seq_lens"])
    R = synth.resident_from_selection(w, sel, inp["seq_lens"].cpu()).to(DEV)
    if tier == "host":
        src_k, src_v = inp["k"].cpu().pin_memory(), inp["v"].cpu().pin_memory()
    else:
        src_k, src_v = inp["k"], inp["v"]
    wset = lib.fill_working_set(d, R, inp["seq_lens"], src_k, src_v)
    rn_pool, rn_full = torch.empty_like(R), torch.empty_like(R)
    pool_out = {key: t.clone() for key, t in
                lib.decode_step_pool(d, inp["q"], summ, src_k, src_v, wset, inp["seq_lens"], R, rn_pool).items()}
    full_out = lib.decode_step_overlapped(d, inp["q"], summ, inp["k"], inp["v"], inp["seq_lens"], R, rn_full)
    torch.cuda.synchronize()
    for key in ("scores", "topk", "plan", "plan_count", "table", "table_count", "out", "lse"):
        assert torch.equal(pool_out[key], full_out[key]), key
    assert torch.equal(rn_pool, rn_full)
    assert int(full_out["plan_count"].sum()) > 0
    expect = lib.fill_working_set(d, rn_full, inp["seq_lens"], inp["k"], inp["v"])
    torch.cuda.synchronize()
    assert torch.equal(wset.pool_k, expect.pool_k) and torch.equal(wset.pool_v, expect.pool_v)
    del inp, summ, wset, expect
    torch.cuda.empty_cache()


@pytest.mark.parametrize("shape", [{"group": 16, "num_drafts": 4},   # 80 query rows, 16 query heads
                                   {"group": 8, "num_drafts": 1}])   # 16 query rows, 8 query heads
def test_step_over_the_working_set_at_wider_groups(lib, shape):
    """Wider GQA groups, whose overlapped step also selects inside its first launch: the
    step over the working set (device tier) gives the full-cache step's outputs bit for
    bit, and its copies leave the pool equal to the gather of the next slot table."""
    w = synth.WORKLOADS["qwen3_235b_32k"].with_(batch=2, num_kv_heads=4, ctx=8192 + 40, **shape)
    _say(f"step over the working set, {shape}")
    inp = {kk: t.to(DEV) for kk, t in synth.generate(w, "cpu").items()}
    d = lib.dims_for(w)
    assert lib.overlapped_selects_in_launch1(d)
    summ = lib.build_summaries(d, inp["k"], inp["seq_lens"])
    sel = lib.topk_blocks(d, lib.score_summaries(d, inp["q"], summ, inp["seq_lens"]), inp["seq_lens"])
    R = synth.resident_from_selection(w, sel, inp["seq_lens"].cpu()).to(DEV)
    wset = lib.fill_working_set(d, R, inp["seq_lens"], inp["k"], inp["v"])
    rn_pool, rn_full = torch.empty_like(R), torch.empty_like(R)
    pool_out = {key: t.clone() for key, t in
                lib.decode_step_pool(d, inp["q"], summ, inp["k"], inp["v"], wset, inp["seq_lens"], R,
                                     rn_pool).items()}
    full_out = lib.decode_step_overlapped(d, inp["q"], summ, inp["k"], inp["v"], inp["seq_lens"], R, rn_full)
    torch.cuda.synchronize()
    for key in ("scores", "topk", "plan", "plan_count", "table", "table_count", "out", "lse"):
        assert torch.equal(pool_out[key], full_out[key]), key
    assert torch.equal(rn_pool, rn_full)
    assert int(full_out["plan_count"].sum()) > 0
    expect = lib.fill_working_set(d, rn_full, inp["seq_lens"], inp["k"], inp["v"])
    torch.cuda.synchronize()
    assert torch.equal(wset.pool_k, expect.pool_k) and torch.equal(wset.pool_v, expect.pool_v)
