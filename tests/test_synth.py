"""The seeded input generator: determinism, shapes, and the stated recipes."""
import numpy as np
import torch

import synth


def test_shapes_and_determinism():
    w = synth.WORKLOADS["tiny_4k"]
    a = synth.generate(w, "cpu")
    b = synth.generate(w, "cpu")
    for key in ("q", "k", "v", "seq_lens", "planted"):
        assert torch.equal(a[key], b[key]), key
    B, H, G, Q, NB = w.batch, w.num_kv_heads, w.group, w.queries, w.max_blocks
    assert a["q"].shape == (B, H, G, Q, 128) and a["q"].dtype == torch.bfloat16
    assert a["k"].shape == (B, H, NB, 16, 128) and a["k"].dtype == torch.bfloat16
    assert a["seq_lens"].dtype == torch.int32 and int(a["seq_lens"][0]) == 4096
    assert w.cap == 0 and w.table_stride == 16 + 5


def test_layers_and_seeds_are_independent():
    w = synth.WORKLOADS["tiny_4k"]
    a = synth.generate(w, "cpu", layer=0, with_kv=False)
    b = synth.generate(w, "cpu", layer=1, with_kv=False)
    c = synth.generate(w.with_(seed=1), "cpu", layer=0, with_kv=False)
    assert not torch.equal(a["q"], b["q"]) and not torch.equal(a["q"], c["q"])


def test_draft_noise_and_planting():
    w = synth.WORKLOADS["tiny_4k"].with_(batch=2, num_kv_heads=4, ctx=2048 + 64)
    inp = synth.generate(w, "cpu")
    q = inp["q"].float()
    diff = q[:, :, :, 1:, :] - q[:, :, :, :1, :]
    assert abs(diff.std().item() - 0.3) < 0.02
    planted = inp["planted"]
    n_cand = synth.first_window_block(int(inp["seq_lens"][0]), w.window)
    assert torch.all(planted.sum(-1) == w.planted)
    assert not planted[..., n_cand:].any()
    # a planted block's keys are shifted by 2 along a unit direction, so its mean key
    # has norm ~ sqrt(4 + 128/16) = 3.46 against ~ sqrt(128/16) = 2.83 for the others
    k = inp["k"].float().mean(dim=3)              # [B, H, NB, d]
    norms = k.norm(dim=-1)
    assert norms[planted].mean() > norms[~planted].mean() + 0.4


def test_heavy_tail_and_lengths():
    w = synth.WORKLOADS["qwen3_235b_32k"].with_(batch=2, ctx=1024 + 128, num_kv_heads=2)
    inp = synth.generate(w, "cpu", with_kv=False)
    n_cand = synth.first_window_block(int(inp["seq_lens"][0]), w.window)
    assert inp["planted"][..., :n_cand].all() and not inp["planted"][..., n_cand:].any()
    r = synth.WORKLOADS["reasoning_36l"]
    lens = synth.seq_lens(r)
    assert lens.shape == (64,) and int(lens.min()) >= 8192 and int(lens.max()) <= 16384
    assert len(set(lens.tolist())) > 32


def test_resident_from_selection_recipes():
    w = synth.WORKLOADS["tiny_4k"].with_(batch=2, num_kv_heads=3, top_k=8, resident="swap", resident_swaps=3)
    lens = torch.tensor([4096, 300], dtype=torch.int32)
    sel = torch.full((2, 3, 8), -1, dtype=torch.int32)
    sel[0] = torch.tensor([50, 3, 9, 100, 7, 21, 60, 2])
    sel[1, :, :5] = torch.tensor([11, 0, 4, 12, 7])        # 14 candidates (300 tokens, W 64)
    r = synth.resident_from_selection(w, sel, lens)
    for b in range(2):
        n_cand = synth.first_window_block(int(lens[b]), w.window)
        for h in range(3):
            s = set(x for x in sel[b, h].tolist() if x >= 0)
            rr = [x for x in r[b, h].tolist() if x >= 0]
            assert len(rr) == len(s) and len(set(rr)) == len(rr)
            assert all(0 <= x < n_cand for x in rr)
            assert len(set(rr) - s) == min(3, len(s), n_cand - len(s))
    # the "prev" recipe keeps the selection, ascending, empties last
    r = synth.resident_from_selection(w.with_(resident="prev"), sel, lens)
    assert r[1, 0].tolist() == [0, 4, 7, 11, 12, -1, -1, -1]


def test_random_scores_distinct():
    s = synth.random_scores((4, 2048), seed=3)
    assert s.dtype == torch.float32 and torch.unique(s).numel() == s.numel()


def test_block_sizes_shapes_planting_and_resident_sets():
    """At 8-, 32- and 64-token blocks: K/V carry blocks of that size, planted blocks sit
    among that size's candidates, and a resident set built from a selection holds
    distinct candidate blocks only."""
    for bs in (8, 32, 64):
        w = synth.WORKLOADS["tiny_4k"].with_(block=bs, batch=2, ctx=2048 + 40, min_len=1000,
                                             top_k=max(4, 256 // bs), planted=6)
        inp = synth.generate(w, "cpu")
        NB = w.max_blocks
        assert NB == -(-(2048 + 40) // bs)
        assert inp["k"].shape == (2, w.num_kv_heads, NB, bs, 128)
        assert inp["v"].shape == inp["k"].shape
        assert w.table_stride == w.top_k + -(-w.window // bs) + 1
        for b in range(2):
            n_cand = synth.first_window_block(int(inp["seq_lens"][b]), w.window, bs)
            assert not inp["planted"][b, :, n_cand:].any()
            assert torch.all(inp["planted"][b].sum(-1) == min(w.planted, n_cand))
        sel = torch.stack([torch.stack([torch.arange(w.top_k, dtype=torch.int32) * 2
                                        for _ in range(w.num_kv_heads)]) for _ in range(2)])
        res = synth.resident_from_selection(w.with_(resident="swap", resident_swaps=1), sel,
                                            inp["seq_lens"])
        for b in range(2):
            n_cand = synth.first_window_block(int(inp["seq_lens"][b]), w.window, bs)
            r = res[b]
            assert torch.all((r == -1) | ((r >= 0) & (r < n_cand)))
            for h in range(w.num_kv_heads):
                vals = [int(x) for x in r[h] if x >= 0]
                assert len(vals) == len(set(vals))
