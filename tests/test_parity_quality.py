"""GPU check of the prediction-quality analysis: the attention shares the analysis
computes on the device equal the oracle's, and the analysis runs end to end.

The analysis is measurement code, not the decode path; its predictions come from
the library's scoring and selection, which test_parity.py holds to the oracle.
"""
import math
import sys

import numpy as np
import pytest
import torch

import bench
from oracle import ref
from tests._helpers import f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(msg):
    print(f"[quality] {msg}", flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("B,H,G,NB,W,lens,bs", [(2, 2, 4, 40, 64, [600, 123], 16), (1, 3, 1, 20, 0, [320], 16),
                                                 (2, 2, 4, 20, 40, [600, 123], 32), (1, 2, 2, 80, 24, [555], 8)])
def test_block_mass_matches_oracle(B, H, G, NB, W, lens, bs):
    _say(f"block mass B={B} H={H} G={G} NB={NB} W={W} bs={bs}")
    g = torch.Generator().manual_seed(9 + G)
    q = torch.randn((B, H, G, 128), generator=g).to(torch.bfloat16)
    k = torch.randn((B, H, NB, bs, 128), generator=g).to(torch.bfloat16)
    L = torch.tensor(lens, dtype=torch.int32)
    scale = 1 / math.sqrt(128)
    got = bench.block_mass_gpu(q.to(DEV), k.to(DEV), L.to(DEV), W, scale, torch)
    torch.cuda.synchronize()
    exp = ref.block_attention_mass(f64(q), f64(k), L.numpy(), W, scale, bs)
    got = f64(got)
    assert np.array_equal(np.isneginf(got), np.isneginf(exp))
    fin = np.isfinite(exp)
    np.testing.assert_allclose(got[fin], exp[fin], rtol=2e-4, atol=1e-9)


@pytest.mark.parametrize("bs", [8, 16, 64])
def test_captured_attention_matches_oracle(bs):
    """The device figure against the oracle's on random selections with -1 pads and
    ids past the candidates (window blocks, past the sequence)."""
    B, H, G, W = 2, 3, 4, 40
    lens = [900, 200]
    NB = -(-max(lens) // bs) + 1
    _say(f"captured attention bs={bs}")
    g = torch.Generator().manual_seed(31 + bs)
    q = torch.randn((B, H, G, 128), generator=g).to(torch.bfloat16)
    k = torch.randn((B, H, NB, bs, 128), generator=g).to(torch.bfloat16)
    L = torch.tensor(lens, dtype=torch.int32)
    r = np.random.default_rng(bs)
    sel = r.integers(-1, NB, size=(B, H, 6))
    for b in range(B):
        for h in range(H):
            row = r.permutation(NB)[:6]
            row[r.random(6) < 0.2] = -1
            sel[b, h] = row
    scale = 1 / math.sqrt(128)
    shares = bench.block_shares_gpu(q.to(DEV), k.to(DEV), L.to(DEV), W, scale, torch)
    got = bench.captured_gpu(shares, torch.from_numpy(sel).to(DEV), L.to(DEV), W, torch)
    torch.cuda.synchronize()
    exp = ref.captured_attention(f64(q), f64(k), L.numpy(), W, scale, sel, bs)
    np.testing.assert_allclose(f64(got), exp, rtol=0, atol=2e-5)


def test_prediction_quality_runs():
    """Two layers of the small workload: every figure is a fraction, and the true
    query's own top-K agrees best with itself among the predictors."""
    _say("prediction quality, small workload")

    class A:
        workload, sets = "tiny_4k", 2

    r = bench.prediction_quality(A())
    assert r["layers"] == 2 and r["top_k"] == 16
    for name, row in r["predictors"].items():
        for key in ("top20_accuracy", "topk_agreement", "top20_min_layer", "topk_min_layer",
                    "agreement_with_true_query_selection"):
            assert 0.0 <= row[key] <= 1.0, (name, key)
    assert r["predictors"]["exact"]["agreement_with_true_query_selection"] == 1.0
    assert r["predictors"]["exact"]["topk_agreement"] >= r["predictors"]["proxy@1.0"]["topk_agreement"]
    assert r["token_budget"] == 256
    by_block = r["captured_attention_by_block_size"]
    assert sorted(by_block, key=int) == ["8", "16", "32", "64"]
    for bs, row in by_block.items():
        assert row["top_k"] == 256 // int(bs)
        assert set(row["captured_attention"]) == {"best possible", "exact", "lookahead@0.3", "proxy@0.3",
                                                  "proxy+lookahead@0.3"}
        for name, v in row["captured_attention"].items():
            assert 0.0 <= v <= 1.0, (bs, name)
