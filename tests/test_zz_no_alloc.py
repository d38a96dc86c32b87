"""oasis_decode_step_overlapped_noalloc (the step with the library's own scratch array as
its workspace, for callers that cannot allocate) against oasis_decode_step_overlapped
with a workspace of its own: two calls in a row on one GPU, the second smaller, then
the first shape again (the array keeps what the last call left, other dims included).
Integer outputs bit-exact, floating point within the parity tolerances."""
import sys

import numpy as np
import pytest
import torch

import synth
from tests._helpers import OUT_ATOL, SCORE_RTOL, f64, i64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(msg):
    print(f"[no-alloc] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import oasis_score_summaries_amd as oa
    oa.load()
    return oa


def _case(oa, w):
    d = oa.dims_for(w)
    assert oa.workspace_bytes(d) <= 16 << 20
    inp = synth.generate(w, DEV)
    summ = oa.build_summaries(d, inp["k"], inp["seq_lens"])
    sel = oa.topk_blocks(d, oa.score_summaries(d, inp["q"], summ, inp["seq_lens"]), inp["seq_lens"])
    resident = synth.resident_from_selection(w, sel, inp["seq_lens"].cpu()).to(DEV)
    return d, inp, summ, resident


def _compare(oa, w, label):
    d, inp, summ, resident = _case(oa, w)
    args = (d, inp["q"], summ, inp["k"], inp["v"], inp["seq_lens"], resident)
    rn_ref, rn_new = torch.empty_like(resident), torch.empty_like(resident)
    exp = oa.decode_step_overlapped(*args, rn_ref, buffers=oa.StepBuffers(d, DEV))
    got = oa.decode_step_overlapped_noalloc(*args, rn_new, outputs=oa.StepBuffers(d, DEV))
    torch.cuda.synchronize()
    _say(f"{label}: compared")
    for key in ("topk", "plan", "plan_count", "table", "table_count"):
        np.testing.assert_array_equal(i64(got[key]), i64(exp[key]), err_msg=f"{label}: {key}")
    np.testing.assert_array_equal(i64(rn_new), i64(rn_ref), err_msg=f"{label}: resident_next")
    es, gs = f64(exp["scores"]), f64(got["scores"])
    fin = np.isfinite(es)
    np.testing.assert_array_equal(np.isfinite(gs), fin, err_msg=f"{label}: scores finiteness")
    np.testing.assert_allclose(gs[fin], es[fin], rtol=SCORE_RTOL, atol=0, err_msg=f"{label}: scores")
    np.testing.assert_allclose(f64(got["out"]), f64(exp["out"]), rtol=0, atol=OUT_ATOL, err_msg=f"{label}: out")
    np.testing.assert_allclose(f64(got["lse"]), f64(exp["lse"]), rtol=0, atol=OUT_ATOL, err_msg=f"{label}: lse")


def test_noalloc_step_matches_the_workspace_step(lib):
    big = synth.WORKLOADS["qwen3_8b_32k"]
    small = synth.WORKLOADS["tiny_4k"].with_(batch=2, fetch_ratio=0.25)
    _say("call 1: Qwen3-8B 32K layer shape")
    _compare(lib, big, "qwen3_8b_32k")
    _say("call 2: smaller input (tiny 4K, batch 2)")
    _compare(lib, small, "tiny_4k")
    _say("call 3: the first shape again")
    _compare(lib, big.with_(batch=2), "qwen3_8b_32k batch 2")
