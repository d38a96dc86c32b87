"""Byte accounting of the benchmark, pinned to the pages' worked capacity example."""
import json
import math
import os

import torch

import bench
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_kv_capacity_worked_example():
    with open(os.path.join(GOLDEN, "eq1_kv_capacity.json")) as f:
        ex = json.load(f)
    per_request = bench.kv_cache_bytes(1, ex["context_tokens"], ex["layers"], ex["kv_heads"],
                                       ex["head_dim"], ex["bytes_per_elem"])
    assert round(per_request / 1e9, 1) == ex["printed_gb_per_request"]
    assert math.floor(ex["hbm_bytes_for_kv"] / per_request) == ex["printed_b_max"]


def test_per_block_units_are_one_instance_of_the_capacity_formula():
    # one 16-token block of one KV head of one layer: the capacity formula with B = 1,
    # L = 16, N_layer = 1, N_kv = 1, d_h = 128, s = 2
    assert bench.BLOCK_KV_BYTES == bench.kv_cache_bytes(1, 16, 1, 1, 128, 2)
    # the summary of a block is 1/16 of its K+V bytes
    assert bench.SUMMARY_BYTES * 16 == bench.BLOCK_KV_BYTES


def test_algorithmic_bytes_by_hand():
    w = synth.WORKLOADS["tiny_4k"]
    lens = torch.tensor([4096])
    tc = torch.tensor([[20, 20]])
    nb = bench.algorithmic_bytes(w, lens, tc)
    cand = (4096 - 64) // 16 * 2                           # 252 candidate blocks x 2 heads
    assert nb["units"] == {"candidate_block_heads": cand, "table_blocks": 40}
    q_all = 1 * 2 * 4 * 4 * 256
    out = 1 * 2 * 4 * 129 * 4
    assert nb["step"] == cand * 512 + 40 * 8192 + q_all + out


def test_percentiles_nearest_rank():
    p = bench.percentiles(list(range(1, 11)))           # 1..10
    assert (p["p10"], p["p50"], p["p90"], p["n"]) == (1, 5.5, 9, 10)
    assert bench.percentiles([3.0])["p90"] == 3.0


def test_cpu_baseline_both_modes_on_the_tiny_workload():
    """The oracle timing leg runs on CPU tensors: one core, then the worker pool."""
    import numpy as np

    from oracle import ref
    w = synth.WORKLOADS["tiny_4k"]
    inp = synth.generate(w, "cpu")
    f64 = lambda t: t.to(torch.float64).numpy()
    lens = inp["seq_lens"].numpy()
    summ = ref.build_summaries(f64(inp["k"]), lens)
    resident = torch.full((w.batch, w.num_kv_heads, w.top_k), -1, dtype=torch.int32)
    sets = [{"q": inp["q"], "k": inp["k"], "v": inp["v"], "seq_lens": inp["seq_lens"],
             "summ": torch.from_numpy(summ).to(torch.bfloat16), "resident": resident}]
    out = bench.cpu_baseline(w, sets, budget_s=1.0, overlapped=True)
    assert out["kind"] == "oracle" and out["cores"] == 1 and out["value"] > 0
    assert out["pool"]["value"] > 0 and 1 <= out["pool"]["cores"] <= 16
    assert np.isfinite(out["pool"]["value"])


def test_analysis_overlap_matches_the_oracle_definition():
    import numpy as np

    from oracle import ref
    r = np.random.default_rng(3)
    for _ in range(200):
        n = int(r.integers(1, 12))
        a = r.permutation(30)[: int(r.integers(0, 12))]
        b = r.permutation(30)[: int(r.integers(0, 12))]
        a = np.concatenate([a, -np.ones(3, dtype=int)])
        b = np.concatenate([b, -np.ones(3, dtype=int)])
        assert bench.top_overlap_rows(a, b, n) == ref.top_overlap(a, b, n)


def test_block_bytes_at_every_block_size():
    """K and V of one block is Eq. (1) at one sequence of `block` tokens, one layer, one
    KV head; the summaries stay two rows whatever the block size."""
    import synth
    for block in (8, 16, 32, 64):
        assert bench.block_kv_bytes(block) == bench.kv_cache_bytes(1, block, 1, 1, 128, 2)
    w = synth.WORKLOADS["qwen3_8b_32k"].with_(block=32, top_k=64)
    lens = [32768] * w.batch
    nb = bench.algorithmic_bytes(w, lens, 10)
    cand = (32768 - 128) // 32 * w.batch * w.num_kv_heads
    assert nb["summaries"] == cand * bench.SUMMARY_BYTES
    assert nb["kv"] == 10 * 32 * 128 * 2 * 2


def _counter_csv(path, rows):
    import csv
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for i, (kernel, counter, value) in enumerate(rows):
            wr.writerow({"Dispatch_Id": i, "Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": value})


def test_summarize_counters_scales_by_the_calibration_copy(tmp_path):
    """Bytes per launch of each step kernel = the counter's mean (KiB) x 1024 x the scale
    that makes the 512 MiB calibration copy read (write) 512 MiB; the step's bytes are
    the sum over its kernels; the file carries the sources' hash and reads back."""
    l1 = "void oasis::step_kernel<2, 4, 2, false>(oasis::ScoreArgs, oasis::TopkPlanArgs, oasis::AttnArgs)"
    l2 = "oasis::attn_merge_kernel(float const*, int, int, float*, float*)"
    other = "void oasis::score_kernel<2>(oasis::ScoreArgs)"
    copy = "__amd_rocclr_copyBuffer"
    fetch_dir, write_dir = str(tmp_path / "f"), str(tmp_path / "w")
    _counter_csv(fetch_dir, [(copy, "FETCH_SIZE", 262144.0)] * 3 + [(copy, "FETCH_SIZE", 4.0)]
                 + [(l1, "FETCH_SIZE", 1000.0), (l1, "FETCH_SIZE", 3000.0), (l2, "FETCH_SIZE", 50.0),
                    (other, "FETCH_SIZE", 9e9)])
    _counter_csv(write_dir, [(copy, "WRITE_SIZE", 524288.0)] * 3
                 + [(l1, "WRITE_SIZE", 10.0), (l1, "WRITE_SIZE", 30.0), (l2, "WRITE_SIZE", 4.0)])
    kernels = ("step_kernel", "attn_merge_kernel")
    text = bench.summarize_counters(fetch_dir, write_dir, "qwen3_8b_32k", "cmd", kernels)
    kv = dict(line.split(" = ", 1) for line in text.splitlines() if " = " in line and not line.startswith("#"))
    assert int(kv["step_kernel.fetch_bytes_per_launch"]) == 2000 * 1024 * 2    # mean 2000 KiB, scale 2
    assert int(kv["step_kernel.write_bytes_per_launch"]) == 20 * 1024          # mean 20 KiB, scale 1
    assert int(kv["step_kernel.traffic_bytes_per_launch"]) == 2000 * 1024 * 2 + 20 * 1024
    assert int(kv["attn_merge_kernel.traffic_bytes_per_launch"]) == 50 * 1024 * 2 + 4 * 1024
    assert int(kv["traffic_bytes_per_step"]) == 2000 * 1024 * 2 + 20 * 1024 + 50 * 1024 * 2 + 4 * 1024
    assert kv["sources_sha256"] == bench.kernel_sources_sha256() and kv["workload"] == "qwen3_8b_32k"
    assert kv["kernels"] == "step_kernel,attn_merge_kernel"
    # read back through measured_traffic (the file is written where bench.py looks, then removed)
    path = bench.traffic_file("unit_test_workload")
    assert not os.path.exists(path)
    try:
        with open(path, "w") as f:
            f.write(text.replace("workload = qwen3_8b_32k", "workload = unit_test_workload"))
        got = bench.measured_traffic("unit_test_workload", kernels)
        assert got == {"step_kernel": 2000 * 1024 * 2 + 20 * 1024, "attn_merge_kernel": 50 * 1024 * 2 + 4 * 1024,
                       "per_step": int(kv["traffic_bytes_per_step"])}
        assert bench.measured_traffic("unit_test_workload", ("score_attn_kernel", "select_merge_kernel")) is None
    finally:
        os.remove(path)


def test_kernel_name_matching():
    assert bench.kernel_matches("void oasis::step_kernel<1, 4, 2, true>(oasis::ScoreArgs)", "step_kernel")
    assert bench.kernel_matches("oasis::attn_merge_kernel(float const*, int)", "attn_merge_kernel")
    assert not bench.kernel_matches("void oasis::select_score_attn_kernel<1, 4, 2>(int)", "score_attn_kernel")
    assert not bench.kernel_matches("void oasis::attn_merge_kernel_x<1>(int)", "attn_merge_kernel")


def test_summarize_occupancy_means_per_kernel(tmp_path):
    a, b = str(tmp_path / "a"), str(tmp_path / "b")
    k1 = "void oasis::score_attn_kernel<2, 4, false>(oasis::ScoreArgs, oasis::AttnArgs, int, int, int, int)"
    k2 = "oasis::attn_merge_kernel(float const*, int, int, float*, float*)"
    _counter_csv(a, [(k1, "OccupancyPercent", 20.0), (k1, "OccupancyPercent", 30.0),
                     (k1, "MeanOccupancyPerCU", 8.0), (k2, "OccupancyPercent", 3.0),
                     ("other_kernel", "OccupancyPercent", 99.0)])
    _counter_csv(b, [(k1, "SQ_WAVES", 13056.0), (k2, "MfmaUtil", 0.0)])
    text = bench.summarize_occupancy([a, b], "qwen3_8b_32k", "cmd")
    rows = {line.split("|")[1].strip(): [c.strip() for c in line.split("|")[2:-1]]
            for line in text.splitlines() if line.startswith("| `")}
    assert set(rows) == {"`oasis::score_attn_kernel<2, 4, false>`", "`oasis::attn_merge_kernel`"}
    r1 = rows["`oasis::score_attn_kernel<2, 4, false>`"]
    assert r1[0] == "2" and r1[1] == "25.0" and r1[2] == "8.0" and r1[5] == "13056.0"
    r2 = rows["`oasis::attn_merge_kernel`"]
    assert r2[1] == "3.0" and r2[3] == "0.0"


def test_empty_timed_region_is_refused(capsys):
    """No timed step (or a negative warm-up, or an empty graph) ends with a message and
    status 2 before any device work."""
    for argv in (["--steps", "0"], ["--warmup", "-1"], ["--graph-steps", "0"]):
        assert bench.main(argv) == 2
        assert "--steps >= 1" in capsys.readouterr().err


def test_more_than_one_gpu_is_refused(capsys, monkeypatch):
    """--gpus above 1 (or a multi-rank launch) ends with a message and status 2 before any
    device work: no multi-GPU path is built."""
    assert bench.main(["--gpus", "2"]) == 2
    assert "exactly one GPU" in capsys.readouterr().err
    monkeypatch.setenv("WORLD_SIZE", "8")
    assert bench.main([]) == 2
