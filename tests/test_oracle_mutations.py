"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that the pins catch each.

Each mutation edits one line of the oracle's source, loads the edited copy as a
separate module, points the pin tests at it and expects at least one of them
to fail.  The oracle file itself is never modified.
"""
import inspect
import types

import pytest

import oracle.ref as ref_mod
from tests import test_oracle as pins

MUTATIONS = {
    "score_swaps_min_and_max": ("kmin = summ[b, h, :n_cand, 0, :]", "kmin = summ[b, h, :n_cand, 1, :]"),
    "score_takes_min_of_products": ("bound = np.maximum(lo, hi).sum(axis=-1)", "bound = np.minimum(lo, hi).sum(axis=-1)"),
    "score_averages_rows": ("s[b, h, :n_cand] = bound.max(axis=0)", "s[b, h, :n_cand] = bound.mean(axis=0)"),
    "topk_ties_prefer_high_index": ("order = np.lexsort((idx, -s))", "order = np.lexsort((-idx, -s))"),
    "window_one_block_late": ("return max(0, (int(seq_len) - int(window)) // block)",
                              "return max(0, (int(seq_len) - int(window)) // block + 1)"),
    "plan_admits_worst_first": ("admit = admit[:n]", "admit = admit[::-1][:n]"),
    "plan_stale_tie_low_index": ("stale.sort(key=lambda i: (s[int(res[i])], -int(res[i])))",
                                 "stale.sort(key=lambda i: (s[int(res[i])], int(res[i])))"),
    "plan_evicts_best_stale": ("stale.sort(key=lambda i: (s[int(res[i])], -int(res[i])))",
                               "stale.sort(key=lambda i: (-s[int(res[i])], -int(res[i])))"),
    "plan_pairs_unsorted": ("zip(sorted(victims), sorted(admit))", "zip(victims, admit)"),
    "plan_ignores_cap": ("n = min(cap, len(admit))", "n = len(admit)"),
    "plan_frees_stale_before_empty": ("victims = (empty + stale)[:n]", "victims = (stale + empty)[:n]"),
    "attention_lse_drops_max": ("lse[b, h, g] = m + math.log(den)", "lse[b, h, g] = math.log(den)"),
    "summaries_read_past_length": ("n_valid = min(bs, L - j * bs)", "n_valid = bs"),
    "attention_drops_scale": ("z = (kt @ q[b, h, g, 0, :]) * scale", "z = (kt @ q[b, h, g, 0, :])"),
    "attention_uses_a_draft": ("z = (kt @ q[b, h, g, 0, :]) * scale", "z = (kt @ q[b, h, g, 1, :]) * scale"),
    "attention_ignores_length": ("if j * block + t < L]", "if True]"),
    "table_drops_window": ("entries = [int(x) for x in r if 0 <= x < w0] + list(range(w0, nb))",
                           "entries = [int(x) for x in r if 0 <= x < w0]"),
    "plan_table_keeps_window_blocks": ("entries = [int(x) for x in r if 0 <= x < w0] + list(range(w0, nb))",
                                       "entries = [int(x) for x in r if x >= 0] + list(range(w0, nb))"),
    "cap_rounds_to_nearest": ("return int(math.floor(float(fetch_ratio) * int(top_k) + 1e-9))",
                              "return int(round(float(fetch_ratio) * int(top_k)))"),
    "resident_table_keeps_window_blocks": (
        "entries = [int(x) for x in resident[b, h] if 0 <= x < w0] + list(range(w0, nb))",
        "entries = [int(x) for x in resident[b, h] if x >= 0] + list(range(w0, nb))"),
    "overlapped_attends_next_set": (
        "table, tcount = resident_table(resident, seq_lens, window, block)",
        "table, tcount = resident_table(build_plan(score_blocks(q, summ, seq_lens, window, block), "
        "topk_blocks(score_blocks(q, summ, seq_lens, window, block), seq_lens, top_k, window, block), "
        "resident, seq_lens, cap, window, block)['resident'], seq_lens, window, block)"),
    "ring_slot_shifted": ("ring_k[b, h, j % WB] = k[b, h, j]", "ring_k[b, h, (j + 1) % WB] = k[b, h, j]"),
    "ring_one_slot_short": ("return -(-int(window) // block) + 1", "return -(-int(window) // block)"),
    "plan_copies_evicted_block": ("slot, new = int(plan[b, h, i, 0]), int(plan[b, h, i, 1])",
                                  "slot, new = int(plan[b, h, i, 0]), int(plan[b, h, i, 2])"),
    "append_never_reopens_block": ("            if t == 0:\n                summ[b, h, j, 0] = k_new[b, h]",
                                   "            if False:\n                summ[b, h, j, 0] = k_new[b, h]"),
    "append_writes_wrong_ring_slot": ("ring_k[b, h, j % WB, t] = k_new[b, h]",
                                      "ring_k[b, h, (j + 1) % WB, t] = k_new[b, h]"),
    "pool_attention_keeps_window_slots": ("if 0 <= int(resident[b, h, s]) < w0:",
                                          "if 0 <= int(resident[b, h, s]):"),
    "pool_attention_reads_whole_last_block": ("n = min(block, L - j * block)", "n = block"),
    "mass_omits_scale": ("z = flat[h] @ q_true[b, h, g] * scale", "z = flat[h] @ q_true[b, h, g]"),
    "mass_normalised_over_candidates_only": ("p /= p.sum()", "p /= p[: n_cand * bs].sum()"),
    "mass_sums_over_the_group": ("best = np.maximum(best, per_block)",
                                 "best = np.where(np.isinf(best), per_block, best + per_block)"),
    "window_assumes_16_token_blocks": ("return max(0, (int(seq_len) - int(window)) // block)",
                                       "return max(0, (int(seq_len) - int(window)) // 16)"),
    "block_count_assumes_16_tokens": ("return (int(seq_len) + block - 1) // block",
                                      "return (int(seq_len) + 15) // 16"),
    "attention_assumes_16_token_blocks": ("for t in range(block) if j * block + t < L]",
                                          "for t in range(min(block, 16)) if j * block + t < L]"),
    "summaries_stride_assumes_16": ("n_valid = min(bs, L - j * bs)", "n_valid = min(bs, L - j * 16)"),
    "captured_over_all_attention": ("fractions.append(per_block[sel].sum() / per_block.sum())",
                                    "fractions.append(per_block[sel].sum())"),
    "captured_best_of_the_group": ("out[b, h] = float(np.mean(fractions))", "out[b, h] = float(np.max(fractions))"),
    "captured_counts_window_blocks": ("for j in selection[b, h] if 0 <= j < n_cand]",
                                      "for j in selection[b, h] if 0 <= j < NB]"),
    "overlap_divides_by_union": ("return 1.0 if m == 0 else len(a & b) / m",
                                 "return 1.0 if m == 0 else len(a & b) / len(a | b)"),
}

# The slowest pins (seconds each) are left out: every planted plan mistake is also
# caught by the smaller exhaustive plan pin.
PIN_TESTS = [getattr(pins, n) for n in dir(pins)
             if n.startswith("test_") and n not in ("test_decode_step_tiny_workload",
                                                    "test_plan_exhaustive_k4_over_12_candidates")]


def _run_pins(mutant, monkeypatch) -> bool:
    """True if some pin fails against ``mutant``."""
    monkeypatch.setattr(pins, "ref", mutant)
    for t in PIN_TESTS:
        params = inspect.signature(t).parameters
        if "distinct" in params:
            variants = [{"distinct": True}, {"distinct": False}]
        elif "cap" in params:
            variants = [{"cap": 0}, {"cap": 4}]
        elif "window" in params:
            variants = [{"window": 0}, {"window": 40}, {"window": 64}]
        elif "block" in params:
            variants = [{"block": 8}, {"block": 32}]
        else:
            variants = [{}]
        for kw in variants:
            try:
                t(**kw)
            except Exception:
                return True
    return False


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, monkeypatch):
    src = inspect.getsource(ref_mod)
    old, new = MUTATIONS[name]
    assert src.count(old) >= 1, name
    mutant = types.ModuleType("oracle_mutant_" + name)
    exec(compile(src.replace(old, new), "<mutant " + name + ">", "exec"), mutant.__dict__)
    assert _run_pins(mutant, monkeypatch), f"mutation {name} went unnoticed"


def test_unmutated_oracle_passes(monkeypatch):
    assert not _run_pins(ref_mod, monkeypatch)
