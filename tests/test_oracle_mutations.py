"""The oracle's pins catch plausible mistakes: each mutation below plants one
mistake in a copy of the oracle's source (the original file is untouched),
and at least one pin of tests/test_oracle.py must then fail.  The unmutated
copy passes every pin used here, so a failure is the mistake's doing."""

import os
import sys
import types

import numpy as np
import pytest

from tests import test_oracle as TO

ORACLE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "oracle", "fsdp_oracle.py")

# name -> [(source fragment, its replacement), ...]; every fragment occurs once
MUTATIONS = {
    "sum instead of average": [("    return acc / np.float32(len(values))", "    return acc")],
    "times 1/R instead of divided by R": [
        ("    return acc / np.float32(len(values))",
         "    return acc * (np.float32(1) / np.float32(len(values)))")],
    "reversed rank order in the sum": [
        ("    acc = _as_f32(values[0]).copy()\n    for q in range(1, len(values)):\n"
         "        acc = acc + _as_f32(values[q])",
         "    acc = _as_f32(values[-1]).copy()\n    for q in range(len(values) - 2, -1, -1):\n"
         "        acc = acc + _as_f32(values[q])")],
    "floor split per parameter": [("        k = (d0 + R - 1) // R          # shard size rounded up",
                                   "        k = max(1, d0 // R)")],
    "floor split of the FlatParameter": [
        ("    pl.S = soff if layout == PER_PARAM else (off + R - 1) // R",
         "    pl.S = soff if layout == PER_PARAM else max(1, off // R)")],
    "padding not zero": [("    shards = np.zeros((pl.R, pl.S), dtype=full.dtype)",
                          "    shards = np.ones((pl.R, pl.S), dtype=full.dtype)")],
    "gather in reverse rank order": [("            valid = [b for b in blocks if b.size > 0]",
                                      "            valid = [b for b in blocks[::-1] if b.size > 0]")],
    "eps inside the square root": [
        ("    p2 = p1 - lr * m_hat / (np.sqrt(v_hat) + eps)",
         "    p2 = p1 - lr * m_hat / np.sqrt(v_hat + eps)")],
    "L2 (coupled) weight decay": [
        ("    p1 = p * (1.0 - lr * weight_decay)", "    p1 = p"),
        ("    g = np.asarray(g, np.float64)", "    g = np.asarray(g, np.float64) + weight_decay * p")],
    "no bias correction": [("    m_hat = m1 / (1.0 - beta1 ** t)", "    m_hat = m1"),
                           ("    v_hat = v1 / (1.0 - beta2 ** t)", "    v_hat = v1")],
    "swapped betas": [("    m1 = beta1 * m + (1.0 - beta1) * g", "    m1 = beta2 * m + (1.0 - beta2) * g"),
                      ("    v1 = beta2 * v + (1.0 - beta2) * g * g",
                       "    v1 = beta1 * v + (1.0 - beta1) * g * g")],
    "second moment of g, not g squared": [
        ("    v1 = beta2 * v + (1.0 - beta2) * g * g", "    v1 = beta2 * v + (1.0 - beta2) * g")],
    "truncating bf16 recast": [("    r = hi + up.astype(np.uint32)", "    r = hi")],
    "bf16 ties away from zero": [
        ("    up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & np.uint32(1)) == 1))",
         "    up = lo >= 0x8000")],
    "bf16 widening drops the sign": [
        ("    return (u16.astype(np.uint32) << np.uint32(16)).view(np.float32)",
         "    return ((u16 & np.uint16(0x7FFF)).astype(np.uint32) << np.uint32(16)).view(np.float32)")],
    "one all-gather per step when resharding after forward": [
        ("    n_ag = 2 if reshard_after_forward else 1", "    n_ag = 1")],
    "R instead of R - 1 in the reduce-scatter ledger": [
        ("    return dict(all_gather=n_ag * ag, reduce_scatter=(pl.R - 1) * pl.S,\n"
         "                optimizer=0, total=n_ag * ag + (pl.R - 1) * pl.S)",
         "    return dict(all_gather=n_ag * ag, reduce_scatter=pl.R * pl.S,\n"
         "                optimizer=0, total=n_ag * ag + pl.R * pl.S)")],
    "ring all-reduce volume without its factor 2": [
        ("    return 2.0 * (R - 1) / R * P", "    return (R - 1) / R * P")],
    "12 instead of 16 state bytes per element": [("    return 16 * pl.S", "    return 12 * pl.S")],
    "peak without the prefetch buffer": [
        ("    return state_total / R + largest_group + prefetch",
         "    return state_total / R + largest_group")],
    "re-shard keeps the old plan": [("    return shard_pack(pl_to, full)",
                                     "    return shard_pack(pl_from, full)")],
    "accumulation skips the first micro-batch": [
        ("    acc = _as_f32(micro_grads[0]).copy()",
         "    acc = np.zeros_like(_as_f32(micro_grads[0]))")],
    "accumulation keeps only the last micro-batch": [
        ("        acc = acc + _as_f32(g)", "        acc = _as_f32(g).copy()")],
    "all-reduce sums instead of averaging": [
        ("    mean = rank_order_mean(grads)",
         "    mean = rank_order_mean(grads) * np.float32(len(grads))")],
}

# The pins run against each mutant, cheapest first: (test function, kwargs).
PINS = [
    (TO.test_walkthrough_toy_shards_gather_rs_and_comm, {}),
    (TO.test_fsdp2_eight_element_hand_calculation, {}),
    (TO.test_fsdp2_exercise_sum_and_mean, {}),
    (TO.test_ceil_split_closed_forms_r3, {}),
    (TO.test_per_param_shard_sizes_match_row_counts, {}),
    (TO.test_block_layout_flat_offsets_and_send_volume, {}),
    (TO.test_memory_accounting_exercise_and_16_bytes, {}),
    (TO.test_block_layout_fsdp2_table_and_rows, {}),
    (TO.test_reduce_scatter_division_correctly_rounded_r3, {}),
    (TO.test_adamw_closed_form_first_step_and_zero_grad, {}),
    (TO.test_adamw_matches_torch_adamw_float64, {"t": 10}),
    (TO.test_bf16_rne_exact_rational_on_edge_cases, {}),
    (TO.test_bf16_to_f32_over_every_bf16_pattern, {}),
    (TO.test_brute_force_layout_pack_gather, {"R": 3, "layout": "per_param"}),
    (TO.test_brute_force_layout_pack_gather, {"R": 8, "layout": "flat"}),
    (TO.test_brute_force_reduce_scatter, {"R": 5}),
    (TO.test_reshard_block_r4_to_r2_matches_the_page_row_table, {}),
    (TO.test_reshard_brute_force_roundtrip_and_layout_change, {"Ra": 3, "Rb": 2}),
    (TO.test_grad_accumulate_order_and_single_micro_batch, {}),
    (TO.test_allreduce_is_gather_of_reduce_scatter_and_ddp_volume, {}),
]


def load_variant(pairs):
    """A fresh module from the oracle's source with `pairs` applied."""
    with open(ORACLE) as f:
        src = f.read()
    for old, new in pairs:
        assert src.count(old) == 1, f"fragment not found exactly once: {old!r}"
        src = src.replace(old, new)
    name = "fsdp_oracle_variant"
    mod = types.ModuleType(name)
    mod.__file__ = ORACLE
    sys.modules[name] = mod       # dataclasses resolve annotations through it
    try:
        exec(compile(src, ORACLE, "exec"), mod.__dict__)
    finally:
        del sys.modules[name]
    return mod


def first_failing_pin(module, monkeypatch):
    monkeypatch.setattr(TO, "O", module)
    for fn, kwargs in PINS:
        try:
            with np.errstate(all="ignore"):
                fn(**kwargs)
        except Exception as e:     # an assertion, or the mistake breaking a shape
            return f"{fn.__name__}{kwargs or ''}: {type(e).__name__}"
    return None


def test_the_unmutated_copy_passes_every_pin(monkeypatch):
    assert first_failing_pin(load_variant([]), monkeypatch) is None


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_each_planted_mistake_fails_a_pin(name, monkeypatch):
    caught = first_failing_pin(load_variant(MUTATIONS[name]), monkeypatch)
    assert caught is not None, f"no pin fails with the mistake: {name}"
