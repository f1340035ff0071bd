"""Pins of the split-planner oracle: the pages' worked wave example, a
brute-force scheduler, exhaustive checks of the wave condition and
hand-derived plans."""

import json
import os

import pytest

import oracle
from oracle import planner as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_pages_wave_example():
    g = _load("wave_example.json")
    S = g["num_sms"]
    for case in g["cases"]:
        total = sum(oracle.waves(c, num_cus=S, ctas_per_cu=g["ctas_per_sm"]) for c in case["ctas"])
        assert total == case["total_waves"], case["what"]
        for c, fill in zip(case["ctas"], case["wave_fill"]):
            assert sum(fill) == c and len(fill) == oracle.waves(c, num_cus=S)
            assert all(f == S for f in fill[:-1]) and 0 < fill[-1] <= S
            assert oracle.simulate_waves(c, S) == len(fill)


def test_pages_split_rule_constants():
    g = _load("split_rule.json")
    assert tuple(g["offsets"]) == oracle.DEFAULT_OFFSETS
    # offset must stay below half: T = 128, half = 64.  Without the guard the
    # offset 64 would "split" into 128 + 0 tokens and pass the wave check.
    p = oracle.split_plan(128, num_cus=32, offsets=[64])
    assert p["reason"] == oracle.REASON_NO_FEASIBLE_OFFSET
    p = oracle.split_plan(128, num_cus=32)   # 128 CTAs on 32 CUs: 4 waves
    assert p["reason"] == oracle.REASON_SPLIT and p["offset"] == 0
    # the per-model thresholds gate splitting
    for thr in g["min_split_tokens"].values():
        assert oracle.split_plan(thr - 1, min_split_tokens=thr)["reason"] == oracle.REASON_BELOW_THRESHOLD
        assert oracle.split_plan(thr, min_split_tokens=thr)["reason"] != oracle.REASON_BELOW_THRESHOLD


def test_simulated_scheduler_equals_ceil_formula():
    for S in range(1, 9):
        for C in range(0, 65):
            assert oracle.simulate_waves(C, S) == oracle.waves(C, num_cus=S), (C, S)
    for S, cpc in ((3, 2), (4, 3)):
        for C in range(0, 40):
            assert oracle.simulate_waves(C, S * cpc) == oracle.waves(C, num_cus=S, ctas_per_cu=cpc)


def test_ctas_tile_model():
    assert oracle.ctas(0, 256, 32) == 0
    assert oracle.ctas(1, 256, 32) == 32
    assert oracle.ctas(4096, 256, 32) == 512
    assert oracle.waves(4096, 256, 32, 256, 1) == 2
    assert oracle.waves(1024, 256, 32, 256, 1) == 1


@pytest.mark.parametrize("T,S,want", [
    (257, 256, (128, 129, 0)),
    (300, 256, (150, 150, 0)),
    (512, 256, (256, 256, 0)),
    (513, 256, (256, 257, 0)),
    (514, 256, (321, 193, 64)),     # 257/257 is 2+2 waves > 3; 321/193 is 2+1
    (600, 256, (364, 236, 64)),
    (300, 132, (214, 86, 64)),      # the pages' example under the half+offset rule
])
def test_hand_derived_plans(T, S, want):
    p = oracle.split_plan(T, num_cus=S)
    assert (p["prefix_tokens"], p["suffix_tokens"], p["offset"]) == want
    assert p["reason"] == oracle.REASON_SPLIT
    assert p["waves_prefix"] + p["waves_suffix"] == p["waves_unsplit"]


def test_hand_derived_no_split_cases():
    for T in (1, 100, 256):
        p = oracle.split_plan(T, num_cus=256)
        assert p["reason"] == oracle.REASON_SINGLE_WAVE and p["prefix_tokens"] == T
        assert p["suffix_tokens"] == 0 and p["offset"] == -1
    for T in (393, 394, 395, 396):   # every offset leaves 4 waves on 132 SMs
        assert oracle.split_plan(T, num_cus=132)["reason"] == oracle.REASON_NO_FEASIBLE_OFFSET
    p = oracle.split_plan(0)
    assert p["reason"] == oracle.REASON_EMPTY and p["prefix_tokens"] == 0


def test_plan_is_smallest_feasible_offset_exhaustive():
    # Independent re-derivation with the simulated scheduler for every T.
    for S in (132, 256, 7):
        for T in range(1, 601):
            p = oracle.split_plan(T, num_cus=S)
            W = oracle.simulate_waves(T, S)
            assert p["waves_unsplit"] == W
            feasible = [o for o in oracle.DEFAULT_OFFSETS
                        if o < T // 2 and oracle.simulate_waves(T // 2 + o, S)
                        + oracle.simulate_waves(T - T // 2 - o, S) <= W]
            if W <= 1:
                assert p["reason"] == oracle.REASON_SINGLE_WAVE
            elif feasible:
                assert p["reason"] == oracle.REASON_SPLIT and p["offset"] == feasible[0]
                assert p["prefix_tokens"] + p["suffix_tokens"] == T
                # half + off and T - half - off: the odd token goes to the suffix
                assert p["prefix_tokens"] - p["suffix_tokens"] == 2 * p["offset"] - T % 2
                assert p["waves_prefix"] + p["waves_suffix"] == W
            else:
                assert p["reason"] == oracle.REASON_NO_FEASIBLE_OFFSET


def test_plan_counts_over_1_to_600():
    def tally(S):
        c = {}
        for T in range(1, 601):
            p = oracle.split_plan(T, num_cus=S)
            key = p["offset"] if p["reason"] == 0 else ("r", p["reason"])
            c[key] = c.get(key, 0) + 1
        return c
    assert tally(256) == {("r", 2): 256, 0: 257, 64: 87}
    assert tally(132) == {("r", 2): 132, 0: 266, 64: 198, ("r", 3): 4}


def test_odd_token_count_keeps_every_token():
    p = oracle.split_plan(1001, num_cus=100)
    assert p["prefix_tokens"] + p["suffix_tokens"] == 1001


def test_custom_offsets_and_tiles():
    p = oracle.split_plan(4096, tokens_per_cta=256, ctas_per_token_tile=32, num_cus=256,
                          min_split_tokens=1024)
    assert (p["prefix_tokens"], p["suffix_tokens"], p["offset"], p["waves_unsplit"]) == (2048, 2048, 0, 2)
    p = oracle.split_plan(514, num_cus=256, offsets=[0, 10, 100])
    assert p["offset"] == 10 and p["prefix_tokens"] == 267


# A per-shape table as the offline sweep of one layer step fills it (the
# fastest offset per token count, -1 for the whole batch): the layer GEMM of a
# Llama-3-70B-shaped rank, 256 x 256 tiles, 32 across h = 8192, 256 CUs,
# threshold 1024.  Any table is a valid input; this one has entries of every
# kind.
MEASURED_SWEEP = {1024: -1, 1536: -1, 2048: -1, 2560: -1, 3072: -1, 3584: -1, 4096: -1,
                  4608: -1, 5120: 512, 5632: 128, 6144: -1, 6656: 192, 7168: 256, 7680: 256,
                  8192: -1}
SWEEP_MODEL = dict(tokens_per_cta=256, ctas_per_token_tile=32, num_cus=256, ctas_per_cu=1,
                   min_split_tokens=1024)


# Under that model a wave is 2048 rows: waves(M) = ceil(ceil(M / 256) * 32 / 256)
# = ceil(M / 2048).  Derived by hand: (prefix, suffix, waves_unsplit,
# waves_prefix, waves_suffix, reason).
@pytest.mark.parametrize("T,want", [
    (1024, (1024, 0, 1, 1, 0, P.REASON_SINGLE_WAVE)),    # one wave: the table is not read
    (2048, (2048, 0, 1, 1, 0, P.REASON_SINGLE_WAVE)),
    (2560, (2560, 0, 2, 2, 0, P.REASON_MEASURED_UNSPLIT)),
    (4608, (4608, 0, 3, 3, 0, P.REASON_MEASURED_UNSPLIT)),
    (5120, (3072, 2048, 3, 2, 1, P.REASON_MEASURED_SPLIT)),     # 2560 + 512 | 2048
    (5632, (5632, 0, 3, 3, 0, P.REASON_MEASURED_OVER_WAVES)),   # 2944 | 2688: 2 + 2 > 3
    (6656, (3520, 3136, 4, 2, 2, P.REASON_MEASURED_SPLIT)),
    (7168, (3840, 3328, 4, 2, 2, P.REASON_MEASURED_SPLIT)),
    (7680, (4096, 3584, 4, 2, 2, P.REASON_MEASURED_SPLIT)),
    (8192, (8192, 0, 4, 4, 0, P.REASON_MEASURED_UNSPLIT)),
])
def test_measured_table_hand_derived(T, want):
    p = oracle.split_plan_measured(T, MEASURED_SWEEP, **SWEEP_MODEL)
    got = (p["prefix_tokens"], p["suffix_tokens"], p["waves_unsplit"], p["waves_prefix"],
           p["waves_suffix"], p["reason"])
    assert got == want
    assert p["offset"] == (MEASURED_SWEEP[T] if p["suffix_tokens"] else -1)


def test_measured_table_properties():
    # Counts not in the table get the analytic plan; every plan keeps every
    # token and never takes more waves than the whole batch, with the wave
    # counts re-derived by the brute-force scheduler.
    S = SWEEP_MODEL["num_cus"]
    for T in list(range(0, 9000, 128)) + list(MEASURED_SWEEP):
        p = oracle.split_plan_measured(T, MEASURED_SWEEP, **SWEEP_MODEL)
        if T not in MEASURED_SWEEP:
            assert p == oracle.split_plan(T, **SWEEP_MODEL)
        assert p["prefix_tokens"] + p["suffix_tokens"] == T
        ctas = [oracle.ctas(m, 256, 32) for m in (T, p["prefix_tokens"], p["suffix_tokens"])]
        assert [oracle.simulate_waves(c, S) for c in ctas] == \
            [p["waves_unsplit"], p["waves_prefix"], p["waves_suffix"]]
        assert p["waves_prefix"] + p["waves_suffix"] <= p["waves_unsplit"]
        if p["suffix_tokens"]:
            assert p["prefix_tokens"] == T // 2 + p["offset"]


def test_measured_table_of_the_analytic_choices_gives_the_analytic_splits():
    for T in range(1, 601):
        a = oracle.split_plan(T, num_cus=132)
        table = {T: a["offset"]} if a["reason"] == P.REASON_SPLIT else {}
        m = oracle.split_plan_measured(T, table, num_cus=132)
        fields = ("prefix_tokens", "suffix_tokens", "offset", "waves_unsplit", "waves_prefix",
                  "waves_suffix")
        assert [m[f] for f in fields] == [a[f] for f in fields]
        assert m["reason"] == (P.REASON_MEASURED_SPLIT if table else a["reason"])


def test_measured_table_rejects_offsets_outside_half():
    for bad in ({100: 50}, {100: -2}, {0: 0}, {101: 50}):
        with pytest.raises(ValueError):
            oracle.split_plan_measured(100, bad)
    # 101 tokens: half = 50, so 49 is the largest offset
    assert oracle.split_plan_measured(101, {101: 49}, num_cus=1)["prefix_tokens"] == 99
