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
