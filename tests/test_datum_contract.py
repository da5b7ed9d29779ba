"""The client-side contract check from Deep Dive - Tinker ('A runnable contract
check'), against the values that page prints (tests/golden)."""
import json
import math
import os
from dataclasses import replace

import pytest

from workloads.datum import RLDatum, center, has_signal, shift_align, validate

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tinker_contract_check.json")))


def test_center_worked_example():
    adv = center(G["clamp_rewards"])
    assert list(adv) == G["advantages"]
    assert sum(G["clamp_rewards"]) / 4 == G["group_mean"]
    assert has_signal(G["clamp_rewards"])
    assert has_signal([1.0] * 4) == G["all_ones_has_signal"]
    assert center([1.0] * 4) == (0.0, 0.0, 0.0, 0.0)


def test_shift_alignment_keeps_first_answer():
    inp, tgt, w = shift_align(G["toy_sequence"], G["toy_action_mask_full"])
    assert list(inp) == G["toy_inputs"] and list(tgt) == G["toy_targets"] and list(w) == G["toy_weights"]
    pos = G["first_answer_position"]
    assert tgt[pos] == G["first_answer_target"] and w[pos] == 1.0
    tot = sum(w)
    assert [x / tot for x in w] == G["toy_reduction_mean_weights"]


def _valid():
    v = G["valid_datum"]
    return RLDatum(tuple(v["input_tokens"]), tuple(v["target_tokens"]), tuple(v["sampled_logprobs"]),
                   tuple(v["advantages"]), tuple(v["mask"]))


def test_validate_rejects_nine_inputs():
    d = _valid()
    validate(d)
    bad = [
        replace(d, input_tokens=(10, 11)),                 # unaligned lengths
        replace(d, advantages=(0.0, math.nan, 0.5)),       # non-finite score
        replace(d, mask=(0.0, 0.5, 1.0)),                  # fractional mask
        replace(d, mask=(0.0, 0.0, 0.0)),                  # nothing trainable
        replace(d, sampled_logprobs=(0.0, 0.4, -0.8)),     # positive action logprob
        replace(d, advantages=(0.5, 0.5, 0.5)),            # masked position with advantage
        replace(d, target_tokens=(11, -1, 21)),            # negative token
    ]
    rejected = 0
    for b in bad:
        with pytest.raises(ValueError):
            validate(b)
        rejected += 1
    for rewards in ((), (math.inf,)):
        with pytest.raises(ValueError):
            center(rewards)
        rejected += 1
    assert rejected == G["rejected_inputs"]
