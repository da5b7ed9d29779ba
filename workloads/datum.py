"""Client-side datum helpers: the caller's contract before the hot path.

These follow the local contract check on the page "Deep Dive - Tinker"
(section "A runnable contract check") and the RL recipe in its section "RL:
preserve tokens, logprobs, and credit": group-centred advantages, the
"has signal" test for a reward group, the datum validation rules, and the
shift that aligns inputs, targets and weights (section "SFT first: a
token-level contract").  They run on the client, upstream of the C-ABI, and are
written here from the rules the page states, not from its listing.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Sequence, Tuple


def center(rewards: Sequence[float]) -> Tuple[float, ...]:
    """Group-relative advantages A_i = R_i - mean(R) (no division by std).

    Empty or non-finite reward groups are rejected with ValueError.
    """
    rewards = tuple(float(r) for r in rewards)
    if len(rewards) == 0:
        raise ValueError("reward group is empty")
    if any(not math.isfinite(r) for r in rewards):
        raise ValueError("reward group holds a non-finite value")
    mean = math.fsum(rewards) / len(rewards)
    return tuple(r - mean for r in rewards)


def has_signal(rewards: Sequence[float]) -> bool:
    """A group whose rewards are all equal centres to all-zero advantages."""
    return len(set(float(r) for r in rewards)) > 1


@dataclass(frozen=True)
class RLDatum:
    input_tokens: Tuple[int, ...]
    target_tokens: Tuple[int, ...]
    sampled_logprobs: Tuple[float, ...]
    advantages: Tuple[float, ...]
    mask: Tuple[float, ...]


def validate(d: RLDatum) -> None:
    """Reject a malformed RL datum with ValueError.

    Rules: all five per-position arrays share one non-zero length; every token
    id is a non-negative Python int; sampled logprobs and advantages are
    finite; mask entries are exactly 0 or 1; at least one position is
    trainable; a trainable position's sampled logprob is not positive; a
    masked position carries zero advantage.
    """
    arrays = (d.input_tokens, d.target_tokens, d.sampled_logprobs, d.advantages, d.mask)
    lengths = {len(a) for a in arrays}
    if len(lengths) != 1 or 0 in lengths:
        raise ValueError(f"per-position arrays are not aligned: lengths {sorted(lengths)}")
    for tok in tuple(d.input_tokens) + tuple(d.target_tokens):
        if type(tok) is not int or tok < 0:
            raise ValueError("token ids must be non-negative ints")
    for val in tuple(d.sampled_logprobs) + tuple(d.advantages):
        if not math.isfinite(val):
            raise ValueError("logprobs and advantages must be finite")
    for m in d.mask:
        if m != 0.0 and m != 1.0:
            raise ValueError("mask entries must be 0 or 1")
    if all(m == 0.0 for m in d.mask):
        raise ValueError("no trainable position in datum")
    for m, lp in zip(d.mask, d.sampled_logprobs):
        if m == 1.0 and lp > 0.0:
            raise ValueError("a trained position has a positive logprob")
    for m, adv in zip(d.mask, d.advantages):
        if m == 0.0 and adv != 0.0:
            raise ValueError("a masked position carries a non-zero advantage")


def shift_align(full_tokens: Sequence[int], full_weights: Sequence[float]):
    """Next-token alignment: inputs drop the last token, targets drop the first,
    and weights follow the target position."""
    full_tokens = tuple(full_tokens)
    full_weights = tuple(full_weights)
    if len(full_tokens) != len(full_weights) or len(full_tokens) < 2:
        raise ValueError("need two or more tokens with one weight each")
    return full_tokens[:-1], full_tokens[1:], full_weights[1:]
