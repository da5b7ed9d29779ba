"""Token-level losses and their gradient with respect to the logprobs (oracle;
test infrastructure only).

Sources
  * Deep Dive - Tinker, "SFT first: a token-level contract": cross-entropy over
    target positions weighted per token, prompt positions weight 0.
  * Deep Dive - Tinker, "The RL datum shape": the backend cross-entropy is
    minus the weighted sum of logprobs; importance_sampling compares current
    and sampler logprobs; ppo adds clipping; a custom loss C(l) is trained by
    sending weights -dC/dl to that cross-entropy.
  * forward_backward_custom post (lovedeathtransformers): the server
    re-forwards and backpropagates sum(logprobs * dLoss/dlogprobs).
  * TPU RL note, section 12 "The instability I have not solved": the RL loss
    exponentiates a difference of logprobs, and a masked token must have its
    value neutralised as well as its weight zeroed (inf * 0 is NaN).
Readings where the pages are silent (their formulas were lost): the loss is a
plain sum over tokens; rho = exp(l - l_sampler); ppo minimises
-min(rho A, clip(rho, 1-eps_lo, 1+eps_hi) A) with inclusive clip bounds; the
custom path reports S = sum g l and returns dl = g.  For cross_entropy the
per-token array is a weight w (may be fractional); for the others it is a mask
m, and rows with w == 0 / m == 0 are removed by selection, so non-finite values
there cannot leak.
Sentinel (TPU RL note, section 12 "The instability I have not solved": a NaN
logprob is caught, and such a token gets its weight zeroed and its value
neutralised).  Reading: a kept row (w != 0) any of whose inputs to its own
loss term is NaN or +-Inf -- l and w for cross_entropy; l, m, A and l_sampler
for importance_sampling and ppo; l, m and g for custom -- is removed by
selection exactly like a masked row (dl = 0, no loss term), and
loss_grad_flagged reports that it happened.  The check is on the inputs, so it
does not depend on the precision the loss is evaluated in.
"""
from __future__ import annotations

import numpy as np

CROSS_ENTROPY, IMPORTANCE_SAMPLING, PPO, CUSTOM = 0, 1, 2, 3


def loss_grad(kind, logp, weights, adv=None, samp=None, g=None, clip_low=0.2, clip_high=0.2):
    """Return (loss float, dlogp float64 [N])."""
    return loss_grad_flagged(kind, logp, weights, adv, samp, g, clip_low, clip_high)[:2]


def _row_inputs(kind, l, w, adv, samp, g):
    """The per-row inputs the kind's loss term reads."""
    if kind == CROSS_ENTROPY:
        return [l, w]
    if kind == CUSTOM:
        return [l, w, np.asarray(g, np.float64)]
    if kind in (IMPORTANCE_SAMPLING, PPO):
        return [l, w, np.asarray(adv, np.float64), np.asarray(samp, np.float64)]
    raise ValueError(f"unknown loss kind {kind}")


def loss_grad_flagged(kind, logp, weights, adv=None, samp=None, g=None, clip_low=0.2,
                      clip_high=0.2):
    """Return (loss float, dlogp float64 [N], sentinel bool): sentinel is True
    when a kept row was removed because one of its inputs was not finite."""
    l = np.asarray(logp, np.float64)
    w = np.asarray(weights, np.float64)
    finite = np.ones(l.shape, bool)
    for a in _row_inputs(kind, l, w, adv, samp, g):
        finite &= np.isfinite(a)
    kept = w != 0.0
    sentinel = bool(np.any(kept & ~finite))
    keep = kept & finite
    dl = np.zeros_like(l)
    if kind == CROSS_ENTROPY:
        dl[keep] = -w[keep]
        return float(-np.sum(w[keep] * l[keep])), dl, sentinel
    if kind == CUSTOM:
        gg = np.asarray(g, np.float64)
        dl[keep] = gg[keep]
        return float(np.sum(gg[keep] * l[keep])), dl, sentinel
    A = np.asarray(adv, np.float64)[keep]
    rho = np.exp(l[keep] - np.asarray(samp, np.float64)[keep])
    if kind == IMPORTANCE_SAMPLING:
        dl[keep] = -rho * A
        return float(-np.sum(rho * A)), dl, sentinel
    clipped = np.clip(rho, 1.0 - clip_low, 1.0 + clip_high)
    obj = np.minimum(rho * A, clipped * A)
    inactive = ((A > 0) & (rho > 1.0 + clip_high)) | ((A < 0) & (rho < 1.0 - clip_low))
    dl[keep] = np.where(inactive, 0.0, -rho * A)
    return float(-np.sum(obj)), dl, sentinel
