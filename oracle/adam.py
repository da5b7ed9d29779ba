"""Per-adapter AdamW step (oracle; test infrastructure only).

Deep Dive - Tinker, "optim_step advances adapter state": the update is
AdamW-equivalent with a default weight decay of zero, and optimizer moments
stay with the service per training client; OpenTinker ("3 Approach") keeps
optimizer state local to each adapter.  The pages give no formula; the reading
taken is the standard bias-corrected AdamW (decoupled decay applied to p
first, epsilon added outside the square root), with each adapter's own step
counter t (1-based):
  m <- b1 m + (1-b1) g ;  v <- b2 v + (1-b2) g^2
  p <- p - lr wd p ;  p <- p - lr (m / (1-b1^t)) / (sqrt(v / (1-b2^t)) + eps)

Non-finite gradients.  TPU RL note, section 12 "The instability I have not
solved", lists among its defences that an optimizer update that is not finite
is skipped outright.  One call here is one adapter's update (its own state and
step counter), so the reading taken is: if any element of the adapter's
gradient is NaN or +-Inf, the whole update is skipped -- p, m and v stay
exactly as they were, and adam_step_flagged reports it so the caller keeps the
adapter's step counter where it was.  adam_step_multi applies that rule to each
adapter's range on its own.
"""
from __future__ import annotations

import numpy as np


def adam_step(p, g, m, v, step, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0):
    """Return new (p, m, v) as float64 arrays; inputs are not modified."""
    return adam_step_flagged(p, g, m, v, step, lr, beta1, beta2, eps, weight_decay)[:3]


def adam_step_flagged(p, g, m, v, step, lr, beta1=0.9, beta2=0.999, eps=1e-8,
                      weight_decay=0.0):
    """(p, m, v, skipped) for one adapter: the step above, or -- when any
    element of g is not finite -- the state unchanged and skipped = True."""
    g = np.asarray(g, np.float64)
    p0 = np.broadcast_to(np.asarray(p, np.float64), g.shape).copy()
    m0 = np.broadcast_to(np.asarray(m, np.float64), g.shape).copy()
    v0 = np.broadcast_to(np.asarray(v, np.float64), g.shape).copy()
    if not np.all(np.isfinite(g)):
        return p0, m0, v0, True
    m1 = beta1 * m0 + (1.0 - beta1) * g
    v1 = beta2 * v0 + (1.0 - beta2) * g * g
    mhat = m1 / (1.0 - beta1 ** step)
    vhat = v1 / (1.0 - beta2 ** step)
    p1 = p0 - lr * weight_decay * p0
    p1 = p1 - lr * mhat / (np.sqrt(vhat) + eps)
    return p1, m1, v1, False


def adam_step_multi(segments, p, g, m, v, lr, beta1=0.9, beta2=0.999, eps=1e-8,
                    weight_decay=0.0):
    """Several adapters' steps over flat arrays.  segments: (offset, count,
    step) per adapter, disjoint.  Returns (p, m, v, skipped list): each range is
    adam_step_flagged of that adapter alone; elements outside every range are
    left as they are."""
    p1 = np.array(p, np.float64)
    m1 = np.array(m, np.float64)
    v1 = np.array(v, np.float64)
    g = np.asarray(g, np.float64)
    skipped = []
    for off, cnt, step in segments:
        sl = slice(int(off), int(off) + int(cnt))
        p1[sl], m1[sl], v1[sl], sk = adam_step_flagged(p1[sl], g[sl], m1[sl], v1[sl], step, lr,
                                                       beta1, beta2, eps, weight_decay)
        skipped.append(sk)
    return p1, m1, v1, skipped
