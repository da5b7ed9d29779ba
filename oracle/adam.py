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

Non-finite gradients (no rule on the pages; the reading taken is to skip the
bad update and keep the state as it was): an element
whose g is NaN or +-Inf keeps its p, m, v unchanged, every other element
updates as above.  adam_step_flagged also reports whether any was skipped.
"""
from __future__ import annotations

import numpy as np


def adam_step(p, g, m, v, step, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0):
    """Return new (p, m, v) as float64 arrays; inputs are not modified."""
    return adam_step_flagged(p, g, m, v, step, lr, beta1, beta2, eps, weight_decay)[:3]


def adam_step_flagged(p, g, m, v, step, lr, beta1=0.9, beta2=0.999, eps=1e-8,
                      weight_decay=0.0):
    """(p, m, v, skipped): the step above, elements with a non-finite g left as
    they were; skipped is True when there was any."""
    g = np.asarray(g, np.float64)
    ok = np.isfinite(g)
    p0 = np.broadcast_to(np.asarray(p, np.float64), g.shape)
    m0 = np.broadcast_to(np.asarray(m, np.float64), g.shape)
    v0 = np.broadcast_to(np.asarray(v, np.float64), g.shape)
    gz = np.where(ok, g, 0.0)   # keeps the skipped lanes free of NaN arithmetic
    m1 = beta1 * m0 + (1.0 - beta1) * gz
    v1 = beta2 * v0 + (1.0 - beta2) * gz * gz
    mhat = m1 / (1.0 - beta1 ** step)
    vhat = v1 / (1.0 - beta2 ** step)
    p1 = p0 - lr * weight_decay * p0
    p1 = p1 - lr * mhat / (np.sqrt(vhat) + eps)
    return (np.where(ok, p1, p0), np.where(ok, m1, m0), np.where(ok, v1, v0),
            bool(not ok.all()))
