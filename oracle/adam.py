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
"""
from __future__ import annotations

import numpy as np


def adam_step(p, g, m, v, step, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0):
    """Return new (p, m, v) as float64 arrays; inputs are not modified."""
    p = np.array(p, np.float64)
    g = np.asarray(g, np.float64)
    m = beta1 * np.asarray(m, np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, np.float64) + (1.0 - beta2) * g * g
    mhat = m / (1.0 - beta1 ** step)
    vhat = v / (1.0 - beta2 ** step)
    p = p - lr * weight_decay * p
    p = p - lr * mhat / (np.sqrt(vhat) + eps)
    return p, m, v
