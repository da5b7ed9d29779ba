"""Target-token logprobs through the lm_head, and their backward (oracle; test
infrastructure only).

TPU RL note ("Tinker API Implementation on TPUs..."), section 10 "The
22,528-token wall":
  * "1 - Score log-probabilities on the training chips": only the target
    token's value is gathered;
  * "3 - Never materialize a log-softmax": a token's logprob is its logit minus
    the logsumexp of the row, with the stable form lse = m + log sum exp(z - m),
    m = max z;
  * "4 - Fused linear cross-entropy": the backward recomputes logits rather
    than keeping them.
The oracle states the result, not the tiling: z_t = U h_t, lse_t as above,
logprob_t = z_t[y_t] - lse_t; for upstream d_t = dL/dlogprob_t,
dh_t = d_t (U[y_t] - sum_v softmax(z_t)_v U[v]).  U is frozen (no dU).
Rows are processed in chunks only to bound memory (an N x V float64 block).
Targets outside [0, V) give a NaN logprob and a zero dh row.
"""
from __future__ import annotations

import numpy as np


def _chunk_rows(n, vocab, budget_bytes=256 << 20):
    return max(1, min(n, budget_bytes // max(1, vocab * 8)))


def token_logprobs(h, U, targets, rows=None):
    """Return (logprobs [N], lse [N]) in float64.  `rows` restricts to a subset."""
    h = np.asarray(h, np.float64)
    U = np.asarray(U, np.float64)
    targets = np.asarray(targets, np.int64)
    idx = np.arange(h.shape[0]) if rows is None else np.asarray(rows, np.int64)
    V = U.shape[0]
    lp = np.empty(idx.size)
    lse = np.empty(idx.size)
    step = _chunk_rows(idx.size, V)
    for s in range(0, idx.size, step):
        sel = idx[s:s + step]
        z = h[sel] @ U.T
        m = z.max(axis=1)
        l = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
        lse[s:s + step] = l
        y = targets[sel]
        ok = (y >= 0) & (y < V)
        zy = np.full(sel.size, np.nan)
        zy[ok] = z[np.arange(sel.size)[ok], y[ok]]
        lp[s:s + step] = zy - l
    return lp, lse


def token_logprobs_backward(h, U, targets, dlogp, rows=None):
    """Return dh [N, H] (float64) for upstream dlogp [N]."""
    h = np.asarray(h, np.float64)
    U = np.asarray(U, np.float64)
    targets = np.asarray(targets, np.int64)
    dlogp = np.asarray(dlogp, np.float64)
    idx = np.arange(h.shape[0]) if rows is None else np.asarray(rows, np.int64)
    V = U.shape[0]
    dh = np.zeros((idx.size, h.shape[1]))
    step = _chunk_rows(idx.size, V)
    for s in range(0, idx.size, step):
        sel = idx[s:s + step]
        z = h[sel] @ U.T
        m = z.max(axis=1)
        p = np.exp(z - m[:, None])
        p /= p.sum(axis=1, keepdims=True)
        d = dlogp[sel]
        y = targets[sel]
        ok = (y >= 0) & (y < V) & (d != 0.0)
        G = -d[:, None] * p
        G[np.arange(sel.size)[ok], y[ok]] += d[ok]
        G[~ok] = 0.0
        dh[s:s + step] = G @ U
    return dh
