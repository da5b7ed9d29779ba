"""Mixed-adapter LoRA linear layer, forward and backward (oracle; test
infrastructure only).

Definitions followed
  * Deep Dive - Tinker, "LoRA is the adaptation boundary" and "Checkpoints and
    export paths": the adapted weight is W' = W + gamma B A with a constant
    scale gamma, commonly alpha / r; the base W is frozen.
  * tinker-ticks, "Forward pass: what actually happens": per user i,
    y_i = x_i W (base) plus x_i A_i B_i (LoRA fix-up), written for row
    vectors.  In PyTorch Linear layout (W [d_out, d_in], A_i [r, d_in],
    B_i [d_out, r]) that is y_t = W x_t + s_a B_a (A_a x_t), s_a = alpha_a/r_a,
    with a = a_t the adapter of token t.
  * OpenTinker (abstract; "3 Approach"): gradients and optimizer state stay
    local to each adapter; TPU RL note, "4. The Tunix backend": only adapter
    gradients exist (the base is frozen, so there is no dW).

Backward, for upstream g_t = dL/dy_t:
  v_t   = B_a^T g_t                       (rank r_a)
  dx_t  = W^T g_t + s_a A_a^T v_t
  dB_a  = s_a sum_{t: a_t=a} g_t u_t^T    with u_t = A_a x_t
  dA_a  = s_a sum_{t: a_t=a} v_t x_t^T
Tokens whose id is outside [0, n_adapters) get the base output only and
contribute to no adapter's gradient.
"""
from __future__ import annotations

import numpy as np


def _rows_of(ids, a):
    return np.nonzero(np.asarray(ids) == a)[0]


def lora_forward(x, W, A, B, scales, ids):
    """y [N, d_out], u [N, r_max] (u_t = A_{a_t} x_t in columns 0..r_a-1, zero after).

    x [N, d_in]; W [d_out, d_in]; A, B lists of per-adapter float64 matrices;
    scales [n_adapters]; ids [N].  The per-adapter loop is the per-user
    reference form; the shared base product is one matmul over all rows.
    """
    x = np.asarray(x, np.float64)
    W = np.asarray(W, np.float64)
    n = x.shape[0]
    r_max = max([a.shape[0] for a in A] + [0])
    y = x @ W.T
    u = np.zeros((n, r_max))
    for a in range(len(A)):
        rows = _rows_of(ids, a)
        if rows.size == 0:
            continue
        ua = x[rows] @ A[a].T
        u[rows, :A[a].shape[0]] = ua
        y[rows] += scales[a] * (ua @ B[a].T)
    return y, u


def lora_backward(dy, x, W, A, B, scales, ids):
    """Return dx [N, d_in], dA list, dB list, v [N, r_max].

    The adapter-local sums run over exactly the tokens routed to that adapter.
    """
    dy = np.asarray(dy, np.float64)
    x = np.asarray(x, np.float64)
    W = np.asarray(W, np.float64)
    n = x.shape[0]
    r_max = max([a.shape[0] for a in A] + [0])
    dx = dy @ W
    v = np.zeros((n, r_max))
    dA = [np.zeros_like(a) for a in A]
    dB = [np.zeros_like(b) for b in B]
    for a in range(len(A)):
        rows = _rows_of(ids, a)
        if rows.size == 0:
            continue
        r = A[a].shape[0]
        g = dy[rows]
        xa = x[rows]
        ua = xa @ A[a].T
        va = g @ B[a]
        v[rows, :r] = va
        dx[rows] += scales[a] * (va @ A[a])
        dB[a] = scales[a] * (g.T @ ua)
        dA[a] = scales[a] * (va.T @ xa)
    return dx, dA, dB, v


def merged_forward(x, W, A, B, scales, ids):
    """Forward through the merged weight W + s_a B_a A_a for each token's
    adapter (the export form W' = W + gamma B A)."""
    x = np.asarray(x, np.float64)
    W = np.asarray(W, np.float64)
    y = x @ W.T
    for a in range(len(A)):
        rows = _rows_of(ids, a)
        if rows.size == 0:
            continue
        Wm = W + scales[a] * (B[a] @ A[a])
        y[rows] = x[rows] @ Wm.T
    return y
