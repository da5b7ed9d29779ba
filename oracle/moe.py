"""Top-k routed expert layer with LoRA on every expert (oracle; test
infrastructure only).

TPU RL note, section 12 "Mixture-of-experts, and where adapters attach": in a
mixture-of-experts model the MLP is the experts, so an adapter that covers the
MLP must cover every expert's projections.  tinker-ticks, "Step time": the MoE
pool is slower than the dense one because every expert weight is touched and
the adapter spans more linear layers.
Readings (the pages give no routing formula): P = softmax(router logits); the
top-k experts are the k largest logits (ties to the lower expert index),
listed by descending probability; their weights are P renormalised over the
top-k; each expert is a SwiGLU MLP down(silu(gate x) * up x), and each of its
three projections carries the token's adapter as y = W x + s B (A x).  The
router and the combine weights are treated as constants in the backward.
Containers: W_gate, W_up [E, F, H]; W_down [E, H, F]; A[p][a][e], B[p][a][e]
for p in ("gate", "up", "down") with gate/up A [r, H], B [F, r] and down
A [r, F], B [H, r].
The functions are the plain definitions above, in float64 throughout.
"""
from __future__ import annotations

import numpy as np


def moe_route(R, k):
    """Return (experts int64 [N, k], weights float64 [N, k])."""
    R = np.asarray(R, np.float64)
    n, E = R.shape
    experts = np.empty((n, k), np.int64)
    weights = np.empty((n, k))
    for t in range(n):
        order = sorted(range(E), key=lambda e: (-R[t, e], e))[:k]
        experts[t] = order
        z = R[t] - R[t].max()
        p = np.exp(z) / np.exp(z).sum()
        weights[t] = p[order] / p[order].sum()
    return experts, weights


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _dsilu(z):
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def _groups(experts, ids):
    """Assignments j = t*k + slot grouped by (expert, adapter)."""
    n, k = experts.shape
    e_flat = experts.reshape(-1)
    a_flat = np.repeat(np.asarray(ids, np.int64), k)
    out = {}
    for j in range(n * k):
        out.setdefault((int(e_flat[j]), int(a_flat[j])), []).append(j)
    return {key: np.asarray(v, np.int64) for key, v in out.items()}


def moe_forward(x, experts, weights, ids, Wg, Wu, Wd, A, B, scale):
    """Return (y [N, H], saved dict with per-assignment g_pre, u_pre, h)."""
    x = np.asarray(x, np.float64)
    n, H = x.shape
    k = experts.shape[1]
    F = Wg.shape[1]
    gpre = np.zeros((n * k, F))
    upre = np.zeros((n * k, F))
    hmid = np.zeros((n * k, F))
    out = np.zeros((n * k, H))
    for (e, a), js in _groups(experts, ids).items():
        xs = x[js // k]
        g = xs @ Wg[e].T + scale * (xs @ A["gate"][a][e].T) @ B["gate"][a][e].T
        u = xs @ Wu[e].T + scale * (xs @ A["up"][a][e].T) @ B["up"][a][e].T
        h = _silu(g) * u
        o = h @ Wd[e].T + scale * (h @ A["down"][a][e].T) @ B["down"][a][e].T
        gpre[js], upre[js], hmid[js], out[js] = g, u, h, o
    y = (out.reshape(n, k, H) * np.asarray(weights)[:, :, None]).sum(axis=1)
    return y, {"gpre": gpre, "upre": upre, "h": hmid}


def moe_backward(dy, x, experts, weights, ids, Wg, Wu, Wd, A, B, scale, saved):
    """Return (dx [N, H], dA, dB) with dA[p][a][e], dB[p][a][e] like A, B."""
    dy = np.asarray(dy, np.float64)
    x = np.asarray(x, np.float64)
    n, H = x.shape
    k = experts.shape[1]
    dA = {p: [[np.zeros_like(m) for m in row] for row in A[p]] for p in A}
    dB = {p: [[np.zeros_like(m) for m in row] for row in B[p]] for p in B}
    dx = np.zeros_like(x)
    w_flat = np.asarray(weights).reshape(-1)
    for (e, a), js in _groups(experts, ids).items():
        ts = js // k
        xs = x[ts]
        do = w_flat[js][:, None] * dy[ts]
        g, u, h = saved["gpre"][js], saved["upre"][js], saved["h"][js]
        Ad, Bd = A["down"][a][e], B["down"][a][e]
        vd = do @ Bd
        dh = do @ Wd[e] + scale * vd @ Ad
        dB["down"][a][e] += scale * do.T @ (h @ Ad.T)
        dA["down"][a][e] += scale * vd.T @ h
        dg = dh * u * _dsilu(g)
        du = dh * _silu(g)
        dxs = np.zeros_like(xs)
        for p, Wp, d in (("gate", Wg, dg), ("up", Wu, du)):
            Ap, Bp = A[p][a][e], B[p][a][e]
            vp = d @ Bp
            dxs += d @ Wp[e] + scale * vp @ Ap
            dB[p][a][e] += scale * d.T @ (xs @ Ap.T)
            dA[p][a][e] += scale * vp.T @ xs
        np.add.at(dx, ts, dxs)
    return dx, dA, dB
