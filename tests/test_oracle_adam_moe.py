"""Pins for oracle.adam, oracle.mlp and oracle.moe (CPU only).

Adam is pinned to torch.optim.AdamW run on the CPU in float64 (an independent
library routine used only here) and to the first-step closed form.  The MoE
layer is pinned by brute-force routing, by its reduction to the dense LoRA
layer (one adapter, top-1), and by float64 finite differences; the SwiGLU MLP by
finite differences.
"""
import numpy as np
import pytest
import torch

import oracle.adam as OA
import oracle.lora as OL
import oracle.mlp as OM
import oracle.moe as OE
import workloads as W


@pytest.mark.parametrize("wd", [0.0, 0.01])
def test_adam_matches_torch_adamw(wd):
    rng = np.random.default_rng(0)
    n = 257
    p0 = rng.standard_normal(n)
    grads = [rng.standard_normal(n) * 10 ** rng.uniform(-4, 0) for _ in range(4)]
    prm = torch.nn.Parameter(torch.tensor(p0, dtype=torch.float64))
    opt = torch.optim.AdamW([prm], lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=wd, foreach=False)
    p, m, v = p0.copy(), np.zeros(n), np.zeros(n)
    for t, g in enumerate(grads, start=1):
        prm.grad = torch.tensor(g)
        opt.step()
        p, m, v = OA.adam_step(p, g, m, v, t, 1e-3, 0.9, 0.999, 1e-8, wd)
        st = opt.state[prm]
        np.testing.assert_allclose(p - p0, prm.detach().numpy() - p0, rtol=1e-12, atol=2e-15)  # torch scales p by (1 - lr wd); fp64 rounding order
        np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-14, atol=0)
        np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-14, atol=0)


def test_adam_first_step_closed_form():
    g = np.array([1e-3, -2.0, 0.0, 5e-9, -7e-7])
    p = np.ones_like(g)
    p1, m, v = OA.adam_step(p, g, np.zeros_like(g), np.zeros_like(g), 1, 1e-4)
    np.testing.assert_allclose(p1 - p, -1e-4 * g / (np.abs(g) + 1e-8), rtol=1e-9, atol=1e-20)


def test_adam_split_run_equals_straight_run():
    rng = np.random.default_rng(1)
    p, m, v = rng.standard_normal(50), np.zeros(50), np.zeros(50)
    gs = [rng.standard_normal(50) for _ in range(6)]
    a = (p, m, v)
    for t, g in enumerate(gs, 1):
        a = OA.adam_step(*a, g, t, 1e-3) if False else OA.adam_step(a[0], g, a[1], a[2], t, 1e-3)
    b = (p, m, v)
    for t, g in enumerate(gs[:3], 1):
        b = OA.adam_step(b[0], g, b[1], b[2], t, 1e-3)
    saved = tuple(x.copy() for x in b)
    for t, g in enumerate(gs[3:], 4):
        saved = OA.adam_step(saved[0], g, saved[1], saved[2], t, 1e-3)
    for x, y in zip(a, saved):
        assert np.array_equal(x, y)


# ---------------------------------------------------------------- MLP
def test_mlp_finite_differences():
    rng = np.random.default_rng(2)
    n, d, f = 10, 8, 12
    ids = rng.integers(0, 2, size=n)
    ranks = [2, 4]
    def proj(di, do):
        Wp = rng.standard_normal((do, di)) * 0.3
        A = [rng.standard_normal((r, di)) * 0.3 for r in ranks]
        B = [rng.standard_normal((do, r)) * 0.3 for r in ranks]
        return (Wp, A, B, np.array([2.0, 0.5]))
    gate, up, down = proj(d, f), proj(d, f), proj(f, d)
    x = rng.standard_normal((n, d))
    dy = rng.standard_normal((n, d))
    y, saved = OM.mlp_forward(x, gate, up, down, ids)
    dx, grads = OM.mlp_backward(dy, x, gate, up, down, ids, saved)
    eps = 1e-6
    D = rng.standard_normal(x.shape)
    L = lambda xx: float(np.sum(OM.mlp_forward(xx, gate, up, down, ids)[0] * dy))
    fd = (L(x + eps * D) - L(x - eps * D)) / (2 * eps)
    assert abs(fd - np.sum(dx * D)) < 1e-7 * max(1, abs(fd))
    # one adapter factor of each projection
    for name, P in (("gate", gate), ("up", up), ("down", down)):
        DA = rng.standard_normal(P[1][1].shape)
        def Lp(e):
            Pn = (P[0], [P[1][0], P[1][1] + e * DA], P[2], P[3])
            args = {"gate": gate, "up": up, "down": down}
            args[name] = Pn
            return float(np.sum(OM.mlp_forward(x, args["gate"], args["up"], args["down"], ids)[0] * dy))
        fd = (Lp(eps) - Lp(-eps)) / (2 * eps)
        an = np.sum(grads[name][0][1] * DA)
        assert abs(fd - an) < 1e-7 * max(1, abs(fd))


# ---------------------------------------------------------------- MoE
def _moe_tiny(seed=3, n=9, H=6, F=5, E=4, k=2, n_ad=2, r=2):
    rng = np.random.default_rng(seed)
    R = rng.standard_normal((n, E)).astype(np.float32).astype(np.float64)
    ids = rng.integers(0, n_ad, size=n)
    Wg = rng.standard_normal((E, F, H)) * 0.4
    Wu = rng.standard_normal((E, F, H)) * 0.4
    Wd = rng.standard_normal((E, H, F)) * 0.4
    A = {p: [[rng.standard_normal((r, F if p == "down" else H)) * 0.4 for _ in range(E)] for _ in range(n_ad)] for p in ("gate", "up", "down")}
    B = {p: [[rng.standard_normal((H if p == "down" else F, r)) * 0.4 for _ in range(E)] for _ in range(n_ad)] for p in ("gate", "up", "down")}
    x = rng.standard_normal((n, H))
    dy = rng.standard_normal((n, H))
    return R, ids, Wg, Wu, Wd, A, B, x, dy, k, rng


def test_moe_route_brute_force_and_ties():
    R = np.array([[0.5, 2.0, 2.0, -1.0, 0.5], [3.0, 3.0, 3.0, 3.0, 3.0]])
    e, w = OE.moe_route(R, 3)
    assert e.tolist() == [[1, 2, 0], [0, 1, 2]]
    np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-15)
    np.testing.assert_allclose(w[1], [1 / 3] * 3, atol=1e-15)
    rng = np.random.default_rng(0)
    R = rng.standard_normal((50, 16)).astype(np.float32)
    e, w = OE.moe_route(R, 4)
    ref = np.argsort(-R.astype(np.float64), axis=1, kind="stable")[:, :4]
    assert np.array_equal(e, ref)
    P = np.exp(R - R.max(1, keepdims=True)); P /= P.sum(1, keepdims=True)
    top = np.take_along_axis(P, ref, 1)
    np.testing.assert_allclose(w, top / top.sum(1, keepdims=True), rtol=1e-6)


def test_moe_reduces_to_dense_lora_at_top1_one_adapter():
    R, ids, Wg, Wu, Wd, A, B, x, dy, _, _ = _moe_tiny(n_ad=1)
    ids = np.zeros_like(ids)
    e, w = OE.moe_route(R, 1)
    assert np.all(w == 1.0)
    y, saved = OE.moe_forward(x, e, w, ids, Wg, Wu, Wd, A, B, 1.5)
    for t in range(x.shape[0]):
        ex = int(e[t, 0])
        lay = lambda p, Wp, inp: OL.lora_forward(inp[None], Wp[ex], [A[p][0][ex]], [B[p][0][ex]], [1.5], [0])[0][0]
        g, u = lay("gate", Wg, x[t]), lay("up", Wu, x[t])
        h = OM.swiglu_forward(g, u)
        np.testing.assert_allclose(y[t], lay("down", Wd, h), rtol=0, atol=1e-12)


def test_moe_backward_finite_differences():
    R, ids, Wg, Wu, Wd, A, B, x, dy, k, rng = _moe_tiny()
    e, w = OE.moe_route(R, k)
    s = 0.7
    y, saved = OE.moe_forward(x, e, w, ids, Wg, Wu, Wd, A, B, s)
    dx, dA, dB = OE.moe_backward(dy, x, e, w, ids, Wg, Wu, Wd, A, B, s, saved)
    L = lambda xx, AA, BB: float(np.sum(OE.moe_forward(xx, e, w, ids, Wg, Wu, Wd, AA, BB, s)[0] * dy))
    eps = 1e-6
    D = rng.standard_normal(x.shape)
    fd = (L(x + eps * D, A, B) - L(x - eps * D, A, B)) / (2 * eps)
    assert abs(fd - np.sum(dx * D)) < 1e-7 * max(1, abs(fd))
    for p in ("gate", "up", "down"):
        for a in range(len(A[p])):
            for ex in range(len(A[p][a])):
                for which, M, G in (("A", A, dA), ("B", B, dB)):
                    DM = rng.standard_normal(M[p][a][ex].shape)
                    def pert(sign):
                        MM = {q: [[m.copy() for m in row] for row in M[q]] for q in M}
                        MM[p][a][ex] = MM[p][a][ex] + sign * eps * DM
                        return L(x, MM, B) if which == "A" else L(x, A, MM)
                    fd = (pert(1) - pert(-1)) / (2 * eps)
                    an = np.sum(G[p][a][ex] * DM)
                    assert abs(fd - an) < 1e-7 * max(1, abs(fd)), (p, a, ex, which)


def test_adam_skips_nonfinite_gradients():
    """NaN and +-Inf gradient elements keep p, m, v as they were; every other
    element takes the ordinary step, checked against torch AdamW run on those
    elements alone from the same state (step 3)."""
    rng = np.random.default_rng(5)
    n = 64
    p0, m0, v0 = rng.standard_normal(n), rng.standard_normal(n) * 1e-3, rng.random(n) * 1e-4
    g = rng.standard_normal(n)
    bad = [3, 17, 40]
    g[bad] = [np.nan, np.inf, -np.inf]
    p, m, v, skipped = OA.adam_step_flagged(p0, g, m0, v0, 3, 1e-3, weight_decay=0.01)
    assert skipped
    for a, a0 in ((p, p0), (m, m0), (v, v0)):
        assert np.array_equal(a[bad], a0[bad])
    ok = np.isfinite(g)
    prm = torch.nn.Parameter(torch.tensor(p0[ok]))
    opt = torch.optim.AdamW([prm], lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01,
                            foreach=False)
    opt.state[prm] = {"step": torch.tensor(2.0, dtype=torch.float64),
                      "exp_avg": torch.tensor(m0[ok]), "exp_avg_sq": torch.tensor(v0[ok])}
    prm.grad = torch.tensor(g[ok])
    opt.step()
    np.testing.assert_allclose(p[ok] - p0[ok], prm.detach().numpy() - p0[ok], rtol=1e-12, atol=2e-15)
    np.testing.assert_allclose(m[ok], opt.state[prm]["exp_avg"].numpy(), rtol=1e-14, atol=0)
    np.testing.assert_allclose(v[ok], opt.state[prm]["exp_avg_sq"].numpy(), rtol=1e-14, atol=0)
    # all finite: nothing skipped, and the plain step
    p2, m2, v2, skipped2 = OA.adam_step_flagged(p0, np.where(ok, g, 0.5), m0, v0, 3, 1e-3)
    assert not skipped2 and np.all(np.isfinite(p2))
