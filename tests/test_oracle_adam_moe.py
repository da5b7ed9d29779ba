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


def _torch_adamw_from(p0, m0, v0, g, prev_steps, lr, wd):
    """torch.optim.AdamW (CPU, float64) one step from a given state; returns
    (p, m, v) after the step."""
    prm = torch.nn.Parameter(torch.tensor(p0))
    opt = torch.optim.AdamW([prm], lr=lr, betas=(0.9, 0.999), eps=1e-8, weight_decay=wd,
                            foreach=False)
    opt.state[prm] = {"step": torch.tensor(float(prev_steps), dtype=torch.float64),
                      "exp_avg": torch.tensor(m0), "exp_avg_sq": torch.tensor(v0)}
    prm.grad = torch.tensor(g)
    opt.step()
    st = opt.state[prm]
    return prm.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


def test_adam_skips_whole_adapter_on_nonfinite_gradient():
    """TPU RL note, section 12: a non-finite optimizer update is skipped
    outright.  Five adapters in one flat buffer; adapter 3's gradient holds one
    NaN (and, in a second round, one -Inf): all of adapter 3 -- p, m and v,
    including every finite element -- stays bit-identical, while each other
    adapter takes the ordinary step, checked against torch AdamW run on that
    adapter alone from the same state.  A per-element skip would move adapter
    3's finite elements and fail here."""
    rng = np.random.default_rng(5)
    counts = [40, 17, 64, 33, 9]
    offs = np.concatenate([[0], np.cumsum(counts)[:-1]])
    n = int(sum(counts))
    steps = [3, 1, 7, 4, 2]
    p0, m0, v0 = rng.standard_normal(n), rng.standard_normal(n) * 1e-3, rng.random(n) * 1e-4
    for bad_value in (np.nan, -np.inf):
        g = rng.standard_normal(n)
        g[offs[3] + 11] = bad_value
        segs = [(int(o), c, t) for o, c, t in zip(offs, counts, steps)]
        p, m, v, skipped = OA.adam_step_multi(segs, p0, g, m0, v0, 1e-3, weight_decay=0.01)
        assert skipped == [False, False, False, True, False]
        sl3 = slice(offs[3], offs[3] + counts[3])
        for a, a0 in ((p, p0), (m, m0), (v, v0)):
            assert np.array_equal(a[sl3], a0[sl3])
        for i in (0, 1, 2, 4):
            sl = slice(offs[i], offs[i] + counts[i])
            tp, tm, tv = _torch_adamw_from(p0[sl], m0[sl], v0[sl], g[sl], steps[i] - 1, 1e-3, 0.01)
            np.testing.assert_allclose(p[sl] - p0[sl], tp - p0[sl], rtol=1e-12, atol=2e-15)
            np.testing.assert_allclose(m[sl], tm, rtol=1e-14, atol=0)
            np.testing.assert_allclose(v[sl], tv, rtol=1e-14, atol=0)
            assert not np.array_equal(p[sl], p0[sl])
    # one adapter alone: +Inf anywhere skips it, all finite steps it
    g1 = rng.standard_normal(8)
    g1[0] = np.inf
    p1, m1, v1, sk = OA.adam_step_flagged(p0[:8], g1, m0[:8], v0[:8], 2, 1e-3)
    assert sk and np.array_equal(p1, p0[:8]) and np.array_equal(m1, m0[:8]) and np.array_equal(v1, v0[:8])
    g1[0] = 0.5
    p1, _, _, sk = OA.adam_step_flagged(p0[:8], g1, m0[:8], v0[:8], 2, 1e-3)
    assert not sk and np.all(p1 != p0[:8])


def test_moe_brute_force_tiny_e4_k2():
    """Brute force on a tiny layer (4 experts, top-2, 2 adapters): per token,
    Python loops pick the two largest logits by scanning (ties to the lower
    index), form their softmax weights from the full softmax, and evaluate each
    chosen expert's SwiGLU MLP with its (expert, adapter) LoRA element by
    element.  Independent of the oracle's grouping by (expert, adapter)."""
    import math
    rng = np.random.default_rng(31)
    n, H, F, E, k, r, s = 7, 5, 6, 4, 2, 2, 0.75
    R = rng.standard_normal((n, E))
    R[2, 1] = R[2, 3] = R[2].max() + 0.5                  # a tie for first place
    ids = rng.integers(0, 2, size=n)
    Wg, Wu = rng.standard_normal((E, F, H)), rng.standard_normal((E, F, H))
    Wd = rng.standard_normal((E, H, F))
    A = {p: [[rng.standard_normal((r, F if p == "down" else H)) for _ in range(E)] for _ in range(2)]
         for p in ("gate", "up", "down")}
    B = {p: [[rng.standard_normal((H if p == "down" else F, r)) for _ in range(E)] for _ in range(2)]
         for p in ("gate", "up", "down")}
    x = rng.standard_normal((n, H))

    def proj(Wm, Am, Bm, z):
        out = []
        for o in range(len(Wm)):
            acc = sum(Wm[o][i] * z[i] for i in range(len(z)))
            for q in range(r):
                acc += s * Bm[o][q] * sum(Am[q][i] * z[i] for i in range(len(z)))
            out.append(acc)
        return out

    experts, weights = OE.moe_route(R, k)
    y = OE.moe_forward(x, experts, weights, ids, Wg, Wu, Wd, A, B, s)[0]
    for t in range(n):
        row = list(R[t])
        picked = []
        for _ in range(k):
            best = None
            for e in range(E):
                if e in picked:
                    continue
                if best is None or row[e] > row[best]:
                    best = e
            picked.append(best)
        assert list(experts[t]) == picked
        mx = max(row)
        z = sum(math.exp(v - mx) for v in row)
        p = [math.exp(row[e] - mx) / z for e in picked]
        wts = [q / sum(p) for q in p]
        a = int(ids[t])
        want = [0.0] * H
        for e, wk in zip(picked, wts):
            gg = proj(Wg[e], A["gate"][a][e], B["gate"][a][e], x[t])
            uu = proj(Wu[e], A["up"][a][e], B["up"][a][e], x[t])
            h = [gi / (1.0 + math.exp(-gi)) * ui for gi, ui in zip(gg, uu)]
            o = proj(Wd[e], A["down"][a][e], B["down"][a][e], h)
            want = [wv + wk * ov for wv, ov in zip(want, o)]
        np.testing.assert_allclose(y[t], want, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(weights[t], wts, rtol=1e-12)
    assert list(experts[2]) == [1, 3]
