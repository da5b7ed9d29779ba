"""Pins for oracle.logprob and oracle.loss (CPU only).

Checks: uniform logits give -ln V; probabilities sum to one; scipy's
log_softmax on small vocabularies; invariance to a common shift of the lm_head
rows; float64 finite differences for the backward; the custom-loss surrogate
identity; closed forms and special cases for each loss; masked rows holding
NaN/Inf contribute exact zeros.
"""
import json
import os

import numpy as np
import pytest
import scipy.special

import oracle.logprob as OP
import oracle.loss as OLs
import workloads as W

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")))


def _case(seed=0, n=16, H=24, V=40):
    rng = np.random.default_rng(seed)
    h = W.round_bf16(rng.standard_normal((n, H)))
    U = W.round_bf16(rng.standard_normal((V, H)) * 0.3)
    y = rng.integers(0, V, size=n)
    return h, U, y, rng


def test_uniform_logits_give_minus_log_vocab():
    g = GOLD["uniform_logprob"]
    V = g["vocab"]
    h = np.random.default_rng(0).standard_normal((3, 8))
    U = np.zeros((V, 8))
    lp, lse = OP.token_logprobs(h, U, np.array([0, 17, V - 1]))
    np.testing.assert_allclose(lp, g["logprob"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("V", [2, 7, 40, 1024])
def test_matches_scipy_log_softmax(V):
    h, U, y, _ = _case(1, V=V)
    y = y % V
    lp, lse = OP.token_logprobs(h, U, y)
    z = h @ U.T
    ref = scipy.special.log_softmax(z, axis=1)[np.arange(len(y)), y]
    np.testing.assert_allclose(lp, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(z, axis=1), rtol=0, atol=1e-12)
    # probabilities normalise
    np.testing.assert_allclose(np.exp(z - lse[:, None]).sum(1), 1.0, rtol=0, atol=1e-12)


def test_shift_invariance():
    h, U, y, rng = _case(2)
    c = rng.standard_normal(U.shape[1])
    lp1, _ = OP.token_logprobs(h, U, y)
    lp2, _ = OP.token_logprobs(h, U + c[None, :], y)
    np.testing.assert_allclose(lp1, lp2, rtol=0, atol=1e-10)


def test_invalid_target_is_nan_and_zero_grad():
    h, U, y, _ = _case(3)
    y = y.copy(); y[2] = U.shape[0]; y[4] = -1
    lp, _ = OP.token_logprobs(h, U, y)
    assert np.isnan(lp[2]) and np.isnan(lp[4]) and np.isfinite(np.delete(lp, [2, 4])).all()
    dh = OP.token_logprobs_backward(h, U, y, np.ones(len(y)))
    assert not dh[2].any() and not dh[4].any()


def test_backward_finite_differences():
    h, U, y, rng = _case(4, n=6, H=10, V=13)
    d = rng.standard_normal(len(y))
    dh = OP.token_logprobs_backward(h, U, y, d)
    f = lambda hh: float(np.sum(d * OP.token_logprobs(hh, U, y)[0]))
    eps = 1e-6
    for _ in range(5):
        D = rng.standard_normal(h.shape)
        fd = (f(h + eps * D) - f(h - eps * D)) / (2 * eps)
        assert abs(fd - np.sum(dh * D)) <= 1e-7 * max(1, abs(fd))


def test_backward_special_cases():
    h, U, y, rng = _case(5)
    Ue = np.tile(U[:1], (U.shape[0], 1))           # every vocab row equal
    assert np.allclose(OP.token_logprobs_backward(h, Ue, y, rng.standard_normal(len(y))), 0, atol=1e-14)
    d = rng.standard_normal(len(y)); d[[1, 3]] = 0
    dh = OP.token_logprobs_backward(h, U, y, d)
    assert not dh[1].any() and not dh[3].any()


def test_custom_surrogate_identity():
    """grad_h sum(g * l(h)) == grad_h C(l(h)) for g = dC/dl, C nonlinear
    (Deep Dive - Tinker, 'The RL datum shape'; forward_backward_custom post)."""
    h, U, y, rng = _case(6, n=5, H=8, V=11)
    C = lambda l: float(np.sum(np.sin(l) + 0.3 * l * l))
    lp, _ = OP.token_logprobs(h, U, y)
    g = np.cos(lp) + 0.6 * lp
    loss, dl = OLs.loss_grad(OLs.CUSTOM, lp, np.ones(len(y)), g=g)
    dh = OP.token_logprobs_backward(h, U, y, dl)
    eps = 1e-6
    for _ in range(4):
        D = rng.standard_normal(h.shape)
        fd = (C(OP.token_logprobs(h + eps * D, U, y)[0]) - C(OP.token_logprobs(h - eps * D, U, y)[0])) / (2 * eps)
        assert abs(fd - np.sum(dh * D)) <= 1e-7 * max(1, abs(fd))


# ---------------------------------------------------------------- losses
def _rl(seed=7, n=64, sigma=0.3):
    rng = np.random.default_rng(seed)
    l = -rng.random(n) * 5
    s = l + rng.standard_normal(n) * sigma
    A = rng.standard_normal(n)
    m = (rng.random(n) < 0.7).astype(np.float64)
    return l, s, A * m, m, rng


def test_ce_closed_form_and_fd():
    l, _, _, m, rng = _rl()
    w = m * rng.random(len(l))
    L, dl = OLs.loss_grad(OLs.CROSS_ENTROPY, l, w)
    assert np.array_equal(dl, np.where(w != 0, -w, 0.0))
    eps = 1e-6
    for t in range(len(l)):
        e = np.zeros(len(l)); e[t] = eps
        fd = (OLs.loss_grad(0, l + e, w)[0] - OLs.loss_grad(0, l - e, w)[0]) / (2 * eps)
        assert abs(fd - dl[t]) < 1e-8


def test_is_at_equal_logprobs():
    l, _, A, m, _ = _rl()
    L, dl = OLs.loss_grad(OLs.IMPORTANCE_SAMPLING, l, m, adv=A, samp=l)
    assert abs(L - (-np.sum(m * A))) < 1e-12
    np.testing.assert_array_equal(dl, np.where(m != 0, -A, 0.0))


@pytest.mark.parametrize("kind", [OLs.IMPORTANCE_SAMPLING, OLs.PPO])
def test_rl_losses_finite_differences(kind):
    l, s, A, m, _ = _rl(8)
    L, dl = OLs.loss_grad(kind, l, m, adv=A, samp=s)
    eps = 1e-7
    rho = np.exp(l - s)
    for t in range(len(l)):
        if kind == OLs.PPO and min(abs(rho[t] - 0.8), abs(rho[t] - 1.2)) < 1e-4:
            continue      # kink of the clipped objective
        e = np.zeros(len(l)); e[t] = eps
        fd = (OLs.loss_grad(kind, l + e, m, adv=A, samp=s)[0] - OLs.loss_grad(kind, l - e, m, adv=A, samp=s)[0]) / (2 * eps)
        assert abs(fd - dl[t]) < 1e-6 * max(1, abs(dl[t])), (t, fd, dl[t])


def test_ppo_equals_is_inside_clip_and_clips_outside():
    l, s, A, m, _ = _rl(9, sigma=0.01)      # every ratio within [0.8, 1.2]
    assert OLs.loss_grad(OLs.PPO, l, m, adv=A, samp=s)[0] == pytest.approx(
        OLs.loss_grad(OLs.IMPORTANCE_SAMPLING, l, m, adv=A, samp=s)[0], abs=1e-12)
    np.testing.assert_array_equal(OLs.loss_grad(OLs.PPO, l, m, adv=A, samp=s)[1],
                                  OLs.loss_grad(OLs.IMPORTANCE_SAMPLING, l, m, adv=A, samp=s)[1])
    # explicit clip cases
    l = np.log(np.array([1.5, 1.5, 0.5, 0.5, 1.19, 0.81]))
    s = np.zeros(6)
    A = np.array([1.0, -1.0, 1.0, -1.0, 1.0, -1.0])
    L, dl = OLs.loss_grad(OLs.PPO, l, np.ones(6), adv=A, samp=s)
    rho = np.exp(l)
    np.testing.assert_allclose(dl, [0.0, 1.5, -0.5, 0.0, -rho[4], rho[5]], rtol=1e-15, atol=0)
    assert L == pytest.approx(-(1.2 - 1.5 + 0.5 - 0.8 + 1.19 - 0.81), abs=1e-12)


def test_custom_with_minus_weights_is_ce():
    l, _, _, m, rng = _rl(10)
    w = m * rng.random(len(l))
    Lc, dc = OLs.loss_grad(OLs.CUSTOM, l, (w != 0).astype(float), g=-w)
    Le, de = OLs.loss_grad(OLs.CROSS_ENTROPY, l, w)
    assert Lc == pytest.approx(Le, abs=1e-12)
    np.testing.assert_array_equal(dc, de)


def test_constant_reward_group_gives_zero_rl_gradient():
    from workloads.datum import center
    A = np.repeat(center([1.0, 1.0, 1.0, 1.0]), 5)
    l = -np.random.default_rng(0).random(20)
    for kind in (OLs.IMPORTANCE_SAMPLING, OLs.PPO):
        L, dl = OLs.loss_grad(kind, l, np.ones(20), adv=A, samp=l + 0.1)
        assert L == 0.0 and not dl.any()


def test_masked_nonfinite_rows_are_exact_zeros():
    l, s, A, m, _ = _rl(11)
    m[:4] = 0
    l, s, A = l.copy(), s.copy(), A.copy()
    l[0], s[1], A[2], l[3] = np.nan, np.inf, np.nan, -np.inf
    for kind in range(4):
        L, dl = OLs.loss_grad(kind, l, m, adv=A, samp=s, g=np.where(m != 0, 1.0, np.nan))
        assert np.isfinite(L) and np.all(dl[:4] == 0.0) and np.isfinite(dl).all()


def test_sentinel_removes_kept_rows_with_nonfinite_inputs():
    """TPU RL note, section 12: a kept row whose own inputs hold NaN or +-Inf is
    neutralised (dl = 0, no loss term) and reported, for every kind; the other
    rows' results equal those of the batch with the bad rows masked out, and a
    bad value in an input the kind does not read changes nothing."""
    l, s, A, m, rng = _rl(12)
    m[:] = 1.0
    g = rng.standard_normal(len(l))
    plant = {  # kind -> rows and inputs to poison
        OLs.CROSS_ENTROPY: [("l", 3, np.nan), ("w", 9, np.inf)],
        OLs.IMPORTANCE_SAMPLING: [("l", 3, -np.inf), ("s", 9, np.nan), ("A", 20, np.inf)],
        OLs.PPO: [("s", 3, -np.inf), ("A", 9, np.nan), ("l", 20, np.nan)],
        OLs.CUSTOM: [("g", 3, np.nan), ("l", 9, np.inf)],
    }
    for kind, items in plant.items():
        arrs = {"l": l.copy(), "s": s.copy(), "A": A.copy(), "w": m.copy(), "g": g.copy()}
        rows = []
        for name, row, val in items:
            arrs[name][row] = val
            rows.append(row)
        L1, dl1, flag = OLs.loss_grad_flagged(kind, arrs["l"], arrs["w"], adv=arrs["A"],
                                              samp=arrs["s"], g=arrs["g"])
        assert flag and np.isfinite(L1) and np.all(np.isfinite(dl1))
        assert np.all(dl1[rows] == 0.0)
        # same as masking those rows by hand on clean inputs
        mm = m.copy()
        mm[rows] = 0.0
        L2, dl2, flag2 = OLs.loss_grad_flagged(kind, l, mm, adv=A, samp=s, g=g)
        assert not flag2
        assert L1 == L2 and np.array_equal(dl1, dl2)
    # inputs a kind does not read: CE ignores A, l_sampler and g
    L1, dl1, flag = OLs.loss_grad_flagged(OLs.CROSS_ENTROPY, l, m, adv=np.full(len(l), np.nan),
                                          samp=np.full(len(l), np.inf), g=np.full(len(l), np.nan))
    assert not flag and np.array_equal(dl1, -m)
    # masked rows never raise the sentinel
    mm = m.copy()
    mm[5] = 0.0
    ll = l.copy()
    ll[5] = np.nan
    assert not OLs.loss_grad_flagged(OLs.PPO, ll, mm, adv=A, samp=s)[2]
