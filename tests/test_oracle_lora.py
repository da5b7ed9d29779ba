"""Pins for oracle.segments and oracle.lora (CPU only).

Each test checks the oracle against something other than itself: brute-force
ordering, the merged-weight form W' = W + gamma B A (Deep Dive - Tinker,
"Checkpoints and export paths"), the frozen-base special case B = 0, finite
differences in float64, and the adapter-isolation property (OpenTinker,
"3 Approach": adapter-local gradients).
"""
import numpy as np
import pytest

import oracle.lora as OL
import oracle.segments as OS
import workloads as W


# ---------------------------------------------------------------- segments
@pytest.mark.parametrize("n,n_keys,seed", [(0, 3, 0), (1, 1, 1), (37, 5, 2), (300, 16, 3), (513, 64, 4)])
def test_segments_brute_force(n, n_keys, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(-2, n_keys + 2, size=n)           # includes invalid ids
    perm, off = OS.segments(ids, n_keys)
    # brute force: Python sort on (key, token index), invalid keys last
    keyed = [(i if 0 <= i < n_keys else n_keys, t) for t, i in enumerate(ids.tolist())]
    want_perm = [t for _, t in sorted(keyed)]
    assert perm.tolist() == want_perm
    want_off = [0]
    for k in range(n_keys):
        want_off.append(want_off[-1] + sum(1 for i in ids.tolist() if i == k))
    assert off.tolist() == want_off


def test_segments_empty_keys_repeat_offsets():
    ids = np.array([0, 0, 3, 3, 3])
    perm, off = OS.segments(ids, 5)
    assert off.tolist() == [0, 2, 2, 2, 5, 5]
    assert perm.tolist() == [0, 1, 2, 3, 4]


# ---------------------------------------------------------------- forward
def _small_case(seed=0, n=40, d_in=24, d_out=20, ranks=(2, 4, 8), order="interleaved"):
    c = W.lora_layer(seed, n, d_in, d_out, list(ranks), [16.0, 8.0, 4.0][:len(ranks)], order=order)
    A = [c.A(i) for i in range(c.n_adapters)]
    B = [c.B(i) for i in range(c.n_adapters)]
    return c, A, B


def test_forward_merged_equals_unmerged():
    c, A, B = _small_case()
    y, _ = OL.lora_forward(c.x(), c.W(), A, B, c.scales, c.ids)
    # merged weight per token, looping over tokens (independent of the grouping)
    x, Wb = c.x(), c.W()
    y2 = np.empty_like(y)
    for t in range(c.n_tokens):
        a = int(c.ids[t])
        Wm = Wb + c.scales[a] * (B[a] @ A[a])
        y2[t] = Wm @ x[t]
    np.testing.assert_allclose(y, y2, rtol=0, atol=1e-12)
    y3 = OL.merged_forward(x, Wb, A, B, c.scales, c.ids)
    np.testing.assert_allclose(y, y3, rtol=0, atol=1e-12)


def test_forward_B_zero_is_base_exactly():
    c, A, B = _small_case(1)
    Bz = [np.zeros_like(b) for b in B]
    y, u = OL.lora_forward(c.x(), c.W(), A, Bz, c.scales, c.ids)
    assert np.array_equal(y, c.x() @ c.W().T)
    assert np.any(u != 0)


def test_forward_single_adapter_is_dense_lora():
    c, A, B = _small_case(2, ranks=(8,))
    ids = np.zeros(c.n_tokens, np.int32)
    y, u = OL.lora_forward(c.x(), c.W(), A, B, c.scales, ids)
    import torch
    xt = torch.from_numpy(c.x())
    lin = torch.nn.functional.linear
    dense = lin(xt, torch.from_numpy(c.W())) + c.scales[0] * lin(lin(xt, torch.from_numpy(A[0])), torch.from_numpy(B[0]))
    np.testing.assert_allclose(y, dense.numpy(), rtol=0, atol=1e-12)


def test_forward_absent_adapter_changes_nothing():
    c, A, B = _small_case(3)
    ids = np.where(c.ids == 1, 0, c.ids).astype(np.int32)   # adapter 1 owns no token
    y, u = OL.lora_forward(c.x(), c.W(), A, B, c.scales, ids)
    B2 = list(B)
    B2[1] = B[1] * 7.0 + 3.0
    A2 = list(A)
    A2[1] = A[1] - 1.0
    y2, u2 = OL.lora_forward(c.x(), c.W(), A2, B2, c.scales, ids)
    assert np.array_equal(y, y2) and np.array_equal(u, u2)


def test_forward_invalid_ids_get_base_only():
    c, A, B = _small_case(4)
    ids = c.ids.copy()
    ids[[0, 5]] = [-1, 99]
    y, u = OL.lora_forward(c.x(), c.W(), A, B, c.scales, ids)
    base = c.x() @ c.W().T
    assert np.array_equal(y[[0, 5]], base[[0, 5]])
    assert np.all(u[[0, 5]] == 0)


def test_forward_permutation_equivariant():
    c, A, B = _small_case(5)
    rng = np.random.default_rng(9)
    p = rng.permutation(c.n_tokens)
    y, u = OL.lora_forward(c.x(), c.W(), A, B, c.scales, c.ids)
    yp, up = OL.lora_forward(c.x()[p], c.W(), A, B, c.scales, c.ids[p])
    np.testing.assert_allclose(yp, y[p], rtol=0, atol=1e-12)
    np.testing.assert_allclose(up, u[p], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- backward
def _objective(x, Wb, A, B, s, ids, dy):
    y, _ = OL.lora_forward(x, Wb, A, B, s, ids)
    return float(np.sum(y * dy))


def test_backward_finite_differences():
    """Central differences of L = sum(y * dY) along seeded random directions and
    on a seeded subset of coordinates."""
    c, A, B = _small_case(6, n=30, d_in=12, d_out=10)
    x, Wb, dy, s, ids = c.x(), c.W(), c.dy(), c.scales, c.ids
    dx, dA, dB, v = OL.lora_backward(dy, x, Wb, A, B, s, ids)
    rng = np.random.default_rng(11)
    h = 1e-5
    for _ in range(4):
        Dx = rng.standard_normal(x.shape)
        DA = [rng.standard_normal(a.shape) for a in A]
        DB = [rng.standard_normal(b.shape) for b in B]
        f = lambda e: _objective(x + e * Dx, Wb, [a + e * da for a, da in zip(A, DA)],
                                 [b + e * db for b, db in zip(B, DB)], s, ids, dy)
        fd = (f(h) - f(-h)) / (2 * h)
        an = np.sum(dx * Dx) + sum(np.sum(g * d) for g, d in zip(dA, DA)) + sum(np.sum(g * d) for g, d in zip(dB, DB))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an))
    # coordinates
    for _ in range(12):
        i = int(rng.integers(0, len(A)))
        which = rng.integers(0, 3)
        if which == 0:
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            E = np.zeros_like(x); E[idx] = 1
            f = lambda e: _objective(x + e * E, Wb, A, B, s, ids, dy)
            an = dx[idx]
        elif which == 1:
            idx = tuple(int(rng.integers(0, n)) for n in A[i].shape)
            E = np.zeros_like(A[i]); E[idx] = 1
            f = lambda e: _objective(x, Wb, [a + e * E if j == i else a for j, a in enumerate(A)], B, s, ids, dy)
            an = dA[i][idx]
        else:
            idx = tuple(int(rng.integers(0, n)) for n in B[i].shape)
            E = np.zeros_like(B[i]); E[idx] = 1
            f = lambda e: _objective(x, Wb, A, [b + e * E if j == i else b for j, b in enumerate(B)], s, ids, dy)
            an = dB[i][idx]
        fd = (f(h) - f(-h)) / (2 * h)
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an))
    # v is B^T dY per token
    for t in range(c.n_tokens):
        a = int(ids[t]); r = A[a].shape[0]
        np.testing.assert_allclose(v[t, :r], B[a].T @ dy[t], rtol=0, atol=1e-12)


def test_backward_no_leak_bitwise():
    """Changing the values (not the routing) of adapter 0's tokens leaves every
    other adapter's dA, dB bitwise unchanged."""
    c, A, B = _small_case(7)
    x, dy = c.x(), c.dy()
    dx, dA, dB, _ = OL.lora_backward(dy, x, c.W(), A, B, c.scales, c.ids)
    rows = c.ids == 0
    x2, dy2 = x.copy(), dy.copy()
    x2[rows] = x2[rows] * -3.0 + 1.0
    dy2[rows] = dy2[rows] * 5.0 - 2.0
    dx2, dA2, dB2, _ = OL.lora_backward(dy2, x2, c.W(), A, B, c.scales, c.ids)
    for j in range(1, c.n_adapters):
        assert np.array_equal(dA[j], dA2[j]) and np.array_equal(dB[j], dB2[j])
    assert not np.array_equal(dA[0], dA2[0])
    assert np.array_equal(dx[~rows], dx2[~rows])


def test_backward_B_zero_and_absent_adapter():
    c, A, B = _small_case(8)
    Bz = [np.zeros_like(b) for b in B]
    dx, dA, dB, v = OL.lora_backward(c.dy(), c.x(), c.W(), A, Bz, c.scales, c.ids)
    assert all(np.array_equal(a, np.zeros_like(a)) for a in dA)
    assert np.array_equal(dx, c.dy() @ c.W())
    ids = np.where(c.ids == 2, 1, c.ids).astype(np.int32)
    _, dA, dB, _ = OL.lora_backward(c.dy(), c.x(), c.W(), A, B, c.scales, ids)
    assert not np.any(dA[2]) and not np.any(dB[2])


def test_closed_form_flop_overhead():
    """tinker-ticks: shrink + expand add 2*r/d of the base GEMM's FLOPs."""
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")))
    r, d = g["lora_flop_overhead"]["rank"], g["lora_flop_overhead"]["hidden"]
    n = 1000
    base = 2 * n * d * d
    lora = 2 * n * d * r + 2 * n * r * d
    assert lora / base == g["lora_flop_overhead"]["fraction"]
    assert round(100 * lora / base, 1) == g["lora_flop_overhead"]["printed_percent"]
    s = g["sgmv_calls_per_forward"]
    assert s["projections_per_layer"] * s["layers"] == s["calls"]


def test_u_is_pinned_by_the_merged_weight_with_identity_B():
    """u_t = A_a x_t: with d_out = r and B_a = I the merged weight W + s A_a
    gives y_t - W x_t = s u_t, so u is checked against the merged form, which
    never forms u."""
    rng = np.random.default_rng(41)
    n, d_in, r = 30, 12, 4
    ids = rng.integers(-1, 3, size=n)                 # includes an invalid id
    A = [rng.standard_normal((r, d_in)) for _ in range(3)]
    B = [np.eye(r) for _ in range(3)]
    s = np.array([2.0, 0.5, 1.25])
    x = rng.standard_normal((n, d_in))
    Wb = rng.standard_normal((r, d_in))
    _, u = OL.lora_forward(x, Wb, A, B, s, ids)
    y_m = OL.merged_forward(x, Wb, A, B, s, ids)
    for t in range(n):
        a = int(ids[t])
        if 0 <= a < 3:
            np.testing.assert_allclose(u[t], (y_m[t] - Wb @ x[t]) / s[a], rtol=0, atol=1e-12)
        else:
            assert not u[t].any()
