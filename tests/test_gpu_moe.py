"""Routed-expert layer (top-k MoE with a LoRA on every expert projection) on the
GPU against oracle.moe.

Two checks per case:
  * end to end: oracle.moe's plain float64 definition on the same inputs and
    the GPU's own routing; y, dx and every (expert, adapter) pair's dA and dB.
    The layer keeps its stage tensors in bf16 (gate/up pre-activations, h, dh,
    dgate, dup), so each result carries several bf16 roundings: the bar is the
    norm-wise relative error within the bf16 tolerance and every element
    within 2.5x it, the latter for pairs of at least 16 assignments
    (gpu_util.check_chained);
  * per stage (diagnostic, per-call parity): each stage the layer stores --
    gate/up pre-activations, h (saved buffer), dh, dgate, dup (backward trace)
    -- against the oracle's projections (oracle.lora) and SwiGLU (oracle.mlp)
    evaluated on the GPU's own previous stage bits, and the gradients of those
    per-call products at the fp32 tolerance.
"""
import numpy as np
import pytest
import torch

import oracle.lora as OL
import oracle.mlp as OM
import oracle.moe as OE
import workloads as W
from gpu_util import TOL_BF16, TOL_F32, bits_of, check_chained, dev_bf16, dev_f32, dev_i32, f64_of, rel_err

pytestmark = pytest.mark.gpu
L = pytest.importorskip("rl_lora_linear_amd.lib")


def _align(n, a=256):
    return (n + a - 1) // a * a


def no_adapter_ids(c, ids):
    """Adapter ids with every out-of-range id mapped to n_adapters ("no adapter")."""
    return np.where((ids >= 0) & (ids < c.n_adapters), ids, c.n_adapters)


def position_of(c, experts, ids):
    """Assignment -> position: stable sort by e*(n_ad+1) + a (valid expert ids)."""
    K = c.top_k
    a = np.repeat(no_adapter_ids(c, ids), K)
    keys = experts.reshape(-1).astype(np.int64) * (c.n_adapters + 1) + a
    perm = np.argsort(keys, kind="stable")
    pos = np.empty_like(perm)
    pos[perm] = np.arange(perm.size)
    return pos


def saved_views(dm, saved):
    """g, u, h (float64 [N*K][F], position order) from the saved buffer: rows of
    [gate | up] pre-activations, then h."""
    c = dm.c
    nk, F = c.n_tokens * c.top_k, c.d_ff
    raw = saved.cpu().numpy()
    gu = W.bf16_bits_to_f64(raw[:nk * 2 * F * 2].view(np.uint16)).reshape(nk, 2 * F)
    off = _align(nk * 2 * F * 2)
    h = W.bf16_bits_to_f64(raw[off:off + nk * F * 2].view(np.uint16)).reshape(nk, F)
    return gu[:, :F], gu[:, F:], h


def trace_views(c, trace):
    """dh, dg, du (float64 [N*K][F], position order) from the backward trace."""
    nk, F = c.n_tokens * c.top_k, c.d_ff
    flat = W.bf16_bits_to_f64(bits_of(trace)).reshape(-1)
    dgu = flat[nk * F:].reshape(nk, 2 * F)
    return flat[:nk * F].reshape(nk, F), dgu[:, :F], dgu[:, F:]


def _pairs(experts, ids):
    """(expert, adapter) -> assignment indices j = t*K + k, in increasing j."""
    n, K = experts.shape
    e_flat = experts.reshape(-1)
    a_flat = np.repeat(np.asarray(ids), K)
    out = {}
    for j in range(n * K):
        out.setdefault((int(e_flat[j]), int(a_flat[j])), []).append(j)
    return {key: np.asarray(v, np.int64) for key, v in out.items()}


def staged_parity(x, dy, experts, weights, ids, Wg, Wu, Wd, A, B, scale, stages, y, dx,
                  grad_of=None, skip_pair=lambda e, a: False):
    """Per-call parity through the fused layer, built from oracle.lora and
    oracle.mlp: every stored stage against the oracle evaluated on the GPU's
    own previous stage.  stages(name, js) -> float64 rows of the GPU's stage
    `name` for assignments js.  y and dx are rebuilt from those per-call
    results and compared at the bf16 tolerance; grad_of(p, e, a) -> the GPU's
    (dA, dB) of that pair, compared with the per-call oracle at the fp32
    tolerance.  y or dx None: not compared (a batch that holds only some of
    its tokens' assignments).  Returns the number of pairs checked."""
    n, K = experts.shape
    w_flat = np.asarray(weights, np.float64).reshape(-1)
    y_st = np.zeros((n, x.shape[1]))
    dx_st = np.zeros_like(y_st)
    got = {nm: [] for nm in ("g", "u", "h", "dh", "dg", "du")}
    want = {nm: [] for nm in got}
    checked = 0
    for (e, a), js in _pairs(experts, ids).items():
        ts = js // K
        xs, s = x[ts], scale(a)
        one = np.zeros(len(js), np.int64)
        def fwd(p, Wp, inp):
            return OL.lora_forward(inp, Wp[e], [A[p][a][e]], [B[p][a][e]], [s], one)[0]
        def bwd(p, Wp, g_up, inp):
            return OL.lora_backward(g_up, inp, Wp[e], [A[p][a][e]], [B[p][a][e]], [s], one)
        gg, uu, hh = stages("g", js), stages("u", js), stages("h", js)
        for nm, gpu, ref in (("g", gg, fwd("gate", Wg, xs)), ("u", uu, fwd("up", Wu, xs)),
                             ("h", hh, OM.swiglu_forward(gg, uu))):
            got[nm].append(gpu)
            want[nm].append(ref)
        o = fwd("down", Wd, hh)
        np.add.at(y_st, ts, w_flat[js][:, None] * o)
        do = w_flat[js][:, None] * dy[ts]
        dh_ref, dA_d, dB_d, _ = bwd("down", Wd, do, hh)
        dh = stages("dh", js)
        dg_ref, du_ref = OM.swiglu_backward(dh, gg, uu)
        dg, du = stages("dg", js), stages("du", js)
        for nm, gpu, ref in (("dh", dh, dh_ref), ("dg", dg, dg_ref), ("du", du, du_ref)):
            got[nm].append(gpu)
            want[nm].append(ref)
        dxg, dA_g, dB_g, _ = bwd("gate", Wg, dg, xs)
        dxu, dA_u, dB_u, _ = bwd("up", Wu, du, xs)
        np.add.at(dx_st, ts, dxg + dxu)
        if grad_of is not None and not skip_pair(e, a):
            for p, dA_r, dB_r in (("gate", dA_g, dB_g), ("up", dA_u, dB_u), ("down", dA_d, dB_d)):
                gA, gB = grad_of(p, e, a)
                assert rel_err(gA, dA_r[0]) < TOL_F32, (p, e, a, "dA per call")
                assert rel_err(gB, dB_r[0]) < TOL_F32, (p, e, a, "dB per call")
            checked += 1
    for nm in got:
        assert rel_err(np.concatenate(got[nm]), np.concatenate(want[nm])) < TOL_BF16, nm
    if y is not None:
        assert rel_err(y, y_st) < TOL_BF16
    if dx is not None:
        assert rel_err(dx, dx_st) < TOL_BF16
    return checked


class DevMoe:
    def __init__(self, c: "W.MoeCase", desc_override=None):
        self.c = c
        E, F, H = c.n_experts, c.d_ff, c.hidden
        self.x = dev_bf16(c.x_bits)
        self.dy = dev_bf16(c.dy_bits)
        self.Wg, self.Wu, self.Wd = dev_bf16(c.Wg_bits), dev_bf16(c.Wu_bits), dev_bf16(c.Wd_bits)
        self.Wgt = torch.empty((E, H, F), dtype=torch.bfloat16, device="cuda")
        self.Wut = torch.empty((E, H, F), dtype=torch.bfloat16, device="cuda")
        self.Wdt = torch.empty((E, F, H), dtype=torch.bfloat16, device="cuda")
        for e in range(E):
            L.lora_transpose_bf16(self.Wg[e], self.Wgt[e])
            L.lora_transpose_bf16(self.Wu[e], self.Wut[e])
            L.lora_transpose_bf16(self.Wd[e], self.Wdt[e])
        self.packs = [dev_bf16(c.pack_g), dev_bf16(c.pack_u), dev_bf16(c.pack_d)]
        s = np.float32(c.alpha / c.rank)
        self.descs = []
        for p in ("gate", "up", "down"):
            a_off, b_off = [], []
            for e in range(E):
                for a in range(c.n_adapters):
                    ao, bo = c.offsets(p, a, e)
                    a_off.append(ao)
                    b_off.append(bo)
            ranks = np.full(len(a_off), c.rank, np.int32)
            if desc_override:
                ranks = desc_override(p, ranks)
            self.descs.append(L.make_desc(a_off, b_off, ranks, np.full(len(a_off), s, np.float32)))
        self.ids = dev_i32(c.ids)
        self.logits = dev_f32(c.router_logits)
        R = max(16, int(np.ceil(c.rank / 16) * 16))
        self.shape = L.MoeShape(c.n_tokens, H, F, c.pack_g.size, c.pack_u.size, c.pack_d.size, E,
                                c.top_k, c.n_adapters, R)
        self.ws = L.empty_workspace(L.moe_workspace_bytes(self.shape))
        self.saved = torch.empty(L.moe_saved_bytes(self.shape), dtype=torch.uint8, device="cuda")

    def route(self):
        n, K = self.c.n_tokens, self.c.top_k
        ex = torch.empty((n, K), dtype=torch.int32, device="cuda")
        w = torch.empty((n, K), dtype=torch.float32, device="cuda")
        L.moe_route(self.logits, K, ex, w)
        return ex, w

    def forward(self, ex, w, ids=None):
        y = torch.empty((self.c.n_tokens, self.c.hidden), dtype=torch.bfloat16, device="cuda")
        L.moe_forward(self.shape, self.x, ex, w, self.ids if ids is None else ids, self.Wg, self.Wu,
                      self.Wd, self.packs, self.descs, y, self.saved, self.ws)
        return y

    def new_trace(self):
        c = self.c
        return torch.empty((3, c.n_tokens * c.top_k, c.d_ff), dtype=torch.bfloat16, device="cuda")

    def backward(self, ex, w, ids=None, accumulate=False, grads=None, trace=None):
        dx = torch.empty((self.c.n_tokens, self.c.hidden), dtype=torch.bfloat16, device="cuda")
        if grads is None:
            grads = [torch.full((p.numel(),), float("nan"), dtype=torch.float32, device="cuda")
                     for p in self.packs]
        L.moe_backward(self.shape, self.dy, self.x, ex, w, self.ids if ids is None else ids,
                       self.Wgt, self.Wut, self.Wdt, self.packs, self.descs, self.saved, dx, grads,
                       accumulate, self.ws, trace=trace)
        return dx, grads

    def oracle_params(self):
        c = self.c
        packs = {"gate": c.pack_g, "up": c.pack_u, "down": c.pack_d}
        A, B = {}, {}
        for p in ("gate", "up", "down"):
            d_in, d_out = (c.d_ff, c.hidden) if p == "down" else (c.hidden, c.d_ff)
            A[p] = [[None] * c.n_experts for _ in range(c.n_adapters)]
            B[p] = [[None] * c.n_experts for _ in range(c.n_adapters)]
            for a in range(c.n_adapters):
                for e in range(c.n_experts):
                    ao, bo = c.offsets(p, a, e)
                    A[p][a][e] = W.bf16_bits_to_f64(packs[p][ao:ao + c.rank * d_in]).reshape(c.rank, d_in)
                    B[p][a][e] = W.bf16_bits_to_f64(packs[p][bo:bo + d_out * c.rank]).reshape(d_out, c.rank)
            # index n_adapters: "no adapter" (zero factors); rank-0 pairs likewise
            A[p].append([np.zeros_like(m) for m in A[p][0]])
            B[p].append([np.zeros_like(m) for m in B[p][0]])
            for (a, e) in getattr(self, "zero_pairs", []):
                A[p][a][e] = np.zeros_like(A[p][a][e])
                B[p][a][e] = np.zeros_like(B[p][a][e])
        Wg = W.bf16_bits_to_f64(c.Wg_bits)
        Wu = W.bf16_bits_to_f64(c.Wu_bits)
        Wd = W.bf16_bits_to_f64(c.Wd_bits)
        return Wg, Wu, Wd, A, B, c.alpha / c.rank

    def split_grad(self, p, g):
        c = self.c
        d_in, d_out = (c.d_ff, c.hidden) if p == "down" else (c.hidden, c.d_ff)
        dA = [[None] * c.n_experts for _ in range(c.n_adapters)]
        dB = [[None] * c.n_experts for _ in range(c.n_adapters)]
        for a in range(c.n_adapters):
            for e in range(c.n_experts):
                ao, bo = c.offsets(p, a, e)
                dA[a][e] = g[ao:ao + c.rank * d_in].reshape(c.rank, d_in)
                dB[a][e] = g[bo:bo + d_out * c.rank].reshape(d_out, c.rank)
        return dA, dB


def _case(n=300, H=256, F=192, E=8, K=2, n_ad=3, r=16, seed=21):
    return W.moe_layer(seed=seed, n_tokens=n, hidden=H, d_ff=F, n_experts=E, top_k=K,
                       n_adapters=n_ad, rank=r)


@pytest.mark.parametrize("E,K", [(8, 2), (128, 8), (40, 3)])
def test_route_matches_oracle(E, K):
    rng = np.random.default_rng(E)
    n = 257
    R = rng.standard_normal((n, E)).astype(np.float32)
    R[5, :] = 0.25                       # all tied: the lowest indices win
    R[6, 3] = R[6, 7] = R[6].max() + 1   # a tie for first place
    ex = torch.empty((n, K), dtype=torch.int32, device="cuda")
    w = torch.empty((n, K), dtype=torch.float32, device="cuda")
    L.moe_route(dev_f32(R), K, ex, w)
    e_ref, w_ref = OE.moe_route(R, K)
    assert np.array_equal(ex.cpu().numpy(), e_ref)
    assert rel_err(w.cpu().numpy(), w_ref) < TOL_F32
    assert list(ex.cpu().numpy()[5]) == list(range(K))


def run_parity(dm, ex, w, y, dx, grads, trace, ids=None):
    c = dm.c
    ids = no_adapter_ids(c, c.ids if ids is None else ids)
    e_np, w_np = ex.cpu().numpy().astype(np.int64), w.cpu().numpy().astype(np.float64)
    Wg, Wu, Wd, A, B, s = dm.oracle_params()
    x = W.bf16_bits_to_f64(c.x_bits)
    dy = W.bf16_bits_to_f64(c.dy_bits)
    yg, dxg = f64_of(y), f64_of(dx)
    zero = set(getattr(dm, "zero_pairs", []))
    # end to end: the plain definition
    y_ref, saved = OE.moe_forward(x, e_np, w_np, ids, Wg, Wu, Wd, A, B, s)
    check_chained(yg, y_ref, "y")
    dx_ref, dA_ref, dB_ref = OE.moe_backward(dy, x, e_np, w_np, ids, Wg, Wu, Wd, A, B, s, saved)
    check_chained(dxg, dx_ref, "dx")
    gv = {p: dm.split_grad(p, gr.cpu().numpy().astype(np.float64))
          for p, gr in zip(("gate", "up", "down"), grads)}
    rows = {key: len(js) for key, js in _pairs(e_np, ids).items()}   # (expert, adapter)
    for p in ("gate", "up", "down"):
        dA, dB = gv[p]
        for a in range(c.n_adapters):
            for e in range(c.n_experts):
                if (a, e) in zero:
                    continue
                t = rows.get((e, a), 0)
                check_chained(dA[a][e], dA_ref[p][a][e], f"{p} dA {a} {e}", terms=t)
                check_chained(dB[a][e], dB_ref[p][a][e], f"{p} dB {a} {e}", terms=t)
    # per stage, from the GPU's own stage bits
    pos = position_of(c, e_np, ids)
    g, u, h = saved_views(dm, dm.saved)
    dh, dg, du = trace_views(c, trace)
    views = {"g": g, "u": u, "h": h, "dh": dh, "dg": dg, "du": du}
    staged_parity(x, dy, e_np, w_np, ids, Wg, Wu, Wd, A, B, lambda a: s,
                  lambda nm, js: views[nm][pos[js]], yg, dxg,
                  grad_of=lambda p, e, a: (gv[p][0][a][e], gv[p][1][a][e]),
                  skip_pair=lambda e, a: a >= c.n_adapters or (a, e) in zero)


@pytest.mark.parametrize("kind", ["small", "mid", "wide", "rank48"])
def test_moe_forward_backward_parity(kind):
    """small/mid/wide: ranks 16 and 32 (gate and up share one pass over x in the
    shrink and the dA reduction); mid: 16 experts, top-4, 3 adapters; rank48:
    max_rank 64, the two-pass path."""
    if kind == "small":
        c = _case()
    elif kind == "mid":
        c = _case(n=1000, H=256, F=192, E=16, K=4, n_ad=3, r=32, seed=26)
    elif kind == "wide":
        c = _case(n=700, H=320, F=128, E=6, K=3, n_ad=2, r=32, seed=22)
    else:
        c = _case(n=400, H=192, F=256, E=5, K=2, n_ad=2, r=48, seed=25)
    dm = DevMoe(c)
    ex, w = dm.route()
    y = dm.forward(ex, w)
    trace = dm.new_trace()
    dx, grads = dm.backward(ex, w, trace=trace)
    assert L.lora_device_status(dm.ws) == 0
    run_parity(dm, ex, w, y, dx, grads, trace)


def test_moe_accumulate_repeatable_and_invalid_ids():
    c = _case(n=200, seed=23)
    dm = DevMoe(c)
    ex, w = dm.route()
    dm.forward(ex, w)
    dx1, g1 = dm.backward(ex, w)
    dx2, g2 = dm.backward(ex, w)
    assert torch.equal(dx1.view(torch.int16), dx2.view(torch.int16))
    assert all(torch.equal(a, b) for a, b in zip(g1, g2))           # bitwise repeatable
    g3 = [g.clone() for g in g1]
    dm.backward(ex, w, accumulate=True, grads=g3)
    for a, b in zip(g3, g1):
        np.testing.assert_allclose(a.cpu().numpy(), 2 * b.cpu().numpy(), rtol=1e-6, atol=0)
    # tokens with an adapter id out of range get the base experts only: the
    # oracle reading is "no adapter" (zero LoRA factors) for those tokens
    ids = c.ids.copy()
    ids[[0, 7]] = [-1, c.n_adapters]
    y = dm.forward(ex, w, ids=dev_i32(ids))
    trace = dm.new_trace()
    dx, grads = dm.backward(ex, w, ids=dev_i32(ids), trace=trace)
    assert L.lora_device_status(dm.ws) & L.FLAG_ID_RANGE
    run_parity(dm, ex, w, y, dx, grads, trace, ids=ids)


def test_moe_rank_zero_pair_is_no_adapter():
    """A (expert, adapter) entry with rank 0 in the tables means no LoRA for that
    pair: its tokens get the base expert, its gradient region is untouched."""
    c = _case(n=256, seed=24)
    def override(p, ranks):
        r = ranks.copy()
        r[1 * c.n_adapters + 2] = 0        # expert 1, adapter 2
        return r
    dm = DevMoe(c, desc_override=override)
    ex, w = dm.route()
    y = dm.forward(ex, w)
    trace = dm.new_trace()
    dx, grads = dm.backward(ex, w, trace=trace)
    assert L.lora_device_status(dm.ws) == 0
    for p, g in zip(("gate", "up", "down"), grads):
        dA, dB = dm.split_grad(p, g.cpu().numpy())
        assert np.all(np.isnan(dA[2][1])) and np.all(np.isnan(dB[2][1]))   # untouched
    dm.zero_pairs = [(2, 1)]
    run_parity(dm, ex, w, y, dx, grads, trace)


@pytest.mark.parametrize("seed", range(8))
def test_moe_random_shapes(seed):
    """Seeded random routed layers: 2-32 experts, top-1 to top-8, H and F
    multiples of 64 up to 384, 1-4 adapters of one rank (a multiple of 8 up to
    64), batches from 1 to 1500 tokens; the end-to-end and per-stage checks of
    the hand-picked cases."""
    rng = np.random.default_rng(500 + seed)
    E = int(rng.integers(2, 33))
    K = int(rng.integers(1, min(8, E) + 1))
    n = int(rng.choice([1, 17, 130, 600, 1500]))
    H, F = 64 * int(rng.integers(1, 7)), 64 * int(rng.integers(1, 7))
    n_ad, r = int(rng.integers(1, 5)), 8 * int(rng.integers(1, 9))
    print(f"[moe random] seed {seed}: n {n} H {H} F {F} E {E} K {K} adapters {n_ad} r {r}",
          flush=True)
    c = _case(n=n, H=H, F=F, E=E, K=K, n_ad=n_ad, r=r, seed=600 + seed)
    dm = DevMoe(c)
    ex, w = dm.route()
    y = dm.forward(ex, w)
    trace = dm.new_trace()
    dx, grads = dm.backward(ex, w, trace=trace)
    assert L.lora_device_status(dm.ws) == 0
    run_parity(dm, ex, w, y, dx, grads, trace)
