"""Routed-expert layer (top-k MoE with a LoRA on every expert projection) on the
GPU against oracle.moe.  Per-call parity through the fused layer: the oracle
runs on the GPU's own routing output and, at every intermediate the layer
stores in bf16, continues from the GPU's stored bits (g, u, h from the saved
buffer; dh, dg, du from the backward's trace), while each of those
intermediates is itself compared with the oracle's value at the bf16
tolerance.  Intermediates the layer does not expose (expert outputs, per-
assignment dx) are rounded to bf16 at the same point."""
import numpy as np
import pytest
import torch

import oracle.moe as OE
import workloads as W
from gpu_util import TOL_BF16, TOL_F32, bits_of, dev_bf16, dev_f32, dev_i32, f64_of, rel_err

pytestmark = pytest.mark.gpu
L = pytest.importorskip("rl_lora_linear_amd.lib")


def _store(name, js, a):
    return W.bf16_bits_to_f64(W.to_bf16_bits(a))


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


class StageStore:
    """oracle.moe `store` hook: continue from the GPU's bits where known, round
    to bf16 elsewhere, and record (gpu, oracle) pairs."""
    def __init__(self, pos, gpu):
        self.pos, self.gpu, self.rec = pos, gpu, {}

    def __call__(self, name, js, v):
        if name in self.gpu:
            g = self.gpu[name][self.pos[js]]
            self.rec.setdefault(name, []).append((g, v))
            return g
        return _store(name, js, v)

    def check(self, names):
        for name in names:
            g = np.concatenate([a for a, _ in self.rec[name]])
            v = np.concatenate([b for _, b in self.rec[name]])
            assert rel_err(g, v) < TOL_BF16, name


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
    pos = position_of(c, e_np, ids)
    g, u, h = saved_views(dm, dm.saved)
    nk, F = c.n_tokens * c.top_k, c.d_ff
    dh, dg, du = trace_views(c, trace)
    Wg, Wu, Wd, A, B, s = dm.oracle_params()
    x = W.bf16_bits_to_f64(c.x_bits)
    st = StageStore(pos, {"g": g, "u": u, "h": h, "dh": dh, "dg": dg, "du": du})
    y_ref, saved = OE.moe_forward(x, e_np, w_np, ids, Wg, Wu, Wd, A, B, s, store=st)
    assert rel_err(f64_of(y), y_ref) < TOL_BF16
    dy = W.bf16_bits_to_f64(c.dy_bits)
    dx_ref, dA_ref, dB_ref = OE.moe_backward(dy, x, e_np, w_np, ids, Wg, Wu, Wd, A, B, s, saved,
                                             store=st)
    st.check(["g", "u", "h", "dh", "dg", "du"])
    assert rel_err(f64_of(dx), dx_ref) < TOL_BF16
    for p, gr in zip(("gate", "up", "down"), grads):
        dA, dB = dm.split_grad(p, gr.cpu().numpy().astype(np.float64))
        for a in range(c.n_adapters):
            for e in range(c.n_experts):
                if (a, e) in getattr(dm, "zero_pairs", []):
                    continue
                assert rel_err(dA[a][e], dA_ref[p][a][e]) < TOL_F32, (p, a, e, "dA")
                assert rel_err(dB[a][e], dB_ref[p][a][e]) < TOL_F32, (p, a, e, "dB")


@pytest.mark.parametrize("kind", ["small", "wide", "rank48"])
def test_moe_forward_backward_parity(kind):
    """small/wide: ranks 16 and 32 (gate and up share one pass over x in the
    shrink and the dA reduction); rank48: max_rank 64, the two-pass path."""
    if kind == "small":
        c = _case()
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
