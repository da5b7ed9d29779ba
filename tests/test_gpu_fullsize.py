"""Full-size parity: the workloads bench.py times, at their sizes and with the
same inputs and launch configuration, checked on sampled outputs the oracle
computes one by one.  Rows are independent through every projection, so a
sampled row's output is exact from the row alone; an adapter's (or an
(expert, adapter) pair's) gradient is the sum over its own rows, computed
whole.  The fused expert and MLP layers are compared with the plain oracle
(end to end, bf16 tolerance) and, per stage, with oracle.lora / oracle.mlp
calls on the GPU's own stored stage bits, as in the small-size tests."""
import numpy as np
import pytest
import torch

import oracle.logprob as OP
import oracle.loss as OLs
import oracle.lora as OL
import oracle.moe as OE
import workloads as W
import workloads.device as WD
from gpu_util import TOL_BF16, TOL_F32, DevLayer, check_chained, f64_of, rel_err
from test_gpu_moe import staged_parity

pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)
L = pytest.importorskip("rl_lora_linear_amd.lib")


# ---------------------------------------------------------------- q/o projection
def test_qo_proj_full_size():
    """8192 tokens, 4096x4096, 16 rank-32 adapters in sorted segments."""
    c = W.attn_proj(seed=2)
    dl = DevLayer(c)
    y, u = dl.forward()
    dx, grad = dl.backward(u)
    assert dl.status() == 0
    x, Wb, A, B, s, ids = dl.oracle_args()
    dy = c.dy()
    rows = np.sort(np.random.default_rng(7).choice(c.n_tokens, 48, replace=False))
    y_ref, u_ref = OL.lora_forward(x[rows], Wb, A, B, s, ids[rows])
    assert rel_err(f64_of(y)[rows], y_ref) < TOL_BF16
    assert rel_err(dl.u_values(u)[rows][:, :u_ref.shape[1]], u_ref) < TOL_F32
    dx_ref, _, _, _ = OL.lora_backward(dy[rows], x[rows], Wb, A, B, s, ids[rows])
    assert rel_err(f64_of(dx)[rows], dx_ref) < TOL_BF16
    dA, dB = dl.split_grad(f64_of(grad))
    for a in (0, 9, 15):
        ra = np.nonzero(ids == a)[0]
        _, dA_ref, dB_ref, _ = OL.lora_backward(dy[ra], x[ra], Wb, A, B, s, ids[ra])
        assert rel_err(dA[a], dA_ref[a]) < TOL_F32, ("dA", a)
        assert rel_err(dB[a], dB_ref[a]) < TOL_F32, ("dB", a)


# ---------------------------------------------------------------- expert layers
def _stage_fetch(saved, trace, NK, F):
    """Row fetchers (positions -> float64 rows) for the saved [gate | up] and h
    rows and the backward trace (dh, [dgate | dup])."""
    sb = saved.view(torch.bfloat16)
    gu = sb[:NK * 2 * F].view(NK, 2 * F)
    h_off = ((NK * 2 * F * 2 + 255) // 256 * 256) // 2
    h = sb[h_off:h_off + NK * F].view(NK, F)
    dh = trace.view(-1)[:NK * F].view(NK, F)
    dgu = trace.view(-1)[NK * F:].view(NK, 2 * F)

    def rows(t, lo=None, hi=None):
        def f(p):
            idx = torch.from_numpy(np.asarray(p, np.int64)).cuda()
            r = t.index_select(0, idx)
            return f64_of(r[:, lo:hi] if lo is not None else r)
        return f
    return {"g": rows(gu, 0, F), "u": rows(gu, F, 2 * F), "h": rows(h), "dh": rows(dh),
            "dg": rows(dgu, 0, F), "du": rows(dgu, F, 2 * F)}


def _positions(experts, ids, n_ad):
    """Position of every assignment: stable sort by expert * (n_ad + 1) + adapter."""
    K = experts.shape[1]
    keys = experts.reshape(-1).astype(np.int64) * (n_ad + 1) + np.repeat(ids.astype(np.int64), K)
    perm = np.argsort(keys, kind="stable")
    pos = np.empty_like(perm)
    pos[perm] = np.arange(perm.size)
    return pos


def _subset_params(Wg, Wu, Wd, pair_AB, experts, ids, scale):
    """oracle.moe parameters for a subset batch, experts and adapters renumbered
    to the ones the subset uses; pair_AB(p, a, e) -> (A, B) float64."""
    e_list = sorted(set(int(e) for e in experts.reshape(-1)))
    a_list = sorted(set(int(a) for a in ids))
    e_loc = {e: i for i, e in enumerate(e_list)}
    a_loc = {a: i for i, a in enumerate(a_list)}
    used = set((int(ids[t]), int(e)) for t in range(len(ids)) for e in experts[t])
    Wg_l = np.stack([f64_of(Wg[e]) for e in e_list])
    Wu_l = np.stack([f64_of(Wu[e]) for e in e_list])
    Wd_l = np.stack([f64_of(Wd[e]) for e in e_list])
    A, B = {}, {}
    for p in ("gate", "up", "down"):
        A[p], B[p] = [], []
        for a in a_list:
            ra, rb = [], []
            for e in e_list:
                if (a, e) in used:
                    Ap, Bp = pair_AB(p, a, e)
                else:       # not touched by the subset
                    Ap, Bp = pair_AB.zeros(p, a)
                ra.append(Ap)
                rb.append(Bp)
            A[p].append(ra)
            B[p].append(rb)
    ex_l = np.vectorize(e_loc.get)(experts)
    ids_l = np.vectorize(a_loc.get)(ids)
    return (Wg_l, Wu_l, Wd_l, A, B, scale), ex_l, ids_l, e_list, a_list


class _PairAB:
    """(A, B) of entry (e, a) of a projection pack, as float64, on demand."""

    def __init__(self, packs, off, rank, dims):
        self.packs, self.off, self.rank, self.dims = packs, off, rank, dims

    def __call__(self, p, a, e):
        i = ("gate", "up", "down").index(p)
        d_in, d_out = self.dims[p]
        r = self.rank(a)
        o = int(self.off(i, e, a))
        A = f64_of(self.packs[i][o:o + r * d_in]).reshape(r, d_in)
        B = f64_of(self.packs[i][o + r * d_in:o + r * d_in + d_out * r]).reshape(d_out, r)
        return A, B

    def zeros(self, p, a):
        d_in, d_out = self.dims[p]
        r = self.rank(a)
        return np.zeros((r, d_in)), np.zeros((d_out, r))


def _expert_parity(x, dy, experts, weights, ids, y, dx, grads, Wg, Wu, Wd, pair, scale_of,
                   pos, fetch, n_ad, K, tokens, pair_key, grad_view):
    """Sampled tokens (y, dx, every stage of their assignments) and one (expert,
    adapter) pair's dA, dB: against oracle.moe's plain definition on subset
    batches (gpu_util.check_chained: the results carry the layer's bf16 stage
    roundings), and per stage against oracle.lora / oracle.mlp on the GPU's own
    stage bits (bf16 stages at the bf16 tolerance, the pair's gradients at the
    fp32 tolerance)."""
    # sampled tokens, all K assignments each
    ts = np.asarray(tokens)
    posmap = pos[(ts[:, None] * K + np.arange(K)[None, :]).reshape(-1)]
    params, ex_l, ids_l, _, _ = _subset_params(Wg, Wu, Wd, pair, experts[ts], ids[ts],
                                               scale_of(int(ids[ts][0])))
    x_s = f64_of(x[torch.from_numpy(ts).cuda()])
    dy_s = f64_of(dy[torch.from_numpy(ts).cuda()])
    y_ref, saved = OE.moe_forward(x_s, ex_l, weights[ts], ids_l, *params)
    check_chained(f64_of(y)[ts], y_ref, "y")
    dx_ref, _, _ = OE.moe_backward(dy_s, x_s, ex_l, weights[ts], ids_l, *params, saved)
    check_chained(f64_of(dx)[ts], dx_ref, "dx")
    Wg_l, Wu_l, Wd_l, A, B, s = params
    staged_parity(x_s, dy_s, ex_l, weights[ts], ids_l, Wg_l, Wu_l, Wd_l, A, B, lambda a: s,
                  lambda nm, js: fetch[nm](posmap[js]), f64_of(y)[ts], f64_of(dx)[ts])
    # one pair: all of its assignments, as a top-1 batch on that expert
    e0, a0 = pair_key
    J = np.nonzero((experts.reshape(-1) == e0) & (np.repeat(ids, K) == a0))[0]
    tp = J // K
    ex1 = np.full((tp.size, 1), e0)
    w1 = weights.reshape(-1)[J][:, None]
    params, ex_l, ids_l, _, _ = _subset_params(Wg, Wu, Wd, pair, ex1, ids[tp], scale_of(a0))
    x_p = f64_of(x[torch.from_numpy(tp).cuda()])
    dy_p = f64_of(dy[torch.from_numpy(tp).cuda()])
    _, saved = OE.moe_forward(x_p, ex_l, w1, ids_l, *params)
    _, dA, dB = OE.moe_backward(dy_p, x_p, ex_l, w1, ids_l, *params, saved)
    for i, p in enumerate(("gate", "up", "down")):
        gA, gB = grad_view(i, e0, a0)
        check_chained(gA, dA[p][0][0], f"{p} dA")
        check_chained(gB, dB[p][0][0], f"{p} dB")
    Wg_l, Wu_l, Wd_l, A, B, s = params
    checked = staged_parity(x_p, dy_p, ex_l, w1, ids_l, Wg_l, Wu_l, Wd_l, A, B, lambda a: s,
                            lambda nm, js: fetch[nm](pos[J][js]), None, None,
                            grad_of=lambda p, e, a: grad_view(("gate", "up", "down").index(p), e0, a0))
    assert checked == 1
    return J.size


def test_moe_full_size():
    """16384 tokens, 128 experts top-8, H 2048, F 768, 8 rank-32 adapters."""
    inp = WD.moe_inputs()
    n, H, F, E, K, n_ad, r = (inp[k] for k in ("n", "H", "F", "E", "K", "n_ad", "r"))
    x, dy = inp["xs"][0], inp["dys"][0]
    Wg, Wu, Wd, packs = inp["Wg"], inp["Wu"], inp["Wd"], inp["packs"]
    Wgt, Wut = (torch.empty((E, H, F), dtype=torch.bfloat16, device="cuda") for _ in range(2))
    Wdt = torch.empty((E, F, H), dtype=torch.bfloat16, device="cuda")
    for e in range(E):
        L.lora_transpose_bf16(Wg[e], Wgt[e])
        L.lora_transpose_bf16(Wu[e], Wut[e])
        L.lora_transpose_bf16(Wd[e], Wdt[e])
    dims = {"gate": (H, F), "up": (H, F), "down": (F, H)}
    descs = [L.make_desc(ao, ao + r * dims[p][0], np.full(ao.size, r, np.int32),
                         np.full(ao.size, 32.0 / r, np.float32))
             for ao, p in zip(inp["a_offs"], ("gate", "up", "down"))]
    shape = L.MoeShape(n, H, F, packs[0].numel(), packs[1].numel(), packs[2].numel(), E, K, n_ad, r)
    ws = L.empty_workspace(L.moe_workspace_bytes(shape))
    saved = torch.empty(L.moe_saved_bytes(shape), dtype=torch.uint8, device="cuda")
    ex = torch.empty((n, K), dtype=torch.int32, device="cuda")
    w = torch.empty((n, K), device="cuda")
    y = torch.empty((n, H), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty_like(y)
    grads = [torch.full((p.numel(),), float("nan"), dtype=torch.float32, device="cuda") for p in packs]
    trace = torch.empty((3, n * K, F), dtype=torch.bfloat16, device="cuda")
    L.moe_route(inp["logits"], K, ex, w)
    L.moe_forward(shape, x, ex, w, inp["ids"], Wg, Wu, Wd, packs, descs, y, saved, ws)
    L.moe_backward(shape, dy, x, ex, w, inp["ids"], Wgt, Wut, Wdt, packs, descs, saved, dx, grads,
                   0, ws, trace=trace)
    assert L.lora_device_status(ws) == 0
    experts = ex.cpu().numpy().astype(np.int64)
    weights = w.cpu().numpy().astype(np.float64)
    ids = inp["ids"].cpu().numpy()
    rng = np.random.default_rng(8)
    ts = np.sort(rng.choice(n, 6, replace=False))
    # routing of the sampled tokens, exact
    e_ref, w_ref = OE.moe_route(inp["logits"][torch.from_numpy(ts).cuda()].cpu().numpy(), K)
    assert np.array_equal(experts[ts], e_ref) and rel_err(weights[ts], w_ref) < TOL_F32
    pos = _positions(experts, ids, n_ad)
    fetch = _stage_fetch(saved, trace, n * K, F)
    pair = _PairAB(packs, lambda i, e, a: inp["a_offs"][i][e * n_ad + a], lambda a: r, dims)

    def grad_view(i, e, a):
        d_in, d_out = (H, F) if i < 2 else (F, H)
        o = int(inp["a_offs"][i][e * n_ad + a])
        gA = f64_of(grads[i][o:o + r * d_in]).reshape(r, d_in)
        gB = f64_of(grads[i][o + r * d_in:o + r * d_in + d_out * r]).reshape(d_out, r)
        return gA, gB

    e0, a0 = int(experts[ts[0], 0]), int(ids[ts[0]])
    count = _expert_parity(x, dy, experts, weights, ids, y, dx, grads, Wg, Wu, Wd, pair,
                           lambda a: 32.0 / r, pos, fetch, n_ad, K, ts, (e0, a0), grad_view)
    assert count > 16


def test_mlp_layer_full_size():
    """32768 tokens, 4096 -> 12288 -> 4096, 64 adapters ranks {8,16,32,64}, interleaved."""
    inp = WD.mlp_inputs()
    n, d, f, n_ad = (inp[k] for k in ("n", "d", "f", "n_ad"))
    ranks, scales = inp["ranks"], inp["scales"]
    x, dy = inp["xs"][0], inp["dys"][0]
    Ws, packs = inp["W"], inp["packs"]
    Wts, descs = [], []
    for Wt, (ao, bo) in zip(Ws, inp["offs"]):
        Wtt = torch.empty((Wt.shape[1], Wt.shape[0]), dtype=torch.bfloat16, device="cuda")
        L.lora_transpose_bf16(Wt, Wtt)
        Wts.append(Wtt)
        descs.append(L.make_desc(ao, bo, ranks, scales))
    shape = L.MlpShape(n, d, f, packs[0].numel(), packs[1].numel(), packs[2].numel(), n_ad, 64)
    ws = L.empty_workspace(L.mlp_workspace_bytes(shape))
    saved = torch.empty(L.mlp_saved_bytes(shape), dtype=torch.uint8, device="cuda")
    y = torch.empty((n, d), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty_like(y)
    grads = [torch.full((p.numel(),), float("nan"), dtype=torch.float32, device="cuda") for p in packs]
    trace = torch.empty((3, n, f), dtype=torch.bfloat16, device="cuda")
    L.mlp_forward(shape, x, inp["ids"], *Ws, packs, descs, y, saved, ws)
    L.mlp_backward(shape, dy, x, inp["ids"], *Wts, packs, descs, saved, dx, grads, 0, ws,
                   trace=trace)
    assert L.lora_device_status(ws) == 0
    ids = inp["ids"].cpu().numpy()
    experts = np.zeros((n, 1), np.int64)
    weights = np.ones((n, 1))
    pos = _positions(experts, ids, n_ad)
    fetch = _stage_fetch(saved, trace, n, f)
    dims = {"gate": (d, f), "up": (d, f), "down": (f, d)}
    offs = inp["offs"]
    pair = _PairAB(packs, lambda i, e, a: offs[i][0][a], lambda a: int(ranks[a]), dims)

    def grad_view(i, e, a):
        d_in, d_out = dims[("gate", "up", "down")[i]]
        r = int(ranks[a])
        oa, ob = int(offs[i][0][a]), int(offs[i][1][a])
        return (f64_of(grads[i][oa:oa + r * d_in]).reshape(r, d_in),
                f64_of(grads[i][ob:ob + d_out * r]).reshape(d_out, r))

    # the adapter with the fewest tokens, and six sampled tokens of one adapter
    counts = np.bincount(ids, minlength=n_ad)
    a0 = int(np.argmin(counts))
    ts = np.sort(np.random.default_rng(9).choice(np.nonzero(ids == a0)[0], 6, replace=False))
    Wg, Wu, Wd = (t.view(1, *t.shape) for t in Ws)
    count = _expert_parity(x, dy, experts, weights, ids, y, dx, grads, Wg, Wu, Wd, pair,
                           lambda a: float(scales[a]), pos, fetch, n_ad, 1, ts, (0, a0), grad_view)
    assert count == counts[a0]


# ---------------------------------------------------------------- logprob
def test_logprob_full_size():
    """16384 tokens, hidden 4096, vocab 151936, PPO: logprobs and dh on sampled tokens,
    the loss and dlogp over every token (per call, from the GPU's logprobs)."""
    inp = WD.logprob_inputs()
    n, H, V = inp["n"], inp["H"], inp["V"]
    h, U, tg = inp["hs"][0], inp["U"], inp["targets"]
    Ut = torch.empty((H, V), dtype=torch.bfloat16, device="cuda")
    L.lora_transpose_bf16(U, Ut)
    lp = torch.empty(n, device="cuda")
    lse = torch.empty(n, device="cuda")
    L.token_logprobs(h, U, tg, lp, lse, L.empty_workspace(L.token_logprobs_workspace_bytes(n, V)))
    samp = (lp + torch.randn(n, generator=inp["gen"], device="cuda") * 0.05 * inp["act"]).contiguous()
    loss = torch.empty(1, device="cuda")
    dl = torch.empty(n, device="cuda")
    L.loss_grad(L.LOSS_PPO, lp, inp["act"], inp["adv"], samp, None, (0.2, 0.2), loss, dl,
                L.empty_workspace(L.loss_grad_workspace_bytes(n)))
    dh = torch.empty((n, H), dtype=torch.bfloat16, device="cuda")
    L.token_logprobs_backward(h, U, Ut, tg, lse, dl, dh,
                              L.empty_workspace(L.token_logprobs_backward_workspace_bytes(n, V, 4096)))
    rows = np.sort(np.random.default_rng(10).choice(n, 8, replace=False))
    h64, U64, t_np = f64_of(h), f64_of(U), tg.cpu().numpy()
    lp_ref, lse_ref = OP.token_logprobs(h64, U64, t_np, rows=rows)
    assert rel_err(lp.cpu().numpy()[rows].astype(np.float64), lp_ref) < TOL_F32
    assert rel_err(lse.cpu().numpy()[rows].astype(np.float64), lse_ref) < TOL_F32
    lp_g, act, adv = lp.cpu().numpy(), inp["act"].cpu().numpy(), inp["adv"].cpu().numpy()
    L_ref, dl_ref = OLs.loss_grad(OLs.PPO, lp_g, act, adv=adv, samp=samp.cpu().numpy(),
                                  clip_low=0.2, clip_high=0.2)
    dlg = dl.cpu().numpy().astype(np.float64)
    rho = np.exp(lp_g.astype(np.float64) - samp.cpu().numpy())
    # where fp32 and fp64 can take the clip decision differently (ratio within
    # 1e-5 of a bound), either valid gradient (clipped: 0; unclipped: -rho A on a
    # kept row) is accepted; every other row is compared
    near = (np.abs(rho - 0.8) < 1e-5) | (np.abs(rho - 1.2) < 1e-5)
    alt = np.where(act != 0, -rho * adv, 0.0)
    ok = (np.abs(dlg - dl_ref) < 1e-5) | (np.abs(dlg - alt) < 1e-5) | (np.abs(dlg) < 1e-30)
    assert ok[near].all()
    assert rel_err(dlg[~near], dl_ref[~near]) < TOL_F32
    assert abs(float(loss.item()) - L_ref) <= TOL_F32 * max(abs(L_ref), 1e-3)
    dh_ref = OP.token_logprobs_backward(h64, U64, t_np, dlg, rows=rows)
    assert rel_err(f64_of(dh)[rows], dh_ref) < TOL_BF16
