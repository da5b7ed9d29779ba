"""GPU parity of the fused lm_head logprob (forward, backward), the token
losses, AdamW and the SwiGLU glue against the oracle, through the C ABI."""
import numpy as np
import pytest

import oracle.adam as OA
import oracle.logprob as OP
import oracle.loss as OLs
import oracle.mlp as OM
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_util import TOL_BF16, TOL_F32, bits_of, dev_bf16, dev_f32, dev_i32, f64_of, rel_err  # noqa: E402
import rl_lora_linear_amd.lib as L  # noqa: E402


def _lp_case(seed=40, n_groups=3, group_size=4, seq_len=50, hidden=320, vocab=1088):
    # 600 tokens (ragged against 256-row tiles), vocab 1088 = 4 full tiles + 64 columns
    return W.logprob_rl(seed=seed, hidden=hidden, vocab=vocab, n_groups=n_groups,
                        group_size=group_size, seq_len=seq_len, sampler_sigma=0.5)


def _run_logprobs(h, U, tgt):
    n, vocab = h.shape[0], U.shape[0]
    lp = torch.empty(n, dtype=torch.float32, device="cuda")
    lse = torch.empty(n, dtype=torch.float32, device="cuda")
    ws = L.empty_workspace(L.token_logprobs_workspace_bytes(n, vocab))
    L.token_logprobs(h, U, tgt, lp, lse, ws)
    return lp, lse, L.lora_device_status(ws)


def test_token_logprobs_parity():
    c = _lp_case()
    h, U, tgt = dev_bf16(c.h_bits), dev_bf16(c.U_bits), dev_i32(c.targets)
    lp, lse, flags = _run_logprobs(h, U, tgt)
    assert flags == 0
    lp_ref, lse_ref = OP.token_logprobs(W.bf16_bits_to_f64(c.h_bits), W.bf16_bits_to_f64(c.U_bits), c.targets)
    assert rel_err(f64_of(lse), lse_ref) < TOL_F32
    assert rel_err(f64_of(lp), lp_ref) < TOL_F32


def test_token_logprobs_uniform_and_invalid_targets():
    g = 1088
    h = dev_bf16(W.to_bf16_bits(np.random.default_rng(0).standard_normal((300, 128))))
    U = torch.zeros((g, 128), dtype=torch.bfloat16, device="cuda")
    tgt = np.arange(300, dtype=np.int32) * 3
    tgt[[5, 77]] = [-1, g]
    lp, lse, flags = _run_logprobs(h, U, dev_i32(tgt))
    assert flags & L.FLAG_TARGET_RANGE
    lpn = lp.cpu().numpy()
    assert np.isnan(lpn[5]) and np.isnan(lpn[77])
    ok = np.ones(300, bool); ok[[5, 77]] = False
    np.testing.assert_allclose(lpn[ok], -np.log(g), rtol=0, atol=2e-6)


@pytest.mark.parametrize("chunk_rows", [256, 1024])
def test_token_logprobs_backward_parity(chunk_rows):
    c = _lp_case(41)
    n, H, V = c.n_tokens, c.hidden, c.vocab
    h, U, tgt = dev_bf16(c.h_bits), dev_bf16(c.U_bits), dev_i32(c.targets)
    Ut = torch.empty((H, V), dtype=torch.bfloat16, device="cuda")
    L.lora_transpose_bf16(U, Ut)
    lp, lse, _ = _run_logprobs(h, U, tgt)
    d = np.random.default_rng(3).standard_normal(n).astype(np.float32)
    d[::7] = 0.0
    dh = torch.empty((n, H), dtype=torch.bfloat16, device="cuda")
    ws = L.empty_workspace(L.token_logprobs_backward_workspace_bytes(n, V, chunk_rows))
    L.token_logprobs_backward(h, U, Ut, tgt, lse, dev_f32(d), dh, ws)
    dh_ref = OP.token_logprobs_backward(W.bf16_bits_to_f64(c.h_bits), W.bf16_bits_to_f64(c.U_bits), c.targets, d)
    dhg = f64_of(dh)
    assert rel_err(dhg, dh_ref) < TOL_BF16
    assert not np.any(dhg[::7])                       # dlogp == 0 rows are exact zeros


@pytest.mark.parametrize("kind", [0, 1, 2, 3])
def test_loss_grad_parity(kind):
    c = _lp_case(42)
    n = c.n_tokens
    rng = np.random.default_rng(kind)
    lp = (-rng.random(n) * 8).astype(np.float32)
    samp = c.sampler_logprobs(lp)
    w = c.action.copy()
    if kind == OLs.CROSS_ENTROPY:
        w = (w * rng.random(n)).astype(np.float32)     # fractional weights
    adv, g = c.advantages, c.custom_g
    # masked rows hold non-finite garbage: selection must keep them out
    lp_in, samp_in, adv_in, g_in = lp.copy(), samp.copy(), adv.copy(), g.copy()
    masked = np.nonzero(w == 0)[0][:5]
    lp_in[masked[0]], samp_in[masked[1]], adv_in[masked[2]], g_in[masked[3]] = np.nan, np.inf, np.nan, -np.inf
    loss = torch.empty(1, dtype=torch.float32, device="cuda")
    dl = torch.empty(n, dtype=torch.float32, device="cuda")
    ws = L.empty_workspace(L.loss_grad_workspace_bytes(n))
    L.loss_grad(kind, dev_f32(lp_in), dev_f32(w), dev_f32(adv_in), dev_f32(samp_in), dev_f32(g_in),
                (0.2, 0.2), loss, dl, ws)
    L_ref, dl_ref = OLs.loss_grad(kind, lp_in, w, adv=adv_in, samp=samp_in, g=g_in, clip_low=0.2, clip_high=0.2)
    dlg = dl.cpu().numpy().astype(np.float64)
    assert np.all(dlg[w == 0] == 0.0) and np.isfinite(dlg).all()
    if kind == OLs.PPO:
        # where fp32 and fp64 can take the clip decision differently (ratio within
        # 1e-5 of a bound), accept either valid gradient; compare the rest
        rho = np.exp(lp.astype(np.float64) - samp)
        near = (np.abs(rho - 0.8) < 1e-5) | (np.abs(rho - 1.2) < 1e-5)
        alt = -rho * adv
        ok = np.where(near, (np.abs(dlg - dl_ref) < 1e-5) | (np.abs(dlg - alt) < 1e-5) | (np.abs(dlg) < 1e-30), True)
        assert ok.all()
        assert rel_err(dlg[~near], dl_ref[~near]) < TOL_F32
        clipped = (dl_ref == 0) & (w != 0) & (adv != 0)
        assert clipped.sum() > 0                        # sigma 0.5 exercises the clip
    else:
        assert rel_err(dlg, dl_ref) < TOL_F32
    assert abs(float(loss.item()) - L_ref) <= TOL_F32 * max(abs(L_ref), 1e-3)


def test_custom_minus_w_is_ce_bitwise():
    c = _lp_case(43)
    n = c.n_tokens
    lp = (-np.random.default_rng(1).random(n) * 8).astype(np.float32)
    w = (c.action * np.random.default_rng(2).random(n)).astype(np.float32)
    ws = L.empty_workspace(L.loss_grad_workspace_bytes(n))
    outs = []
    for kind, weights, g in ((OLs.CROSS_ENTROPY, w, None), (OLs.CUSTOM, (w != 0).astype(np.float32), -w)):
        loss = torch.empty(1, dtype=torch.float32, device="cuda")
        dl = torch.empty(n, dtype=torch.float32, device="cuda")
        L.loss_grad(kind, dev_f32(lp), dev_f32(weights), None, None, None if g is None else dev_f32(g),
                    None, loss, dl, ws)
        outs.append((loss.cpu().numpy(), dl.cpu().numpy()))
    assert np.array_equal(outs[0][0].view(np.uint32), outs[1][0].view(np.uint32))
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))


@pytest.mark.parametrize("n", [1, 7, 4096 + 3, 262144])
def test_adam_parity_and_resume(n):
    rng = np.random.default_rng(n)
    p0 = rng.uniform(-1 / 64, 1 / 64, n).astype(np.float32)      # LoRA-A-like initial values
    grads = [(rng.standard_normal(n) * 10 ** rng.uniform(-4, -1)).astype(np.float32) for _ in range(4)]
    p, m, v = dev_f32(p0), torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
    pb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    po, mo, vo = p0.astype(np.float64), np.zeros(n), np.zeros(n)
    snap = None
    for t, g in enumerate(grads, start=1):
        pre = p.cpu().numpy().astype(np.float64)
        L.adam_step(p, dev_f32(g), m, v, t, 1e-4, 0.9, 0.999, 1e-8, 0.01, pb)
        # per-call parity: the oracle steps from the GPU's own state
        po, mo2, vo2 = OA.adam_step(pre, g, mo, vo, t, 1e-4, 0.9, 0.999, 1e-8, 0.01)
        # Delta p at 1e-4 of its scale, plus the fp32 spacing of p itself: the
        # stored parameter cannot resolve a step finer than one ulp of p
        dp, dp_ref = p.cpu().numpy() - pre, po - pre
        scale = np.maximum(np.abs(dp_ref), np.sqrt(np.mean(dp_ref ** 2)))
        ulp = np.spacing(np.abs(po).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(dp - dp_ref) <= TOL_F32 * scale + ulp)
        assert rel_err(m.cpu().numpy(), mo2) < TOL_F32 and rel_err(v.cpu().numpy(), vo2) < TOL_F32
        mo, vo = m.cpu().numpy().astype(np.float64), v.cpu().numpy().astype(np.float64)
        assert np.array_equal(bits_of(pb), W.to_bf16_bits(p.cpu().numpy()))
        if t == 2:
            snap = (p.clone(), m.clone(), v.clone())
    # resume from the step-2 snapshot: bitwise identical to the straight run
    p2, m2, v2 = snap
    for t, g in enumerate(grads[2:], start=3):
        L.adam_step(p2, dev_f32(g), m2, v2, t, 1e-4, 0.9, 0.999, 1e-8, 0.01, None)
    assert torch.equal(p2, p) and torch.equal(m2, m) and torch.equal(v2, v)


def test_adam_multi_matches_per_segment():
    """One batched launch over many adapters == one adam_step per adapter,
    bitwise; elements outside every segment stay untouched.  70 segments
    (more than one launch's worth), unaligned offsets, an empty segment and
    per-segment step counters."""
    rng = np.random.default_rng(70)
    counts = [int(c) for c in rng.integers(0, 9000, 70)]
    counts[5] = 0
    counts[6] = 3
    segs, off = [], 5                              # offset 5: float4 path off for some segments
    for i, c in enumerate(counts):
        segs.append((off, c, 1 + (i * 7) % 13))
        off += c + int(rng.integers(0, 3))         # gaps between segments
    n = off + 11
    p0 = rng.uniform(-0.02, 0.02, n).astype(np.float32)
    g0 = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    m0 = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v0 = (rng.uniform(0, 1e-5, n)).astype(np.float32)
    args = (1e-4, 0.9, 0.999, 1e-8, 0.01)
    p, m, v, g = dev_f32(p0), dev_f32(m0), dev_f32(v0), dev_f32(g0)
    pb = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    L.adam_step_multi(segs, p, g, m, v, *args, p_bf16=pb)
    p2, m2, v2 = dev_f32(p0), dev_f32(m0), dev_f32(v0)
    pb2 = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    for o, c, t in segs:
        L.adam_step(p2[o:o + c], g[o:o + c], m2[o:o + c], v2[o:o + c], t, *args, pb2[o:o + c])
    torch.cuda.synchronize()
    assert torch.equal(p, p2) and torch.equal(m, m2) and torch.equal(v, v2)
    assert np.array_equal(bits_of(pb), bits_of(pb2))
    inside = np.zeros(n, bool)
    for o, c, _ in segs:
        inside[o:o + c] = True
    assert np.array_equal(p.cpu().numpy()[~inside], p0[~inside])
    assert np.all(bits_of(pb)[~inside] == 0)
    # one segment against the oracle directly
    o, c, t = segs[9]
    po, mo, vo = OA.adam_step(p0[o:o + c].astype(np.float64), g0[o:o + c], m0[o:o + c], v0[o:o + c],
                              t, *args)
    assert rel_err(m.cpu().numpy()[o:o + c], mo) < TOL_F32
    assert rel_err(v.cpu().numpy()[o:o + c], vo) < TOL_F32
    dp, dp_ref = p.cpu().numpy()[o:o + c] - p0[o:o + c], po - p0[o:o + c]
    scale = np.maximum(np.abs(dp_ref), np.sqrt(np.mean(dp_ref ** 2)))
    ulp = np.spacing(np.abs(po).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(dp - dp_ref) <= TOL_F32 * scale + ulp)


def test_swiglu_parity():
    rng = np.random.default_rng(7)
    n = 3 * 1000 + 5
    gb = W.to_bf16_bits(rng.standard_normal(n) * 3)
    ub = W.to_bf16_bits(rng.standard_normal(n))
    db = W.to_bf16_bits(rng.standard_normal(n))
    g, u, d = dev_bf16(gb), dev_bf16(ub), dev_bf16(db)
    h = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    L.swiglu_forward(g, u, h)
    gf, uf, df = (W.bf16_bits_to_f64(x) for x in (gb, ub, db))
    assert rel_err(f64_of(h), OM.swiglu_forward(gf, uf)) < TOL_BF16
    dg = torch.empty_like(h); du = torch.empty_like(h)
    L.swiglu_backward(d, g, u, dg, du)
    rg, ru = OM.swiglu_backward(df, gf, uf)
    assert rel_err(f64_of(dg), rg) < TOL_BF16 and rel_err(f64_of(du), ru) < TOL_BF16


def _adam_close(pn, mn, vn, p0, po, mo, vo):
    """Delta p at 1e-4 of its scale plus what the fp32 parameter cannot resolve:
    p is rounded twice (after the decay, after the step), half an ulp each, of
    the larger of the old and new magnitudes."""
    p0 = np.asarray(p0, np.float64)
    dp, dp_ref = np.asarray(pn, np.float64) - p0, po - p0
    scale = np.maximum(np.abs(dp_ref), np.sqrt(np.mean(dp_ref ** 2)))
    ulp = np.spacing(np.maximum(np.abs(p0), np.abs(po)).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(dp - dp_ref) <= TOL_F32 * scale + ulp)
    assert rel_err(mn, mo) < TOL_F32 and rel_err(vn, vo) < TOL_F32


@pytest.mark.parametrize("layout", ["five", "seventy", "single_big"])
def test_adam_skips_whole_adapter_on_nonfinite_gradient(layout):
    """TPU RL note, section 12: a non-finite optimizer update is skipped
    outright.  An adapter whose gradient holds one NaN or Inf keeps ALL of its
    p, m, v and bf16 copy bit for bit; every other adapter steps as the oracle
    does; the status word gets FLAG_NONFINITE_GRAD and the workspace's skip
    flags name exactly the skipped adapters.  five: one launch, adapter 3 bad;
    seventy: two launches' worth of segments with unaligned offsets, bad ones in
    both launches; single_big: adam_step on one 262149-element adapter whose
    only bad element sits in its last block.  A second call on the same
    workspace with clean gradients steps everything and clears the flags."""
    rng = np.random.default_rng(9)
    if layout == "five":
        counts, gaps, bad_segs = [1003, 4096, 17, 5000, 64], [0] * 5, [3]
    elif layout == "seventy":
        counts = [int(c) for c in rng.integers(1, 3000, 70)]
        gaps, bad_segs = [int(x) for x in rng.integers(0, 3, 70)], [2, 40, 66]
    else:
        counts, gaps, bad_segs = [262149], [0], [0]
    segs, off = [], 3 if layout == "seventy" else 0
    for i, (c, gp) in enumerate(zip(counts, gaps)):
        segs.append((off, c, 1 + (i * 5) % 11))
        off += c + gp
    n = off + 7
    p0 = rng.standard_normal(n).astype(np.float32)
    m0 = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v0 = (rng.random(n) * 1e-6).astype(np.float32)
    pb0 = W.to_bf16_bits(p0)
    g = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    for j, i in enumerate(bad_segs):
        o, c, _ = segs[i]
        g[o + c - 1 - (j % c)] = [np.nan, np.inf, -np.inf][j % 3]
    ws = L.empty_workspace(L.adam_workspace_bytes(len(segs)))
    for gg, bad in ((g, set(bad_segs)), (np.nan_to_num(g, nan=0.3, posinf=0.1, neginf=-0.1), set())):
        p, m, v = dev_f32(p0), dev_f32(m0), dev_f32(v0)
        pb = dev_bf16(pb0)
        if layout == "single_big":
            o, c, t = segs[0]
            L.adam_step(p[o:o + c], dev_f32(gg[o:o + c]), m[o:o + c], v[o:o + c], t, 1e-4,
                        weight_decay=0.01, p_bf16=pb[o:o + c], ws=ws)
        else:
            L.adam_step_multi(segs, p, dev_f32(gg), m, v, 1e-4, weight_decay=0.01, p_bf16=pb, ws=ws)
        flags = L.adam_skip_flags(ws, len(segs))
        assert L.lora_device_status(ws) == (L.FLAG_NONFINITE_GRAD if bad else 0)
        assert set(np.nonzero(flags)[0].tolist()) == bad and set(flags.tolist()) <= {0, 1}
        pn, mn, vn, pbn = p.cpu().numpy(), m.cpu().numpy(), v.cpu().numpy(), bits_of(pb)
        for i, (o, c, t) in enumerate(segs):
            sl = slice(o, o + c)
            po, mo, vo, skipped = OA.adam_step_flagged(p0[sl], gg[sl], m0[sl], v0[sl], t, 1e-4,
                                                       weight_decay=0.01)
            assert skipped == (i in bad)
            if i in bad:
                for a, a0 in ((pn, p0), (mn, m0), (vn, v0)):
                    assert np.array_equal(a[sl].view(np.int32), a0[sl].view(np.int32)), i
                assert np.array_equal(pbn[sl], pb0[sl])
            else:
                _adam_close(pn[sl], mn[sl], vn[sl], p0[sl], po, mo, vo)
                assert np.array_equal(pbn[sl], W.to_bf16_bits(pn[sl]))
        inside = np.zeros(n, bool)
        for o, c, _ in segs:
            inside[o:o + c] = True
        assert np.array_equal(pn[~inside].view(np.int32), p0[~inside].view(np.int32))


@pytest.mark.parametrize("kind", [0, 1, 2, 3])
def test_loss_grad_sentinel(kind):
    """TPU RL note, section 12: kept rows whose inputs hold NaN or +-Inf (in
    every input the kind reads) are removed by selection -- dlogp 0, no loss
    term -- and FLAG_NONFINITE_LOSS is raised; the rest matches the oracle.  A
    clean batch leaves the flag clear."""
    c = _lp_case(44)
    n = c.n_tokens
    rng = np.random.default_rng(10 + kind)
    lp = (-rng.random(n) * 8).astype(np.float32)
    samp = c.sampler_logprobs(lp).astype(np.float32)
    w = c.action.astype(np.float32).copy()
    adv, g = c.advantages.astype(np.float32).copy(), c.custom_g.astype(np.float32).copy()
    kept = np.nonzero(w != 0)[0]
    rows = kept[[3, 50, 100, 200, 300]]
    arrs = {"l": lp.copy(), "w": w.copy(), "A": adv.copy(), "s": samp.copy(), "g": g.copy()}
    names = {0: ["l", "w", "l"], 1: ["l", "A", "s", "w"], 2: ["s", "A", "l", "w", "s"],
             3: ["g", "l", "w"]}[kind]
    vals = [np.nan, np.inf, -np.inf]
    for j, (r, nm) in enumerate(zip(rows, names)):
        arrs[nm][r] = vals[j % 3]
    ws = L.empty_workspace(L.loss_grad_workspace_bytes(n))
    for clean in (False, True):
        src = {"l": lp, "w": w, "A": adv, "s": samp, "g": g} if clean else arrs
        loss = torch.empty(1, dtype=torch.float32, device="cuda")
        dl = torch.empty(n, dtype=torch.float32, device="cuda")
        L.loss_grad(kind, dev_f32(src["l"]), dev_f32(src["w"]), dev_f32(src["A"]), dev_f32(src["s"]),
                    dev_f32(src["g"]), (0.2, 0.2), loss, dl, ws)
        L_ref, dl_ref, flag = OLs.loss_grad_flagged(kind, src["l"], src["w"], adv=src["A"],
                                                    samp=src["s"], g=src["g"])
        assert flag == (not clean)
        assert L.lora_device_status(ws) == (0 if clean else L.FLAG_NONFINITE_LOSS)
        dlg = dl.cpu().numpy().astype(np.float64)
        assert np.isfinite(dlg).all() and np.isfinite(loss.item())
        if not clean:
            assert np.all(dlg[rows[:len(names)]] == 0.0)
        rho = np.exp(src["l"].astype(np.float64) - src["s"])
        near = (np.abs(rho - 0.8) < 1e-5) | (np.abs(rho - 1.2) < 1e-5) if kind == OLs.PPO else \
            np.zeros(n, bool)
        assert rel_err(dlg[~near], dl_ref[~near]) < TOL_F32
        assert abs(float(loss.item()) - L_ref) <= TOL_F32 * max(abs(L_ref), 1e-3)
