"""Timed runs of the workloads beside the q/o projection step, each next to the
oracle timed on the host cores, plus whole-model AdamW and the chip's measured
peaks.  Used by bench.py; every timed step runs through the library's C entry
points on seeded synthetic inputs drawn on the device (workloads.device).

  mlp      Qwen3-8B-width SwiGLU MLP, 64 adapters r{8,16,32,64}, 32768 tokens
           with interleaved ids: mlp_forward + mlp_backward
  logprob  fused lm_head logprob (H 4096, V 151936) + PPO loss + logprob
           backward over 16 groups x 4 x 256 tokens; the custom-loss path timed
           two ways (one forward reusing lse; the two-forward protocol)
  moe      Qwen3-30B-A3B-style routed layer (128 experts, top-8, H 2048, F 768,
           8 rank-32 adapters on every expert): route + forward + backward
  decode   rollout-shaped forward: 256 tokens over 64 adapters, 4096 -> 4096
  adam     AdamW over one whole rank-32 Qwen3-8B adapter (87,293,952 params)
  peaks    register-only MFMA loop, streaming copy and read: the chip's own peaks

CPU baselines run the oracle (NumPy float64) on a bounded sample of the same
workload -- rows are independent through every projection, the lm_head and
the loss, so tokens/s scales with the sample -- and say what the sample was.
"""
from __future__ import annotations

import os
import time

import numpy as np
import torch

import rl_lora_linear_amd.lib as L
import workloads as W
import workloads.device as WD

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)


# ------------------------------------------------------------------ host / timing helpers
def host_info():
    """BLAS threads the oracle uses, CPUs this process may run on, CPU model."""
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cores": int(threads), "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": model}


def cpu_entry(tokens, seconds, sample, unit="tokens/s"):
    d = {"value": round(tokens / seconds, 2), "unit": unit, "kind": "oracle", "sample": sample,
         "seconds": round(seconds, 2)}
    d.update(host_info())
    return d


def f64(t: torch.Tensor) -> np.ndarray:
    """Host float64 copy of a device tensor (bf16 bits decoded exactly)."""
    if t.dtype == torch.bfloat16:
        return W.bf16_bits_to_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return t.detach().cpu().numpy().astype(np.float64)


def timed(step, steps, warmup, log, name):
    """ms per step with no instrumentation, then a second pass of `steps` with
    the library's HIP-event timers on (kernel durations)."""
    for k in range(warmup):
        step(k)
    torch.cuda.synchronize()

    def run(instrumented):
        L.lora_timing_reset()
        L.lora_timing_enable(instrumented)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            step(k)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        L.lora_timing_enable(False)
        return (t1 - t0) * 1e3 / steps

    log(f"[bench] {name}: timing {steps} steps, then {steps} instrumented steps")
    ms = run(False)
    return ms, run(True)


def timer(tid):
    """(average ms per record, records) of a library timer since the last reset."""
    tot, cnt = L.lora_timing_read(tid)
    return tot / max(cnt, 1), cnt


def roofline(bound, kernel, work, ms, peaks, unit_work):
    """work per launch (flop or byte) over the launch's average ms, against the
    published peak and, when measured, the chip's own."""
    if bound == "mfma":
        achieved = work / (ms / 1e3) / 1e12
        peak, unit = PEAK_BF16_TFLOPS, "TFLOP/s"
        mp = (peaks or {}).get("mfma_bf16_tflops")
    else:
        achieved = work / (ms / 1e3) / 1e9
        peak, unit = PEAK_HBM_GBS, "GB/s"
        mp = (peaks or {}).get("hbm_stream_gbs")
    r = {"bound": bound, "kernel": kernel, "achieved": round(achieved, 1), "peak": peak,
         "unit": unit, "frac": round(achieved / peak, 4), "traffic": None,
         "work_per_launch": work, "work_unit": unit_work, "avg_ms": round(ms, 5)}
    if mp:
        r["measured_peak"] = round(mp, 1)
        r["frac_measured_peak"] = round(achieved / mp, 4)
    return r


def _free(*ts):
    for t in ts:
        del t
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ peaks
def peaks(log):
    """The chip's own peaks, each timed with events after a warm-up launch (the
    clock settles under the load): a register-only MFMA loop with enough
    blocks to keep every SIMD's matrix pipe fed, and 1 GiB streaming copy and
    read kernels."""
    log("[bench] peaks: MFMA loop, streaming copy and read")
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    blocks = 256 * 8
    sink = torch.empty(blocks, device="cuda")
    L.lora_probe_mfma(20000, blocks, sink)          # ~20 ms: the clock ramps up under load
    iters = 10000
    t_mfma = None
    for _ in range(3):                              # the best of three ~10 ms runs
        s.record()
        flops = L.lora_probe_mfma(iters, blocks, sink)
        e.record()
        torch.cuda.synchronize()
        t = s.elapsed_time(e) / 1e3
        t_mfma = t if t_mfma is None else min(t_mfma, t)
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    isink = torch.zeros(1, dtype=torch.int32, device="cuda")
    reps = 5

    def rate(fn):
        fn()
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / 1e3 / reps

    t_copy = rate(lambda: L.lora_probe_copy(src, dst))
    t_read = rate(lambda: L.lora_probe_read(src, isink))
    _free(src, dst, sink, isink)
    copy_gbs, read_gbs = 2 * n / t_copy / 1e9, n / t_read / 1e9
    return {"mfma_bf16_tflops": round(flops / t_mfma / 1e12, 1),
            "hbm_copy_gbs": round(copy_gbs, 1), "hbm_read_gbs": round(read_gbs, 1),
            "hbm_stream_gbs": round(max(copy_gbs, read_gbs), 1),
            "how": f"MFMA: {blocks} blocks x 8 waves x 4 independent v_mfma_f32_32x32x16_bf16 chains "
                   f"on register operands, best of 3 runs of {iters} rounds ({t_mfma * 1e3:.1f} ms) after a "
                   "20000-round warm-up; copy: 1 GiB -> "
                   "1 GiB, read + write bytes over its time; read: 1 GiB read-only stream; "
                   "hbm_stream_gbs = the better of the two (the measured HBM peak)"}


# ------------------------------------------------------------------ MLP
def _mlp_cpu(inp, target_s):
    """oracle.mlp forward + backward on the first S tokens (whole workload's
    weights and adapters; per-adapter sums over the sample's tokens)."""
    import oracle.mlp as OM
    ranks, scales = inp["ranks"], inp["scales"].astype(np.float64)
    projs = []
    for Wt, pack, (ao, bo) in zip(inp["W"], inp["packs"], inp["offs"]):
        Wd = f64(Wt)
        d_out, d_in = Wd.shape
        p = f64(pack)
        A = [p[ao[i]:ao[i] + r * d_in].reshape(r, d_in) for i, r in enumerate(ranks)]
        B = [p[bo[i]:bo[i] + d_out * r].reshape(d_out, r) for i, r in enumerate(ranks)]
        projs.append((Wd, A, B, scales))
    x, dy, ids = inp["xs"][0], inp["dys"][0], inp["ids"].cpu().numpy()
    S, spent, tokens = 256, 0.0, 0
    while True:
        xs, dys = f64(x[tokens:tokens + S]), f64(dy[tokens:tokens + S])
        t0 = time.perf_counter()
        y, saved = OM.mlp_forward(xs, *projs, ids[tokens:tokens + S])
        OM.mlp_backward(dys, xs, *projs, ids[tokens:tokens + S], saved)
        spent += time.perf_counter() - t0
        tokens += S
        if spent > target_s or tokens + S > x.shape[0]:
            break
    return cpu_entry(tokens, spent, f"oracle.mlp fwd+bwd on the first {tokens} of the {x.shape[0]} "
                                    f"tokens, in batches of {S}, full weights and 64 adapters")


def mlp(steps, warmup, log, peaks_=None, cpu_s=8.0, n=32768, d=4096, f=12288, n_ad=64):
    inp = WD.mlp_inputs(n, d, f, n_ad)
    ranks, ids, xs, dys = inp["ranks"], inp["ids"], inp["xs"], inp["dys"]
    R = 64
    Ws, packs = inp["W"], inp["packs"]
    Wts, descs = [], []
    for Wt, (ao, bo) in zip(Ws, inp["offs"]):
        Wtt = torch.empty((Wt.shape[1], Wt.shape[0]), dtype=torch.bfloat16, device="cuda")
        L.lora_transpose_bf16(Wt, Wtt)
        Wts.append(Wtt)
        descs.append(L.make_desc(ao, bo, ranks, inp["scales"]))
    shape = L.MlpShape(n, d, f, packs[0].numel(), packs[1].numel(), packs[2].numel(), n_ad, R)
    ws = L.empty_workspace(L.mlp_workspace_bytes(shape))
    saved = torch.empty(L.mlp_saved_bytes(shape), dtype=torch.uint8, device="cuda")
    grads = [torch.zeros(p.numel(), dtype=torch.float32, device="cuda") for p in packs]
    y = torch.empty((n, d), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty_like(y)

    def step(k):
        x, dyy = xs[k % 2], dys[k % 2]
        L.mlp_forward(shape, x, ids, *Ws, packs, descs, y, saved, ws)
        L.mlp_backward(shape, dyy, x, ids, *Wts, packs, descs, saved, dx, grads, 0, ws)

    ms, ms_instr = timed(step, steps, warmup, log, f"mlp {n} tokens")
    if L.lora_device_status(ws):
        raise RuntimeError("mlp: device status flags set")
    gemm_ms, gemm_n = timer(L.TIMER_BASE_GEMM)
    shr_ms, shr_n = timer(L.TIMER_SHRINK)
    grd_ms, grd_n = timer(L.TIMER_GRAD)
    flops_step = 6 * 2.0 * n * d * f
    per_step = gemm_n / steps
    out = {
        "tokens_per_s": round(n / (ms / 1e3), 1), "ms_per_step": round(ms, 4),
        "ms_per_step_instrumented": round(ms_instr, 4),
        "config": {"workload": f"qwen3-8b MLP gate/up {d}->{f}, down {f}->{d}, {n_ad} adapters "
                               f"ranks {{8,16,32,64}} alpha 32, {n} tokens interleaved ids, fwd+bwd",
                   "rank_counts": {int(r): int((ranks == r).sum()) for r in (8, 16, 32, 64)}},
        # 6 projections of 2 N d f per step in 4 grouped launches: work per launch
        # is the step's flops over its launches
        "roofline": roofline("mfma", "base GEMMs (gate+up with SwiGLU, down; dh with the SwiGLU "
                             "backward; gate/up dX K-concatenated): 6 x 2*N*d*d_ff per step in 4 "
                             "launches", flops_step / per_step, gemm_ms, peaks_, "flop"),
        "kernels": {"shrink_ms_per_step": round(shr_ms * shr_n / steps, 4),
                    "grad_ms_per_step": round(grd_ms * grd_n / steps, 4),
                    "gemm_ms_per_step": round(gemm_ms * gemm_n / steps, 4)},
    }
    if cpu_s > 0:
        log("[bench] mlp: cpu baseline (oracle)")
        out["cpu_baseline"] = _mlp_cpu(inp, cpu_s)
    _free(ws, saved, y, dx, *grads, *Wts)
    return out


# ------------------------------------------------------------------ logprob + loss
def _logprob_cpu(h, U, tg, lp_dev, act, adv, samp, target_s):
    """oracle.logprob forward + backward and oracle.loss (PPO) on sampled rows."""
    import oracle.logprob as OP
    import oracle.loss as OLs
    t0 = time.perf_counter()
    U64 = f64(U)
    conv = time.perf_counter() - t0
    n = h.shape[0]
    rng = np.random.default_rng(0)
    tgt = tg.cpu().numpy()
    actn, advn, sampn = act.cpu().numpy(), adv.cpu().numpy(), samp.cpu().numpy()
    S, spent, tokens = 64, 0.0, 0
    while True:
        rows = np.sort(rng.choice(n, S, replace=False))
        hs = f64(h[torch.from_numpy(rows).cuda()])
        t1 = time.perf_counter()
        lp, lse = OP.token_logprobs(hs, U64, tgt[rows])
        _, dl = OLs.loss_grad(OLs.PPO, lp, actn[rows], adv=advn[rows], samp=sampn[rows])
        OP.token_logprobs_backward(hs, U64, tgt[rows], dl)
        spent += time.perf_counter() - t1
        tokens += S
        if spent > target_s or tokens >= n:
            break
    del U64
    return cpu_entry(tokens, spent, f"oracle logprob fwd + PPO loss + logprob bwd on {tokens} "
                                    f"sampled rows (batches of {S}) against the full V={U.shape[0]} "
                                    f"lm_head (its float64 conversion, {conv:.1f} s, not timed)")


def logprob(steps, warmup, log, peaks_=None, cpu_s=8.0, n_seq=64, seq=256, H=4096, V=151936,
            chunk=4096):
    inp = WD.logprob_inputs(n_seq, seq, H, V)
    n, hs, U, tg, act, adv, gen = (inp[k] for k in ("n", "hs", "U", "targets", "act", "adv", "gen"))
    Ut = torch.empty((H, V), dtype=torch.bfloat16, device="cuda")
    L.lora_transpose_bf16(U, Ut)
    lp = torch.empty(n, device="cuda")
    lse = torch.empty(n, device="cuda")
    ws_f = L.empty_workspace(L.token_logprobs_workspace_bytes(n, V))
    L.token_logprobs(hs[0], U, tg, lp, lse, ws_f)
    samp = (lp + torch.randn(n, generator=gen, device="cuda") * 0.05 * act).contiguous()
    g_custom = (torch.randn(n, generator=gen, device="cuda") * act).contiguous()
    ws_l = L.empty_workspace(L.loss_grad_workspace_bytes(n))
    ws_b = L.empty_workspace(L.token_logprobs_backward_workspace_bytes(n, V, chunk))
    loss = torch.empty(1, device="cuda")
    dl = torch.empty(n, device="cuda")
    dh = torch.empty((n, H), dtype=torch.bfloat16, device="cuda")
    lp2 = torch.empty_like(lp)

    def step_ppo(k):
        h = hs[k % 2]
        L.token_logprobs(h, U, tg, lp, lse, ws_f)
        L.loss_grad(L.LOSS_PPO, lp, act, adv, samp, None, (0.2, 0.2), loss, dl, ws_l)
        L.token_logprobs_backward(h, U, Ut, tg, lse, dl, dh, ws_b)

    def step_custom_one(k):       # the custom path reusing the forward's lse
        h = hs[k % 2]
        L.token_logprobs(h, U, tg, lp, lse, ws_f)
        L.loss_grad(L.LOSS_CUSTOM, lp, act, None, None, g_custom, None, loss, dl, ws_l)
        L.token_logprobs_backward(h, U, Ut, tg, lse, dl, dh, ws_b)

    def step_custom_two(k):       # forward for the client's dLoss/dlogprob, then the
        h = hs[k % 2]             # server's own forward and backward of sum(logprob * g)
        L.token_logprobs(h, U, tg, lp2, lse, ws_f)
        L.token_logprobs(h, U, tg, lp, lse, ws_f)
        L.loss_grad(L.LOSS_CUSTOM, lp, act, None, None, g_custom, None, loss, dl, ws_l)
        L.token_logprobs_backward(h, U, Ut, tg, lse, dl, dh, ws_b)

    ms, ms_instr = timed(step_ppo, steps, warmup, log, f"logprob {n} tokens (PPO)")
    if L.lora_device_status(ws_f) or L.lora_device_status(ws_l):
        raise RuntimeError("logprob: device status flags set")
    f_ms, f_n = timer(L.TIMER_LOGPROB_FWD)
    b_ms, b_n = timer(L.TIMER_LOGPROB_BWD)     # one record per token chunk (two GEMMs)
    chunks = b_n // steps
    rows_per_chunk = n / max(chunks, 1)
    flops_fwd = 2.0 * n * V * H
    ms1, _ = timed(step_custom_one, steps, warmup, log, "custom loss, one forward")
    ms2, _ = timed(step_custom_two, steps, warmup, log, "custom loss, two forwards")
    out = {
        "tokens_per_s": round(n / (ms / 1e3), 1), "ms_per_step": round(ms, 4),
        "ms_per_step_instrumented": round(ms_instr, 4),
        "config": {"workload": f"hidden {H} -> vocab {V}, {n} tokens = 16 groups x 4 x {seq}, "
                               f"prompt {inp['prompt']}/{seq}, PPO clip 0.2, backward chunk "
                               f"{chunk} rows"},
        # dominant kernel: the backward chunk (logits recomputed into G, then dh = G U):
        # 2 x 2 x rows x V x H flops per record
        "roofline": roofline("mfma", "logprob backward chunk: EPI_GRAD GEMM + dh GEMM",
                             2 * 2.0 * rows_per_chunk * V * H, b_ms, peaks_, "flop"),
        "kernels": {"logprob_forward": roofline("mfma", "lm_head GEMM with online logsumexp",
                                                flops_fwd, f_ms, peaks_, "flop")},
        "custom_loss": {
            "ms_one_forward": round(ms1, 4), "ms_two_forward": round(ms2, 4),
            "ms_ppo_step": round(ms, 4),
            "ratio_two_forward_vs_ppo": round(ms2 / ms, 4),
            "ratio_two_vs_one_forward": round(ms2 / ms1, 4),
            "flop_ratio_expected": round(4.0 / 3.0, 4),
            "note": "the pages quote 1.5x FLOPs for the whole model, where the frozen-base backward "
                    "costs about one forward; on this path the backward (recompute + dh) is two "
                    "forwards, so the two-forward protocol costs (2F + 2F) / (F + 2F) = 4/3"},
    }
    if cpu_s > 0:
        log("[bench] logprob: cpu baseline (oracle)")
        out["cpu_baseline"] = _logprob_cpu(hs[0], U, tg, lp, act, adv, samp, cpu_s)
    _free(Ut, ws_f, ws_l, ws_b, dh)
    return out


# ------------------------------------------------------------------ MoE
def _moe_cpu(inp, ex, w, target_s):
    """oracle.moe route + forward + backward on S sampled tokens (all of their K
    assignments), the full expert weights and adapters."""
    import oracle.moe as OE
    E, n_ad, r, H, F = inp["E"], inp["n_ad"], inp["r"], inp["H"], inp["F"]
    t0 = time.perf_counter()
    Wg, Wu, Wd = f64(inp["Wg"]), f64(inp["Wu"]), f64(inp["Wd"])
    A, B = {}, {}
    for p, pack, aoffs, (di, do) in zip(("gate", "up", "down"), inp["packs"], inp["a_offs"],
                                        ((H, F), (H, F), (F, H))):
        pk = f64(pack)
        A[p] = [[None] * E for _ in range(n_ad)]
        B[p] = [[None] * E for _ in range(n_ad)]
        for e in range(E):
            for a in range(n_ad):
                o = int(aoffs[e * n_ad + a])
                A[p][a][e] = pk[o:o + r * di].reshape(r, di)
                B[p][a][e] = pk[o + r * di:o + r * di + do * r].reshape(do, r)
        del pk
    conv = time.perf_counter() - t0
    n = inp["n"]
    ids = inp["ids"].cpu().numpy()
    logits = inp["logits"]
    rng = np.random.default_rng(1)
    S, spent, tokens = 256, 0.0, 0
    while True:
        ts = np.sort(rng.choice(n, S, replace=False))
        sel = torch.from_numpy(ts).cuda()
        xs, dys = f64(inp["xs"][0][sel]), f64(inp["dys"][0][sel])
        R = logits[sel].cpu().numpy()
        t1 = time.perf_counter()
        e_s, w_s = OE.moe_route(R, inp["K"])
        y, saved = OE.moe_forward(xs, e_s, w_s, ids[ts], Wg, Wu, Wd, A, B, 32.0 / r)
        OE.moe_backward(dys, xs, e_s, w_s, ids[ts], Wg, Wu, Wd, A, B, 32.0 / r, saved)
        spent += time.perf_counter() - t1
        tokens += S
        if spent > target_s or tokens >= n:
            break
    return cpu_entry(tokens, spent, f"oracle.moe route + fwd + bwd on {tokens} sampled tokens "
                                    f"(batches of {S}, all K assignments each) over the full "
                                    f"expert weights and adapters (float64 conversion {conv:.1f} s, "
                                    "not timed)")


def moe(steps, warmup, log, peaks_=None, cpu_s=8.0, n=16384, H=2048, F=768, E=128, K=8, n_ad=8,
        r=32):
    inp = WD.moe_inputs(n, H, F, E, K, n_ad, r)
    logits, ids, Wg, Wu, Wd, xs, dys = (inp[k] for k in ("logits", "ids", "Wg", "Wu", "Wd", "xs",
                                                          "dys"))
    Wgt, Wut = (torch.empty((E, H, F), dtype=torch.bfloat16, device="cuda") for _ in range(2))
    Wdt = torch.empty((E, F, H), dtype=torch.bfloat16, device="cuda")
    for e in range(E):
        L.lora_transpose_bf16(Wg[e], Wgt[e])
        L.lora_transpose_bf16(Wu[e], Wut[e])
        L.lora_transpose_bf16(Wd[e], Wdt[e])
    packs = inp["packs"]
    descs = [L.make_desc(a_off, a_off + r * di, np.full(a_off.size, r, np.int32),
                         np.full(a_off.size, 32.0 / r, np.float32))
             for a_off, di in zip(inp["a_offs"], (H, H, F))]
    shape = L.MoeShape(n, H, F, packs[0].numel(), packs[1].numel(), packs[2].numel(), E, K, n_ad, r)
    ws = L.empty_workspace(L.moe_workspace_bytes(shape))
    saved = torch.empty(L.moe_saved_bytes(shape), dtype=torch.uint8, device="cuda")
    ex = torch.empty((n, K), dtype=torch.int32, device="cuda")
    w = torch.empty((n, K), device="cuda")
    y = torch.empty((n, H), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty_like(y)
    grads = [torch.zeros(p.numel(), dtype=torch.float32, device="cuda") for p in packs]

    def step(k):
        L.moe_route(logits, K, ex, w)
        L.moe_forward(shape, xs[k % 2], ex, w, ids, Wg, Wu, Wd, packs, descs, y, saved, ws)
        L.moe_backward(shape, dys[k % 2], xs[k % 2], ex, w, ids, Wgt, Wut, Wdt, packs, descs, saved,
                       dx, grads, 0, ws)

    ms, ms_instr = timed(step, steps, warmup, log, f"moe {n} tokens")
    if L.lora_device_status(ws):
        raise RuntimeError("moe: device status flags set")
    gemm_ms, gemm_n = timer(L.TIMER_BASE_GEMM)
    shr_ms, shr_n = timer(L.TIMER_SHRINK)
    grd_ms, grd_n = timer(L.TIMER_GRAD)
    flops_step = 6 * 2.0 * n * K * H * F
    per_step = gemm_n / steps
    out = {
        "tokens_per_s": round(n / (ms / 1e3), 1), "ms_per_step": round(ms, 4),
        "ms_per_step_instrumented": round(ms_instr, 4),
        "config": {"workload": f"qwen3-30b-a3b-style MoE: {E} experts top-{K}, hidden {H}, expert "
                               f"intermediate {F}, {n_ad} adapters r{r} alpha 32 on every expert's "
                               f"gate/up/down, {n} tokens random adapter ids; route + fwd + bwd"},
        "roofline": roofline("mfma", "grouped expert GEMMs: 6 x 2*N*K*H*F per step in 4 launches",
                             flops_step / per_step, gemm_ms, peaks_, "flop"),
        "kernels": {"shrink_ms_per_step": round(shr_ms * shr_n / steps, 4),
                    "grad_ms_per_step": round(grd_ms * grd_n / steps, 4),
                    "gemm_ms_per_step": round(gemm_ms * gemm_n / steps, 4)},
    }
    if cpu_s > 0:
        log("[bench] moe: cpu baseline (oracle)")
        out["cpu_baseline"] = _moe_cpu(inp, ex, w, cpu_s)
    _free(Wgt, Wut, Wdt, ws, saved, y, dx, *grads)
    return out


# ------------------------------------------------------------------ decode
def decode(steps, warmup, log, peaks_=None, cpu_s=3.0, n=256, d=4096, n_ad=64):
    inp = WD.decode_inputs(n, d, n_ad)
    R = 64
    shape = L.make_shape(n, d, d, inp["pack"].numel(), inp["pack"].numel(), n_ad, R,
                         L.IDS_INTERLEAVED)
    desc = L.make_desc(inp["a_off"], inp["b_off"], inp["ranks"], inp["scales"])
    ws = L.empty_workspace(L.lora_workspace_bytes(shape))
    y = torch.empty((n, d), dtype=torch.bfloat16, device="cuda")
    u = torch.empty((2, n, R), dtype=torch.bfloat16, device="cuda")

    def step(k):
        L.lora_forward(shape, inp["xs"][k % 4], inp["W"], inp["pack"], inp["pack"], desc,
                       inp["ids"], y, u, ws)

    ms, ms_instr = timed(step, steps, warmup, log, f"decode forward {n} tokens")
    if L.lora_device_status(ws):
        raise RuntimeError("decode: device status flags set")
    gemm_ms, _ = timer(L.TIMER_BASE_GEMM)
    shr_ms, _ = timer(L.TIMER_SHRINK)
    gemm_bytes = d * d * 2 + 2 * n * d * 2          # W once, x read, y written
    out = {
        "tokens_per_s": round(n / (ms / 1e3), 1), "ms_per_step": round(ms, 4),
        "ms_per_step_instrumented": round(ms_instr, 4),
        "config": {"workload": f"decode-step forward: {n} tokens (one per sequence), {n_ad} "
                               f"adapters r8-64 alpha 32, interleaved ids, d {d} -> {d}"},
        "roofline": roofline("hbm", "few-row base GEMM with the fused expand (W read once)",
                             gemm_bytes, gemm_ms, peaks_, "byte"),
        "kernels": {"shrink_avg_ms": round(shr_ms, 5)},
    }
    if cpu_s > 0:
        import oracle.lora as OL
        log("[bench] decode: cpu baseline (oracle)")
        Wd = f64(inp["W"])
        p = f64(inp["pack"])
        ranks = inp["ranks"]
        A = [p[inp["a_off"][i]:inp["a_off"][i] + r * d].reshape(r, d) for i, r in enumerate(ranks)]
        B = [p[inp["b_off"][i]:inp["b_off"][i] + d * r].reshape(d, r) for i, r in enumerate(ranks)]
        x64, ids = f64(inp["xs"][0]), inp["ids"].cpu().numpy()
        spent, reps = 0.0, 0
        while spent < cpu_s:
            t0 = time.perf_counter()
            OL.lora_forward(x64, Wd, A, B, inp["scales"].astype(np.float64), ids)
            spent += time.perf_counter() - t0
            reps += 1
        out["cpu_baseline"] = cpu_entry(reps * n, spent, f"oracle.lora forward on the whole "
                                                         f"{n}-token batch, {reps} times")
    _free(ws, y, u)
    return out


# ------------------------------------------------------------------ AdamW over a whole adapter
ADAPTER_PARAMS_8B_R32 = 87_293_952   # 36 layers x 32 x (2(4096+4096) + 2(4096+1024) + 3(4096+12288))


def adam(steps, warmup, log, peaks_=None, cpu_s=3.0, n=ADAPTER_PARAMS_8B_R32):
    """One adapter's AdamW step over all of a rank-32 Qwen3-8B adapter (every
    projection of every layer as one flat range), with the bf16 copy."""
    gen = torch.Generator(device="cuda").manual_seed(6)
    p = torch.randn(n, generator=gen, device="cuda") * 0.02
    g = torch.randn(n, generator=gen, device="cuda") * 1e-3
    m = torch.zeros(n, device="cuda")
    v = torch.zeros(n, device="cuda")
    pb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    ws = L.empty_workspace(L.adam_workspace_bytes(1))
    t = [0]

    def step(k):
        t[0] += 1
        L.adam_step(p, g, m, v, t[0], 1e-4, 0.9, 0.999, 1e-8, 0.0, p_bf16=pb, ws=ws)

    ms, ms_instr = timed(step, steps, warmup, log, f"adam {n} params")
    if L.lora_device_status(ws):
        raise RuntimeError("adam: device status flags set")
    a_ms, _ = timer(L.TIMER_ADAM)
    out = {"params": n, "ms_per_step": round(ms, 4), "ms_per_step_instrumented": round(ms_instr, 4),
           # algorithmic bytes: p, m, v read and written, g read, bf16 copy written
           "roofline": roofline("hbm", "AdamW (flag clear, gradient scan, update) over one adapter",
                                30.0 * n, a_ms, peaks_, "byte"),
           "config": {"workload": "one AdamW step over a whole rank-32 Qwen3-8B adapter "
                                  f"({n} params) with its bf16 copy"}}
    if cpu_s > 0:
        import oracle.adam as OA
        k = n // 16
        pp, gg = p[:k].cpu().numpy().astype(np.float64), g[:k].cpu().numpy().astype(np.float64)
        zz = np.zeros(k)
        spent, reps = 0.0, 0
        while spent < cpu_s:
            t0 = time.perf_counter()
            OA.adam_step(pp, gg, zz, zz, 1, 1e-4)
            spent += time.perf_counter() - t0
            reps += 1
        out["cpu_baseline"] = cpu_entry(reps * k, spent, f"oracle.adam on the first {k} params "
                                                         f"(1/16 of the adapter), {reps} times",
                                        unit="params/s")
    _free(p, g, m, v, pb, ws)
    return out
