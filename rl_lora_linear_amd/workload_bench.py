"""Timed steps of the MLP, fused-logprob and routed-expert workloads (device
inputs, seeded and synthetic, generated on the GPU).  Used by bench.py
--workload; every step runs through the library's C entry points."""
from __future__ import annotations

import time

import numpy as np
import torch

from . import lib as L

import workloads.device as WD

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def _timed(step, steps, warmup, log):
    """ms per step with no instrumentation; then a second pass of `steps`
    steps with the library's HIP-event timers on (kernel durations, read with
    _timer).  Returns (ms, instrumented ms)."""
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

    log(f"[bench] timing {steps} steps, then {steps} instrumented steps")
    ms = run(False)
    return ms, run(True)


def _timer(tid):
    tot, cnt = L.lora_timing_read(tid)
    return tot / max(cnt, 1), cnt


def mlp(steps, warmup, log, n=32768, d=4096, f=12288, n_ad=64):
    """SwiGLU MLP layer (mlp_forward + mlp_backward), 64 adapters with ranks from
    {8,16,32,64} on each projection, interleaved ids."""
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

    log(f"[bench] mlp {n} tokens, d {d}, d_ff {f}, {n_ad} adapters")
    ms, ms_instr = _timed(step, steps, warmup, log)
    if L.lora_device_status(ws):
        raise RuntimeError("device status flags set")
    gemm_ms, gemm_n = _timer(L.TIMER_BASE_GEMM)
    # 6 projections of 2*N*d*d_ff per step in 4 GEMM launches (gate+up with the
    # SwiGLU, down; dh with the SwiGLU backward, the gate/up dX K-concatenated)
    flops_step = 6 * 2.0 * n * d * f
    gemm_step_ms = gemm_ms * gemm_n / steps
    tf = flops_step / (gemm_step_ms / 1e3) / 1e12
    return {
        "metric": "tokens/s mixed-adapter LoRA MLP fwd+bwd", "value": round(n / (ms / 1e3), 1),
        "unit": "tokens/s", "ms_per_step": round(ms, 4), "ms_per_step_instrumented": round(ms_instr, 4),
        "config": {"workload": f"qwen3-8b MLP gate/up {d}->{f}, down {f}->{d}, {n_ad} adapters "
                               f"ranks {{8,16,32,64}} alpha 32, {n} tokens interleaved ids, fwd+bwd",
                   "rank_counts": {int(r): int((ranks == r).sum()) for r in (8, 16, 32, 64)}},
        "roofline": {"bound": "mfma",
                     "kernel": "base GEMMs (6 projections of 2*N*d*d_ff per step in 4 launches)",
                     "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4), "avg_ms": round(gemm_ms, 4),
                     "gemm_ms_per_step": round(gemm_step_ms, 4), "launches": gemm_n},
    }


def logprob(steps, warmup, log, n_seq=64, seq=256, H=4096, V=151936, chunk=4096):
    """Fused lm_head logprob + PPO loss + logprob backward, 16 groups x 4 x 256."""
    inp = WD.logprob_inputs(n_seq, seq, H, V)
    n, hs, U, tg, act, adv, gen = (inp[k] for k in ("n", "hs", "U", "targets", "act", "adv", "gen"))
    prompt = inp["prompt"]
    Ut = torch.empty((H, V), dtype=torch.bfloat16, device="cuda")
    L.lora_transpose_bf16(U, Ut)
    lp = torch.empty(n, device="cuda")
    lse = torch.empty(n, device="cuda")
    ws_f = L.empty_workspace(L.token_logprobs_workspace_bytes(n, V))
    L.token_logprobs(hs[0], U, tg, lp, lse, ws_f)
    samp = (lp + torch.randn(n, generator=gen, device="cuda") * 0.05 * act).contiguous()
    ws_l = L.empty_workspace(L.loss_grad_workspace_bytes(n))
    ws_b = L.empty_workspace(L.token_logprobs_backward_workspace_bytes(n, V, chunk))
    loss = torch.empty(1, device="cuda")
    dl = torch.empty(n, device="cuda")
    dh = torch.empty((n, H), dtype=torch.bfloat16, device="cuda")

    def step(k):
        h = hs[k % 2]
        L.token_logprobs(h, U, tg, lp, lse, ws_f)
        L.loss_grad(L.LOSS_PPO, lp, act, adv, samp, None, (0.2, 0.2), loss, dl, ws_l)
        L.token_logprobs_backward(h, U, Ut, tg, lse, dl, dh, ws_b)   # chunk from ws size

    log(f"[bench] logprob {n} tokens, H {H}, V {V}")
    ms, ms_instr = _timed(step, steps, warmup, log)
    f_ms, f_n = _timer(L.TIMER_LOGPROB_FWD)
    b_ms, b_n = _timer(L.TIMER_LOGPROB_BWD)     # one record per token chunk
    b_step_ms = b_ms * b_n / steps
    flops = 2.0 * n * V * H
    tf_f = flops / (f_ms / 1e3) / 1e12
    tf_b = 2 * flops / (b_step_ms / 1e3) / 1e12
    return {
        "metric": "tokens/s fused lm_head logprob + PPO loss + logprob backward",
        "value": round(n / (ms / 1e3), 1), "unit": "tokens/s", "ms_per_step": round(ms, 4), "ms_per_step_instrumented": round(ms_instr, 4),
        "config": {"workload": f"hidden {H} -> vocab {V}, {n} tokens = 16 groups x 4 x {seq}, "
                               f"prompt {prompt}/{seq}, PPO clip 0.2, backward chunk {chunk} rows"},
        "roofline": {"bound": "mfma", "kernel": "lm_head GEMM with online logsumexp (forward)",
                     "achieved": round(tf_f, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf_f / PEAK_BF16_TFLOPS, 4), "avg_ms": round(f_ms, 4)},
        "kernels": {"logprob_backward": {"ms_per_step": round(b_step_ms, 4), "chunks": b_n // steps,
                                         "TFLOP_s": round(tf_b, 1),
                                         "frac_mfma": round(tf_b / PEAK_BF16_TFLOPS, 4)}},
    }


def decode(steps, warmup, log, n=256, d=4096, n_ad=64):
    """Rollout-shaped mixed-adapter forward (lora_forward only): 256 tokens, one
    per sequence of a decode step, over 64 adapters with ranks from
    {8,16,32,64}, interleaved ids, d 4096 -> 4096.  The base GEMM at this
    height reads the whole weight for few rows, so its bound is HBM."""
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

    log(f"[bench] decode forward {n} tokens, d {d}, {n_ad} adapters")
    ms, ms_instr = _timed(step, steps, warmup, log)
    if L.lora_device_status(ws):
        raise RuntimeError("device status flags set")
    gemm_ms, gemm_n = _timer(L.TIMER_BASE_GEMM)
    gemm_bytes = d * d * 2 + 2 * n * d * 2   # W once, x and y
    gbs = gemm_bytes / (gemm_ms / 1e3) / 1e9
    return {
        "metric": "tokens/s mixed-adapter LoRA forward at decode batch",
        "value": round(n / (ms / 1e3), 1), "unit": "tokens/s", "ms_per_step": round(ms, 4),
        "ms_per_step_instrumented": round(ms_instr, 4),
        "config": {"workload": f"decode-step forward: {n} tokens (one per sequence), {n_ad} "
                               f"adapters r8-64 alpha 32, interleaved ids, d {d} -> {d}"},
        "roofline": {"bound": "hbm", "kernel": "base GEMM with the fused expand (W read once)",
                     "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "avg_ms": round(gemm_ms, 4)},
    }


def moe(steps, warmup, log, n=16384, H=2048, F=768, E=128, K=8, n_ad=8, r=32):
    """Qwen3-30B-A3B-style routed layer: top-8 of 128 experts, 8 rank-32 adapters
    on every expert's gate/up/down; route + forward + backward."""
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

    log(f"[bench] moe {n} tokens, {E} experts top-{K}, H {H}, F {F}, {n_ad} adapters r{r}")
    ms, ms_instr = _timed(step, steps, warmup, log)
    if L.lora_device_status(ws):
        raise RuntimeError("device status flags set")
    gemm_ms, gemm_n = _timer(L.TIMER_BASE_GEMM)
    # 6 expert projections of 2*N*K*H*F each per step, run as 4 grouped GEMM
    # launches (gate+up fused in the forward, the gate and up dX in one K-concatenated GEMM)
    flops_step = 6 * 2.0 * n * K * H * F
    gemm_step_ms = gemm_ms * gemm_n / steps
    tf = flops_step / (gemm_step_ms / 1e3) / 1e12
    return {
        "metric": "tokens/s mixed-adapter LoRA routed-expert layer fwd+bwd",
        "value": round(n / (ms / 1e3), 1), "unit": "tokens/s", "ms_per_step": round(ms, 4), "ms_per_step_instrumented": round(ms_instr, 4),
        "config": {"workload": f"qwen3-30b-a3b-style MoE: {E} experts top-{K}, hidden {H}, "
                               f"expert intermediate {F}, {n_ad} adapters r{r} alpha 32 on every "
                               f"expert's gate/up/down, {n} tokens random adapter ids; "
                               "route + fwd + bwd"},
        "roofline": {"bound": "mfma",
                     "kernel": "grouped expert GEMMs (6 projections of 2*N*K*H*F per step in "
                               "4 launches)",
                     "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4), "avg_ms": round(gemm_ms, 4),
                     "gemm_ms_per_step": round(gemm_step_ms, 4), "launches": gemm_n},
    }
