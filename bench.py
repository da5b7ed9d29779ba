"""Benchmark of the mixed-adapter LoRA training hot path on one MI355X.

Headline step (`value`): one pass of the hot path over a Qwen3-8B-width q/o
projection (4096 -> 4096, bf16, fp32 accumulate) with 16 rank-32 adapters
(alpha 32) over 8192 tokens in sorted 512-token segments -- segment build,
shrink and the base GEMM with the LoRA expand in its epilogue (forward), the
same for dX plus the adapter-gradient reductions (backward), and one AdamW
step per adapter (lr 1e-4, betas 0.9/0.999, eps 1e-8) writing the bf16 copy
the next forward reads.  Inputs are seeded synthetic data resident in HBM
before timing; four rotated copies of (x, dY) keep the 256 MB Infinity Cache
from serving repeat reads.  `tokens_per_s_fwd_bwd` times the same step
without the AdamW launch (tokens / (t_fwd + t_bwd)).

Prints ONE JSON line on stdout.  `roofline` is for the dominant kernel (the
base GEMM), timed live with HIP events the library records around each of its
launches on the launch stream, in a second pass of the same number of steps
(reported as ms_per_step_instrumented).  `cpu_baseline` times the oracle
(NumPy float64) on the host cores.  Unless --quick, `configs` carries the MLP,
fused logprob + RL loss (with the custom-loss path timed two ways), routed
expert and decode workloads, each with its own roofline and CPU baseline,
`adam_whole_model` an AdamW step over a whole rank-32 Qwen3-8B adapter, and
`measured_peaks` the chip's own MFMA and copy rates (bench_workloads.py).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E

METRIC = "tokens/s mixed-adapter LoRA fwd+bwd at 8B shapes; % MFMA / HBM peak"

# HBM bytes per base-GEMM launch at this workload, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE passes scaled by a 512 MiB copy's readings (x2 fetch, x1 write):
# profiles/gemm_nt_traffic_8192x4096x4096.md.  Valid only for the kernel source the
# counters were taken on (sha256 prefix of gemm.hip + common.hpp); else reported null.
GEMM_TRAFFIC = {"bytes_per_launch": 476.6e6, "src_sha256": "24e916bb20ed11bf"}


def gemm_traffic():
    import hashlib
    csrc = os.path.join(ROOT, "rl_lora_linear_amd", "csrc")
    h = hashlib.sha256()
    for f in ("gemm.hip", "common.hpp"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return GEMM_TRAFFIC["bytes_per_launch"] if h.hexdigest()[:16] == GEMM_TRAFFIC["src_sha256"] else None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--tokens", type=int, default=8192)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target wall time of the oracle sample")
    ap.add_argument("--workload", default="qo_proj",
                    choices=["qo_proj", "mlp", "logprob", "moe", "decode", "adam", "peaks"],
                    help="qo_proj (default): the headline step, with every other workload in "
                         "`configs` unless --quick; mlp / logprob / moe / decode / adam / peaks: "
                         "that workload alone, one JSON line")
    ap.add_argument("--quick", action="store_true",
                    help="headline step only (no other workloads, no measured peaks)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="only run a plain device copy of MB megabytes 5 times (calibrates "
                         "the FETCH_SIZE / WRITE_SIZE counters against known bytes) and exit")
    return ap.parse_args()


def cpu_baseline(case, target_s):
    """Time the oracle's forward + backward (+ Adam prorated) on the host."""
    import numpy as np
    import bench_workloads as BW
    import oracle.adam as OA
    import oracle.lora as OL

    x = case.x()
    Wb = case.W()
    dy = case.dy()
    A = [case.A(i) for i in range(case.n_adapters)]
    B = [case.B(i) for i in range(case.n_adapters)]
    s = case.scales
    # sample: whole adapters' segments (gradients need every token of an adapter)
    per = case.n_tokens // case.n_adapters
    n_ad_sample = case.n_adapters
    t_layer = 0.0
    reps = 0
    t0 = time.perf_counter()
    while True:
        a = reps % case.n_adapters
        rows = np.nonzero(case.ids == a)[0]
        ts = time.perf_counter()
        y, u = OL.lora_forward(x[rows], Wb, A, B, s, case.ids[rows])
        OL.lora_backward(dy[rows], x[rows], Wb, A, B, s, case.ids[rows])
        t_layer += time.perf_counter() - ts
        reps += 1
        if time.perf_counter() - t0 > target_s or reps >= 4 * n_ad_sample:
            break
    tokens_done = reps * per
    # Adam for one adapter, prorated per token
    r0, r1 = case.adapter_range(0)
    n_par = r1 - r0
    g = np.random.default_rng(0).standard_normal(n_par)
    ts = time.perf_counter()
    OA.adam_step(np.zeros(n_par), g, np.zeros(n_par), np.zeros(n_par), 1, 1e-4)
    t_adam_one = time.perf_counter() - ts
    t_adam_per_token = t_adam_one * case.n_adapters / case.n_tokens
    tps = tokens_done / (t_layer + t_adam_per_token * tokens_done)
    out = {"value": round(tps, 2), "unit": "tokens/s", "kind": "oracle",
           "sample": f"{reps} adapter segments x {per} tokens of the same workload "
                     f"(fp64 NumPy fwd+bwd, {t_layer:.1f} s) + one adapter's AdamW prorated per token",
           "tokens_per_s_fwd_bwd": round(tokens_done / t_layer, 2)}
    out.update(BW.host_info())
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the path runs on "
              "one MI355X; sharding it over several GPUs is designed, not built or measured.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 5}))
        return

    import bench_workloads as BW
    cpu_s = 0.0 if args.no_cpu_baseline else 8.0
    if args.workload != "qo_proj":
        torch.cuda.set_device(0)
        if args.workload == "peaks":
            out = BW.peaks(log)
        else:
            out = getattr(BW, args.workload)(args.steps, args.warmup, log, None, cpu_s)
        out.update({"workload": args.workload, "n_gpus": 1, "steps": args.steps,
                    "warmup": args.warmup, "dtype": "bf16",
                    "data": "synthetic (seeded, generated on the device)"})
        print(json.dumps(out), flush=True)
        return

    import rl_lora_linear_amd.lib as L
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    peaks = None if args.quick else BW.peaks(log)
    log(f"[bench] generating inputs ({args.tokens} tokens)")
    case = W.attn_proj(seed=2, n_tokens=args.tokens)
    N, d_in, d_out = case.n_tokens, case.d_in, case.d_out
    n_ad = case.n_adapters
    max_rank = max(16, -(-int(case.ranks.max()) // 16) * 16)

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    shape = L.make_shape(N, d_in, d_out, case.pack_elems, case.pack_elems, n_ad, max_rank,
                         L.IDS_SORTED)
    x0, dy0, Wm = dev_bf16(case.x_bits), dev_bf16(case.dy_bits), dev_bf16(case.W_bits)
    Wt = torch.empty((d_in, d_out), dtype=torch.bfloat16, device=dev)
    L.lora_transpose_bf16(Wm, Wt)
    pack = dev_bf16(case.pack_bits)
    desc = L.make_desc(case.a_off, case.b_off, case.ranks, case.scales.astype(np.float32))
    ids = torch.from_numpy(case.ids.astype(np.int32)).to(dev)
    ws = L.empty_workspace(L.lora_workspace_bytes(shape))
    # rotated input sets
    sets = []
    for k in range(4):
        xs = torch.roll(x0, shifts=k * 97, dims=0).contiguous()
        dys = torch.roll(dy0, shifts=k * 89, dims=0).contiguous()
        sets.append((xs, dys))
    y = torch.empty((N, d_out), dtype=torch.bfloat16, device=dev)
    u = torch.empty((2, N, max_rank), dtype=torch.bfloat16, device=dev)   # hi/lo planes
    dx = torch.empty((N, d_in), dtype=torch.bfloat16, device=dev)
    grad = torch.zeros(case.pack_elems, dtype=torch.float32, device=dev)
    master = pack.float().clone()
    m = torch.zeros_like(master)
    v = torch.zeros_like(master)
    ranges = [case.adapter_range(i) for i in range(n_ad)]
    ws_adam = L.empty_workspace(L.adam_workspace_bytes(n_ad))
    steps_done = [0]

    def step(k, with_adam=True):
        xs, dys = sets[k % len(sets)]
        L.lora_forward(shape, xs, Wm, pack, pack, desc, ids, y, u, ws)
        L.lora_backward(shape, dys, xs, Wt, pack, pack, desc, ids, u, dx, grad, grad, 0, ws)
        if not with_adam:
            return
        t = steps_done[0] + 1
        # every adapter in the batch takes its own AdamW step
        L.adam_step_multi([(a0, a1 - a0, t) for (a0, a1) in ranges], master, grad, m, v, 1e-4,
                          0.9, 0.999, 1e-8, 0.0, p_bf16=pack, ws=ws_adam)
        steps_done[0] = t

    log(f"[bench] warmup {args.warmup}")
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    flags = L.lora_device_status(ws) | L.lora_device_status(ws_adam)
    if flags:
        raise RuntimeError(f"device status flags {flags:#x}")

    def timed(instrumented, with_adam=True):
        L.lora_timing_reset()
        L.lora_timing_enable(instrumented)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            step(k, with_adam)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        L.lora_timing_enable(False)
        return (t1 - t0) * 1e3 / args.steps

    log(f"[bench] timing {args.steps} steps")
    ms_step = timed(False)
    tokens_s = N / (ms_step / 1e3)
    log(f"[bench] timing {args.steps} steps without the AdamW launch")
    ms_fwd_bwd = timed(False, with_adam=False)
    log(f"[bench] timing {args.steps} instrumented steps (kernel durations)")
    ms_step_instr = timed(True)

    timers = {}
    for name, tid in (("base_gemm", L.TIMER_BASE_GEMM), ("shrink", L.TIMER_SHRINK),
                      ("grad", L.TIMER_GRAD), ("adam", L.TIMER_ADAM)):
        tot, cnt = L.lora_timing_read(tid)
        timers[name] = (tot, cnt)
    gemm_ms, gemm_n = timers["base_gemm"]
    gemm_avg_ms = gemm_ms / max(gemm_n, 1)
    gemm_flops = 2.0 * N * d_in * d_out
    achieved = gemm_flops / (gemm_avg_ms / 1e3) / 1e12

    # algorithmic bytes of the HBM-bound kernels (per launch)
    r = int(case.ranks[0])
    shrink_bytes = (N * d_in * 2 + n_ad * r * d_in * 2 + N * max_rank * 4)
    grad_bytes = (N * d_out * 2 + N * max_rank * 4 + n_ad * d_out * r * 4) + \
                 (N * d_in * 2 + N * max_rank * 4 + n_ad * r * d_in * 4)
    adam_bytes = 30 * sum(a1 - a0 for a0, a1 in ranges)   # p,m,v r+w, g r, bf16 copy w

    def kentry(name, bytes_per_launch, launches_per_step):
        tot, cnt = timers[name]
        avg = tot / max(cnt, 1)
        gbs = bytes_per_launch / (avg / 1e3) / 1e9 if avg > 0 else 0.0
        return {"avg_ms": round(avg, 5), "launches": cnt, "bytes_per_launch": int(bytes_per_launch),
                "GB_s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}

    kernels = {
        "base_gemm": {"avg_ms": round(gemm_avg_ms, 5), "launches": gemm_n,
                      "TFLOP_s": round(achieved, 1), "frac_mfma": round(achieved / PEAK_BF16_TFLOPS, 4)},
        "shrink": kentry("shrink", shrink_bytes, 2),
        "grad_dA_dB": kentry("grad", grad_bytes, 1),
        "adam_all_adapters": kentry("adam", adam_bytes, 1),
    }
    out = {
        "metric": METRIC,
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_instrumented": round(ms_step_instr, 4),
        "tokens_per_s_fwd_bwd": round(N / (ms_fwd_bwd / 1e3), 1),
        "ms_fwd_bwd": round(ms_fwd_bwd, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; random-init Qwen3-8B-width projection and adapters)",
        "config": {"workload": "qwen3-8b q/o projection 4096->4096, 16 adapters rank 32 alpha 32, "
                               f"{N} tokens (16 sorted segments), fwd+bwd+AdamW",
                   "tokens": N, "d_in": d_in, "d_out": d_out, "adapters": n_ad, "rank": r},
        "roofline": {"bound": "mfma", "kernel": "base GEMM (y = x W^T and dx = dy W, bf16 MFMA)",
                     "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": gemm_traffic(),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 counters)"},
        "kernels": kernels,
    }
    if peaks:
        out["measured_peaks"] = peaks
        out["roofline"]["measured_peak"] = peaks["mfma_bf16_tflops"]
        out["roofline"]["frac_measured_peak"] = round(achieved / peaks["mfma_bf16_tflops"], 4)
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    if not args.quick:
        del sets, y, u, dx, grad, master, m, v, ws
        torch.cuda.empty_cache()
        cfgs = {}
        for name in ("mlp", "logprob", "moe", "decode"):
            cfgs[name] = getattr(BW, name)(args.steps, args.warmup, log, peaks, cpu_s)
        out["configs"] = cfgs
        out["adam_whole_model"] = BW.adam(args.steps, args.warmup, log, peaks,
                                          0.0 if args.no_cpu_baseline else 3.0)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
