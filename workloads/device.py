"""Seeded synthetic inputs drawn on the GPU (torch's Philox generator) for the
full-size workloads, shared by bench.py and the full-size parity tests.

Drawing 10^8-10^9 values with numpy takes minutes; these generators draw them on
the device in seconds.  They hold none of the hot path's arithmetic: random
draws, bf16 rounding and packing only.  Distributions are those of the
host-side generators: activations N(0, 1), frozen weights N(0, 0.02), LoRA A
uniform +-1/sqrt(d_in), B N(0, 0.01) (pack tests) or N(0, 0.01) for both in the
expert packs, router logits N(0, 1), adapter ids uniform.  A caller needs a
GPU build of torch.
"""
from __future__ import annotations

import numpy as np


def _torch():
    import torch
    return torch


def randn(gen, shape, std, dtype=None):
    torch = _torch()
    dtype = dtype or torch.bfloat16
    return (torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32) * std).to(dtype)


def adapter_pack(gen, ranks, d_in, d_out):
    """One projection's adapter pack (A_i then B_i per adapter) and its offsets:
    A uniform +-1/sqrt(d_in), B N(0, 0.01)."""
    torch = _torch()
    a_off, b_off, off = [], [], 0
    for r in ranks:
        a_off.append(off)
        b_off.append(off + r * d_in)
        off += r * (d_in + d_out)
    pack = torch.empty(off, dtype=torch.bfloat16, device="cuda")
    for i, r in enumerate(ranks):
        pack[a_off[i]:b_off[i]] = ((torch.rand(r * d_in, generator=gen, device="cuda") * 2 - 1)
                                   / np.sqrt(d_in)).to(torch.bfloat16)
        pack[b_off[i]:b_off[i] + d_out * r] = randn(gen, (d_out * r,), 0.01)
    return pack, np.asarray(a_off), np.asarray(b_off)


def mlp_inputs(n=32768, d=4096, f=12288, n_ad=64, seed=3, rank_choices=(8, 16, 32, 64)):
    """Qwen3-8B-width SwiGLU MLP: gate/up d->f, down f->d, n_ad adapters with
    ranks from rank_choices (alpha 32) on each projection, interleaved ids.
    Returns a dict: ids, ranks, scales, W (gate, up, down; [d_out][d_in]),
    packs, a_off/b_off per projection, xs and dys (two rotated sets each)."""
    torch = _torch()
    gen = torch.Generator(device="cuda").manual_seed(seed)
    rng = np.random.default_rng(seed)
    ranks = rng.choice(np.asarray(rank_choices), size=n_ad).astype(np.int32)
    scales = (32.0 / ranks).astype(np.float32)
    ids = torch.from_numpy(rng.integers(0, n_ad, size=n).astype(np.int32)).cuda()
    Ws, packs, offs = [], [], []
    for di, do in ((d, f), (d, f), (f, d)):
        Ws.append(randn(gen, (do, di), 0.02))
        pack, ao, bo = adapter_pack(gen, ranks, di, do)
        packs.append(pack)
        offs.append((ao, bo))
    xs = [randn(gen, (n, d), 1.0) for _ in range(2)]
    dys = [randn(gen, (n, d), 1.0) for _ in range(2)]
    return dict(n=n, d=d, f=f, n_ad=n_ad, ids=ids, ranks=ranks, scales=scales, W=Ws,
                packs=packs, offs=offs, xs=xs, dys=dys)


def decode_inputs(n=256, d=4096, n_ad=64, seed=7, rank_choices=(8, 16, 32, 64)):
    """Rollout-shaped forward: n tokens (one per sequence in a decode step) over
    n_ad adapters with ranks from rank_choices (alpha 32), interleaved ids, one
    Qwen3-8B-width projection d -> d.  Returns a dict: ids, ranks, scales, W
    ([d][d]), pack, a_off, b_off, xs (four rotated sets)."""
    torch = _torch()
    gen = torch.Generator(device="cuda").manual_seed(seed)
    rng = np.random.default_rng(seed)
    ranks = rng.choice(np.asarray(rank_choices), size=n_ad).astype(np.int32)
    scales = (32.0 / ranks).astype(np.float32)
    ids = torch.from_numpy(rng.integers(0, n_ad, size=n).astype(np.int32)).cuda()
    W = randn(gen, (d, d), 0.02)
    pack, a_off, b_off = adapter_pack(gen, ranks, d, d)
    xs = [randn(gen, (n, d), 1.0) for _ in range(4)]
    return dict(n=n, d=d, n_ad=n_ad, ids=ids, ranks=ranks, scales=scales, W=W, pack=pack,
                a_off=a_off, b_off=b_off, xs=xs)


def moe_inputs(n=16384, H=2048, F=768, E=128, K=8, n_ad=8, r=32, seed=5):
    """Qwen3-30B-A3B-style routed layer: E experts, top-K, rank-r LoRA (alpha 32)
    on every expert's gate/up/down for each of n_ad adapters, random ids.
    Pack layout: entry (e, a) at ((a * E + e) * r * (d_in + d_out)), A then B.
    Returns a dict: logits, ids, Wg, Wu ([E][F][H]), Wd ([E][H][F]), packs,
    a_off (per projection, [E * n_ad] in (e, a) order), xs, dys."""
    torch = _torch()
    gen = torch.Generator(device="cuda").manual_seed(seed)
    rng = np.random.default_rng(seed)
    logits = torch.randn((n, E), generator=gen, device="cuda")
    ids = torch.from_numpy(rng.integers(0, n_ad, size=n).astype(np.int32)).cuda()
    Wg, Wu = randn(gen, (E, F, H), 0.02), randn(gen, (E, F, H), 0.02)
    Wd = randn(gen, (E, H, F), 0.02)
    packs, a_offs = [], []
    for (di, do) in ((H, F), (H, F), (F, H)):
        per = r * (di + do)
        pack = torch.empty(n_ad * E * per, dtype=torch.bfloat16, device="cuda")
        pack.copy_(randn(gen, (pack.numel(),), 0.01))
        packs.append(pack)
        a_offs.append(np.array([(a * E + e) * per for e in range(E) for a in range(n_ad)]))
    xs = [randn(gen, (n, H), 1.0) for _ in range(2)]
    dys = [randn(gen, (n, H), 1.0) for _ in range(2)]
    return dict(n=n, H=H, F=F, E=E, K=K, n_ad=n_ad, r=r, logits=logits, ids=ids, Wg=Wg, Wu=Wu,
                Wd=Wd, packs=packs, a_offs=a_offs, xs=xs, dys=dys)


def logprob_inputs(n_seq=64, seq=256, H=4096, V=151936, seed=4, groups=16):
    """Fused lm_head logprob workload: n_seq sequences of seq tokens in groups of
    n_seq / groups completions; hidden states N(0, 1), lm_head N(0, 0.02),
    uniform targets, prompt mask on the first 40% of each sequence, advantages
    = group-normalised Bernoulli(0.3) rewards on the completion tokens.
    Returns a dict: hs (two sets), U, targets, act, adv, gen (for the sampler
    noise, drawn after the first logprobs)."""
    torch = _torch()
    gen = torch.Generator(device="cuda").manual_seed(seed)
    n = n_seq * seq
    hs = [randn(gen, (n, H), 1.0) for _ in range(2)]
    U = randn(gen, (V, H), 0.02)
    tg = torch.randint(0, V, (n,), generator=gen, device="cuda", dtype=torch.int32)
    prompt = int(0.4 * seq)
    act = torch.zeros(n_seq, seq, device="cuda")
    act[:, prompt:] = 1
    act = act.reshape(-1).contiguous()
    rew = (torch.rand(n_seq, generator=gen, device="cuda") < 0.3).float().reshape(groups, -1)
    adv = (rew - rew.mean(dim=1, keepdim=True)).reshape(n_seq, 1).expand(n_seq, seq).reshape(-1)
    adv = (adv * act).contiguous()
    return dict(n=n, H=H, V=V, seq=seq, prompt=prompt, hs=hs, U=U, targets=tg, act=act, adv=adv,
                gen=gen)
