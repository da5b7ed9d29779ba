"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and
the benchmark.

This module draws random inputs and packs them; it holds none of the hot path's
arithmetic.  Every tensor is drawn with numpy's PCG64 generator from a fixed
seed, rounded once to bf16 (round-to-nearest-even) where the kernels take bf16,
and handed to both sides as the same bits.  Shapes follow the workloads the
pages describe: Qwen3-8B/4B-width projections with rank-32 adapters over
1024-token completions (tinker-ticks, "Step time" and "How the SGMV kernel
works"), groups of 4-16 completions (Deep Dive - Tinker, "RL: preserve
tokens, logprobs, and credit"), a 151,936-entry lm_head (the Qwen3 vocabulary)
and Qwen3-30B-A3B-style experts.

Layout conventions (PyTorch Linear): W [d_out, d_in]; adapter i has
A_i [r_i, d_in] and B_i [d_out, r_i]; the adapter pack stores, per adapter,
A_i row-major followed immediately by B_i row-major, so one adapter's
parameters (and gradients, and Adam moments) form one contiguous range.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from .bf16 import bf16_bits_to_f32, bf16_bits_to_f64, round_bf16, to_bf16_bits, to_bf16_bits_f32
from .datum import center

__all__ = [
    "LoraLayerCase", "LogprobCase", "MoeCase", "lora_layer", "tiny_chain",
    "attn_proj", "mlp_block", "logprob_rl", "moe_layer", "bf16_bits_to_f64",
    "bf16_bits_to_f32", "round_bf16", "to_bf16_bits", "to_bf16_bits_f32",
]


def _normal_bits(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    """N(0, std^2) in float32, rounded once to bf16; returns uint16 bits."""
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return to_bf16_bits_f32(a).reshape(shape)


def _uniform_bits(rng: np.random.Generator, shape, bound: float) -> np.ndarray:
    a = rng.uniform(-bound, bound, size=shape).astype(np.float32)
    return to_bf16_bits_f32(a).reshape(shape)


@dataclass
class LoraLayerCase:
    """One LoRA-adapted linear layer over a mixed-adapter token batch."""
    n_tokens: int
    d_in: int
    d_out: int
    ranks: np.ndarray          # int32 [n_adapters]
    alphas: np.ndarray         # float64 [n_adapters]
    ids: np.ndarray            # int32 [n_tokens]
    x_bits: np.ndarray         # uint16 [N, d_in]
    W_bits: np.ndarray         # uint16 [d_out, d_in]
    pack_bits: np.ndarray      # uint16 [P]: per adapter A_i then B_i
    a_off: np.ndarray          # int64 [n_adapters]
    b_off: np.ndarray          # int64 [n_adapters]
    dy_bits: Optional[np.ndarray] = None   # uint16 [N, d_out]
    order: str = "sorted"

    @property
    def n_adapters(self) -> int:
        return int(self.ranks.size)

    @property
    def scales(self) -> np.ndarray:
        return self.alphas / self.ranks.astype(np.float64)

    @property
    def max_rank(self) -> int:
        return int(self.ranks.max())

    @property
    def pack_elems(self) -> int:
        return int(self.pack_bits.size)

    def A(self, i: int) -> np.ndarray:
        r = int(self.ranks[i])
        o = int(self.a_off[i])
        return bf16_bits_to_f64(self.pack_bits[o:o + r * self.d_in]).reshape(r, self.d_in)

    def B(self, i: int) -> np.ndarray:
        r = int(self.ranks[i])
        o = int(self.b_off[i])
        return bf16_bits_to_f64(self.pack_bits[o:o + self.d_out * r]).reshape(self.d_out, r)

    def x(self) -> np.ndarray:
        return bf16_bits_to_f64(self.x_bits)

    def W(self) -> np.ndarray:
        return bf16_bits_to_f64(self.W_bits)

    def dy(self) -> np.ndarray:
        return bf16_bits_to_f64(self.dy_bits)

    def adapter_range(self, i: int):
        """[start, end) of adapter i's parameters in the pack."""
        r = int(self.ranks[i])
        return int(self.a_off[i]), int(self.a_off[i]) + r * (self.d_in + self.d_out)


def _pack_offsets(ranks, d_in, d_out):
    a_off = np.zeros(len(ranks), np.int64)
    b_off = np.zeros(len(ranks), np.int64)
    o = 0
    for i, r in enumerate(ranks):
        a_off[i] = o
        b_off[i] = o + int(r) * d_in
        o += int(r) * (d_in + d_out)
    return a_off, b_off, o


def sorted_ids_from_lengths(lengths) -> np.ndarray:
    return np.repeat(np.arange(len(lengths), dtype=np.int32), np.asarray(lengths, np.int64))


def lora_layer(seed: int, n_tokens: int, d_in: int, d_out: int, ranks, alphas,
               ids: Optional[np.ndarray] = None, order: str = "sorted",
               w_std: float = 0.02, b_std: float = 0.01, x_std: float = 1.0,
               with_dy: bool = True, rng: Optional[np.random.Generator] = None) -> LoraLayerCase:
    """Draw one layer: W~N(0,w_std), A_i~U(+-1/sqrt(d_in)), B_i~N(0,b_std),
    x~N(0,x_std), upstream dY~N(0,1).

    `ids` defaults to equal sorted segments; with order="interleaved" and no
    ids, ids are iid uniform over the adapters.  Draw order: ids, W, adapters
    (A_i then B_i, i ascending), x, dY.
    """
    rng = rng if rng is not None else np.random.default_rng(seed)
    ranks = np.asarray(ranks, dtype=np.int32)
    alphas = np.asarray(alphas, dtype=np.float64)
    n_ad = ranks.size
    if ids is None:
        if order == "sorted":
            base = n_tokens // n_ad
            lengths = [base + (1 if i < n_tokens % n_ad else 0) for i in range(n_ad)]
            ids = sorted_ids_from_lengths(lengths)
        else:
            ids = rng.integers(0, n_ad, size=n_tokens).astype(np.int32)
    ids = np.asarray(ids, dtype=np.int32)
    W_bits = _normal_bits(rng, (d_out, d_in), w_std)
    a_off, b_off, total = _pack_offsets(ranks, d_in, d_out)
    pack = np.empty(total, np.uint16)
    bound = 1.0 / np.sqrt(d_in)
    for i, r in enumerate(ranks):
        r = int(r)
        pack[a_off[i]:a_off[i] + r * d_in] = _uniform_bits(rng, (r * d_in,), bound)
        pack[b_off[i]:b_off[i] + d_out * r] = _normal_bits(rng, (d_out * r,), b_std)
    x_bits = _normal_bits(rng, (n_tokens, d_in), x_std)
    dy_bits = _normal_bits(rng, (n_tokens, d_out), 1.0) if with_dy else None
    return LoraLayerCase(n_tokens, d_in, d_out, ranks, alphas, ids, x_bits, W_bits,
                         pack, a_off, b_off, dy_bits, order)


# --------------------------------------------------------------------------
# Tiny end-to-end case: one layer, lm_head, cross-entropy.
# --------------------------------------------------------------------------
@dataclass
class TinyChain:
    layer: LoraLayerCase
    U_bits: np.ndarray       # uint16 [V, d]
    targets: np.ndarray      # int32 [N]
    weights: np.ndarray      # float32 [N]: 0 on the prompt half of each segment, 1 after
    seg_lengths: np.ndarray  # int64 [n_adapters]

    def U(self):
        return bf16_bits_to_f64(self.U_bits)


def tiny_chain(seed: int = 1, d: int = 256, n_tokens: int = 512, n_adapters: int = 4,
               rank: int = 8, alpha: float = 16.0, vocab: int = 1024) -> TinyChain:
    """Tiny fp32 oracle check: d_in=d_out=d, 4 rank-8 adapters (alpha 16) over
    contiguous segments of seeded random lengths, lm_head V=1024, the first half
    (floor) of each segment masked as prompt, cross-entropy weights 1 after."""
    rng = np.random.default_rng(seed)
    cuts = np.sort(rng.choice(np.arange(1, n_tokens), size=n_adapters - 1, replace=False))
    bounds = np.concatenate([[0], cuts, [n_tokens]])
    lengths = np.diff(bounds).astype(np.int64)
    ids = sorted_ids_from_lengths(lengths)
    layer = lora_layer(seed, n_tokens, d, d, [rank] * n_adapters, [alpha] * n_adapters,
                       ids=ids, with_dy=False, rng=rng)
    U_bits = _normal_bits(rng, (vocab, d), 0.02)
    targets = rng.integers(0, vocab, size=n_tokens).astype(np.int32)
    weights = np.zeros(n_tokens, np.float32)
    for i in range(n_adapters):
        s, L = int(bounds[i]), int(lengths[i])
        weights[s + L // 2:s + L] = 1.0
    return TinyChain(layer, U_bits, targets, weights, lengths)


def attn_proj(seed: int = 2, n_tokens: int = 8192, d: int = 4096, n_adapters: int = 16,
              rank: int = 32, alpha: float = 32.0) -> LoraLayerCase:
    """Qwen3-8B-width q/o projection: d->d, 16 rank-32 adapters (alpha 32) in
    sorted equal segments (8192 tokens = 16 x 512)."""
    return lora_layer(seed, n_tokens, d, d, [rank] * n_adapters, [alpha] * n_adapters,
                      order="sorted")


@dataclass
class MlpCase:
    gate: LoraLayerCase
    up: LoraLayerCase
    down: LoraLayerCase


def mlp_block(seed: int = 3, n_tokens: int = 32768, d: int = 4096, d_ff: int = 12288,
              n_adapters: int = 64, rank_choices=(8, 16, 32, 64), alpha: float = 32.0) -> MlpCase:
    """Qwen3-8B-width MLP: gate/up d->d_ff and down d_ff->d, 64 adapters with
    ranks drawn from {8,16,32,64}, per-token ids iid uniform (interleaved).
    The three projections share ids, ranks and the token batch; each has its
    own base weight and adapter factors.  dY is drawn for the down output."""
    rng = np.random.default_rng(seed)
    ranks = rng.choice(np.asarray(rank_choices), size=n_adapters).astype(np.int32)
    alphas = np.full(n_adapters, alpha)
    ids = rng.integers(0, n_adapters, size=n_tokens).astype(np.int32)
    gate = lora_layer(seed, n_tokens, d, d_ff, ranks, alphas, ids=ids, order="interleaved",
                      with_dy=False, rng=rng)
    up = lora_layer(seed, n_tokens, d, d_ff, ranks, alphas, ids=ids, order="interleaved",
                    with_dy=False, rng=rng)
    up.x_bits = gate.x_bits          # the MLP input is shared
    down = lora_layer(seed, n_tokens, d_ff, d, ranks, alphas, ids=ids, order="interleaved",
                      with_dy=True, rng=rng)
    return MlpCase(gate, up, down)


# --------------------------------------------------------------------------
# Fused target logprob + RL loss.
# --------------------------------------------------------------------------
@dataclass
class LogprobCase:
    hidden: int
    vocab: int
    h_bits: np.ndarray        # uint16 [N, H]
    U_bits: np.ndarray        # uint16 [V, H]
    targets: np.ndarray       # int32 [N]
    action: np.ndarray        # float32 [N]: 0 prompt, 1 action
    rewards: np.ndarray       # float64 [n_seq]
    advantages: np.ndarray    # float32 [N]: group-centred reward on action tokens, 0 on prompt
    noise: np.ndarray         # float32 [N]: N(0, sigma) on action tokens, 0 on prompt
    custom_g: np.ndarray      # float32 [N]: N(0,1) on action tokens, 0 on prompt
    seq_len: int
    group_size: int
    n_groups: int

    @property
    def n_tokens(self):
        return int(self.targets.size)

    def sampler_logprobs(self, model_logprobs: np.ndarray) -> np.ndarray:
        """Sampler logprobs = model logprobs + noise on action tokens, 0 on the
        prompt (observation positions carry zero logprob)."""
        lp = np.asarray(model_logprobs, np.float32)
        return np.where(self.action > 0, lp + self.noise, np.float32(0.0)).astype(np.float32)


def logprob_rl(seed: int = 4, hidden: int = 4096, vocab: int = 151936, n_groups: int = 16,
               group_size: int = 4, seq_len: int = 256, prompt_frac: float = 0.4,
               reward_p: float = 0.3, sampler_sigma: float = 0.05,
               h_std: float = 1.0, u_std: float = 0.02) -> LogprobCase:
    """16 groups x 4 completions x 256 tokens; prompt = first floor(0.4*256)
    positions; targets uniform; rewards Bernoulli(0.3) per completion,
    advantages centred within each group; sampler noise N(0, 0.05)."""
    rng = np.random.default_rng(seed)
    n_seq = n_groups * group_size
    N = n_seq * seq_len
    n_prompt = int(np.floor(prompt_frac * seq_len))
    h_bits = _normal_bits(rng, (N, hidden), h_std)
    U_bits = _normal_bits(rng, (vocab, hidden), u_std)
    targets = rng.integers(0, vocab, size=N).astype(np.int32)
    rewards = (rng.random(n_seq) < reward_p).astype(np.float64)
    action = np.zeros(N, np.float32)
    adv = np.zeros(N, np.float32)
    for g in range(n_groups):
        a_grp = center(rewards[g * group_size:(g + 1) * group_size])
        for j in range(group_size):
            s = (g * group_size + j) * seq_len
            action[s + n_prompt:s + seq_len] = 1.0
            adv[s + n_prompt:s + seq_len] = np.float32(a_grp[j])
    noise = (rng.standard_normal(N) * sampler_sigma).astype(np.float32) * action
    g = rng.standard_normal(N).astype(np.float32) * action
    return LogprobCase(hidden, vocab, h_bits, U_bits, targets, action, rewards, adv, noise,
                       g, seq_len, group_size, n_groups)


# --------------------------------------------------------------------------
# Mixture-of-experts layer with per-(expert, adapter) LoRA.
# --------------------------------------------------------------------------
@dataclass
class MoeCase:
    n_tokens: int
    hidden: int
    d_ff: int
    n_experts: int
    top_k: int
    n_adapters: int
    rank: int
    alpha: float
    router_logits: np.ndarray   # float32 [N, E]
    ids: np.ndarray             # int32 [N] adapter id per token
    x_bits: np.ndarray          # uint16 [N, H]
    dy_bits: np.ndarray         # uint16 [N, H]
    Wg_bits: np.ndarray         # uint16 [E, d_ff, H]
    Wu_bits: np.ndarray         # uint16 [E, d_ff, H]
    Wd_bits: np.ndarray         # uint16 [E, H, d_ff]
    # adapter packs, per projection: [adapter][expert] A then B, contiguous per adapter
    pack_g: np.ndarray
    pack_u: np.ndarray
    pack_d: np.ndarray

    def adapter_elems(self, proj: str) -> int:
        """Parameters of one adapter over all experts for one projection."""
        r, H, F = self.rank, self.hidden, self.d_ff
        return self.n_experts * r * (H + F)

    def offsets(self, proj: str, a: int, e: int):
        """(a_off, b_off) of adapter a, expert e in that projection's pack.
        gate/up: A [r, H], B [F, r]; down: A [r, F], B [H, r]."""
        r, H, F = self.rank, self.hidden, self.d_ff
        d_in, d_out = (F, H) if proj == "down" else (H, F)
        per = r * (d_in + d_out)
        base = a * self.n_experts * per + e * per
        return base, base + r * d_in


def moe_layer(seed: int = 5, n_tokens: int = 16384, hidden: int = 2048, d_ff: int = 768,
              n_experts: int = 128, top_k: int = 8, n_adapters: int = 8, rank: int = 32,
              alpha: float = 32.0) -> MoeCase:
    """Qwen3-30B-A3B-style layer: 128 experts, top-8, hidden 2048, expert
    intermediate 768; router logits N(0,1) fp32; 8 rank-32 adapters on every
    expert's gate/up/down; adapter ids iid uniform per token."""
    rng = np.random.default_rng(seed)
    R = rng.standard_normal((n_tokens, n_experts), dtype=np.float32)
    ids = rng.integers(0, n_adapters, size=n_tokens).astype(np.int32)
    Wg = _normal_bits(rng, (n_experts, d_ff, hidden), 0.02)
    Wu = _normal_bits(rng, (n_experts, d_ff, hidden), 0.02)
    Wd = _normal_bits(rng, (n_experts, hidden, d_ff), 0.02)

    def pack(d_in, d_out):
        per = rank * (d_in + d_out)
        p = np.empty(n_adapters * n_experts * per, np.uint16)
        for a in range(n_adapters):
            for e in range(n_experts):
                base = (a * n_experts + e) * per
                p[base:base + rank * d_in] = _uniform_bits(rng, (rank * d_in,), 1.0 / np.sqrt(d_in))
                p[base + rank * d_in:base + per] = _normal_bits(rng, (d_out * rank,), 0.01)
        return p
    pg = pack(hidden, d_ff)
    pu = pack(hidden, d_ff)
    pd = pack(d_ff, hidden)
    x = _normal_bits(rng, (n_tokens, hidden), 1.0)
    dy = _normal_bits(rng, (n_tokens, hidden), 1.0)
    return MoeCase(n_tokens, hidden, d_ff, n_experts, top_k, n_adapters, rank, alpha, R, ids,
                   x, dy, Wg, Wu, Wd, pg, pu, pd)
