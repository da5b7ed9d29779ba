"""Helpers shared by the GPU parity tests: upload seeded cases, run the C-ABI
calls through the binding, and the parity metric.

Parity metric: max_e |gpu_e - ora_e| / max(|ora_e|, rms(ora)), compared with
2e-2 for bf16 outputs and 1e-4 for fp32 outputs.
"""
from __future__ import annotations

import numpy as np
import torch

import workloads as W

TOL_BF16 = 2e-2
TOL_F32 = 1e-4


def rel_err(gpu, ora) -> float:
    g = np.asarray(gpu, np.float64).reshape(-1)
    o = np.asarray(ora, np.float64).reshape(-1)
    if o.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(o * o)))
    den = np.maximum(np.abs(o), rms)
    den[den == 0] = 1.0
    return float(np.max(np.abs(g - o) / den))


def l2_rel(gpu, ora) -> float:
    """||gpu - ora||_2 / ||ora||_2 (0 for an all-zero reference matched exactly)."""
    g = np.asarray(gpu, np.float64).reshape(-1)
    o = np.asarray(ora, np.float64).reshape(-1)
    n = float(np.linalg.norm(o))
    d = float(np.linalg.norm(g - o))
    return d / n if n > 0 else d


def check_chained(gpu, ora, what="", terms=None):
    """An fp32 result that the fused layers derive from bf16 stage tensors,
    against the plain float64 definition: the norm-wise relative error within
    the bf16 tolerance, and no element beyond 2.5x that tolerance (the
    elementwise metric's maximum over ~10^6 elements of a sum of bf16 rounding
    errors reaches ~4.5 standard deviations).  terms: the number of rows each
    element sums (a routed pair's assignments); under 16 the elementwise bar
    is not applied -- a gradient element summed over a few rows carries its
    largest product's stage rounding (a few bf16 ulps of silu' or of the
    scaled vector) without averaging, which can exceed 2.5x the tolerance of
    the matrix's rms, and the per-call checks at the fp32 tolerance cover those
    pairs exactly."""
    m, l2 = rel_err(gpu, ora), l2_rel(gpu, ora)
    print(f"[chained] {what}: max {m:.3g} l2 {l2:.3g}" + (f" ({terms} rows)" if terms else ""),
          flush=True)
    assert l2 < TOL_BF16, (what, m, l2)
    if terms is None or terms >= 16:
        assert m < 2.5 * TOL_BF16, (what, m, l2)


def dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64_of(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return W.bf16_bits_to_f64(bits_of(t))
    return t.detach().cpu().numpy().astype(np.float64)


def dev_f32(a, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def dev_i32(a, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


class DevLayer:
    """A LoraLayerCase resident on the GPU, with its workspace."""

    def __init__(self, case: "W.LoraLayerCase", order: int = None, max_rank: int = None):
        import rl_lora_linear_amd.lib as L
        self.L = L
        self.case = case
        if order is None:
            order = L.IDS_SORTED if case.order == "sorted" else L.IDS_INTERLEAVED
        self.max_rank = max_rank or max(16, int(np.ceil(case.max_rank / 16) * 16))
        self.shape = L.make_shape(case.n_tokens, case.d_in, case.d_out, case.pack_elems,
                                  case.pack_elems, case.n_adapters, self.max_rank, order)
        self.scales32 = case.scales.astype(np.float32)
        self.x = dev_bf16(case.x_bits)
        self.W = dev_bf16(case.W_bits)
        self.Wt = torch.empty((case.d_in, case.d_out), dtype=torch.bfloat16, device="cuda")
        L.lora_transpose_bf16(self.W, self.Wt)
        self.pack = dev_bf16(case.pack_bits)
        self.desc = L.make_desc(case.a_off, case.b_off, case.ranks, self.scales32)
        self.ids = dev_i32(case.ids)
        self.ws = L.empty_workspace(L.lora_workspace_bytes(self.shape))
        self.dy = dev_bf16(case.dy_bits) if case.dy_bits is not None else None

    def forward(self, x=None, pack=None, ids=None):
        N, d_out = self.case.n_tokens, self.case.d_out
        y = torch.empty((N, d_out), dtype=torch.bfloat16, device="cuda")
        # saved vector: bf16 hi/lo planes of s_a u_t, poisoned with NaN first
        u = torch.full((2, N, self.max_rank), float("nan"), dtype=torch.bfloat16, device="cuda")
        p = self.pack if pack is None else pack
        self.L.lora_forward(self.shape, self.x if x is None else x, self.W, p, p, self.desc,
                            self.ids if ids is None else ids, y, u, self.ws)
        return y, u

    def backward(self, u, dy=None, x=None, pack=None, ids=None, accumulate=False, grad=None):
        N = self.case.n_tokens
        dx = torch.empty((N, self.case.d_in), dtype=torch.bfloat16, device="cuda")
        if grad is None:
            grad = torch.full((self.case.pack_elems,), float("nan"), dtype=torch.float32, device="cuda")
        p = self.pack if pack is None else pack
        self.L.lora_backward(self.shape, self.dy if dy is None else dy, self.x if x is None else x,
                             self.Wt, p, p, self.desc, self.ids if ids is None else ids, u, dx,
                             grad, grad, accumulate, self.ws)
        return dx, grad

    def u_values(self, u, ids=None) -> np.ndarray:
        """u_t = A_a x_t (float64, [N][max_rank]) from the saved hi/lo planes of
        s_a u_t; tokens without a valid adapter keep the stored value (zero)."""
        planes = f64_of(u)
        su = planes[0] + planes[1]
        ids = self.case.ids if ids is None else np.asarray(ids)
        ok = (ids >= 0) & (ids < self.case.n_adapters)
        s = np.ones(len(ids))
        s[ok] = self.scales32[ids[ok]].astype(np.float64)
        return su / s[:, None]

    def status(self) -> int:
        return self.L.lora_device_status(self.ws)

    # oracle-side views (float64)
    def oracle_args(self):
        c = self.case
        A = [c.A(i) for i in range(c.n_adapters)]
        B = [c.B(i) for i in range(c.n_adapters)]
        return c.x(), c.W(), A, B, self.scales32.astype(np.float64), c.ids

    def split_grad(self, grad: np.ndarray):
        """Per-adapter (dA, dB) views of a flat gradient pack."""
        c = self.case
        dA, dB = [], []
        for i in range(c.n_adapters):
            r = int(c.ranks[i])
            a, b = int(c.a_off[i]), int(c.b_off[i])
            dA.append(grad[a:a + r * c.d_in].reshape(r, c.d_in))
            dB.append(grad[b:b + c.d_out * r].reshape(c.d_out, r))
        return dA, dB
