"""Dense SwiGLU MLP with a LoRA on each projection (oracle; test infrastructure
only).

The MLP projections are where LoRA must attach for RL to match full
fine-tuning (TPU RL note, section 4 "The Tunix backend"; Deep Dive - Tinker,
"LoRA is the adaptation boundary"), and tinker-ticks ("How the SGMV kernel
works") counts gate/up/down among the seven adapted projections per layer.
Reading: the glue between the projections is SwiGLU, h = silu(gate x) * up x,
out = down h, silu(z) = z * sigmoid(z); each projection is the mixed-adapter
layer of oracle.lora with the same per-token adapter ids.
"""
from __future__ import annotations

import numpy as np

from .lora import lora_backward, lora_forward


def silu(z):
    return z / (1.0 + np.exp(-z))


def dsilu(z):
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def swiglu_forward(g, u):
    return silu(np.asarray(g, np.float64)) * np.asarray(u, np.float64)


def swiglu_backward(dh, g, u):
    """Return (dg, du) for h = silu(g) * u."""
    dh = np.asarray(dh, np.float64)
    g = np.asarray(g, np.float64)
    u = np.asarray(u, np.float64)
    return dh * u * dsilu(g), dh * silu(g)


def mlp_forward(x, gate, up, down, ids):
    """gate/up/down are (W, A list, B list, scales) tuples."""
    g, ug = lora_forward(x, gate[0], gate[1], gate[2], gate[3], ids)
    u, uu = lora_forward(x, up[0], up[1], up[2], up[3], ids)
    h = swiglu_forward(g, u)
    y, ud = lora_forward(h, down[0], down[1], down[2], down[3], ids)
    return y, {"g": g, "u": u, "h": h}


def mlp_backward(dy, x, gate, up, down, ids, saved):
    """Return dx and per-projection (dA, dB) lists."""
    dh, dAd, dBd, _ = lora_backward(dy, saved["h"], down[0], down[1], down[2], down[3], ids)
    dg, du = swiglu_backward(dh, saved["g"], saved["u"])
    dxg, dAg, dBg, _ = lora_backward(dg, x, gate[0], gate[1], gate[2], gate[3], ids)
    dxu, dAu, dBu, _ = lora_backward(du, x, up[0], up[1], up[2], up[3], ids)
    return dxg + dxu, {"gate": (dAg, dBg), "up": (dAu, dBu), "down": (dAd, dBd)}
