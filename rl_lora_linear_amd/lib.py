"""ctypes binding of liblora_mi355x.so (include/lora_mi355x.h).

Argument marshalling only: every function below forwards torch tensors'
device pointers, sizes and the current HIP stream to the C entry point of the
same name and raises LoraError on a non-zero status.  All computation runs in
the library's gfx950 kernels; there is no fallback path.  If the library is
missing the import of this module raises, loudly.  LORA_MI355X_LIB, when set,
names another build of the same library to load instead (the host-sanitizer
build of `python -m rl_lora_linear_amd.build --host-asan`).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("LORA_MI355X_LIB") or os.path.join(_HERE, "liblora_mi355x.so")

# status codes and flags (include/lora_mi355x.h)
LORA_OK, LORA_E_INVALID_ARG, LORA_E_UNSUPPORTED, LORA_E_WORKSPACE, LORA_E_HIP, LORA_E_DEVICE_CHECK = range(6)
FLAG_ID_RANGE, FLAG_UNSORTED, FLAG_TARGET_RANGE, FLAG_BAD_DESC = 0x1, 0x2, 0x4, 0x8
FLAG_NONFINITE_GRAD, FLAG_NONFINITE_LOSS = 0x10, 0x20
IDS_SORTED, IDS_INTERLEAVED = 0, 1
LOSS_CROSS_ENTROPY, LOSS_IMPORTANCE_SAMPLING, LOSS_PPO, LOSS_CUSTOM = range(4)
TIMER_BASE_GEMM, TIMER_LOGPROB_FWD, TIMER_LOGPROB_BWD, TIMER_SHRINK, TIMER_EXPAND, TIMER_GRAD, TIMER_ADAM = range(7)

EXPORTS = [
    "lora_workspace_bytes", "lora_workspace_init", "lora_device_status", "lora_last_error",
    "lora_segments_workspace_bytes", "lora_segments", "lora_transpose_bf16", "lora_forward",
    "lora_backward", "token_logprobs_workspace_bytes", "token_logprobs",
    "token_logprobs_backward_workspace_bytes", "token_logprobs_backward",
    "loss_grad_workspace_bytes", "loss_grad", "adam_workspace_bytes", "adam_step",
    "adam_step_multi", "swiglu_forward",
    "swiglu_backward", "bf16_add", "moe_route", "moe_workspace_bytes", "moe_saved_bytes", "moe_forward",
    "moe_backward", "mlp_workspace_bytes", "mlp_saved_bytes", "mlp_forward", "mlp_backward",
    "lora_timing_enable", "lora_timing_reset", "lora_timing_read",
    "lora_forward_noalloc_scratch_bytes", "lora_forward_noalloc",
    "lora_probe_mfma_flops_per_iter", "lora_probe_mfma", "lora_probe_copy", "lora_probe_read",
]


class LoraError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"status {status}: {msg}")
        self.status = status


class LoraShape(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int64), ("d_in", ctypes.c_int64), ("d_out", ctypes.c_int64),
                ("a_pack_elems", ctypes.c_int64), ("b_pack_elems", ctypes.c_int64),
                ("n_adapters", ctypes.c_int32), ("max_rank", ctypes.c_int32),
                ("order", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class MoeShape(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int64), ("hidden", ctypes.c_int64), ("d_ff", ctypes.c_int64),
                ("gate_pack_elems", ctypes.c_int64), ("up_pack_elems", ctypes.c_int64),
                ("down_pack_elems", ctypes.c_int64), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("n_adapters", ctypes.c_int32),
                ("max_rank", ctypes.c_int32)]


class MlpShape(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int64), ("hidden", ctypes.c_int64), ("d_ff", ctypes.c_int64),
                ("gate_pack_elems", ctypes.c_int64), ("up_pack_elems", ctypes.c_int64),
                ("down_pack_elems", ctypes.c_int64), ("n_adapters", ctypes.c_int32),
                ("max_rank", ctypes.c_int32)]


class AdamSegment(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_int64), ("count", ctypes.c_int64), ("step", ctypes.c_int64)]


class LossConfig(ctypes.Structure):
    _fields_ = [("clip_low", ctypes.c_float), ("clip_high", ctypes.c_float)]


DESC_DTYPE = np.dtype([("a_off", "<i8"), ("b_off", "<i8"), ("rank", "<i4"), ("scale", "<f4")])
assert DESC_DTYPE.itemsize == 24

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_F = ctypes.c_float
_SZ = ctypes.c_size_t


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m rl_lora_linear_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "lora_workspace_bytes": (_SZ, [ctypes.POINTER(LoraShape)]),
        "lora_workspace_init": (_I32, [_P, _SZ, _P]),
        "lora_device_status": (_I32, [_P, ctypes.POINTER(_I32), _P]),
        "lora_last_error": (ctypes.c_char_p, []),
        "lora_segments_workspace_bytes": (_SZ, [_I64, _I32]),
        "lora_segments": (_I32, [_P, _I64, _I32, _I32, _P, _P, _P, _SZ, _P]),
        "lora_transpose_bf16": (_I32, [_P, _P, _I64, _I64, _P]),
        "lora_forward": (_I32, [ctypes.POINTER(LoraShape), _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
        "lora_backward": (_I32, [ctypes.POINTER(LoraShape), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                 _P, _I32, _P, _SZ, _P]),
        "token_logprobs_workspace_bytes": (_SZ, [_I64, _I64]),
        "token_logprobs": (_I32, [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _SZ, _P]),
        "token_logprobs_backward_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
        "token_logprobs_backward": (_I32, [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
        "loss_grad_workspace_bytes": (_SZ, [_I64]),
        "loss_grad": (_I32, [_I32, _I64, _P, _P, _P, _P, _P, ctypes.POINTER(LossConfig), _P, _P, _P,
                             _SZ, _P]),
        "adam_workspace_bytes": (_SZ, [_I32]),
        "adam_step": (_I32, [_I64, _P, _P, _P, _P, _I64, _F, _F, _F, _F, _F, _P, _P, _SZ, _P]),
        "adam_step_multi": (_I32, [_I32, ctypes.POINTER(AdamSegment), _P, _P, _P, _P, _F, _F, _F, _F,
                                   _F, _P, _P, _SZ, _P]),
        "swiglu_forward": (_I32, [_I64, _P, _P, _P, _P]),
        "bf16_add": (_I32, [_I64, _P, _P, _P, _P]),
        "moe_route": (_I32, [_I64, _I32, _I32, _P, _P, _P, _P]),
        "moe_workspace_bytes": (_SZ, [ctypes.POINTER(MoeShape)]),
        "moe_saved_bytes": (_SZ, [ctypes.POINTER(MoeShape)]),
        "moe_forward": (_I32, [ctypes.POINTER(MoeShape)] + [_P] * 16 + [_SZ, _P]),
        "moe_backward": (_I32, [ctypes.POINTER(MoeShape)] + [_P] * 19 + [_I32, _P, _P, _SZ, _P]),
        "mlp_workspace_bytes": (_SZ, [ctypes.POINTER(MlpShape)]),
        "mlp_saved_bytes": (_SZ, [ctypes.POINTER(MlpShape)]),
        "mlp_forward": (_I32, [ctypes.POINTER(MlpShape)] + [_P] * 14 + [_SZ, _P]),
        "mlp_backward": (_I32, [ctypes.POINTER(MlpShape)] + [_P] * 17 + [_I32, _P, _P, _SZ, _P]),
        "swiglu_backward": (_I32, [_I64, _P, _P, _P, _P, _P, _P]),
        "lora_forward_noalloc_scratch_bytes": (_SZ, []),
        "lora_forward_noalloc": (_I32, [ctypes.POINTER(LoraShape), _P, _P, _P, _P, _P, _P, _P, _P,
                                        _P, _P]),
        "lora_probe_mfma_flops_per_iter": (_I64, [_I32]),
        "lora_probe_mfma": (_I32, [_I64, _I32, _P, _P]),
        "lora_probe_copy": (_I32, [_P, _P, _I64, _P]),
        "lora_probe_read": (_I32, [_P, _I64, _P, _P]),
        "lora_timing_enable": (None, [_I32]),
        "lora_timing_reset": (None, []),
        "lora_timing_read": (_I32, [_I32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_I64)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()


def _check(st: int):
    if st != LORA_OK:
        raise LoraError(st, LIB.lora_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


# ------------------------------------------------------------------ helpers
def make_shape(n_tokens, d_in, d_out, a_pack_elems, b_pack_elems, n_adapters, max_rank,
               order=IDS_SORTED) -> LoraShape:
    return LoraShape(n_tokens, d_in, d_out, a_pack_elems, b_pack_elems, n_adapters, max_rank, order, 0)


def make_desc(a_off, b_off, ranks, scales, device="cuda") -> torch.Tensor:
    """Device descriptor table (24-byte records) as a uint8 tensor."""
    d = np.zeros(len(ranks), DESC_DTYPE)
    d["a_off"], d["b_off"], d["rank"], d["scale"] = a_off, b_off, ranks, scales
    return torch.from_numpy(d.view(np.uint8).copy()).to(device)


def empty_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace (its status word starts cleared)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ C entry points
def lora_workspace_bytes(shape: LoraShape) -> int:
    n = LIB.lora_workspace_bytes(ctypes.byref(shape))
    if n == 0:
        raise LoraError(LORA_E_INVALID_ARG, LIB.lora_last_error().decode())
    return n


def lora_workspace_init(ws: torch.Tensor, stream=None):
    _check(LIB.lora_workspace_init(_ptr(ws), _nbytes(ws), _stream(stream)))


def lora_device_status(ws: torch.Tensor, stream=None) -> int:
    """Synchronise, read and clear the workspace status word; returns the flags
    (does not raise on content errors)."""
    flags = _I32(0)
    st = LIB.lora_device_status(_ptr(ws), ctypes.byref(flags), _stream(stream))
    if st not in (LORA_OK, LORA_E_DEVICE_CHECK):
        _check(st)
    return flags.value


def lora_segments_workspace_bytes(n: int, n_keys: int) -> int:
    return LIB.lora_segments_workspace_bytes(n, n_keys)


def lora_segments(ids, n_keys, order, perm, offsets, ws, stream=None):
    _check(LIB.lora_segments(_ptr(ids), ids.numel(), n_keys, order, _ptr(perm), _ptr(offsets),
                             _ptr(ws), _nbytes(ws), _stream(stream)))


def lora_transpose_bf16(src, dst, stream=None):
    rows, cols = src.shape
    _check(LIB.lora_transpose_bf16(_ptr(src), _ptr(dst), rows, cols, _stream(stream)))


def lora_forward(shape, x, W, A_pack, B_pack, desc, ids, y, u_saved, ws, stream=None):
    _check(LIB.lora_forward(ctypes.byref(shape), _ptr(x), _ptr(W), _ptr(A_pack), _ptr(B_pack),
                            _ptr(desc), _ptr(ids), _ptr(y), _ptr(u_saved), _ptr(ws), _nbytes(ws),
                            _stream(stream)))


def lora_forward_noalloc_scratch_bytes() -> int:
    return LIB.lora_forward_noalloc_scratch_bytes()


def lora_forward_noalloc(shape, x, W, A_pack, B_pack, desc, ids, y, u_saved, status=None,
                         stream=None):
    """lora_forward on the library's fixed scratch array (no workspace); status:
    optional device int32 tensor the call's flags are OR-ed into."""
    _check(LIB.lora_forward_noalloc(ctypes.byref(shape), _ptr(x), _ptr(W), _ptr(A_pack),
                                    _ptr(B_pack), _ptr(desc), _ptr(ids), _ptr(y), _ptr(u_saved),
                                    _ptr(status), _stream(stream)))


def lora_backward(shape, dy, x, W_t, A_pack, B_pack, desc, ids, u_saved, dx, dA_pack, dB_pack,
                  accumulate, ws, stream=None):
    _check(LIB.lora_backward(ctypes.byref(shape), _ptr(dy), _ptr(x), _ptr(W_t), _ptr(A_pack),
                             _ptr(B_pack), _ptr(desc), _ptr(ids), _ptr(u_saved), _ptr(dx),
                             _ptr(dA_pack), _ptr(dB_pack), int(accumulate), _ptr(ws), _nbytes(ws),
                             _stream(stream)))


def token_logprobs_workspace_bytes(n, vocab) -> int:
    return LIB.token_logprobs_workspace_bytes(n, vocab)


def token_logprobs(h, lm_head, targets, logprobs, lse, ws, stream=None):
    n, hidden = h.shape
    vocab = lm_head.shape[0]
    _check(LIB.token_logprobs(n, hidden, vocab, _ptr(h), _ptr(lm_head), _ptr(targets),
                              _ptr(logprobs), _ptr(lse), _ptr(ws), _nbytes(ws), _stream(stream)))


def token_logprobs_backward_workspace_bytes(n, vocab, chunk_rows) -> int:
    return LIB.token_logprobs_backward_workspace_bytes(n, vocab, chunk_rows)


def token_logprobs_backward(h, lm_head, lm_head_t, targets, lse, dlogp, dh, ws, stream=None):
    n, hidden = h.shape
    vocab = lm_head.shape[0]
    _check(LIB.token_logprobs_backward(n, hidden, vocab, _ptr(h), _ptr(lm_head), _ptr(lm_head_t),
                                       _ptr(targets), _ptr(lse), _ptr(dlogp), _ptr(dh), _ptr(ws),
                                       _nbytes(ws), _stream(stream)))


def loss_grad_workspace_bytes(n) -> int:
    return LIB.loss_grad_workspace_bytes(n)


def loss_grad(kind, logprobs, weights, advantages, sampler_logprobs, custom_g, clip, loss_out,
              dlogp, ws, stream=None):
    cfg = LossConfig(*clip) if clip is not None else None
    _check(LIB.loss_grad(kind, logprobs.numel(), _ptr(logprobs), _ptr(weights), _ptr(advantages),
                         _ptr(sampler_logprobs), _ptr(custom_g),
                         ctypes.byref(cfg) if cfg is not None else None, _ptr(loss_out), _ptr(dlogp),
                         _ptr(ws), _nbytes(ws), _stream(stream)))


def adam_workspace_bytes(n_seg: int) -> int:
    return LIB.adam_workspace_bytes(n_seg)


def adam_skip_flags(ws: torch.Tensor, n_seg: int) -> np.ndarray:
    """Per-segment skip flags of the latest AdamW call on this workspace
    (int32 at byte 256 + 4 i: 1 = skipped, 0 = stepped); synchronises."""
    torch.cuda.synchronize()
    return ws[256:256 + 4 * n_seg].cpu().numpy().view(np.int32).copy()


def adam_step(p, g, m, v, step, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
              p_bf16=None, ws=None, stream=None):
    """ws: workspace of adam_workspace_bytes(1) (a fresh zeroed one if None).
    A gradient holding NaN or Inf skips the whole step and sets
    FLAG_NONFINITE_GRAD in the workspace status word."""
    if ws is None:
        ws = empty_workspace(adam_workspace_bytes(1), device=p.device)
    _check(LIB.adam_step(p.numel(), _ptr(p), _ptr(g), _ptr(m), _ptr(v), int(step), lr, beta1,
                         beta2, eps, weight_decay, _ptr(p_bf16), _ptr(ws), _nbytes(ws),
                         _stream(stream)))
    return ws


def adam_step_multi(segments, p, g, m, v, lr, beta1=0.9, beta2=0.999, eps=1e-8,
                    weight_decay=0.0, p_bf16=None, ws=None, stream=None):
    """segments: list of (offset, count, step) into the flat p/g/m/v buffers.
    ws: workspace of adam_workspace_bytes(len(segments)) (fresh if None)."""
    n = p.numel()
    for t in (g, m, v):
        if t.numel() != n:
            raise LoraError(LORA_E_INVALID_ARG, "p, g, m, v must have the same length")
    if p_bf16 is not None and p_bf16.numel() != n:
        raise LoraError(LORA_E_INVALID_ARG, "p_bf16 must have the length of p")
    for o, c, _ in segments:
        if o < 0 or c < 0 or o + c > n:
            raise LoraError(LORA_E_INVALID_ARG, f"segment ({o}, {c}) outside a buffer of {n}")
    if ws is None:
        ws = empty_workspace(adam_workspace_bytes(len(segments)), device=p.device)
    arr = (AdamSegment * max(1, len(segments)))(*[AdamSegment(int(o), int(c), int(t)) for o, c, t in segments])
    _check(LIB.adam_step_multi(len(segments), arr, _ptr(p), _ptr(g), _ptr(m), _ptr(v), lr, beta1,
                               beta2, eps, weight_decay, _ptr(p_bf16), _ptr(ws), _nbytes(ws),
                               _stream(stream)))
    return ws


def bf16_add(a, b, out, stream=None):
    _check(LIB.bf16_add(a.numel(), _ptr(a), _ptr(b), _ptr(out), _stream(stream)))


def moe_route(logits, top_k, experts, weights, stream=None):
    n, E = logits.shape
    _check(LIB.moe_route(n, E, top_k, _ptr(logits), _ptr(experts), _ptr(weights), _stream(stream)))


def moe_workspace_bytes(shape: MoeShape) -> int:
    n = LIB.moe_workspace_bytes(ctypes.byref(shape))
    if n == 0:
        raise LoraError(LORA_E_INVALID_ARG, LIB.lora_last_error().decode())
    return n


def moe_saved_bytes(shape: MoeShape) -> int:
    n = LIB.moe_saved_bytes(ctypes.byref(shape))
    if n == 0:
        raise LoraError(LORA_E_INVALID_ARG, LIB.lora_last_error().decode())
    return n


def moe_forward(shape, x, experts, weights, ids, W_gate, W_up, W_down, packs, descs, y, saved, ws,
                stream=None):
    """packs, descs: (gate, up, down) triples."""
    _check(LIB.moe_forward(ctypes.byref(shape), _ptr(x), _ptr(experts), _ptr(weights), _ptr(ids),
                           _ptr(W_gate), _ptr(W_up), _ptr(W_down), *[_ptr(p) for p in packs],
                           *[_ptr(d) for d in descs], _ptr(y), _ptr(saved), _ptr(ws), _nbytes(ws),
                           _stream(stream)))


def moe_backward(shape, dy, x, experts, weights, ids, W_gate_t, W_up_t, W_down_t, packs, descs,
                 saved, dx, grads, accumulate, ws, trace=None, stream=None):
    """packs, descs, grads: (gate, up, down) triples; trace: optional bf16 [3][N*K][F]."""
    _check(LIB.moe_backward(ctypes.byref(shape), _ptr(dy), _ptr(x), _ptr(experts), _ptr(weights),
                            _ptr(ids), _ptr(W_gate_t), _ptr(W_up_t), _ptr(W_down_t),
                            *[_ptr(p) for p in packs], *[_ptr(d) for d in descs], _ptr(saved),
                            _ptr(dx), *[_ptr(g) for g in grads], int(accumulate), _ptr(trace),
                            _ptr(ws), _nbytes(ws), _stream(stream)))


def mlp_workspace_bytes(shape: MlpShape) -> int:
    n = LIB.mlp_workspace_bytes(ctypes.byref(shape))
    if n == 0:
        raise LoraError(LORA_E_INVALID_ARG, LIB.lora_last_error().decode())
    return n


def mlp_saved_bytes(shape: MlpShape) -> int:
    n = LIB.mlp_saved_bytes(ctypes.byref(shape))
    if n == 0:
        raise LoraError(LORA_E_INVALID_ARG, LIB.lora_last_error().decode())
    return n


def mlp_forward(shape, x, ids, W_gate, W_up, W_down, packs, descs, y, saved, ws, stream=None):
    """packs, descs: (gate, up, down) triples."""
    _check(LIB.mlp_forward(ctypes.byref(shape), _ptr(x), _ptr(ids), _ptr(W_gate), _ptr(W_up),
                           _ptr(W_down), *[_ptr(p) for p in packs], *[_ptr(d) for d in descs],
                           _ptr(y), _ptr(saved), _ptr(ws), _nbytes(ws), _stream(stream)))


def mlp_backward(shape, dy, x, ids, W_gate_t, W_up_t, W_down_t, packs, descs, saved, dx, grads,
                 accumulate, ws, trace=None, stream=None):
    """packs, descs, grads: (gate, up, down) triples; trace: optional bf16 [3 * N * F]."""
    _check(LIB.mlp_backward(ctypes.byref(shape), _ptr(dy), _ptr(x), _ptr(ids), _ptr(W_gate_t),
                            _ptr(W_up_t), _ptr(W_down_t), *[_ptr(p) for p in packs],
                            *[_ptr(d) for d in descs], _ptr(saved), _ptr(dx),
                            *[_ptr(g) for g in grads], int(accumulate), _ptr(trace), _ptr(ws),
                            _nbytes(ws), _stream(stream)))


def swiglu_forward(gate, up, h, stream=None):
    _check(LIB.swiglu_forward(gate.numel(), _ptr(gate), _ptr(up), _ptr(h), _stream(stream)))


def swiglu_backward(dh, gate, up, dgate, dup, stream=None):
    _check(LIB.swiglu_backward(gate.numel(), _ptr(dh), _ptr(gate), _ptr(up), _ptr(dgate), _ptr(dup),
                               _stream(stream)))


def lora_probe_mfma(iters, blocks, sink, stream=None):
    """Register-only bf16 MFMA loop; returns its flop count."""
    _check(LIB.lora_probe_mfma(int(iters), int(blocks), _ptr(sink), _stream(stream)))
    return LIB.lora_probe_mfma_flops_per_iter(int(blocks)) * int(iters)


def lora_probe_copy(src, dst, stream=None):
    """Streaming device copy of src's bytes into dst."""
    _check(LIB.lora_probe_copy(_ptr(src), _ptr(dst), _nbytes(src), _stream(stream)))


def lora_probe_read(src, sink, stream=None):
    """Read-only stream over src's bytes (sink: a device int32 tensor)."""
    _check(LIB.lora_probe_read(_ptr(src), _nbytes(src), _ptr(sink), _stream(stream)))


def lora_timing_enable(on: bool):
    LIB.lora_timing_enable(1 if on else 0)


def lora_timing_reset():
    LIB.lora_timing_reset()


def lora_timing_read(timer: int):
    ms = ctypes.c_double(0)
    n = _I64(0)
    _check(LIB.lora_timing_read(timer, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value
