"""CPU-only checks of the C-ABI library: it loads, exports every function
include/lora_mi355x.h declares, and rejects bad host-side arguments before
enqueuing anything (no GPU is touched: every call here fails validation)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lora_mi355x.h")


def _ensure_built():
    from rl_lora_linear_amd import build as B
    srcs = [os.path.join(B.CSRC, f) for f in os.listdir(B.CSRC)] + [HEADER]
    if not os.path.exists(B.LIB) or os.path.getmtime(B.LIB) < max(os.path.getmtime(s) for s in srcs):
        B.build()


@pytest.fixture(scope="module")
def L():
    _ensure_built()
    import rl_lora_linear_amd.lib as lib
    return lib


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\**\s+\**([a-z_][\w]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if not n.startswith("LORA")))


def test_header_parsed():
    names = _declared_functions()
    assert "lora_forward" in names and "adam_step" in names and len(names) >= 20


def test_library_exports_every_declared_symbol(L):
    cdll = ctypes.CDLL(L.LIB_PATH)
    missing = [n for n in _declared_functions() if not hasattr(cdll, n)]
    assert missing == []
    assert sorted(L.EXPORTS) == _declared_functions()


def test_host_validation_returns_before_any_launch(L):
    lib = L.LIB
    sh = L.make_shape(512, 256, 256, 4096, 4096, 4, 16)
    assert L.lora_workspace_bytes(sh) > 0
    P = ctypes.c_void_p(16)     # never dereferenced: validation fails first
    st = lib.lora_forward(ctypes.byref(sh), P, None, P, P, P, P, P, P, P, 1 << 30, None)
    assert st == L.LORA_E_INVALID_ARG and b"non-NULL" in lib.lora_last_error()
    bad = L.make_shape(512, 100, 256, 4096, 4096, 4, 16)
    st = lib.lora_forward(ctypes.byref(bad), P, P, P, P, P, P, P, P, P, 1 << 30, None)
    assert st == L.LORA_E_UNSUPPORTED
    for r_bad in (8, 12, 24, 80):       # max_rank must be a multiple of 16 in [16, 64]
        bad = L.make_shape(512, 256, 256, 4096, 4096, 4, r_bad)
        assert lib.lora_workspace_bytes(ctypes.byref(bad)) == 0
    st = lib.lora_forward(ctypes.byref(sh), P, P, P, P, P, P, P, P, P, 64, None)
    assert st == L.LORA_E_WORKSPACE
    st = lib.lora_backward(ctypes.byref(sh), P, P, P, P, P, P, P, P, P, P, P, 0, P, 64, None)
    assert st == L.LORA_E_WORKSPACE
    assert lib.token_logprobs(10, 100, 1024, P, P, P, P, P, P, 1 << 30, None) == L.LORA_E_UNSUPPORTED
    assert lib.token_logprobs(10, 128, 1024, P, P, P, P, P, P, 16, None) == L.LORA_E_WORKSPACE
    assert lib.loss_grad(9, 10, P, P, P, P, P, None, P, P, P, 1 << 20, None) == L.LORA_E_INVALID_ARG
    assert lib.loss_grad(L.LOSS_PPO, 10, P, P, P, P, P, None, P, P, P, 1 << 20, None) == L.LORA_E_INVALID_ARG
    assert lib.adam_step(10, P, P, P, P, 0, 1e-3, 0.9, 0.999, 1e-8, 0.0, None, P, 1 << 12, None) == L.LORA_E_INVALID_ARG
    assert lib.adam_step(10, P, P, P, P, 1, 1e-3, 0.9, 0.999, 1e-8, 0.0, None, P, 16, None) == L.LORA_E_WORKSPACE
    assert lib.adam_step(10, P, P, P, P, 1, 1e-3, 0.9, 0.999, 1e-8, 0.0, None, None, 1 << 12, None) == L.LORA_E_WORKSPACE
    assert lib.adam_workspace_bytes(70) >= 256 + 4 * 70 and lib.adam_workspace_bytes(-1) == 0
    assert lib.lora_segments(P, 10, 0, 0, P, P, P, 1 << 20, None) == L.LORA_E_INVALID_ARG
    assert lib.lora_transpose_bf16(P, ctypes.c_void_p(32), 100, 64, None) == L.LORA_E_UNSUPPORTED
    assert lib.lora_timing_read(99, None, None) == L.LORA_E_INVALID_ARG


def test_workspace_sizes_monotone(L):
    small = L.lora_workspace_bytes(L.make_shape(512, 256, 256, 4096, 4096, 4, 16))
    big = L.lora_workspace_bytes(L.make_shape(8192, 4096, 4096, 16 * 32 * 8192, 16 * 32 * 8192, 16, 32))
    assert 0 < small < big
    assert L.lora_segments_workspace_bytes(0, 4) > 0 and L.lora_segments_workspace_bytes(-1, 4) == 0
    assert L.token_logprobs_backward_workspace_bytes(100, 1024, 255) == 0
    assert L.token_logprobs_backward_workspace_bytes(100, 1024, 256) >= 256 * 1024 * 2


def test_expert_layer_size_queries_and_validation(L):
    lib = L.LIB
    mlp = L.MlpShape(256, 512, 1024, 1 << 16, 1 << 16, 1 << 16, 4, 16)
    moe1 = L.MoeShape(256, 512, 1024, 1 << 16, 1 << 16, 1 << 16, 1, 1, 4, 16)
    # The MLP layer is the one-expert layer without routing: same saved activations, no
    # routed-copy buffers in its workspace.
    assert L.mlp_saved_bytes(mlp) == L.moe_saved_bytes(moe1) > 0
    assert 0 < L.mlp_workspace_bytes(mlp) <= L.moe_workspace_bytes(moe1)
    bigger = L.MlpShape(1024, 512, 1024, 1 << 16, 1 << 16, 1 << 16, 4, 16)
    assert L.mlp_saved_bytes(bigger) > L.mlp_saved_bytes(mlp)
    for bad in (L.MlpShape(256, 500, 1024, 1, 1, 1, 4, 16),     # hidden not a multiple of 64
                L.MlpShape(256, 512, 1024, 1, 1, 1, 4, 24),      # rank not a multiple of 16
                L.MlpShape(-1, 512, 1024, 1, 1, 1, 4, 16),       # negative token count
                L.MlpShape(256, 512, 1024, -1, 1, 1, 4, 16)):    # negative pack size
        assert lib.mlp_workspace_bytes(ctypes.byref(bad)) == 0
        assert lib.mlp_saved_bytes(ctypes.byref(bad)) == 0
    for bad in (L.MoeShape(256, 512, 1024, 1, 1, 1, 8, 9, 4, 16),    # top_k > n_experts
                L.MoeShape(256, 512, 1024, 1, 1, 1, 2048, 2, 4, 16)):  # too many experts
        assert lib.moe_workspace_bytes(ctypes.byref(bad)) == 0
    P = ctypes.c_void_p(16)     # never dereferenced: validation fails first
    st = lib.moe_forward(ctypes.byref(moe1), P, None, None, P, P, P, P, P, P, P, P, P, P, P, P, P,
                         1 << 30, None)
    assert st == L.LORA_E_INVALID_ARG and b"experts and weights" in lib.lora_last_error()
    st = lib.mlp_forward(ctypes.byref(mlp), P, P, P, P, P, P, P, P, P, P, P, P, P, P, 64, None)
    assert st == L.LORA_E_WORKSPACE
    st = lib.mlp_backward(ctypes.byref(mlp), P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P,
                          0, None, P, 64, None)
    assert st == L.LORA_E_WORKSPACE
