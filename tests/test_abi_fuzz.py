"""Property checks of the C ABI's host side (CPU only, no GPU touched).

Random shapes, including negative, zero and very large sizes, go through every
size query and every layer entry point with no workspace:

* a size query either rejects the shape (0) or returns a size that is
  deterministic, at least the bytes of the per-token tables it must hold, and
  far from wrapping around;
* an entry point given no workspace returns an error status and enqueues
  nothing, whatever the shape (it must fail on the host before any launch).

test_host_asan.py runs this file again with the host code under
AddressSanitizer, so an out-of-bounds host access on any of these paths fails.
"""
import ctypes

import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

SET = settings(max_examples=250, deadline=None, derandomize=True,
               suppress_health_check=[HealthCheck.too_slow])

I64 = st.one_of(st.integers(-5, 70000), st.sampled_from([0, 1, 63, 64, 65, 4096, 1 << 20, 1 << 30,
                                                         (1 << 31) - 1, 1 << 40, -(1 << 40)]))
I32 = st.one_of(st.integers(-3, 20000), st.sampled_from([0, 1, 8, 15, 16, 32, 48, 64, 65, 1 << 30,
                                                         -(1 << 30)]))
DIM = st.one_of(st.sampled_from([0, 1, 63, 64, 128, 4096, 12288, 1 << 20, (1 << 20) + 64]),
                st.integers(-64, 5000))
P = ctypes.c_void_p(64)   # never dereferenced: every call below fails validation first
HUGE = 1 << 62


@pytest.fixture(scope="module")
def L():
    from test_abi_host import _ensure_built
    _ensure_built()
    import rl_lora_linear_amd.lib as lib
    return lib


def _sane(size, floor):
    assert size == 0 or floor <= size < HUGE, (size, floor)


@SET
@given(n=I64, d_in=DIM, d_out=DIM, a=I64, b=I64, n_ad=I32, r=I32, order=st.integers(-1, 2),
       reserved=st.sampled_from([0, 0, 0, 1]))
def test_layer_size_and_validation(L, n, d_in, d_out, a, b, n_ad, r, order, reserved):
    lib = L.LIB
    sh = L.LoraShape(n, d_in, d_out, a, b, n_ad, r, order, reserved)
    size = lib.lora_workspace_bytes(ctypes.byref(sh))
    assert size == lib.lora_workspace_bytes(ctypes.byref(sh))
    _sane(size, 8 * max(n, 0))
    if size and (reserved or not 0 <= order <= 1 or n < 0 or r % 16 or not 16 <= r <= 64):
        pytest.fail(f"accepted an invalid shape {n, d_in, d_out, n_ad, r, order, reserved}")
    st_f = lib.lora_forward(ctypes.byref(sh), P, P, P, P, P, P, P, P, None, 0, None)
    st_b = lib.lora_backward(ctypes.byref(sh), P, P, P, P, P, P, P, P, P, P, P, 0, None, 0, None)
    assert st_f != L.LORA_OK and st_b != L.LORA_OK


@SET
@given(n=I64, k=I32, v=I64, rows=I64, nseg=I32)
def test_other_size_queries(L, n, k, v, rows, nseg):
    lib = L.LIB
    _sane(lib.lora_segments_workspace_bytes(n, k), 4)   # status word (perm, offsets: caller)
    _sane(lib.token_logprobs_workspace_bytes(n, v), 0)
    _sane(lib.token_logprobs_backward_workspace_bytes(n, v, rows), 0)
    _sane(lib.loss_grad_workspace_bytes(n), 0)
    _sane(lib.adam_workspace_bytes(nseg), 4 * max(nseg, 0))
    assert lib.lora_segments(P, n, k, 0, P, P, None, 0, None) != L.LORA_OK
    assert lib.token_logprobs(n, 4096, v, P, P, P, P, P, None, 0, None) != L.LORA_OK
    assert lib.loss_grad(0, n, P, P, None, None, None, None, P, P, None, 0, None) != L.LORA_OK


@SET
@given(n=I64, h=DIM, f=DIM, g=I64, u=I64, dn=I64, e=I32, k=I32, n_ad=I32, r=I32)
def test_expert_layer_size_and_validation(L, n, h, f, g, u, dn, e, k, n_ad, r):
    lib = L.LIB
    moe = L.MoeShape(n, h, f, g, u, dn, e, k, n_ad, r)
    mlp = L.MlpShape(n, h, f, g, u, dn, n_ad, r)
    for q in (lib.moe_workspace_bytes, lib.moe_saved_bytes):
        size = q(ctypes.byref(moe))
        assert size == q(ctypes.byref(moe))
        _sane(size, 0)
    for q in (lib.mlp_workspace_bytes, lib.mlp_saved_bytes):
        size = q(ctypes.byref(mlp))
        assert size == q(ctypes.byref(mlp))
        _sane(size, 0)
    assert lib.moe_forward(ctypes.byref(moe), P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, None,
                           0, None) != L.LORA_OK
    assert lib.mlp_forward(ctypes.byref(mlp), P, P, P, P, P, P, P, P, P, P, P, P, P, None, 0,
                           None) != L.LORA_OK


def test_size_queries_match_entry_point_ranges(L):
    lib = L.LIB
    assert lib.token_logprobs_workspace_bytes(10, 100) == 0          # vocab not a multiple of 64
    assert lib.token_logprobs_workspace_bytes(1 << 30, 128) == 0     # n beyond 2^30 - 1
    assert lib.loss_grad_workspace_bytes(1 << 30) == 0
    assert lib.loss_grad_workspace_bytes((1 << 30) - 1) > 0
    # A chunk never runs longer than n rounded up to 256 rows, so asking for more sizes the same.
    one = lib.token_logprobs_backward_workspace_bytes(100, 128, 256)
    assert one >= 256 * 128 * 2
    assert lib.token_logprobs_backward_workspace_bytes(100, 128, 1 << 20) == one
    assert lib.token_logprobs_backward_workspace_bytes(1000, 128, 300) == \
        lib.token_logprobs_backward_workspace_bytes(1000, 128, 512)
