"""lora_forward_noalloc (the forward on the library's fixed scratch array, for
callers that cannot allocate) against lora_forward through the C ABI: two
calls in a row, the second with a smaller input, each bit for bit equal to
lora_forward on the same inputs; the content flags reach the caller's status
word; a shape beyond the array is refused before anything runs."""
import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_util import DevLayer, bits_of, dev_i32  # noqa: E402
import rl_lora_linear_amd.lib as L  # noqa: E402


def _decode_case():
    # rollout-shaped: 256 tokens over 64 adapters with ranks 8-64, interleaved
    rng = np.random.default_rng(51)
    ranks = rng.choice(np.array([8, 16, 32, 64]), size=64).astype(np.int32)
    ids = rng.integers(0, 64, size=256).astype(np.int32)
    return W.lora_layer(51, 256, 1024, 512, ranks, [32.0] * 64, ids=ids, order="interleaved",
                        with_dy=False)


def _small_case():
    ids = W.sorted_ids_from_lengths([40, 0, 57, 3])
    return W.lora_layer(52, len(ids), 192, 320, [16, 8, 64, 32], [16.0, 8.0, 32.0, 32.0], ids=ids,
                        with_dy=False)


def _both(dl, ids=None):
    """(y, u) from lora_forward and from lora_forward_noalloc, and the flags of each."""
    y_ref, u_ref = dl.forward(ids=ids)
    flags_ref = dl.status()
    N, d_out = dl.case.n_tokens, dl.case.d_out
    y = torch.full((N, d_out), float("nan"), dtype=torch.bfloat16, device="cuda")
    u = torch.full((2, N, dl.max_rank), float("nan"), dtype=torch.bfloat16, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    L.lora_forward_noalloc(dl.shape, dl.x, dl.W, dl.pack, dl.pack, dl.desc,
                           dl.ids if ids is None else ids, y, u, status=st)
    torch.cuda.synchronize()
    return (y_ref, u_ref, flags_ref), (y, u, int(st.item()))


def test_noalloc_forward_equals_forward_twice_then_smaller():
    assert L.lora_forward_noalloc_scratch_bytes() == 2 << 20
    for case in (_decode_case(), _small_case()):          # the second call is smaller
        dl = DevLayer(case, max_rank=64)
        (y_ref, u_ref, f_ref), (y, u, f) = _both(dl)
        assert f_ref == 0 and f == 0
        assert np.array_equal(bits_of(y), bits_of(y_ref))
        assert np.array_equal(bits_of(u), bits_of(u_ref))


def test_noalloc_forward_flags_and_limits():
    case = _small_case()
    dl = DevLayer(case, max_rank=64)
    ids = case.ids.copy()
    ids[[0, 50]] = [-3, 99]                                # out of range: base output, flagged
    (y_ref, u_ref, f_ref), (y, u, f) = _both(dl, ids=dev_i32(ids))
    assert f_ref & L.FLAG_ID_RANGE and f == f_ref
    assert np.array_equal(bits_of(y), bits_of(y_ref))
    assert np.array_equal(bits_of(u), bits_of(u_ref))
    # the next call starts from a clear status word in the scratch array
    (_, _, _), (_, _, f2) = _both(dl)
    assert f2 == 0
    # a shape whose scratch exceeds the array is refused on the host
    big = L.make_shape(1 << 20, 64, 64, 1 << 20, 1 << 20, 1024, 16, L.IDS_INTERLEAVED)
    t = torch.empty(64, dtype=torch.bfloat16, device="cuda")
    i = torch.empty(64, dtype=torch.int32, device="cuda")
    with pytest.raises(L.LoraError) as e:
        L.lora_forward_noalloc(big, t, t, t, t, dl.desc, i, t, t)
    assert e.value.status == L.LORA_E_UNSUPPORTED
