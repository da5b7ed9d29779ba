"""GPU parity of the segment builder and the mixed-adapter LoRA layer against
the oracle, through the C ABI.  Sizes span several 256-row/column tiles and a
ragged tail; edge cases: empty input, absent adapters, invalid ids, invalid
descriptors, mixed ranks, sorted and interleaved ids."""
import numpy as np
import pytest

import oracle.lora as OL
import oracle.segments as OS
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_util import TOL_BF16, TOL_F32, DevLayer, bits_of, dev_i32, f64_of, rel_err  # noqa: E402
import rl_lora_linear_amd.lib as L  # noqa: E402


# ---------------------------------------------------------------- segments
@pytest.mark.parametrize("n,n_keys,order,seed", [
    (0, 4, L.IDS_INTERLEAVED, 0), (1, 1, L.IDS_SORTED, 1), (255, 3, L.IDS_INTERLEAVED, 2),
    (257, 16, L.IDS_SORTED, 3), (4097, 64, L.IDS_INTERLEAVED, 4), (3000, 200, L.IDS_INTERLEAVED, 7),
    (16384, 16, L.IDS_SORTED, 8), (20000, 1024, L.IDS_INTERLEAVED, 5),
    (131072, 1024, L.IDS_INTERLEAVED, 6)])
def test_segments_bit_exact(n, n_keys, order, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, n_keys, size=n).astype(np.int32)
    if order == L.IDS_SORTED:
        ids = np.sort(ids)
    perm = torch.full((max(n, 1),), -7, dtype=torch.int32, device="cuda")
    offs = torch.full((n_keys + 1,), -7, dtype=torch.int32, device="cuda")
    ws = L.empty_workspace(L.lora_segments_workspace_bytes(n, n_keys))
    L.lora_segments(dev_i32(ids), n_keys, order, perm, offs, ws)
    assert L.lora_device_status(ws) == 0
    p_ref, o_ref = OS.segments(ids, n_keys)
    assert np.array_equal(offs.cpu().numpy(), o_ref)
    assert np.array_equal(perm.cpu().numpy()[:n], p_ref)


def test_segments_flags_invalid_and_unsorted():
    ids = np.array([0, 1, 5, 1, -1, 2, 2], np.int32)
    ws = L.empty_workspace(L.lora_segments_workspace_bytes(7, 3))
    perm = torch.zeros(7, dtype=torch.int32, device="cuda")
    offs = torch.zeros(4, dtype=torch.int32, device="cuda")
    L.lora_segments(dev_i32(ids), 3, L.IDS_SORTED, perm, offs, ws)
    flags = L.lora_device_status(ws)
    assert flags & L.FLAG_ID_RANGE and flags & L.FLAG_UNSORTED
    p_ref, o_ref = OS.segments(ids, 3)
    assert np.array_equal(offs.cpu().numpy(), o_ref) and np.array_equal(perm.cpu().numpy(), p_ref)
    assert L.lora_device_status(ws) == 0          # read-and-clear


# ---------------------------------------------------------------- layer cases
def _case(kind):
    if kind == "tiny":        # the tiny oracle-check layer: d=256, 4 x r8, 512 sorted tokens
        lay = W.tiny_chain(1).layer
        lay.dy_bits = W.to_bf16_bits(np.random.default_rng(11).standard_normal((lay.n_tokens, lay.d_out)))
        return lay
    if kind == "ragged":      # 5 adapters, mixed ranks, interleaved, ragged everything
        rng = np.random.default_rng(21)
        ids = rng.integers(0, 5, size=700).astype(np.int32)
        ids[ids == 3] = 1                         # adapter 3 owns no token
        return W.lora_layer(21, 700, 320, 192, [8, 16, 24, 40, 64], [16, 32, 8, 40, 64], ids=ids,
                            order="interleaved")
    if kind == "multi":       # several 256-tiles with a ragged tail, sorted uneven segments
        ids = W.sorted_ids_from_lengths([300, 1, 0, 450, 249])
        return W.lora_layer(22, 1000, 512, 768, [32, 8, 16, 64, 32], [32.0] * 5, ids=ids)
    if kind == "big_chunks":  # an adapter with > 1024 tokens (several gradient chunks)
        ids = W.sorted_ids_from_lengths([2500, 700])
        return W.lora_layer(23, 3200, 256, 320, [32, 16], [32.0, 16.0], ids=ids)
    if kind == "many":        # 130 one-token adapters, then three more: a tile half with more
        # distinct adapters than the epilogue's tables hold, and factor blocks over several rounds
        lengths = [1] * 130 + [40, 0, 90]
        ids = W.sorted_ids_from_lengths(lengths)
        ranks = [[64, 8, 32, 64, 16, 48][i % 6] for i in range(len(lengths))]
        return W.lora_layer(24, len(ids), 192, 320, ranks, [float(r) for r in ranks], ids=ids)
    if kind == "tall":        # a batch large enough for 128-row shrink tiles: interleaved ids,
        # mixed ranks, an adapter with no token, segments that end mid-tile
        rng = np.random.default_rng(25)
        ids = rng.integers(0, 8, size=65536).astype(np.int32)
        ids[ids == 5] = 2                         # adapter 5 owns no token
        ranks = [8, 64, 16, 40, 32, 24, 48, 56]
        return W.lora_layer(25, 65536, 128, 192, ranks, [float(r) for r in ranks], ids=ids,
                            order="interleaved")
    if kind == "small_segs":  # 600 adapters of 1-12 tokens: enough chunks that a reduction item
        # takes all of a chunk's column blocks; column counts that end mid-block
        rng = np.random.default_rng(26)
        lengths = rng.integers(1, 13, size=600)
        ids = W.sorted_ids_from_lengths(lengths)
        ranks = [[8, 16, 24, 32, 40, 48, 56, 64][i % 8] for i in range(600)]
        return W.lora_layer(26, len(ids), 320, 448, ranks, [float(r) for r in ranks], ids=ids)
    if kind == "split_k":     # few tokens over many adapters, K over 2 and 3 chunks of 1024
        # with partial last chunks: both shrinks split K over blocks and fold the chunk sums
        rng = np.random.default_rng(27)
        ids = rng.integers(0, 24, size=300).astype(np.int32)
        ids[ids == 7] = 3                         # adapter 7 owns no token
        ranks = [[8, 16, 24, 32, 40, 48, 56, 64][i % 8] for i in range(24)]
        return W.lora_layer(27, 300, 1536, 2560, ranks, [32.0] * 24, ids=ids, order="interleaved")
    if kind == "mixed_chunks":   # many small adapters (finalize blocks check 256 keys each)
        # with one adapter over two gradient chunks and one with no token
        lengths = [1500] + [190] * 19 + [0] + [190] * 19
        ids = W.sorted_ids_from_lengths(lengths)
        ranks = [[16, 32, 8, 64][i % 4] for i in range(len(lengths))]
        return W.lora_layer(28, len(ids), 256, 320, ranks, [32.0] * len(lengths), ids=ids)
    if kind == "huge_keys":   # 5000 adapters of 0-3 tokens: the tile -> adapter lookups
        # search a 5001-entry prefix array (three rounds of the wave search)
        rng = np.random.default_rng(29)
        lengths = rng.integers(0, 4, size=5000)
        ids = W.sorted_ids_from_lengths(lengths)
        ranks = [[8, 16, 32, 64][i % 4] for i in range(5000)]
        return W.lora_layer(29, len(ids), 128, 192, ranks, [16.0] * 5000, ids=ids)
    if kind == "wide":        # 8192 interleaved tokens over 8 adapters at d 2048 -> 2560: the
        # headline tiling (32-row shrink tiles, about one per CU; 256x256 GEMM tiles) with a
        # partial last k chunk in the backward shrink; an adapter with no token
        rng = np.random.default_rng(30)
        ids = rng.integers(0, 8, size=8192).astype(np.int32)
        ids[ids == 6] = 1                         # adapter 6 owns no token
        ranks = [16, 64, 8, 32, 24, 48, 40, 56]
        return W.lora_layer(30, 8192, 2048, 2560, ranks, [float(r) for r in ranks], ids=ids,
                            order="interleaved")
    raise KeyError(kind)


CASES = ["tiny", "ragged", "multi", "big_chunks", "many", "tall", "small_segs", "split_k",
         "mixed_chunks", "huge_keys", "wide"]


@pytest.mark.parametrize("kind", CASES)
def test_forward_parity(kind):
    c = _case(kind)
    dl = DevLayer(c)
    y, u = dl.forward()
    assert dl.status() == 0
    x, Wb, A, B, s, ids = dl.oracle_args()
    y_ref, u_ref = OL.lora_forward(x, Wb, A, B, s, ids)
    assert rel_err(f64_of(y), y_ref) < TOL_BF16
    u_g = dl.u_values(u)
    assert rel_err(u_g[:, :u_ref.shape[1]], u_ref) < TOL_F32
    assert not np.any(u_g[:, u_ref.shape[1]:])


@pytest.mark.parametrize("kind", CASES)
def test_backward_parity(kind):
    c = _case(kind)
    dl = DevLayer(c)
    y, u = dl.forward()
    dx, grad = dl.backward(u)
    assert dl.status() == 0
    x, Wb, A, B, s, ids = dl.oracle_args()
    dx_ref, dA_ref, dB_ref, v_ref = OL.lora_backward(c.dy(), x, Wb, A, B, s, ids)
    assert rel_err(f64_of(dx), dx_ref) < TOL_BF16
    dA, dB = dl.split_grad(f64_of(grad))
    for i in range(c.n_adapters):
        assert rel_err(dA[i], dA_ref[i]) < TOL_F32, (kind, "dA", i)
        assert rel_err(dB[i], dB_ref[i]) < TOL_F32, (kind, "dB", i)


def test_backward_accumulate_and_repeatable():
    c = _case("big_chunks")
    dl = DevLayer(c)
    y, u = dl.forward()
    dx1, g1 = dl.backward(u)
    dx2, g2 = dl.backward(u)
    assert torch.equal(bits_of_t(dx1), bits_of_t(dx2)) and torch.equal(g1, g2)   # bitwise repeatable
    g3 = g1.clone()
    dl.backward(u, accumulate=True, grad=g3)
    np.testing.assert_allclose(g3.cpu().numpy(), 2 * g1.cpu().numpy(), rtol=1e-6, atol=0)


def bits_of_t(t):
    return t.view(torch.int16)


def test_no_leak_bitwise():
    """Changing the values of adapter 0's tokens leaves every other adapter's
    dA, dB bitwise unchanged (OpenTinker: adapter-local gradients)."""
    c = _case("ragged")
    dl = DevLayer(c)
    y, u = dl.forward()
    _, g1 = dl.backward(u)
    rows = np.nonzero(c.ids == 0)[0]
    x2 = c.x_bits.copy()
    x2[rows] = np.random.default_rng(5).integers(0x3000, 0x4000, size=x2[rows].shape).astype(np.uint16)
    dy2 = c.dy_bits.copy()
    dy2[rows] = dy2[rows[::-1]]
    from gpu_util import dev_bf16
    xd, dyd = dev_bf16(x2), dev_bf16(dy2)
    _, u2 = dl.forward(x=xd)
    _, g2 = dl.backward(u2, dy=dyd, x=xd)
    a1, b1 = dl.split_grad(g1.cpu().numpy())
    a2, b2 = dl.split_grad(g2.cpu().numpy())
    for j in range(1, c.n_adapters):
        assert np.array_equal(a1[j], a2[j]) and np.array_equal(b1[j], b2[j]), j
    assert not np.array_equal(a1[0], a2[0])


def test_B_zero_is_base_output_bitwise():
    c = _case("multi")
    dl = DevLayer(c)
    pack = c.pack_bits.copy()
    for i in range(c.n_adapters):
        r = int(c.ranks[i])
        pack[c.b_off[i]:c.b_off[i] + c.d_out * r] = 0
    from gpu_util import dev_bf16
    y0, u0 = dl.forward(pack=dev_bf16(pack))
    # base-only output: every token routed to an id outside [0, n_adapters)
    bad = dev_i32(np.full(c.n_tokens, c.n_adapters, np.int32))
    yb, ub = dl.forward(ids=bad)
    assert dl.status() & L.FLAG_ID_RANGE
    a, b = bits_of(y0), bits_of(yb)
    zeros = ((a & 0x7FFF) == 0) & ((b & 0x7FFF) == 0)     # signed zero aside
    assert np.all((a == b) | zeros)
    assert not torch.any(ub != 0)
    _, g = dl.backward(u0, pack=dev_bf16(pack))
    dA, dB = dl.split_grad(g.cpu().numpy())
    assert all(not a.any() for a in dA)


@pytest.mark.parametrize("kind", ["ragged", "split_k"])
def test_invalid_ids_and_descriptors(kind):
    # split_k: the same with both shrinks splitting K (inactive adapters own no tile)
    c = _case(kind)
    ids = c.ids.copy()
    ids[[3, 10, c.n_tokens - 1]] = [-5, c.n_adapters, 1 << 20]
    dl = DevLayer(c)
    # adapter 2 gets an invalid descriptor (rank 12: not a multiple of 8)
    bad_desc = L.make_desc(c.a_off, c.b_off, np.where(np.arange(c.n_adapters) == 2, 12, c.ranks),
                           dl.scales32)
    dl.desc = bad_desc
    y, u = dl.forward(ids=dev_i32(ids))
    flags = dl.status()
    assert flags & L.FLAG_ID_RANGE and flags & L.FLAG_BAD_DESC
    x, Wb, A, B, s, _ = dl.oracle_args()
    eff = ids.copy()
    eff[eff == 2] = -1                      # adapter 2 inactive
    y_ref, u_ref = OL.lora_forward(x, Wb, A, B, s, eff)
    assert rel_err(f64_of(y), y_ref) < TOL_BF16
    assert rel_err(dl.u_values(u, ids)[:, :u_ref.shape[1]], u_ref) < TOL_F32
    dx, g = dl.backward(u, ids=dev_i32(ids))
    dx_ref, dA_ref, dB_ref, _ = OL.lora_backward(c.dy(), x, Wb, A, B, s, eff)
    assert rel_err(f64_of(dx), dx_ref) < TOL_BF16
    dA, dB = dl.split_grad(f64_of(g))
    for i in range(c.n_adapters):
        if i != 2:
            assert rel_err(dA[i], dA_ref[i]) < TOL_F32 and rel_err(dB[i], dB_ref[i]) < TOL_F32


def test_empty_batch():
    c = W.lora_layer(30, 0, 64, 128, [8, 16], [8.0, 16.0])
    dl = DevLayer(c)
    y, u = dl.forward()
    dx, g = dl.backward(u)
    assert dl.status() == 0
    # no token: every adapter's gradient region is overwritten with zeros
    assert not torch.any(g != 0)


def test_host_validation_errors():
    c = _case("tiny")
    dl = DevLayer(c)
    bad = L.make_shape(c.n_tokens, 100, c.d_out, c.pack_elems, c.pack_elems, c.n_adapters, 16)
    with pytest.raises(L.LoraError) as e:
        L.lora_forward(bad, dl.x, dl.W, dl.pack, dl.pack, dl.desc, dl.ids,
                       torch.empty(1, device="cuda"), torch.empty(1, device="cuda"), dl.ws)
    assert e.value.status == L.LORA_E_UNSUPPORTED
    small = L.empty_workspace(1024)
    y = torch.empty((c.n_tokens, c.d_out), dtype=torch.bfloat16, device="cuda")
    u = torch.empty((2, c.n_tokens, 16), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(L.LoraError) as e:
        L.lora_forward(dl.shape, dl.x, dl.W, dl.pack, dl.pack, dl.desc, dl.ids, y, u, small)
    assert e.value.status == L.LORA_E_WORKSPACE
