"""Two GPU parity cases that follow the data through more than one call.

* The tiny check end to end: the oracle runs from the inputs alone through
  layer forward -> lm_head logprobs -> cross-entropy -> logprob backward ->
  layer backward -> AdamW, and the GPU chain (each call fed the previous GPU
  call's outputs) is compared with it at every stage at the bf16 tolerance
  (the chain carries bf16 activations).  Sorted segments as drawn, and the same
  tokens with shuffled adapter ids (a rollout-shaped batch; OpenTinker,
  "3 Approach").  The AdamW step runs at t = 3 from seeded moments, a
  mid-training state, so that the update is a smooth function of the gradient
  (at t = 1 from zero moments it is about -lr sign(g), which no tolerance on g
  can bound where g is near zero).
* The decode-shaped forward (rollout batches are small per adapter; OpenTinker,
  "3 Approach"): 256 tokens, one per sequence, over 64 adapters with ranks from
  {8, 16, 32, 64}, interleaved ids, a 4096 x 4096 projection -- every row's y
  and u against the oracle, and every row bitwise equal to the same token in a
  4096-row batch that runs the tiled GEMM (batch invariance across the two
  GEMM kernels at the full width).
"""
import numpy as np
import pytest

import oracle.adam as OA
import oracle.logprob as OP
import oracle.lora as OL
import oracle.loss as OLs
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_util import TOL_BF16, TOL_F32, DevLayer, bits_of, dev_bf16, dev_f32, dev_i32, f64_of, rel_err  # noqa: E402
import rl_lora_linear_amd.lib as L  # noqa: E402


@pytest.mark.parametrize("ids_kind", ["sorted", "shuffled"])
def test_tiny_chain_end_to_end(ids_kind):
    c = W.tiny_chain(1)
    lay = c.layer
    targets, weights = c.targets, c.weights
    if ids_kind == "shuffled":
        perm = np.random.default_rng(3).permutation(lay.n_tokens)
        lay.ids = lay.ids[perm].copy()
    dl = DevLayer(lay, order=L.IDS_SORTED if ids_kind == "sorted" else L.IDS_INTERLEAVED)
    n, d, V = lay.n_tokens, lay.d_out, c.U_bits.shape[0]
    x, Wb, A, B, s, ids = dl.oracle_args()
    U64 = c.U()

    # ---- oracle chain, from the inputs alone
    y_o, _ = OL.lora_forward(x, Wb, A, B, s, ids)
    lp_o, lse_o = OP.token_logprobs(y_o, U64, targets)
    L_o, dl_o = OLs.loss_grad(OLs.CROSS_ENTROPY, lp_o, weights)
    dh_o = OP.token_logprobs_backward(y_o, U64, targets, dl_o)
    dx_o, dA_o, dB_o, _ = OL.lora_backward(dh_o, x, Wb, A, B, s, ids)

    # ---- GPU chain
    y, u = dl.forward()
    U = dev_bf16(c.U_bits)
    Ut = torch.empty((d, V), dtype=torch.bfloat16, device="cuda")
    L.lora_transpose_bf16(U, Ut)
    tgt = dev_i32(targets)
    lp = torch.empty(n, device="cuda")
    lse = torch.empty(n, device="cuda")
    ws_lp = L.empty_workspace(L.token_logprobs_workspace_bytes(n, V))
    L.token_logprobs(y, U, tgt, lp, lse, ws_lp)
    loss = torch.empty(1, device="cuda")
    dlp = torch.empty(n, device="cuda")
    ws_l = L.empty_workspace(L.loss_grad_workspace_bytes(n))
    L.loss_grad(L.LOSS_CROSS_ENTROPY, lp, dev_f32(weights), None, None, None, None, loss, dlp, ws_l)
    dh = torch.empty((n, d), dtype=torch.bfloat16, device="cuda")
    ws_b = L.empty_workspace(L.token_logprobs_backward_workspace_bytes(n, V, 256))
    L.token_logprobs_backward(y, U, Ut, tgt, lse, dlp, dh, ws_b)
    dx, grad = dl.backward(u, dy=dh)
    assert dl.status() == 0 and L.lora_device_status(ws_lp) == 0 and L.lora_device_status(ws_l) == 0

    assert rel_err(f64_of(y), y_o) < TOL_BF16
    assert rel_err(f64_of(lp), lp_o) < TOL_BF16
    assert rel_err(f64_of(lse), lse_o) < TOL_BF16
    assert abs(loss.item() - L_o) <= TOL_BF16 * abs(L_o)
    assert np.array_equal(f64_of(dlp), dl_o)          # CE: dl = -w exactly
    assert rel_err(f64_of(dh), dh_o) < TOL_BF16
    assert rel_err(f64_of(dx), dx_o) < TOL_BF16
    dA, dB = dl.split_grad(f64_of(grad))
    for i in range(lay.n_adapters):
        assert rel_err(dA[i], dA_o[i]) < TOL_BF16, ("dA", i)
        assert rel_err(dB[i], dB_o[i]) < TOL_BF16, ("dB", i)

    # ---- AdamW at t = 3 from seeded moments, every adapter in one call
    rng = np.random.default_rng(4)
    g_o = np.zeros(lay.pack_elems)
    for i in range(lay.n_adapters):
        a0, a1 = lay.adapter_range(i)
        r = int(lay.ranks[i])
        g_o[a0:a0 + r * lay.d_in] = dA_o[i].reshape(-1)
        g_o[a0 + r * lay.d_in:a1] = dB_o[i].reshape(-1)
    segs = [(lay.adapter_range(i)[0], lay.adapter_range(i)[1] - lay.adapter_range(i)[0], 3)
            for i in range(lay.n_adapters)]
    p0 = W.bf16_bits_to_f32(lay.pack_bits).astype(np.float32)
    m0 = np.zeros(lay.pack_elems, np.float32)
    v0 = np.zeros(lay.pack_elems, np.float32)
    for o, cnt, _ in segs:               # moments of the right size for each adapter
        rms = np.sqrt(np.mean(g_o[o:o + cnt] ** 2))
        m0[o:o + cnt] = rng.standard_normal(cnt) * 0.5 * rms
        v0[o:o + cnt] = rng.uniform(0.5, 1.5, cnt) * rms * rms
    p, m, v = dev_f32(p0), dev_f32(m0), dev_f32(v0)
    ws_a = L.adam_step_multi(segs, p, grad, m, v, 1e-4, 0.9, 0.999, 1e-8, 0.0)
    assert L.lora_device_status(ws_a) == 0
    p_o, m_o, v_o, skipped = OA.adam_step_multi(segs, p0.astype(np.float64), g_o, m0, v0, 1e-4)
    assert not any(skipped)
    dp, dp_o = p.cpu().numpy().astype(np.float64) - p0, p_o - p0
    for o, cnt, _ in segs:
        sl = slice(o, o + cnt)
        # the stored fp32 parameter resolves the step only to one ulp of p
        ulp = np.spacing(np.abs(p_o[sl]).astype(np.float32)).astype(np.float64)
        scale = np.maximum(np.abs(dp_o[sl]), np.sqrt(np.mean(dp_o[sl] ** 2)))
        assert np.all(np.abs(dp[sl] - dp_o[sl]) <= TOL_BF16 * scale + ulp)
        assert rel_err(m.cpu().numpy()[sl], m_o[sl]) < TOL_BF16
        assert rel_err(v.cpu().numpy()[sl], v_o[sl]) < TOL_BF16


def _decode_case(n_tokens, seed=7, n_ad=64, d=4096):
    rng = np.random.default_rng(seed)
    ranks = rng.choice(np.array([8, 16, 32, 64]), size=n_ad).astype(np.int32)
    ids = rng.integers(0, n_ad, size=n_tokens).astype(np.int32)
    return W.lora_layer(seed, n_tokens, d, d, ranks, [32.0] * n_ad, ids=ids,
                        order="interleaved", with_dy=False)


def test_decode_shape_every_row():
    """256 tokens over 64 adapters (ranks 8-64), interleaved, 4096 -> 4096: every
    row's y (bf16 tolerance) and u (fp32 tolerance) against the oracle."""
    c = _decode_case(256)
    assert len(set(c.ids.tolist())) > 40
    dl = DevLayer(c, max_rank=64)
    y, u = dl.forward()
    assert dl.status() == 0
    x, Wb, A, B, s, ids = dl.oracle_args()
    y_ref, u_ref = OL.lora_forward(x, Wb, A, B, s, ids)
    assert rel_err(f64_of(y), y_ref) < TOL_BF16
    ug = dl.u_values(u)
    assert rel_err(ug[:, :u_ref.shape[1]], u_ref) < TOL_F32
    # per row too: no row may hide behind the batch's rms
    yg = f64_of(y)
    for t in range(c.n_tokens):
        assert rel_err(yg[t], y_ref[t]) < TOL_BF16, t


def test_decode_rows_bitwise_equal_in_a_tiled_batch():
    """The decode batch (few-row GEMM) and a 4096-row batch whose first 256 rows
    are the same tokens with the same adapter ids (tiled GEMM): those rows' y
    and saved u planes carry the same bits."""
    big = _decode_case(4096, seed=8)
    small = _decode_case(256, seed=8)
    small.x_bits = big.x_bits[:256].copy()
    small.ids = big.ids[:256].copy()
    small.W_bits, small.pack_bits = big.W_bits, big.pack_bits
    small.ranks, small.a_off, small.b_off = big.ranks, big.a_off, big.b_off
    y_b, u_b = DevLayer(big, max_rank=64).forward()
    y_s, u_s = DevLayer(small, max_rank=64).forward()
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(y_s), bits_of(y_b)[:256])
    assert np.array_equal(bits_of(u_s), bits_of(u_b)[:, :256])
