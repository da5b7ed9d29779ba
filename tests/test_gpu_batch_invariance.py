"""Batch invariance: a token's per-row results do not depend on the batch it
is in.  On-policy RL compares the logprobs of a rollout with those of the
training step over the same tokens, so row t must come out bit for bit the
same whether it is computed among few tokens or many (tinker-ticks, "Why RL
needs batch-invariant kernels").

Each test runs a large batch and a prefix of it as a batch of its own and
compares the prefix rows bitwise: the dense layer's y, saved u and dx, with the
large batch past the size at which the shrink switches from 32-row to 128-row
tiles and a prefix small enough for the few-row GEMM; the routed-expert layer's y and dx, likewise past the switch in
(expert, adapter) assignments; the lm_head logprob, logsumexp and dh.
Per-adapter gradient sums are sums over the batch and are not compared."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import DevLayer

pytestmark = pytest.mark.gpu
L = pytest.importorskip("rl_lora_linear_amd.lib")

TALL_ROWS = 128 * 256 // 2   # rows from which the shrink takes 128-row tiles (256 CUs)


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 \
        else t.contiguous().view(torch.int32).cpu().numpy()


def _assert_same_bits(a, b, what):
    da, db = _bits(a), _bits(b)
    bad = np.argwhere(da != db)
    assert bad.size == 0, f"{what}: {len(bad)} elements differ, first at {bad[0].tolist()}"


# the 256-row prefix runs its forward GEMM in the few-row kernel, the batch in
# the 256x256-tile kernel.  With d_in 2048 and d_out 3072 the shrinks sum over
# 2 and 3 k chunks: the batch in 128-row tiles, the 4096-row prefix in 32-row
# tiles, and the 256-row prefix with K split over blocks (chunk sums folded in
# a second launch), forward and backward.
@pytest.mark.parametrize("n_small", [4096, 256])
@pytest.mark.parametrize("d_in,d_out", [(256, 320), (2048, 3072)])
def test_dense_layer_rows_batch_invariant(n_small, d_in, d_out):
    n_big = TALL_ROWS + 4096
    c = W.lora_layer(seed=27, n_tokens=n_big, d_in=d_in, d_out=d_out, ranks=[8, 64, 16, 32, 48],
                     alphas=[16.0, 32.0, 8.0, 64.0, 32.0], order="interleaved")
    dl = DevLayer(c)
    y_b, u_b = dl.forward()
    dx_b, _ = dl.backward(u_b)
    assert dl.status() == 0

    sh = L.make_shape(n_small, c.d_in, c.d_out, c.pack_elems, c.pack_elems, c.n_adapters,
                      dl.max_rank, L.IDS_INTERLEAVED)
    ws = L.empty_workspace(L.lora_workspace_bytes(sh))
    x, ids, dy = dl.x[:n_small].contiguous(), dl.ids[:n_small].contiguous(), dl.dy[:n_small].contiguous()
    y_s = torch.empty((n_small, c.d_out), dtype=torch.bfloat16, device="cuda")
    u_s = torch.full((2, n_small, dl.max_rank), float("nan"), dtype=torch.bfloat16, device="cuda")
    L.lora_forward(sh, x, dl.W, dl.pack, dl.pack, dl.desc, ids, y_s, u_s, ws)
    dx_s = torch.empty((n_small, c.d_in), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((c.pack_elems,), dtype=torch.float32, device="cuda")
    L.lora_backward(sh, dy, x, dl.Wt, dl.pack, dl.pack, dl.desc, ids, u_s, dx_s, g, g, False, ws)
    assert L.lora_device_status(ws) == 0

    _assert_same_bits(y_s, y_b[:n_small], "y")
    _assert_same_bits(u_s, u_b[:, :n_small], "u (both planes)")
    _assert_same_bits(dx_s, dx_b[:n_small], "dx")


def test_moe_layer_rows_batch_invariant():
    from test_gpu_moe import DevMoe
    top_k = 8
    n_big, n_small = TALL_ROWS // top_k + 808, 500   # 8 assignments per token
    c = W.moe_layer(seed=29, n_tokens=n_big, hidden=256, d_ff=192, n_experts=16, top_k=top_k,
                    n_adapters=3, rank=32)
    dm = DevMoe(c)
    ex, w = dm.route()
    y_b = dm.forward(ex, w)
    dx_b, _ = dm.backward(ex, w)
    assert L.lora_device_status(dm.ws) == 0

    s = dm.shape
    sh = L.MoeShape(n_small, s.hidden, s.d_ff, s.gate_pack_elems, s.up_pack_elems,
                    s.down_pack_elems, s.n_experts, s.top_k, s.n_adapters, s.max_rank)
    ws = L.empty_workspace(L.moe_workspace_bytes(sh))
    saved = torch.empty(L.moe_saved_bytes(sh), dtype=torch.uint8, device="cuda")
    x, dy = dm.x[:n_small].contiguous(), dm.dy[:n_small].contiguous()
    ex_s, w_s, ids = ex[:n_small].contiguous(), w[:n_small].contiguous(), dm.ids[:n_small].contiguous()
    y_s = torch.empty((n_small, s.hidden), dtype=torch.bfloat16, device="cuda")
    L.moe_forward(sh, x, ex_s, w_s, ids, dm.Wg, dm.Wu, dm.Wd, dm.packs, dm.descs, y_s, saved, ws)
    dx_s = torch.empty_like(y_s)
    grads = [torch.zeros((p.numel(),), dtype=torch.float32, device="cuda") for p in dm.packs]
    L.moe_backward(sh, dy, x, ex_s, w_s, ids, dm.Wgt, dm.Wut, dm.Wdt, dm.packs, dm.descs, saved,
                   dx_s, grads, False, ws)
    assert L.lora_device_status(ws) == 0

    _assert_same_bits(y_s, y_b[:n_small], "y")
    _assert_same_bits(dx_s, dx_b[:n_small], "dx")


def test_logprob_rows_batch_invariant():
    n_big, n_small, H, V = 1280, 300, 320, 1088
    gen = torch.Generator(device="cuda").manual_seed(31)
    h = torch.randn((n_big, H), generator=gen, device="cuda").bfloat16()
    U = (0.05 * torch.randn((V, H), generator=gen, device="cuda")).bfloat16()
    tgt = torch.randint(0, V, (n_big,), generator=gen, device="cuda", dtype=torch.int32)
    d = torch.randn((n_big,), generator=gen, device="cuda")
    Ut = torch.empty((H, V), dtype=torch.bfloat16, device="cuda")
    L.lora_transpose_bf16(U, Ut)

    def run(n):
        hh, tt, dd = h[:n].contiguous(), tgt[:n].contiguous(), d[:n].contiguous()
        lp = torch.empty(n, dtype=torch.float32, device="cuda")
        lse = torch.empty(n, dtype=torch.float32, device="cuda")
        ws = L.empty_workspace(L.token_logprobs_workspace_bytes(n, V))
        L.token_logprobs(hh, U, tt, lp, lse, ws)
        assert L.lora_device_status(ws) == 0
        dh = torch.empty((n, H), dtype=torch.bfloat16, device="cuda")
        wsb = L.empty_workspace(L.token_logprobs_backward_workspace_bytes(n, V, 256))
        L.token_logprobs_backward(hh, U, Ut, tt, lse, dd, dh, wsb)
        assert L.lora_device_status(wsb) == 0
        return lp, lse, dh

    lp_b, lse_b, dh_b = run(n_big)
    lp_s, lse_s, dh_s = run(n_small)
    _assert_same_bits(lp_s, lp_b[:n_small], "logprob")
    _assert_same_bits(lse_s, lse_b[:n_small], "lse")
    _assert_same_bits(dh_s, dh_b[:n_small], "dh")
