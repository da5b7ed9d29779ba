"""The fused SwiGLU MLP layer (mlp_forward / mlp_backward) on the GPU.

It is the expert layer with one expert and no routing, so the oracle is
oracle.moe with every token routed to expert 0 at weight 1, which is the plain
SwiGLU MLP with a LoRA on each projection: compared end to end (y, dx, every
adapter's dA and dB at the bf16 tolerance) and per stage from the GPU's own
stored stage bits, as for the routed layer.  The layer must also equal
moe_forward / moe_backward with one expert, top-1, weight 1: y, dx and the
gate/up gradients bit for bit (the routed combine of one weight-1 expert is a
copy)."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import dev_i32

pytestmark = pytest.mark.gpu
L = pytest.importorskip("rl_lora_linear_amd.lib")

from test_gpu_moe import DevMoe, run_parity  # noqa: E402  (shared device setup and parity)


def _mlp_shape(dm):
    sh = dm.shape
    return L.MlpShape(sh.n_tokens, sh.hidden, sh.d_ff, sh.gate_pack_elems, sh.up_pack_elems,
                      sh.down_pack_elems, sh.n_adapters, sh.max_rank)


def _routing(c):
    ex = torch.zeros((c.n_tokens, 1), dtype=torch.int32, device="cuda")
    w = torch.ones((c.n_tokens, 1), dtype=torch.float32, device="cuda")
    return ex, w


def _mlp_run(dm, ids=None, trace=None, grads=None, accumulate=False):
    c = dm.c
    ids = dm.ids if ids is None else ids
    sh = _mlp_shape(dm)
    ws = L.empty_workspace(L.mlp_workspace_bytes(sh))
    saved = torch.empty(L.mlp_saved_bytes(sh), dtype=torch.uint8, device="cuda")
    y = torch.empty((c.n_tokens, c.hidden), dtype=torch.bfloat16, device="cuda")
    L.mlp_forward(sh, dm.x, ids, dm.Wg, dm.Wu, dm.Wd, dm.packs, dm.descs, y, saved, ws)
    dx = torch.empty_like(y)
    if grads is None:
        grads = [torch.full((p.numel(),), float("nan"), dtype=torch.float32, device="cuda")
                 for p in dm.packs]
    L.mlp_backward(sh, dm.dy, dm.x, ids, dm.Wgt, dm.Wut, dm.Wdt, dm.packs, dm.descs, saved, dx,
                   grads, accumulate, ws, trace=trace)
    return y, dx, grads, saved, ws


# the last two cases: 200 adapters over 2000 tokens, so a 256-row tile holds
# ~25 adapter runs and the fused LoRA expand stages their factor blocks in
# several batches in every launch (gate/up, down, dh, the K-split dX); at rank 32
# the gate/up and K-split launches stage both LoRA sets per round, at rank 64
# one set per round
@pytest.mark.parametrize("n,H,F,n_ad,r,seed", [(600, 256, 320, 5, 32, 41), (777, 192, 256, 3, 48, 42),
                                               (2000, 256, 320, 200, 64, 43),
                                               (2000, 256, 320, 200, 32, 44)])
def test_mlp_layer_parity(n, H, F, n_ad, r, seed):
    c = W.moe_layer(seed=seed, n_tokens=n, hidden=H, d_ff=F, n_experts=1, top_k=1,
                    n_adapters=n_ad, rank=r)
    dm = DevMoe(c)
    trace = dm.new_trace()
    y, dx, grads, saved, ws = _mlp_run(dm, trace=trace)
    assert L.lora_device_status(ws) == 0
    dm.saved = saved
    ex, w = _routing(c)
    run_parity(dm, ex, w, y, dx, grads, trace)


def test_mlp_layer_equals_one_expert_moe_and_invalid_ids():
    c = W.moe_layer(seed=43, n_tokens=500, hidden=256, d_ff=192, n_experts=1, top_k=1,
                    n_adapters=4, rank=16)
    dm = DevMoe(c)
    ids = c.ids.copy()
    ids[[3, 11]] = [-2, c.n_adapters]          # base MLP only for these tokens
    ids_d = dev_i32(ids)
    y, dx, grads, _, ws = _mlp_run(dm, ids=ids_d)
    assert L.lora_device_status(ws) & L.FLAG_ID_RANGE
    ex, w = _routing(c)
    y2 = dm.forward(ex, w, ids=ids_d)
    dx2, grads2 = dm.backward(ex, w, ids=ids_d)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(dx.view(torch.int16), dx2.view(torch.int16))
    # gate and up gradients bit for bit; the routed down dB takes u_down through
    # the weight-scaled planes (re-split after the weight), so it may differ in
    # the last bits of the lo plane
    for a, b in zip(grads[:2], grads2[:2]):
        assert torch.equal(torch.nan_to_num(a, nan=7.0), torch.nan_to_num(b, nan=7.0))
    a, b = grads[2].cpu().numpy(), grads2[2].cpu().numpy()
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-5 * np.abs(b).max())
    # accumulate adds into the packs
    g3 = [g.clone() for g in grads]
    _mlp_run(dm, ids=ids_d, grads=g3, accumulate=True)
    for a, b in zip(g3, grads):
        np.testing.assert_allclose(torch.nan_to_num(a).cpu().numpy(),
                                   2 * torch.nan_to_num(b).cpu().numpy(), rtol=1e-6, atol=0)


def test_empty_batch_moe_and_mlp():
    """No tokens: both layers return at once, and the backward overwrites every
    active pair's gradient region with zeros (accumulate = 0)."""
    c = W.moe_layer(seed=44, n_tokens=64, hidden=128, d_ff=128, n_experts=3, top_k=2,
                    n_adapters=2, rank=16)
    dm = DevMoe(c)
    for routed in (True, False):
        grads = [torch.full((p.numel(),), float("nan"), dtype=torch.float32, device="cuda")
                 for p in dm.packs]
        empty = torch.empty((0, c.hidden), dtype=torch.bfloat16, device="cuda")
        none = torch.empty(0, dtype=torch.int32, device="cuda")
        if routed:
            sh = L.MoeShape(0, c.hidden, c.d_ff, *(p.numel() for p in dm.packs), c.n_experts,
                            c.top_k, c.n_adapters, dm.shape.max_rank)
            ws = L.empty_workspace(L.moe_workspace_bytes(sh))
            saved = torch.empty(L.moe_saved_bytes(sh), dtype=torch.uint8, device="cuda")
            ex = torch.empty((0, c.top_k), dtype=torch.int32, device="cuda")
            w = torch.empty((0, c.top_k), dtype=torch.float32, device="cuda")
            L.moe_forward(sh, empty, ex, w, none, dm.Wg, dm.Wu, dm.Wd, dm.packs, dm.descs, empty,
                          saved, ws)
            L.moe_backward(sh, empty, empty, ex, w, none, dm.Wgt, dm.Wut, dm.Wdt, dm.packs,
                           dm.descs, saved, empty, grads, 0, ws)
        else:
            dm1 = DevMoe(W.moe_layer(seed=45, n_tokens=64, hidden=128, d_ff=128, n_experts=1,
                                     top_k=1, n_adapters=2, rank=16))
            sh = L.MlpShape(0, c.hidden, c.d_ff, *(p.numel() for p in dm1.packs), 2,
                            dm1.shape.max_rank)
            ws = L.empty_workspace(L.mlp_workspace_bytes(sh))
            saved = torch.empty(L.mlp_saved_bytes(sh), dtype=torch.uint8, device="cuda")
            grads = [torch.full((p.numel(),), float("nan"), dtype=torch.float32, device="cuda")
                     for p in dm1.packs]
            L.mlp_forward(sh, empty, none, dm1.Wg, dm1.Wu, dm1.Wd, dm1.packs, dm1.descs, empty,
                          saved, ws)
            L.mlp_backward(sh, empty, empty, none, dm1.Wgt, dm1.Wut, dm1.Wdt, dm1.packs,
                           dm1.descs, saved, empty, grads, 0, ws)
        torch.cuda.synchronize()
        assert L.lora_device_status(ws) == 0
        for g in grads:
            assert not torch.any(g != 0)          # NaN-poisoned before: all overwritten
