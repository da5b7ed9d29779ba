"""The layer calls replayed from a captured HIP graph give the eager results,
bit for bit, on every replay.

Every entry point of a training step's forward and backward launches only
kernels (no allocation, no memset node, no host synchronisation) with launch
shapes fixed by the call's sizes, so a caller may capture a step once and
replay it.  Each case runs the calls eagerly for the reference, captures them
into a graph, and replays it three times with other eager work and
synchronisations between the replays, comparing every output after every
replay with the eager bits:
  * the dense mixed-adapter layer, forward + backward (interleaved ids, mixed
    ranks, a ragged row tile);
  * a decode-shaped forward (the few-row GEMM and the K-split shrink with its
    fold launch);
  * the routed-expert layer: routing, forward and backward.
"""
import numpy as np
import pytest
import torch

import workloads as W
import workloads.device as WD
from gpu_util import DevLayer, bits_of

pytestmark = pytest.mark.gpu
L = pytest.importorskip("rl_lora_linear_amd.lib")


def _snap(ts):
    return [bits_of(t) if t.dtype == torch.bfloat16 else t.detach().cpu().numpy().copy() for t in ts]


def _same(a, b, what):
    for i, (x, y) in enumerate(zip(a, b)):
        assert x.shape == y.shape and np.array_equal(x.view(np.uint8), y.view(np.uint8)), (what, i)


def _replay_check(run, outs, other):
    """run(): the calls; outs: their output tensors; other(): unrelated eager
    work run between replays."""
    torch.cuda.synchronize()
    run()
    torch.cuda.synchronize()
    ref = _snap(outs)
    for t in outs:
        t.fill_(float("nan") if t.is_floating_point() else -1)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        print(f"[graph] replay {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        _same(_snap(outs), ref, f"replay {rep}")
        for t in outs:
            t.fill_(float("nan") if t.is_floating_point() else -1)
        other()
        torch.cuda.synchronize()


def test_dense_layer_step_graph():
    ranks = [8, 16, 32, 64, 24]
    ids = np.random.default_rng(41).integers(-1, 6, size=3000).astype(np.int32)
    c = W.lora_layer(41, len(ids), 512, 768, ranks, [float(r) for r in ranks], ids=ids,
                     order="interleaved")
    dl = DevLayer(c)
    N = c.n_tokens
    y = torch.empty((N, c.d_out), dtype=torch.bfloat16, device="cuda")
    u = torch.empty((2, N, dl.max_rank), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty((N, c.d_in), dtype=torch.bfloat16, device="cuda")
    grad = torch.empty(c.pack_elems, dtype=torch.float32, device="cuda")

    def run():
        L.lora_forward(dl.shape, dl.x, dl.W, dl.pack, dl.pack, dl.desc, dl.ids, y, u, dl.ws)
        L.lora_backward(dl.shape, dl.dy, dl.x, dl.Wt, dl.pack, dl.pack, dl.desc, dl.ids, u, dx,
                        grad, grad, 0, dl.ws)

    other_c = W.lora_layer(42, 700, 256, 320, [16, 32], [16.0, 32.0])
    other = DevLayer(other_c)
    _replay_check(run, [y, u, dx, grad], lambda: other.forward())
    assert dl.status() == L.FLAG_ID_RANGE   # the ids -1 and 5 (no adapter)


def test_decode_forward_graph():
    ranks = [8, 16, 32, 64] * 4
    ids = np.tile(np.arange(16, dtype=np.int32), 16)
    c = W.lora_layer(43, len(ids), 2048, 1024, ranks, [32.0] * 16, ids=ids, order="interleaved")
    dl = DevLayer(c)
    y = torch.empty((c.n_tokens, c.d_out), dtype=torch.bfloat16, device="cuda")
    u = torch.empty((2, c.n_tokens, dl.max_rank), dtype=torch.bfloat16, device="cuda")

    def run():
        L.lora_forward(dl.shape, dl.x, dl.W, dl.pack, dl.pack, dl.desc, dl.ids, y, u, dl.ws)

    scratch = torch.empty(1 << 20, device="cuda")
    _replay_check(run, [y, u], lambda: scratch.normal_())
    assert dl.status() == 0


def test_routed_layer_step_graph():
    n, H, F, E, K, n_ad, r = 1500, 256, 192, 16, 4, 3, 16
    inp = WD.moe_inputs(n, H, F, E, K, n_ad, r, seed=44)
    Wgt, Wut = (torch.empty((E, H, F), dtype=torch.bfloat16, device="cuda") for _ in range(2))
    Wdt = torch.empty((E, F, H), dtype=torch.bfloat16, device="cuda")
    for e in range(E):
        L.lora_transpose_bf16(inp["Wg"][e], Wgt[e])
        L.lora_transpose_bf16(inp["Wu"][e], Wut[e])
        L.lora_transpose_bf16(inp["Wd"][e], Wdt[e])
    packs = inp["packs"]
    descs = [L.make_desc(a_off, a_off + r * di, np.full(a_off.size, r, np.int32),
                         np.full(a_off.size, 2.0, np.float32))
             for a_off, di in zip(inp["a_offs"], (H, H, F))]
    shape = L.MoeShape(n, H, F, packs[0].numel(), packs[1].numel(), packs[2].numel(), E, K, n_ad, r)
    ws = L.empty_workspace(L.moe_workspace_bytes(shape))
    saved = torch.empty(L.moe_saved_bytes(shape), dtype=torch.uint8, device="cuda")
    ex = torch.empty((n, K), dtype=torch.int32, device="cuda")
    w = torch.empty((n, K), device="cuda")
    y = torch.empty((n, H), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty_like(y)
    grads = [torch.empty(p.numel(), dtype=torch.float32, device="cuda") for p in packs]

    def run():
        L.moe_route(inp["logits"], K, ex, w)
        L.moe_forward(shape, inp["xs"][0], ex, w, inp["ids"], inp["Wg"], inp["Wu"], inp["Wd"],
                      packs, descs, y, saved, ws)
        L.moe_backward(shape, inp["dys"][0], inp["xs"][0], ex, w, inp["ids"], Wgt, Wut, Wdt, packs,
                       descs, saved, dx, grads, 0, ws)

    scratch = torch.empty(1 << 20, device="cuda")
    _replay_check(run, [ex, w, y, dx, *grads], lambda: scratch.normal_())
    assert L.lora_device_status(ws) == 0
