"""The base GEMM runs one block per compute unit, each looping over its XCD's
tiles; these shapes give it more tiles than blocks, unevenly: 257 row tiles
(one XCD gets 33 tiles for its 32 blocks, so one block runs two) and 521 (two
or three tiles per block), with a ragged last tile.  d_in = 64 and d_out = 256
keep the oracle cheap enough to check every output of the forward (y, u) and
the backward (dX, dA, dB), for sorted segments and for interleaved ids.
"""
import numpy as np
import pytest

import oracle.lora as OL
import workloads as W
from gpu_util import TOL_BF16, TOL_F32, DevLayer, f64_of, rel_err

pytestmark = pytest.mark.gpu
L = pytest.importorskip("rl_lora_linear_amd.lib")


@pytest.mark.parametrize("n,order", [(256 * 257 - 100, "sorted"), (256 * 520 + 7, "interleaved")])
def test_more_tiles_than_blocks(n, order):
    print(f"[persistent] n {n} {order}", flush=True)
    ranks = [16, 32, 8, 64]
    rng = np.random.default_rng(n)
    if order == "sorted":
        ids = W.sorted_ids_from_lengths(rng.multinomial(n, np.full(len(ranks), 1 / len(ranks))))
    else:
        ids = rng.integers(0, len(ranks), size=n).astype(np.int32)
    c = W.lora_layer(77, n, 64, 256, ranks, [float(r) for r in ranks], ids=ids, order=order)
    dl = DevLayer(c)
    y, u = dl.forward()
    dx, grad = dl.backward(u)
    assert dl.status() == 0
    x, Wb, A, B, s, idv = dl.oracle_args()
    y_ref, u_ref = OL.lora_forward(x, Wb, A, B, s, idv)
    assert rel_err(f64_of(y), y_ref) < TOL_BF16
    u_g = dl.u_values(u)
    assert rel_err(u_g[:, :u_ref.shape[1]], u_ref) < TOL_F32
    dx_ref, dA_ref, dB_ref, _ = OL.lora_backward(c.dy(), x, Wb, A, B, s, idv)
    assert rel_err(f64_of(dx), dx_ref) < TOL_BF16
    dA, dB = dl.split_grad(f64_of(grad))
    for i in range(c.n_adapters):
        assert rel_err(dA[i], dA_ref[i]) < TOL_F32, ("dA", i)
        assert rel_err(dB[i], dB_ref[i]) < TOL_F32, ("dB", i)
