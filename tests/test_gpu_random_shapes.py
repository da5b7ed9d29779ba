"""Seeded random shapes through the dense mixed-adapter layer on the GPU,
against the oracle (oracle.lora), forward and backward.

Each seed draws a batch size from a list that straddles the tile edges (1 to
3000 tokens), d_in and d_out as multiples of 64 up to 1024, 1 to 12 adapters
with ranks that are multiples of 8 up to 64 and alphas from {8, 16, 32, 64},
and either sorted segments of Dirichlet-random lengths (some empty) or
interleaved ids that include ids with no adapter (-1 and n_adapters).  The bar
is the one of the hand-picked layer cases: y and dX within the bf16 tolerance,
u, dA and dB within the fp32 one, and the status word flags exactly the ids
outside the adapter range.
"""
import numpy as np
import pytest

import oracle.lora as OL
import workloads as W
from gpu_util import TOL_BF16, TOL_F32, DevLayer, f64_of, rel_err

pytestmark = pytest.mark.gpu
L = pytest.importorskip("rl_lora_linear_amd.lib")


def _draw(seed):
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.choice([1, 7, 31, 33, 255, 257, 513, 1000, 2049, 3000]))
    d_in = 64 * int(rng.integers(1, 17))
    d_out = 64 * int(rng.integers(1, 17))
    n_ad = int(rng.integers(1, 13))
    ranks = [8 * int(rng.integers(1, 9)) for _ in range(n_ad)]
    alphas = [float(rng.choice([8, 16, 32, 64])) for _ in range(n_ad)]
    if rng.random() < 0.5:
        order = "sorted"
        ids = W.sorted_ids_from_lengths(rng.multinomial(n, rng.dirichlet(np.ones(n_ad))))
    else:
        order = "interleaved"
        ids = rng.integers(-1, n_ad + 1, size=n).astype(np.int32)
    return W.lora_layer(2000 + seed, n, d_in, d_out, ranks, alphas, ids=ids, order=order)


@pytest.mark.parametrize("seed", range(24))
def test_random_layer_parity(seed):
    c = _draw(seed)
    ranks = [int(r) for r in c.ranks]
    print(f"[random] seed {seed}: n {c.n_tokens} d {c.d_in}->{c.d_out} ranks {ranks} {c.order}",
          flush=True)
    dl = DevLayer(c)
    y, u = dl.forward()
    dx, grad = dl.backward(u)
    x, Wb, A, B, s, ids = dl.oracle_args()
    valid = bool(np.all((ids >= 0) & (ids < c.n_adapters)))
    assert dl.status() == (0 if valid else L.FLAG_ID_RANGE)
    y_ref, u_ref = OL.lora_forward(x, Wb, A, B, s, ids)
    assert rel_err(f64_of(y), y_ref) < TOL_BF16
    u_g = dl.u_values(u)
    assert rel_err(u_g[:, :u_ref.shape[1]], u_ref) < TOL_F32
    assert not np.any(u_g[:, u_ref.shape[1]:])
    dx_ref, dA_ref, dB_ref, _ = OL.lora_backward(c.dy(), x, Wb, A, B, s, ids)
    assert rel_err(f64_of(dx), dx_ref) < TOL_BF16
    dA, dB = dl.split_grad(f64_of(grad))
    for i in range(c.n_adapters):
        assert rel_err(dA[i], dA_ref[i]) < TOL_F32, ("dA", i)
        assert rel_err(dB[i], dB_ref[i]) < TOL_F32, ("dB", i)
