"""SwiGLU MLP with a LoRA on each projection (gate, up, down; mixed ranks,
interleaved ids) on the GPU against oracle.lora / oracle.mlp, call by call:
each library call is compared with the oracle evaluated on the same input bits,
including the GPU's own outputs of the previous call."""
import numpy as np
import pytest

import oracle.lora as OL
import oracle.mlp as OM
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_util import TOL_BF16, TOL_F32, DevLayer, bits_of, dev_bf16, f64_of, rel_err  # noqa: E402
import rl_lora_linear_amd.lib as L  # noqa: E402


def _oracle_args(dl, x=None):
    xx, Wb, A, B, s, ids = dl.oracle_args()
    return (xx if x is None else x), Wb, A, B, s, ids


@pytest.mark.parametrize("n,d,f,n_ad", [(600, 256, 320, 6), (1500, 192, 448, 9)])
def test_mlp_call_by_call(n, d, f, n_ad):
    c = W.mlp_block(seed=31, n_tokens=n, d=d, d_ff=f, n_adapters=n_ad)
    gate, up, down = DevLayer(c.gate), DevLayer(c.up), DevLayer(c.down)
    # forward: gate and up share x
    g, ug = gate.forward()
    u, uu = up.forward(x=gate.x)
    h = torch.empty_like(g)
    L.swiglu_forward(g, u, h)
    y, ud = down.forward(x=h)
    for dl, out in ((gate, g), (up, u)):
        y_ref, _ = OL.lora_forward(*_oracle_args(dl, x=W.bf16_bits_to_f64(c.gate.x_bits)))
        assert rel_err(f64_of(out), y_ref) < TOL_BF16
    h_ref = OM.swiglu_forward(f64_of(g), f64_of(u))
    assert rel_err(f64_of(h), h_ref) < TOL_BF16
    y_ref, u_ref = OL.lora_forward(*_oracle_args(down, x=f64_of(h)))
    assert rel_err(f64_of(y), y_ref) < TOL_BF16
    assert rel_err(down.u_values(ud)[:, :u_ref.shape[1]], u_ref) < TOL_F32
    # backward: down, SwiGLU, gate and up, dx = dx_gate + dx_up
    dh, gd = down.backward(ud, x=h)
    dx_ref, dA_ref, dB_ref, _ = OL.lora_backward(c.down.dy(), *_oracle_args(down, x=f64_of(h)))
    assert rel_err(f64_of(dh), dx_ref) < TOL_BF16
    dA, dB = down.split_grad(gd.cpu().numpy().astype(np.float64))
    for i in range(n_ad):
        assert rel_err(dA[i], dA_ref[i]) < TOL_F32 and rel_err(dB[i], dB_ref[i]) < TOL_F32, ("down", i)
    dg, du = torch.empty_like(g), torch.empty_like(u)
    L.swiglu_backward(dh, g, u, dg, du)
    dg_ref, du_ref = OM.swiglu_backward(f64_of(dh), f64_of(g), f64_of(u))
    assert rel_err(f64_of(dg), dg_ref) < TOL_BF16 and rel_err(f64_of(du), du_ref) < TOL_BF16
    dxs = []
    for name, dl, d_up, uv in (("gate", gate, dg, ug), ("up", up, du, uu)):
        dxp, gp = dl.backward(uv, dy=d_up, x=gate.x)
        dx_ref, dA_ref, dB_ref, _ = OL.lora_backward(f64_of(d_up), *_oracle_args(
            dl, x=W.bf16_bits_to_f64(c.gate.x_bits)))
        assert rel_err(f64_of(dxp), dx_ref) < TOL_BF16, name
        dA, dB = dl.split_grad(gp.cpu().numpy().astype(np.float64))
        for i in range(n_ad):
            assert rel_err(dA[i], dA_ref[i]) < TOL_F32 and rel_err(dB[i], dB_ref[i]) < TOL_F32, (name, i)
        dxs.append(dxp)
    dx = torch.empty_like(dxs[0])
    L.bf16_add(dxs[0], dxs[1], dx)
    # one rounding of the exact sum (two bf16 values add exactly in fp64)
    assert np.array_equal(bits_of(dx), W.to_bf16_bits(f64_of(dxs[0]) + f64_of(dxs[1])))
    assert gate.status() == 0 and up.status() == 0 and down.status() == 0
