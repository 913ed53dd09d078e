"""CPU checks of the composed decoder layer's oracle side (used by
test_gpu_layer.py): the oracle projection wrapped as an autograd function
gives, through the whole composition, the same output and gradients as torch
autograd of the same fp64 formulas written out with plain matmuls, so the
wrapper's forward and backward wiring (shapes, operand order, the scale) is
pinned independently of the GPU."""
import numpy as np
import pytest

from oracle import nf4
from tests import decoder_layer as dl
from tests.test_gpu_layer import _oracle_layer


def test_oracle_layer_matches_torch_autograd():
    torch = pytest.importorskip("torch")
    spec = dl.LayerSpec(d=128, f=192, heads=2, r=8, alpha=16.0)
    params = dl.make_params(spec, seed=3)
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 12, spec.d), dtype=np.float32)
    dy = rng.standard_normal((2, 12, spec.d), dtype=np.float32)
    ry, rdx, rgrads = _oracle_layer(spec, params, x, dy)

    cb = nf4.nf4_codebook()
    W = {n: torch.from_numpy(nf4.dequantize(nf4.quantize(params[n][0], cb), cb).astype(np.float64)) for n in dl.NAMES}
    A = {n: torch.from_numpy(params[n][1].astype(np.float64)).requires_grad_(True) for n in dl.NAMES}
    B = {n: torch.from_numpy(params[n][2].astype(np.float64)).requires_grad_(True) for n in dl.NAMES}
    x64 = torch.from_numpy(x.astype(np.float64)).requires_grad_(True)

    def lin(n, h):
        return h @ W[n].T + spec.scale * ((h @ A[n].T) @ B[n].T)

    y = dl.layer_forward(x64, lin, torch.from_numpy(params["g1"].astype(np.float64)),
                         torch.from_numpy(params["g2"].astype(np.float64)), spec.heads)
    y.backward(torch.from_numpy(dy.astype(np.float64)))
    np.testing.assert_allclose(ry, y.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(rdx, x64.grad.numpy(), rtol=1e-10, atol=1e-12)
    for n in dl.NAMES:
        np.testing.assert_allclose(rgrads[n][0], A[n].grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(rgrads[n][1], B[n].grad.numpy(), rtol=1e-10, atol=1e-12)
