"""Pins for the oracle's RMSNorm (the normalisation feeding the LM head).

y = bf16(bf16(x r) gamma), r = 1 / sqrt(mean(x^2) + eps) per row.  Checked
against torch's CPU rms_norm in fp64 followed by torch's own fp64 -> fp32 ->
bf16 casts, closed forms for constant and alternating rows (which catch a sum
used in place of the mean, a missing square root or a missing eps), exact
scale invariance at eps = 0, and the exact effect of doubling gamma.
"""

import numpy as np
import pytest

from invariant_selected_token_amd import synth
from oracle import oracle as orc


def _bits(x):
    return synth.f32_exact_to_bf16_bits(np.asarray(x, np.float32))


def _rows(T=8, H=256, seed=31, std=1.0):
    return synth.normal_bf16(seed, 0, T, H, std)


@pytest.mark.parametrize("H", [64, 4096])
@pytest.mark.parametrize("c", [2.0, -0.375, 3.0])
def test_constant_row_normalises_to_gamma(H, c):
    """x = c everywhere: mean(x^2) = c^2, x r = c / sqrt(c^2 + eps) rounds to
    sign(c) in bf16 (within 2^-20 of it), so y = sign(c) gamma exactly."""
    x = _bits(np.full((2, H), c))
    g = synth.f32_to_bf16_bits(np.linspace(-2, 2, H).astype(np.float32))
    y = orc.rmsnorm(x, g, 1e-6)
    want = _bits(np.sign(c) * synth.bf16_bits_to_f32(g))
    assert np.array_equal(y, np.broadcast_to(want, y.shape))


def test_alternating_row_and_mean_not_sum():
    H = 1024
    x = _bits(np.tile(np.array([1.5, -1.5], np.float32), (1, H // 2)))
    y = orc.rmsnorm(x, _bits(np.ones(H)), 0.0)
    assert np.array_equal(synth.bf16_bits_to_f32(y)[0], np.tile([1.0, -1.0], H // 2))


def test_eps_enters_under_the_root():
    """x = 2^-10 everywhere with eps = 3 * 2^-20: x r = 2^-10 / sqrt(4 * 2^-20) = 1/2."""
    H = 64
    x = _bits(np.full((1, H), 2.0 ** -10))
    y, xr = orc.rmsnorm(x, _bits(np.ones(H)), 3 * 2.0 ** -20, want_xr=True)
    assert np.all(xr == 0.5) and np.all(synth.bf16_bits_to_f32(y) == 0.5)


def test_scale_invariance_exact_without_eps():
    x = _rows()
    x2 = _bits(2.0 * synth.bf16_bits_to_f32(x))
    g = _rows(1, 256, 32)[0]
    assert np.array_equal(orc.rmsnorm(x, g, 0.0), orc.rmsnorm(x2, g, 0.0))


def test_doubling_gamma_doubles_y_exactly():
    x = _rows()
    g = _rows(1, 256, 33)[0]
    g2 = _bits(2.0 * synth.bf16_bits_to_f32(g))
    y1 = synth.bf16_bits_to_f32(orc.rmsnorm(x, g, 1e-6))
    y2 = synth.bf16_bits_to_f32(orc.rmsnorm(x, g2, 1e-6))
    assert np.array_equal(y2, 2.0 * y1)


@pytest.mark.parametrize("H,eps", [(256, 1e-6), (4096, 1e-6), (192, 1e-5)])
def test_matches_torch_rms_norm_and_casts(H, eps):
    torch = pytest.importorskip("torch")
    x = _rows(16, H, 40 + H)
    g = _rows(1, H, 41 + H, 0.5)[0]
    xt = torch.from_numpy(synth.bf16_bits_to_f32(x).astype(np.float64))
    xr = torch.nn.functional.rms_norm(xt, (H,), eps=eps)
    n = xr.to(torch.float32).to(torch.bfloat16).to(torch.float32)
    gt = torch.from_numpy(synth.bf16_bits_to_f32(g))
    yt = (n * gt).to(torch.bfloat16)                   # bf16 * bf16 is exact in fp32
    want = yt.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.rmsnorm(x, g, eps), want)
