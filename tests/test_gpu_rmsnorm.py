"""GPU parity and invariance of the RMSNorm feeding the LM head.

The kernel's r = 1/sqrt(mean(x^2) + eps) carries the fp32 error of a sum of
positive squares (per-lane chains of H/64 terms, then 6 tree levels: at most
(H/64 + 6) 2^-24 relative), then /H, + eps, sqrt and the division (half an
ulp each) and the product x r: at most (H/64 + 16) 2^-24 relative in x r.
Its first bf16 rounding can therefore differ from the oracle's only where
the oracle's x r lies that close to a bf16 rounding midpoint; there the
kernel must give the other rounding, everywhere else the same bits.
"""

import numpy as np
import pytest

import invariant_selected_token_amd as rlk
from invariant_selected_token_amd import synth
from oracle import oracle as orc

from conftest import to_dev_bf16, to_dev_i32

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _inputs(T, H, seed, scale=3.0):
    x = synth.normal_bf16(seed, 0, T, H, scale)
    g = synth.f32_to_bf16_bits(
        1.0 + 0.1 * np.random.Generator(np.random.PCG64(seed + 1)).normal(size=H).astype(np.float32))
    return x, g


def _gpu(x, g, eps, dev):
    y = rlk.rlk_rmsnorm(to_dev_bf16(x, dev), to_dev_bf16(g.reshape(1, -1), dev)[0], eps)
    torch.cuda.synchronize()
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


def _alternatives(xr, g):
    """Per element: the bits the oracle gives, the bits of the other rounding
    of x r, and whether x r is close enough to a midpoint for either."""
    x32 = xr.astype(np.float32).astype(np.float64)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.abs(x32)))
    step = np.where(x32 == 0, 2.0 ** -133, np.exp2(e - 7))
    lo = np.floor(x32 / step) * step
    hi = lo + step
    mid = lo + step / 2
    n_ref = orc.round_bf16(x32.astype(np.float32))
    other = np.where(n_ref == lo, hi, lo)
    gf = synth.bf16_bits_to_f32(g).astype(np.float64)
    y_other = synth.f32_to_bf16_bits((other * gf).astype(np.float32))   # exact product
    return mid, y_other


# H up to 4096 and up to 8192 keep the row in registers (8 or 16 chunks per
# lane), larger H reads it twice: all three paths, with ragged chunk counts.
@pytest.mark.parametrize("T,H,eps", [(1, 64, 1e-6), (300, 4096, 1e-6), (77, 192, 1e-5),
                                     (513, 2056, 1e-6), (64, 8192, 0.0), (33, 4104, 1e-6),
                                     (9, 16392, 1e-6)])
def test_rmsnorm_parity(dev, T, H, eps):
    x, g = _inputs(T, H, 500 + H)
    got = _gpu(x, g, eps, dev)
    ref, xr = orc.rmsnorm(x, g, eps, want_xr=True)
    mid, y_other = _alternatives(xr, g)
    near = np.abs(xr - mid) <= (H / 64 + 16) * 2.0 ** -24 * np.abs(xr) + 2.0 ** -140
    diff = got != ref
    print(f"rmsnorm T={T} H={H}: {int(diff.sum())} of {diff.size} elements take the other "
          f"rounding, {int(near.sum())} are near a midpoint", flush=True)
    assert not (diff & ~near).any(), "a difference away from a rounding midpoint"
    assert np.array_equal(got[diff], y_other[diff])


def test_rmsnorm_batch_invariant(dev):
    x, g = _inputs(256, 4096, 77)
    full = _gpu(x, g, 1e-6, dev)
    for t in (0, 3, 255):
        one = _gpu(x[t:t + 1], g, 1e-6, dev)
        assert np.array_equal(one[0], full[t])
    perm = np.random.Generator(np.random.PCG64(5)).permutation(256)
    assert np.array_equal(_gpu(x[perm], g, 1e-6, dev), full[perm])


def test_rmsnorm_feeding_the_lm_head(prefill, dev):
    """Pre-norm hidden states -> RMSNorm -> selected-token logp, against the
    oracle's RMSNorm -> oracle's logp on sampled rows, and bitwise invariant
    to packing."""
    c = prefill.case
    x, g = _inputs(c.T, c.H, 91)
    xd = to_dev_bf16(x, dev)
    gd = to_dev_bf16(g.reshape(1, -1), dev)[0]
    h = rlk.rlk_rmsnorm(xd, gd, 1e-6)
    lp, lse = rlk.rlk_selected_logp(h, prefill.weight, prefill.targets)
    torch.cuda.synchronize()
    rows = np.array([0, 511, 512, 4095])
    hn = orc.rmsnorm(x[rows], g, 1e-6)
    r_lp, r_lse = orc.selected_logp(hn, c.weight, c.targets[rows])
    assert np.abs(lp.cpu().numpy()[rows] - r_lp).max() <= 1e-3
    assert np.abs(lse.cpu().numpy()[rows] - r_lse).max() <= 1e-3
    h2 = rlk.rlk_rmsnorm(xd[512:1024], gd, 1e-6)
    lp2, _ = rlk.rlk_selected_logp(h2, prefill.weight, prefill.targets[512:1024])
    torch.cuda.synchronize()
    assert torch.equal(lp2.view(torch.int32), lp[512:1024].view(torch.int32))
