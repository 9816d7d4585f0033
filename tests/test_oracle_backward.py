"""Pins for the oracle's backward of the selected-token log-probability.

L = sum_t g[t] logp[t]; the oracle's grad_hidden and grad_weight are checked
against torch's CPU autograd (fp64) of log_softmax(inv_tau h w^T) gathered
at the targets, against central finite differences of scipy's log_softmax,
and against identities the mathematics fixes: the logit gradient of each row
sums to zero, so grad_hidden vanishes when all weight rows are equal and the
rows of grad_weight sum to zero; rows with g = 0 or an out-of-range target
contribute nothing; 1/tau = 2 equals a doubled weight.  A dropped softmax
term, a sign error, a missing temperature factor or a transposed product
each fails one of them.
"""

import numpy as np
import pytest
import scipy.special

from invariant_selected_token_amd import synth
from oracle import oracle as orc


def _case(T=6, H=64, V=40, seed=5):
    c = synth.normal_case("bwd_small", seed, T, H, V, hidden_std=1.0, weight_std=0.2)
    g = np.random.Generator(np.random.PCG64(seed + 1)).normal(size=T)
    return c, g


def _f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("inv_tau", [1.0, 0.7])
def test_backward_matches_torch_autograd(inv_tau):
    torch = pytest.importorskip("torch")
    c, g = _case()
    h = torch.tensor(_f64(c.hidden), dtype=torch.float64, requires_grad=True)
    w = torch.tensor(_f64(c.weight), dtype=torch.float64, requires_grad=True)
    ls = torch.log_softmax(inv_tau * (h @ w.T), dim=1)
    y = torch.tensor(c.targets, dtype=torch.int64)
    loss = (torch.tensor(g) * ls[torch.arange(c.T), y]).sum()
    loss.backward()
    gh, gw = orc.selected_logp_backward(c.hidden, c.weight, c.targets, g, inv_tau)
    np.testing.assert_allclose(gh, h.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(gw, w.grad.numpy(), rtol=0, atol=1e-12)


def test_backward_finite_differences():
    c, g = _case(T=3, H=64, V=30, seed=9)
    hf, wf = _f64(c.hidden), _f64(c.weight)
    inv_tau = 0.8

    def loss(hh, ww):
        ls = scipy.special.log_softmax(inv_tau * (hh @ ww.T), axis=1)
        return float((g * ls[np.arange(c.T), c.targets]).sum())

    gh, gw = orc.selected_logp_backward(c.hidden, c.weight, c.targets, g, inv_tau)
    eps = 1e-6
    rng = np.random.Generator(np.random.PCG64(3))
    for _ in range(12):
        t, k = rng.integers(0, c.T), rng.integers(0, 64)
        d = np.zeros_like(hf)
        d[t, k] = eps
        fd = (loss(hf + d, wf) - loss(hf - d, wf)) / (2 * eps)
        assert abs(fd - gh[t, k]) < 1e-7
        v = rng.integers(0, c.V)
        d = np.zeros_like(wf)
        d[v, k] = eps
        fd = (loss(hf, wf + d) - loss(hf, wf - d)) / (2 * eps)
        assert abs(fd - gw[v, k]) < 1e-7


def test_logit_gradient_rows_sum_to_zero_and_target_term():
    c, g = _case(T=8, V=100)
    dz = orc.grad_logits(c.hidden, c.weight, c.targets, g)
    np.testing.assert_allclose(dz.sum(1), 0.0, atol=1e-14)
    ls = orc.log_softmax(c.hidden, c.weight)
    p = np.exp(ls)
    rows = np.arange(c.T)
    np.testing.assert_allclose(dz[rows, c.targets], g * (1 - p[rows, c.targets]),
                               rtol=0, atol=1e-14)
    off = np.ones_like(dz, dtype=bool)
    off[rows, c.targets] = False
    np.testing.assert_allclose(dz[off], (-g[:, None] * p)[off], rtol=0, atol=1e-15)


def test_equal_weight_rows_give_zero_hidden_gradient():
    c, g = _case(T=5, H=64, V=50)
    w = np.repeat(c.weight[:1], 50, axis=0)          # every vocabulary row equal
    gh, gw = orc.selected_logp_backward(c.hidden, w, c.targets, g)
    assert np.abs(gh).max() < 1e-14
    # and the rows of grad_weight always sum to zero
    gh2, gw2 = orc.selected_logp_backward(c.hidden, c.weight, c.targets, g)
    np.testing.assert_allclose(gw2.sum(0), 0.0, atol=1e-13)


def test_ignored_rows_contribute_nothing():
    c, g = _case(T=6)
    y = c.targets.copy()
    y[1] = -1
    y[4] = c.V
    g2 = g.copy()
    g2[2] = 0.0
    gh, gw = orc.selected_logp_backward(c.hidden, c.weight, y, g2)
    assert not gh[[1, 2, 4]].any()
    keep = [0, 3, 5]
    _, gw_keep = orc.selected_logp_backward(c.hidden[keep], c.weight, y[keep], g2[keep])
    np.testing.assert_allclose(gw, gw_keep, rtol=0, atol=1e-14)


def test_inverse_temperature_two_equals_doubled_weight():
    """logp(h, w, 1/tau = 2) = logp(h, 2w, 1): the hidden gradients agree
    exactly, and grad_w at 1/tau = 2 is twice the gradient with respect to 2w."""
    c, g = _case()
    w2 = synth.f32_exact_to_bf16_bits(2.0 * synth.bf16_bits_to_f32(c.weight))
    gh_a, gw_a = orc.selected_logp_backward(c.hidden, c.weight, c.targets, g, 2.0)
    gh_b, gw_b = orc.selected_logp_backward(c.hidden, w2, c.targets, g, 1.0)
    assert np.array_equal(gh_a, gh_b)
    assert np.array_equal(gw_a, 2.0 * gw_b)
