"""Pins for the oracle's contract options: temperature, bf16 logits, entropy.

Each option is checked against something other than the oracle itself:
hand-derived round-to-nearest-even values and torch's CPU fp32 -> bf16 cast
for the rounding; closed forms for the entropy of uniform and two-level
distributions; scipy's log-softmax and entropy on small rows; an exact
identity (multiplying the logits by 2 equals doubling the weight, both exact
in binary floating point).  A misplaced temperature (applied after the LSE or
to the LSE only), a rounding that truncates or rounds ties away, an entropy
with a wrong sign or a dropped vocabulary term each fail one of these.
"""

import math

import numpy as np
import pytest
import scipy.special
import scipy.stats

from invariant_selected_token_amd import synth
from oracle import oracle as orc


def _bf16(x):
    return synth.f32_exact_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _logit_inputs(zvec, H=64):
    """hidden = e0, weight[v, 0] = z_v: logits equal z exactly (z bf16-exact)."""
    V = len(zvec)
    hidden = np.zeros((1, H), np.float32)
    hidden[0, 0] = 1.0
    weight = np.zeros((V, H), np.float32)
    weight[:, 0] = zvec
    return _bf16(hidden), _bf16(weight)


# --------------------------------------------------------------- rounding --

def _f32(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


# (fp32 input, expected bf16 value), each worked out by hand from the format:
# 8 significant bits, so the spacing just above 1 is 2^-7.
HAND_ROUND = [
    (1.0 + 2.0 ** -8, 1.0),                        # midpoint, 1 is even
    (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),        # midpoint, 1 + 2/128 is even
    (1.0 + 2.0 ** -8 + 2.0 ** -20, 1.0 + 2.0 ** -7),   # just above the midpoint
    (1.0 + 2.0 ** -8 - 2.0 ** -20, 1.0),           # just below it
    (-(1.0 + 3 * 2.0 ** -8), -(1.0 + 2.0 ** -6)),  # symmetric for negatives
    (3.0, 3.0),
    (0.1, 0.10009765625),                          # 0x3DCCCCCD -> 0x3DCD
    (255.0 * 2.0 ** 120, 255.0 * 2.0 ** 120),      # largest finite bf16
    (-0.0, -0.0),
    (2.0 ** -130, 2.0 ** -130),                    # bf16 subnormal, exact
    (2.0 ** -134, 0.0),                            # half the smallest subnormal: tie -> 0
    (3 * 2.0 ** -134, 2.0 ** -132),                # 1.5 steps: tie -> 2 steps
]


@pytest.mark.parametrize("x,want", HAND_ROUND)
def test_round_bf16_hand_values(x, want):
    got = orc.round_bf16(np.array([x], np.float32))[0]
    assert got == want and math.copysign(1.0, got) == math.copysign(1.0, want)


def test_round_bf16_overflow_and_specials():
    fmax = _f32(0x7F7FFFFF)           # above the midpoint past bf16's largest
    below = _f32(0x7F7F7FFF)          # below that midpoint
    got = orc.round_bf16(np.array([fmax, -fmax, below, np.inf, -np.inf, np.nan],
                                  np.float32))
    assert got[0] == np.inf and got[1] == -np.inf
    assert got[2] == 255.0 * 2.0 ** 120
    assert got[3] == np.inf and got[4] == -np.inf and np.isnan(got[5])


def test_round_bf16_matches_torch_cpu_cast():
    torch = pytest.importorskip("torch")
    rng = np.random.Generator(np.random.PCG64(2024))
    bits = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    # half of them exactly on a rounding midpoint (low 16 bits 0x8000)
    bits[::2] = (bits[::2] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    got = orc.round_bf16(x)
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all(), x[~same][:5]
    assert (np.signbit(got) == np.signbit(want)).all()


# ------------------------------------------------------------- options ----

def test_no_options_equals_plain_path_bitwise():
    c = synth.tiny_case()
    lp, lse = orc.selected_logp(c.hidden, c.weight, c.targets)
    lp2, lse2, _ = orc.selected_logp_ex(c.hidden, c.weight, c.targets, 1.0, False)
    assert np.array_equal(lp.view(np.uint64), lp2.view(np.uint64))
    assert np.array_equal(lse.view(np.uint64), lse2.view(np.uint64))


def test_inverse_temperature_two_equals_doubled_weight_exactly():
    """z (2 w) = 2 z (w) exactly (every product and partial sum doubles), and
    z * 2.0 is exact, so the two must agree to the bit."""
    c = synth.tiny_case()
    w2 = synth.f32_exact_to_bf16_bits(2.0 * synth.bf16_bits_to_f32(c.weight))
    a = orc.selected_logp_ex(c.hidden, c.weight, c.targets, 2.0, False)
    b = orc.selected_logp_ex(c.hidden, w2, c.targets, 1.0, False)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint64), y.view(np.uint64))


@pytest.mark.parametrize("inv_tau", [0.7, 1.0 / 0.6, 1.25])
def test_temperature_against_scipy_log_softmax(inv_tau):
    c = synth.tiny_case()
    z = orc.logits(c.hidden, c.weight)
    ref = scipy.special.log_softmax(z * inv_tau, axis=1)
    lp, lse, ent = orc.selected_logp_ex(c.hidden, c.weight, c.targets, inv_tau, False)
    rows = np.arange(c.T)
    np.testing.assert_allclose(lp, ref[rows, c.targets], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(z * inv_tau, axis=1),
                               rtol=0, atol=1e-12)
    p = np.exp(ref)
    np.testing.assert_allclose(ent, scipy.stats.entropy(p, axis=1), rtol=0, atol=1e-10)


@pytest.mark.parametrize("inv_tau", [1.0, 0.7])
def test_bf16_mode_equals_torch_rounded_logits(inv_tau):
    """bf16 mode = the plain LSE of logits cast fp64 -> fp32 -> bf16 by torch."""
    torch = pytest.importorskip("torch")
    c = synth.tiny_case()
    z = orc.logits(c.hidden, c.weight) * inv_tau
    zb = torch.from_numpy(z.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    lp_ref, lse_ref = orc.lse_from_logits(zb, c.targets)
    lp, lse, ent = orc.selected_logp_ex(c.hidden, c.weight, c.targets, inv_tau, True)
    np.testing.assert_allclose(lp, lp_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-13)
    # rounding really happened: the bf16 logits differ from the fp64 ones
    assert np.abs(zb - z).max() > 1e-4


# ------------------------------------------------------------- entropy ----

@pytest.mark.parametrize("V", [4, 4096, 151936])
def test_entropy_uniform_is_log_v(V):
    hidden, weight = _logit_inputs(np.zeros(V, np.float32))
    _, _, ent = orc.selected_logp_ex(hidden, weight, np.array([0], np.int32))
    assert abs(ent[0] - math.log(V)) <= 1e-12 * math.log(V)


@pytest.mark.parametrize("a", [1.0, 5.0, -3.0, 40.0])
def test_entropy_two_level_closed_form(a):
    """z = a at one entry, 0 at the other V - 1: with Z = e^a + V - 1,
    H = log Z - a e^a / Z (worked out by hand from -sum p log p)."""
    V = 1000
    zvec = np.zeros(V, np.float32)
    zvec[17] = a
    hidden, weight = _logit_inputs(zvec)
    _, _, ent = orc.selected_logp_ex(hidden, weight, np.array([17], np.int32))
    Z = math.exp(a) + V - 1
    want = math.log(Z) - a * math.exp(a) / Z
    assert abs(ent[0] - want) <= 1e-12 * max(1.0, abs(want))


def test_entropy_bruteforce_scipy_small_rows():
    rng = np.random.Generator(np.random.PCG64(77))
    for V in (2, 3, 37, 129):
        z = rng.normal(0.0, 3.0, size=(5, V))
        y = rng.integers(0, V, size=5).astype(np.int32)
        _, _, ent = orc.ex_from_logits(z, y)
        want = scipy.stats.entropy(scipy.special.softmax(z, axis=1), axis=1)
        np.testing.assert_allclose(ent, want, rtol=0, atol=1e-12)
        assert (ent >= 0).all() and (ent <= math.log(V) + 1e-12).all()


def test_entropy_permutation_invariant_and_temperature_limits():
    rng = np.random.Generator(np.random.PCG64(78))
    z = rng.normal(0.0, 2.0, size=(4, 500))
    y = np.zeros(4, np.int32)
    _, _, e0 = orc.ex_from_logits(z, y)
    _, _, e1 = orc.ex_from_logits(z[:, rng.permutation(500)], y)
    np.testing.assert_allclose(e0, e1, rtol=0, atol=1e-12)
    _, _, hot = orc.ex_from_logits(z, y, inv_tau=0.0)       # tau -> infinity
    np.testing.assert_allclose(hot, math.log(500), rtol=0, atol=1e-12)
    _, _, cold = orc.ex_from_logits(z, y, inv_tau=1e4)      # tau -> 0: one-hot
    assert (cold < 1e-6).all()


def test_entropy_nonfinite_policy():
    z = np.zeros((4, 8))
    z[0, 3] = np.nan                     # NaN logit -> NaN everything
    z[1, :] = -np.inf                    # all -inf -> lse -inf, entropy NaN
    z[2, :] = -np.inf
    z[2, 5] = 1.5                        # one finite logit -> entropy 0
    z[3, :4] = -np.inf                   # -inf entries carry no probability
    y = np.array([0, 0, 5, 6], np.int32)
    lp, lse, ent = orc.ex_from_logits(z, y)
    assert np.isnan(ent[0]) and np.isnan(lse[0])
    assert lse[1] == -np.inf and np.isnan(ent[1])
    assert ent[2] == 0.0 and lse[2] == 1.5 and lp[2] == 0.0
    assert abs(ent[3] - math.log(4)) < 1e-15
