"""Pins for the fp64 CPU oracle: closed forms, brute force and invariants.

The oracle is the plain definition of the selected-token log-probability from
the RL-Kernel blog (section 四, Linear-LogP over the vocabulary; the LSE in its
max-shifted form).  Each test below checks it against something other than
itself: exact integer arithmetic, an unshifted softmax computed a different
way, closed forms, or printed numbers.  A dropped vocabulary term, a wrong
sign, a wrong gather index or a transposed operand each fails at least one.
"""

import math
import os

import numpy as np
import pytest

from invariant_selected_token_amd import synth
from oracle import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


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


# Hand-worked V = 4 examples.  Each closed form is simplified by hand, not
# evaluated with the oracle's max-shift algorithm.
HAND = [
    ((0.0, 0.0, 0.0, 0.0), lambda: math.log(4.0)),
    ((0.0, 1.0, 2.0, 3.0),
     lambda: 3.0 + math.log(1.0 + math.exp(-1.0) + math.exp(-2.0) + math.exp(-3.0))),
    ((40.0, 0.0, 0.0, 0.0), lambda: 40.0),  # 3e^-40 is below half an ulp of 40
    ((-1.0, -1.0, 2.0, 2.0), lambda: 2.0 + math.log(2.0 + 2.0 * math.exp(-3.0))),
    ((0.5, -0.25, 0.125, 0.0),
     lambda: 0.5 + math.log(1.0 + math.exp(-0.75) + math.exp(-0.375) + math.exp(-0.5))),
]


@pytest.mark.parametrize("zvec,lse_closed", HAND)
def test_v4_hand_examples(zvec, lse_closed):
    lse_ref = lse_closed()
    hidden, weight = _logit_inputs(zvec)
    for y in range(4):
        logp, lse = orc.selected_logp(hidden, weight, np.array([y], np.int32))
        assert abs(lse[0] - lse_ref) <= 1e-14 * max(1.0, abs(lse_ref))
        assert abs(logp[0] - (zvec[y] - lse_ref)) <= 1e-14 * max(1.0, abs(lse_ref))


def test_v4_worked_values():
    # A few of the values spelled out (ln 4 and the (40,0,0,0) row).
    hidden, weight = _logit_inputs((0.0, 0.0, 0.0, 0.0))
    logp, lse = orc.selected_logp(hidden, weight, np.array([2], np.int32))
    assert lse[0] == pytest.approx(1.3862943611198906, abs=1e-15)
    assert logp[0] == pytest.approx(-1.3862943611198906, abs=1e-15)
    hidden, weight = _logit_inputs((40.0, 0.0, 0.0, 0.0))
    lp = [orc.selected_logp(hidden, weight, np.array([y], np.int32))[0][0]
          for y in range(4)]
    assert lp == [0.0, -40.0, -40.0, -40.0]


@pytest.mark.parametrize("H,V", [(256, 4096), (4096, 151936)])
def test_all_equal_logits_closed_form(H, V):
    """hidden = 0 gives z = 0 for every v: lse = log V, logp = -log V."""
    hidden = np.zeros((2, H), np.uint16)
    rng = np.random.Generator(np.random.PCG64(7))
    weight = synth.f32_to_bf16_bits(
        rng.standard_normal((V, H), dtype=np.float32) * np.float32(0.02))
    targets = np.array([0, V - 1], np.int32)
    logp, lse = orc.selected_logp(hidden, weight, targets)
    assert np.all(lse == math.log(V))
    assert np.all(logp == -math.log(V))


def test_constant_logits_closed_form():
    """z = c for every v: lse = c + log V."""
    V, H, c = 1000, 64, 3.0
    hidden, weight = _logit_inputs(np.full(V, c), H)
    logp, lse = orc.selected_logp(hidden, weight, np.array([17], np.int32))
    assert lse[0] == pytest.approx(c + math.log(V), abs=1e-14)
    assert logp[0] == pytest.approx(-math.log(V), abs=1e-14)


def test_logits_exact_on_grid_vs_integer_matmul():
    """On {-1,0,1}*2^-4 inputs every partial sum is exact: compare to int64."""
    rng = np.random.Generator(np.random.PCG64(11))
    T, H, V = 5, 192, 37  # non-square, V not a multiple of 8
    hi = rng.integers(-1, 2, size=(T, H))
    wi = rng.integers(-1, 2, size=(V, H))
    hidden = _bf16(hi.astype(np.float32) / 16)
    weight = _bf16(wi.astype(np.float32) / 16)
    z_exact = (hi @ wi.T).astype(np.float64) / 256.0
    z = orc.logits(hidden, weight)
    assert z.shape == (T, V)
    assert np.array_equal(z, z_exact)


def test_interleaved_dot_products_equal_naive_loop():
    rng = np.random.Generator(np.random.PCG64(12))
    hidden = synth.f32_to_bf16_bits(rng.standard_normal((3, 320), dtype=np.float32))
    weight = synth.f32_to_bf16_bits(
        rng.standard_normal((45, 320), dtype=np.float32) * np.float32(0.02))
    a = orc.logits(hidden, weight)
    b = orc.logits_naive(hidden, weight)
    assert np.array_equal(a.view(np.uint64), b.view(np.uint64))


@pytest.mark.parametrize("V", [1, 2, 5, 16])
def test_bruteforce_softmax_tiny_vocab(V):
    """Unshifted softmax over an independently computed fp64 matmul."""
    rng = np.random.Generator(np.random.PCG64(100 + V))
    T, H = 6, 64
    hidden = synth.f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    weight = synth.f32_to_bf16_bits(
        rng.standard_normal((V, H), dtype=np.float32) * np.float32(0.3))
    targets = rng.integers(0, V, size=T, dtype=np.int32)
    h64 = synth.bf16_bits_to_f32(hidden).astype(np.float64)
    w64 = synth.bf16_bits_to_f32(weight).astype(np.float64)
    z = h64 @ w64.T
    assert np.abs(z).max() <= 20.0
    p = np.exp(z) / np.exp(z).sum(axis=1, keepdims=True)
    ref = np.log(p[np.arange(T), targets])
    logp, lse = orc.selected_logp(hidden, weight, targets)
    np.testing.assert_allclose(logp, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.log(np.exp(z).sum(axis=1)), rtol=0, atol=1e-12)


def test_sum_to_one_and_gather_consistency():
    c = synth.tiny_case()
    ls = orc.log_softmax(c.hidden, c.weight)
    np.testing.assert_allclose(np.exp(ls).sum(axis=1), 1.0, rtol=0, atol=1e-12)
    logp, lse = orc.selected_logp(c.hidden, c.weight, c.targets)
    np.testing.assert_allclose(logp, ls[np.arange(c.T), c.targets], rtol=0, atol=1e-13)
    assert np.all(logp <= 0.0)


def test_thread_count_does_not_change_bits():
    c = synth.tiny_case()
    a = orc.selected_logp(c.hidden, c.weight, c.targets, nthreads=1)
    b = orc.selected_logp(c.hidden, c.weight, c.targets, nthreads=max(2, orc.max_threads()))
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint64), y.view(np.uint64))


def test_vocab_permutation_equivariance():
    c = synth.tiny_case()
    perm = np.random.Generator(np.random.PCG64(5)).permutation(c.V)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(c.V)
    a_lp, a_lse = orc.selected_logp(c.hidden, c.weight, c.targets)
    b_lp, b_lse = orc.selected_logp(c.hidden, c.weight[perm], inv[c.targets].astype(np.int32))
    np.testing.assert_allclose(b_lp, a_lp, rtol=0, atol=1e-13)
    np.testing.assert_allclose(b_lse, a_lse, rtol=0, atol=1e-13)


@pytest.mark.parametrize("c", [-512.0, -3.0, 0.75, 64.0, 4096.0])
def test_shift_equivariance(c):
    """Adding c to every logit of a row adds c to its lse and leaves its logp
    unchanged (the softmax is invariant under a common shift).  The shift is
    built from the inputs: 64 more hidden columns (1, 0, ..., 0) and weight
    columns (c, 0, ..., 0), so every logit gains c exactly (c is bf16-exact
    and the fp64 sums stay exact).  A max shift applied twice or not at all,
    or an lse that drops the max, fails this."""
    k = synth.tiny_case()
    T, V = k.hidden.shape[0], k.weight.shape[0]
    hx = np.zeros((T, 64), np.float32)
    hx[:, 0] = 1.0
    wx = np.zeros((V, 64), np.float32)
    wx[:, 0] = c
    hidden2 = np.concatenate([k.hidden, _bf16(hx)], axis=1)
    weight2 = np.concatenate([k.weight, _bf16(wx)], axis=1)
    lp, lse = orc.selected_logp(k.hidden, k.weight, k.targets)
    lp2, lse2 = orc.selected_logp(hidden2, weight2, k.targets)
    ulp = np.spacing(np.maximum(np.abs(lse2), abs(c)))
    assert np.all(np.abs(lse2 - (lse + c)) <= 4 * ulp)
    assert np.all(np.abs(lp2 - lp) <= 4 * ulp)


def test_row_independence():
    """A row's result does not depend on the other rows passed with it."""
    c = synth.tiny_case()
    full = orc.selected_logp(c.hidden, c.weight, c.targets)
    for t in (0, 17, 63):
        one = orc.selected_logp(c.hidden[t:t + 1], c.weight, c.targets[t:t + 1])
        assert one[0][0] == full[0][t] and one[1][0] == full[1][t]


def _dominant_row(H, V, gap_scale, seed):
    """Grid weight, hidden = gap_scale*sign(w[v*, k]) on 1280 of its non-zeros."""
    rng = np.random.Generator(np.random.PCG64(seed))
    wi = rng.integers(-1, 2, size=(V, H))
    vstar = int(rng.integers(0, V))
    nz = np.flatnonzero(wi[vstar])[:1280]
    hi = np.zeros((1, H), np.int64)
    hi[0, nz] = np.sign(wi[vstar, nz])
    hidden = _bf16(hi.astype(np.float32) * np.float32(gap_scale))
    weight = _bf16(wi.astype(np.float32) / 16)
    z = (hi @ wi.T).astype(np.float64) * gap_scale / 16.0  # exact
    return hidden, weight, vstar, z[0]


@pytest.mark.parametrize("scale,zmax", [(0.5, 40.0), (1.25, 100.0)])
def test_dominant_logit(scale, zmax):
    """One logit far above the rest (40, and 100 where e^100 > FLT_MAX)."""
    H, V = 4096, 512
    hidden, weight, vstar, z = _dominant_row(H, V, scale, 21)
    assert z[vstar] == zmax
    others = np.delete(z, vstar)
    tail = np.exp(others - zmax).sum()  # independent of the oracle's loop
    logp, lse = orc.selected_logp(hidden, weight, np.array([vstar], np.int32))
    assert lse[0] == pytest.approx(zmax + math.log1p(tail), abs=1e-12)
    assert logp[0] == pytest.approx(-math.log1p(tail), abs=1e-12)
    assert -V * math.exp(-(zmax - others.max())) <= logp[0] <= 0.0
    y = int(np.argmin(z))
    logp2, _ = orc.selected_logp(hidden, weight, np.array([y], np.int32))
    assert logp2[0] == pytest.approx(z[y] - zmax - math.log1p(tail), abs=1e-12)


def test_nonfinite_and_range_policy():
    H, V = 64, 8
    rng = np.random.Generator(np.random.PCG64(3))
    weight = synth.f32_to_bf16_bits(
        rng.standard_normal((V, H), dtype=np.float32) * np.float32(0.5))
    hidden = synth.f32_to_bf16_bits(rng.standard_normal((5, H), dtype=np.float32))
    hidden[1, 3] = 0x7FC0            # NaN
    hidden[2, 5] = 0x7F80            # +Inf -> +/-Inf logits
    targets = np.array([0, 1, 2, -1, V], np.int32)
    logp, lse = orc.selected_logp(hidden, weight, targets)
    assert np.isfinite(logp[0]) and np.isfinite(lse[0])
    assert np.isnan(logp[1]) and np.isnan(lse[1])
    assert np.isnan(logp[2]) and np.isnan(lse[2])
    assert np.isnan(logp[3]) and np.isfinite(lse[3])   # target < 0
    assert np.isnan(logp[4]) and np.isfinite(lse[4])   # target >= V


def test_minus_inf_logits_carry_zero_probability():
    z = np.array([[-np.inf, 0.0, 0.0],
                  [-np.inf, -np.inf, -np.inf]])
    logp, lse = orc.lse_from_logits(z, np.array([0, 1], np.int32))
    assert lse[0] == math.log(2.0) and logp[0] == -np.inf
    assert lse[1] == -np.inf and np.isnan(logp[1])
    logp, _ = orc.lse_from_logits(z[:1], np.array([1], np.int32))
    assert logp[0] == -math.log(2.0)


def test_sample_targets_inverse_cdf():
    lp = np.log(np.array([[0.1, 0.2, 0.7]] * 5))
    u = np.array([0.0, 0.05, 0.15, 0.5, 0.999])
    assert orc.sample_targets(lp, u).tolist() == [0, 0, 1, 2, 2]


def _golden_ratio_rows():
    rows = []
    with open(os.path.join(GOLDEN, "ratio_worked_example.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, ro, tr, n, printed, digits = line.split()
                rows.append((name, float(ro), float(tr), int(n), float(printed), int(digits)))
    return rows


@pytest.mark.parametrize("row", _golden_ratio_rows(), ids=lambda r: r[0])
def test_ratio_worked_example_from_the_pages(row):
    """compare_stats' k3 uses r = exp(train - rollout) as the page defines it."""
    _, rollout, train, n, printed, digits = row
    a = np.full(n, train, np.float32)
    b = np.full(n, rollout, np.float32)
    st = orc.compare_stats(a, b)
    d = float(np.float32(train)) - float(np.float32(rollout))
    r_total = math.exp(n * d)            # ratio over n tokens: log-ratios add
    assert round(r_total, digits) == pytest.approx(printed, abs=10 ** -digits / 2)
    assert st["mismatch_count"] == n
    assert st["max_abs_diff"] == pytest.approx(abs(d), rel=1e-12)
    r = math.exp(d)
    assert st["k3_mean"] == pytest.approx(r - 1.0 - math.log(r), rel=1e-9)
    assert not (0.8 <= r_total <= 1.2) if n == 200 else (0.8 <= r_total <= 1.2)


def test_compare_stats_bitwise_semantics():
    a = np.array([1.0, -0.0, np.nan, 2.0], np.float32)
    b = np.array([1.0, 0.0, np.nan, np.nextafter(np.float32(2.0), np.float32(3.0))], np.float32)
    st = orc.compare_stats(a, b)
    assert st["mismatch_count"] == 2          # -0 vs +0 and the last ulp
    assert st["max_abs_diff"] == pytest.approx(2.0 ** -22)
