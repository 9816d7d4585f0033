"""GPU parity and invariance of the contract options: temperature, bf16
logits, entropy (rlk_selected_logp_ex and the two-stage _ex calls).

Tolerance 1e-3 against the fp64 oracle, as for the plain path, with one
exception derived from the arithmetic: in bf16 mode a logit is rounded to
bf16 from its fp32 value, and the kernel's fp32 value differs from the
oracle's by the fp32 summation error, at most H 2^-24 sum_k |h_k w_k|.  Where
the oracle's logit lies within that distance of a bf16 rounding midpoint the
two sides may round it to neighbouring bf16 values; only there the test
allows a change of that logit by its bf16 step (doubled, for second-order
terms), propagated to first order: by p_v to the lse, by p_v |z_v - E z| to
the entropy (dH/dz_v = -p_v (z_v - E z)), and in full to the target logit.
On grid inputs, where every fp32 sum is exact, no slack is allowed.
"""

import math

import numpy as np
import pytest

import invariant_selected_token_amd as rlk
from invariant_selected_token_amd import synth
from oracle import oracle as orc

from conftest import to_dev_bf16, to_dev_i32

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

TOL = 1e-3


def _np(*ts):
    torch.cuda.synchronize()
    return [None if t is None else t.cpu().numpy().astype(np.float64) for t in ts]


def _bits(x):
    return x.contiguous().view(torch.int32)


def _close(got, ref, what, tol=TOL):
    nan = np.isnan(got)
    assert np.array_equal(nan, np.isnan(ref)), f"{what}: NaN pattern differs"
    d = np.where(nan, 0.0, np.abs(np.where(nan, 0.0, got) - np.where(nan, 0.0, ref)))
    tol = np.broadcast_to(tol, d.shape)
    worst = np.max(d - tol) if d.size else 0.0
    print(f"{what}: max |diff| = {d.max():.3e}, worst excess over tolerance {worst:.3e}",
          flush=True)
    assert (d <= tol).all(), f"{what}: max |diff| {d.max()}"


def _ex(h, w, y, inv_tau=1.0, bf16=False, ent=True):
    lp, lse, e = rlk.rlk_selected_logp_ex(h, w, y, inv_temperature=inv_tau,
                                          logits_bf16=bf16, entropy=ent)
    return lp, lse, e


def _bf16_slack(hidden, weight, targets, inv_tau):
    """Per-row allowance for logp and lse in bf16 mode (see module doc)."""
    z = orc.logits(hidden, weight) * inv_tau
    habs = synth.f32_exact_to_bf16_bits(np.abs(synth.bf16_bits_to_f32(hidden)))
    wabs = synth.f32_exact_to_bf16_bits(np.abs(synth.bf16_bits_to_f32(weight)))
    bound = hidden.shape[1] * 2.0 ** -24 * orc.logits(habs, wabs) * abs(inv_tau) * 1.0001
    z32 = z.astype(np.float32).astype(np.float64)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.abs(z32)))
    step = np.where(z32 == 0, 2.0 ** -133, np.exp2(e - 7))
    mid = (np.floor(z32 / step) + 0.5) * step
    near = np.abs(z32 - mid) <= bound + 2.0 ** -40
    zb = orc.round_bf16(z32.astype(np.float32))
    m = zb.max(1, keepdims=True)
    p = np.exp(zb - m)
    p /= p.sum(1, keepdims=True)
    dz = step * 2 * near                      # possible change of each logit
    slack_lse = (p * dz).sum(1)
    ez = (p * zb).sum(1, keepdims=True)
    slack_ent = (p * np.abs(zb - ez) * dz).sum(1)
    rows = np.arange(len(targets))
    slack_lp = dz[rows, targets] + slack_lse
    return slack_lp, slack_lse, slack_ent, near


# sampled rows of the grid case: zero rows, dominant rows, duplicates, others
ADV_ROWS = np.array([0, 15, 16, 20, 24, 31, 32, 40, 64, 72, 500, 1023])


# ---------------------------------------------------------------- identity --

def test_unit_temperature_with_entropy_keeps_plain_bits(tiny, prefill):
    """The option kernel at 1/tau = 1 without rounding gives the plain bits."""
    for c in (tiny, prefill):
        lp0, lse0 = rlk.rlk_selected_logp(c.hidden, c.weight, c.targets)
        lp1, lse1, _ = _ex(c.hidden, c.weight, c.targets, 1.0, False, True)
        torch.cuda.synchronize()
        assert torch.equal(_bits(lp0), _bits(lp1)) and torch.equal(_bits(lse0), _bits(lse1))


# ---------------------------------------------------------------- parity ----

@pytest.mark.parametrize("inv_tau", [1.0, 0.7, 1.0 / 0.6, 2.0])
def test_temperature_and_entropy_tiny(tiny, inv_tau):
    c = tiny.case
    lp, lse, ent = _np(*_ex(tiny.hidden, tiny.weight, tiny.targets, inv_tau))
    r_lp, r_lse, r_ent = orc.selected_logp_ex(c.hidden, c.weight, c.targets, inv_tau, False)
    _close(lp, r_lp, f"logp 1/tau={inv_tau}")
    _close(lse, r_lse, f"lse 1/tau={inv_tau}")
    _close(ent, r_ent, f"entropy 1/tau={inv_tau}")
    assert (ent >= 0).all() and (ent <= math.log(c.V) + 1e-5).all()


@pytest.mark.parametrize("T,H,V", [(1, 64, 5), (255, 256, 129), (300, 192, 1000),
                                   (513, 128, 4133), (64, 128, 769), (100, 320, 2000)])
def test_options_ragged_shapes(dev, T, H, V):
    c = synth.normal_case(f"opt_{T}x{H}x{V}", 900 + T, T, H, V)
    h, w, y = to_dev_bf16(c.hidden, dev), to_dev_bf16(c.weight, dev), to_dev_i32(c.targets, dev)
    lp, lse, ent = _np(*_ex(h, w, y, 0.8, False, True))
    r_lp, r_lse, r_ent = orc.selected_logp_ex(c.hidden, c.weight, c.targets, 0.8, False)
    _close(lp, r_lp, f"logp {T}x{H}x{V}")
    _close(lse, r_lse, f"lse {T}x{H}x{V}")
    _close(ent, r_ent, f"entropy {T}x{H}x{V}")


def test_inverse_temperature_two_equals_doubled_weight_bitwise(tiny, dev):
    """z * 2 is exact and z(2 w) = 2 z(w) exactly in fp32 too."""
    c = tiny.case
    w2 = synth.f32_exact_to_bf16_bits(2.0 * synth.bf16_bits_to_f32(c.weight))
    a = _ex(tiny.hidden, tiny.weight, tiny.targets, 2.0, False, True)
    b = _ex(tiny.hidden, to_dev_bf16(w2, dev), tiny.targets, 1.0, False, True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(_bits(x), _bits(y))


def _dense_grid(T=64, H=4096, V=4096, seed=4242):
    """h in {0, 1} 2^-4 (density 0.9), w in {-1, 0, 1} 2^-4 (0.05 / 0.1 /
    0.85): every logit is an integer multiple of 2^-8 near 11.5 that needs
    about 12 significant bits, exact in fp32, so the bf16 rounding changes
    almost every logit and both sides decide it on the same value."""
    rng = np.random.Generator(np.random.PCG64(seed))
    h = (rng.random((T, H)) < 0.9).astype(np.float32) / 16
    w = rng.choice(np.array([-1.0, 0.0, 1.0], np.float32), size=(V, H),
                   p=[0.05, 0.1, 0.85]) / 16
    y = rng.integers(0, V, size=T).astype(np.int32)
    return synth.f32_exact_to_bf16_bits(h), synth.f32_exact_to_bf16_bits(w), y


@pytest.mark.parametrize("inv_tau", [1.0, 0.5])
def test_bf16_logits_exact_on_dense_grid(dev, inv_tau):
    hb, wb, y = _dense_grid()
    lp, lse, ent = _np(*_ex(to_dev_bf16(hb, dev), to_dev_bf16(wb, dev), to_dev_i32(y, dev),
                            inv_tau, True, True))
    r_lp, r_lse, r_ent = orc.selected_logp_ex(hb, wb, y, inv_tau, True)
    _close(lp, r_lp, "dense grid bf16 logp", 1e-4)
    _close(lse, r_lse, "dense grid bf16 lse", 1e-4)
    _close(ent, r_ent, "dense grid bf16 entropy", 1e-4)
    n_lp, _, _ = orc.selected_logp_ex(hb, wb, y, inv_tau, False)
    assert np.abs(n_lp - r_lp).max() > 1e-2      # the rounding changes results


@pytest.mark.parametrize("inv_tau", [1.0, 0.5])
def test_bf16_logits_exact_on_grid(adversarial, inv_tau):
    """Coarse grid (zero, dominant and duplicate rows): exact fp32 sums, no
    slack; most of these logits are already bf16 values."""
    c = adversarial.case
    lp, lse, ent = _np(*_ex(adversarial.hidden, adversarial.weight, adversarial.targets,
                            inv_tau, True, True))
    rows = ADV_ROWS
    r_lp, r_lse, r_ent = orc.selected_logp_ex(c.hidden[rows], c.weight, c.targets[rows],
                                              inv_tau, True)
    _close(lp[rows], r_lp, "grid bf16 logp")
    _close(lse[rows], r_lse, "grid bf16 lse")
    _close(ent[rows], r_ent, "grid bf16 entropy")


@pytest.mark.parametrize("inv_tau", [1.0, 0.7])
def test_bf16_logits_random(tiny, inv_tau):
    c = tiny.case
    lp, lse, ent = _np(*_ex(tiny.hidden, tiny.weight, tiny.targets, inv_tau, True, True))
    r_lp, r_lse, r_ent = orc.selected_logp_ex(c.hidden, c.weight, c.targets, inv_tau, True)
    s_lp, s_lse, s_ent, near = _bf16_slack(c.hidden, c.weight, c.targets, inv_tau)
    print(f"bf16 mode: {near.mean() * 100:.3f} % of logits within the fp32 bound of a "
          f"rounding midpoint; target slack on {int((s_lp > s_lse).sum())} rows", flush=True)
    _close(lp, r_lp, "bf16 logp", TOL + s_lp)
    _close(lse, r_lse, "bf16 lse", TOL + s_lse)
    _close(ent, r_ent, "bf16 entropy", TOL + s_ent)


def test_entropy_prefill_sampled_rows(prefill, dev):
    c = prefill.case
    rows = np.array([0, 1, 255, 256, 2047, 4095], dtype=np.int64)
    lp, lse, ent = _np(*_ex(prefill.hidden, prefill.weight, prefill.targets, 0.9, False, True))
    r_lp, r_lse, r_ent = orc.selected_logp_ex(c.hidden[rows], c.weight, c.targets[rows],
                                              0.9, False)
    _close(lp[rows], r_lp, "prefill logp 1/tau=0.9")
    _close(lse[rows], r_lse, "prefill lse 1/tau=0.9")
    _close(ent[rows], r_ent, "prefill entropy 1/tau=0.9")


def test_entropy_adversarial_rows(adversarial):
    """Zero rows (uniform: entropy log V), dominant rows (entropy ~ 0) and
    duplicated rows (equal bits)."""
    c = adversarial.case
    lp, lse, ent = _np(*_ex(adversarial.hidden, adversarial.weight, adversarial.targets))
    rows = ADV_ROWS
    r_lp, r_lse, r_ent = orc.selected_logp_ex(c.hidden[rows], c.weight, c.targets[rows],
                                              1.0, False)
    _close(ent[rows], r_ent, "adversarial entropy")
    assert np.abs(ent[:16] - math.log(c.V)).max() < 1e-4
    assert np.array_equal(ent[32:64].view(np.uint64), ent[64:96].view(np.uint64))


def test_entropy_nonfinite_rows(tiny, dev):
    c = tiny.case
    hid = c.hidden.copy()
    hid[3, 10] = 0x7FC0      # NaN
    hid[5, 20] = 0x7F80      # +Inf
    lp, lse, ent = _np(*_ex(to_dev_bf16(hid, dev), tiny.weight, tiny.targets, 0.7, True, True))
    assert np.isnan(ent[3]) and np.isnan(ent[5])
    clean = _np(*_ex(tiny.hidden, tiny.weight, tiny.targets, 0.7, True, True))[2]
    others = [t for t in range(c.T) if t not in (3, 5)]
    assert np.array_equal(ent[others].view(np.uint64), clean[others].view(np.uint64))
    # all logits -inf: lse -inf, entropy NaN
    H, V = 64, 300
    w = np.zeros((V, H), np.float32)
    w[:, 0] = 0.5
    h = np.zeros((1, H), np.float32)
    h[0, 0] = -np.inf
    lp, lse, ent = _np(*_ex(to_dev_bf16(synth.f32_to_bf16_bits(h), dev),
                            to_dev_bf16(synth.f32_to_bf16_bits(w), dev),
                            to_dev_i32(np.array([4], np.int32), dev), 0.7, False, True))
    assert lse[0] == -np.inf and np.isnan(ent[0]) and np.isnan(lp[0])


# ------------------------------------------------------------- invariance ---

OPTS = [(0.7, False, True), (1.0, True, True), (1.0 / 0.6, True, False)]


@pytest.mark.parametrize("inv_tau,bf16,ent", OPTS)
def test_options_batch_one_vs_batch(tiny, inv_tau, bf16, ent):
    full = _ex(tiny.hidden, tiny.weight, tiny.targets, inv_tau, bf16, ent)
    for t in (0, 17, 63):
        one = _ex(tiny.hidden[t:t + 1], tiny.weight, tiny.targets[t:t + 1], inv_tau, bf16, ent)
        for a, b in zip(full, one):
            if a is not None:
                assert torch.equal(_bits(a[t:t + 1]), _bits(b))


@pytest.mark.parametrize("inv_tau,bf16,ent", OPTS[:2])
def test_options_prefill_packed_vs_per_sequence(prefill, inv_tau, bf16, ent):
    full = _ex(prefill.hidden, prefill.weight, prefill.targets, inv_tau, bf16, ent)
    for s in range(8):
        sl = slice(512 * s, 512 * (s + 1))
        part = _ex(prefill.hidden[sl], prefill.weight, prefill.targets[sl], inv_tau, bf16, ent)
        for a, b in zip(full, part):
            if a is not None:
                assert torch.equal(_bits(a[sl]), _bits(b))


def test_options_vocab_slices_merge_to_unsliced_bits(prefill):
    c = prefill.case
    T, V = c.T, c.V
    flags = rlk.RLK_LOGITS_BF16 | rlk.RLK_ENTROPY
    full = _ex(prefill.hidden, prefill.weight, prefill.targets, 0.7, True, True)
    ws = torch.empty(rlk.rlk_workspace_bytes_ex(T, V, flags), dtype=torch.uint8,
                     device=prefill.hidden.device)
    ws.fill_(0xFF)
    cols = (V + 255) // 256
    cuts = [0] + [round(i * cols / 4) * 256 for i in range(1, 4)] + [V]
    for a, b in zip(cuts[:-1], cuts[1:]):
        rlk.rlk_vocab_stats_ex(prefill.hidden, prefill.weight[a:b], prefill.targets, ws, V, a,
                               inv_temperature=0.7, logits_bf16=True, entropy=True)
    part = rlk.rlk_vocab_merge_ex(prefill.targets, ws, V, logits_bf16=True, entropy=True)
    for a, b in zip(full, part):
        assert torch.equal(_bits(a), _bits(b))


@pytest.mark.parametrize("rows", [1, 16, 32, 33, 200, 256])
def test_options_small_batches_match_the_full_batch(prefill, rows):
    """Decode-size batches (one token tile, mostly padding) against the same
    rows inside the 4096-row batch: same bits, options on."""
    full = _ex(prefill.hidden, prefill.weight, prefill.targets, 0.7, True, True)
    part = _ex(prefill.hidden[:rows], prefill.weight, prefill.targets[:rows], 0.7, True, True)
    for a, b in zip(full, part):
        assert torch.equal(_bits(a[:rows]), _bits(b))
