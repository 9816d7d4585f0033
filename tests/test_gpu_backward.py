"""GPU parity and invariance of the backward (rlk_selected_logp_backward,
rlk_logp_grad_logits) against the fp64 oracle.

Tolerance, from the arithmetic of the HIP path: dz is formed in fp32 and
rounded to bf16 (relative error <= 2^-9; 2^-8 allowed), then contracted with
fp32 accumulation over K terms (error <= K 2^-24 of the sum of absolute
terms).  So per output element

    |grad - oracle| <= (2^-8 + (K + 16) 2^-24) * (|dz| |w|)  (grad_hidden, K = V)
                       (2^-8 + (K + 16) 2^-24) * (|dz|^T |h|) (grad_weight, K = T)

plus 1e-6 |g| for the fp32 exponent and lse.  Gross mistakes (sign, missing
softmax term, transposed operand, missing temperature) are O(1) of the same
scale.  The tests print the fraction of that bound actually used.
"""

import numpy as np
import pytest

import invariant_selected_token_amd as rlk
from invariant_selected_token_amd import synth
from oracle import oracle as orc

from conftest import to_dev_bf16, to_dev_i32

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def _grads_dev(g, dev):
    return torch.from_numpy(np.ascontiguousarray(g, dtype=np.float32)).to(dev)


def _upstream(T, seed):
    return np.random.Generator(np.random.PCG64(seed)).normal(size=T).astype(np.float32)


def _run(h, w, y, g, inv_tau=1.0, want_hidden=True, want_weight=True):
    _, lse, _ = rlk.rlk_selected_logp_ex(h, w, y, inv_temperature=inv_tau)
    gh, gw = rlk.rlk_selected_logp_backward(h, w, y, lse, g, inv_temperature=inv_tau,
                                            want_hidden=want_hidden, want_weight=want_weight)
    torch.cuda.synchronize()
    return lse, gh, gw


def _check(got, ref, bound, what):
    err = np.abs(got.astype(np.float64) - ref)
    assert np.isfinite(got).all(), what
    ratio = (err / np.maximum(bound, 1e-300)).max()
    rel = err.max() / max(np.abs(ref).max(), 1e-300)
    print(f"{what}: max |err| {err.max():.3e} (rel to max |ref| {rel:.2e}), "
          f"{ratio:.3f} of the bound", flush=True)
    assert (err <= bound).all(), f"{what}: max |err| {err.max()} exceeds the bound"


def _bounds(hidden, weight, y, g, inv_tau, rows_h=None):
    dz = orc.grad_logits(hidden, weight, y, g.astype(np.float64), inv_tau)
    ad = np.abs(dz)
    T, V = dz.shape
    bh = (2.0 ** -8 + (V + 16) * 2.0 ** -24) * (ad @ np.abs(_f64(weight))) \
        + 1e-6 * np.abs(g)[:, None]
    bw = (2.0 ** -8 + (T + 16) * 2.0 ** -24) * (ad.T @ np.abs(_f64(hidden))) + 1e-6
    return dz, bh, bw


# ------------------------------------------------------------------ stage ---

@pytest.mark.parametrize("inv_tau", [1.0, 0.7])
def test_grad_logits_stage(tiny, dev, inv_tau):
    c = tiny.case
    g = _upstream(c.T, 11)
    _, lse, _ = rlk.rlk_selected_logp_ex(tiny.hidden, tiny.weight, tiny.targets,
                                         inv_temperature=inv_tau)
    dz = rlk.rlk_logp_grad_logits(tiny.hidden, tiny.weight, tiny.targets, lse,
                                  _grads_dev(g, dev), inv_temperature=inv_tau)
    torch.cuda.synchronize()
    got = dz.float().cpu().numpy().astype(np.float64)
    ref = orc.grad_logits(c.hidden, c.weight, c.targets, g.astype(np.float64), inv_tau)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-6 * np.abs(g)[:, None]
    _check(got[:, :c.V], ref, bound, f"dz 1/tau={inv_tau}")
    assert np.array_equal(np.sign(got[:, :c.V]) * (np.abs(ref) > 1e-30),
                          np.sign(ref) * (np.abs(ref) > 1e-30))


# ---------------------------------------------------------------- parity ----

@pytest.mark.parametrize("inv_tau", [1.0, 0.7])
def test_backward_tiny(tiny, dev, inv_tau):
    c = tiny.case
    g = _upstream(c.T, 12)
    _, gh, gw = _run(tiny.hidden, tiny.weight, tiny.targets, _grads_dev(g, dev), inv_tau)
    rh, rw = orc.selected_logp_backward(c.hidden, c.weight, c.targets, g.astype(np.float64),
                                        inv_tau)
    _, bh, bw = _bounds(c.hidden, c.weight, c.targets, g, inv_tau)
    _check(gh.cpu().numpy(), rh, bh, f"grad_hidden 1/tau={inv_tau}")
    _check(gw.cpu().numpy(), rw, bw, f"grad_weight 1/tau={inv_tau}")


@pytest.mark.parametrize("T,H,V", [(1, 64, 5), (70, 192, 1000), (300, 64, 257),
                                   (513, 128, 4133)])
def test_backward_ragged(dev, T, H, V):
    c = synth.normal_case(f"bwd_{T}x{H}x{V}", 700 + T, T, H, V, weight_std=0.1)
    g = _upstream(T, 13 + T)
    h, w, y = to_dev_bf16(c.hidden, dev), to_dev_bf16(c.weight, dev), to_dev_i32(c.targets, dev)
    _, gh, gw = _run(h, w, y, _grads_dev(g, dev), 0.9)
    rh, rw = orc.selected_logp_backward(c.hidden, c.weight, c.targets, g.astype(np.float64),
                                        0.9)
    _, bh, bw = _bounds(c.hidden, c.weight, c.targets, g, 0.9)
    _check(gh.cpu().numpy(), rh, bh, f"grad_hidden {T}x{H}x{V}")
    _check(gw.cpu().numpy(), rw, bw, f"grad_weight {T}x{H}x{V}")


@pytest.mark.parametrize("T,H,V", [(70, 192, 1000), (1, 64, 5), (300, 64, 257)])
def test_grad_weight_stays_in_bounds(dev, T, H, V):
    """grad_weight's tiles are stored transposed, as 16-byte pieces of its rows,
    through a range-checked resource per 32 rows (rows past V and columns past
    H dropped): written into the middle of a sentinel-filled buffer, the floats
    around it keep the sentinel and the values equal a plain output's bits."""
    c = synth.normal_case(f"bwd_bounds_{T}x{H}x{V}", 900 + T, T, H, V, weight_std=0.1)
    g = _grads_dev(_upstream(T, 31 + T), dev)
    h, w, y = to_dev_bf16(c.hidden, dev), to_dev_bf16(c.weight, dev), to_dev_i32(c.targets, dev)
    lse, _, gw_ref = _run(h, w, y, g, 0.9, want_hidden=False)
    pad = 1024   # floats on each side (4 KiB: keeps the output 16-byte aligned)
    sentinel = -7.25
    buf = torch.full((V * H + 2 * pad,), sentinel, dtype=torch.float32, device=dev)
    gw = buf[pad:pad + V * H].view(V, H)
    _, got = rlk.rlk_selected_logp_backward(h, w, y, lse, g, inv_temperature=0.9,
                                            want_hidden=False, grad_weight=gw)
    torch.cuda.synchronize()
    assert torch.all(buf[:pad] == sentinel) and torch.all(buf[pad + V * H:] == sentinel)
    assert torch.equal(got.view(torch.int32), gw_ref.view(torch.int32))


def test_grad_weight_must_be_16_byte_aligned(tiny, dev):
    """Its rows leave as 16-byte pieces: a 4-byte-aligned grad_weight is refused
    before any launch (RLK_ERR_MISALIGNED, raised by the binding)."""
    h, w, y = tiny.hidden, tiny.weight, tiny.targets
    T, H, V = h.shape[0], h.shape[1], w.shape[0]
    _, lse, _ = rlk.rlk_selected_logp_ex(h, w, y)
    g = torch.ones(T, dtype=torch.float32, device=dev)
    buf = torch.zeros(V * H + 1, dtype=torch.float32, device=dev)
    with pytest.raises(RuntimeError, match="misaligned"):
        rlk.rlk_selected_logp_backward(h, w, y, lse, g, want_hidden=False,
                                       grad_weight=buf[1:].view(V, H))
    torch.cuda.synchronize()


@pytest.mark.parametrize("T,H,V", [(70, 192, 1000), (300, 128, 4133)])
def test_backward_strided_operands_same_bits(dev, T, H, V):
    """hidden and weight as views into wider rows whose extra columns hold NaN:
    the row strides reach the hidden-row transpose, the dz pass and both
    products' K-major reads, and the gradients keep the contiguous call's bits
    (any read of a padding column would bring a NaN in)."""
    c = synth.normal_case(f"bwd_strided_{T}x{H}x{V}", 950 + T, T, H, V, weight_std=0.1)
    g = _grads_dev(_upstream(T, 41 + T), dev)
    h, w, y = to_dev_bf16(c.hidden, dev), to_dev_bf16(c.weight, dev), to_dev_i32(c.targets, dev)
    _, gh, gw = _run(h, w, y, g, 0.8)
    hb = torch.full((T, H + 64), float("nan"), dtype=h.dtype, device=dev)
    wb = torch.full((V, H + 128), float("nan"), dtype=w.dtype, device=dev)
    hb[:, :H] = h
    wb[:, :H] = w
    _, gh2, gw2 = _run(hb[:, :H], wb[:, :H], y, g, 0.8)
    assert torch.equal(gh.view(torch.int32), gh2.view(torch.int32)), "grad_hidden"
    assert torch.equal(gw.view(torch.int32), gw2.view(torch.int32)), "grad_weight"


def test_backward_medium_full_grad_weight(dev):
    """A bigger vocabulary and depth: T=512, H=1024, V=8192."""
    c = synth.normal_case("bwd_medium", 4321, 512, 1024, 8192)
    g = _upstream(512, 14)
    h, w, y = to_dev_bf16(c.hidden, dev), to_dev_bf16(c.weight, dev), to_dev_i32(c.targets, dev)
    _, gh, gw = _run(h, w, y, _grads_dev(g, dev))
    rh, rw = orc.selected_logp_backward(c.hidden, c.weight, c.targets, g.astype(np.float64))
    _, bh, bw = _bounds(c.hidden, c.weight, c.targets, g, 1.0)
    _check(gh.cpu().numpy(), rh, bh, "grad_hidden medium")
    _check(gw.cpu().numpy(), rw, bw, "grad_weight medium")


def test_backward_prefill_sampled_hidden_rows(prefill, dev):
    """Full Qwen3-8B shape; grad_hidden on sampled rows against the oracle,
    grad_weight finite everywhere."""
    c = prefill.case
    g = _upstream(c.T, 15)
    _, gh, gw = _run(prefill.hidden, prefill.weight, prefill.targets, _grads_dev(g, dev))
    rows = np.array([0, 255, 256, 2048, 4095])
    rh, _ = orc.selected_logp_backward(c.hidden[rows], c.weight, c.targets[rows],
                                       g[rows].astype(np.float64), want_weight=False)
    dz = orc.grad_logits(c.hidden[rows], c.weight, c.targets[rows], g[rows].astype(np.float64))
    bh = (2.0 ** -8 + (c.V + 16) * 2.0 ** -24) * (np.abs(dz) @ np.abs(_f64(c.weight))) \
        + 1e-6 * np.abs(g[rows])[:, None]
    _check(gh.cpu().numpy()[rows], rh, bh, "prefill grad_hidden rows")
    assert bool(torch.isfinite(gw).all())


# ------------------------------------------------------------- invariance ---

def _bits(x):
    return x.contiguous().view(torch.int32)


def test_grad_hidden_batch_invariant(tiny, dev):
    c = tiny.case
    g = _grads_dev(_upstream(c.T, 16), dev)
    _, gh, _ = _run(tiny.hidden, tiny.weight, tiny.targets, g, 0.8, want_weight=False)
    for t in (0, 31, 63):
        _, g1, _ = _run(tiny.hidden[t:t + 1], tiny.weight, tiny.targets[t:t + 1], g[t:t + 1],
                        0.8, want_weight=False)
        assert torch.equal(_bits(gh[t:t + 1]), _bits(g1))


def test_grad_hidden_packed_vs_per_sequence(prefill, dev):
    g = _grads_dev(_upstream(prefill.case.T, 17), dev)
    _, gh, _ = _run(prefill.hidden, prefill.weight, prefill.targets, g, want_weight=False)
    for s in (0, 3, 7):
        sl = slice(512 * s, 512 * (s + 1))
        _, part, _ = _run(prefill.hidden[sl], prefill.weight, prefill.targets[sl], g[sl],
                          want_weight=False)
        assert torch.equal(_bits(gh[sl]), _bits(part))


def test_grad_weight_repeatable_and_zero_rows_appended(prefill, dev):
    """Same rows -> same bits; appending rows with g = 0 or an ignored target
    adds exact zeros at the end of every sum -> same bits."""
    c = prefill.case
    g = _grads_dev(_upstream(c.T, 18), dev)
    _, gh_a, gw_a = _run(prefill.hidden, prefill.weight, prefill.targets, g)
    _, gh_b, gw_b = _run(prefill.hidden, prefill.weight, prefill.targets, g)
    assert torch.equal(_bits(gw_a), _bits(gw_b)) and torch.equal(_bits(gh_a), _bits(gh_b))
    extra = 100
    h2 = torch.cat([prefill.hidden, prefill.hidden[:extra]])
    y2 = torch.cat([prefill.targets, prefill.targets[:extra]])
    y2[c.T + extra // 2:] = -1                       # ignored targets
    g2 = torch.cat([g, torch.zeros(extra, dtype=torch.float32, device=dev)])
    g2[c.T + extra // 2:] = 1.0                      # nonzero g, but ignored rows
    _, gh_c, gw_c = _run(h2, prefill.weight, y2, g2)
    assert torch.equal(_bits(gw_a), _bits(gw_c))
    assert torch.equal(_bits(gh_a), _bits(gh_c[:c.T]))
    assert not bool(gh_c[c.T:].any())


def test_inverse_temperature_two_equals_doubled_weight(tiny, dev):
    c = tiny.case
    g = _grads_dev(_upstream(c.T, 19), dev)
    w2 = to_dev_bf16(synth.f32_exact_to_bf16_bits(2.0 * synth.bf16_bits_to_f32(c.weight)), dev)
    _, gh_a, gw_a = _run(tiny.hidden, tiny.weight, tiny.targets, g, 2.0)
    _, gh_b, gw_b = _run(tiny.hidden, w2, tiny.targets, g, 1.0)
    assert torch.equal(_bits(gh_a), _bits(gh_b))
    assert torch.equal(_bits(gw_a), _bits(2.0 * gw_b))


def test_ignored_rows_and_zero_batch(tiny, dev):
    c = tiny.case
    y = c.targets.copy()
    y[[2, 40]] = [-1, c.V]
    g = _upstream(c.T, 20)
    _, gh, gw = _run(tiny.hidden, tiny.weight, to_dev_i32(y, dev), _grads_dev(g, dev))
    assert not bool(gh[[2, 40]].any())
    rh, rw = orc.selected_logp_backward(c.hidden, c.weight, y, g.astype(np.float64))
    _, bh, bw = _bounds(c.hidden, c.weight, y, g, 1.0)
    _check(gw.cpu().numpy(), rw, bw, "grad_weight with ignored rows")
    # T == 0: grad_weight is zero-filled
    gw0 = torch.full((c.V, c.hidden.shape[1]), 7.0, device=dev)
    empty = torch.empty(0, dtype=torch.float32, device=dev)
    rlk.rlk_selected_logp_backward(tiny.hidden[:0], tiny.weight, tiny.targets[:0], empty, empty,
                                   want_hidden=False, grad_weight=gw0)
    torch.cuda.synchronize()
    assert not bool(gw0.any())
