"""GPU parity: the HIP path against the fp64 CPU oracle, through the C ABI.

Tolerance: |logp - oracle| <= 1e-3 and |lse - oracle| <= 1e-3 per row, the
bound the design fixes for this path (fp32 accumulation over H <= 4096 with
logits of O(1) magnitude stays orders of magnitude below it).  NaN must meet
NaN.  Where floating point is exact (grid inputs), the logits must match the
oracle bit for bit.
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


def _run(h, w, y):
    lp, lse = rlk.rlk_selected_logp(h, w, y)
    torch.cuda.synchronize()
    return lp.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _assert_close(got, ref, what):
    both_nan = np.isnan(got) & np.isnan(ref)
    assert np.array_equal(np.isnan(got), np.isnan(ref)), f"{what}: NaN pattern differs"
    d = np.where(both_nan, 0.0, np.abs(got - ref))
    d = np.where(np.isinf(got) & (got == ref), 0.0, d)
    print(f"{what}: max |diff| = {d.max():.3e} over {d.size} rows", flush=True)
    assert d.max() <= TOL, f"{what}: max |diff| {d.max()} > {TOL}"


def test_tiny_all_rows(tiny):
    c = tiny.case
    lp, lse = _run(tiny.hidden, tiny.weight, tiny.targets)
    ref_lp, ref_lse = orc.selected_logp(c.hidden, c.weight, c.targets)
    _assert_close(lp, ref_lp, "tiny logp")
    _assert_close(lse, ref_lse, "tiny lse")
    assert np.all(lp <= 0.0)


RAGGED = [
    # (T, H, V): tails in every dimension, single rows, sub-tile vocabularies
    (1, 64, 1), (1, 64, 5), (3, 128, 127), (7, 64, 128), (255, 256, 129),
    (256, 256, 256), (257, 64, 257), (300, 192, 1000), (513, 128, 4133),
    (70, 4096, 3000), (600, 64, 640),
    # partly filled tiles whose last live row group is partly (65) or wholly
    # (64, 128) filled, with odd K-block counts
    (64, 128, 769), (65, 64, 1031), (128, 320, 2000),
]


@pytest.mark.parametrize("T,H,V", RAGGED)
def test_ragged_shapes(dev, T, H, V):
    c = synth.normal_case(f"ragged_{T}_{H}_{V}", 4000 + T + V, T, H, V,
                          hidden_std=1.0, weight_std=0.1)
    h, w, y = to_dev_bf16(c.hidden, dev), to_dev_bf16(c.weight, dev), to_dev_i32(c.targets, dev)
    lp, lse = _run(h, w, y)
    ref_lp, ref_lse = orc.selected_logp(c.hidden, c.weight, c.targets)
    _assert_close(lp, ref_lp, f"T={T} H={H} V={V} logp")
    _assert_close(lse, ref_lse, f"T={T} H={H} V={V} lse")
    # the logits stage against the fp64 logits, with the worst-case fp32
    # summation bound H * 2^-24 * sum_k |h_k w_k| (plus one rounding)
    z = rlk.rlk_logits(h, w)
    torch.cuda.synchronize()
    zg = z.cpu().numpy().astype(np.float64)
    zo = orc.logits(c.hidden, c.weight)
    habs = np.abs(synth.bf16_bits_to_f32(c.hidden).astype(np.float64))
    wabs = np.abs(synth.bf16_bits_to_f32(c.weight).astype(np.float64))
    bound = (H + 1) * 2.0 ** -24 * (habs @ wabs.T)
    assert np.all(np.abs(zg - zo) <= bound + 1e-30)


@pytest.mark.parametrize("T,V", [(300, 1000), (257, 4133), (70, 3000), (1, 5), (600, 640)])
def test_logits_store_paths_agree_and_stay_in_bounds(dev, T, V):
    """The logits land at any 4-byte aligned address: a 16-byte aligned view
    with V a multiple of 4 takes the 16-byte stores, a view one float further
    on the one-column stores.  Both hold the same bits, and the floats around
    each view (rows past T and columns past V are dropped, not redirected)
    keep their sentinel."""
    H = 128
    c = synth.normal_case(f"store_{T}_{V}", 4100 + T + V, T, H, V,
                          hidden_std=1.0, weight_std=0.1)
    h, w = to_dev_bf16(c.hidden, dev), to_dev_bf16(c.weight, dev)
    n = T * V
    got = []
    for start in (4, 1):          # 16-byte aligned, then 4-byte aligned
        buf = torch.full((n + 8 + 64,), -7.25, dtype=torch.float32, device=dev)
        view = buf[start:start + n].view(T, V)
        rlk.rlk_logits(h, w, logits=view)
        torch.cuda.synchronize()
        b = buf.cpu().numpy()
        assert np.all(b[:start] == -7.25) and np.all(b[start + n:] == -7.25), start
        got.append(b[start:start + n].reshape(T, V).copy())
    assert np.array_equal(got[0].view(np.uint32), got[1].view(np.uint32))
    zo = orc.logits(c.hidden, c.weight)
    habs = np.abs(synth.bf16_bits_to_f32(c.hidden).astype(np.float64))
    wabs = np.abs(synth.bf16_bits_to_f32(c.weight).astype(np.float64))
    bound = (H + 1) * 2.0 ** -24 * (habs @ wabs.T)
    assert np.all(np.abs(got[0].astype(np.float64) - zo) <= bound + 1e-30)


def test_strided_operands(dev):
    """Row strides larger than H (views into wider buffers)."""
    c = synth.normal_case("strided", 77, 40, 128, 700, weight_std=0.1)
    hb = np.zeros((40, 200), np.uint16)
    hb[:, :128] = c.hidden
    wb = np.zeros((700, 136), np.uint16)
    wb[:, :128] = c.weight
    h = to_dev_bf16(hb, dev)[:, :128]
    w = to_dev_bf16(wb, dev)[:, :128]
    lp, lse = _run(h, w, to_dev_i32(c.targets, dev))
    ref_lp, ref_lse = orc.selected_logp(c.hidden, c.weight, c.targets)
    _assert_close(lp, ref_lp, "strided logp")
    _assert_close(lse, ref_lse, "strided lse")


def test_padded_vocabulary_rows_are_left_out(dev):
    """V smaller than weight's row count: rows >= V take no part."""
    c = synth.normal_case("padded", 78, 33, 128, 1000, weight_std=0.1)
    h, w = to_dev_bf16(c.hidden, dev), to_dev_bf16(c.weight, dev)
    y = np.minimum(c.targets, 899).astype(np.int32)
    lp, lse = rlk.rlk_selected_logp(h, w, to_dev_i32(y, dev), V=900)
    torch.cuda.synchronize()
    ref_lp, ref_lse = orc.selected_logp(c.hidden, c.weight[:900], y)
    _assert_close(lp.cpu().numpy().astype(np.float64), ref_lp, "padded logp")
    _assert_close(lse.cpu().numpy().astype(np.float64), ref_lse, "padded lse")


PREFILL_SAMPLE = [0, 1, 31, 32, 127, 128, 255, 256, 257, 511, 512, 1023, 2047,
                  2048, 3071, 4094, 4095]


def test_prefill_full_size_sampled_rows(prefill):
    """T=4096, H=4096, V=151936 in the benchmark's launch configuration."""
    c = prefill.case
    lp, lse = _run(prefill.hidden, prefill.weight, prefill.targets)
    rng = np.random.Generator(np.random.PCG64(99))
    rows = np.unique(np.concatenate([PREFILL_SAMPLE, rng.choice(c.T, 31, replace=False)]))
    ref_lp, ref_lse = orc.selected_logp(c.hidden[rows], c.weight, c.targets[rows])
    _assert_close(lp[rows], ref_lp, "prefill logp")
    _assert_close(lse[rows], ref_lse, "prefill lse")
    # properties that hold on every row: finite, logp <= 0 (the target's
    # logit is one of the summed terms and the max term contributes exactly 1)
    assert np.all(np.isfinite(lp)) and np.all(np.isfinite(lse))
    assert np.all(lp <= 0.0)


def test_adversarial_grid(adversarial, dev):
    """Coarse grid: exact logits, exact ties, all-equal and dominant rows."""
    a = adversarial
    c = a.case
    lp, lse = _run(a.hidden, a.weight, a.targets)
    rows = np.array([0, 5, 15, 16, 20, 23, 24, 31, 32, 40, 63, 64, 72, 95, 96,
                     500, 1023])
    # exact logits: every partial sum is a multiple of 2^-8 below 2^8
    z = rlk.rlk_logits(a.hidden[rows.tolist()], a.weight)
    torch.cuda.synchronize()
    zo = orc.logits(c.hidden[rows], c.weight)
    assert np.array_equal(z.cpu().numpy().astype(np.float64), zo)
    ref_lp, ref_lse = orc.selected_logp(c.hidden[rows], c.weight, c.targets[rows])
    _assert_close(lp[rows], ref_lp, "adversarial logp")
    _assert_close(lse[rows], ref_lse, "adversarial lse")
    # all-equal rows: lse = log V, logp = -log V
    assert np.all(np.abs(lse[0:16] - math.log(c.V)) <= 1e-5)
    assert np.all(np.abs(lp[0:16] + math.log(c.V)) <= 1e-5)
    # dominant rows targeting v*: logp in [-V e^-gap, 0]
    assert np.all(lp[16:24] <= 0.0) and np.all(lp[16:24] >= -1e-3)
    # duplicated hidden rows share lse bit for bit
    lse32 = lse.astype(np.float32)
    assert np.array_equal(lse32[32:64].view(np.uint32), lse32[64:96].view(np.uint32))
    assert np.all(lp <= 0.0)


def test_large_logit_no_overflow(dev):
    """A +100 logit (e^100 > FLT_MAX) on a grid weight: lse ~ 100, no inf."""
    H, V = 4096, 2048
    rng = np.random.Generator(np.random.PCG64(31))
    wi = rng.integers(-1, 2, size=(V, H))
    vstar = 777
    nz = np.flatnonzero(wi[vstar])[:1280]
    hi = np.zeros((2, H))
    hi[0, nz] = np.sign(wi[vstar, nz]) * 1.25
    hidden = synth.f32_exact_to_bf16_bits(hi.astype(np.float32))
    weight = synth.f32_exact_to_bf16_bits((wi / 16).astype(np.float32))
    y = np.array([vstar, 3], np.int32)
    lp, lse = _run(to_dev_bf16(hidden, dev), to_dev_bf16(weight, dev), to_dev_i32(y, dev))
    ref_lp, ref_lse = orc.selected_logp(hidden, weight, y)
    assert ref_lse[0] >= 100.0 and np.all(np.isfinite(lse))
    _assert_close(lp, ref_lp, "+100 logp")
    _assert_close(lse, ref_lse, "+100 lse")


def test_nonfinite_and_out_of_range_rows(tiny, dev):
    c = tiny.case
    hid = c.hidden.copy()
    hid[3, 10] = 0x7FC0      # NaN
    hid[5, 20] = 0x7F80      # +Inf
    y = c.targets.copy()
    y[7] = -1
    y[9] = c.V
    clean_lp, clean_lse = rlk.rlk_selected_logp(tiny.hidden, tiny.weight, tiny.targets)
    lp, lse = rlk.rlk_selected_logp(to_dev_bf16(hid, dev), tiny.weight, to_dev_i32(y, dev))
    torch.cuda.synchronize()
    lp, lse = lp.cpu().numpy(), lse.cpu().numpy()
    clean_lp, clean_lse = clean_lp.cpu().numpy(), clean_lse.cpu().numpy()
    ref_lp, ref_lse = orc.selected_logp(hid, c.weight, y)
    for r in (3, 5):
        assert np.isnan(lp[r]) and np.isnan(lse[r]) and np.isnan(ref_lp[r])
    for r in (7, 9):
        assert np.isnan(lp[r]) and np.isnan(ref_lp[r])
        assert lse[r].view(np.uint32) == clean_lse[r].view(np.uint32)
    others = [t for t in range(c.T) if t not in (3, 5, 7, 9)]
    assert np.array_equal(lp[others].view(np.uint32), clean_lp[others].view(np.uint32))
    assert np.array_equal(lse[others].view(np.uint32), clean_lse[others].view(np.uint32))


def test_all_minus_inf_row(dev):
    """hidden = -Inf at k=0 with w[:, 0] > 0: every logit -Inf -> lse -Inf, logp NaN."""
    H, V = 64, 300
    w = np.zeros((V, H), np.float32)
    w[:, 0] = 0.5
    w[:, 1] = np.linspace(-1, 1, V).astype(np.float32)
    h = np.zeros((2, H), np.float32)
    h[0, 0] = -np.inf
    h[1, 1] = 2.0
    hb = synth.f32_to_bf16_bits(h)
    wb = synth.f32_to_bf16_bits(w)
    y = np.array([4, 4], np.int32)
    lp, lse = _run(to_dev_bf16(hb, dev), to_dev_bf16(wb, dev), to_dev_i32(y, dev))
    ref_lp, ref_lse = orc.selected_logp(hb, wb, y)
    assert lse[0] == -np.inf and ref_lse[0] == -np.inf
    assert np.isnan(lp[0]) and np.isnan(ref_lp[0])
    _assert_close(lp[1:], ref_lp[1:], "finite row logp")


def test_compare_kernel_matches_oracle_stats(dev):
    rng = np.random.Generator(np.random.PCG64(8))
    n = 5000
    b = (rng.standard_normal(n) * 3 - 5).astype(np.float32)
    a = b.copy()
    idx = rng.choice(n, 700, replace=False)
    a[idx] = a[idx] + (rng.standard_normal(700) * 1e-3).astype(np.float32)

    def both(x, y):
        st = rlk.consistency_report(rlk.rlk_compare(torch.from_numpy(x).to(dev),
                                                    torch.from_numpy(y).to(dev)))
        return st, orc.compare_stats(x, y)

    st, ref = both(a, b)
    assert st["n"] == ref["n"]
    assert st["mismatch_count"] == ref["mismatch_count"]
    assert st["max_abs_diff"] == ref["max_abs_diff"]
    for k in ("mean_abs_diff", "k3_mean"):
        assert st[k] == pytest.approx(ref[k], rel=1e-9, abs=1e-15)
    assert st["std_abs_diff"] == pytest.approx(ref["std_abs_diff"], rel=1e-6)
    # special values: NaN on both sides (equal bits), NaN on one side (+inf
    # difference), -0 vs +0 (a mismatch of size 0), equal infinities
    a2, b2 = a.copy(), b.copy()
    a2[10], b2[10] = np.nan, np.nan
    a2[11] = np.nan
    a2[12], b2[12] = -0.0, 0.0
    a2[13], b2[13] = -np.inf, -np.inf
    st, ref = both(a2, b2)
    assert st["mismatch_count"] == ref["mismatch_count"]
    assert st["max_abs_diff"] == ref["max_abs_diff"] == np.inf
    assert st["k3_mean"] == pytest.approx(ref["k3_mean"], rel=1e-9, abs=1e-15)
    # a vs itself: zero everything
    t = torch.from_numpy(b).to(dev)
    st0 = rlk.consistency_report(rlk.rlk_compare(t, t))
    assert st0["mismatch_count"] == 0 and st0["max_abs_diff"] == 0.0


def test_long_rollout_softmax_targets(rollout, dev):
    """T=16384 (32 responses x 512): sampled rows get targets drawn from the
    oracle's own softmax (inverse CDF with one seeded uniform per row); the
    other rows keep uniform targets, which cannot affect the sampled rows."""
    c = rollout.case
    rng = np.random.Generator(np.random.PCG64(77))
    rows = np.unique(np.concatenate([[0, 255, 256, 511, 8191, 8192, 16383],
                                     rng.choice(c.T, 25, replace=False)]))
    ls = orc.log_softmax(c.hidden[rows], c.weight)
    y = c.targets.copy()
    y[rows] = orc.sample_targets(ls, c.meta["u"][rows])
    lp, lse = _run(rollout.hidden, rollout.weight, to_dev_i32(y, dev))
    ref_lp, ref_lse = orc.selected_logp(c.hidden[rows], c.weight, y[rows])
    np.testing.assert_allclose(ref_lp, ls[np.arange(rows.size), y[rows]], rtol=0, atol=1e-12)
    _assert_close(lp[rows], ref_lp, "rollout logp")
    _assert_close(lse[rows], ref_lse, "rollout lse")
    assert np.all(np.isfinite(lp)) and np.all(lp <= 0.0)


@pytest.mark.parametrize("T,H,V", [(3, 65536, 300), (4, 64, 1_000_003), (70_000, 64, 300)])
def test_maximum_sizes(dev, T, H, V):
    """The limits of the contract: H at its maximum (1024 K blocks), a vocabulary
    of a million rows (7813 statistics tiles, ragged last tile), 70 000 rows
    (274 token tiles); every row against the oracle, targets including 0 and
    V - 1."""
    c = synth.normal_case(f"max_{T}x{H}x{V}", 880 + T % 97, T, H, V)
    y = c.targets.copy()
    y[0], y[-1] = 0, V - 1
    lp, lse = _run(to_dev_bf16(c.hidden, dev), to_dev_bf16(c.weight, dev), to_dev_i32(y, dev))
    ref_lp, ref_lse = orc.selected_logp(c.hidden, c.weight, y)
    _assert_close(lp, ref_lp, f"logp {T}x{H}x{V}")
    _assert_close(lse, ref_lse, f"lse {T}x{H}x{V}")


@pytest.mark.parametrize("V", [163_840, 163_841, 200_000])
def test_merge_register_limit(dev, V):
    """The merge holds a row's group of statistics tiles in registers while the
    group has at most 80 tiles (16 groups: V <= 163 840) and reads them in
    chunks beyond that; both must fold to the oracle's lse, logp and entropy,
    and the rows with and without the entropy partials must share their bits."""
    T, H = 40, 64
    c = synth.normal_case(f"merge_limit_{V}", 771 + V % 1000, T, H, V)
    y = c.targets.copy()
    y[0], y[1] = 0, V - 1
    h, w, yd = to_dev_bf16(c.hidden, dev), to_dev_bf16(c.weight, dev), to_dev_i32(y, dev)
    lp, lse = _run(h, w, yd)
    lp2, lse2, ent = rlk.rlk_selected_logp_ex(h, w, yd, inv_temperature=0.9, entropy=True)
    lp1, lse1, _ = rlk.rlk_selected_logp_ex(h, w, yd, inv_temperature=0.9, entropy=False)
    torch.cuda.synchronize()
    ref_lp, ref_lse = orc.selected_logp(c.hidden, c.weight, y)
    _assert_close(lp, ref_lp, f"V={V} logp")
    _assert_close(lse, ref_lse, f"V={V} lse")
    rlp, rlse, rent = orc.selected_logp_ex(c.hidden, c.weight, y, inv_tau=0.9)
    _assert_close(lp2.cpu().numpy().astype(np.float64), rlp, f"V={V} logp tau")
    _assert_close(lse2.cpu().numpy().astype(np.float64), rlse, f"V={V} lse tau")
    _assert_close(ent.cpu().numpy().astype(np.float64), rent, f"V={V} entropy")
    assert torch.equal(lp1.view(torch.int32), lp2.view(torch.int32))
    assert torch.equal(lse1.view(torch.int32), lse2.view(torch.int32))


def test_empty_batches_through_every_entry_point(tiny, dev):
    """T = 0: every call returns empty results (grad_weight zero-filled)."""
    h0, y0 = tiny.hidden[:0], tiny.targets[:0]
    lp, lse = rlk.rlk_selected_logp(h0, tiny.weight, y0)
    assert lp.shape == (0,) and lse.shape == (0,)
    lp, lse, ent = rlk.rlk_selected_logp_ex(h0, tiny.weight, y0, inv_temperature=0.5,
                                            logits_bf16=True, entropy=True)
    assert ent.shape == (0,)
    z = rlk.rlk_logits(h0, tiny.weight)
    assert z.shape == (0, tiny.case.V)
    e = torch.empty(0, dtype=torch.float32, device=dev)
    gh, gw = rlk.rlk_selected_logp_backward(h0, tiny.weight, y0, e, e)
    torch.cuda.synchronize()
    assert gh.shape == (0, tiny.case.H) and not bool(gw.any())
    assert rlk.rlk_rmsnorm(h0, tiny.weight[0], 1e-6).shape == (0, tiny.case.H)
    ws = rlk.workspace_for(1, tiny.case.V, dev)
    tl, ti = rlk.rlk_topk_logp(z, e, ws, 5)
    assert tl.shape == (0, 5) and ti.shape == (0, 5)


def test_single_entry_vocabulary_with_options(dev):
    """V = 1: lse = z, logp = 0, entropy = 0, top-1 is that entry."""
    c = synth.normal_case("v1", 4, 5, 64, 1)
    h, w = to_dev_bf16(c.hidden, dev), to_dev_bf16(c.weight, dev)
    y = to_dev_i32(np.zeros(5, np.int32), dev)
    lp, lse, ent = rlk.rlk_selected_logp_ex(h, w, y, inv_temperature=0.7, entropy=True)
    torch.cuda.synchronize()
    assert bool((lp == 0).all()) and bool((ent == 0).all())
    z = orc.logits(c.hidden, c.weight)[:, 0] * 0.7
    assert np.abs(lse.cpu().numpy() - z).max() <= 1e-5
    lp2, lse2, tl, ti = rlk.topk_logprobs(h, w, y, 1, inv_temperature=0.7)
    assert bool((ti == 0).all()) and bool((tl == 0).all())
