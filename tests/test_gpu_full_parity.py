"""Every row of the full-size workloads against the fp64 oracle, through the
C ABI, in the benchmark's launch configuration.

The oracle's values for the Qwen3-8B-shaped workloads (4096 prefill rows,
1024 coarse-grid rows, 16384 long-rollout rows with targets drawn from the
oracle's own softmax) take minutes of CPU time, so they are stored in
tests/golden/full_size_oracle.npz by tests/golden/make_full_oracle.py, which
calls only the oracle and the seeded generators; each workload's stored
values carry a fingerprint of the input bytes, and a test whose regenerated
inputs do not match the fingerprint fails rather than compare against values
of other inputs.

Tolerance: |logp - oracle| <= 1e-3 and |lse - oracle| <= 1e-3 on every row
(and the entropy with the options), NaN meeting NaN; on the coarse grid the
logits are exact in any summation order, so their per-row integer checksums
must equal the oracle's exactly.  The definition is the RL-Kernel blog's
section 四 (Linear LogP: the selected token's logit minus the vocabulary LSE).
"""

import math
import os

import numpy as np
import pytest

import invariant_selected_token_amd as rlk
from invariant_selected_token_amd import synth
from oracle import oracle as orc

from conftest import to_dev_bf16, to_dev_i32

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

TOL = 1e-3
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "full_size_oracle.npz")


@pytest.fixture(scope="module")
def golden():
    with np.load(GOLDEN, allow_pickle=False) as d:
        return {k: d[k] for k in d.files}


def _fingerprint_ok(golden, key, case, targets=None):
    got = synth.fingerprint(case, targets)
    assert str(golden[key]) == got, (
        f"{key}: the stored oracle values are for other inputs ({golden[key]} != {got}); "
        "rerun tests/golden/make_full_oracle.py")


def _np(x):
    return x.cpu().numpy().astype(np.float64)


def _assert_close(got, ref, what, tol=TOL):
    assert got.shape == ref.shape, what
    assert np.array_equal(np.isnan(got), np.isnan(ref)), f"{what}: NaN pattern differs"
    d = np.where(np.isnan(got) & np.isnan(ref), 0.0, np.abs(got - ref))
    print(f"{what}: max |diff| = {d.max():.3e} over all {d.size} rows", flush=True)
    assert d.max() <= tol, f"{what}: max |diff| {d.max()} > {tol} at row {int(d.argmax())}"


def _bench_call(dc, targets=None, V=None):
    """The two stages exactly as the benchmark times them."""
    T, V = dc.hidden.shape[0], int(dc.weight.shape[0] if V is None else V)
    y = dc.targets if targets is None else targets
    ws = rlk.workspace_for(T, V, dc.hidden.device)
    rlk.rlk_vocab_stats(dc.hidden, dc.weight, y, ws)
    lp, lse = rlk.rlk_vocab_merge(y, ws, V)
    torch.cuda.synchronize()
    return lp, lse


def test_prefill_topk_every_row(prefill, golden):
    """The top 20 log-probabilities of all 4096 prefill rows (the path that
    recomputes the candidate tiles) against the oracle's top 32: the values
    rank by rank within 1e-3; the same id wherever the oracle's value at that
    rank stands more than 2e-3 from both neighbours (closer values may swap
    within fp32 rounding); and every returned id among the oracle's top 32,
    with its value within 1e-3 of the oracle's for that id."""
    _fingerprint_ok(golden, "prefill_fingerprint", prefill.case)
    k = 20
    _, _, tl, ti = rlk.topk_logprobs(prefill.hidden, prefill.weight, prefill.targets, k)
    torch.cuda.synchronize()
    tl, ti = _np(tl), ti.cpu().numpy()
    ol, oi = golden["prefill_topk_logp"], golden["prefill_topk_ids"]
    T = tl.shape[0]
    _assert_close(tl, ol[:, :k], "prefill top-20 values by rank")
    d = ol[:, :-1] - ol[:, 1:]                        # >= 0, ranks r and r + 1
    before = np.concatenate([np.full((T, 1), np.inf), d[:, :k - 1]], axis=1)
    sep = (before > 2e-3) & (d[:, :k] > 2e-3)
    print(f"prefill top-20: {int(sep.sum())} of {sep.size} ranks separated", flush=True)
    assert np.array_equal(ti[sep], oi[:, :k][sep]), "an id differs at a separated rank"
    match = ti[:, :, None] == oi[:, None, :]           # [T, k, 32]
    assert match.any(axis=2).all(), "a returned id is not among the oracle's top 32"
    ov = np.where(match, ol[:, None, :], 0.0).sum(axis=2)
    assert np.abs(tl - ov).max() <= TOL, "a returned id's value is off the oracle's"


def test_prefill_every_row(prefill, golden):
    """T = 4096 packed rows (8 x 512), H = 4096, V = 151936: all 4096 rows."""
    _fingerprint_ok(golden, "prefill_fingerprint", prefill.case)
    lp, lse = _bench_call(prefill)
    _assert_close(_np(lp), golden["prefill_logp"], "prefill logp")
    _assert_close(_np(lse), golden["prefill_lse"], "prefill lse")
    assert bool((lp <= 0).all())


def test_decode_batches_every_row(prefill, golden):
    """The decode sweep (batches of 1 .. 256 rows from the 256-vector pool at
    random positions): every row of every batch against the oracle."""
    plan = synth.decode_plan(prefill_T=prefill.case.T)
    dev = prefill.hidden.device
    pool = plan["pool"]
    for B, slots in plan["batches"].items():
        rows = pool[slots]
        idx = torch.from_numpy(rows).to(dev)
        lp, lse = rlk.rlk_selected_logp(prefill.hidden[idx].contiguous(), prefill.weight,
                                        prefill.targets[idx].contiguous())
        torch.cuda.synchronize()
        _assert_close(_np(lp), golden["prefill_logp"][rows], f"decode B={B} logp")
        _assert_close(_np(lse), golden["prefill_lse"][rows], f"decode B={B} lse")


def test_prefill_options_every_row(prefill, golden):
    """Inverse temperature 0.7 with the entropy, all 4096 rows."""
    _fingerprint_ok(golden, "prefill_fingerprint", prefill.case)
    inv_tau = float(golden["prefill_opt_inv_tau"])
    lp, lse, ent = rlk.rlk_selected_logp_ex(prefill.hidden, prefill.weight, prefill.targets,
                                            inv_temperature=inv_tau, entropy=True)
    torch.cuda.synchronize()
    _assert_close(_np(lp), golden["prefill_opt_logp"], "prefill 1/tau=0.7 logp")
    _assert_close(_np(lse), golden["prefill_opt_lse"], "prefill 1/tau=0.7 lse")
    _assert_close(_np(ent), golden["prefill_opt_entropy"], "prefill 1/tau=0.7 entropy")


def test_adversarial_every_row(adversarial, golden):
    """The coarse grid (T = 1024): logp and lse on every row; the logits of
    every row exact (integer checksums of 256 z equal to the oracle's)."""
    a = adversarial
    c = a.case
    _fingerprint_ok(golden, "adversarial_fingerprint", c)
    lp, lse = _bench_call(a)
    lp, lse = _np(lp), _np(lse)
    _assert_close(lp, golden["adversarial_logp"], "adversarial logp")
    _assert_close(lse, golden["adversarial_lse"], "adversarial lse")
    # closed forms: all-equal rows give lse = log V, logp = -log V
    assert np.all(np.abs(lse[0:16] - math.log(c.V)) <= 1e-5)
    assert np.all(np.abs(lp[0:16] + math.log(c.V)) <= 1e-5)
    dev = a.hidden.device
    w = torch.arange(1, c.V + 1, dtype=torch.int64, device=dev)
    sums = np.empty((c.T, 3), np.int64)
    for r0 in range(0, c.T, 128):
        z = rlk.rlk_debug_logits(a.hidden[r0:r0 + 128], a.weight)
        q = z.double() * 256.0
        qi = torch.round(q).to(torch.int64)
        assert bool((qi.double() == q).all()), f"rows {r0}..: a logit off the 2^-8 grid"
        sums[r0:r0 + 128, 0] = qi.sum(dim=1).cpu().numpy()
        sums[r0:r0 + 128, 1] = (qi * qi).sum(dim=1).cpu().numpy()
        sums[r0:r0 + 128, 2] = (qi * w).sum(dim=1).cpu().numpy()
        del z, q, qi
    bad = np.flatnonzero((sums != golden["adversarial_logit_sums"]).any(axis=1))
    assert bad.size == 0, f"exact logits differ from the oracle's on rows {bad[:10]}"


def _bits_equal(a, b, what):
    st = rlk.consistency_report(rlk.rlk_compare(a.contiguous(), b.contiguous()))
    print(f"{what}: mismatch_count={st['mismatch_count']} "
          f"max_abs_diff={st['max_abs_diff']:.3e}", flush=True)
    assert st["mismatch_count"] == 0 and st["max_abs_diff"] == 0.0, what


def test_adversarial_invariance(adversarial):
    """Ties, all-equal, dominant and duplicated rows: bitwise the same when
    run alone, in sub-batches at other positions, permuted, and repeated 100
    times (RL-Kernel blog, section 五: bitwise, not a tolerance)."""
    a = adversarial
    T = a.case.T
    dev = a.hidden.device
    lp, lse = rlk.rlk_selected_logp(a.hidden, a.weight, a.targets)
    # batch 1: the structured rows and some grid rows
    rows = list(range(0, 96, 3)) + [15, 16, 23, 24, 31, 32, 63, 64, 95, 96, 500, 1023]
    for t in rows:
        x, s = rlk.rlk_selected_logp(a.hidden[t:t + 1], a.weight, a.targets[t:t + 1])
        _bits_equal(x, lp[t:t + 1], f"adversarial batch-1 row {t} logp")
        _bits_equal(s, lse[t:t + 1], f"adversarial batch-1 row {t} lse")
    # sub-batches at other positions, ragged tile tails included
    for n, shift in ((1, 600), (64, 3), (128, 900), (255, 17), (256, 1), (257, 700)):
        idx = (torch.arange(n, device=dev) + shift) % T
        x, s = rlk.rlk_selected_logp(a.hidden[idx].contiguous(), a.weight,
                                     a.targets[idx].contiguous())
        _bits_equal(x, lp[idx], f"adversarial T={n} logp")
        _bits_equal(s, lse[idx], f"adversarial T={n} lse")
    rng = np.random.Generator(np.random.PCG64(41))
    for _ in range(3):
        p = torch.from_numpy(rng.permutation(T)).to(dev)
        x, s = rlk.rlk_selected_logp(a.hidden[p].contiguous(), a.weight,
                                     a.targets[p].contiguous())
        _bits_equal(x, lp[p], "adversarial permuted logp")
        _bits_equal(s, lse[p], "adversarial permuted lse")
    stats = torch.zeros((100, 2, 8), dtype=torch.float64, device=dev)
    x = torch.empty_like(lp)
    s = torch.empty_like(lse)
    for i in range(100):
        rlk.rlk_selected_logp(a.hidden, a.weight, a.targets, logp=x, lse=s)
        rlk.rlk_compare(x, lp, stats=stats[i, 0])
        rlk.rlk_compare(s, lse, stats=stats[i, 1])
    st = stats.cpu().numpy()
    print(f"adversarial 100 repeats: mismatches {st[:, :, 1].sum()}", flush=True)
    assert st[:, :, 1].sum() == 0 and st[:, :, 2].max() == 0.0


def test_rollout_every_row(rollout, golden):
    """T = 16384 rows (32 x 512) with targets drawn from the oracle's own
    softmax: all rows."""
    c = rollout.case
    y = golden["rollout_targets"]
    _fingerprint_ok(golden, "rollout_fingerprint", c, y)
    yd = to_dev_i32(y, rollout.hidden.device)
    lp, lse = _bench_call(rollout, targets=yd)
    _assert_close(_np(lp), golden["rollout_logp"], "rollout logp")
    _assert_close(_np(lse), golden["rollout_lse"], "rollout lse")
    # the sampled targets are likely tokens: their logp is far above uniform
    assert float(np.median(golden["rollout_logp"])) > -math.log(c.V)


def test_prefill_grad_weight_rows(prefill, golden):
    """The backward at the full prefill shape: 24 rows of grad_weight (targets
    of some row, nobody's target, tile edges) against the oracle within the
    backward's bound, and grad_hidden on 16 rows against the oracle."""
    c = prefill.case
    _fingerprint_ok(golden, "prefill_fingerprint", c)
    g = synth.upstream_grad(c.T, int(golden["prefill_gw_seed"]))
    dev = prefill.hidden.device
    gd = torch.from_numpy(g).to(dev)
    _, lse = rlk.rlk_selected_logp(prefill.hidden, prefill.weight, prefill.targets)
    gh, gw = rlk.rlk_selected_logp_backward(prefill.hidden, prefill.weight, prefill.targets,
                                            lse, gd)
    torch.cuda.synchronize()
    rows = golden["prefill_gw_rows"]
    got = gw[torch.from_numpy(rows).to(dev)].cpu().numpy().astype(np.float64)
    err = np.abs(got - golden["prefill_gw"])
    bound = golden["prefill_gw_bound"].astype(np.float64)
    print(f"prefill grad_weight rows: max |err| {err.max():.3e}, "
          f"{(err / bound).max():.3f} of the bound", flush=True)
    assert np.isfinite(got).all() and (err <= bound).all()
    assert bool(torch.isfinite(gw).all()) and bool(torch.isfinite(gh).all())
    hrows = np.array([0, 1, 255, 256, 511, 512, 1000, 2047, 2048, 3000, 3071, 3072, 4000,
                      4093, 4094, 4095])
    rh, _ = orc.selected_logp_backward(c.hidden[hrows], c.weight, c.targets[hrows],
                                       g[hrows].astype(np.float64), want_weight=False)
    dz = orc.grad_logits(c.hidden[hrows], c.weight, c.targets[hrows], g[hrows].astype(np.float64))
    wabs = np.abs(synth.bf16_bits_to_f32(c.weight).astype(np.float64))
    bh = (2.0 ** -8 + (c.V + 16) * 2.0 ** -24) * (np.abs(dz) @ wabs) \
        + 1e-6 * np.abs(g[hrows])[:, None]
    errh = np.abs(gh.cpu().numpy()[hrows].astype(np.float64) - rh)
    print(f"prefill grad_hidden rows: {(errh / bh).max():.3f} of the bound", flush=True)
    assert (errh <= bh).all()


# -------------------------------------------- vocabulary slices vs the oracle

def _tp_cuts(V, P):
    cols = (V + 255) // 256
    return [0] + [round(i * cols / P) * 256 for i in range(1, P)] + [V]


def _sliced(dc, cuts, V):
    T = dc.hidden.shape[0]
    ws = rlk.workspace_for(T, V, dc.hidden.device)
    ws.fill_(0xFF)
    for a, b in zip(cuts[:-1], cuts[1:]):
        rlk.rlk_vocab_stats_shard(dc.hidden, dc.weight[a:b], dc.targets, ws, V, a)
    lp, lse = rlk.rlk_vocab_merge(dc.targets, ws, V)
    torch.cuda.synchronize()
    return lp, lse


@pytest.mark.parametrize("P", [2, 3, 8])
def test_vocab_slices_against_oracle_small(dev, P):
    """Statistics of P vocabulary slices merged once, against the oracle: the
    tiny workload and a ragged one (V not a multiple of 256, T not of 256)."""
    for case in (synth.tiny_case(), synth.normal_case("slices_ragged", 321, 300, 192, 4133,
                                                       weight_std=0.1)):

        class D:
            hidden = to_dev_bf16(case.hidden, dev)
            weight = to_dev_bf16(case.weight, dev)
            targets = to_dev_i32(case.targets, dev)

        lp, lse = _sliced(D, _tp_cuts(case.V, P), case.V)
        ref_lp, ref_lse = orc.selected_logp(case.hidden, case.weight, case.targets)
        _assert_close(_np(lp), ref_lp, f"{case.name} {P} slices logp")
        _assert_close(_np(lse), ref_lse, f"{case.name} {P} slices lse")


def test_vocab_slices_against_oracle_prefill(prefill, golden):
    """Four tensor-parallel slices of the Qwen3-8B head, every row."""
    _fingerprint_ok(golden, "prefill_fingerprint", prefill.case)
    lp, lse = _sliced(prefill, _tp_cuts(prefill.case.V, 4), prefill.case.V)
    _assert_close(_np(lp), golden["prefill_logp"], "prefill 4 slices logp")
    _assert_close(_np(lse), golden["prefill_lse"], "prefill 4 slices lse")


def test_tp_exchange_through_the_documented_layout(prefill, golden):
    """Four 'ranks', each with a workspace of its own, compute the statistics
    of their vocabulary shard; the exchange an all-gather would do is done by
    copying, per rank, its contiguous tile rows of part_m and part_s (the
    offsets rlk_workspace_layout documents) and the xt entries of the rows
    whose target it owns into one workspace; one merge then gives the
    unsharded bits and the oracle's values."""
    c = prefill.case
    T, V = c.T, c.V
    dev = prefill.hidden.device
    lay = rlk.rlk_workspace_layout(T, V)
    full_lp, full_lse = rlk.rlk_selected_logp(prefill.hidden, prefill.weight, prefill.targets)
    cuts = _tp_cuts(V, 4)
    merged = rlk.workspace_for(T, V, dev)
    merged.fill_(0xFF)
    f32 = lambda ws, off, n: ws[off:off + 4 * n].view(torch.float32)
    for a, b in zip(cuts[:-1], cuts[1:]):
        own = rlk.workspace_for(T, V, dev)
        own.fill_(0xFF)
        rlk.rlk_vocab_stats_shard(prefill.hidden, prefill.weight[a:b], prefill.targets, own, V, a)
        j0, j1 = a // 128, (b + 127) // 128
        for region in ("part_m", "part_s"):
            lo, hi = lay[region] + 4 * j0 * T, lay[region] + 4 * j1 * T
            merged[lo:hi].copy_(own[lo:hi])
        mine = (prefill.targets >= a) & (prefill.targets < b)
        xt_m, xt_o = f32(merged, lay["xt"], T), f32(own, lay["xt"], T)
        xt_m[mine] = xt_o[mine]
        del own
    lp, lse = rlk.rlk_vocab_merge(prefill.targets, merged, V)
    torch.cuda.synchronize()
    _bits_equal(lp, full_lp, "exchanged shards logp")
    _bits_equal(lse, full_lse, "exchanged shards lse")
    _assert_close(_np(lp), golden["prefill_logp"], "exchanged shards logp vs oracle")
