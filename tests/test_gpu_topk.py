"""GPU parity and invariance of the top-k log-probabilities.

Several answers are correct where values tie within the fp32 / fp64
difference, so the test compares what is unique and checks the rest is
valid: every returned (id, value) matches the oracle's log-softmax at that
id within 1e-3, ids are distinct and values non-increasing, and no id left
out has an oracle value above the k-th returned one by more than 2e-3.  The
entry at a row's target equals that row's logp bit for bit (same logits,
same subtraction), and a row's result does not depend on its batch.
"""

import numpy as np
import pytest
import scipy.special

import invariant_selected_token_amd as rlk
from invariant_selected_token_amd import synth
from oracle import oracle as orc

from conftest import to_dev_bf16, to_dev_i32

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _check_valid(tl, ti, ls, k, what, tol=1e-3):
    T = tl.shape[0]
    for t in range(T):
        ids = ti[t]
        assert len(set(ids.tolist())) == k, f"{what}: duplicate ids in row {t}"
        assert np.all(np.diff(tl[t]) <= 0), f"{what}: not decreasing in row {t}"
        assert np.abs(tl[t] - ls[t, ids]).max() <= tol, f"{what}: value off in row {t}"
        rest = np.ones(ls.shape[1], bool)
        rest[ids] = False
        if rest.any():
            assert ls[t, rest].max() <= ls[t, ids].min() + 2 * tol, f"{what}: missed an entry"


def _run(h, w, y, k, inv_tau=1.0, bf16=False):
    lp, lse, tl, ti = rlk.topk_logprobs(h, w, y, k, inv_temperature=inv_tau, logits_bf16=bf16)
    torch.cuda.synchronize()
    return lp, lse, tl, ti


@pytest.mark.parametrize("k", [1, 5, 20, 64])
def test_topk_tiny(tiny, k):
    c = tiny.case
    lp, lse, tl, ti = _run(tiny.hidden, tiny.weight, tiny.targets, k)
    ls = orc.log_softmax(c.hidden, c.weight)
    tl, ti = tl.cpu().numpy().astype(np.float64), ti.cpu().numpy()
    _check_valid(tl, ti, ls, k, f"tiny k={k}")
    rlp, rids = orc.topk_logp(c.hidden, c.weight, k)
    # where the oracle's consecutive values are well separated the ids agree
    sep = np.abs(np.diff(np.concatenate([rlp, np.full((c.T, 1), -np.inf)], 1), axis=1)) > 1e-4
    assert np.array_equal(ti[sep], rids[sep])


@pytest.mark.parametrize("inv_tau,bf16", [(0.7, False), (1.0, True)])
def test_topk_options_and_target_entry_bitwise(tiny, inv_tau, bf16):
    c = tiny.case
    lp, lse, tl, ti = _run(tiny.hidden, tiny.weight, tiny.targets, 8, inv_tau, bf16)
    zs = orc.logits(c.hidden, c.weight) * inv_tau
    if bf16:
        zs = orc.round_bf16(zs.astype(np.float32))
    ls = scipy.special.log_softmax(zs, axis=1)
    # bf16 mode: a logit near a rounding midpoint may round the other way on
    # the kernel's fp32 value, moving it by one bf16 step (< 0.01 here)
    tol = 0.01 if bf16 else 1e-3
    _check_valid(tl.cpu().numpy().astype(np.float64), ti.cpu().numpy(), ls, 8,
                 f"1/tau={inv_tau} bf16={bf16}", tol)
    # the entry at any returned id is that id's logp, bit for bit
    lp2, _, _ = rlk.rlk_selected_logp_ex(tiny.hidden, tiny.weight, ti[:, 2].contiguous(),
                                         inv_temperature=inv_tau, logits_bf16=bf16)
    torch.cuda.synchronize()
    assert torch.equal(lp2.view(torch.int32), tl[:, 2].contiguous().view(torch.int32))
    tl_np, ti_np, lp_np = tl.cpu().numpy(), ti.cpu().numpy(), lp.cpu().numpy()
    for t in range(c.T):
        hit = np.flatnonzero(ti_np[t] == c.targets[t])
        if hit.size:
            assert tl_np[t, hit[0]].view(np.uint32) == lp_np[t].view(np.uint32)


def test_topk_prefill_sampled_rows_and_batch_invariance(prefill):
    c = prefill.case
    lp, lse, tl, ti = _run(prefill.hidden[:1024], prefill.weight, prefill.targets[:1024], 20)
    rows = np.array([0, 255, 256, 1023])
    ls = orc.log_softmax(c.hidden[rows], c.weight)
    _check_valid(tl.cpu().numpy()[rows].astype(np.float64), ti.cpu().numpy()[rows], ls, 20,
                 "prefill rows")
    _, _, tl1, ti1 = _run(prefill.hidden[256:257], prefill.weight, prefill.targets[256:257], 20)
    assert torch.equal(tl1.view(torch.int32), tl[256:257].view(torch.int32))
    assert torch.equal(ti1, ti[256:257])


def test_topk_ties_nan_and_short_rows(dev):
    """Grid logits with many exact ties (smaller id first), a row of NaN
    logits, and k = V."""
    H, V = 64, 40
    w = np.zeros((V, H), np.float32)
    w[:, 0] = np.repeat(np.array([1.0, 0.5, -0.5, 0.25], np.float32), 10)
    h = np.zeros((3, H), np.float32)
    h[0, 0] = 1.0
    h[1, 0] = np.nan
    h[2, 0] = -2.0
    hb, wb = synth.f32_to_bf16_bits(h), synth.f32_to_bf16_bits(w)
    y = np.zeros(3, np.int32)
    lp, lse, tl, ti = _run(to_dev_bf16(hb, dev), to_dev_bf16(wb, dev), to_dev_i32(y, dev), V)
    rlp, rids = orc.topk_logp(hb, wb, V)
    ti_np = ti.cpu().numpy()
    assert np.array_equal(ti_np[[0, 2]], rids[[0, 2]])       # exact ties: ids in order
    np.testing.assert_allclose(tl.cpu().numpy()[[0, 2]], rlp[[0, 2]], rtol=0, atol=1e-5)
    # every logit of row 1 is NaN: nothing can be selected, so all k entries
    # are the short-row filler (id -1, -inf), as in the oracle
    assert np.array_equal(ti_np[1], rids[1]) and np.all(ti_np[1] == -1)
    assert np.all(tl.cpu().numpy()[1] == -np.inf)


@pytest.mark.parametrize("k", [17, 25, 33])
def test_topk_boundary_inside_a_tie_group(dev, k):
    """Groups of 10 exactly equal logits with the k-th place inside a group:
    the smaller ids of that group are taken, as in the oracle (k >= 17 takes
    the bisection path)."""
    H, V = 64, 40
    w = np.zeros((V, H), np.float32)
    w[:, 0] = np.repeat(np.array([1.0, 0.5, -0.5, 0.25], np.float32), 10)
    h = np.zeros((2, H), np.float32)
    h[0, 0] = 1.0
    h[1, 0] = -2.0
    hb, wb = synth.f32_to_bf16_bits(h), synth.f32_to_bf16_bits(w)
    y = np.zeros(2, np.int32)
    lp, lse, tl, ti = _run(to_dev_bf16(hb, dev), to_dev_bf16(wb, dev), to_dev_i32(y, dev), k)
    rlp, rids = orc.topk_logp(hb, wb, k)
    assert np.array_equal(ti.cpu().numpy(), rids)
    np.testing.assert_allclose(tl.cpu().numpy(), rlp, rtol=0, atol=1e-5)


def test_topk_tie_cut_at_ids_above_2_pow_25(dev):
    """The tie cut at the k-th value bisects over the token ids; ids of a
    vocabulary past 2^25 need its 26th bit.  Logits given directly (the
    store kernel stops at V = 2^24): row t of V = 2^25 + 4096 entries holds 30
    tied maxima 1.0 at ids 2^25 .. 2^25 + 29 and, in every other 128-wide
    tile j, the value -1 - j 1e-6; so the candidate tiles are that tile and
    tiles 0 .. 18 (20 tiles: the bisection path at k = 20) and the answer is
    ids 2^25 .. 2^25 + 19, each with the value 1.0 - lse."""
    T, V, k = 2, 2 ** 25 + 4096, 20
    nst = V // 128
    tile = torch.arange(nst, device=dev, dtype=torch.float32)
    z = (-1.0 - tile * 1e-6).repeat_interleave(128).unsqueeze(0).repeat(T, 1).contiguous()
    a = 2 ** 25
    z[:, a:a + 128] = -5.0
    z[:, a:a + 30] = 1.0
    lse = torch.logsumexp(z, dim=1).contiguous()
    part_m = z.view(T, nst, 128).amax(dim=2).t().contiguous()     # [nST][T], tile-major
    ws = torch.zeros((nst * T + 64,), dtype=torch.float32, device=dev)
    ws[:nst * T] = part_m.view(-1)
    tl, ti = rlk.rlk_topk_logp(z, lse, ws, k)
    torch.cuda.synchronize()
    want_ids = torch.arange(a, a + k, dtype=torch.int32, device=dev).unsqueeze(0).repeat(T, 1)
    assert torch.equal(ti, want_ids), ti[:, :k].tolist()
    want_v = (1.0 - lse).unsqueeze(1).expand(T, k)
    assert torch.equal(tl.view(torch.int32), want_v.contiguous().view(torch.int32))
    del z
