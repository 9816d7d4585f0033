"""Pins for the oracle's top-k log-probabilities.

Checked against numpy's stable argsort of scipy's log_softmax (an
independent selection and normalisation), hand-worked rows with ties (the
smaller id first), k equal to the vocabulary size (the whole sorted
log-softmax), the consistency of the entry at the target with the oracle's
selected-token logp, NaN entries never selected, and fewer finite entries
than k.
"""

import numpy as np
import pytest
import scipy.special

from invariant_selected_token_amd import synth
from oracle import oracle as orc


def _ref(z, k):
    ls = scipy.special.log_softmax(z, axis=1)
    order = np.argsort(-ls, axis=1, kind="stable")[:, :k]   # stable: ties keep id order
    return np.take_along_axis(ls, order, 1), order


@pytest.mark.parametrize("k", [1, 5, 20])
def test_matches_argsort_of_log_softmax(k):
    rng = np.random.Generator(np.random.PCG64(41))
    z = rng.normal(0, 2, size=(7, 300))
    lp, ids = orc.topk_from_logits(z, k)
    rlp, rids = _ref(z, k)
    assert np.array_equal(ids, rids)
    np.testing.assert_allclose(lp, rlp, rtol=0, atol=1e-12)


def test_ties_go_to_the_smaller_id():
    z = np.array([[0.5, 2.0, 2.0, -1.0, 2.0, 0.5]])
    lp, ids = orc.topk_from_logits(z, 5)
    assert ids[0].tolist() == [1, 2, 4, 0, 5]
    assert lp[0, 0] == lp[0, 1] == lp[0, 2]
    lse = np.log(3 * np.exp(2.0) + 2 * np.exp(0.5) + np.exp(-1.0))
    assert abs(lp[0, 0] - (2.0 - lse)) < 1e-14


def test_k_equal_to_vocabulary_is_the_sorted_log_softmax():
    c = synth.tiny_case()
    lp, ids = orc.topk_logp(c.hidden[:3], c.weight[:50], 50)
    ls = orc.log_softmax(c.hidden[:3], c.weight[:50])
    for t in range(3):
        assert sorted(ids[t].tolist()) == list(range(50))
        np.testing.assert_allclose(lp[t], ls[t, ids[t]], rtol=0, atol=1e-14)
        assert np.all(np.diff(lp[t]) <= 0)
    np.testing.assert_allclose(np.exp(lp).sum(1), 1.0, rtol=0, atol=1e-12)


def test_entry_at_the_target_equals_selected_logp_and_options():
    c = synth.tiny_case()
    for inv_tau, bf16 in [(1.0, False), (0.7, True)]:
        lp, ids = orc.topk_logp(c.hidden, c.weight, 8, inv_tau, bf16)
        sel, _, _ = orc.selected_logp_ex(c.hidden, c.weight, ids[:, 3].copy(), inv_tau, bf16)
        np.testing.assert_array_equal(lp[:, 3], sel)


def test_nan_never_selected_and_short_rows():
    z = np.array([[np.nan, 1.0, -np.inf, 0.0], [-np.inf, -np.inf, 3.0, -np.inf]])
    lp, ids = orc.topk_from_logits(z, 3)
    assert ids[0].tolist() == [1, 3, 2]        # NaN skipped; lse is NaN for that row
    assert np.all(np.isnan(lp[0]))
    assert ids[1].tolist() == [2, 0, 1] and lp[1, 0] == 0.0 and lp[1, 1] == -np.inf
    lp2, ids2 = orc.topk_from_logits(z[:1], 4)
    assert ids2[0, 3] == -1 and lp2[0, 3] == -np.inf
