"""The top-k log-probabilities without stored logits (rlk_topk_logp_direct)
against the same selection over the logits stored whole (rlk_debug_logits +
rlk_topk_logp), bit for bit.

The direct path recomputes only the candidate tiles of each row with the
logit GEMM's MFMA chain, so every returned value and id must equal the stored
path's: the comparison is exact, on ragged vocabularies, an odd number of
64-deep K blocks (the GEMM's appended zero block), the options, rows with many
exactly tied tile maxima (the coarse grid), rows of NaN and infinities, and
the full prefill shape.  The stored path itself is checked against the fp64
oracle in test_gpu_topk.py (which now runs the direct path through
topk_logprobs).
"""

import numpy as np
import pytest

import invariant_selected_token_amd as rlk
from invariant_selected_token_amd import synth

from conftest import to_dev_bf16, to_dev_i32

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _both(h, w, y, k, inv_tau=1.0, bf16=False, dcap=16):
    """(direct logp, direct ids, stored logp, stored ids) for the same rows."""
    T, V = h.shape[0], w.shape[0]
    flags = rlk.RLK_LOGITS_BF16 if bf16 else 0
    ws = rlk.workspace_for(T, V, h.device, flags)
    _, lse, _ = rlk.rlk_selected_logp_ex(h, w, y, inv_temperature=inv_tau, logits_bf16=bf16,
                                         workspace=ws)
    dl, di = rlk.rlk_topk_logp_direct(h, w, lse, ws, k, inv_tau, bf16, max_degenerate_rows=dcap)
    z = rlk.rlk_debug_logits(h, w)
    sl, si = rlk.rlk_topk_logp(z, lse, ws, k, inv_tau, bf16)
    torch.cuda.synchronize()
    del z
    return dl, di, sl, si


def _same(dl, di, sl, si, what):
    assert torch.equal(di, si), f"{what}: ids differ in rows " \
        f"{torch.nonzero((di != si).any(dim=1)).flatten()[:8].tolist()}"
    assert torch.equal(dl.view(torch.int32), sl.view(torch.int32)), f"{what}: values differ"


def _rand(T, H, V, seed, dev, scale=1.0):
    g = np.random.Generator(np.random.PCG64(seed))
    h = synth.f32_to_bf16_bits(g.standard_normal((T, H), dtype=np.float32) * scale)
    w = synth.f32_to_bf16_bits(g.standard_normal((V, H), dtype=np.float32) * 0.02)
    y = g.integers(0, V, T).astype(np.int32)
    return to_dev_bf16(h, dev), to_dev_bf16(w, dev), to_dev_i32(y, dev)


@pytest.mark.parametrize("k", [1, 5, 8, 9, 16, 17, 20, 24, 25, 32, 33, 64])
def test_direct_equals_stored_tiny(tiny, k):
    _same(*_both(tiny.hidden, tiny.weight, tiny.targets, k), f"tiny k={k}")


@pytest.mark.parametrize("T,H,V,k", [
    (300, 256, 1000, 5),     # 8 tiles, ragged last tile
    (300, 256, 1000, 20),    # fewer tiles than k: every tile of every row
    (257, 192, 4095, 20),    # H / 64 odd: the GEMM's appended zero block
    (1, 320, 6000, 64),      # one row, 47 tiles, the largest k
    (130, 128, 16385, 33),   # a one-entry last tile
])
def test_direct_equals_stored_ragged(dev, T, H, V, k):
    h, w, y = _rand(T, H, V, 1000 + T + H + V + k, dev)
    _same(*_both(h, w, y, k), f"T={T} H={H} V={V} k={k}")


@pytest.mark.parametrize("inv_tau,bf16,k", [(0.7, False, 8), (1.0, True, 20), (1.3, True, 64)])
def test_direct_equals_stored_options(tiny, inv_tau, bf16, k):
    _same(*_both(tiny.hidden, tiny.weight, tiny.targets, k, inv_tau, bf16),
          f"1/tau={inv_tau} bf16={bf16} k={k}")


@pytest.mark.parametrize("k", [1, 20, 32, 64])
def test_direct_equals_stored_tied_tile_maxima(dev, k):
    """Coarse-grid operands: logits are multiples of 2^-8 over a small range,
    so many tiles share the same maximum and the first-k-by-index rule for
    the tied tiles decides the candidates."""
    T, H, V = 96, 256, 8192
    g = np.random.Generator(np.random.PCG64(77 + k))
    h = (g.integers(-1, 2, (T, H)) * 0.0625).astype(np.float32)
    w = (g.integers(-1, 2, (V, H)) * 0.0625).astype(np.float32)
    w[:, 8:] = 0.0                       # 8 terms: few distinct logit values
    hb, wb = synth.f32_to_bf16_bits(h), synth.f32_to_bf16_bits(w)
    y = g.integers(0, V, T).astype(np.int32)
    _same(*_both(to_dev_bf16(hb, dev), to_dev_bf16(wb, dev), to_dev_i32(y, dev), k),
          f"tied k={k}")


def _poisoned(dev, V=4096, H=128, T=8):
    """Rows whose k-th largest tile maximum is -inf: a row of NaN, a row
    whose logits are -inf or NaN tile by tile (an infinite hidden value
    against weights of both signs and zeros), a row with -inf logits only
    past its first tile; the other rows ordinary."""
    g = np.random.Generator(np.random.PCG64(5))
    h = g.standard_normal((T, H), dtype=np.float32)
    w = g.standard_normal((V, H), dtype=np.float32) * 0.02
    w[:, 0] = 0.0
    w[256:, 0] = -1.0                       # from row 256 on, h[:, 0] = inf gives -inf
    w[1000:1100, 0] = 0.0                   # ... and NaN (inf * 0) for ids 1000 .. 1099
    h[1, :] = np.nan
    h[3, 0] = np.inf
    h[5, 0] = np.inf
    h[5, 1:] = 0.0
    y = np.zeros(T, np.int32)
    return (to_dev_bf16(synth.f32_to_bf16_bits(h), dev),
            to_dev_bf16(synth.f32_to_bf16_bits(w), dev), to_dev_i32(y, dev))


@pytest.mark.parametrize("k", [4, 20, 40])
def test_direct_equals_stored_poisoned_rows(dev, k):
    h, w, y = _poisoned(dev)
    dl, di, sl, si = _both(h, w, y, k, dcap=8)
    _same(dl, di, sl, si, f"poisoned k={k}")


def test_direct_marks_rows_without_room(dev):
    """With no room for rows whose m* is -inf (and more tiles than k), those
    rows get id -2 and NaN in every place; every other row is untouched."""
    h, w, y = _poisoned(dev)
    k = 4
    dl, di, sl, si = _both(h, w, y, k, dcap=0)
    bad = [1, 3, 5]
    good = [t for t in range(h.shape[0]) if t not in bad]
    assert torch.all(di[bad] == -2) and torch.all(torch.isnan(dl[bad]))
    _same(dl[good], di[good], sl[good], si[good], "rows with room")
    # room for one: the first such row in row order is served
    dl1, di1, _, _ = _both(h, w, y, k, dcap=1)
    _same(dl1[[1]], di1[[1]], sl[[1]], si[[1]], "the served row")
    assert torch.all(di1[[3, 5]] == -2)


def test_direct_repeats_and_batch_invariance(tiny):
    h, w, y = tiny.hidden, tiny.weight, tiny.targets
    dl, di, _, _ = _both(h, w, y, 20)
    for _ in range(3):
        dl2, di2, _, _ = _both(h, w, y, 20)
        _same(dl2, di2, dl, di, "repeat")
    for a, b in [(0, 1), (5, 6), (17, 64)]:
        dl3, di3, _, _ = _both(h[a:b], w, y[a:b], 20)
        _same(dl3, di3, dl[a:b], di[a:b], f"rows {a}:{b} alone")


@pytest.mark.parametrize("k", [20, 64])
def test_direct_equals_stored_prefill(prefill, k):
    """The full prefill shape (T = 4096, H = 4096, V = 151936)."""
    _same(*_both(prefill.hidden, prefill.weight, prefill.targets, k), f"prefill k={k}")


def test_direct_equals_stored_rollout(rollout):
    """The long rollout (T = 16384 packed rows), k = 20 and 64."""
    for k in (20, 64):
        _same(*_both(rollout.hidden, rollout.weight, rollout.targets, k), f"rollout k={k}")


def test_direct_error_paths(tiny):
    h, w, y = tiny.hidden, tiny.weight, tiny.targets
    T, V = h.shape[0], w.shape[0]
    ws = rlk.workspace_for(T, V, h.device)
    _, lse = rlk.rlk_selected_logp(h, w, y, workspace=ws)
    L = rlk.lib()
    need = rlk.rlk_topk_logp_direct_workspace_bytes(T, V, 8, 4)
    buf = torch.empty(need, dtype=torch.uint8, device=h.device)
    out_l = torch.empty((T, 8), dtype=torch.float32, device=h.device)
    out_i = torch.empty((T, 8), dtype=torch.int32, device=h.device)
    H = h.shape[1]

    def call(k=8, dcap=4, wsb=need, stats=ws.numel() * ws.element_size()):
        return L.rlk_topk_logp_direct(h.data_ptr(), H, w.data_ptr(), H, lse.data_ptr(),
                                      ws.data_ptr(), stats, T, H, V, k, 1.0, 0, dcap,
                                      buf.data_ptr(), wsb, out_l.data_ptr(), out_i.data_ptr(),
                                      None)
    assert call(k=0) == rlk.RLK_ERR_INVALID_VALUE
    assert call(k=65) == rlk.RLK_ERR_INVALID_VALUE
    assert call(dcap=-1) == rlk.RLK_ERR_INVALID_VALUE
    assert call(wsb=need - 1) == rlk.RLK_ERR_WORKSPACE_TOO_SMALL
    assert call(stats=16) == rlk.RLK_ERR_WORKSPACE_TOO_SMALL
    assert call() == rlk.RLK_OK
    torch.cuda.synchronize()
