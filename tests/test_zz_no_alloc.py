"""The allocation-free entry point rlk_selected_logp_noalloc against the
workspace entry point rlk_selected_logp it varies, through the C ABI.

Both run the same kernels, so the outputs must agree bit for bit (a stronger
bar than the path's 1e-3 tolerance to the oracle, which is checked too on
sampled rows).  Two calls in a row, the second with fewer rows, so that the
second call runs on a scratch array that still holds the first call's
statistics and counters.  The error paths are CPU checks: they return before
any HIP call.
"""

import ctypes

import numpy as np
import pytest

import invariant_selected_token_amd as rlk
from invariant_selected_token_amd import synth

FAKE = 0x10000


def _noalloc(hidden, ldh, weight, ldw, targets, logp, lse, T, H, V, stream=None):
    return rlk.lib().rlk_selected_logp_noalloc(hidden, ldh, weight, ldw, targets, logp, lse,
                                               T, H, V, stream)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), rlk.RLK_ERR_INVALID_SHAPE),
    (dict(H=100, ldh=256, ldw=256), rlk.RLK_ERR_UNSUPPORTED),
    (dict(hidden=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(logp=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(targets=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(lse=FAKE + 2), rlk.RLK_ERR_MISALIGNED),
    (dict(weight=FAKE + 8), rlk.RLK_ERR_MISALIGNED),
    # 8000 rows at the Qwen3-8B vocabulary need about 76 MB of statistics
    (dict(T=8000, V=151936), rlk.RLK_ERR_SCRATCH_LIMIT),
    (dict(T=8000, V=151936, hidden=None), rlk.RLK_ERR_SCRATCH_LIMIT),
    (dict(T=0, hidden=None, weight=None, targets=None, logp=None, lse=None), rlk.RLK_OK),
])
def test_noalloc_error_paths(kw, status):
    a = dict(hidden=FAKE, ldh=256, weight=FAKE, ldw=256, targets=FAKE, logp=FAKE, lse=FAKE,
             T=4, H=256, V=1000)
    a.update(kw)
    assert _noalloc(**a) == status
    assert rlk.rlk_last_hip_error() == 0


def test_scratch_limit_matches_the_workspace_size():
    """The largest T that fits is the largest whose workspace fits the array."""
    V, H = 151936, 4096
    lo, hi = 1, 1 << 20                    # ws(lo) fits, ws(hi) does not
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if rlk.rlk_selected_logp_workspace_bytes(mid, H, V) <= rlk.RLK_NOALLOC_SCRATCH_BYTES:
            lo = mid
        else:
            hi = mid
    assert 7000 <= lo < 7100
    # T = lo passes the size check (then stops at the NULL pointers), lo + 1 does not
    assert _noalloc(None, H, None, H, None, None, None, lo, H, V) == rlk.RLK_ERR_NULL_POINTER
    assert _noalloc(None, H, None, H, None, None, None, lo + 1, H, V) == \
        rlk.RLK_ERR_SCRATCH_LIMIT


@pytest.mark.gpu
def test_noalloc_matches_the_workspace_entry_point():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    c = synth.prefill_case()
    to_dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev)
    h_all, w = to_dev(c.hidden), to_dev(c.weight)
    y_all = torch.from_numpy(c.targets).to(dev)
    H, V = c.H, c.V
    stream = torch.cuda.current_stream(dev).cuda_stream
    # two calls in a row, the second smaller and at other rows
    for T, r0 in ((4096, 0), (1000, 2500)):
        print(f"noalloc: T={T} rows {r0}.. H={H} V={V}", flush=True)
        h, y = h_all[r0:r0 + T].contiguous(), y_all[r0:r0 + T].contiguous()
        lp_n = torch.full((T,), float("nan"), dtype=torch.float32, device=dev)
        lse_n = torch.full((T,), float("nan"), dtype=torch.float32, device=dev)
        st = _noalloc(h.data_ptr(), H, w.data_ptr(), H, y.data_ptr(), lp_n.data_ptr(),
                      lse_n.data_ptr(), T, H, V, ctypes.c_void_p(stream))
        assert st == rlk.RLK_OK, rlk.rlk_status_string(st)
        ws = torch.empty(rlk.rlk_selected_logp_workspace_bytes(T, H, V), dtype=torch.uint8,
                         device=dev)
        lp_w = torch.empty(T, dtype=torch.float32, device=dev)
        lse_w = torch.empty(T, dtype=torch.float32, device=dev)
        st = rlk.lib().rlk_selected_logp(h.data_ptr(), H, w.data_ptr(), H, y.data_ptr(),
                                         lp_w.data_ptr(), lse_w.data_ptr(), T, H, V,
                                         ws.data_ptr(), ws.numel(), ctypes.c_void_p(stream))
        assert st == rlk.RLK_OK
        torch.cuda.synchronize()
        assert torch.equal(lp_n.view(torch.int32), lp_w.view(torch.int32)), T
        assert torch.equal(lse_n.view(torch.int32), lse_w.view(torch.int32)), T
        # and the path's tolerance to the oracle on a few rows
        from oracle import oracle as orc
        rows = np.array([0, T // 2, T - 1])
        ref_lp, ref_lse = orc.selected_logp(c.hidden[r0 + rows], c.weight, c.targets[r0 + rows])
        got = lp_n.cpu().numpy()[rows].astype(np.float64)
        assert np.abs(got - ref_lp).max() <= 1e-3
        assert np.abs(lse_n.cpu().numpy()[rows].astype(np.float64) - ref_lse).max() <= 1e-3
        del ws


@pytest.mark.gpu
def test_noalloc_replays_in_a_hip_graph():
    """The caller it is for: a captured graph.  The capture holds only kernel
    launches (the scratch's counters are cleared by a kernel); every replay,
    with an eager call on other rows in between that overwrites the scratch,
    gives the bits of the workspace entry point."""
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    c = synth.prefill_case(T=2048)
    to_dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(
        torch.bfloat16)
    h_all, w = to_dev(c.hidden), to_dev(c.weight)
    y_all = torch.from_numpy(c.targets).to(dev)
    h, y = h_all[:1024].contiguous(), y_all[:1024].contiguous()
    h2, y2 = h_all[1024:].contiguous(), y_all[1024:].contiguous()
    ref_lp, ref_lse = rlk.rlk_selected_logp(h, w, y)
    torch.cuda.synchronize()
    lp = torch.empty(1024, dtype=torch.float32, device=dev)
    lse = torch.empty_like(lp)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):        # warm-up on the capture stream (looks up the scratch)
        rlk.rlk_selected_logp_noalloc(h, w, y, lp, lse, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        rlk.rlk_selected_logp_noalloc(h, w, y, lp, lse, stream=s)
    lp2 = torch.empty(1024, dtype=torch.float32, device=dev)
    lse2 = torch.empty_like(lp2)
    for rep in range(4):
        lp.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(lp.view(torch.int32), ref_lp.view(torch.int32)), rep
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), rep
        rlk.rlk_selected_logp_noalloc(h2, w, y2, lp2, lse2)     # eager, other rows
        torch.cuda.synchronize()
