"""Calls on a side stream that let the binding allocate the workspace and the
outputs: those allocations belong to the side stream, so memory the caching
allocator hands out on the current stream meanwhile cannot be the workspace
(whose tile-claim counters the running kernels update).  The side-stream
results must carry the current-stream bits."""

import numpy as np
import pytest

import invariant_selected_token_amd as rlk

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def test_side_stream_without_workspace(prefill):
    dev = prefill.hidden.device
    ref_lp, ref_lse = rlk.rlk_selected_logp(prefill.hidden, prefill.weight, prefill.targets)
    g = torch.from_numpy(np.random.default_rng(3).standard_normal(512).astype(np.float32)).to(dev)
    ref_gh, _ = rlk.rlk_selected_logp_backward(prefill.hidden[:512], prefill.weight,
                                               prefill.targets[:512], ref_lse[:512], g,
                                               want_weight=False)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        # the current stream stays the default one: only stream= names the side
        lp, lse = rlk.rlk_selected_logp(prefill.hidden, prefill.weight, prefill.targets,
                                        stream=side)
        gh, _ = rlk.rlk_selected_logp_backward(prefill.hidden[:512], prefill.weight,
                                               prefill.targets[:512], ref_lse[:512], g,
                                               want_weight=False, stream=side)
        outs.append((lp, lse, gh))
        # meanwhile the current stream allocates and overwrites memory of the
        # same sizes as the workspaces
        for n in (rlk.rlk_selected_logp_workspace_bytes(4096, 4096, 151936),
                  rlk.rlk_selected_logp_backward_workspace_bytes(512, 4096, 151936)):
            junk = torch.empty(n, dtype=torch.uint8, device=dev)
            junk.fill_(0xA5)
            del junk
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for lp, lse, gh in outs:
        assert torch.equal(lp.view(torch.int32), ref_lp.view(torch.int32))
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))
        assert torch.equal(gh.view(torch.int32), ref_gh.view(torch.int32))


def test_direct_topk_on_a_side_stream_without_workspace(prefill):
    """The top-k path without stored logits allocates its pair buffers and
    tables on the side stream (the plan's counters live there)."""
    dev = prefill.hidden.device
    h, w, y = prefill.hidden[:1024], prefill.weight, prefill.targets[:1024]
    T, V, k = 1024, prefill.case.V, 20
    ws = rlk.workspace_for(T, V, dev)
    _, lse = rlk.rlk_selected_logp(h, w, y, workspace=ws)
    ref_l, ref_i = rlk.rlk_topk_logp_direct(h, w, lse, ws, k)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        outs.append(rlk.rlk_topk_logp_direct(h, w, lse, ws, k, stream=side))
        junk = torch.empty(rlk.rlk_topk_logp_direct_workspace_bytes(T, V, k), dtype=torch.uint8,
                           device=dev)
        junk.fill_(0x5A)
        del junk
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for tl, ti in outs:
        assert torch.equal(ti, ref_i)
        assert torch.equal(tl.view(torch.int32), ref_l.view(torch.int32))
