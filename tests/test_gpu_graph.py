"""The entry points inside a captured HIP graph (serving loops replay the
scoring step as a graph).  The library allocates nothing, never
synchronises and clears memory only with kernels, so its launches can be
captured.  Each replay, with the program's own eager work in between, must
give the eager bits."""

import numpy as np
import pytest

import invariant_selected_token_amd as rlk

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _bits(x):
    return x.contiguous().view(torch.int32)


def test_forward_with_options_replays_bitwise(prefill):
    h, w, y = prefill.hidden[:1024], prefill.weight, prefill.targets[:1024]
    T, V = 1024, prefill.case.V
    flags = rlk.RLK_ENTROPY
    ws = torch.empty(rlk.rlk_workspace_bytes_ex(T, V, flags), dtype=torch.uint8,
                     device=h.device)
    lp = torch.empty(T, dtype=torch.float32, device=h.device)
    lse, ent = torch.empty_like(lp), torch.empty_like(lp)
    ref = rlk.rlk_selected_logp_ex(h, w, y, inv_temperature=0.7, entropy=True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):        # warm-up on the capture stream
        rlk.rlk_selected_logp_ex(h, w, y, inv_temperature=0.7, entropy=ent, logp=lp, lse=lse,
                                 workspace=ws, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        rlk.rlk_selected_logp_ex(h, w, y, inv_temperature=0.7, entropy=ent, logp=lp, lse=lse,
                                 workspace=ws, stream=s)
    for rep in range(4):
        lp.fill_(np.nan)
        ent.fill_(np.nan)
        g.replay()
        torch.cuda.synchronize()
        _ = (h[:16].float() @ w[:16].float().T).sum()     # unrelated eager work
        for a, b in zip((lp, lse, ent), ref):
            assert torch.equal(_bits(a), _bits(b)), f"replay {rep}"


def test_backward_replays_bitwise(tiny):
    h, w, y = tiny.hidden, tiny.weight, tiny.targets
    T, H, V = tiny.case.T, tiny.case.H, tiny.case.V
    gl = torch.linspace(-1, 1, T, dtype=torch.float32, device=h.device)
    _, lse = rlk.rlk_selected_logp(h, w, y)
    ws = torch.empty(rlk.rlk_selected_logp_backward_workspace_bytes(T, H, V),
                     dtype=torch.uint8, device=h.device)
    gh = torch.empty((T, H), dtype=torch.float32, device=h.device)
    gw = torch.empty((V, H), dtype=torch.float32, device=h.device)
    ref_h, ref_w = rlk.rlk_selected_logp_backward(h, w, y, lse, gl)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        rlk.rlk_selected_logp_backward(h, w, y, lse, gl, grad_hidden=gh, grad_weight=gw,
                                       workspace=ws, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        rlk.rlk_selected_logp_backward(h, w, y, lse, gl, grad_hidden=gh, grad_weight=gw,
                                       workspace=ws, stream=s)
    for rep in range(3):
        gh.fill_(np.nan)
        gw.fill_(np.nan)
        ws.fill_(0xFF)                      # stale workspace must not matter
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(gh), _bits(ref_h)) and torch.equal(_bits(gw), _bits(ref_w))


def test_direct_topk_replays_bitwise(prefill):
    """The top-k path without stored logits (six launches, counters cleared
    by a kernel and by its plan step) captured and replayed: each replay
    gives the eager bits, with the workspace scribbled over in between."""
    h, w, y = prefill.hidden[:512], prefill.weight, prefill.targets[:512]
    T, V, k = 512, prefill.case.V, 20
    ws = rlk.workspace_for(T, V, h.device)
    _, lse = rlk.rlk_selected_logp(h, w, y, workspace=ws)
    wsd = torch.empty(rlk.rlk_topk_logp_direct_workspace_bytes(T, V, k), dtype=torch.uint8,
                      device=h.device)
    tl = torch.empty((T, k), dtype=torch.float32, device=h.device)
    ti = torch.empty((T, k), dtype=torch.int32, device=h.device)
    ref_l, ref_i = rlk.rlk_topk_logp_direct(h, w, lse, ws, k)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        rlk.rlk_topk_logp_direct(h, w, lse, ws, k, workspace=wsd, topk_logp=tl, topk_ids=ti,
                                 stream=s)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        rlk.rlk_topk_logp_direct(h, w, lse, ws, k, workspace=wsd, topk_logp=tl, topk_ids=ti,
                                 stream=s)
    for rep in range(4):
        tl.fill_(np.nan)
        ti.fill_(-7)
        wsd.fill_(0xA5)                                   # stale counters and tables
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _ = (h[:16].float() @ w[:16].float().T).sum()     # unrelated eager work
        assert torch.equal(ti, ref_i), f"replay {rep}"
        assert torch.equal(_bits(tl), _bits(ref_l)), f"replay {rep}"
