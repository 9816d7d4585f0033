"""Bitwise self-consistency of the HIP path (the pages' 0-mismatch criterion).

A row's fp32 logp and lse must be bit-for-bit the same whatever batch it is
in, wherever it sits, packed or per sequence, prefill or decode, and across
repeated calls (RL-Kernel blog, sections 五-七: bitwise, not a tolerance; the
vLLM blog summary's batch independence and phase consistency).  Bits are
compared on the device by rlk_compare and on the host by integer views.
"""

import numpy as np
import pytest

import invariant_selected_token_amd as rlk
from invariant_selected_token_amd import synth

from conftest import to_dev_bf16, to_dev_i32

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _bits(x):
    return x.contiguous().view(torch.int32)


def _assert_bits_equal(a, b, what):
    st = rlk.consistency_report(rlk.rlk_compare(a.contiguous(), b.contiguous()))
    print(f"{what}: mismatch_count={st['mismatch_count']} "
          f"max_abs_diff={st['max_abs_diff']:.3e} over {st['n']}", flush=True)
    assert st["mismatch_count"] == 0 and st["max_abs_diff"] == 0.0, what
    assert torch.equal(_bits(a), _bits(b)), what


def test_tiny_batch_one_vs_batch(tiny):
    lp, lse = rlk.rlk_selected_logp(tiny.hidden, tiny.weight, tiny.targets)
    lp1 = torch.empty_like(lp)
    lse1 = torch.empty_like(lse)
    for t in range(tiny.case.T):
        a, b = rlk.rlk_selected_logp(tiny.hidden[t:t + 1], tiny.weight, tiny.targets[t:t + 1])
        lp1[t:t + 1] = a
        lse1[t:t + 1] = b
    _assert_bits_equal(lp1, lp, "tiny batch-1 vs batch-64 logp")
    _assert_bits_equal(lse1, lse, "tiny batch-1 vs batch-64 lse")


def test_tiny_repeats_and_permutations(tiny):
    lp, lse = rlk.rlk_selected_logp(tiny.hidden, tiny.weight, tiny.targets)
    for _ in range(100):
        a, b = rlk.rlk_selected_logp(tiny.hidden, tiny.weight, tiny.targets)
        _assert_bits_equal(a, lp, "tiny repeat logp")
        _assert_bits_equal(b, lse, "tiny repeat lse")
    rng = np.random.Generator(np.random.PCG64(17))
    for _ in range(8):
        p = torch.from_numpy(rng.permutation(tiny.case.T)).to(lp.device)
        a, b = rlk.rlk_selected_logp(tiny.hidden[p].contiguous(), tiny.weight,
                                     tiny.targets[p].contiguous())
        _assert_bits_equal(a, lp[p], "tiny permuted logp")
        _assert_bits_equal(b, lse[p], "tiny permuted lse")


def test_every_tile_position_same_bits(prefill):
    """One vector copied into all 512 rows (every position of two token
    tiles): all rows must carry identical bits."""
    h = prefill.hidden[1234:1235].expand(512, -1).contiguous()
    y = prefill.targets[1234:1235].expand(512).contiguous()
    lp, lse = rlk.rlk_selected_logp(h, prefill.weight, y)
    _assert_bits_equal(lp, lp[0:1].expand(512).contiguous(), "all positions logp")
    _assert_bits_equal(lse, lse[0:1].expand(512).contiguous(), "all positions lse")


def test_prefill_packed_vs_per_sequence(prefill):
    lp, lse = rlk.rlk_selected_logp(prefill.hidden, prefill.weight, prefill.targets)
    parts_lp, parts_lse = [], []
    for s in range(8):
        sl = slice(512 * s, 512 * (s + 1))
        a, b = rlk.rlk_selected_logp(prefill.hidden[sl], prefill.weight, prefill.targets[sl])
        parts_lp.append(a)
        parts_lse.append(b)
    _assert_bits_equal(torch.cat(parts_lp), lp, "packed vs per-sequence logp")
    _assert_bits_equal(torch.cat(parts_lse), lse, "packed vs per-sequence lse")


def test_prefill_repeats(prefill):
    lp, lse = rlk.rlk_selected_logp(prefill.hidden, prefill.weight, prefill.targets)
    stats = torch.zeros((100, 8), dtype=torch.float64, device=lp.device)
    a = torch.empty_like(lp)
    b = torch.empty_like(lse)
    for i in range(100):
        rlk.rlk_selected_logp(prefill.hidden, prefill.weight, prefill.targets, logp=a, lse=b)
        rlk.rlk_compare(a, lp, stats=stats[i])
    s = stats.cpu().numpy()
    print(f"100 repeats: total mismatch {s[:, 1].sum()} max diff {s[:, 2].max()}", flush=True)
    assert s[:, 1].sum() == 0 and s[:, 2].max() == 0.0
    _assert_bits_equal(b, lse, "repeat lse")


def test_prefill_permuted_rows(prefill):
    lp, lse = rlk.rlk_selected_logp(prefill.hidden, prefill.weight, prefill.targets)
    rng = np.random.Generator(np.random.PCG64(23))
    p = torch.from_numpy(rng.permutation(prefill.case.T)).to(lp.device)
    a, b = rlk.rlk_selected_logp(prefill.hidden[p].contiguous(), prefill.weight,
                                 prefill.targets[p].contiguous())
    _assert_bits_equal(a, lp[p], "permuted logp")
    _assert_bits_equal(b, lse[p], "permuted lse")


def test_decode_sweep_matches_batch_one_and_prefill(prefill):
    """Decode batches of {1,2,3,7,16,64,255,256} rows from a pool of 256
    prefill vectors, at random positions: each row's bits equal its batch-1
    bits and its bits inside the 4096-row prefill call."""
    plan = synth.decode_plan(prefill_T=prefill.case.T)
    dev = prefill.hidden.device
    pool = torch.from_numpy(plan["pool"]).to(dev)
    lp_pre, lse_pre = rlk.rlk_selected_logp(prefill.hidden, prefill.weight, prefill.targets)
    ph = prefill.hidden[pool].contiguous()
    py = prefill.targets[pool].contiguous()
    lp1 = torch.empty(256, dtype=torch.float32, device=dev)
    lse1 = torch.empty_like(lp1)
    for i in range(256):
        a, b = rlk.rlk_selected_logp(ph[i:i + 1], prefill.weight, py[i:i + 1])
        lp1[i:i + 1] = a
        lse1[i:i + 1] = b
    _assert_bits_equal(lp1, lp_pre[pool], "batch-1 vs prefill logp")
    _assert_bits_equal(lse1, lse_pre[pool], "batch-1 vs prefill lse")
    for B, slots in plan["batches"].items():
        s = torch.from_numpy(slots).to(dev)
        a, b = rlk.rlk_selected_logp(ph[s].contiguous(), prefill.weight, py[s].contiguous())
        _assert_bits_equal(a, lp1[s], f"decode B={B} logp")
        _assert_bits_equal(b, lse1[s], f"decode B={B} lse")


def test_every_batch_size_to_257_same_bits(prefill):
    """One 256 x 256 tile serves every batch size; rows past T are predicated
    off inside it.  Every batch of T = 1 .. 257 rows (the last one a full tile
    plus a tile of one row) must give each row the bits the same vector gets
    in the 4096-row call: plain, with the options (1/tau = 0.7, bf16 logits,
    entropy), and the stored logits.  Row i of the batch of T holds prefill
    vector (i + 37 T) mod 4096, so the rows land at all tile positions.  (The
    vLLM blog summary's dense-GEMM lesson: no small-batch kernels, or a
    request's bits depend on its batch.)"""
    dev = prefill.hidden.device
    N = prefill.case.T
    lp_pre, lse_pre = rlk.rlk_selected_logp(prefill.hidden, prefill.weight, prefill.targets)
    lp2, lse2, ent2 = rlk.rlk_selected_logp_ex(prefill.hidden, prefill.weight, prefill.targets,
                                              inv_temperature=0.7, logits_bf16=True,
                                              entropy=True)
    sizes = list(range(1, 258))
    stats = torch.zeros((len(sizes), 5, 8), dtype=torch.float64, device=dev)
    for k, T in enumerate(sizes):
        idx = (torch.arange(T, device=dev) + 37 * T) % N
        h = prefill.hidden[idx].contiguous()
        y = prefill.targets[idx].contiguous()
        a, b = rlk.rlk_selected_logp(h, prefill.weight, y)
        rlk.rlk_compare(a, lp_pre[idx].contiguous(), stats=stats[k, 0])
        rlk.rlk_compare(b, lse_pre[idx].contiguous(), stats=stats[k, 1])
        a, b, e = rlk.rlk_selected_logp_ex(h, prefill.weight, y, inv_temperature=0.7,
                                           logits_bf16=True, entropy=True)
        rlk.rlk_compare(a, lp2[idx].contiguous(), stats=stats[k, 2])
        rlk.rlk_compare(b, lse2[idx].contiguous(), stats=stats[k, 3])
        rlk.rlk_compare(e, ent2[idx].contiguous(), stats=stats[k, 4])
    st = stats.cpu().numpy()
    bad = [(sizes[k], v) for k in range(len(sizes)) for v in range(5) if st[k, v, 1] != 0]
    print(f"T = 1 .. 257: {len(bad)} mismatching (size, output) pairs", flush=True)
    assert not bad, bad[:10]
    # stored logits: 1 .. 257 rows against the 4096-row call
    z_ref = rlk.rlk_debug_logits(prefill.hidden, prefill.weight)
    zst = torch.zeros((len(sizes), 8), dtype=torch.float64, device=dev)
    for k, T in enumerate(sizes):
        idx = (torch.arange(T, device=dev) + 37 * T) % N
        z = rlk.rlk_debug_logits(prefill.hidden[idx].contiguous(), prefill.weight)
        rlk.rlk_compare(z.view(-1), z_ref[idx].contiguous().view(-1), stats=zst[k])
    zs = zst.cpu().numpy()
    assert zs[:, 1].sum() == 0, [sizes[k] for k in np.flatnonzero(zs[:, 1])][:10]


@pytest.mark.parametrize("V", [151936, 151935])
def test_logits_and_grad_hidden_small_batches_same_bits(prefill, V):
    """The stored logits (whole-row stores for V a multiple of 4, one column
    per store otherwise) and the backward's grad_hidden -- a row's gradient
    depends on that row alone -- carry the same bits in batches of 1 .. 257
    rows as in a 512-row call."""
    dev = prefill.hidden.device
    w = prefill.weight[:V]
    h512 = prefill.hidden[:512].contiguous()
    y512 = torch.remainder(prefill.targets[:512], V).to(torch.int32).contiguous()
    z_ref = rlk.rlk_debug_logits(h512, w)
    for T, shift in ((1, 300), (64, 5), (65, 400), (128, 200), (200, 3), (257, 100)):
        idx = (torch.arange(T, device=dev) + shift) % 512
        z = rlk.rlk_debug_logits(h512[idx].contiguous(), w)
        _assert_bits_equal(z, z_ref[idx].contiguous(), f"T={T} V={V} logits")
    del z_ref
    if V != 151936:
        return
    g = torch.from_numpy(np.random.default_rng(77).standard_normal(512).astype(np.float32)).to(dev)
    _, lse512 = rlk.rlk_selected_logp(h512, w, y512)
    gh_ref, _ = rlk.rlk_selected_logp_backward(h512, w, y512, lse512, g, want_weight=False)
    stats = torch.zeros((257, 8), dtype=torch.float64, device=dev)
    for T in range(1, 258):
        idx = (torch.arange(T, device=dev) + 11 * T) % 512
        gh, _ = rlk.rlk_selected_logp_backward(h512[idx].contiguous(), w, y512[idx].contiguous(),
                                               lse512[idx].contiguous(), g[idx].contiguous(),
                                               want_weight=False)
        rlk.rlk_compare(gh.view(-1), gh_ref[idx].contiguous().view(-1), stats=stats[T - 1])
    st = stats.cpu().numpy()
    bad = [T for T in range(1, 258) if st[T - 1, 1] != 0]
    print(f"grad_hidden T = 1 .. 257: {len(bad)} mismatching sizes", flush=True)
    assert not bad, bad[:10]


def test_other_rows_do_not_matter(tiny, dev):
    """Replacing every other row's contents and targets leaves a row's bits."""
    lp, lse = rlk.rlk_selected_logp(tiny.hidden, tiny.weight, tiny.targets)
    c = synth.normal_case("noise", 555, tiny.case.T, tiny.case.H, tiny.case.V)
    h2 = to_dev_bf16(c.hidden, dev)
    y2 = to_dev_i32(c.targets, dev)
    keep = [0, 13, 40]
    h2[keep] = tiny.hidden[keep]
    y2[keep] = tiny.targets[keep]
    a, b = rlk.rlk_selected_logp(h2, tiny.weight, y2)
    _assert_bits_equal(a[keep], lp[keep], "content independence logp")
    _assert_bits_equal(b[keep], lse[keep], "content independence lse")


def test_negative_control_order_change_is_visible(prefill):
    """Reversing the K order (same mathematics, other fp32 rounding) must be
    seen by the harness as last-bit drift: mismatches > 0, tiny differences.
    This shows the bitwise checks above can see the drift the pages warn
    about (RL-Kernel blog, section 二: summation order changes the last bits)."""
    rows = slice(0, 512)
    lp, _ = rlk.rlk_selected_logp(prefill.hidden[rows], prefill.weight, prefill.targets[rows])
    hr = prefill.hidden[rows].flip(1).contiguous()
    wr = prefill.weight.flip(1).contiguous()
    a, _ = rlk.rlk_selected_logp(hr, wr, prefill.targets[rows])
    st = rlk.consistency_report(rlk.rlk_compare(a, lp))
    print(f"negative control: {st}", flush=True)
    assert st["mismatch_count"] > 0
    assert 0.0 < st["max_abs_diff"] < 1e-3


def test_two_stages_equal_one_call(prefill):
    """rlk_vocab_stats + rlk_vocab_merge reproduce rlk_selected_logp bitwise."""
    lp, lse = rlk.rlk_selected_logp(prefill.hidden, prefill.weight, prefill.targets)
    ws = rlk.workspace_for(prefill.case.T, prefill.case.V, lp.device)
    rlk.rlk_vocab_stats(prefill.hidden, prefill.weight, prefill.targets, ws)
    a, b = rlk.rlk_vocab_merge(prefill.targets, ws, prefill.case.V)
    _assert_bits_equal(a, lp, "two-stage logp")
    _assert_bits_equal(b, lse, "two-stage lse")


def test_rollout_packed_vs_per_response(rollout):
    """T=16384 packed vs 32 per-response calls of 512 rows, bitwise."""
    lp, lse = rlk.rlk_selected_logp(rollout.hidden, rollout.weight, rollout.targets)
    parts_lp, parts_lse = [], []
    for s in range(32):
        sl = slice(512 * s, 512 * (s + 1))
        a, b = rlk.rlk_selected_logp(rollout.hidden[sl], rollout.weight, rollout.targets[sl])
        parts_lp.append(a)
        parts_lse.append(b)
    _assert_bits_equal(torch.cat(parts_lp), lp, "rollout packed vs per-response logp")
    _assert_bits_equal(torch.cat(parts_lse), lse, "rollout packed vs per-response lse")


def _slices(V, cuts):
    """[v_begin, v_end) slices of [0, V) cut at the given 256-aligned rows."""
    edges = [0] + sorted(set(cuts)) + [V]
    return [(a, b) for a, b in zip(edges[:-1], edges[1:]) if b > a]


def _tp_cuts(V, P):
    cols = (V + 255) // 256
    return [round(i * cols / P) * 256 for i in range(1, P)]


@pytest.mark.parametrize("name", ["tp2", "tp4", "tp8", "uneven", "single_columns"])
def test_vocab_slices_merge_to_the_unsliced_bits(prefill, name):
    """Statistics computed per slice of the vocabulary (tensor-parallel LM-head
    shards, RL-Kernel blog section 七) and merged once give the unsliced bits
    for any slice count.  The workspace starts as NaN so that a tile or target
    logit that no slice writes shows up as a mismatch."""
    c = prefill.case
    T, V = c.T, c.V
    cuts = {"tp2": _tp_cuts(V, 2), "tp4": _tp_cuts(V, 4), "tp8": _tp_cuts(V, 8),
            "uneven": [256, 512, 75776, 151552],
            "single_columns": [256 * j for j in range(1, 12)] + [V - V % 256]}[name]
    sl = _slices(V, cuts)
    assert all(a % 256 == 0 for a, _ in sl) and sl[-1][1] == V
    lp, lse = rlk.rlk_selected_logp(prefill.hidden, prefill.weight, prefill.targets)
    ws = rlk.workspace_for(T, V, lp.device)
    ws.view(torch.uint8).fill_(0xFF)          # all-ones bits: NaN in every float slot
    for a, b in sl:
        rlk.rlk_vocab_stats_shard(prefill.hidden, prefill.weight[a:b], prefill.targets,
                                  ws, V, a)
    s_lp, s_lse = rlk.rlk_vocab_merge(prefill.targets, ws, V)
    _assert_bits_equal(s_lp, lp, f"{name} ({len(sl)} slices) logp")
    _assert_bits_equal(s_lse, lse, f"{name} ({len(sl)} slices) lse")


def test_vocab_slices_on_two_streams(tiny):
    """Two slices launched on different streams, joined before the merge."""
    c = tiny.case
    T, V = c.T, c.V
    lp, lse = rlk.rlk_selected_logp(tiny.hidden, tiny.weight, tiny.targets)
    ws = rlk.workspace_for(T, V, lp.device)
    ws.view(torch.uint8).fill_(0xFF)
    cut = (V // 512) * 256
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    ready = torch.cuda.current_stream().record_event()
    s1.wait_event(ready)
    s2.wait_event(ready)
    with torch.cuda.stream(s1):
        rlk.rlk_vocab_stats_shard(tiny.hidden, tiny.weight[:cut], tiny.targets, ws, V, 0,
                                  stream=s1)
    with torch.cuda.stream(s2):
        rlk.rlk_vocab_stats_shard(tiny.hidden, tiny.weight[cut:], tiny.targets, ws, V, cut,
                                  stream=s2)
    torch.cuda.current_stream().wait_stream(s1)
    torch.cuda.current_stream().wait_stream(s2)
    s_lp, s_lse = rlk.rlk_vocab_merge(tiny.targets, ws, V)
    _assert_bits_equal(s_lp, lp, "two-stream slices logp")
    _assert_bits_equal(s_lse, lse, "two-stream slices lse")


@pytest.mark.parametrize("H", [192, 4096])
def test_odd_block_count_and_zero_rows_batch_invariant(dev, H):
    """1024 rows (280 tiles over 70 columns of 256: more than one round of
    the persistent grid) against four 256-row calls.  H = 192 has an odd
    number of 64-deep K blocks (a phantom zero block is appended), and rows of
    zeros make logits of exactly 0, whose sign must agree too."""
    T, V = 1024, 256 * 70 - 37
    c = synth.normal_case(f"tail_{H}", 990 + H, T, H, V)
    hid = c.hidden.copy()
    hid[[5, 300, 777, 1023]] = 0
    h, w, y = to_dev_bf16(hid, dev), to_dev_bf16(c.weight, dev), to_dev_i32(c.targets, dev)
    lp, lse = rlk.rlk_selected_logp(h, w, y)
    for s in range(4):
        sl = slice(256 * s, 256 * (s + 1))
        a, b = rlk.rlk_selected_logp(h[sl], w, y[sl])
        _assert_bits_equal(a, lp[sl], f"H={H} logp rows {sl}")
        _assert_bits_equal(b, lse[sl], f"H={H} lse rows {sl}")
    _, _, e_full = rlk.rlk_selected_logp_ex(h, w, y, inv_temperature=0.8, entropy=True)
    _, _, e_part = rlk.rlk_selected_logp_ex(h[:256], w, y[:256], inv_temperature=0.8,
                                            entropy=True)
    _assert_bits_equal(e_part, e_full[:256], f"H={H} entropy")
