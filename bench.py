#!/usr/bin/env python3
"""Benchmark of the batch-invariant selected-token log-probability path.

Workload: the Qwen3-8B LM-head shape on the training-side recompute, T = 4096
packed rows (8 sequences x 512 tokens), H = 4096, V = 151936, bf16 hidden and
weight (synthetic, seeded), uniform targets.  One step is one pass of the
whole hot path on one batch, with inputs already resident in HBM:
  1. rlk_vocab_stats  logit GEMM (bf16 MFMA, fp32 accumulation) with the fused
                      per-(row, 128-wide vocabulary tile) max / sum of
                      exponentials and the target-logit capture;
  2. rlk_vocab_merge  fixed-order fold of the tile statistics -> lse, logp;
  3. rlk_compare      bitwise consistency of this step's logp and lse (one
                      buffer, one launch) against the first call's (mismatch
                      count, max |diff|).
Prints one JSON line.  Only one GPU is used; --gpus N > 1 exits.

After the timed region (never inside it) the line also gets: per-step median
and minimum times; the shader clock sampled while the statistics kernel runs
(amd-smi); the invariance report of every workload (batch 1 vs batch N, row
positions, packing, decode vs prefill, repeats, and a negative control), as
mismatch count, max / mean / std of |diff| and the k3 estimator per variant;
the vendor path (hipBLASLt GEMM + logsumexp + gather) as context; the other
entry points' timings; and the fp64 oracle timed on the host.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import shutil
import statistics
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X's published dense bf16 MFMA peak (2.5 PFLOP/s; 256 CU x 4096 FLOP/clk x 2.4 GHz
# = 2516.6 TFLOP/s before rounding)
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
KERNEL_SRC = os.path.join(ROOT, "invariant_selected_token_amd", "csrc", "kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_stats_prefill_T4096_traffic.md")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_digest() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the GEMM kernel from the committed rocprofv3
    counter summary, or None when the kernel source changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not b or m.group(1) != kernel_source_digest():
        return None
    return float(b.group(1))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(case, seconds: float) -> dict:
    """The fp64 oracle, as it stands, on a bounded sample of the same rows;
    plus the single-thread time of the whole tiny workload."""
    import numpy as np

    from invariant_selected_token_amd import synth
    from oracle import oracle as orc

    # every call names its thread count: a count given to the oracle stays
    # its OpenMP default for later calls
    cores = orc.max_threads()
    tiny = synth.tiny_case()
    t0 = time.perf_counter()
    orc.selected_logp(tiny.hidden, tiny.weight, tiny.targets, nthreads=1)
    tiny_s = time.perf_counter() - t0
    probe = max(2, min(cores, 16))
    t0 = time.perf_counter()
    orc.selected_logp(case.hidden[:probe], case.weight, case.targets[:probe], nthreads=cores)
    per_row = (time.perf_counter() - t0) / probe
    n = int(max(probe, min(case.T, round(seconds / max(per_row, 1e-9)))))
    rng = np.random.Generator(np.random.PCG64(4321))
    rows = np.sort(rng.choice(case.T, size=n, replace=False))
    t0 = time.perf_counter()
    orc.selected_logp(case.hidden[rows], case.weight, case.targets[rows], nthreads=cores)
    wall = time.perf_counter() - t0
    return {"value": n / wall, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{n} of {case.T} rows of the same workload (seeded choice), "
                      f"full vocabulary V={case.V}, fp64, {wall:.1f} s wall",
            "tiny_T64_H256_V4096_single_thread_s": tiny_s}


def sample_sclk(torch, fn, seconds: float = 3.0):
    """Shader clock (MHz, mean over the XCDs' GFX clocks, median over the
    samples) and socket power (W) read with amd-smi while `fn` keeps the GPU
    busy; None when the tool is missing or prints no clock."""
    tool = shutil.which("amd-smi")
    if tool is None:
        return None
    samples, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            try:
                r = subprocess.run([tool, "metric", "-g", "0", "-c", "-p"], capture_output=True,
                                   text=True, timeout=10)
            except (OSError, subprocess.SubprocessError):
                return
            mhz = [int(x) for x in re.findall(r"GFX_\d+:\s*CLK:\s*(\d+)\s*MHz", r.stdout)]
            pw = re.findall(r"SOCKET_POWER:\s*([\d.]+)\s*W", r.stdout)
            if mhz:
                samples.append((sum(mhz) / len(mhz), float(pw[0]) if pw else None))

    for _ in range(5):
        fn()
    torch.cuda.synchronize()
    th = threading.Thread(target=poll, daemon=True)
    th.start()
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=15)
    # the first sample may straddle the start of the load
    use = samples[1:] if len(samples) > 2 else samples
    if not use:
        return None
    mhz = [u[0] for u in use]
    watts = [u[1] for u in use if u[1] is not None]
    return {"median_MHz": statistics.median(mhz), "min_MHz": min(mhz), "max_MHz": max(mhz),
            "socket_power_W_median": statistics.median(watts) if watts else None,
            "samples": len(use), "source": "amd-smi metric -c -p: GFX clocks of the XCDs "
                                            "and socket power"}


VARIANTS = ("options", "slices", "backward", "rmsnorm", "topk20", "long_rollout", "decode")
WORKLOADS = ("tiny", "prefill", "decode", "adversarial", "rollout", "negative_control")


class Harness:
    """Collects rlk_compare statistics per (workload, variant, output) on the
    device and folds them on the host at the end: one synchronisation."""

    def __init__(self, rlk, torch, dev):
        self.rlk, self.torch, self.dev = rlk, torch, dev
        self.parts = {}

    def add(self, workload, variant, a, b, what="logp"):
        st = self.torch.empty(8, dtype=self.torch.float64, device=self.dev)
        self.rlk.rlk_compare(a.contiguous().view(-1), b.contiguous().view(-1), stats=st)
        self.parts.setdefault((workload, variant, what), []).append(st)

    def report(self):
        out = {}
        for (w, v, what), sts in self.parts.items():
            s = self.torch.stack(sts).cpu().numpy()
            n, k3n = s[:, 0].sum(), s[:, 6].sum()
            mean = s[:, 3].sum() / n if n else 0.0
            var = max(s[:, 4].sum() / n - mean * mean, 0.0) if n else 0.0
            out.setdefault(w, {}).setdefault(v, {})[what] = {
                "compared": int(n), "mismatch_count": int(s[:, 1].sum()),
                "max_abs_diff": float(s[:, 2].max()), "mean_abs_diff": float(mean),
                "std_abs_diff": float(var ** 0.5),
                "k3_mean": float(s[:, 5].sum() / k3n) if k3n else 0.0}
        return out


def invariance_report(rlk, torch, np, prefill_dev, only=WORKLOADS):
    """Bitwise self-consistency of every workload, per variant (the pages'
    mismatch count and max |diff|; the vLLM blog summary's mean / std of
    |diff| and k3).  prefill_dev = (hidden, weight, targets) on the device."""
    from invariant_selected_token_amd import synth

    hidden, weight, targets = prefill_dev
    dev = hidden.device
    H = Harness(rlk, torch, dev)

    def to_dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)

    def both(w, v, got, ref):
        H.add(w, v, got[0], ref[0], "logp")
        H.add(w, v, got[1], ref[1], "lse")

    def call(h, W, y):
        return rlk.rlk_selected_logp(h, W, y)

    rng = np.random.Generator(np.random.PCG64(2468))
    if "tiny" in only:
        c = synth.tiny_case()
        h, W, y = to_dev(c.hidden), to_dev(c.weight), torch.from_numpy(c.targets).to(dev)
        ref = call(h, W, y)
        for t in range(c.T):
            both("tiny_T64", "batch1_vs_batch64", call(h[t:t + 1], W, y[t:t + 1]),
                 (ref[0][t:t + 1], ref[1][t:t + 1]))
        for _ in range(100):
            both("tiny_T64", "repeats_100", call(h, W, y), ref)
        for _ in range(8):
            p = torch.from_numpy(rng.permutation(c.T)).to(dev)
            both("tiny_T64", "permutations_8", call(h[p].contiguous(), W, y[p].contiguous()),
                 (ref[0][p], ref[1][p]))
    T = hidden.shape[0]
    ref_pre = call(hidden, weight, targets)
    if "prefill" in only:
        w = "prefill_T4096"
        for sq in range(T // 512):
            sl = slice(512 * sq, 512 * (sq + 1))
            both(w, "per_sequence_vs_packed", call(hidden[sl], weight, targets[sl]),
                 (ref_pre[0][sl], ref_pre[1][sl]))
        for _ in range(20):
            both(w, "repeats_20", call(hidden, weight, targets), ref_pre)
        p = torch.from_numpy(rng.permutation(T)).to(dev)
        both(w, "permuted", call(hidden[p].contiguous(), weight, targets[p].contiguous()),
             (ref_pre[0][p], ref_pre[1][p]))
        for n in (1, 7, 100, 255, 257, 1000):
            idx = (torch.arange(n, device=dev) + 13 * n) % T
            both(w, "sub_batches_at_other_positions",
                 call(hidden[idx].contiguous(), weight, targets[idx].contiguous()),
                 (ref_pre[0][idx], ref_pre[1][idx]))
    if "decode" in only:
        plan = synth.decode_plan(prefill_T=T)
        pool = torch.from_numpy(plan["pool"]).to(dev)
        ph, py = hidden[pool].contiguous(), targets[pool].contiguous()
        one_lp = torch.empty(pool.numel(), dtype=torch.float32, device=dev)
        one_lse = torch.empty_like(one_lp)
        for i in range(pool.numel()):
            a, b = call(ph[i:i + 1], weight, py[i:i + 1])
            one_lp[i:i + 1], one_lse[i:i + 1] = a, b
        both("decode_sweep", "batch1_vs_prefill", (one_lp, one_lse),
             (ref_pre[0][pool], ref_pre[1][pool]))
        for B, slots in plan["batches"].items():
            sl = torch.from_numpy(slots).to(dev)
            got = call(ph[sl].contiguous(), weight, py[sl].contiguous())
            both("decode_sweep", f"B={B}_vs_batch1", got, (one_lp[sl], one_lse[sl]))
            both("decode_sweep", f"B={B}_vs_prefill", got,
                 (ref_pre[0][pool[sl]], ref_pre[1][pool[sl]]))
    if "adversarial" in only:
        c = synth.adversarial_case()
        h, W, y = to_dev(c.hidden), to_dev(c.weight), torch.from_numpy(c.targets).to(dev)
        w = "adversarial_T1024"
        ref = call(h, W, y)
        for t in list(range(0, 96)) + [500, 1023]:
            both(w, "batch1_vs_batch", call(h[t:t + 1], W, y[t:t + 1]),
                 (ref[0][t:t + 1], ref[1][t:t + 1]))
        for _ in range(100):
            both(w, "repeats_100", call(h, W, y), ref)
        for _ in range(3):
            p = torch.from_numpy(rng.permutation(c.T)).to(dev)
            both(w, "permutations_3", call(h[p].contiguous(), W, y[p].contiguous()),
                 (ref[0][p], ref[1][p]))
        del W
    if "rollout" in only:
        c = synth.long_rollout_case()
        h, y = to_dev(c.hidden), torch.from_numpy(c.targets).to(dev)
        w = "rollout_T16384"
        ref = call(h, weight, y)
        for sq in range(c.T // 512):
            sl = slice(512 * sq, 512 * (sq + 1))
            both(w, "per_response_vs_packed", call(h[sl], weight, y[sl]),
                 (ref[0][sl], ref[1][sl]))
        for _ in range(5):
            both(w, "repeats_5", call(h, weight, y), ref)
        p = torch.from_numpy(rng.permutation(c.T)).to(dev)
        both(w, "permuted", call(h[p].contiguous(), weight, y[p].contiguous()),
             (ref[0][p], ref[1][p]))
        del h
    if "negative_control" in only:
        # the same mathematics in another summation order (K reversed in both
        # operands) must show up as drift: mismatches > 0 (RL-Kernel blog,
        # section 二: accumulation order changes the last bits)
        rows = slice(0, 512)
        got = call(hidden[rows].flip(1).contiguous(), weight.flip(1).contiguous(), targets[rows])
        both("negative_control", "K_order_reversed_prefill_512_rows", got,
             (ref_pre[0][rows], ref_pre[1][rows]))
    return H.report()


def vendor_context(torch, hidden, weight, targets, steps):
    """The vendor path on the same GPU, as context (not a target): the bf16
    logits GEMM of torch (hipBLASLt), logsumexp in fp32, gather.  Timed, and
    checked for batch invariance (rows alone and in sub-batches against the
    full batch)."""
    import torch.nn.functional as F

    def path(h, y):
        z = F.linear(h, weight).float()
        lse = torch.logsumexp(z, dim=1)
        return z.gather(1, y.long()[:, None])[:, 0] - lse, lse

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms = timed(lambda: path(hidden, targets))
    gemm_ms = timed(lambda: F.linear(hidden, weight))
    lp, _ = path(hidden, targets)
    mism, maxd, n = 0, 0.0, 0
    for rows in (slice(0, 1), slice(100, 101), slice(0, 7), slice(0, 64), slice(1000, 1255),
                 slice(0, 512)):
        a, _ = path(hidden[rows], targets[rows])
        d = (a - lp[rows]).abs()
        mism += int((a.view(torch.int32) != lp[rows].view(torch.int32)).sum())
        maxd = max(maxd, float(d.max()))
        n += a.numel()
    return {"ms": ms, "what": "F.linear bf16 (hipBLASLt) + logsumexp fp32 + gather",
            "gemm_only_ms": gemm_ms,
            "gemm_only_frac_of_bf16_peak": 2.0 * hidden.shape[0] * hidden.shape[1]
            * weight.shape[0] / (gemm_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "batch_invariance": {"compared": n, "mismatch_count": mism, "max_abs_diff": maxd,
                                 "variants": "rows 0, 100, 0-6, 0-63, 1000-1254, 0-511 "
                                             "alone vs in the 4096-row batch"}}


def time_variants(rlk, torch, np, hidden, weight, targets, T, H, V, steps, flops,
                  only=VARIANTS):
    """The same workload through the other entry points, timed after (never
    inside) the headline region: the contract options (1/tau = 0.7, bf16
    logits, entropy), the statistics computed as 4 vocabulary slices plus one
    merge, the backward, the RMSNorm, top-k, the long rollout and decode
    batches (`only` names a subset).  Mean milliseconds per call over `steps`
    calls after 2 warm-up calls."""
    dev = hidden.device
    out = {}

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    if "options" in only:
        flags = rlk.RLK_LOGITS_BF16 | rlk.RLK_ENTROPY
        ws_ex = torch.empty(rlk.rlk_workspace_bytes_ex(T, V, flags), dtype=torch.uint8,
                            device=dev)

        def opts_stats():
            rlk.rlk_vocab_stats_ex(hidden, weight, targets, ws_ex, V, 0, inv_temperature=0.7,
                                   logits_bf16=True, entropy=True)

        def opts_merge():
            rlk.rlk_vocab_merge_ex(targets, ws_ex, V, logits_bf16=True, entropy=True)

        st = timed(opts_stats)
        mg = timed(opts_merge)
        del ws_ex
        out["options_tau0.7_bf16_entropy"] = {"gemm_stats_ms": st, "merge_ms": mg,
                                              "gemm_TFLOP/s": flops / (st * 1e-3) / 1e12}

    if "slices" in only:
        ws = rlk.workspace_for(T, V, dev)
        cols = (V + 255) // 256
        cuts = [0] + [round(i * cols / 4) * 256 for i in range(1, 4)] + [V]

        def slices():
            for a, b in zip(cuts[:-1], cuts[1:]):
                rlk.rlk_vocab_stats_shard(hidden, weight[a:b], targets, ws, V, a)
            rlk.rlk_vocab_merge(targets, ws, V)

        out["vocab_slices_4_plus_merge_ms"] = timed(slices)
        del ws

    if "backward" in only:
        # hidden-row transpose, dz pass, grad_hidden (weight read K-major) and
        # grad_weight GEMMs
        g = torch.linspace(-1.0, 1.0, T, dtype=torch.float32, device=dev)
        _, lse = rlk.rlk_selected_logp(hidden, weight, targets)
        gh = torch.empty((T, H), dtype=torch.float32, device=dev)
        gw = torch.empty((V, H), dtype=torch.float32, device=dev)
        ws_b = torch.empty(rlk.rlk_selected_logp_backward_workspace_bytes(T, H, V),
                           dtype=torch.uint8, device=dev)

        def backward():
            rlk.rlk_selected_logp_backward(hidden, weight, targets, lse, g, grad_hidden=gh,
                                           grad_weight=gw, workspace=ws_b)

        bw = timed(backward)
        del ws_b, gw
        out["backward"] = {"ms": bw, "TFLOP/s": 3 * flops / (bw * 1e-3) / 1e12,
                           "frac_of_bf16_peak": 3 * flops / (bw * 1e-3) / 1e12
                           / PEAK_BF16_TFLOPS}

    if "rmsnorm" in only:
        # RMSNorm feeding the LM head, on the same [T, H] shape (HBM-bound)
        gamma = torch.ones(H, dtype=torch.bfloat16, device=dev)
        xn = torch.empty_like(hidden)

        def rmsnorm():
            rlk.rlk_rmsnorm(hidden, gamma, 1e-6, y=xn)

        rn = timed(rmsnorm)
        rn_bytes = 2.0 * T * H * 2 + 2.0 * H
        out["rmsnorm"] = {"ms": rn, "GB/s": rn_bytes / (rn * 1e-3) / 1e9,
                          "frac_of_hbm_peak": rn_bytes / (rn * 1e-3) / 1e9 / PEAK_HBM_GBS,
                          "bytes": rn_bytes}

    if "topk20" in only:
        # top-k log-probabilities (k = 20): logits stored once, then the selection
        z = torch.empty((T, V), dtype=torch.float32, device=dev)
        tl = torch.empty((T, 20), dtype=torch.float32, device=dev)
        ti = torch.empty((T, 20), dtype=torch.int32, device=dev)
        ws_t = rlk.workspace_for(T, V, dev)
        _, lse_t = rlk.rlk_selected_logp(hidden, weight, targets, workspace=ws_t)

        def store_logits():
            rlk.rlk_logits(hidden, weight, logits=z)

        def select():
            rlk.rlk_topk_logp(z, lse_t, ws_t, 20, topk_logp=tl, topk_ids=ti)

        lg = timed(store_logits)
        sel = timed(select)
        del z
        # the same top-k without the stored logits: the candidate tiles'
        # logits recomputed (bitwise the same entries)
        ws_d = torch.empty(rlk.rlk_topk_logp_direct_workspace_bytes(T, V, 20),
                           dtype=torch.uint8, device=dev)

        def direct():
            rlk.rlk_topk_logp_direct(hidden, weight, lse_t, ws_t, 20, workspace=ws_d,
                                     topk_logp=tl, topk_ids=ti)

        dr = timed(direct)
        del ws_d
        # the two paths' entries, bit for bit
        z = torch.empty((T, V), dtype=torch.float32, device=dev)
        rlk.rlk_logits(hidden, weight, logits=z)
        sl, si = rlk.rlk_topk_logp(z, lse_t, ws_t, 20)
        del z
        dl, di = rlk.rlk_topk_logp_direct(hidden, weight, lse_t, ws_t, 20)
        torch.cuda.synchronize()
        mism = int(((di != si) | (dl.view(torch.int32) != sl.view(torch.int32))).sum().item())

        # context: the vendor route, torch's bf16 linear layer then torch.topk of
        # the log-softmax (not batch-invariant; ties in its own order)
        def vendor():
            zz = torch.nn.functional.linear(hidden, weight).float()
            torch.topk(torch.log_softmax(zz, dim=1), 20, dim=1)

        vd = timed(vendor)
        out["topk20"] = {"logits_store_ms": lg, "select_ms": sel,
                         "select_GB/s": 4.0 * T * V / (sel * 1e-3) / 1e9,
                         "direct_ms": dr, "direct_vs_stored": (lg + sel) / dr,
                         "direct_vs_stored_mismatches": mism,
                         "vendor_linear_topk_ms": vd}

    if "long_rollout" in only:
        # 16384 rows (32 responses x 512 tokens) through the same path
        from invariant_selected_token_amd import synth as _synth
        lr = _synth.long_rollout_case()
        to_dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(
            dev).view(torch.bfloat16)
        h_lr, y_lr = to_dev(lr.hidden), torch.from_numpy(lr.targets).to(dev)
        T_lr = lr.T
        ws_lr = rlk.workspace_for(T_lr, V, dev)
        lp_lr = torch.empty(T_lr, dtype=torch.float32, device=dev)
        lse_lr = torch.empty_like(lp_lr)

        def rollout_stats():
            rlk.rlk_vocab_stats(h_lr, weight, y_lr, ws_lr)

        def rollout_merge():
            rlk.rlk_vocab_merge(y_lr, ws_lr, V, logp=lp_lr, lse=lse_lr)

        ro_g = timed(rollout_stats)
        ro_m = timed(rollout_merge)
        ro_bytes = 8.0 * ((V + 127) // 128) * T_lr + 16.0 * T_lr
        out["long_rollout"] = {
            "T": T_lr, "gemm_stats_ms": ro_g, "merge_ms": ro_m,
            "tokens/s": T_lr / ((ro_g + ro_m) * 1e-3),
            "gemm_TFLOP/s": 2.0 * T_lr * H * V / (ro_g * 1e-3) / 1e12,
            "gemm_frac_of_bf16_peak": 2.0 * T_lr * H * V / (ro_g * 1e-3) / 1e12
            / PEAK_BF16_TFLOPS,
            "merge_GB/s": ro_bytes / (ro_m * 1e-3) / 1e9}
        del h_lr, ws_lr

    if "decode" in only:
        # decode batches: the whole head is streamed for a handful of rows
        decode = {}
        for B in (1, 16, 64, 256):
            hb, yb = hidden[:B].contiguous(), targets[:B].contiguous()
            lpb = torch.empty(B, dtype=torch.float32, device=dev)
            lseb = torch.empty_like(lpb)
            wsb = rlk.workspace_for(B, V, dev)

            def dec():
                rlk.rlk_selected_logp(hb, weight, yb, logp=lpb, lse=lseb, workspace=wsb)

            ms = timed(dec)
            decode[f"B={B}"] = {"ms": ms, "weight_GB/s": 2.0 * V * H / (ms * 1e-3) / 1e9}
        out["decode"] = decode
    out["steps"] = steps
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed steps first (the shader clock settles over ~8 launches)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-time budget of the oracle CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--variants", default=",".join(VARIANTS),
                    help="comma-separated subset of: " + ", ".join(VARIANTS))
    ap.add_argument("--variant-steps", type=int, default=10,
                    help="timed calls per variant (options, vocabulary slices); 0 skips")
    ap.add_argument("--no-harness", action="store_true",
                    help="skip the per-workload invariance report")
    ap.add_argument("--harness", default=",".join(WORKLOADS),
                    help="comma-separated subset of: " + ", ".join(WORKLOADS))
    ap.add_argument("--no-vendor", action="store_true",
                    help="skip the vendor-path context timing")
    ap.add_argument("--no-sclk", action="store_true",
                    help="skip sampling the shader clock under load")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="run one plain device copy of this many MiB before the "
                         "timed region (reference kernel for HBM counters)")
    args = ap.parse_args()
    variants = tuple(x for x in args.variants.split(",") if x)
    unknown = [x for x in variants if x not in VARIANTS]
    unknown += [x for x in args.harness.split(",") if x and x not in WORKLOADS]
    if unknown:
        print(f"bench.py: unknown variants {unknown}; choose from {VARIANTS} "
              f"and {WORKLOADS}", file=sys.stderr)
        return 2

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this path is measured on one GPU only; the row-sharded "
              "multi-GPU layout is described in the design notes but not run. "
              "Use --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import invariant_selected_token_amd as rlk
    from invariant_selected_token_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    case = synth.prefill_case()
    T, H, V = case.T, case.H, case.V
    log(f"bench: workload {case.name} on {torch.cuda.get_device_name(dev)}")

    def to_dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)

    hidden, weight = to_dev(case.hidden), to_dev(case.weight)
    targets = torch.from_numpy(case.targets).to(dev)
    ws = rlk.workspace_for(T, V, dev)
    # logp and lse in one buffer, so that one compare covers both
    out = torch.empty(2 * T, dtype=torch.float32, device=dev)
    logp, lse = out[:T], out[T:]
    ref_lp, ref_lse = rlk.rlk_selected_logp(hidden, weight, targets)
    ref = torch.cat([ref_lp, ref_lse])
    stats = torch.zeros((max(args.steps, 1), 8), dtype=torch.float64, device=dev)

    def step(i):
        rlk.rlk_vocab_stats(hidden, weight, targets, ws)
        rlk.rlk_vocab_merge(targets, ws, V, logp=logp, lse=lse)
        rlk.rlk_compare(out, ref, stats=stats[i])

    if args.calib_copy_mb > 0:
        n = args.calib_copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for i in range(args.warmup):
        step(0)
    torch.cuda.synchronize()
    stats.zero_()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        e = ev[i]
        e[0].record()
        rlk.rlk_vocab_stats(hidden, weight, targets, ws)
        e[1].record()
        rlk.rlk_vocab_merge(targets, ws, V, logp=logp, lse=lse)
        e[2].record()
        rlk.rlk_compare(out, ref, stats=stats[i])
        e[3].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    g_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(K)]
    m_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in range(K)]
    c_ms = [ev[i][2].elapsed_time(ev[i][3]) for i in range(K)]
    s_ms = [ev[i][0].elapsed_time(ev[i][3]) for i in range(K)]
    gemm_ms = sum(g_ms) / K
    merge_ms = sum(m_ms) / K
    check_ms = sum(c_ms) / K
    s_all = stats.cpu().numpy()
    mismatch = int(s_all[:, 1].sum())
    max_diff = float(s_all[:, 2].max())

    flops = 2.0 * T * H * V                      # algorithmic work per launch
    achieved = flops / (gemm_ms * 1e-3) / 1e12   # TFLOP/s
    nst = (V + 127) // 128
    merge_bytes = 8.0 * nst * T + 4.0 * T * 2 + 8.0 * T   # partials + xt + targets, logp + lse
    traffic = measured_traffic()
    out = {
        "metric": "selected-token logp tokens/s + % bf16 MFMA peak, Qwen3-8B LM head, 0 mismatch",
        "value": T * K / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": wall / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": case.name, "T": T, "H": H, "V": V,
                   "seq_len": 512, "n_seqs": T // 512, "seed": case.meta["seed"],
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic},
        "stages_ms": {"gemm_stats": gemm_ms, "merge": merge_ms, "consistency_check": check_ms},
        "stages_ms_median_min": {
            "gemm_stats": [statistics.median(g_ms), min(g_ms)],
            "merge": [statistics.median(m_ms), min(m_ms)],
            "step_on_device": [statistics.median(s_ms), min(s_ms)]},
        "merge_hbm": {"GB/s": merge_bytes / (merge_ms * 1e-3) / 1e9,
                      "peak": PEAK_HBM_GBS, "bytes": merge_bytes},
        "consistency": {"mismatch_count": mismatch, "max_abs_diff": max_diff,
                        "compared": 2 * T * K},
        "kernel_source": kernel_source_digest(),
    }
    if not args.no_sclk:
        log("bench: sampling the shader clock under the statistics kernel")
        clk = sample_sclk(torch, lambda: rlk.rlk_vocab_stats(hidden, weight, targets, ws))
        out["sclk"] = clk
        if clk:
            # the same achieved rate against the peak at the clock the load sustained
            peak_at = PEAK_BF16_TFLOPS * clk["median_MHz"] / 2400.0
            out["roofline"]["frac_at_measured_sclk"] = achieved / peak_at
            out["roofline"]["peak_at_measured_sclk"] = peak_at
    if not args.no_harness:
        log("bench: invariance report")
        hs = tuple(x for x in args.harness.split(",") if x)
        out["invariance"] = invariance_report(rlk, torch, np, (hidden, weight, targets), hs)
        torch.cuda.empty_cache()
    if not args.no_vendor:
        log("bench: vendor path (context)")
        out["vendor_context"] = vendor_context(torch, hidden, weight, targets, 10)
        torch.cuda.empty_cache()
    if args.variant_steps > 0:
        out["variants"] = time_variants(rlk, torch, np, hidden, weight, targets, T, H, V,
                                        args.variant_steps, flops, variants)
    if not args.no_cpu_baseline:
        log("bench: timing the fp64 oracle on the host")
        out["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0 if mismatch == 0 else 1


if __name__ == "__main__":
    sys.exit(main())
