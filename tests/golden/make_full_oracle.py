#!/usr/bin/env python3
"""Writes tests/golden/full_size_oracle.npz: the fp64 oracle's outputs for
EVERY row of the full-size workloads, so that the GPU tests can compare every
row without running the oracle for minutes inside a test.

Only the oracle (oracle/) and the seeded input generators (synth) are called;
the stored values are the oracle's, for inputs named by a fingerprint of their
bytes (a test refuses a file whose fingerprint does not match the generator).
Parts (all by default; --parts a,b recomputes only those and keeps the rest
of an existing file):

  prefill          T = 4096 packed rows, H = 4096, V = 151936: logp, lse;
  prefill_gw       24 rows of grad_weight for an upstream gradient N(0, 1)
                   (seed 15), with each element's tolerance, the backward's
                   bound (2^-8 + (T + 16) 2^-24) (|dz|^T |h|) + 1e-6 computed
                   from the oracle's dz;
  prefill_options  logp, lse and entropy with inverse temperature 0.7;
  prefill_topk     the 32 largest log-probabilities of every row and their ids
                   (decreasing, ties to the smaller id);
  adversarial      T = 1024 coarse-grid rows: logp, lse;
  adversarial_sums per row, three exact integer checksums of the oracle's
                   logits q = 256 z (every coarse-grid logit is a multiple of
                   2^-8 below 2^12 in magnitude, so q is an exact integer):
                   sum_v q, sum_v q^2 and sum_v (v + 1) q;
  rollout          T = 16384 rows: targets drawn from the oracle's own softmax
                   by inverse CDF with the workload's one uniform per row,
                   then logp, lse.

Run:  python tests/golden/make_full_oracle.py [--parts ...] [--dry]
(all parts: about 40 minutes on 8 cores; --dry runs every step on small
versions of the workloads and writes to /tmp).
"""

from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from invariant_selected_token_amd import synth  # noqa: E402
from oracle import oracle as orc  # noqa: E402

OUT = os.path.join(HERE, "full_size_oracle.npz")
DRY_OUT = "/tmp/full_size_oracle_dry.npz"
PARTS = ("prefill", "prefill_gw", "prefill_options", "prefill_topk", "adversarial",
         "adversarial_sums", "rollout")
ROLLOUT_CHUNK = 512
GW_SEED = 15
N_GW_ROWS = 24
OPTIONS_INV_TAU = 0.7
TOPK_STORED = 32


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


def grad_weight_rows(c, rng):
    """24 vocabulary rows: 11 that are targets of some row (the one-hot term
    matters there), 8 that are nobody's target, and rows at tile edges."""
    tgt = np.unique(c.targets)
    non = np.setdiff1d(np.arange(c.V), tgt)
    edges = np.array([0, 127, 128, 255, c.V - 1], np.int64)
    rows = np.concatenate([edges, rng.choice(tgt, 11, replace=False),
                           rng.choice(non, 8, replace=False)])
    rows = np.unique(rows)
    assert rows.size == N_GW_ROWS, rows.size
    return rows


def part_prefill(c, out):
    lp, lse = orc.selected_logp(c.hidden, c.weight, c.targets)
    out["prefill_logp"], out["prefill_lse"] = lp, lse


def part_prefill_gw(c, out):
    g = synth.upstream_grad(c.T, GW_SEED).astype(np.float64)
    rows = grad_weight_rows(c, np.random.Generator(np.random.PCG64(2025)))
    _, gw = orc.selected_logp_backward(c.hidden, c.weight, c.targets, g,
                                       want_hidden=False, want_weight=True)
    out["prefill_gw_rows"] = rows
    out["prefill_gw"] = np.ascontiguousarray(gw[rows])
    del gw
    dz = orc.grad_logits(c.hidden, c.weight, c.targets, g)
    habs = np.abs(synth.bf16_bits_to_f32(c.hidden).astype(np.float64))
    bound = (2.0 ** -8 + (c.T + 16) * 2.0 ** -24) * (np.abs(dz[:, rows]).T @ habs) + 1e-6
    # a tolerance, stored in fp32 rounded outwards
    out["prefill_gw_bound"] = (bound * (1.0 + 2.0 ** -20)).astype(np.float32)
    out["prefill_gw_seed"] = np.array(GW_SEED, np.int32)


def part_prefill_options(c, out):
    lp, lse, ent = orc.selected_logp_ex(c.hidden, c.weight, c.targets, inv_tau=OPTIONS_INV_TAU)
    out["prefill_opt_inv_tau"] = np.array(OPTIONS_INV_TAU)
    out["prefill_opt_logp"], out["prefill_opt_lse"], out["prefill_opt_entropy"] = lp, lse, ent


def part_prefill_topk(c, out, chunk=512):
    lp = np.empty((c.T, TOPK_STORED))
    ids = np.empty((c.T, TOPK_STORED), np.int32)
    for r0 in range(0, c.T, chunk):
        r1 = min(c.T, r0 + chunk)
        lp[r0:r1], ids[r0:r1] = orc.topk_logp(c.hidden[r0:r1], c.weight, TOPK_STORED)
    out["prefill_topk_logp"], out["prefill_topk_ids"] = lp, ids


def part_adversarial(c, out):
    lp, lse = orc.selected_logp(c.hidden, c.weight, c.targets)
    out["adversarial_logp"], out["adversarial_lse"] = lp, lse


def part_adversarial_sums(c, out, chunk=128):
    sums = np.empty((c.T, 3), np.int64)
    w = np.arange(1, c.V + 1, dtype=np.int64)
    for r0 in range(0, c.T, chunk):
        r1 = min(c.T, r0 + chunk)
        q = orc.logits(c.hidden[r0:r1], c.weight) * 256.0
        qi = np.rint(q).astype(np.int64)
        assert np.array_equal(qi.astype(np.float64), q), "a grid logit is not a multiple of 2^-8"
        sums[r0:r1, 0] = qi.sum(axis=1)
        sums[r0:r1, 1] = (qi * qi).sum(axis=1)
        sums[r0:r1, 2] = (qi * w).sum(axis=1)
    out["adversarial_logit_sums"] = sums


def part_rollout(c, out):
    u = c.meta["u"]
    y = np.empty(c.T, np.int32)
    lp = np.empty(c.T)
    lse = np.empty(c.T)
    t0 = time.time()
    for r0 in range(0, c.T, ROLLOUT_CHUNK):
        r1 = min(c.T, r0 + ROLLOUT_CHUNK)
        z = orc.logits(c.hidden[r0:r1], c.weight)
        _, lse0 = orc.lse_from_logits(z, np.zeros(r1 - r0, np.int32))
        ls = z - lse0[:, None]                    # log-softmax, to draw targets from
        if r0 == 0:                               # the same bits as the oracle's own
            ref = orc.log_softmax(c.hidden[:4], c.weight)
            assert np.array_equal(ref, ls[:4]), "log-softmax recipe differs"
        y[r0:r1] = orc.sample_targets(ls, u[r0:r1])
        del ls
        lp[r0:r1], lse[r0:r1] = orc.lse_from_logits(z, y[r0:r1])
        del z
        log(f"rollout rows {r0}..{r1 - 1} done ({time.time() - t0:.0f} s)")
    out["rollout_fingerprint"] = np.array(synth.fingerprint(c, y))
    out["rollout_targets"], out["rollout_logp"], out["rollout_lse"] = y, lp, lse


def main(parts, dry=False):
    path = DRY_OUT if dry else OUT
    out = {}
    if os.path.exists(path) and set(parts) != set(PARTS):
        with np.load(path, allow_pickle=False) as old:
            out = {k: old[k] for k in old.files}
    out["oracle_version"] = np.array(orc._load().oracle_version(), np.int32)
    kw = (lambda T: {"T": T}) if dry else (lambda T: {})
    t_all = time.time()
    log(f"parts {parts} on {orc.max_threads()} threads")
    if any(p.startswith("prefill") for p in parts):
        c = synth.prefill_case(**kw(128))
        out["prefill_fingerprint"] = np.array(synth.fingerprint(c))
        for p, fn in (("prefill", part_prefill), ("prefill_gw", part_prefill_gw),
                      ("prefill_options", part_prefill_options),
                      ("prefill_topk", part_prefill_topk)):
            if p in parts:
                t0 = time.time()
                fn(c, out)
                log(f"{p} done in {time.time() - t0:.0f} s")
        del c
    if any(p.startswith("adversarial") for p in parts):
        c = synth.adversarial_case(**kw(128))
        out["adversarial_fingerprint"] = np.array(synth.fingerprint(c))
        for p, fn in (("adversarial", part_adversarial),
                      ("adversarial_sums", part_adversarial_sums)):
            if p in parts:
                t0 = time.time()
                fn(c, out)
                log(f"{p} done in {time.time() - t0:.0f} s")
        del c
    if "rollout" in parts:
        part_rollout(synth.long_rollout_case(**kw(1024)), out)
    np.savez(path, **out)
    log(f"wrote {path} ({os.path.getsize(path)} bytes) in {time.time() - t_all:.0f} s")


if __name__ == "__main__":
    args = sys.argv[1:]
    sel = PARTS
    if "--parts" in args:
        sel = tuple(args[args.index("--parts") + 1].split(","))
        unknown = set(sel) - set(PARTS)
        if unknown:
            sys.exit(f"unknown parts {sorted(unknown)}; choose from {PARTS}")
    main(sel, dry="--dry" in args)
