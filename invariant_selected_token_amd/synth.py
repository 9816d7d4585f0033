"""Seeded synthetic inputs for the selected-token log-probability path.

This module is shared by the tests, the benchmark and the smoke check.  It
holds no arithmetic of the method itself: it only draws random numbers and
rounds them to bfloat16 bit patterns, so that the HIP path and the CPU oracle
can be fed the very same bytes.

Recipe.  Every draw comes from numpy ``Generator(PCG64(SeedSequence(key)))``
with key = [seed, stream, chunk]; stream 0 = hidden, 1 = weight, 2 = targets,
3 = extra structure.  Matrices are drawn in chunks of 8192 rows, chunk c from
its own stream key (so chunks can be drawn in parallel and the bytes do not
depend on the thread count):
  * hidden ~ N(0, 1) as float32, rounded to bfloat16 (round to nearest even,
    done with integer arithmetic on the fp32 bit pattern).
  * weight ~ N(0, 0.02^2) as float32 (standard normal times 0.02 in fp32),
    rounded to bfloat16 the same way.
  * targets ~ uniform integers in [0, V) (stream 2, chunk 0).
The shapes are the Qwen3-8B LM-head shape (H = 4096, V = 151936) that the
RL-Kernel blog's experiments use (sections 六 and 七: Qwen3-8B dense, seed
1234); base seed 1234, workload i uses 1234 + i.
"""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

QWEN3_8B_H = 4096
QWEN3_8B_V = 151936
BASE_SEED = 1234
CHUNK_ROWS = 8192
S_HIDDEN, S_WEIGHT, S_TARGETS, S_EXTRA = 0, 1, 2, 3
_THREADS = 8


def rng_for(seed: int, stream: int, chunk: int = 0) -> np.random.Generator:
    """The generator for one (seed, stream, chunk) key."""
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([seed, stream, chunk])))


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_exact_to_bf16_bits(x) -> np.ndarray:
    """float32 values that are already bfloat16-representable -> bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("value not representable in bfloat16")
    return (u >> np.uint32(16)).astype(np.uint16)


def _chunked(rows: int, fill) -> None:
    """Run fill(chunk_index, r0, r1) over 8192-row chunks on a thread pool."""
    jobs = [(c, r0, min(rows, r0 + CHUNK_ROWS))
            for c, r0 in enumerate(range(0, rows, CHUNK_ROWS))]
    if len(jobs) <= 1:
        for j in jobs:
            fill(*j)
        return
    with ThreadPoolExecutor(min(_THREADS, len(jobs))) as ex:
        list(ex.map(lambda j: fill(*j), jobs))


def normal_bf16(seed: int, stream: int, rows: int, cols: int,
                std: float) -> np.ndarray:
    """N(0, std^2) rounded to bfloat16 bits, [rows, cols]."""
    out = np.empty((rows, cols), dtype=np.uint16)

    def fill(c, r0, r1):
        x = rng_for(seed, stream, c).standard_normal((r1 - r0, cols),
                                                    dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[r0:r1] = f32_to_bf16_bits(x)

    _chunked(rows, fill)
    return out


def grid_bf16(seed: int, stream: int, rows: int, cols: int) -> np.ndarray:
    """Uniform over {-1, 0, 1} * 2^-4 as bfloat16 bits, [rows, cols]."""
    out = np.empty((rows, cols), dtype=np.uint16)
    lut = f32_exact_to_bf16_bits(np.array([-1, 0, 1], np.float32) *
                                 np.float32(2.0 ** -4))

    def fill(c, r0, r1):
        i = rng_for(seed, stream, c).integers(0, 3, size=(r1 - r0, cols),
                                             dtype=np.int8)
        out[r0:r1] = lut[i]

    _chunked(rows, fill)
    return out


@dataclass
class Case:
    name: str
    hidden: np.ndarray          # uint16 [T, H] bfloat16 bits
    weight: np.ndarray          # uint16 [V, H] bfloat16 bits
    targets: np.ndarray         # int32 [T]
    meta: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return int(self.hidden.shape[0])

    @property
    def H(self) -> int:
        return int(self.hidden.shape[1])

    @property
    def V(self) -> int:
        return int(self.weight.shape[0])


def normal_case(name: str, seed: int, T: int, H: int, V: int,
                hidden_std: float = 1.0, weight_std: float = 0.02) -> Case:
    """hidden ~ N(0,1), weight ~ N(0, 0.02^2), targets uniform in [0, V)."""
    hidden = normal_bf16(seed, S_HIDDEN, T, H, hidden_std)
    weight = normal_bf16(seed, S_WEIGHT, V, H, weight_std)
    targets = rng_for(seed, S_TARGETS).integers(0, V, size=T, dtype=np.int32)
    return Case(name, hidden, weight, targets,
                {"seed": seed, "hidden_std": hidden_std,
                 "weight_std": weight_std})


def tiny_case(seed: int = BASE_SEED + 1) -> Case:
    """T=64 rows, H=256, V=4096."""
    return normal_case("tiny_T64_H256_V4096", seed, 64, 256, 4096)


def prefill_case(seed: int = BASE_SEED + 2, T: int = 4096) -> Case:
    """Training-side recompute: T=4096 packed rows (8 sequences x 512)."""
    c = normal_case(f"qwen3_8b_lm_head_prefill_T{T}", seed, T, QWEN3_8B_H,
                    QWEN3_8B_V)
    c.meta["seq_len"] = 512
    c.meta["n_seqs"] = T // 512
    return c


DECODE_BATCH_SIZES = (1, 2, 3, 7, 16, 64, 255, 256)


def decode_plan(prefill_T: int = 4096, pool_size: int = 256,
                batch_sizes=DECODE_BATCH_SIZES,
                seed: int = BASE_SEED + 3) -> dict:
    """Rollout/decode sweep: a pool of prefill rows and one batch per size.

    The pool is ``pool_size`` distinct row indices of the prefill workload
    (drawn without replacement).  Batch B takes the first B entries of a fresh
    permutation of the pool, so each pooled vector lands at a random position.
    Returns {"pool": int64[pool_size], "batches": {B: int64[B] pool slots}}.
    """
    rng = rng_for(seed, S_EXTRA)
    pool = rng.choice(prefill_T, size=pool_size, replace=False).astype(np.int64)
    batches = {}
    for b in batch_sizes:
        batches[int(b)] = rng.permutation(pool_size)[:b].astype(np.int64)
    return {"pool": pool, "batches": batches}


def adversarial_case(seed: int = BASE_SEED + 4, T: int = 1024,
                     H: int = QWEN3_8B_H, V: int = QWEN3_8B_V) -> Case:
    """Coarse-grid contract stress (many exact ties, exact logits).

    hidden and weight are uniform over {-1, 0, 1} * 2^-4, so every product is
    a multiple of 2^-8 and every partial sum is exact in fp32.  Rows 0-15 are
    all zero (all logits equal).  Rows 16-31 are "dominant" rows: for a drawn
    index v*, hidden takes 0.5*sign(w[v*, k]) on the first 1280 k where
    w[v*, k] != 0 (zero elsewhere), so z[v*] = 1280 * 0.5 * 2^-4 = 40 exactly;
    rows 16-23 target v*, rows 24-31 a uniform target.  Rows 32-63 copy rows
    64-95 and get different targets.  H must allow 1280 non-zeros in w[v*].
    """
    hidden_f = bf16_bits_to_f32(grid_bf16(seed, S_HIDDEN, T, H))
    weight = grid_bf16(seed, S_WEIGHT, V, H)
    targets = rng_for(seed, S_TARGETS).integers(0, V, size=T, dtype=np.int32)
    rng = rng_for(seed, S_EXTRA)
    hidden_f[0:16] = 0.0
    vstar = rng.integers(0, V, size=16).astype(np.int64)
    for i, r in enumerate(range(16, 32)):
        wrow = bf16_bits_to_f32(weight[vstar[i]])
        nz = np.flatnonzero(wrow != 0.0)
        if nz.size < 1280:
            raise ValueError("weight row has fewer than 1280 non-zeros")
        sel = nz[:1280]
        hidden_f[r] = 0.0
        wf_sign = np.sign(wrow[sel]).astype(np.float32)
        hidden_f[r, sel] = np.float32(0.5) * wf_sign
        if r < 24:
            targets[r] = np.int32(vstar[i])
    hidden_f[32:64] = hidden_f[64:96]
    dup_targets = rng.integers(0, V, size=32, dtype=np.int32)
    same = dup_targets == targets[64:96]
    dup_targets[same] = (dup_targets[same] + 1) % V
    targets[32:64] = dup_targets
    hidden = f32_exact_to_bf16_bits(hidden_f)
    return Case(f"adversarial_grid_T{T}", hidden, weight, targets,
                {"seed": seed, "vstar": vstar, "zero_rows": (0, 16),
                 "dominant_rows": (16, 32), "dup_rows": (32, 64),
                 "dup_of": (64, 96)})


def long_rollout_case(seed: int = BASE_SEED + 5, T: int = 16384) -> Case:
    """Long rollout: T=16384 rows (32 responses x 512), config-2 distributions.

    ``targets`` here are uniform placeholders; ``meta["u"]`` holds one uniform
    draw per row in [0, 1) for drawing the targets from the model's own
    softmax (done by the caller that owns a softmax).
    """
    c = normal_case(f"qwen3_8b_lm_head_rollout_T{T}", seed, T, QWEN3_8B_H,
                    QWEN3_8B_V)
    c.meta["u"] = rng_for(seed, S_EXTRA).random(T)
    c.meta["seq_len"] = 512
    c.meta["n_seqs"] = T // 512
    return c


def upstream_grad(T: int, seed: int) -> np.ndarray:
    """An upstream gradient dL/dlogp for the backward: N(0, 1) as float32."""
    return np.random.Generator(np.random.PCG64(seed)).normal(size=T).astype(np.float32)


def fingerprint(case: Case, targets=None) -> str:
    """A short digest of a workload's bytes (hidden, weight, targets), so that
    values stored for it can tell when the generator has changed."""
    import hashlib
    h = hashlib.sha256()
    for a in (case.hidden, case.weight,
              case.targets if targets is None else np.asarray(targets, np.int32)):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()[:24]
