"""ctypes wrapper around the fp64 CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library.

What the oracle computes is the selected-token log-probability as the
RL-Kernel blog defines it (section 四, the Linear-LogP reduction class): logits
``z = h . w_v`` over the whole vocabulary, ``lse = log sum_v exp(z_v)`` in the
max-shifted form ``m + log sum exp(z - m)``, and ``logp = z_y - lse`` read at
the target token.  All arithmetic is fp64 in ``oracle.c``; this module only
marshals numpy arrays.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

# Plain C, no fast-math, no FMA contraction; OpenMP over rows only.
BUILD_CMD = [
    "gcc", "-O3", "-std=c11", "-fopenmp", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-march=x86-64-v3",
    _SRC, "-o", _LIB_PATH, "-lm",
]

_lib = None


def build() -> str:
    """Compile ``liboracle.so`` next to its source (always recompiles)."""
    subprocess.run(BUILD_CMD, check=True)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, c_int = ctypes.c_int64, ctypes.c_int
    vp = ctypes.c_void_p
    lib.oracle_version.restype = c_int
    lib.oracle_max_threads.restype = c_int
    lib.oracle_logits.argtypes = [vp, i64, vp, i64, i64, i64, i64, vp, c_int]
    lib.oracle_logits.restype = c_int
    lib.oracle_logits_naive.argtypes = [vp, i64, vp, i64, i64, i64, i64, vp]
    lib.oracle_logits_naive.restype = c_int
    lib.oracle_lse_from_logits.argtypes = [vp, vp, i64, i64, vp, vp]
    lib.oracle_lse_from_logits.restype = None
    lib.oracle_selected_logp.argtypes = [vp, i64, vp, i64, vp, i64, i64, i64,
                                         vp, vp, c_int]
    lib.oracle_selected_logp.restype = c_int
    lib.oracle_log_softmax.argtypes = [vp, i64, vp, i64, i64, i64, i64, vp,
                                       c_int]
    lib.oracle_log_softmax.restype = c_int
    lib.oracle_round_bf16.argtypes = [vp, i64, vp]
    lib.oracle_round_bf16.restype = None
    lib.oracle_ex_from_logits.argtypes = [vp, vp, i64, i64, ctypes.c_double, c_int,
                                          vp, vp, vp]
    lib.oracle_ex_from_logits.restype = None
    lib.oracle_selected_logp_ex.argtypes = [vp, i64, vp, i64, vp, i64, i64, i64,
                                            ctypes.c_double, c_int, vp, vp, vp, c_int]
    lib.oracle_selected_logp_ex.restype = c_int
    lib.oracle_logp_grad_logits.argtypes = [vp, i64, vp, i64, vp, vp, i64, i64, i64,
                                            ctypes.c_double, vp, c_int]
    lib.oracle_logp_grad_logits.restype = c_int
    lib.oracle_selected_logp_backward.argtypes = [vp, i64, vp, i64, vp, vp, i64, i64, i64,
                                                  ctypes.c_double, vp, vp, c_int]
    lib.oracle_selected_logp_backward.restype = c_int
    lib.oracle_rmsnorm.argtypes = [vp, i64, vp, ctypes.c_double, i64, i64, vp, vp]
    lib.oracle_rmsnorm.restype = None
    lib.oracle_topk_logp.argtypes = [vp, i64, vp, i64, i64, i64, i64, c_int, ctypes.c_double,
                                     c_int, vp, vp, c_int]
    lib.oracle_topk_logp.restype = c_int
    lib.oracle_topk_from_logits.argtypes = [vp, i64, i64, c_int, ctypes.c_double, c_int, vp, vp]
    lib.oracle_topk_from_logits.restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _bf16_2d(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16 or a.ndim != 2:
        raise TypeError("expected a 2-D uint16 array of bfloat16 bit patterns")
    return a


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def logits(hidden, weight, nthreads: int = 0) -> np.ndarray:
    """fp64 logits z[t, v] = sum_k h[t, k] w[v, k]."""
    lib = _load()
    h, w = _bf16_2d(hidden), _bf16_2d(weight)
    T, H = h.shape
    V = w.shape[0]
    if w.shape[1] != H:
        raise ValueError("hidden and weight disagree on H")
    z = np.empty((T, V), dtype=np.float64)
    if lib.oracle_logits(_ptr(h), H, _ptr(w), H, T, H, V, _ptr(z), nthreads):
        raise MemoryError("oracle_logits failed")
    return z


def logits_naive(hidden, weight) -> np.ndarray:
    """Same logits, one dot product at a time (single thread)."""
    lib = _load()
    h, w = _bf16_2d(hidden), _bf16_2d(weight)
    T, H = h.shape
    V = w.shape[0]
    z = np.empty((T, V), dtype=np.float64)
    if lib.oracle_logits_naive(_ptr(h), H, _ptr(w), H, T, H, V, _ptr(z)):
        raise MemoryError("oracle_logits_naive failed")
    return z


def lse_from_logits(z, targets):
    """(logp, lse) of logits given directly, shape [T, V] fp64."""
    lib = _load()
    z = np.ascontiguousarray(z, dtype=np.float64)
    if z.ndim != 2:
        raise ValueError("z must be 2-D")
    T, V = z.shape
    y = np.ascontiguousarray(targets, dtype=np.int32)
    if y.shape != (T,):
        raise ValueError("targets must have shape [T]")
    logp = np.empty(T, dtype=np.float64)
    lse = np.empty(T, dtype=np.float64)
    lib.oracle_lse_from_logits(_ptr(z), _ptr(y), T, V, _ptr(logp), _ptr(lse))
    return logp, lse


def selected_logp(hidden, weight, targets, nthreads: int = 0):
    """(logp[T], lse[T]) in fp64 for bf16 hidden [T, H], weight [V, H]."""
    lib = _load()
    h, w = _bf16_2d(hidden), _bf16_2d(weight)
    T, H = h.shape
    V = w.shape[0]
    if w.shape[1] != H:
        raise ValueError("hidden and weight disagree on H")
    y = np.ascontiguousarray(targets, dtype=np.int32)
    if y.shape != (T,):
        raise ValueError("targets must have shape [T]")
    logp = np.empty(T, dtype=np.float64)
    lse = np.empty(T, dtype=np.float64)
    if lib.oracle_selected_logp(_ptr(h), H, _ptr(w), H, _ptr(y), T, H, V,
                                _ptr(logp), _ptr(lse), nthreads):
        raise MemoryError("oracle_selected_logp failed")
    return logp, lse


def log_softmax(hidden, weight, nthreads: int = 0) -> np.ndarray:
    """Full-row fp64 log-softmax [T, V]."""
    lib = _load()
    h, w = _bf16_2d(hidden), _bf16_2d(weight)
    T, H = h.shape
    V = w.shape[0]
    out = np.empty((T, V), dtype=np.float64)
    if lib.oracle_log_softmax(_ptr(h), H, _ptr(w), H, T, H, V, _ptr(out),
                              nthreads):
        raise MemoryError("oracle_log_softmax failed")
    return out


def round_bf16(x) -> np.ndarray:
    """fp32 values rounded to bfloat16 (to nearest, ties to even), as fp64."""
    lib = _load()
    a = np.ascontiguousarray(x, dtype=np.float32).ravel()
    out = np.empty(a.size, dtype=np.float64)
    lib.oracle_round_bf16(_ptr(a), a.size, _ptr(out))
    return out.reshape(np.shape(x))


def ex_from_logits(z, targets, inv_tau: float = 1.0, bf16: bool = False):
    """(logp, lse, entropy) of fp64 logits [T, V] given directly, after the
    contract options (z * inv_tau, then optionally fp32 -> bf16 rounding)."""
    lib = _load()
    z = np.ascontiguousarray(z, dtype=np.float64)
    if z.ndim != 2:
        raise ValueError("z must be 2-D")
    T, V = z.shape
    y = np.ascontiguousarray(targets, dtype=np.int32)
    if y.shape != (T,):
        raise ValueError("targets must have shape [T]")
    logp, lse, ent = (np.empty(T, dtype=np.float64) for _ in range(3))
    lib.oracle_ex_from_logits(_ptr(z), _ptr(y), T, V, float(inv_tau), int(bool(bf16)),
                              _ptr(logp), _ptr(lse), _ptr(ent))
    return logp, lse, ent


def selected_logp_ex(hidden, weight, targets, inv_tau: float = 1.0, bf16: bool = False,
                     nthreads: int = 0):
    """(logp, lse, entropy) in fp64 with the contract options: every logit
    multiplied by ``inv_tau`` and, with ``bf16``, rounded fp32 -> bf16."""
    lib = _load()
    h, w = _bf16_2d(hidden), _bf16_2d(weight)
    T, H = h.shape
    V = w.shape[0]
    if w.shape[1] != H:
        raise ValueError("hidden and weight disagree on H")
    y = np.ascontiguousarray(targets, dtype=np.int32)
    if y.shape != (T,):
        raise ValueError("targets must have shape [T]")
    logp, lse, ent = (np.empty(T, dtype=np.float64) for _ in range(3))
    if lib.oracle_selected_logp_ex(_ptr(h), H, _ptr(w), H, _ptr(y), T, H, V,
                                   float(inv_tau), int(bool(bf16)), _ptr(logp),
                                   _ptr(lse), _ptr(ent), nthreads):
        raise MemoryError("oracle_selected_logp_ex failed")
    return logp, lse, ent


def _bwd_args(hidden, weight, targets, grad_logp):
    h, w = _bf16_2d(hidden), _bf16_2d(weight)
    T, H = h.shape
    V = w.shape[0]
    if w.shape[1] != H:
        raise ValueError("hidden and weight disagree on H")
    y = np.ascontiguousarray(targets, dtype=np.int32)
    g = np.ascontiguousarray(grad_logp, dtype=np.float64)
    if y.shape != (T,) or g.shape != (T,):
        raise ValueError("targets and grad_logp must have shape [T]")
    return h, w, y, g, T, H, V


def grad_logits(hidden, weight, targets, grad_logp, inv_tau: float = 1.0,
                nthreads: int = 0) -> np.ndarray:
    """dz [T, V] = g inv_tau (onehot(y) - softmax(inv_tau z)), fp64; rows with
    an out-of-range target are 0."""
    lib = _load()
    h, w, y, g, T, H, V = _bwd_args(hidden, weight, targets, grad_logp)
    dz = np.empty((T, V), dtype=np.float64)
    if lib.oracle_logp_grad_logits(_ptr(h), H, _ptr(w), H, _ptr(y), _ptr(g), T, H, V,
                                   float(inv_tau), _ptr(dz), nthreads):
        raise MemoryError("oracle_logp_grad_logits failed")
    return dz


def selected_logp_backward(hidden, weight, targets, grad_logp, inv_tau: float = 1.0,
                           want_hidden: bool = True, want_weight: bool = True,
                           nthreads: int = 0):
    """(grad_hidden [T, H] or None, grad_weight [V, H] or None) in fp64 for
    L = sum_t grad_logp[t] logp[t]."""
    lib = _load()
    h, w, y, g, T, H, V = _bwd_args(hidden, weight, targets, grad_logp)
    gh = np.empty((T, H), dtype=np.float64) if want_hidden else None
    gw = np.empty((V, H), dtype=np.float64) if want_weight else None
    if lib.oracle_selected_logp_backward(_ptr(h), H, _ptr(w), H, _ptr(y), _ptr(g), T, H, V,
                                         float(inv_tau),
                                         _ptr(gh) if gh is not None else None,
                                         _ptr(gw) if gw is not None else None, nthreads):
        raise MemoryError("oracle_selected_logp_backward failed")
    return gh, gw


def rmsnorm(x, gamma, eps: float = 1e-6, want_xr: bool = False):
    """bf16 bits [T, H] of y = bf16(bf16(x r) gamma), r = 1/sqrt(mean(x^2) + eps)
    per row (fp64 arithmetic, roundings as the module doc states); with
    ``want_xr`` also the unrounded x r (fp64)."""
    lib = _load()
    xb = _bf16_2d(x)
    T, H = xb.shape
    g = np.ascontiguousarray(gamma)
    if g.dtype != np.uint16 or g.shape != (H,):
        raise TypeError("gamma must be a uint16 [H] array of bfloat16 bit patterns")
    out = np.empty((T, H), dtype=np.uint16)
    xr = np.empty((T, H), dtype=np.float64) if want_xr else None
    lib.oracle_rmsnorm(_ptr(xb), H, _ptr(g), float(eps), T, H, _ptr(out),
                       _ptr(xr) if xr is not None else None)
    return (out, xr) if want_xr else out


def topk_logp(hidden, weight, k: int, inv_tau: float = 1.0, bf16: bool = False,
              nthreads: int = 0):
    """(logp [T, k] fp64, ids [T, k] int32): the k largest entries of
    log softmax(z') per row, decreasing, ties to the smaller id."""
    lib = _load()
    h, w = _bf16_2d(hidden), _bf16_2d(weight)
    T, H = h.shape
    V = w.shape[0]
    lp = np.empty((T, k), dtype=np.float64)
    ids = np.empty((T, k), dtype=np.int32)
    if lib.oracle_topk_logp(_ptr(h), H, _ptr(w), H, T, H, V, int(k), float(inv_tau),
                            int(bool(bf16)), _ptr(lp), _ptr(ids), nthreads):
        raise MemoryError("oracle_topk_logp failed")
    return lp, ids


def topk_from_logits(z, k: int, inv_tau: float = 1.0, bf16: bool = False):
    """The same selection on fp64 logits [T, V] given directly."""
    lib = _load()
    z = np.ascontiguousarray(z, dtype=np.float64)
    T, V = z.shape
    lp = np.empty((T, k), dtype=np.float64)
    ids = np.empty((T, k), dtype=np.int32)
    lib.oracle_topk_from_logits(_ptr(z), T, V, int(k), float(inv_tau), int(bool(bf16)),
                                _ptr(lp), _ptr(ids))
    return lp, ids


def sample_targets(log_probs: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Draw one target per row from the oracle's softmax by inverse CDF.

    ``u`` holds one uniform draw in [0, 1) per row (an input, supplied by the
    seeded generator).  The target is the smallest v whose fp64 cumulative
    probability, summed in index order, reaches ``u * total``.
    """
    p = np.exp(np.asarray(log_probs, dtype=np.float64))
    c = np.cumsum(p, axis=1)
    thresh = np.asarray(u, dtype=np.float64) * c[:, -1]
    idx = np.array([np.searchsorted(c[i], thresh[i], side="left")
                    for i in range(c.shape[0])], dtype=np.int64)
    return np.minimum(idx, c.shape[1] - 1).astype(np.int32)


def compare_stats(a, b) -> dict:
    """Consistency statistics of two fp32 log-probability arrays.

    ``a`` plays the training side, ``b`` the rollout side.  Definitions follow
    the pages: the mismatch count and the maximum absolute logp difference
    (RL-Kernel blog, sections 六 and 七), and the per-token absolute
    difference's max, mean and standard deviation plus the k3 estimator
    ``r - 1 - log r`` with ``r = p_train / p_rollout = exp(a - b)`` (vLLM
    blog summary on papercache.org, "diff = 0" definition).

    A row is a mismatch when the two fp32 bit patterns differ.  Absolute
    differences are taken in fp64; a row whose bit patterns are equal counts
    0, a row where exactly one side is NaN counts +inf.  The k3 sum runs over
    rows where both sides are finite.
    """
    a = np.ascontiguousarray(a, dtype=np.float32).ravel()
    b = np.ascontiguousarray(b, dtype=np.float32).ravel()
    if a.shape != b.shape:
        raise ValueError("shape mismatch")
    n = a.size
    same = a.view(np.uint32) == b.view(np.uint32)
    a64, b64 = a.astype(np.float64), b.astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        d = np.abs(a64 - b64)
    d = np.where(same, 0.0, d)
    d = np.where(np.isnan(d), np.inf, d)
    fin = np.isfinite(a64) & np.isfinite(b64)
    lr = a64[fin] - b64[fin]
    k3 = np.exp(lr) - 1.0 - lr
    out = {
        "n": int(n),
        "mismatch_count": int(n - np.count_nonzero(same)),
        "max_abs_diff": float(d.max()) if n else 0.0,
        "mean_abs_diff": float(d.mean()) if n else 0.0,
        "std_abs_diff": float(d.std()) if n else 0.0,
        "k3_mean": float(k3.mean()) if k3.size else 0.0,
    }
    return out
