"""Python binding of the batch-invariant selected-token log-probability library.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``librlk.so`` (built from ``csrc/`` for gfx950).  Function names
match the C entry points declared in ``include/rlk.h``.  There is no fallback:
if the library is missing, every call raises.

Tensors are PyTorch device tensors (PyTorch provides device memory and
streams).  bfloat16 operands may be given as ``torch.bfloat16`` or as 16-bit
integer tensors holding the bit patterns.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librlk.so")

RLK_OK = 0
RLK_ERR_NULL_POINTER = 1
RLK_ERR_INVALID_SHAPE = 2
RLK_ERR_UNSUPPORTED = 3
RLK_ERR_MISALIGNED = 4
RLK_ERR_WORKSPACE_TOO_SMALL = 5
RLK_ERR_HIP = 6
RLK_ERR_INVALID_VALUE = 7
RLK_ERR_SCRATCH_LIMIT = 8
RLK_NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024

RLK_LOGITS_BF16 = 1
RLK_ENTROPY = 2

EXPORTED = (
    "rlk_abi_version", "rlk_status_string", "rlk_last_hip_error",
    "rlk_vocab_tile", "rlk_selected_logp_workspace_bytes", "rlk_workspace_layout",
    "rlk_selected_logp", "rlk_vocab_stats", "rlk_vocab_stats_shard",
    "rlk_vocab_merge", "rlk_debug_logits", "rlk_logits", "rlk_compare",
    "rlk_workspace_bytes_ex",
    "rlk_selected_logp_ex", "rlk_vocab_stats_ex", "rlk_vocab_merge_ex",
    "rlk_selected_logp_backward_workspace_bytes", "rlk_selected_logp_backward",
    "rlk_logp_grad_logits", "rlk_rmsnorm", "rlk_topk_logp", "rlk_selected_logp_noalloc",
    "rlk_topk_logp_direct_workspace_bytes", "rlk_topk_logp_direct",
)

_lib = None


class RLKError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: status {status}: {rlk_status_string(status)}"
        if status == RLK_ERR_HIP:
            msg += f" (hipError {rlk_last_hip_error()})"
        super().__init__(msg)


def lib() -> ctypes.CDLL:
    """The loaded ``librlk.so`` (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m invariant_selected_token_amd.build`")
    # torch's HIP runtime must be the process's only one: librlk.so asks for
    # libamdhip64.so.7, which binds to torch's copy (same soname) when torch is
    # loaded first; loaded the other way round, torch would map a second
    # runtime next to the system one and the two would not share devices.
    _torch()
    L = ctypes.CDLL(LIB_PATH)
    i64, sz, vp, c_int = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int
    L.rlk_abi_version.restype = c_int
    L.rlk_status_string.argtypes = [c_int]
    L.rlk_status_string.restype = ctypes.c_char_p
    L.rlk_last_hip_error.restype = c_int
    L.rlk_vocab_tile.restype = c_int
    L.rlk_selected_logp_workspace_bytes.argtypes = [i64, i64, i64]
    L.rlk_selected_logp_workspace_bytes.restype = sz
    psz = ctypes.POINTER(sz)
    L.rlk_workspace_layout.argtypes = [i64, i64, c_int, psz, psz, psz, psz]
    L.rlk_workspace_layout.restype = c_int
    L.rlk_selected_logp.argtypes = [vp, i64, vp, i64, vp, vp, vp, i64, i64, i64,
                                    vp, sz, vp]
    L.rlk_selected_logp.restype = c_int
    L.rlk_selected_logp_noalloc.argtypes = [vp, i64, vp, i64, vp, vp, vp, i64, i64, i64, vp]
    L.rlk_selected_logp_noalloc.restype = c_int
    L.rlk_vocab_stats.argtypes = [vp, i64, vp, i64, vp, i64, i64, i64, vp, sz, vp]
    L.rlk_vocab_stats.restype = c_int
    L.rlk_vocab_stats_shard.argtypes = [vp, i64, vp, i64, vp, i64, i64, i64, i64, i64,
                                        vp, sz, vp]
    L.rlk_vocab_stats_shard.restype = c_int
    L.rlk_vocab_merge.argtypes = [vp, vp, vp, i64, i64, vp, sz, vp]
    L.rlk_vocab_merge.restype = c_int
    for name in ("rlk_debug_logits", "rlk_logits"):
        getattr(L, name).argtypes = [vp, i64, vp, i64, vp, i64, i64, i64, vp]
        getattr(L, name).restype = c_int
    L.rlk_compare.argtypes = [vp, vp, i64, vp, vp]
    L.rlk_compare.restype = c_int
    f32 = ctypes.c_float
    L.rlk_workspace_bytes_ex.argtypes = [i64, i64, c_int]
    L.rlk_workspace_bytes_ex.restype = sz
    L.rlk_selected_logp_ex.argtypes = [vp, i64, vp, i64, vp, vp, vp, vp, i64, i64, i64,
                                       f32, c_int, vp, sz, vp]
    L.rlk_selected_logp_ex.restype = c_int
    L.rlk_vocab_stats_ex.argtypes = [vp, i64, vp, i64, vp, i64, i64, i64, i64, i64, f32,
                                     c_int, vp, sz, vp]
    L.rlk_vocab_stats_ex.restype = c_int
    L.rlk_vocab_merge_ex.argtypes = [vp, vp, vp, vp, i64, i64, c_int, vp, sz, vp]
    L.rlk_vocab_merge_ex.restype = c_int
    L.rlk_selected_logp_backward_workspace_bytes.argtypes = [i64, i64, i64]
    L.rlk_selected_logp_backward_workspace_bytes.restype = sz
    L.rlk_selected_logp_backward.argtypes = [vp, i64, vp, i64, vp, vp, vp, vp, vp, i64, i64,
                                             i64, f32, vp, sz, vp]
    L.rlk_selected_logp_backward.restype = c_int
    L.rlk_logp_grad_logits.argtypes = [vp, i64, vp, i64, vp, vp, vp, vp, i64, i64, i64, i64,
                                       f32, vp]
    L.rlk_logp_grad_logits.restype = c_int
    L.rlk_rmsnorm.argtypes = [vp, i64, vp, f32, vp, i64, i64, i64, vp]
    L.rlk_rmsnorm.restype = c_int
    L.rlk_topk_logp.argtypes = [vp, i64, vp, vp, sz, i64, i64, c_int, f32, c_int, vp, vp, vp]
    L.rlk_topk_logp.restype = c_int
    L.rlk_topk_logp_direct_workspace_bytes.argtypes = [i64, i64, c_int, i64]
    L.rlk_topk_logp_direct_workspace_bytes.restype = sz
    L.rlk_topk_logp_direct.argtypes = [vp, i64, vp, i64, vp, vp, sz, i64, i64, i64, c_int, f32,
                                       c_int, i64, vp, sz, vp, vp, vp]
    L.rlk_topk_logp_direct.restype = c_int
    _lib = L
    return L


def rlk_abi_version() -> int:
    return int(lib().rlk_abi_version())


def rlk_status_string(status: int) -> str:
    return lib().rlk_status_string(int(status)).decode()


def rlk_last_hip_error() -> int:
    return int(lib().rlk_last_hip_error())


def rlk_vocab_tile() -> int:
    return int(lib().rlk_vocab_tile())


def rlk_selected_logp_workspace_bytes(T: int, H: int, V: int) -> int:
    return int(lib().rlk_selected_logp_workspace_bytes(int(T), int(H), int(V)))


def rlk_workspace_layout(T: int, V: int, flags: int = 0) -> dict:
    """Byte offsets of the workspace regions for (T, V, flags): part_m and
    part_s ([ceil(V/128)][T] fp32, tile-major), xt ([T] fp32) and part_u."""
    offs = [ctypes.c_size_t(0) for _ in range(4)]
    _call("rlk_workspace_layout", lib().rlk_workspace_layout(
        int(T), int(V), int(flags), *[ctypes.byref(o) for o in offs]))
    return dict(zip(("part_m", "part_s", "xt", "part_u"), (int(o.value) for o in offs)))


def rlk_workspace_bytes_ex(T: int, V: int, flags: int) -> int:
    return int(lib().rlk_workspace_bytes_ex(int(T), int(V), int(flags)))


# ---------------------------------------------------------------- tensors --

def _torch():
    import torch
    return torch


def _check_device(name, t, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (cuda) tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _bf16_operand(name, t, device=None):
    torch = _torch()
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must be bfloat16 (or 16-bit bit patterns)")
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit column stride")
    _check_device(name, t, device)
    return t.data_ptr(), t.stride(0)


def _on(stream):
    """Allocations made inside belong to ``stream`` (the side stream the call
    runs on), so the caching allocator does not hand their memory to other
    work while that stream's kernels still use it."""
    import contextlib
    return _torch().cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _stream_ptr(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _call(where, status):
    if status != RLK_OK:
        raise RLKError(status, where)


def _prepare(hidden, weight, targets, V):
    torch = _torch()
    dev = hidden.device
    hp, ldh = _bf16_operand("hidden", hidden, dev)
    wp, ldw = _bf16_operand("weight", weight, dev)
    T, H = hidden.shape
    if weight.shape[1] != H:
        raise ValueError("hidden and weight disagree on H")
    V = int(weight.shape[0] if V is None else V)
    if V > weight.shape[0]:
        raise ValueError("V exceeds the rows of weight")
    if targets.dtype != torch.int32 or targets.shape != (T,) or not targets.is_contiguous():
        raise ValueError("targets must be a contiguous int32 [T] tensor")
    _check_device("targets", targets, dev)
    return dev, hp, ldh, wp, ldw, T, H, V


def _outputs(dev, T, logp, lse, stream=None):
    torch = _torch()
    with _on(stream):
        if logp is None:
            logp = torch.empty(T, dtype=torch.float32, device=dev)
        if lse is None:
            lse = torch.empty(T, dtype=torch.float32, device=dev)
    for name, t in (("logp", logp), ("lse", lse)):
        if t.dtype != torch.float32 or t.shape != (T,) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 [T] tensor")
        _check_device(name, t, dev)
    return logp, lse


def workspace_for(T: int, V: int, device, flags: int = 0, stream=None):
    """A device workspace tensor large enough for T rows and vocabulary V
    (allocated for ``stream`` when one is given)."""
    torch = _torch()
    need = rlk_workspace_bytes_ex(T, V, flags)
    with _on(stream):
        return torch.empty(max(need, 1), dtype=torch.uint8, device=device)


def _workspace(dev, T, V, workspace, stream=None):
    if workspace is None:
        workspace = workspace_for(T, V, dev, stream=stream)
    _check_device("workspace", workspace, dev)
    return workspace, workspace.numel() * workspace.element_size()


def rlk_selected_logp(hidden, weight, targets, logp=None, lse=None,
                      workspace=None, V=None, stream=None):
    """logp[T], lse[T] (fp32) for hidden [T, H], weight [>=V, H], targets [T].

    ``V`` defaults to ``weight.shape[0]``; pass the real vocabulary size when
    ``weight`` carries padding rows.  Outputs and the workspace are allocated
    on ``hidden.device`` when not given.  Runs on ``stream`` (default: the
    current torch stream) without synchronising.
    """
    dev, hp, ldh, wp, ldw, T, H, V = _prepare(hidden, weight, targets, V)
    logp, lse = _outputs(dev, T, logp, lse, stream)
    ws, ws_bytes = _workspace(dev, T, V, workspace, stream)
    _call("rlk_selected_logp", lib().rlk_selected_logp(
        hp, ldh, wp, ldw, targets.data_ptr(), logp.data_ptr(), lse.data_ptr(),
        T, H, V, ws.data_ptr(), ws_bytes, _stream_ptr(stream, dev)))
    return logp, lse


def rlk_selected_logp_noalloc(hidden, weight, targets, logp, lse, V=None, stream=None):
    """rlk_selected_logp with the library's static device scratch as its
    workspace: the call itself allocates nothing (the caller passes the
    outputs).  Calls that may overlap on one GPU must be serialised."""
    dev, hp, ldh, wp, ldw, T, H, V = _prepare(hidden, weight, targets, V)
    logp, lse = _outputs(dev, T, logp, lse, stream)
    _call("rlk_selected_logp_noalloc", lib().rlk_selected_logp_noalloc(
        hp, ldh, wp, ldw, targets.data_ptr(), logp.data_ptr(), lse.data_ptr(),
        T, H, V, _stream_ptr(stream, dev)))
    return logp, lse


def rlk_vocab_stats(hidden, weight, targets, workspace, V=None, stream=None):
    """Stage 1: logit GEMM + per-tile statistics + target capture into
    ``workspace`` (see :func:`workspace_for`)."""
    dev, hp, ldh, wp, ldw, T, H, V = _prepare(hidden, weight, targets, V)
    ws, ws_bytes = _workspace(dev, T, V, workspace, stream)
    _call("rlk_vocab_stats", lib().rlk_vocab_stats(
        hp, ldh, wp, ldw, targets.data_ptr(), T, H, V, ws.data_ptr(), ws_bytes,
        _stream_ptr(stream, dev)))
    return ws


def rlk_vocab_stats_shard(hidden, weight_shard, targets, workspace, V, v_begin,
                          stream=None):
    """Stage 1 on the weight rows [v_begin, v_begin + weight_shard.shape[0])
    of a V-row LM head, into a workspace sized for (T, V)."""
    torch = _torch()
    dev = hidden.device
    hp, ldh = _bf16_operand("hidden", hidden, dev)
    wp, ldw = _bf16_operand("weight_shard", weight_shard, dev)
    T, H = hidden.shape
    if weight_shard.shape[1] != H:
        raise ValueError("hidden and weight_shard disagree on H")
    if targets.dtype != torch.int32 or targets.shape != (T,) or not targets.is_contiguous():
        raise ValueError("targets must be a contiguous int32 [T] tensor")
    _check_device("targets", targets, dev)
    _check_device("workspace", workspace, dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    _call("rlk_vocab_stats_shard", lib().rlk_vocab_stats_shard(
        hp, ldh, wp, ldw, targets.data_ptr(), T, H, int(V), int(v_begin),
        int(weight_shard.shape[0]), workspace.data_ptr(), ws_bytes,
        _stream_ptr(stream, dev)))
    return workspace


def rlk_vocab_merge(targets, workspace, V, logp=None, lse=None, stream=None):
    """Stage 2: fixed-order fold of the tile statistics -> (logp, lse)."""
    torch = _torch()
    dev = targets.device
    _check_device("targets", targets, dev)
    if targets.dtype != torch.int32 or targets.dim() != 1 or not targets.is_contiguous():
        raise ValueError("targets must be a contiguous int32 [T] tensor")
    T = targets.shape[0]
    logp, lse = _outputs(dev, T, logp, lse, stream)
    _check_device("workspace", workspace, dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    _call("rlk_vocab_merge", lib().rlk_vocab_merge(
        targets.data_ptr(), logp.data_ptr(), lse.data_ptr(), T, int(V),
        workspace.data_ptr(), ws_bytes, _stream_ptr(stream, dev)))
    return logp, lse


def _flags(logits_bf16, entropy):
    return (RLK_LOGITS_BF16 if logits_bf16 else 0) | (RLK_ENTROPY if entropy else 0)


def _entropy_out(dev, T, entropy, want, stream=None):
    torch = _torch()
    if not want:
        return None
    if entropy is None or entropy is True:
        with _on(stream):
            entropy = torch.empty(T, dtype=torch.float32, device=dev)
    if entropy.dtype != torch.float32 or entropy.shape != (T,) or not entropy.is_contiguous():
        raise ValueError("entropy must be a contiguous float32 [T] tensor")
    _check_device("entropy", entropy, dev)
    return entropy


def rlk_selected_logp_ex(hidden, weight, targets, inv_temperature=1.0, logits_bf16=False,
                         entropy=False, logp=None, lse=None, workspace=None, V=None,
                         stream=None):
    """(logp, lse, entropy) with the contract options: logits times
    ``inv_temperature``, optionally rounded to bf16; ``entropy`` True (or an
    output tensor) also returns the per-row entropy, else None."""
    dev, hp, ldh, wp, ldw, T, H, V = _prepare(hidden, weight, targets, V)
    logp, lse = _outputs(dev, T, logp, lse, stream)
    flags = _flags(logits_bf16, entropy is not False and entropy is not None)
    ent = _entropy_out(dev, T, entropy, flags & RLK_ENTROPY, stream)
    if workspace is None:
        workspace = workspace_for(T, V, dev, flags, stream)
    _check_device("workspace", workspace, dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    _call("rlk_selected_logp_ex", lib().rlk_selected_logp_ex(
        hp, ldh, wp, ldw, targets.data_ptr(), logp.data_ptr(), lse.data_ptr(),
        ent.data_ptr() if ent is not None else None, T, H, V, float(inv_temperature),
        flags, workspace.data_ptr(), ws_bytes, _stream_ptr(stream, dev)))
    return logp, lse, ent


def rlk_vocab_stats_ex(hidden, weight_shard, targets, workspace, V, v_begin=0,
                       inv_temperature=1.0, logits_bf16=False, entropy=False, stream=None):
    """Stage 1 with the contract options on weight rows [v_begin, v_begin +
    weight_shard.shape[0]) of a V-row head; workspace sized by
    rlk_workspace_bytes_ex(T, V, flags)."""
    torch = _torch()
    dev = hidden.device
    hp, ldh = _bf16_operand("hidden", hidden, dev)
    wp, ldw = _bf16_operand("weight_shard", weight_shard, dev)
    T, H = hidden.shape
    if weight_shard.shape[1] != H:
        raise ValueError("hidden and weight_shard disagree on H")
    if targets.dtype != torch.int32 or targets.shape != (T,) or not targets.is_contiguous():
        raise ValueError("targets must be a contiguous int32 [T] tensor")
    _check_device("targets", targets, dev)
    _check_device("workspace", workspace, dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    _call("rlk_vocab_stats_ex", lib().rlk_vocab_stats_ex(
        hp, ldh, wp, ldw, targets.data_ptr(), T, H, int(V), int(v_begin),
        int(weight_shard.shape[0]), float(inv_temperature), _flags(logits_bf16, entropy),
        workspace.data_ptr(), ws_bytes, _stream_ptr(stream, dev)))
    return workspace


def rlk_vocab_merge_ex(targets, workspace, V, logits_bf16=False, entropy=False, logp=None,
                       lse=None, stream=None):
    """Stage 2 with the same flags as stage 1 -> (logp, lse, entropy or None)."""
    torch = _torch()
    dev = targets.device
    _check_device("targets", targets, dev)
    if targets.dtype != torch.int32 or targets.dim() != 1 or not targets.is_contiguous():
        raise ValueError("targets must be a contiguous int32 [T] tensor")
    T = targets.shape[0]
    logp, lse = _outputs(dev, T, logp, lse, stream)
    flags = _flags(logits_bf16, entropy is not False and entropy is not None)
    ent = _entropy_out(dev, T, entropy, flags & RLK_ENTROPY, stream)
    _check_device("workspace", workspace, dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    _call("rlk_vocab_merge_ex", lib().rlk_vocab_merge_ex(
        targets.data_ptr(), logp.data_ptr(), lse.data_ptr(),
        ent.data_ptr() if ent is not None else None, T, int(V), flags,
        workspace.data_ptr(), ws_bytes, _stream_ptr(stream, dev)))
    return logp, lse, ent


def rlk_selected_logp_backward_workspace_bytes(T: int, H: int, V: int) -> int:
    return int(lib().rlk_selected_logp_backward_workspace_bytes(int(T), int(H), int(V)))


def _f32_vec(name, t, T, dev):
    torch = _torch()
    if t.dtype != torch.float32 or t.shape != (T,) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 [T] tensor")
    _check_device(name, t, dev)
    return t.data_ptr()


def rlk_selected_logp_backward(hidden, weight, targets, lse, grad_logp, inv_temperature=1.0,
                               want_hidden=True, want_weight=True, grad_hidden=None,
                               grad_weight=None, workspace=None, V=None, stream=None):
    """(grad_hidden [T, H] or None, grad_weight [V, H] or None), fp32, of
    L = sum_t grad_logp[t] logp[t], using the forward's ``lse``."""
    torch = _torch()
    dev, hp, ldh, wp, ldw, T, H, V = _prepare(hidden, weight, targets, V)
    lp_ = _f32_vec("lse", lse, T, dev)
    gp_ = _f32_vec("grad_logp", grad_logp, T, dev)
    with _on(stream):
        if want_hidden and grad_hidden is None:
            grad_hidden = torch.empty((T, H), dtype=torch.float32, device=dev)
        if want_weight and grad_weight is None:
            grad_weight = torch.empty((V, H), dtype=torch.float32, device=dev)
    for name, t, shape in (("grad_hidden", grad_hidden if want_hidden else None, (T, H)),
                           ("grad_weight", grad_weight if want_weight else None, (V, H))):
        if t is not None:
            if t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous float32 {list(shape)} tensor")
            _check_device(name, t, dev)
    gh = grad_hidden if want_hidden else None
    gw = grad_weight if want_weight else None
    if workspace is None:
        with _on(stream):
            workspace = torch.empty(max(rlk_selected_logp_backward_workspace_bytes(T, H, V), 1),
                                    dtype=torch.uint8, device=dev)
    _check_device("workspace", workspace, dev)
    _call("rlk_selected_logp_backward", lib().rlk_selected_logp_backward(
        hp, ldh, wp, ldw, targets.data_ptr(), lp_, gp_,
        gh.data_ptr() if gh is not None else None, gw.data_ptr() if gw is not None else None,
        T, H, V, float(inv_temperature), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream_ptr(stream, dev)))
    return gh, gw


def rlk_logp_grad_logits(hidden, weight, targets, lse, grad_logp, inv_temperature=1.0,
                         dz=None, V=None, stream=None):
    """bf16 dz [T, Vp] (Vp = V rounded up to 64, padding columns 0)."""
    torch = _torch()
    dev, hp, ldh, wp, ldw, T, H, V = _prepare(hidden, weight, targets, V)
    Vp = (V + 63) // 64 * 64
    if dz is None:
        with _on(stream):
            dz = torch.empty((T, Vp), dtype=torch.bfloat16, device=dev)
    if dz.dim() != 2 or dz.shape[0] != T or dz.stride(1) != 1 or dz.element_size() != 2:
        raise ValueError("dz must be a 2-D 16-bit [T, >= Vp] tensor with unit column stride")
    _check_device("dz", dz, dev)
    _call("rlk_logp_grad_logits", lib().rlk_logp_grad_logits(
        hp, ldh, wp, ldw, targets.data_ptr(), _f32_vec("lse", lse, T, dev),
        _f32_vec("grad_logp", grad_logp, T, dev), dz.data_ptr(), dz.stride(0), T, H, V,
        float(inv_temperature), _stream_ptr(stream, dev)))
    return dz


def rlk_rmsnorm(x, gamma, eps=1e-6, y=None, stream=None):
    """bf16 y [T, H] = RMSNorm(x) * gamma (the LM head's input)."""
    torch = _torch()
    dev = x.device
    xp, ldx = _bf16_operand("x", x, dev)
    T, H = x.shape
    if gamma.dim() != 1 or gamma.shape[0] != H or not gamma.is_contiguous():
        raise ValueError("gamma must be a contiguous [H] tensor")
    gp, _ = _bf16_operand("gamma", gamma.view(1, H), dev)
    if y is None:
        with _on(stream):
            y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    yp, ldy = _bf16_operand("y", y, dev)
    if tuple(y.shape) != (T, H):
        raise ValueError("y must have shape [T, H]")
    _call("rlk_rmsnorm", lib().rlk_rmsnorm(xp, ldx, gp, float(eps), yp, ldy, T, H,
                                           _stream_ptr(stream, dev)))
    return y


def rlk_topk_logp(logits, lse, workspace, k, inv_temperature=1.0, logits_bf16=False, V=None,
                  topk_logp=None, topk_ids=None, stream=None):
    """(topk_logp [T, k] fp32, topk_ids [T, k] int32) from stored logits and
    the statistics pass's lse and workspace (same options)."""
    torch = _torch()
    dev = logits.device
    _check_device("logits", logits, dev)
    if logits.dtype != torch.float32 or logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be a 2-D float32 tensor with unit column stride")
    T = logits.shape[0]
    V = int(logits.shape[1] if V is None else V)
    lp_ = _f32_vec("lse", lse, T, dev)
    _check_device("workspace", workspace, dev)
    with _on(stream):
        if topk_logp is None:
            topk_logp = torch.empty((T, k), dtype=torch.float32, device=dev)
        if topk_ids is None:
            topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    _call("rlk_topk_logp", lib().rlk_topk_logp(
        logits.data_ptr(), logits.stride(0), lp_, workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), T, V, int(k), float(inv_temperature),
        RLK_LOGITS_BF16 if logits_bf16 else 0, topk_logp.data_ptr(), topk_ids.data_ptr(),
        _stream_ptr(stream, dev)))
    return topk_logp, topk_ids


def rlk_topk_logp_direct_workspace_bytes(T, V, k, max_degenerate_rows=16) -> int:
    return int(lib().rlk_topk_logp_direct_workspace_bytes(int(T), int(V), int(k),
                                                          int(max_degenerate_rows)))


def rlk_topk_logp_direct(hidden, weight, lse, stats_workspace, k, inv_temperature=1.0,
                         logits_bf16=False, max_degenerate_rows=16, workspace=None,
                         topk_logp=None, topk_ids=None, V=None, stream=None):
    """(topk_logp [T, k] fp32, topk_ids [T, k] int32) without stored logits:
    the candidate tiles' logits are recomputed from hidden and weight; the
    statistics pass's lse and workspace (same options) select them."""
    torch = _torch()
    dev = hidden.device
    hp, ldh = _bf16_operand("hidden", hidden, dev)
    wp, ldw = _bf16_operand("weight", weight, dev)
    T, H = hidden.shape
    V = int(weight.shape[0] if V is None else V)
    lp_ = _f32_vec("lse", lse, T, dev)
    _check_device("stats_workspace", stats_workspace, dev)
    need = rlk_topk_logp_direct_workspace_bytes(T, V, k, max_degenerate_rows) if T > 0 else 0
    with _on(stream):
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        if topk_logp is None:
            topk_logp = torch.empty((T, k), dtype=torch.float32, device=dev)
        if topk_ids is None:
            topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    _check_device("workspace", workspace, dev)
    _call("rlk_topk_logp_direct", lib().rlk_topk_logp_direct(
        hp, ldh, wp, ldw, lp_, stats_workspace.data_ptr(),
        stats_workspace.numel() * stats_workspace.element_size(), T, H, V, int(k),
        float(inv_temperature), RLK_LOGITS_BF16 if logits_bf16 else 0, int(max_degenerate_rows),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        topk_logp.data_ptr(), topk_ids.data_ptr(), _stream_ptr(stream, dev)))
    return topk_logp, topk_ids


def topk_logprobs(hidden, weight, targets, k, inv_temperature=1.0, logits_bf16=False,
                  stored_logits=False, stream=None):
    """Selected-token logp and lse plus the top-k log-probabilities of every
    row: the statistics pass, then the selection over the candidate tiles'
    recomputed logits (or, with stored_logits, over the logits stored whole:
    the same bits, at the cost of a [T, V] fp32 array)."""
    dev, _, _, _, _, T, _, V = _prepare(hidden, weight, targets, None)
    flags = RLK_LOGITS_BF16 if logits_bf16 else 0
    ws = workspace_for(T, V, dev, flags, stream)
    logp, lse, _ = rlk_selected_logp_ex(hidden, weight, targets,
                                        inv_temperature=inv_temperature,
                                        logits_bf16=logits_bf16, workspace=ws, stream=stream)
    if stored_logits:
        z = rlk_logits(hidden, weight, stream=stream)
        tl, ti = rlk_topk_logp(z, lse, ws, k, inv_temperature, logits_bf16, stream=stream)
    else:
        tl, ti = rlk_topk_logp_direct(hidden, weight, lse, ws, k, inv_temperature, logits_bf16,
                                      V=V, stream=stream)
    return logp, lse, tl, ti


def rlk_debug_logits(hidden, weight, logits=None, V=None, stream=None):
    """fp32 logits [T, V] from the same GEMM main loop (stage comparison)."""
    torch = _torch()
    dev = hidden.device
    hp, ldh = _bf16_operand("hidden", hidden, dev)
    wp, ldw = _bf16_operand("weight", weight, dev)
    T, H = hidden.shape
    V = int(weight.shape[0] if V is None else V)
    if logits is None:
        with _on(stream):
            logits = torch.empty((T, V), dtype=torch.float32, device=dev)
    if logits.dtype != torch.float32 or logits.shape != (T, V) or not logits.is_contiguous():
        raise ValueError("logits must be a contiguous float32 [T, V] tensor")
    _check_device("logits", logits, dev)
    _call("rlk_debug_logits", lib().rlk_debug_logits(hp, ldh, wp, ldw, logits.data_ptr(),
                                                     T, H, V, _stream_ptr(stream, dev)))
    return logits


rlk_logits = rlk_debug_logits


def rlk_compare(a, b, stats=None, stream=None):
    """fp64 [8] statistics of a vs b (see rlk.h), computed on the device."""
    torch = _torch()
    dev = a.device
    if a.dtype != torch.float32 or b.dtype != torch.float32 or a.shape != b.shape:
        raise ValueError("a and b must be float32 tensors of one shape")
    _check_device("a", a, dev)
    _check_device("b", b, dev)
    with _on(stream):
        a = a.contiguous()
        b = b.contiguous()
        if stats is None:
            stats = torch.empty(8, dtype=torch.float64, device=dev)
    _check_device("stats", stats, dev)
    _call("rlk_compare", lib().rlk_compare(a.data_ptr(), b.data_ptr(), a.numel(),
                                           stats.data_ptr(), _stream_ptr(stream, dev)))
    return stats


def consistency_report(stats) -> dict:
    """Host-side view of rlk_compare's statistics (synchronises)."""
    s = [float(x) for x in stats.cpu().tolist()]
    n = s[0]
    mean = s[3] / n if n else 0.0
    var = max(s[4] / n - mean * mean, 0.0) if n else 0.0
    return {
        "n": int(n),
        "mismatch_count": int(s[1]),
        "max_abs_diff": s[2],
        "mean_abs_diff": mean,
        "std_abs_diff": var ** 0.5,
        "k3_mean": s[5] / s[6] if s[6] else 0.0,
    }


selected_logp = rlk_selected_logp
