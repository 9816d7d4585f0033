"""CPU tests of the C-ABI library: exports, constants and every error path.

No test here launches a kernel: each call either returns before its first
HIP call (validation) or touches no device at all.  Pointer values used on
the error paths are never dereferenced by the library.
"""

import ctypes
import os
import re

import pytest

import invariant_selected_token_amd as rlk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rlk.h")

FAKE = 0x10000          # a 64 KiB-aligned non-null address, never dereferenced
WS_FAKE = 1 << 40


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rlk_\w+)\s*\(", text)))


def test_header_declares_what_the_binding_knows():
    assert _declared_functions() == sorted(rlk.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = rlk.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name


SURVEY_CALLS = {
    # the boundary's calls and their C signatures, as the hot path's scope
    # table lists them (argument names may differ; types and order may not)
    "rlk_abi_version": "int rlk_abi_version(void)",
    "rlk_status_string": "const char *rlk_status_string(int status)",
    "rlk_selected_logp_workspace_bytes":
        "size_t rlk_selected_logp_workspace_bytes(int64_t T, int64_t H, int64_t V)",
    "rlk_selected_logp":
        "int rlk_selected_logp(const void *hidden, int64_t ld_hidden, const void *weight, "
        "int64_t ld_weight, const int32_t *targets, float *logp, float *lse, int64_t T, "
        "int64_t H, int64_t V, void *workspace, size_t workspace_bytes, void *stream)",
    "rlk_debug_logits":
        "int rlk_debug_logits(const void *hidden, int64_t ld_hidden, const void *weight, "
        "int64_t ld_weight, float *logits, int64_t T, int64_t H, int64_t V, void *stream)",
}


def _types_of(decl):
    """(return type, [argument types]) of a C declaration, names dropped."""
    decl = re.sub(r"\s+", " ", decl).strip().rstrip(";")
    head, args = decl.split("(", 1)
    args = args.rsplit(")", 1)[0]
    ret = head.rsplit(" ", 1)[0].replace(" *", "*").strip()
    if head.rstrip().split(" ")[-1].startswith("*"):
        ret += "*"
    out = []
    for a in ([] if args.strip() == "void" else args.split(",")):
        a = a.strip()
        m = re.match(r"(.*?)(\w+)$", a)
        out.append(re.sub(r"\s+", "", m.group(1)))
    return ret.replace(" ", ""), out


def test_boundary_calls_of_the_scope_table():
    """Every call of the boundary the hot-path scope table lists is declared
    with its signature and exported."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    text = "\n".join(l for l in text.splitlines() if not l.lstrip().startswith("#"))
    decls = [re.sub(r"\s+", " ", d).strip() for d in re.split(r"[;{}]", text)]
    L = rlk.lib()
    for name, want in SURVEY_CALLS.items():
        found = [d for d in decls if re.search(r"\b" + name + r"\s*\(", d)]
        assert len(found) == 1, (name, found)
        assert _types_of(found[0]) == _types_of(want), (name, found[0])
        assert hasattr(L, name), name


def test_constants():
    assert rlk.rlk_abi_version() == 5
    assert rlk.rlk_vocab_tile() == 128
    msgs = {rlk.rlk_status_string(s) for s in range(9)}
    assert len(msgs) == 9 and all(msgs)
    assert rlk.rlk_status_string(99) == "unknown status"


def test_workspace_size():
    def ws(T, V, H=4096):
        return rlk.rlk_selected_logp_workspace_bytes(T, H, V)

    assert ws(0, 151936) == 0 and ws(-1, 10) == 0 and ws(5, 0) == 0
    assert ws(5, 10, H=0) == 0 and ws(5, 10, H=-64) == 0
    # H does not change the size
    assert ws(64, 4096, H=256) == ws(64, 4096, H=4096) == ws(64, 4096, H=64)
    # the size limits: T and V up to 2^31 - 4096
    assert ws(2 ** 31 - 4096, 1) > 0 and ws(2 ** 31 - 4095, 1) == 0
    assert ws(1, 2 ** 31 - 4096) > 0 and ws(1, 2 ** 31 - 4095) == 0

    def expect(T, V):
        r = lambda x: (x + 255) // 256 * 256
        return 2 * r(((V + 127) // 128) * T * 4) + r(T * 4) + 256   # + tile-claim counters

    for T, V in [(1, 1), (1, 151936), (64, 4096), (4096, 151936), (16384, 151936),
                 (257, 129)]:
        assert ws(T, V) == expect(T, V)
    prev = 0
    for T in range(1, 600, 37):
        assert ws(T, 151936) >= prev
        prev = ws(T, 151936)


def _call(hidden=FAKE, ldh=256, weight=FAKE, ldw=256, targets=FAKE, logp=FAKE,
          lse=FAKE, T=4, H=256, V=1000, ws=WS_FAKE, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = max(rlk.rlk_selected_logp_workspace_bytes(T, 256, V), 0)
    return rlk.lib().rlk_selected_logp(hidden, ldh, weight, ldw, targets, logp, lse,
                                       T, H, V, ws, ws_bytes, stream)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), rlk.RLK_ERR_INVALID_SHAPE),
    (dict(H=0), rlk.RLK_ERR_INVALID_SHAPE),
    (dict(H=-64), rlk.RLK_ERR_INVALID_SHAPE),
    (dict(V=0), rlk.RLK_ERR_INVALID_SHAPE),
    (dict(ldh=128), rlk.RLK_ERR_INVALID_SHAPE),
    (dict(ldw=192), rlk.RLK_ERR_INVALID_SHAPE),
    (dict(H=200, ldh=256, ldw=256), rlk.RLK_ERR_UNSUPPORTED),
    (dict(H=65536 + 64, ldh=65536 + 64, ldw=65536 + 64), rlk.RLK_ERR_UNSUPPORTED),
    (dict(ldh=(1 << 21) + 8), rlk.RLK_ERR_UNSUPPORTED),
    (dict(T=1 << 31), rlk.RLK_ERR_UNSUPPORTED),
    (dict(V=1 << 31), rlk.RLK_ERR_UNSUPPORTED),
    # past the last row index every kernel forms in int
    (dict(T=2 ** 31 - 4095, V=64), rlk.RLK_ERR_UNSUPPORTED),
    (dict(T=1, V=2 ** 31 - 4095), rlk.RLK_ERR_UNSUPPORTED),
    # the largest T is accepted (stops at the workspace check)
    (dict(T=2 ** 31 - 4096, V=64, ws_bytes=100), rlk.RLK_ERR_WORKSPACE_TOO_SMALL),
    # 8388607 x 256 = 2^31 - 256 workgroup tiles: T and V are in range, but a
    # tile index plus a grid of workgroups would pass 2^31
    (dict(T=(2 ** 23 - 1) * 256, V=65536), rlk.RLK_ERR_UNSUPPORTED),
    (dict(hidden=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(weight=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(targets=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(logp=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(lse=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(ws=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(hidden=FAKE + 8), rlk.RLK_ERR_MISALIGNED),
    (dict(weight=FAKE + 2), rlk.RLK_ERR_MISALIGNED),
    (dict(ldh=260), rlk.RLK_ERR_MISALIGNED),
    (dict(ldw=257), rlk.RLK_ERR_MISALIGNED),
    (dict(targets=FAKE + 2), rlk.RLK_ERR_MISALIGNED),
    (dict(logp=FAKE + 1), rlk.RLK_ERR_MISALIGNED),
    (dict(lse=FAKE + 3), rlk.RLK_ERR_MISALIGNED),
    (dict(ws=WS_FAKE + 4), rlk.RLK_ERR_MISALIGNED),
    (dict(ws_bytes=100), rlk.RLK_ERR_WORKSPACE_TOO_SMALL),
])
def test_selected_logp_error_paths(kw, status):
    assert _call(**kw) == status
    assert rlk.rlk_last_hip_error() == 0


def test_selected_logp_empty_batch_is_a_no_op():
    assert _call(T=0, hidden=None, weight=None, targets=None, logp=None, lse=None,
                 ws=None, ws_bytes=0) == rlk.RLK_OK


def test_workspace_one_byte_short():
    need = rlk.rlk_selected_logp_workspace_bytes(4, 256, 1000)
    assert _call(ws_bytes=need - 1) == rlk.RLK_ERR_WORKSPACE_TOO_SMALL


@pytest.mark.parametrize("kw,status", [
    (dict(T=-5), rlk.RLK_ERR_INVALID_SHAPE),
    (dict(H=96, ldh=96, ldw=96), rlk.RLK_ERR_UNSUPPORTED),
    (dict(logits=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(hidden=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(logits=FAKE + 2), rlk.RLK_ERR_MISALIGNED),
    (dict(T=0, logits=None, hidden=None, weight=None), rlk.RLK_OK),
    (dict(V=(1 << 24) + 1), rlk.RLK_ERR_UNSUPPORTED),   # 32 output rows past 2^31 bytes
    (dict(V=(1 << 24) + 1, T=0), rlk.RLK_ERR_UNSUPPORTED),
])
@pytest.mark.parametrize("name", ["rlk_debug_logits", "rlk_logits"])
def test_logits_error_paths(kw, status, name):
    a = dict(hidden=FAKE, ldh=256, weight=FAKE, ldw=256, logits=FAKE, T=4, H=256,
             V=100, stream=None)
    a.update(kw)
    fn = getattr(rlk.lib(), name)
    assert fn(a["hidden"], a["ldh"], a["weight"], a["ldw"],
              a["logits"], a["T"], a["H"], a["V"], a["stream"]) == status


@pytest.mark.parametrize("a,b,n,stats,status", [
    (FAKE, FAKE, -1, FAKE, rlk.RLK_ERR_INVALID_SHAPE),
    (FAKE, FAKE, 1 << 31, FAKE, rlk.RLK_ERR_UNSUPPORTED),
    # the largest n is accepted (indices are 64-bit on the device)
    (FAKE, FAKE, (1 << 31) - 1, None, rlk.RLK_ERR_NULL_POINTER),
    (FAKE, FAKE, 10, None, rlk.RLK_ERR_NULL_POINTER),
    (None, FAKE, 10, FAKE, rlk.RLK_ERR_NULL_POINTER),
    (FAKE, FAKE, 10, FAKE + 4, rlk.RLK_ERR_MISALIGNED),
    (FAKE + 1, FAKE, 10, FAKE, rlk.RLK_ERR_MISALIGNED),
])
def test_compare_error_paths(a, b, n, stats, status):
    assert rlk.lib().rlk_compare(a, b, n, stats, None) == status


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    h = torch.zeros((2, 64), dtype=torch.bfloat16)
    w = torch.zeros((8, 64), dtype=torch.bfloat16)
    y = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError):
        rlk.rlk_selected_logp(h, w, y)
    with pytest.raises(ValueError):
        rlk.rlk_logits(h, w)


def test_status_error_type_carries_the_message():
    e = rlk.RLKError(rlk.RLK_ERR_MISALIGNED, "where")
    assert "misaligned" in str(e) and e.status == rlk.RLK_ERR_MISALIGNED


def _stats(hidden=FAKE, ldh=256, weight=FAKE, ldw=256, targets=FAKE, T=4, H=256,
           V=1000, ws=WS_FAKE, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = rlk.rlk_selected_logp_workspace_bytes(T, 256, V)
    return rlk.lib().rlk_vocab_stats(hidden, ldh, weight, ldw, targets, T, H, V, ws,
                                     ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), rlk.RLK_ERR_INVALID_SHAPE),
    (dict(H=100, ldh=104, ldw=104), rlk.RLK_ERR_UNSUPPORTED),
    (dict(targets=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(ws=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(hidden=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(targets=FAKE + 1), rlk.RLK_ERR_MISALIGNED),
    (dict(ws=WS_FAKE + 8), rlk.RLK_ERR_MISALIGNED),
    (dict(ws_bytes=64), rlk.RLK_ERR_WORKSPACE_TOO_SMALL),
    (dict(T=0, hidden=None, weight=None, targets=None, ws=None, ws_bytes=0), rlk.RLK_OK),
])
def test_vocab_stats_error_paths(kw, status):
    assert _stats(**kw) == status


def _merge(targets=FAKE, logp=FAKE, lse=FAKE, T=4, V=1000, ws=WS_FAKE, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = rlk.rlk_selected_logp_workspace_bytes(T, 256, V)
    return rlk.lib().rlk_vocab_merge(targets, logp, lse, T, V, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), rlk.RLK_ERR_INVALID_SHAPE),
    (dict(V=0), rlk.RLK_ERR_INVALID_SHAPE),
    (dict(V=1 << 31), rlk.RLK_ERR_UNSUPPORTED),
    (dict(targets=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(logp=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(lse=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(ws=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(lse=FAKE + 2), rlk.RLK_ERR_MISALIGNED),
    (dict(ws=WS_FAKE + 4), rlk.RLK_ERR_MISALIGNED),
    (dict(ws_bytes=16), rlk.RLK_ERR_WORKSPACE_TOO_SMALL),
    (dict(T=0, targets=None, logp=None, lse=None, ws=None, ws_bytes=0), rlk.RLK_OK),
])
def test_vocab_merge_error_paths(kw, status):
    assert _merge(**kw) == status


def _shard(hidden=FAKE, ldh=256, weight=FAKE, ldw=256, targets=FAKE, T=4, H=256,
           V=1000, v_begin=256, v_count=256, ws=WS_FAKE, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = rlk.rlk_selected_logp_workspace_bytes(T, 256, V)
    return rlk.lib().rlk_vocab_stats_shard(hidden, ldh, weight, ldw, targets, T, H, V,
                                           v_begin, v_count, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(v_begin=-256), rlk.RLK_ERR_INVALID_SHAPE),
    (dict(v_count=0), rlk.RLK_ERR_INVALID_SHAPE),
    (dict(v_count=-1), rlk.RLK_ERR_INVALID_SHAPE),
    (dict(v_begin=768, v_count=256), rlk.RLK_ERR_INVALID_SHAPE),   # past V
    (dict(v_begin=128), rlk.RLK_ERR_UNSUPPORTED),                  # not 256-aligned
    (dict(v_count=200), rlk.RLK_ERR_UNSUPPORTED),                  # ragged, not last
    (dict(H=100, ldh=104, ldw=104), rlk.RLK_ERR_UNSUPPORTED),
    (dict(T=-1), rlk.RLK_ERR_INVALID_SHAPE),
    (dict(targets=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(weight=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(ws=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(ws=WS_FAKE + 4), rlk.RLK_ERR_MISALIGNED),
    (dict(T=1000, ws_bytes=("for", 1000, 512)), rlk.RLK_ERR_WORKSPACE_TOO_SMALL),  # slice-sized
    (dict(T=0, hidden=None, weight=None, targets=None, ws=None, ws_bytes=0), rlk.RLK_OK),
])
def test_vocab_stats_shard_error_paths(kw, status):
    kw = dict(kw)
    if isinstance(kw.get("ws_bytes"), tuple):     # sized in the test, not at collection
        _, t, v = kw["ws_bytes"]
        kw["ws_bytes"] = rlk.rlk_selected_logp_workspace_bytes(t, 256, v)
        assert kw["ws_bytes"] < rlk.rlk_selected_logp_workspace_bytes(kw["T"], 256, 1000)
    assert _shard(**kw) == status
    assert rlk.rlk_last_hip_error() == 0


def test_vocab_stats_shard_accepts_the_ragged_last_slice():
    # 768 + 232 = V: validation passes up to the operands (a null hidden).
    assert _shard(hidden=None, v_begin=768, v_count=232) == rlk.RLK_ERR_NULL_POINTER
    assert _shard(hidden=None, v_begin=0, v_count=1000) == rlk.RLK_ERR_NULL_POINTER


def test_one_hip_runtime_in_the_process():
    """The library binds to torch's HIP runtime instead of mapping a second one
    (two runtimes in one process do not share devices).  Run in a fresh
    interpreter that loads the library before anything imports torch."""
    import subprocess
    import sys
    code = ("import invariant_selected_token_amd as r; r.lib(); "
            "import re; maps = open('/proc/self/maps').read(); "
            "print(sorted(set(re.findall(r'\\S*libamdhip64\\S*', maps))))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True,
                         text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    paths = eval(out.stdout.strip().splitlines()[-1])
    assert len(paths) == 1, paths


# ------------------------------------------------------ contract options --

def test_workspace_size_ex():
    wx = rlk.rlk_workspace_bytes_ex
    ws = lambda T, V: rlk.rlk_selected_logp_workspace_bytes(T, 4096, V)
    r = lambda x: (x + 255) // 256 * 256
    for T, V in [(1, 1), (64, 4096), (4096, 151936), (257, 129)]:
        assert wx(T, V, 0) == ws(T, V)
        assert wx(T, V, rlk.RLK_LOGITS_BF16) == ws(T, V)
        stats = r(((V + 127) // 128) * T * 4)
        assert wx(T, V, rlk.RLK_ENTROPY) == ws(T, V) + stats
        assert wx(T, V, rlk.RLK_ENTROPY | rlk.RLK_LOGITS_BF16) == ws(T, V) + stats
    assert wx(4, 1000, 4) == 0 and wx(4, 1000, -1) == 0 and wx(0, 10, 0) == 0


def _ex(hidden=FAKE, ldh=256, weight=FAKE, ldw=256, targets=FAKE, logp=FAKE, lse=FAKE,
        entropy=FAKE, T=4, H=256, V=1000, inv_tau=1.0, flags=rlk.RLK_ENTROPY, ws=WS_FAKE,
        ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = rlk.rlk_workspace_bytes_ex(T, V, flags if flags in (0, 1, 2, 3) else 0)
    return rlk.lib().rlk_selected_logp_ex(hidden, ldh, weight, ldw, targets, logp, lse,
                                          entropy, T, H, V, inv_tau, flags, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(inv_tau=0.0), rlk.RLK_ERR_INVALID_VALUE),
    (dict(inv_tau=-1.0), rlk.RLK_ERR_INVALID_VALUE),
    (dict(inv_tau=float("inf")), rlk.RLK_ERR_INVALID_VALUE),
    (dict(inv_tau=float("nan")), rlk.RLK_ERR_INVALID_VALUE),
    (dict(flags=4), rlk.RLK_ERR_INVALID_VALUE),
    (dict(flags=-1), rlk.RLK_ERR_INVALID_VALUE),
    (dict(T=0, inv_tau=0.0), rlk.RLK_ERR_INVALID_VALUE),          # options before T == 0
    (dict(entropy=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(entropy=FAKE + 2), rlk.RLK_ERR_MISALIGNED),
    (dict(H=100, ldh=104, ldw=104), rlk.RLK_ERR_UNSUPPORTED),
    (dict(T=-1), rlk.RLK_ERR_INVALID_SHAPE),
    (dict(logp=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(ws=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(T=0, hidden=None, weight=None, targets=None, logp=None, lse=None, entropy=None,
          ws=None, ws_bytes=0), rlk.RLK_OK),
])
def test_selected_logp_ex_error_paths(kw, status):
    assert _ex(**kw) == status
    assert rlk.rlk_last_hip_error() == 0


def test_selected_logp_ex_entropy_needs_the_larger_workspace():
    T, V = 1000, 1000
    plain = rlk.rlk_workspace_bytes_ex(T, V, 0)
    assert plain < rlk.rlk_workspace_bytes_ex(T, V, rlk.RLK_ENTROPY)
    assert _ex(T=T, V=V, ws_bytes=plain) == rlk.RLK_ERR_WORKSPACE_TOO_SMALL
    # without the entropy flag the entropy pointer is ignored (may be NULL),
    # and validation gets as far as the workspace size
    assert _ex(T=T, V=V, flags=rlk.RLK_LOGITS_BF16, entropy=None,
               ws_bytes=plain - 1) == rlk.RLK_ERR_WORKSPACE_TOO_SMALL


@pytest.mark.parametrize("kw,status", [
    (dict(inv_tau=0.0), rlk.RLK_ERR_INVALID_VALUE),
    (dict(flags=8), rlk.RLK_ERR_INVALID_VALUE),
    (dict(v_begin=128, v_count=256), rlk.RLK_ERR_UNSUPPORTED),
    (dict(v_begin=128), rlk.RLK_ERR_INVALID_SHAPE),                 # past V
    (dict(ws_bytes=64), rlk.RLK_ERR_WORKSPACE_TOO_SMALL),
    (dict(targets=None), rlk.RLK_ERR_NULL_POINTER),
])
def test_vocab_stats_ex_error_paths(kw, status):
    a = dict(hidden=FAKE, ldh=256, weight=FAKE, ldw=256, targets=FAKE, T=4, H=256, V=1000,
             v_begin=0, v_count=1000, inv_tau=1.0, flags=rlk.RLK_ENTROPY, ws=WS_FAKE,
             ws_bytes=None)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = rlk.rlk_workspace_bytes_ex(4, 1000, rlk.RLK_ENTROPY)
    assert rlk.lib().rlk_vocab_stats_ex(
        a["hidden"], a["ldh"], a["weight"], a["ldw"], a["targets"], a["T"], a["H"], a["V"],
        a["v_begin"], a["v_count"], a["inv_tau"], a["flags"], a["ws"], a["ws_bytes"],
        None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(flags=4), rlk.RLK_ERR_INVALID_VALUE),
    (dict(entropy=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(entropy=FAKE + 1), rlk.RLK_ERR_MISALIGNED),
    (dict(ws_bytes=("plain",)), rlk.RLK_ERR_WORKSPACE_TOO_SMALL),
    (dict(T=0, targets=None, logp=None, lse=None, entropy=None, ws=None, ws_bytes=0),
     rlk.RLK_OK),
])
def test_vocab_merge_ex_error_paths(kw, status):
    a = dict(targets=FAKE, logp=FAKE, lse=FAKE, entropy=FAKE, T=1000, V=1000,
             flags=rlk.RLK_ENTROPY, ws=WS_FAKE, ws_bytes=None)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = rlk.rlk_workspace_bytes_ex(1000, 1000, rlk.RLK_ENTROPY)
    elif isinstance(a["ws_bytes"], tuple):
        a["ws_bytes"] = rlk.rlk_workspace_bytes_ex(1000, 1000, 0)
    assert rlk.lib().rlk_vocab_merge_ex(a["targets"], a["logp"], a["lse"], a["entropy"],
                                        a["T"], a["V"], a["flags"], a["ws"], a["ws_bytes"],
                                        None) == status


# --------------------------------------------------------------- backward --

def test_backward_workspace_size():
    wb = rlk.rlk_selected_logp_backward_workspace_bytes
    r = lambda x: (x + 255) // 256 * 256
    p = lambda x: (x + 63) // 64 * 64
    for T, H, V in [(1, 64, 1), (64, 256, 4096), (4096, 4096, 151936), (300, 192, 1000)]:
        # dz, hidden^T (the weight and dz are read as stored), then the
        # tile-claim counters
        want = r(T * p(V) * 2) + r(H * p(T) * 2) + 256
        assert wb(T, H, V) == want
    assert wb(0, 64, 10) == 0 and wb(4, 0, 10) == 0 and wb(4, 64, 0) == 0


def _bwd(hidden=FAKE, ldh=256, weight=FAKE, ldw=256, targets=FAKE, lse=FAKE, grad=FAKE,
         gh=FAKE, gw=FAKE, T=4, H=256, V=1000, inv_tau=1.0, ws=WS_FAKE, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = rlk.rlk_selected_logp_backward_workspace_bytes(T, H, V)
    return rlk.lib().rlk_selected_logp_backward(hidden, ldh, weight, ldw, targets, lse, grad,
                                                gh, gw, T, H, V, inv_tau, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(inv_tau=0.0), rlk.RLK_ERR_INVALID_VALUE),
    (dict(inv_tau=float("nan")), rlk.RLK_ERR_INVALID_VALUE),
    (dict(T=-1), rlk.RLK_ERR_INVALID_SHAPE),
    (dict(H=100, ldh=104, ldw=104), rlk.RLK_ERR_UNSUPPORTED),
    (dict(V=(1 << 21) + 1), rlk.RLK_ERR_UNSUPPORTED),              # V becomes a GEMM depth
    (dict(gh=None, gw=None), rlk.RLK_OK),                         # nothing asked for
    (dict(gh=FAKE + 2), rlk.RLK_ERR_MISALIGNED),
    (dict(gw=FAKE + 1), rlk.RLK_ERR_MISALIGNED),
    (dict(gw=FAKE + 4), rlk.RLK_ERR_MISALIGNED),                  # 16-byte pieces of its rows
    (dict(hidden=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(lse=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(grad=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(targets=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(ws=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(lse=FAKE + 2), rlk.RLK_ERR_MISALIGNED),
    (dict(ws=WS_FAKE + 8), rlk.RLK_ERR_MISALIGNED),
    (dict(ws_bytes=1024), rlk.RLK_ERR_WORKSPACE_TOO_SMALL),
    (dict(T=0, gw=None, hidden=None, weight=None, targets=None, lse=None, grad=None, ws=None,
          ws_bytes=0), rlk.RLK_OK),
])
def test_backward_error_paths(kw, status):
    assert _bwd(**kw) == status
    assert rlk.rlk_last_hip_error() == 0


def test_backward_workspace_shrinks_with_one_output():
    """Only grad_hidden: the h^T region is not needed."""
    T, H, V = 300, 192, 1000
    full = rlk.rlk_selected_logp_backward_workspace_bytes(T, H, V)
    r = lambda x: (x + 255) // 256 * 256
    only_h = r(T * 1024 * 2) + 256
    # one byte short of the grad_hidden-only layout is refused before any launch
    # (a call that passes validation would launch, so the exact size is not probed)
    assert _bwd(T=T, H=H, V=V, ldh=H, ldw=H, gw=None,
                ws_bytes=only_h - 1) == rlk.RLK_ERR_WORKSPACE_TOO_SMALL
    assert only_h < full


@pytest.mark.parametrize("kw,status", [
    (dict(inv_tau=-1.0), rlk.RLK_ERR_INVALID_VALUE),
    (dict(ld_dz=960), rlk.RLK_ERR_INVALID_SHAPE),                 # < V rounded up to 64
    (dict(ld_dz=1028), rlk.RLK_ERR_MISALIGNED),
    (dict(dz=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(dz=FAKE + 8), rlk.RLK_ERR_MISALIGNED),
    (dict(T=0, dz=None), rlk.RLK_OK),
])
def test_grad_logits_error_paths(kw, status):
    a = dict(hidden=FAKE, ldh=256, weight=FAKE, ldw=256, targets=FAKE, lse=FAKE, grad=FAKE,
             dz=FAKE, ld_dz=1024, T=4, H=256, V=1000, inv_tau=1.0)
    a.update(kw)
    assert rlk.lib().rlk_logp_grad_logits(a["hidden"], a["ldh"], a["weight"], a["ldw"],
                                          a["targets"], a["lse"], a["grad"], a["dz"],
                                          a["ld_dz"], a["T"], a["H"], a["V"], a["inv_tau"],
                                          None) == status


# ---------------------------------------------------------------- rmsnorm --

@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), rlk.RLK_ERR_INVALID_SHAPE),
    (dict(H=0), rlk.RLK_ERR_INVALID_SHAPE),
    (dict(ldx=56), rlk.RLK_ERR_INVALID_SHAPE),
    (dict(ldy=56), rlk.RLK_ERR_INVALID_SHAPE),
    (dict(H=60, ldx=64, ldy=64), rlk.RLK_ERR_UNSUPPORTED),
    (dict(eps=-1.0), rlk.RLK_ERR_INVALID_VALUE),
    (dict(eps=float("nan")), rlk.RLK_ERR_INVALID_VALUE),
    (dict(eps=float("inf")), rlk.RLK_ERR_INVALID_VALUE),
    (dict(x=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(gamma=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(y=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(x=FAKE + 8), rlk.RLK_ERR_MISALIGNED),
    (dict(gamma=FAKE + 4), rlk.RLK_ERR_MISALIGNED),
    (dict(ldy=68), rlk.RLK_ERR_MISALIGNED),
    (dict(T=0, x=None, gamma=None, y=None), rlk.RLK_OK),
])
def test_rmsnorm_error_paths(kw, status):
    a = dict(x=FAKE, ldx=64, gamma=FAKE, eps=1e-6, y=FAKE, ldy=64, T=4, H=64)
    a.update(kw)
    assert rlk.lib().rlk_rmsnorm(a["x"], a["ldx"], a["gamma"], a["eps"], a["y"], a["ldy"],
                                 a["T"], a["H"], None) == status


# ------------------------------------------------------------------ top-k --

@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), rlk.RLK_ERR_INVALID_SHAPE),
    (dict(V=0), rlk.RLK_ERR_INVALID_SHAPE),
    (dict(ld=999), rlk.RLK_ERR_INVALID_SHAPE),
    (dict(k=0), rlk.RLK_ERR_INVALID_VALUE),
    (dict(k=65), rlk.RLK_ERR_INVALID_VALUE),
    (dict(k=20, V=10, ld=10), rlk.RLK_ERR_INVALID_VALUE),
    (dict(inv_tau=0.0), rlk.RLK_ERR_INVALID_VALUE),
    (dict(flags=8), rlk.RLK_ERR_INVALID_VALUE),
    (dict(logits=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(lse=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(out_lp=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(out_id=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(logits=FAKE + 2), rlk.RLK_ERR_MISALIGNED),
    (dict(out_id=FAKE + 1), rlk.RLK_ERR_MISALIGNED),
    (dict(ws=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(ws=WS_FAKE + 4), rlk.RLK_ERR_MISALIGNED),
    (dict(ws_bytes=64), rlk.RLK_ERR_WORKSPACE_TOO_SMALL),
    (dict(T=0, logits=None, lse=None, ws=None, out_lp=None, out_id=None), rlk.RLK_OK),
])
def test_topk_error_paths(kw, status):
    a = dict(logits=FAKE, ld=1000, lse=FAKE, ws=WS_FAKE, ws_bytes=1 << 20, T=4, V=1000, k=5,
             inv_tau=1.0, flags=0, out_lp=FAKE, out_id=FAKE)
    a.update(kw)
    assert rlk.lib().rlk_topk_logp(a["logits"], a["ld"], a["lse"], a["ws"], a["ws_bytes"],
                                   a["T"], a["V"], a["k"], a["inv_tau"], a["flags"],
                                   a["out_lp"], a["out_id"], None) == status


def test_topk_direct_workspace_size():
    """k pair slots of 128 fp32 logits per row, then room for the rows whose
    k-th largest tile maximum is -inf (all ceil(V / 128) tiles each) when
    there are more tiles than k; 0 for invalid arguments."""
    wb = rlk.rlk_topk_logp_direct_workspace_bytes
    r = lambda x: (x + 255) // 256 * 256
    for T, V, k, d in [(4096, 151936, 20, 16), (300, 1000, 20, 7), (1, 128, 1, 0)]:
        nst = (V + 127) // 128
        d = d if nst > k else 0
        P = T * k + d * nst
        per_item = 256 if k > 32 else 128
        items = (P + per_item - 1) // per_item + nst
        want = (r(P * 512) + r(P * 4) + r(T * k * 4) + 2 * r(T * 4) + r(max(d, 1) * 4)
                + 3 * r(nst * 4) + r((nst + 1) * 4) + r(items * 4) + r(16))
        assert wb(T, V, k, d) == want, (T, V, k, d)
    assert wb(4096, 151936, 20, 17) > wb(4096, 151936, 20, 16)
    assert wb(300, 1000, 20, 1000) == wb(300, 1000, 20, 0)     # 8 tiles <= k: no extra room
    assert wb(0, 10, 1, 0) == 0 and wb(4, 0, 1, 0) == 0
    assert wb(4, 1000, 0, 0) == 0 and wb(4, 1000, 65, 0) == 0 and wb(4, 10, 20, 0) == 0
    assert wb(4, 1000, 5, -1) == 0
    assert wb(1 << 25, 151936, 64, 0) == 0                    # more than 2^30 pairs


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), rlk.RLK_ERR_INVALID_SHAPE),
    (dict(V=0), rlk.RLK_ERR_INVALID_SHAPE),
    (dict(H=100, ldh=104, ldw=104), rlk.RLK_ERR_UNSUPPORTED),
    (dict(k=0), rlk.RLK_ERR_INVALID_VALUE),
    (dict(k=65), rlk.RLK_ERR_INVALID_VALUE),
    (dict(k=20, V=10), rlk.RLK_ERR_INVALID_VALUE),
    (dict(dcap=-1), rlk.RLK_ERR_INVALID_VALUE),
    (dict(inv_tau=float("inf")), rlk.RLK_ERR_INVALID_VALUE),
    (dict(flags=4), rlk.RLK_ERR_INVALID_VALUE),
    (dict(T=1 << 25, k=64), rlk.RLK_ERR_UNSUPPORTED),
    (dict(hidden=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(lse=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(stats=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(ws=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(out_id=None), rlk.RLK_ERR_NULL_POINTER),
    (dict(hidden=FAKE + 8), rlk.RLK_ERR_MISALIGNED),
    (dict(stats=WS_FAKE + 4), rlk.RLK_ERR_MISALIGNED),
    (dict(out_lp=FAKE + 2), rlk.RLK_ERR_MISALIGNED),
    (dict(stats_bytes=64), rlk.RLK_ERR_WORKSPACE_TOO_SMALL),
    (dict(ws_bytes=64), rlk.RLK_ERR_WORKSPACE_TOO_SMALL),
    (dict(T=0, hidden=None, weight=None, lse=None, stats=None, ws=None, out_lp=None,
          out_id=None), rlk.RLK_OK),
])
def test_topk_direct_error_paths(kw, status):
    a = dict(hidden=FAKE, ldh=256, weight=FAKE, ldw=256, lse=FAKE, stats=WS_FAKE,
             stats_bytes=1 << 20, T=4, H=256, V=1000, k=5, inv_tau=1.0, flags=0, dcap=2,
             ws=WS_FAKE, ws_bytes=1 << 24, out_lp=FAKE, out_id=FAKE)
    a.update(kw)
    assert rlk.lib().rlk_topk_logp_direct(
        a["hidden"], a["ldh"], a["weight"], a["ldw"], a["lse"], a["stats"], a["stats_bytes"],
        a["T"], a["H"], a["V"], a["k"], a["inv_tau"], a["flags"], a["dcap"], a["ws"],
        a["ws_bytes"], a["out_lp"], a["out_id"], None) == status
    assert rlk.rlk_last_hip_error() == 0


def test_binding_type_errors_before_any_device_work():
    torch = pytest.importorskip("torch")
    h = torch.zeros((2, 64), dtype=torch.float32)
    w = torch.zeros((8, 64), dtype=torch.bfloat16)
    y = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(TypeError):
        rlk.rlk_selected_logp(h, w, y)                 # fp32 hidden
    with pytest.raises(TypeError):
        rlk.rlk_selected_logp_ex(h, w, y, entropy=True)  # fp32 hidden, option path
    with pytest.raises(ValueError):
        rlk.rlk_selected_logp(w[:2], w, y)             # host tensors


def test_workspace_layout():
    """The documented carve-up: part_m at 0, part_s and xt after whole
    256-byte-rounded regions, part_u after xt; the entropy workspace is the
    plain one plus one statistics region."""
    r = lambda x: (x + 255) // 256 * 256
    for T, V in [(1, 1), (64, 4096), (4096, 151936), (257, 129)]:
        st = r(((V + 127) // 128) * T * 4)
        lay = rlk.rlk_workspace_layout(T, V)
        assert lay == {"part_m": 0, "part_s": st, "xt": 2 * st, "part_u": 2 * st + r(4 * T)}
        assert rlk.rlk_workspace_layout(T, V, rlk.RLK_ENTROPY) == lay
        # the counters after the regions are the library's
        assert rlk.rlk_workspace_bytes_ex(T, V, 0) >= lay["part_u"]
        assert rlk.rlk_workspace_bytes_ex(T, V, rlk.RLK_ENTROPY) >= lay["part_u"] + st
    L = rlk.lib()
    assert L.rlk_workspace_layout(0, 10, 0, None, None, None, None) == rlk.RLK_ERR_INVALID_SHAPE
    assert L.rlk_workspace_layout(4, 0, 0, None, None, None, None) == rlk.RLK_ERR_INVALID_SHAPE
    assert L.rlk_workspace_layout(2 ** 31, 10, 0, None, None, None, None) == \
        rlk.RLK_ERR_UNSUPPORTED
    assert L.rlk_workspace_layout(4, 10, 8, None, None, None, None) == rlk.RLK_ERR_INVALID_VALUE
    assert L.rlk_workspace_layout(4, 10, 0, None, None, None, None) == rlk.RLK_OK
