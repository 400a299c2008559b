"""C-ABI checks that need no GPU: the library loads, exports every symbol that
include/w4a16_moe.h declares, and rejects bad arguments on the host before
anything is enqueued (no HIP call is reached on these paths)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER_DIR = os.path.join(ROOT, "include")


def declared_functions():
    names = []
    for fn in sorted(os.listdir(HEADER_DIR)):
        if not fn.endswith(".h"):
            continue
        src = open(os.path.join(HEADER_DIR, fn)).read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        src = re.sub(r"^\s*#.*$", " ", src, flags=re.M)
        src = re.sub(r"typedef\s+struct\s*\{.*?\}\s*\w+\s*;", " ", src, flags=re.S)
        src = re.sub(r"enum\s+\w*\s*\{.*?\}\s*;", " ", src, flags=re.S)
        for m in re.finditer(r"(?:^|;)\s*(?:const\s+)?[A-Za-z_][\w]*\s*\**\s+\**\s*([A-Za-z_]\w*)\s*\(", src, re.M):
            names.append(m.group(1))
    return names


@pytest.fixture(scope="module")
def L():
    from w4a16_grouped_expert_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail(f"library not built: {_lib.LIB_PATH}")
    return _lib.lib()


def test_header_declares_the_five_entry_points():
    names = set(declared_functions())
    for n in ("moe_route", "moe_align", "moe_w4a16_grouped_ffn", "pack_w4_g128", "slot_cache_load"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 15
    raw = ctypes.CDLL(os.path.join(ROOT, "w4a16_grouped_expert_amd", "lib", "libw4a16moe.so"))
    missing = [n for n in names if not hasattr(raw, n)]
    assert not missing, missing


def test_binding_covers_every_declared_symbol(L):
    from w4a16_grouped_expert_amd import _lib
    assert set(declared_functions()) == set(_lib.SIGNATURES)


def test_status_strings(L):
    assert L.moe_status_string(0) == b"MOE_OK"
    assert L.moe_status_string(2) == b"MOE_ERR_UNSUPPORTED_SHAPE"
    assert L.moe_abi_version() == 1


def test_layout_matches_oracle_blob_layout(L):
    from oracle import quant
    from w4a16_grouped_expert_amd import _lib
    for d, I in ((256, 512), (2048, 1024), (4096, 14336), (128, 128)):
        lay = _lib.ExpertLayout()
        assert L.moe_expert_layout_get(d, I, ctypes.byref(lay)) == 0
        offs, total = quant.blob_layout(d, I)
        assert (lay.w13_codes, lay.w13_scales, lay.w2_codes, lay.w2_scales) == offs
        assert lay.blob_bytes == total
    lay = _lib.ExpertLayout()
    assert L.moe_expert_layout_get(2000, 1024, ctypes.byref(lay)) == 2
    assert b"multiples of 128" in L.moe_last_error()


def test_host_side_argument_checks(L):
    vp = ctypes.c_void_p(16)  # never dereferenced: every call below fails its host checks first
    # pack: K not a multiple of 128, N not a multiple of 16, interleave needs N % 32
    assert L.pack_w4_g128(vp, 1, 16, 100, 0, vp, 0, vp, 0, None) == 2
    assert L.pack_w4_g128(vp, 1, 24, 128, 0, vp, 0, vp, 0, None) == 2
    assert L.pack_w4_g128(vp, 1, 48, 128, 1, vp, 0, vp, 0, None) == 2
    assert L.pack_w4_g128(vp, -1, 16, 128, 0, vp, 0, vp, 0, None) == 1
    assert L.pack_w4_g128(None, 1, 16, 128, 0, vp, 0, vp, 0, None) == 1
    assert L.pack_w4_g128(None, 0, 16, 128, 0, None, 0, None, 0, None) == 0   # empty: no-op
    # route: k > E, E > 1024, d % 8, null outputs
    assert L.moe_route(vp, vp, 4, 64, 8, 9, 1, vp, vp, vp, None) == 2
    assert L.moe_route(vp, vp, 4, 64, 2000, 8, 1, vp, vp, vp, None) == 2
    assert L.moe_route(vp, vp, 4, 60, 8, 2, 1, vp, vp, vp, None) == 2
    assert L.moe_route(vp, vp, 4, 64, 8, 2, 1, None, vp, vp, None) == 1
    assert L.moe_route(None, None, 0, 64, 8, 2, 1, None, None, None, None) == 0  # T = 0: no-op
    # align: E > 1024, k > 16, block_m without tile_offsets
    assert L.moe_align(vp, 4, 2, 1025, 0, vp, vp, vp, vp, None, None) == 2
    assert L.moe_align(vp, 4, 17, 64, 0, vp, vp, vp, vp, None, None) == 2
    assert L.moe_align(vp, 4, 2, 8, 64, vp, vp, vp, vp, None, None) == 1
    # ffn: null args, bad shapes, small workspace
    from w4a16_grouped_expert_amd import _lib
    assert L.moe_w4a16_grouped_ffn(None, None) == 1
    a = _lib.FfnArgs()
    a.T, a.d, a.I, a.E, a.k = 4, 200, 512, 8, 2
    assert L.moe_w4a16_grouped_ffn(ctypes.byref(a), None) == 2
    a.d = 256
    assert L.moe_w4a16_grouped_ffn(ctypes.byref(a), None) == 1            # null pointers
    for f in ("x", "topk_ids", "topk_weights", "expert_offsets", "sorted_pairs", "pair_pos", "active_experts",
              "out"):
        setattr(a, f, 256)
    a.bank, a.bank_stride, a.workspace, a.combine = 256, 202752, 256, 1
    a.workspace_bytes = 16
    assert L.moe_w4a16_grouped_ffn(ctypes.byref(a), None) == 3           # workspace too small
    assert b"workspace" in L.moe_last_error()
    a.bank_stride = 1000
    assert L.moe_w4a16_grouped_ffn(ctypes.byref(a), None) == 1           # stride below one blob
    # slot cache: argument validation before any allocation
    h = ctypes.c_void_p()
    assert L.moe_slot_cache_create(0, 16, 100, vp, vp, ctypes.byref(h)) == 1
    assert L.moe_slot_cache_create(64, 16, 100, None, vp, ctypes.byref(h)) == 1
    assert L.slot_cache_load(None, None, None, None, None, None, None, None, None) == 1
    assert L.moe_slot_cache_configure(None, 0, 0.9, 1) == 1
    assert L.slot_cache_begin_step(None, None) == 1
    assert L.moe_timing_read(99, None, None) == 1


def test_workspace_bytes_sizes(L):
    # h [T*k, I] bf16 + y [ksplit, T*k, d] fp32, each rounded up to 256 bytes
    ws = L.moe_ffn_workspace_bytes(16, 2048, 1024, 64, 8, 1)
    assert ws >= 16 * 8 * 1024 * 2 + 16 * 8 * 2048 * 4
    assert L.moe_ffn_workspace_bytes(-1, 2048, 1024, 64, 8, 0) == -1


def test_decode_layer_host_checks(L):
    """moe_decode_layer: argument errors are reported before anything is enqueued."""
    from w4a16_grouped_expert_amd import _lib
    vp = 256
    assert L.moe_decode_layer(None, None) == 1
    a = _lib.LayerArgs()
    a.T, a.d, a.I, a.E, a.k, a.renormalize = 17, 256, 512, 8, 2, 1
    assert L.moe_decode_layer(ctypes.byref(a), None) == 2                # T > 16
    a.T, a.d = 4, 8192
    assert L.moe_decode_layer(ctypes.byref(a), None) == 2                # d > 4096
    a.d = 256
    assert L.moe_decode_layer(ctypes.byref(a), None) == 1                # null pointers
    for f in ("x", "w_router", "bank", "logits", "topk_ids", "topk_weights", "out", "workspace", "counters"):
        setattr(a, f, vp)
    a.bank_stride = 202752
    a.workspace_bytes = 16
    assert L.moe_decode_layer(ctypes.byref(a), None) == 3                # workspace too small
    a.workspace_bytes = L.moe_decode_layer_workspace_bytes(4, 256, 512, 8, 2)
    a.bank_stride = 1000
    assert L.moe_decode_layer(ctypes.byref(a), None) == 1                # stride below one blob
    a.T = 0
    assert L.moe_decode_layer(ctypes.byref(a), None) == 0                # T = 0: no-op
    # workspace: h [T*k, I] bf16 + the down pass's partial sums, 256-byte granules
    ws = L.moe_decode_layer_workspace_bytes(16, 2048, 1024, 64, 8)
    assert ws >= 16 * 8 * 1024 * 2 + (2048 // 32) * 32 * 512 * 4
    assert L.moe_decode_layer_workspace_bytes(-1, 2048, 1024, 64, 8) == -1


def test_mat_decode_layer_host_checks(L):
    """moe_mat_decode_layer: argument errors are reported before anything is enqueued."""
    from w4a16_grouped_expert_amd import _lib
    vp = 256
    assert L.moe_mat_decode_layer(None, 0.0, None) == 1
    a = _lib.LayerArgs()
    a.T, a.d, a.I, a.E, a.k, a.renormalize = 17, 256, 512, 8, 2, 1
    assert L.moe_mat_decode_layer(ctypes.byref(a), 0.0, None) == 2       # T > 16
    a.T, a.d = 4, 384
    assert L.moe_mat_decode_layer(ctypes.byref(a), 0.0, None) == 2       # d not a multiple of 256
    a.d = 256
    assert L.moe_mat_decode_layer(ctypes.byref(a), float("nan"), None) == 1  # NaN tau
    assert L.moe_mat_decode_layer(ctypes.byref(a), 0.5, None) == 1       # null pointers
    for f in ("x", "w_router", "bank", "logits", "topk_ids", "topk_weights", "out", "workspace", "counters"):
        setattr(a, f, vp)
    a.bank_stride = 202752
    a.workspace_bytes = 16
    assert L.moe_mat_decode_layer(ctypes.byref(a), 2.0, None) == 3       # workspace too small
    a.workspace_bytes = L.moe_decode_layer_workspace_bytes(4, 256, 512, 8, 2)
    a.bank_stride = 1000
    assert L.moe_mat_decode_layer(ctypes.byref(a), 0.0, None) == 1       # stride below one blob
    a.T = 0
    assert L.moe_mat_decode_layer(ctypes.byref(a), 0.1, None) == 0       # T = 0: no-op


def test_noalloc_host_checks(L):
    """moe_w4a16_grouped_ffn_noalloc: a caller workspace or a step whose workspace
    exceeds the scratch is refused on the host, before any device call."""
    from w4a16_grouped_expert_amd import _lib
    assert L.moe_w4a16_grouped_ffn_noalloc(None, None) == 1
    a = _lib.FfnArgs()
    a.T, a.d, a.I, a.E, a.k, a.mode = 4096, 2048, 1024, 64, 8, 2
    a.workspace, a.workspace_bytes = 256, 1 << 20
    assert L.moe_w4a16_grouped_ffn_noalloc(ctypes.byref(a), None) == 1   # caller workspace given
    a.workspace, a.workspace_bytes = None, 0
    assert L.moe_w4a16_grouped_ffn_noalloc(ctypes.byref(a), None) == 3   # needs more than the scratch
    assert b"scratch" in L.moe_last_error()
    a.T = 0
    assert L.moe_w4a16_grouped_ffn_noalloc(ctypes.byref(a), None) == 0   # T = 0: no-op


def test_mat_layout_matches_oracle(L):
    """Layout m1 on the host: section offsets, blob size and the two-bit prefix equal
    the oracle's (the prefix holds the high planes and scales, the low planes follow)."""
    from oracle import matryoshka as omat
    from w4a16_grouped_expert_amd import _lib
    for d, I in ((256, 512), (2048, 1024), (4096, 14336)):
        lay = _lib.MatLayout()
        assert L.moe_mat_layout_get(d, I, ctypes.byref(lay)) == 0
        offs, total = omat.blob_layout_m1(d, I)
        assert (lay.w13_hi, lay.w13_lo, lay.w13_scales, lay.w2_hi, lay.w2_lo, lay.w2_scales) == offs
        assert lay.blob_bytes == total and lay.two_bit_bytes == omat.two_bit_prefix_m1(d, I)


def _run_with_log(level):
    import subprocess
    import sys
    code = (
        "import ctypes\n"
        "from w4a16_grouped_expert_amd import _lib\n"
        "L = _lib.lib()\n"
        "vp = ctypes.c_void_p(16)\n"
        "assert L.moe_route(vp, vp, 4, 64, 8, 9, 1, vp, vp, vp, None) == 2\n"
        "print('msg=' + L.moe_last_error().decode())\n"
    )
    env = dict(os.environ)
    env.pop("MOE_W4A16_LOG", None)
    if level is not None:
        env["MOE_W4A16_LOG"] = str(level)
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    msg = r.stdout.strip().splitlines()[-1][len("msg="):]
    return msg, [l for l in r.stderr.splitlines() if l.startswith("[w4a16_moe]")]


def test_log_level_env():
    """MOE_W4A16_LOG=1 echoes each recorded error message to stderr; unset, the
    library prints nothing (the message stays available through moe_last_error)."""
    msg, lines = _run_with_log(None)
    assert msg and lines == []
    msg1, lines1 = _run_with_log(1)
    assert msg1 == msg
    assert lines1 == ["[w4a16_moe] error: " + msg]
