"""C-ABI checks that need no GPU: the library loads, exports every function that
include/lla.h declares, and rejects bad arguments with the documented status before any
HIP call (the pointers passed here are never dereferenced)."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lla.h")


def _lib():
    from local_linear_attention_amd import lla
    if not os.path.exists(lla.library_path()):
        pytest.fail("liblla.so is not built (run __graft_entry__.build())")
    return lla.load_library()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(lla_\w+)\s*\(", src, flags=re.M)))


def declared_enums():
    src = open(HEADER).read()
    return {name: int(val) for name, val in re.findall(r"\b(LLA_\w+)\s*=\s*(\d+)", src)}


def test_header_declares_the_entry_points():
    assert declared_functions() == ["lla_decode", "lla_decode_workspace_size", "lla_decode_ws",
                                    "lla_forward", "lla_forward_ex", "lla_forward_fallback_rows",
                                    "lla_forward_noalloc",
                                    "lla_forward_workspace_bytes",
                                    "lla_forward_ws",
                                    "lla_parallax_backward", "lla_parallax_backward_workspace_size",
                                    "lla_parallax_decode", "lla_parallax_decode_workspace_size",
                                    "lla_parallax_decode_ws",
                                    "lla_parallax_forward", "lla_parallax_forward_ex",
                                    "lla_parallax_forward_stats",
                                    "lla_parallax_forward_ws", "lla_parallax_path_available",
                                    "lla_parallax_workspace_size",
                                    "lla_path_available", "lla_pool_trim", "lla_profile_collect",
                                    "lla_profile_enable", "lla_status_string", "lla_version",
                                    "lla_workspace_size"]


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_codes_match_header_and_binding():
    from local_linear_attention_amd import lla
    enums = declared_enums()
    for code, name in lla.STATUS.items():
        assert enums[name] == code
    assert enums["LLA_PATH_AUTO"] == lla.PATHS["auto"]
    assert enums["LLA_PATH_EXACT"] == lla.PATHS["exact"]
    assert enums["LLA_PATH_FAST"] == lla.PATHS["fast"]
    assert enums["LLA_PATH_CG"] == lla.PATHS["cg"]
    assert enums["LLA_DTYPE_F32"] == lla.DTYPES["f32"]
    assert enums["LLA_DTYPE_BF16"] == lla.DTYPES["bf16"]


def test_version_and_status_strings():
    lib = _lib()
    assert lib.lla_version() >= 100
    for s in range(9):
        assert lib.lla_status_string(s)
    assert lib.lla_status_string(99) == b"unknown status"


# Distinct fake device addresses, far apart, so only the tested fault triggers.
Q, K, V, OUT = 0x10000000, 0x20000000, 0x30000000, 0x40000000


def call(lib, q=Q, k=K, v=V, out=OUT, B=1, H=2, n=16, d=64, h=8.0, lam=0.1, dtype=1, path=None):
    args = [ctypes.c_void_p(q), ctypes.c_void_p(k), ctypes.c_void_p(v), ctypes.c_void_p(out),
            B, H, n, d, h, lam, dtype, None]
    if path is None:
        return lib.lla_forward(*args)
    return lib.lla_forward_ex(*args, path)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=0), 1), (dict(k=0), 1), (dict(v=0), 1), (dict(out=0), 1),
    (dict(B=0), 2), (dict(H=-1), 2), (dict(n=0), 2), (dict(n=2 ** 31), 2),
    (dict(B=2 ** 16, H=2 ** 16, n=2), 2),
    (dict(h=0.0), 3), (dict(h=-1.0), 3), (dict(h=math.inf), 3), (dict(h=math.nan), 3),
    (dict(lam=-1e-3), 3), (dict(lam=math.nan), 3), (dict(lam=math.inf), 3),
    (dict(d=48), 4), (dict(d=256), 4), (dict(d=0), 4), (dict(dtype=2), 4),
    (dict(out=Q + 64), 7), (dict(out=V - 64), 7),
])
def test_invalid_arguments_are_rejected_before_any_launch(kw, expect):
    lib = _lib()
    assert call(lib, **kw) == expect
    assert call(lib, path=1, **kw) == expect


def test_unknown_path_is_rejected():
    lib = _lib()
    assert call(lib, path=7) == 4


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from local_linear_attention_amd import lla
    monkeypatch.setattr(lla, "_LIB", None)
    monkeypatch.setattr(lla, "library_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        lla.load_library()


def test_path_availability_query():
    from local_linear_attention_amd import lla
    for dt in ("f32", "bf16"):
        for d in (16, 32, 64, 128):
            assert lla.lla_path_available("auto", dt, d)
            assert lla.lla_path_available("exact", dt, d)
        for d in (0, 8, 48, 256):
            assert not lla.lla_path_available("exact", dt, d)
    assert not lla.lla_path_available("fast", "f32", 64)  # the matrix-core path is bf16-only
    assert lla.lla_path_available("fast", "bf16", 64)


def test_workspace_size():
    from local_linear_attention_amd import lla
    from parity_util import fast_workspace_bytes as fast_bytes
    assert lla.lla_workspace_size(2, 16, 4096, 64, "bf16", "fast") == fast_bytes(32, 4096)
    assert lla.lla_workspace_size(2, 16, 4096, 64, "bf16", "auto") == fast_bytes(32, 4096)
    assert lla.lla_workspace_size(1, 1, 130, 64, "bf16", "fast") == fast_bytes(1, 130)
    assert lla.lla_workspace_size(1, 3, 300, 64, "bf16", "fast") == fast_bytes(3, 300)
    assert lla.lla_workspace_size(1, 8, 16384, 128, "bf16", "auto") == fast_bytes(8, 16384, 128)
    assert lla.lla_workspace_size(2, 3, 777, 128, "bf16", "fast") == fast_bytes(6, 777, 128)
    assert lla.lla_workspace_size(1, 2, 512, 128, "bf16", "fast") == 0     # every row is short (i < 4d)
    assert lla.lla_workspace_size(1, 2, 513, 128, "bf16", "fast") == fast_bytes(2, 513, 128) > 0
    assert lla.lla_workspace_size(1, 2, 192, 64, "bf16", "fast") == 0      # every row is short (i < 3d)
    assert lla.lla_workspace_size(1, 2, 193, 64, "bf16", "fast") == fast_bytes(2, 193) > 0
    # beyond the fast path's sequence limit AUTO falls back to the exact path (no scratch)
    assert lla.lla_workspace_size(1, 1, (1 << 22) + 1, 64, "bf16", "fast") == 0
    assert lla.lla_workspace_size(1, 1, (1 << 22) + 1, 64, "bf16", "auto") == 0
    assert lla.lla_workspace_size(1, 1, 100, 64, "bf16", "fast") == 0      # every row is short
    assert lla.lla_workspace_size(2, 16, 4096, 64, "bf16", "exact") == 0
    assert lla.lla_workspace_size(2, 16, 4096, 64, "f32", "auto") == 0
    assert lla.lla_workspace_size(2, 16, 4096, 48, "bf16", "auto") == 0     # unsupported d
    assert lla.lla_workspace_size(0, 16, 4096, 64, "bf16", "auto") == 0     # bad shape


def test_boundary_contract_names():
    # The boundary: lla_forward with the operation's own arguments (then dtype and stream),
    # the caller-workspace pair, status strings and the version.
    lib = _lib()
    for name in ("lla_forward", "lla_forward_workspace_bytes", "lla_forward_ws", "lla_status_string",
                 "lla_version"):
        assert name in declared_functions() and hasattr(lib, name), name
    from local_linear_attention_amd import lla
    for args in ((2, 16, 4096, 64, "bf16"), (1, 8, 16384, 128, "bf16"), (1, 4, 1024, 64, "f32"),
                 (4, 12, 2048, 64, "bf16"), (1, 1, 64, 16, "f32"), (1, 1, 100, 64, "bf16")):
        assert lla.lla_forward_workspace_bytes(*args) == lla.lla_workspace_size(*args, "auto"), args
    assert lla.lla_forward_workspace_bytes(0, 16, 4096, 64, "bf16") == 0


def test_forward_ws_rejects_overlapping_workspace():
    lib = _lib()
    args = [ctypes.c_void_p(Q), ctypes.c_void_p(K), ctypes.c_void_p(V), ctypes.c_void_p(OUT),
            1, 2, 4096, 64, 8.0, 0.1, 1, None, 2]
    from local_linear_attention_amd import lla
    need = lla.lla_workspace_size(1, 2, 4096, 64, "bf16", "fast")
    in_bytes, out_bytes = 2 * 4096 * 64 * 2, 2 * 4096 * 64 * 4
    assert need > 0
    # one byte of overlap is enough, at either end of any argument
    for ws in (Q, K + in_bytes - 1, V - need + 1, OUT + out_bytes // 2, Q - 256):
        assert lib.lla_forward_ws(*args, ctypes.c_void_p(ws), need) == 7, hex(ws)
    # a short workspace is reported as such first
    assert lib.lla_forward_ws(*args, ctypes.c_void_p(Q), need - 1) == 5
    # every other workspace-taking entry point checks the same way
    assert lib.lla_parallax_forward_ws(ctypes.c_void_p(Q), ctypes.c_void_p(K), ctypes.c_void_p(V),
                                       ctypes.c_void_p(RHO), ctypes.c_void_p(OUT), 1, 2, 4096, 64, 8.0, 1, None, 2,
                                       ctypes.c_void_p(RHO + 64),
                                       lla.lla_parallax_workspace_size(1, 2, 4096, 64, "bf16", "fast")) == 7
    dbytes = lla.lla_decode_workspace_size(1, 2, 4096, 64, "bf16")
    assert dbytes > 0
    assert lib.lla_decode_ws(ctypes.c_void_p(Q), ctypes.c_void_p(K), ctypes.c_void_p(V), ctypes.c_void_p(OUT),
                             1, 2, 4096, 64, 8.0, 0.01, 1, None, ctypes.c_void_p(K + 128), dbytes) == 7


def test_fallback_rows_query_validation_before_any_copy():
    # Every case returns before the library touches the device (no GPU here).
    lib = _lib()
    rows = ctypes.c_int64(-1)
    ws = ctypes.c_void_p(0x7f0000000000)
    def q(ws_ptr, nbytes, B=1, H=2, n=4096, d=64, dtype=1, path=0, out=ctypes.byref(rows)):
        return lib.lla_forward_fallback_rows(ws_ptr, nbytes, B, H, n, d, dtype, path, out, None)
    assert q(ws, 1 << 30, out=None) == 1                      # NULL result pointer
    assert q(ws, 1 << 30, d=48) == 4                          # unsupported head dimension
    assert q(ws, 1 << 30, B=0) == 2                           # bad shape
    rows.value = -1
    assert q(ws, 1 << 30, path=1) == 0 and rows.value == 0    # exact path: no workspace, no rows
    rows.value = -1
    assert q(ws, 1 << 30, dtype=0) == 0 and rows.value == 0   # fp32 resolves to the exact path
    rows.value = -1
    assert q(ws, 1 << 30, n=100) == 0 and rows.value == 0     # every row short: no workspace
    assert q(None, 0) == 5                                     # fast path needs its workspace
    from local_linear_attention_amd import lla
    need = lla.lla_workspace_size(1, 2, 4096, 64, "bf16", "auto")
    assert q(ws, need - 1) == 5


def test_forward_ws_validation_before_launch():
    lib = _lib()
    args = [ctypes.c_void_p(Q), ctypes.c_void_p(K), ctypes.c_void_p(V), ctypes.c_void_p(OUT),
            1, 2, 4096, 64, 8.0, 0.1, 1, None, 2]
    # fast path needs scratch: none or too little is refused before any launch
    assert lib.lla_forward_ws(*args, None, 0) == 5
    assert lib.lla_forward_ws(*args, ctypes.c_void_p(0x50000000), 1024) == 5
    bad = list(args)
    bad[7] = 32
    assert lib.lla_forward_ws(*bad, None, 0) == 4  # fast path does not cover d = 32


def test_profile_collect_without_launches():
    from local_linear_attention_amd import lla
    prev = lla.lla_profile_enable(True)
    assert lla.lla_profile_collect() == []
    lla.lla_profile_enable(prev)


# ---------------------------------------------------------------- Parallax entry points
RHO = 0x60000000


def call_parallax(lib, q=Q, k=K, v=V, rho=RHO, out=OUT, B=1, H=2, n=16, d=64, h=8.0, dtype=1, path=None):
    args = [ctypes.c_void_p(q), ctypes.c_void_p(k), ctypes.c_void_p(v), ctypes.c_void_p(rho),
            ctypes.c_void_p(out), B, H, n, d, h, dtype, None]
    if path is None:
        return lib.lla_parallax_forward(*args)
    return lib.lla_parallax_forward_ex(*args, path)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=0), 1), (dict(k=0), 1), (dict(v=0), 1), (dict(rho=0), 1), (dict(out=0), 1),
    (dict(B=0), 2), (dict(n=0), 2), (dict(n=2 ** 31), 2),
    (dict(h=0.0), 3), (dict(h=-2.0), 3), (dict(h=math.nan), 3), (dict(h=math.inf), 3),
    (dict(d=48), 4), (dict(d=256), 4), (dict(dtype=2), 4),
    (dict(out=Q + 64), 7), (dict(out=RHO - 64), 7), (dict(out=RHO + 128), 7),
])
def test_parallax_invalid_arguments_are_rejected_before_any_launch(kw, expect):
    lib = _lib()
    assert call_parallax(lib, **kw) == expect
    assert call_parallax(lib, path=1, **kw) == expect
    assert call_parallax(lib, path=2, **kw) == expect


def test_parallax_unknown_or_uncovered_path_is_rejected():
    lib = _lib()
    assert call_parallax(lib, path=7) == 4
    assert call_parallax(lib, path=2, d=32) == 4      # the matrix-core path is d = 64 only
    assert call_parallax(lib, path=2, dtype=0) == 4   # and bf16 only
    assert call_parallax(lib, path=3) == 4            # CG solves the LLA system; Parallax has none


def test_cg_path_is_an_lla_path_with_a_row_list_scratch():
    # The CG path keeps no d x d state; its scratch is the list of rows whose iteration did not
    # converge (a count, then one 32-bit entry per row), which the direct solve then takes.
    from local_linear_attention_amd import lla
    lib = _lib()
    for dt in ("f32", "bf16"):
        for d in (16, 32, 64, 128):
            assert lla.lla_path_available("cg", dt, d)
            assert lla.lla_workspace_size(2, 3, 500, d, dt, "cg") == 256 + (6 * 500 * 4 + 255) // 256 * 256
    assert not lla.lla_path_available("cg", "bf16", 48)
    assert not lla.lla_parallax_path_available("cg", "bf16", 64)
    # validation happens before any launch on the CG path too
    assert call(lib, path=3, q=0) == 1
    assert call(lib, path=3, n=0) == 2
    assert call(lib, path=3, lam=-1.0) == 3
    assert call(lib, path=3, d=48) == 4
    assert call(lib, path=3, out=Q + 16) == 7
    # the _ws entry point needs that scratch on the CG path
    need = lla.lla_workspace_size(1, 2, 4096, 64, "bf16", "cg")
    args = [ctypes.c_void_p(Q), ctypes.c_void_p(K), ctypes.c_void_p(V), ctypes.c_void_p(OUT),
            1, 2, 4096, 64, 8.0, 0.1, 1, None, 3]
    assert lib.lla_forward_ws(*args, None, 0) == 5
    assert lib.lla_forward_ws(*args, ctypes.c_void_p(0x7e0000000000), need - 1) == 5


def parallax_workspace_bytes(BH, n):
    """Scratch of the Parallax matrix-core path: per head and 64-key tile the image (bf16 K
    key-major with 72-half rows, fp16 V feature-major with 68-half rows, padded to whole KiB),
    the tile key sum (64 floats), the largest key norm and the largest |v| (one float each);
    then the count of heads left to the fp64 fallback (one unsigned) and their list (one int
    per head); each region rounded up to 256 B."""
    up = lambda x: (x + 255) // 256 * 256
    tiles = -(-n // 64)
    image = -(-(64 * 72 * 2 + 64 * 68 * 2) // 1024) * 1024
    return (up(BH * tiles * image) + up(BH * tiles * 64 * 4) + 2 * up(BH * tiles * 4) + up(4)
            + up(BH * 4))


def test_parallax_workspace_size_and_paths():
    from local_linear_attention_amd import lla
    assert lla.lla_parallax_workspace_size(2, 16, 4096, 64, "bf16", "fast") == parallax_workspace_bytes(32, 4096)
    assert lla.lla_parallax_workspace_size(2, 16, 4096, 64, "bf16", "auto") == parallax_workspace_bytes(32, 4096)
    assert lla.lla_parallax_workspace_size(1, 3, 1, 64, "bf16", "fast") == parallax_workspace_bytes(3, 1)
    assert lla.lla_parallax_workspace_size(1, 1, 300, 64, "bf16", "exact") == 0
    assert lla.lla_parallax_workspace_size(1, 1, 300, 64, "f32", "auto") == 0
    assert lla.lla_parallax_workspace_size(1, 1, (1 << 22) + 1, 64, "bf16", "auto") == 0
    assert lla.lla_parallax_workspace_size(1, 1, 300, 48, "bf16", "auto") == 0
    for dt in ("f32", "bf16"):
        for d in (16, 32, 64, 128):
            assert lla.lla_parallax_path_available("auto", dt, d)
            assert lla.lla_parallax_path_available("exact", dt, d)
        assert not lla.lla_parallax_path_available("exact", dt, 48)
    assert lla.lla_parallax_path_available("fast", "bf16", 64)
    assert not lla.lla_parallax_path_available("fast", "bf16", 128)
    assert not lla.lla_parallax_path_available("fast", "f32", 64)


def test_parallax_ws_validation_before_launch():
    lib = _lib()
    args = [ctypes.c_void_p(Q), ctypes.c_void_p(K), ctypes.c_void_p(V), ctypes.c_void_p(RHO),
            ctypes.c_void_p(OUT), 1, 2, 4096, 64, 8.0, 1, None, 2]
    assert lib.lla_parallax_forward_ws(*args, None, 0) == 5
    assert lib.lla_parallax_forward_ws(*args, ctypes.c_void_p(0x50000000), 4096) == 5


# ---------------------------------------------------------------- Parallax decode
def call_decode(lib, q=Q, k=K, v=V, rho=RHO, out=OUT, B=2, H=3, L=100, d=64, h=8.0, dtype=1):
    return lib.lla_parallax_decode(ctypes.c_void_p(q), ctypes.c_void_p(k), ctypes.c_void_p(v),
                                   ctypes.c_void_p(rho), ctypes.c_void_p(out), B, H, L, d, h, dtype, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=0), 1), (dict(k=0), 1), (dict(v=0), 1), (dict(rho=0), 1), (dict(out=0), 1),
    (dict(B=0), 2), (dict(H=0), 2), (dict(L=0), 2), (dict(L=2 ** 31), 2),
    (dict(h=0.0), 3), (dict(h=math.inf), 3), (dict(h=math.nan), 3),
    (dict(d=48), 4), (dict(d=256), 4), (dict(dtype=2), 4),
    (dict(out=Q + 64), 7), (dict(out=RHO - 64), 7), (dict(out=K + 4096), 7), (dict(out=V + 64), 7),
])
def test_decode_invalid_arguments_are_rejected_before_any_launch(kw, expect):
    assert call_decode(_lib(), **kw) == expect


def decode_split(BH, L):
    """Chunks per head of the decode kernels: about 1024 blocks in all, chunks of 256 to 2048
    keys, none empty."""
    s = max(1, -(-1024 // BH))
    s = min(s, -(-L // 256))
    s = max(s, -(-L // 2048))
    c = -(-L // s)
    return -(-L // c), c


def test_decode_workspace_size():
    from local_linear_attention_amd import lla
    for B, H, L, d in ((8, 16, 8192, 64), (1, 16, 32768, 64), (64, 16, 1024, 64), (8, 8, 8192, 128),
                       (1, 1, 300, 16), (4, 4, 200, 32), (512, 16, 256, 64)):
        S, _ = decode_split(B * H, L)
        expect = 0 if S == 1 else B * H * S * (4 + 2 * d) * 4
        assert lla.lla_parallax_decode_workspace_size(B, H, L, d, "bf16") == expect, (B, H, L, d)
        assert lla.lla_parallax_decode_workspace_size(B, H, L, d, "f32") == expect
    assert lla.lla_parallax_decode_workspace_size(1, 1, 1, 64, "bf16") == 0
    assert lla.lla_parallax_decode_workspace_size(1, 1, 100, 48, "bf16") == 0


def test_decode_ws_validation_before_launch():
    lib = _lib()
    args = [ctypes.c_void_p(Q), ctypes.c_void_p(K), ctypes.c_void_p(V), ctypes.c_void_p(RHO),
            ctypes.c_void_p(OUT), 1, 2, 4096, 64, 8.0, 1, None]
    assert lib.lla_parallax_decode_ws(*args, None, 0) == 5
    assert lib.lla_parallax_decode_ws(*args, ctypes.c_void_p(0x50000000), 64) == 5


# ---------------------------------------------------------------- LLA decode
def call_lla_decode(lib, q=Q, k=K, v=V, out=OUT, B=2, H=3, L=100, d=64, h=8.0, lam=0.01, dtype=1):
    return lib.lla_decode(ctypes.c_void_p(q), ctypes.c_void_p(k), ctypes.c_void_p(v), ctypes.c_void_p(out),
                          B, H, L, d, h, lam, dtype, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=0), 1), (dict(k=0), 1), (dict(v=0), 1), (dict(out=0), 1),
    (dict(B=0), 2), (dict(L=0), 2), (dict(L=2 ** 31), 2),
    (dict(h=0.0), 3), (dict(h=math.nan), 3), (dict(lam=-1.0), 3), (dict(lam=math.inf), 3),
    (dict(d=48), 4), (dict(dtype=2), 4),
    (dict(out=Q + 64), 7), (dict(out=K + 4096), 7), (dict(out=V - 64), 7),
])
def test_lla_decode_invalid_arguments_are_rejected_before_any_launch(kw, expect):
    assert call_lla_decode(_lib(), **kw) == expect


def lla_decode_split(BH, L):
    """Chunks per head of the LLA decode kernels: about 1024 blocks in all, chunks of 512 to
    2048 keys, none empty."""
    s = -(-1024 // BH)
    s = min(s, -(-L // 512))
    s = max(s, -(-L // 2048), 1)
    c = -(-L // s)
    return -(-L // c)


def test_lla_decode_workspace_size():
    from local_linear_attention_amd import lla
    for B, H, L, d, dt in ((8, 16, 8192, 64, "bf16"), (1, 1, 100, 64, "bf16"), (2, 3, 700, 16, "f32"),
                           (1, 2, 5000, 128, "bf16"), (4, 4, 1000, 32, "f32"), (64, 16, 1024, 64, "bf16")):
        S = lla_decode_split(B * H, L)
        nb = d // 16
        nt = nb * (nb + 1) // 2 + nb * nb
        ta = 8 if (dt == "f32" or L < 2 * d) else 4
        e = nt * 256 + d
        stats = -(-(B * H * S * (2 + d) * 8) // 256) * 256
        scores = -(-(B * H * L * 4) // 256) * 256 if ta == 4 else 0   # split-operand moments
        mom = -(-(B * H * S * e * ta) // 256) * 256
        summed = B * H * e * 8 if S > 1 else 0
        assert lla.lla_decode_workspace_size(B, H, L, d, dt) == stats + scores + mom + summed, (B, H, L, d)
    assert lla.lla_decode_workspace_size(1, 1, 100, 48, "bf16") == 0


def test_lla_decode_ws_validation_before_launch():
    lib = _lib()
    args = [ctypes.c_void_p(Q), ctypes.c_void_p(K), ctypes.c_void_p(V), ctypes.c_void_p(OUT),
            1, 2, 4096, 64, 8.0, 0.01, 1, None]
    assert lib.lla_decode_ws(*args, None, 0) == 5
    assert lib.lla_decode_ws(*args, ctypes.c_void_p(0x50000000), 64) == 5


# ---- Parallax forward with statistics and backward: validation happens before any launch
# (the fake addresses are never dereferenced).
RHO, DOUT, STATS, DQ, DK, DV, DR = (0x50000000, 0x60000000, 0x70000000, 0x80000000, 0x90000000, 0xA0000000,
                                    0xB0000000)


def stats_call(lib, stats=STATS, out=OUT, q=Q, B=1, H=2, n=16, d=64, h=8.0, dtype=1, path=0, ws=None, wsb=0):
    return lib.lla_parallax_forward_stats(ctypes.c_void_p(q), ctypes.c_void_p(K), ctypes.c_void_p(V),
                                          ctypes.c_void_p(RHO), ctypes.c_void_p(out),
                                          ctypes.c_void_p(stats) if stats else None, B, H, n, d, h, dtype, None,
                                          path, ws, wsb)


def bwd_call(lib, dq=DQ, dk=DK, dv=DV, dr=DR, dout=DOUT, stats=STATS, B=1, H=2, n=16, d=64, h=8.0, dtype=1,
             path=0, ws=None, wsb=0):
    p = [ctypes.c_void_p(x) if x else None for x in (Q, K, V, RHO, dout, stats, dq, dk, dv, dr)]
    return lib.lla_parallax_backward(*p, B, H, n, d, h, dtype, None, path, ws, wsb)


def test_parallax_forward_stats_validation():
    lib = _lib()
    assert stats_call(lib, stats=0) == 1
    assert stats_call(lib, q=0) == 1
    assert stats_call(lib, n=0) == 2
    assert stats_call(lib, h=0.0) == 3
    assert stats_call(lib, d=48) == 4
    assert stats_call(lib, dtype=0, path=2) == 4            # FAST is bf16 only
    assert stats_call(lib, stats=Q + 64) == 7               # stats overlaps q
    assert stats_call(lib, stats=OUT + 1024) == 7           # lse overlaps out
    # a caller workspace that is too small
    assert stats_call(lib, n=4096, path=2, ws=ctypes.c_void_p(0xC0000000), wsb=64) == 5


def test_parallax_backward_validation():
    lib = _lib()
    for kw in ({"dq": 0}, {"dk": 0}, {"dv": 0}, {"dr": 0}, {"dout": 0}, {"stats": 0}):
        assert bwd_call(lib, **kw) == 1, kw
    assert bwd_call(lib, B=0) == 2
    assert bwd_call(lib, h=-1.0) == 3
    assert bwd_call(lib, h=float("nan")) == 3
    assert bwd_call(lib, d=96) == 4
    assert bwd_call(lib, dtype=0, path=2) == 4
    assert bwd_call(lib, d=32, path=2) == 4
    assert bwd_call(lib, dq=DOUT + 8) == 7                  # gradient over an input
    assert bwd_call(lib, dk=DQ + 16) == 7                   # two gradients overlap
    assert bwd_call(lib, dr=STATS + 4) == 7                 # gradient over the log-sum-exp
    assert bwd_call(lib, n=4096, path=2, ws=ctypes.c_void_p(0xC0000000), wsb=1024) == 5
    assert bwd_call(lib, n=100, path=1, ws=ctypes.c_void_p(0xC0000000), wsb=8) == 5


def test_parallax_backward_workspace_size():
    from local_linear_attention_amd import lla
    for B, H, n in ((2, 16, 4096), (1, 1, 1), (3, 2, 130)):
        tiles = -(-n // 64)
        assert lla.lla_parallax_backward_workspace_size(B, H, n, 64, "bf16", "fast") == B * H * tiles * (55296 + 27648)
        assert lla.lla_parallax_backward_workspace_size(B, H, n, 64, "bf16", "auto") == B * H * tiles * (55296 + 27648)
        assert lla.lla_parallax_backward_workspace_size(B, H, n, 64, "bf16", "exact") == B * H * n * 32
        assert lla.lla_parallax_backward_workspace_size(B, H, n, 32, "f32", "auto") == B * H * n * 32
    assert lla.lla_parallax_backward_workspace_size(1, 1, 10, 32, "bf16", "fast") == 0
    assert lla.lla_parallax_backward_workspace_size(1, 1, 10, 48, "bf16", "auto") == 0
