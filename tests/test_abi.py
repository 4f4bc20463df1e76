"""The C ABI on the CPU: libfp4q.so loads, exports every function include/fp4q.h
declares, and rejects bad arguments with the documented status before any
launch (no GPU is touched: every call here fails validation or is an empty
no-op)."""
import ctypes
import os
import re
import threading

import pytest

import microscaling_fp4_quantization_amd as fq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4q.h")

OK, ARG, SHAPE, ALIGN, WS = 0, 1, 2, 3, 4
A16 = 0x10000  # fake, suitably aligned device addresses (never dereferenced)
A16b = 0x20000
A16c = 0x30000
WSB = 1 << 20


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fq.LIB_PATH):
        from microscaling_fp4_quantization_amd import build
        build.build()
    return fq.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    assert names == sorted(fq.EXPORTS), names


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name
    assert L.fp4q_abi_version() == 2
    assert L.fp4q_workspace_bytes(1, 32, 32) > 0


def mx(L, x=A16, xt=0, rows=4, cols=64, rot=0, codes=A16b, scales=A16c, bm=None, kind=0,
       stats=None, ws=None, wsb=0):
    return L.mxfp4_quantize(x, xt, rows, cols, rot, codes, scales, bm, kind, stats, ws, wsb, None)


def nv(L, x=A16, xt=0, rows=4, cols=64, block=16, fmt=1, gmode=0, g=None, rot=0, codes=A16b,
       scales=A16c, bm=None, kind=0, stats=None, ws=None, wsb=0):
    return L.nvfp4_quantize(x, xt, rows, cols, block, fmt, gmode, g, rot, codes, scales, bm, kind,
                            stats, ws, wsb, None)


def err(L):
    return L.fp4q_last_error().decode()


def test_mxfp4_validation(L):
    assert mx(L, x=None) == ARG and "NULL" in err(L)
    assert mx(L, codes=None) == ARG
    assert mx(L, xt=7) == ARG and "dtype" in err(L)
    assert mx(L, cols=48) == SHAPE and "multiple" in err(L)
    assert mx(L, rows=-1) == SHAPE
    assert mx(L, rows=1 << 62, cols=1 << 10) == SHAPE and "overflow" in err(L)
    assert mx(L, rows=1 << 31, cols=512) == SHAPE and "limit" in err(L)
    assert mx(L, rot=16) == SHAPE
    assert mx(L, x=A16 + 8) == ALIGN
    assert mx(L, codes=A16b + 4) == ALIGN
    assert mx(L, bm=A16 + 2) == ALIGN
    assert mx(L, kind=5) == ARG
    assert mx(L, stats=A16) == WS and "workspace" in err(L)
    assert mx(L, stats=A16, ws=A16b, wsb=100) == WS
    assert mx(L, stats=A16, ws=A16b + 16, wsb=WSB) == ALIGN
    assert mx(L, stats=A16 + 4, ws=A16b, wsb=WSB) == ALIGN


def test_nvfp4_validation(L):
    assert nv(L, block=24, cols=48) == SHAPE
    assert nv(L, block=16, cols=40) == SHAPE
    assert nv(L, block=64, rot=64, cols=128) == SHAPE
    assert nv(L, block=16, rot=32) == SHAPE and "equal" in err(L)
    assert nv(L, fmt=0) == ARG and "scale_fmt" in err(L)
    assert nv(L, fmt=2, gmode=1, g=A16, ws=A16b, wsb=WSB) == ARG and "UE5M3" in err(L)
    assert nv(L, gmode=2, g=None) == ARG
    assert nv(L, gmode=1, g=A16) == WS
    assert nv(L, gmode=2, g=A16 + 2) == ALIGN
    assert nv(L, gmode=4, g=A16) == ARG and "ROW" in err(L)
    assert nv(L, gmode=3, g=None) == ARG
    assert nv(L, fmt=2, gmode=3, g=A16) == ARG and "UE5M3" in err(L)
    assert nv(L, gmode=3, g=A16, stats=A16b) == WS


def srch(L, x=A16, xt=0, rows=4, cols=64, fmt=1, block=16, gmode=0, g=None, rot=0, radius=1,
         codes=A16b, scales=A16c, bm=None, kind=0, stats=None, ws=None, wsb=0):
    return L.fp4_quantize_search(x, xt, rows, cols, fmt, block, gmode, g, rot, radius, codes,
                                 scales, bm, kind, stats, ws, wsb, None)


def test_search_validation(L):
    assert srch(L, radius=-1) == ARG and "radius" in err(L)
    assert srch(L, radius=9) == ARG and "radius" in err(L)
    assert srch(L, fmt=0, block=16) == SHAPE
    assert srch(L, fmt=0, block=32, gmode=2, g=A16) == ARG and "MXFP4" in err(L)
    assert srch(L, fmt=2, gmode=1, g=A16, ws=A16b, wsb=WSB) == ARG and "UE5M3" in err(L)
    assert srch(L, fmt=5) == ARG
    assert srch(L, x=None) == ARG
    assert srch(L, stats=A16) == WS
    assert srch(L, gmode=1, g=A16) == WS
    assert srch(L, rows=0, radius=3) == OK
    assert srch(L, gmode=3, g=A16) == ARG and "per-row" in err(L)


def test_gemm_validation(L):
    gm = lambda a, sa, b, sb, m, n, k, c, ct, ws=A16, wsb=1 << 20: L.fp4_gemm_mxfp4(
        a, sa, b, sb, m, n, k, c, ct, ws, wsb, None)
    assert gm(A16, A16b, A16c, A16, 4, 4, 48, A16b, 1) == SHAPE and "multiple of 32" in err(L)
    assert gm(A16, A16b, A16c, A16, 4, 4, -32, A16b, 1) == SHAPE
    assert gm(A16, A16b, A16c, A16, 4, 4, 1 << 24, A16b, 1) == SHAPE and "2^23" in err(L)
    assert gm(A16, A16b, A16c, A16, 4, 1 << 21, 64, A16b, 1) == SHAPE
    assert gm(A16, A16b, A16c, A16, 1 << 31, 4, 64, A16b, 1) == SHAPE
    assert gm(A16, A16b, A16c, A16, 4, 4, 64, None, 1) == ARG
    assert gm(None, A16b, A16c, A16, 4, 4, 64, A16b, 1) == ARG
    assert gm(A16 + 8, A16b, A16c, A16, 4, 4, 64, A16b, 1) == ALIGN
    assert gm(A16, A16b, A16c, A16, 4, 4, 64, A16b + 2, 1) == ALIGN
    assert gm(A16, A16b, A16c, A16, 4, 4, 64, A16b, 5) == ARG
    assert gm(A16, A16b, A16c, A16, 4, 4, 64, A16b, 1, ws=None) == WS and "workspace" in err(L)
    need = L.fp4_gemm_workspace_bytes(4, 4, 64)
    assert need == 256 * 2
    assert gm(A16, A16b, A16c, A16, 4, 4, 64, A16b, 1, wsb=need - 1) == WS
    assert gm(A16, A16b, A16c, A16, 4, 4, 64, A16b, 1, ws=A16 + 4, wsb=need) == ALIGN
    assert gm(A16, A16b, A16c, A16, 0, 4, 64, A16b, 1, ws=None, wsb=0) == OK


def test_gemm_nvfp4_validation(L):
    gn = lambda a, sa, b, sb, m, n, k, c, ct, ga=None, gb=None, ws=A16, wsb=1 << 20: L.fp4_gemm_nvfp4(
        a, sa, ga, b, sb, gb, m, n, k, c, ct, ws, wsb, None)
    assert gn(A16, A16b, A16c, A16, 4, 4, 96, A16b, 1) == SHAPE and "multiple of 64" in err(L)
    assert gn(A16, A16b, A16c, A16, 4, 4, -64, A16b, 1) == SHAPE
    assert gn(A16, A16b, A16c, A16, 4, 4, 1 << 24, A16b, 1) == SHAPE and "2^23" in err(L)
    assert gn(A16, A16b, A16c, A16, 4, 1 << 21, 64, A16b, 1) == SHAPE
    assert gn(A16, A16b, A16c, A16, 4, 4, 64, None, 1) == ARG
    assert gn(A16, None, A16c, A16, 4, 4, 64, A16b, 1) == ARG
    assert gn(A16 + 8, A16b, A16c, A16, 4, 4, 64, A16b, 1) == ALIGN
    assert gn(A16, A16b + 2, A16c, A16, 4, 4, 64, A16b, 1) == ALIGN and "4-byte" in err(L)
    assert gn(A16, A16b, A16c, A16, 4, 4, 64, A16b, 1, ga=A16 + 2) == ALIGN
    assert gn(A16, A16b, A16c, A16, 4, 4, 64, A16b, 7) == ARG
    assert gn(A16, A16b, A16c, A16, 0, 4, 64, A16b, 1, ws=None, wsb=0) == OK
    # Products with enough tiles need no workspace; few tiles split K.
    assert L.fp4_gemm_nvfp4_workspace_bytes(8192, 18944, 3584) == 0
    wb = L.fp4_gemm_nvfp4_workspace_bytes(16, 3584, 18944)
    assert wb > 0 and wb % (16 * 3584 * 4) == 0 and 2 <= wb // (16 * 3584 * 4) <= 18944 // 256
    assert L.fp4_gemm_nvfp4_workspace_bytes(0, 5, 64) == 0


def test_gemm_workspace_bytes(L):
    """Packed scales: 256 B per 32-row fragment of A and B per 256-wide K stage,
    padded to 256 B; then, when K is split into ranges, one binary32 M x N
    partial product per range (at most one range per stage)."""
    wb = L.fp4_gemm_workspace_bytes
    assert wb(0, 5, 64) == 0 and wb(5, 5, 0) == 0
    assert wb(1, 1, 32) == 2 * 256
    assert wb(8192, 18944, 3584) == (256 + 592) * 14 * 256   # enough tiles: no split
    for m, n, k in [(33, 64, 257 * 32), (1, 18944, 3584), (16, 3584, 18944), (300, 517, 384),
                    (256, 18944, 3584), (1024, 18944, 3584)]:
        stages = -(-k // 256)
        packed = -(-((-(-m // 32) + -(-n // 32)) * stages * 256) // 256) * 256
        extra = wb(m, n, k) - packed
        assert extra >= 0 and extra % (m * n * 4) == 0, (m, n, k)
        splits = extra // (m * n * 4)
        assert splits == 0 or 2 <= splits <= stages, (m, n, k, splits)
    # Decode-sized products split K; a full-chip one does not.
    assert wb(1, 18944, 3584) > (1 + 592) * 14 * 256
    assert wb(1024, 18944, 3584) == (32 + 592) * 14 * 256


def test_other_entry_points_validation(L):
    deq = L.fp4_dequantize
    assert deq(A16, A16b, 0, 16, None, 4, 64, 0, A16c, 1, None) == SHAPE  # MXFP4 needs block 32
    assert deq(A16, A16b, 3, 16, None, 4, 64, 0, A16c, 1, None) == ARG
    assert deq(A16, A16b, 1, 16, None, 4, 64, 0, A16c, 9, None) == ARG
    assert deq(A16, A16b, 1, 16, None, 4, 64, 0, None, 1, None) == ARG
    assert deq(A16 + 1, A16b, 1, 16, None, 4, 64, 0, A16c, 1, None) == ALIGN
    mse = L.fp4_block_mse
    assert mse(A16, 0, A16b, A16c, 1, 16, None, 4, 64, 0, None, 2, None, None, 0, None) == ARG
    assert mse(A16, 0, A16b, A16c, 1, 16, None, 4, 64, 0, None, 0, A16, None, 0, None) == WS
    rot = L.hadamard_block_rotate
    assert rot(A16, 0, 4, 64, 8, A16b, None) == SHAPE
    assert rot(A16, 0, 4, 40, 16, A16b, None) == SHAPE
    assert rot(A16, 0, 4, 64, 16, A16b + 4, None) == ALIGN


def test_empty_tensor_without_outputs_is_a_noop(L):
    assert mx(L, rows=0, x=None, codes=None, scales=None) == OK
    assert err(L) == ""
    assert nv(L, rows=3, cols=0, x=None, codes=None, scales=None) == OK


def test_last_error_is_thread_local(L):
    assert mx(L, xt=9) == ARG
    main_msg = err(L)
    seen = {}

    def worker():
        seen["before"] = L.fp4q_last_error().decode()
        seen["rc"] = mx(L, cols=48)
        seen["after"] = L.fp4q_last_error().decode()

    t = threading.Thread(target=worker)
    t.start()
    t.join()
    assert seen["before"] == "" and seen["rc"] == SHAPE and "multiple" in seen["after"]
    assert err(L) == main_msg


def test_product_path_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "microscaling_fp4_quantization_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f


def test_missing_library_raises(tmp_path, monkeypatch):
    monkeypatch.setattr(fq, "LIB_PATH", str(tmp_path / "absent.so"))
    monkeypatch.setattr(fq, "_lib", None)
    with pytest.raises(fq.Fp4qError):
        fq.lib()


def test_profile_events_validation(L):
    assert L.fp4q_profile_events(None, -1) == ARG and "negative" in err(L)
    assert L.fp4q_profile_events(None, 0) == OK
    assert L.fp4q_profile_count() == 0
    # Recording on, but an argument error launches nothing, so nothing is recorded.
    handles = (ctypes.c_void_p * 2)(A16, A16b)
    assert L.fp4q_profile_events(handles, 1) == OK
    assert mx(L, x=None) == ARG
    assert L.fp4q_profile_count() == 0
    assert L.fp4q_profile_events(None, 0) == OK


def test_noalloc_validation(L):
    """Argument errors come back before the scratch is looked up (no GPU touched)."""
    def nva(x=A16, fmt=1, gmode=0, g=None, block=16, cols=64, kind=0, stats=None):
        return L.nvfp4_quantize_noalloc(x, 0, 4, cols, block, fmt, gmode, g, 0, A16b, A16c, None,
                                        kind, stats, None)
    assert nva(x=None) == ARG
    assert nva(fmt=0) == ARG and "scale_fmt" in err(L)
    assert nva(cols=40) == SHAPE
    assert nva(gmode=2) == ARG and "g pointer" in err(L)
    assert nva(kind=3) == ARG
    assert nva(stats=A16 + 4) == ALIGN


def test_mx_nv_validation(L):
    """fp4_quantize_mx_nv checks both passes' arguments before launching anything."""
    def pair(x=A16, xt=0, rows=4, cols=64, mxc=A16b, mxs=A16c, block=16, g=A16, nvc=A16b,
             nvs=A16c, kind=0, mst=None, nst=None, ws=A16, wsb=WSB):
        return L.fp4_quantize_mx_nv(x, xt, rows, cols, mxc, mxs, None, mst, block, g, nvc, nvs,
                                    None, nst, kind, ws, wsb, None)
    assert pair(xt=5) == ARG
    assert pair(cols=48) == SHAPE                       # not a multiple of 32 (MXFP4)
    assert pair(block=12) == SHAPE
    assert pair(cols=96, block=64) == SHAPE             # 96 % 64
    assert pair(g=None) == ARG and "g pointer" in err(L)  # the dynamic scale needs g
    assert pair(ws=None) == WS                          # always needs a workspace
    assert pair(wsb=16) == WS
    assert pair(kind=2) == ARG
    assert pair(nvc=None) == ARG
    assert pair(mxc=A16b + 8) == ALIGN
    assert pair(mst=A16 + 4) == ALIGN


def test_mx_nv_batch_validation(L):
    """fp4_quantize_mx_nv_batch validates every tensor (naming it) before launching."""
    def t(cols=64, bm=None, x=A16):
        return fq.MxNvTensor(x, 4, cols, A16b, A16c, bm, None, A16, A16b, A16c, bm, None)

    def batch(ts, n=None, block=16, ws=A16, kind=0):
        arr = (fq.MxNvTensor * max(1, len(ts)))(*ts)
        return L.fp4_quantize_mx_nv_batch(arr, len(ts) if n is None else n, 0, block, kind, ws, WSB, None)
    assert batch([t()], n=0) == ARG
    assert batch([t()] * 17) == ARG and "n_tensors" in err(L)
    assert L.fp4_quantize_mx_nv_batch(None, 1, 0, 16, 0, A16, WSB, None) == ARG
    assert batch([t()], block=8) == SHAPE
    assert batch([t(), t(cols=48)]) == SHAPE and "tensor 1" in err(L)
    assert batch([t(), t(bm=A16)]) == ARG and "every tensor" in err(L)
    assert batch([t()], ws=None) == WS
    assert batch([t(x=A16 + 8)]) == ALIGN
