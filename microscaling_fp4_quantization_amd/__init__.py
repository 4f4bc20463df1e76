"""Python binding of libfp4q.so, the gfx950 microscaling FP4 quantization library.

The functions here carry the C ABI's names (include/fp4q.h) and only marshal
arguments: they check tensor shapes, allocate outputs with torch when the caller
does not pass them, and hand device pointers and torch's current HIP stream to
the library.  Every step of the computation runs in the library's kernels.
There is no fallback: if libfp4q.so is missing, importing the functions works but
every call raises.

Layouts (row-major, blocks of b consecutive elements along a row):
  codes      uint8 rows x cols/2; byte j holds element 2j (low nibble) and 2j+1
  scales     uint8 rows x cols/b; E8M0 (MXFP4) or UE4M3/UE5M3 bytes
  block_mse  float32 rows x cols/b
  stats      float64[6] device tensor laid out as the C struct fp4q_stats
             (sse_nonmax, sse_max, sse_zero, sum_x2, then two int64 counts);
             read it with stats_dict().
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfp4q.so")

BF16, F32 = 0, 1
FMT_MXFP4, FMT_UE4M3, FMT_UE5M3 = 0, 1, 2
G_NONE, G_DYNAMIC, G_GIVEN, G_ROW = 0, 1, 2, 3
MSE_ABS, MSE_REL = 0, 1
STATUS = {0: "OK", 1: "ERR_ARG", 2: "ERR_SHAPE", 3: "ERR_ALIGN", 4: "ERR_WORKSPACE", 5: "ERR_HIP"}

EXPORTS = ("mxfp4_quantize", "nvfp4_quantize", "nvfp4_quantize_noalloc", "fp4_quantize_mx_nv",
           "fp4_quantize_mx_nv_batch", "fp4_quantize_search",
           "fp4_dequantize",
           "fp4_block_mse", "hadamard_block_rotate", "fp4_gemm_mxfp4", "fp4_gemm_workspace_bytes",
           "fp4_gemm_nvfp4", "fp4_gemm_nvfp4_workspace_bytes",
           "fp4q_workspace_bytes",
           "fp4q_last_error", "fp4q_abi_version", "fp4q_profile_events", "fp4q_profile_count")


class Fp4qError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib():
    """The loaded libfp4q.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise Fp4qError(5, f"{LIB_PATH} is missing; build it with "
                               "`python -m microscaling_fp4_quantization_amd.build`")
        _lib = _bind(ctypes.CDLL(LIB_PATH))
    return _lib


def _bind(l):
    c = ctypes
    P, i32, i64, sz = c.c_void_p, c.c_int32, c.c_int64, c.c_size_t
    l.mxfp4_quantize.argtypes = [P, i32, i64, i64, i32, P, P, P, i32, P, P, sz, P]
    l.nvfp4_quantize.argtypes = [P, i32, i64, i64, i32, i32, i32, P, i32, P, P, P, i32, P, P, sz, P]
    l.nvfp4_quantize_noalloc.argtypes = [P, i32, i64, i64, i32, i32, i32, P, i32, P, P, P, i32, P, P]
    l.nvfp4_quantize_noalloc.restype = c.c_int
    l.fp4_quantize_mx_nv.argtypes = [P, i32, i64, i64, P, P, P, P, i32, P, P, P, P, P, i32, P, sz, P]
    l.fp4_quantize_mx_nv.restype = c.c_int
    l.fp4_quantize_mx_nv_batch.argtypes = [P, i32, i32, i32, i32, P, sz, P]
    l.fp4_quantize_mx_nv_batch.restype = c.c_int
    l.fp4_dequantize.argtypes = [P, P, i32, i32, P, i64, i64, i32, P, i32, P]
    l.fp4_quantize_search.argtypes = [P, i32, i64, i64, i32, i32, i32, P, i32, i32, P, P, P, i32,
                                      P, P, sz, P]
    l.fp4_gemm_mxfp4.argtypes = [P, P, P, P, i64, i64, i64, P, i32, P, sz, P]
    l.fp4_gemm_workspace_bytes.argtypes = [i64, i64, i64]
    l.fp4_gemm_workspace_bytes.restype = sz
    l.fp4_gemm_nvfp4.argtypes = [P, P, P, P, P, P, i64, i64, i64, P, i32, P, sz, P]
    l.fp4_gemm_nvfp4_workspace_bytes.argtypes = [i64, i64, i64]
    l.fp4_gemm_nvfp4_workspace_bytes.restype = sz
    l.fp4_block_mse.argtypes = [P, i32, P, P, i32, i32, P, i64, i64, i32, P, i32, P, P, sz, P]
    l.hadamard_block_rotate.argtypes = [P, i32, i64, i64, i32, P, P]
    for name in ("mxfp4_quantize", "nvfp4_quantize", "fp4_dequantize", "fp4_block_mse",
                 "hadamard_block_rotate"):
        getattr(l, name).restype = c.c_int
    l.fp4q_workspace_bytes.argtypes = [i64, i64, i32]
    l.fp4q_workspace_bytes.restype = sz
    l.fp4q_last_error.argtypes = []
    l.fp4q_last_error.restype = c.c_char_p
    l.fp4q_abi_version.argtypes = []
    l.fp4q_abi_version.restype = c.c_int32
    l.fp4q_profile_events.argtypes = [P, i32]
    l.fp4q_profile_events.restype = c.c_int
    l.fp4q_profile_count.argtypes = []
    l.fp4q_profile_count.restype = c.c_int32
    return l


def _check(rc: int):
    if rc != 0:
        raise Fp4qError(rc, lib().fp4q_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16 or float32")


def _matrix(x: torch.Tensor, what: str = "x") -> torch.Tensor:
    if x.dim() != 2:
        raise ValueError(f"{what} must be 2-D (rows x cols)")
    if not x.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if not x.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    return x


_workspaces = {}


def workspace_bytes(rows: int = 0, cols: int = 0, block: int = 32) -> int:
    return int(lib().fp4q_workspace_bytes(rows, cols, block))


def workspace(device) -> torch.Tensor:
    """A zero-filled workspace for `device` and torch's current stream on it.
    Calls made on one stream share it (stream order keeps them apart); calls
    made on another stream get a workspace of their own."""
    dev = torch.device(device)
    key = (dev.index, torch.cuda.current_stream(dev).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None:
        ws = torch.zeros(workspace_bytes(), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def new_stats(device) -> torch.Tensor:
    return torch.zeros(6, dtype=torch.float64, device=device)


def stats_dict(stats: torch.Tensor) -> dict:
    """Copy an fp4q_stats tensor to the host (synchronises)."""
    h = stats.detach().cpu()
    f = h[:4].tolist()
    i = h.view(torch.int64)[4:6].tolist()
    return {"sse_nonmax": f[0], "sse_max": f[1], "sse_zero": f[2], "sum_x2": f[3],
            "n_blocks": i[0], "n_zero_blocks": i[1]}


@dataclass
class Quantized:
    codes: torch.Tensor
    scales: torch.Tensor
    block_mse: Optional[torch.Tensor]
    stats: Optional[torch.Tensor]
    g: Optional[torch.Tensor]


def _outputs(x, block, codes, scales, block_mse, stats):
    rows, cols = x.shape
    dev = x.device
    if codes is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((rows, cols // block), dtype=torch.uint8, device=dev)
    if block_mse is True:
        block_mse = torch.empty((rows, cols // block), dtype=torch.float32, device=dev)
    elif block_mse is False:
        block_mse = None
    if stats is True:
        stats = new_stats(dev)
    elif stats is False:
        stats = None
    return codes, scales, block_mse, stats


def mxfp4_quantize(x: torch.Tensor, rotate: int = 0, *, codes=None, scales=None,
                   block_mse=True, mse_kind: int = MSE_ABS, stats=True,
                   ws: Optional[torch.Tensor] = None) -> Quantized:
    """MXFP4 (block 32, E8M0) quantize + pack + dequantize + error split.

    ``block_mse`` / ``stats``: True to allocate, False to skip, or a tensor to fill.
    """
    x = _matrix(x)
    codes, scales, block_mse, stats = _outputs(x, 32, codes, scales, block_mse, stats)
    ws = ws if ws is not None else (workspace(x.device) if stats is not None else None)
    _check(lib().mxfp4_quantize(_ptr(x), _dtype_code(x), x.shape[0], x.shape[1], rotate,
                                _ptr(codes), _ptr(scales), _ptr(block_mse), mse_kind,
                                _ptr(stats), _ptr(ws), 0 if ws is None else ws.numel(),
                                _stream(x.device)))
    return Quantized(codes, scales, block_mse, stats, None)


def nvfp4_quantize(x: torch.Tensor, block: int = 16, scale_fmt: int = FMT_UE4M3,
                   gmode: int = G_DYNAMIC, g: Optional[torch.Tensor] = None, rotate: int = 0, *,
                   codes=None, scales=None, block_mse=True, mse_kind: int = MSE_ABS, stats=True,
                   ws: Optional[torch.Tensor] = None) -> Quantized:
    """UE4M3/UE5M3 block quantize (NVFP4 at block 16) + pack + dequantize + error split.

    ``g``: one-element float32 device tensor; written in the dynamic mode (allocated
    when not given), read in the given mode.  With ``G_ROW`` it holds one scale per
    row (allocated with ``rows`` elements when not given) and is written.
    """
    x = _matrix(x)
    codes, scales, block_mse, stats = _outputs(x, block, codes, scales, block_mse, stats)
    if gmode != G_NONE and g is None:
        g = torch.empty(x.shape[0] if gmode == G_ROW else 1, dtype=torch.float32, device=x.device)
    need_ws = stats is not None or gmode == G_DYNAMIC
    ws = ws if ws is not None else (workspace(x.device) if need_ws else None)
    _check(lib().nvfp4_quantize(_ptr(x), _dtype_code(x), x.shape[0], x.shape[1], block,
                                scale_fmt, gmode, _ptr(g), rotate, _ptr(codes), _ptr(scales),
                                _ptr(block_mse), mse_kind, _ptr(stats), _ptr(ws),
                                0 if ws is None else ws.numel(), _stream(x.device)))
    return Quantized(codes, scales, block_mse, stats, g)


def nvfp4_quantize_noalloc(x: torch.Tensor, block: int = 16, scale_fmt: int = FMT_UE4M3,
                           gmode: int = G_DYNAMIC, g: Optional[torch.Tensor] = None,
                           rotate: int = 0, *, codes=None, scales=None, block_mse=True,
                           mse_kind: int = MSE_ABS, stats=True) -> Quantized:
    """nvfp4_quantize on the library's static device scratch (no workspace).
    The library allocates nothing; pass preallocated outputs (``codes``,
    ``scales``, ``block_mse``, ``stats``, ``g``) to allocate nothing here either."""
    x = _matrix(x)
    codes, scales, block_mse, stats = _outputs(x, block, codes, scales, block_mse, stats)
    if gmode != G_NONE and g is None:
        g = torch.empty(x.shape[0] if gmode == G_ROW else 1, dtype=torch.float32, device=x.device)
    _check(lib().nvfp4_quantize_noalloc(_ptr(x), _dtype_code(x), x.shape[0], x.shape[1], block,
                                        scale_fmt, gmode, _ptr(g), rotate, _ptr(codes), _ptr(scales),
                                        _ptr(block_mse), mse_kind, _ptr(stats), _stream(x.device)))
    return Quantized(codes, scales, block_mse, stats, g)


def fp4_quantize_mx_nv(x: torch.Tensor, nv_block: int = 16, *, mse_kind: int = MSE_ABS,
                       block_mse=True, stats=True, mx=None, nv=None, g=None,
                       ws: Optional[torch.Tensor] = None):
    """MXFP4 and dynamic NVFP4 (UE4M3 scales) of one unrotated tensor in one call;
    the NVFP4 per-tensor scale comes from the MXFP4 pass (no separate amax pass).

    ``mx`` / ``nv``: optional dicts of preallocated outputs (keys ``codes``,
    ``scales``, ``block_mse``, ``stats``).  Returns (Quantized MXFP4, Quantized
    NVFP4); the NVFP4 one carries ``g``."""
    x = _matrix(x)
    mx, nv = dict(mx or {}), dict(nv or {})
    m = _outputs(x, 32, mx.get("codes"), mx.get("scales"), mx.get("block_mse", block_mse),
                 mx.get("stats", stats))
    v = _outputs(x, nv_block, nv.get("codes"), nv.get("scales"), nv.get("block_mse", block_mse),
                 nv.get("stats", stats))
    if g is None:
        g = torch.empty(1, dtype=torch.float32, device=x.device)
    ws = ws if ws is not None else workspace(x.device)
    _check(lib().fp4_quantize_mx_nv(_ptr(x), _dtype_code(x), x.shape[0], x.shape[1],
                                    _ptr(m[0]), _ptr(m[1]), _ptr(m[2]), _ptr(m[3]), nv_block, _ptr(g),
                                    _ptr(v[0]), _ptr(v[1]), _ptr(v[2]), _ptr(v[3]), mse_kind,
                                    _ptr(ws), ws.numel(), _stream(x.device)))
    return Quantized(*m, None), Quantized(*v, g)


class MxNvTensor(ctypes.Structure):
    """fp4q_mx_nv_tensor: one tensor of a batched fp4_quantize_mx_nv call."""
    _fields_ = [("x", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("mx_codes", ctypes.c_void_p), ("mx_scales", ctypes.c_void_p),
                ("mx_block_mse", ctypes.c_void_p), ("mx_stats", ctypes.c_void_p),
                ("g", ctypes.c_void_p), ("nv_codes", ctypes.c_void_p), ("nv_scales", ctypes.c_void_p),
                ("nv_block_mse", ctypes.c_void_p), ("nv_stats", ctypes.c_void_p)]


MAX_BATCH = 16


def fp4_quantize_mx_nv_batch(xs, nv_block: int = 16, *, mse_kind: int = MSE_ABS, block_mse=True,
                             stats=True, outs=None, ws: Optional[torch.Tensor] = None):
    """fp4_quantize_mx_nv for up to MAX_BATCH tensors (same dtype, same device) in
    one launch per pass.  ``outs``: optional list of (mx dict, nv dict, g) of
    preallocated outputs per tensor.  Returns a list of (Quantized MXFP4,
    Quantized NVFP4 with g) per tensor."""
    xs = [_matrix(x) for x in xs]
    if not xs:
        raise ValueError("xs is empty")
    if any(x.dtype != xs[0].dtype or x.device != xs[0].device for x in xs):
        raise ValueError("every tensor of a batch must have the same dtype and device")
    res = []
    arr = (MxNvTensor * len(xs))()
    for i, x in enumerate(xs):
        mx, nv, g = outs[i] if outs is not None else ({}, {}, None)
        m = _outputs(x, 32, mx.get("codes"), mx.get("scales"), mx.get("block_mse", block_mse),
                     mx.get("stats", stats))
        v = _outputs(x, nv_block, nv.get("codes"), nv.get("scales"), nv.get("block_mse", block_mse),
                     nv.get("stats", stats))
        if g is None:
            g = torch.empty(1, dtype=torch.float32, device=x.device)
        ptr = lambda t: None if t is None else t.data_ptr()
        arr[i] = MxNvTensor(ptr(x), x.shape[0], x.shape[1], ptr(m[0]), ptr(m[1]), ptr(m[2]), ptr(m[3]),
                            ptr(g), ptr(v[0]), ptr(v[1]), ptr(v[2]), ptr(v[3]))
        res.append((Quantized(*m, None), Quantized(*v, g)))
    ws = ws if ws is not None else workspace(xs[0].device)
    _check(lib().fp4_quantize_mx_nv_batch(arr, len(xs), _dtype_code(xs[0]), nv_block, mse_kind,
                                          _ptr(ws), ws.numel(), _stream(xs[0].device)))
    return res


def fp4_quantize_search(x: torch.Tensor, fmt: int = FMT_UE4M3, block: int = 16,
                        gmode: int = G_DYNAMIC, g: Optional[torch.Tensor] = None, rotate: int = 0,
                        radius: int = 1, *, codes=None, scales=None, block_mse=True,
                        mse_kind: int = MSE_ABS, stats=True,
                        ws: Optional[torch.Tensor] = None) -> Quantized:
    """Block quantize with the per-block scale search (the max-based scale code and
    its neighbours within ``radius``, lowest block SSE) + pack + error split.
    ``fmt`` is FMT_MXFP4 (block 32, gmode G_NONE), FMT_UE4M3 or FMT_UE5M3."""
    x = _matrix(x)
    codes, scales, block_mse, stats = _outputs(x, block, codes, scales, block_mse, stats)
    if gmode != G_NONE and g is None:
        g = torch.empty(1, dtype=torch.float32, device=x.device)
    need_ws = stats is not None or gmode == G_DYNAMIC
    ws = ws if ws is not None else (workspace(x.device) if need_ws else None)
    _check(lib().fp4_quantize_search(_ptr(x), _dtype_code(x), x.shape[0], x.shape[1], fmt, block,
                                     gmode, _ptr(g), rotate, radius, _ptr(codes), _ptr(scales),
                                     _ptr(block_mse), mse_kind, _ptr(stats), _ptr(ws),
                                     0 if ws is None else ws.numel(), _stream(x.device)))
    return Quantized(codes, scales, block_mse, stats, g)


_gemm_workspaces = {}


def gemm_workspace(device, nbytes: int) -> torch.Tensor:
    """A device workspace of at least `nbytes` for the GEMMs, kept per device
    and current stream and grown on demand (calls on one stream are ordered, so
    they can share it)."""
    dev = torch.device(device)
    key = (dev.index, torch.cuda.current_stream(dev).cuda_stream)
    ws = _gemm_workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _gemm_workspaces[key] = ws
    return ws


def fp4_gemm_mxfp4(a_codes: torch.Tensor, a_scales: torch.Tensor, b_codes: torch.Tensor,
                   b_scales: torch.Tensor, out_dtype=torch.float32,
                   out: Optional[torch.Tensor] = None,
                   ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = A_hat @ B_hat.T for MXFP4 operands as mxfp4_quantize writes them:
    codes (rows x K/2 uint8) and E8M0 scales (rows x K/32 uint8)."""
    a_codes, a_scales = _matrix(a_codes, "a_codes"), _matrix(a_scales, "a_scales")
    b_codes, b_scales = _matrix(b_codes, "b_codes"), _matrix(b_scales, "b_scales")
    m, k = a_codes.shape[0], a_codes.shape[1] * 2
    n = b_codes.shape[0]
    if b_codes.shape[1] * 2 != k or a_scales.shape != (m, k // 32) or b_scales.shape != (n, k // 32):
        raise ValueError("operand shapes do not match: codes rows x K/2, scales rows x K/32")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=a_codes.device)
    need = int(lib().fp4_gemm_workspace_bytes(m, n, k))
    if ws is None and need:
        ws = gemm_workspace(a_codes.device, need)
    _check(lib().fp4_gemm_mxfp4(_ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), m, n,
                                k, _ptr(out), _dtype_code(out), _ptr(ws),
                                0 if ws is None else ws.numel(), _stream(a_codes.device)))
    return out


def fp4_gemm_nvfp4(a_codes: torch.Tensor, a_scales: torch.Tensor, a_g: Optional[torch.Tensor],
                   b_codes: torch.Tensor, b_scales: torch.Tensor, b_g: Optional[torch.Tensor],
                   out_dtype=torch.float32, out: Optional[torch.Tensor] = None,
                   ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = A_hat @ B_hat.T for NVFP4 operands as nvfp4_quantize writes them with
    block 16 and UE4M3 scales: codes (rows x K/2 uint8), scale bytes (rows x
    K/16 uint8) and the per-tensor scale (a 1-element float32 device tensor, or
    None for 1)."""
    a_codes, a_scales = _matrix(a_codes, "a_codes"), _matrix(a_scales, "a_scales")
    b_codes, b_scales = _matrix(b_codes, "b_codes"), _matrix(b_scales, "b_scales")
    m, k = a_codes.shape[0], a_codes.shape[1] * 2
    n = b_codes.shape[0]
    if b_codes.shape[1] * 2 != k or a_scales.shape != (m, k // 16) or b_scales.shape != (n, k // 16):
        raise ValueError("operand shapes do not match: codes rows x K/2, scales rows x K/16")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=a_codes.device)
    need = int(lib().fp4_gemm_nvfp4_workspace_bytes(m, n, k))
    if ws is None and need:
        ws = gemm_workspace(a_codes.device, need)
    _check(lib().fp4_gemm_nvfp4(_ptr(a_codes), _ptr(a_scales), _ptr(a_g), _ptr(b_codes),
                                _ptr(b_scales), _ptr(b_g), m, n, k, _ptr(out), _dtype_code(out),
                                _ptr(ws), 0 if ws is None else ws.numel(),
                                _stream(a_codes.device)))
    return out


def fp4_dequantize(codes: torch.Tensor, scales: torch.Tensor, fmt: int, block: int,
                   g: Optional[torch.Tensor] = None, rotate: int = 0,
                   out_dtype=torch.float32, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x_hat from codes and scale bytes (fmt FMT_MXFP4, FMT_UE4M3 or FMT_UE5M3;
    ``g`` the one-element per-tensor scale of UE4M3 codes, None for 1, ignored
    for the other formats), back in the original domain when ``rotate`` is the
    block size the codes were rotated with; float32 or bf16 (round to nearest
    even)."""
    codes = _matrix(codes, "codes")
    rows, cols = codes.shape[0], codes.shape[1] * 2
    if out is None:
        out = torch.empty((rows, cols), dtype=out_dtype, device=codes.device)
    _check(lib().fp4_dequantize(_ptr(codes), _ptr(scales), fmt, block, _ptr(g), rows, cols,
                                rotate, _ptr(out), _dtype_code(out), _stream(codes.device)))
    return out


def fp4_block_mse(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, fmt: int,
                  block: int, g: Optional[torch.Tensor] = None, rotate: int = 0, *,
                  block_mse=True, mse_kind: int = MSE_ABS, stats=True,
                  ws: Optional[torch.Tensor] = None):
    """Error split of stored codes against x; returns (block_mse, stats)."""
    x = _matrix(x)
    _, _, block_mse, stats = _outputs(x, block, codes, scales, block_mse, stats)
    ws = ws if ws is not None else (workspace(x.device) if stats is not None else None)
    _check(lib().fp4_block_mse(_ptr(x), _dtype_code(x), _ptr(codes), _ptr(scales), fmt, block,
                               _ptr(g), x.shape[0], x.shape[1], rotate, _ptr(block_mse),
                               mse_kind, _ptr(stats), _ptr(ws), 0 if ws is None else ws.numel(),
                               _stream(x.device)))
    return block_mse, stats


def hadamard_block_rotate(x: torch.Tensor, n: int, out: Optional[torch.Tensor] = None):
    """Each run of ``n`` (16 or 32) consecutive elements of a row times the
    normalized Sylvester Hadamard matrix, in float32 (its own inverse)."""
    x = _matrix(x)
    if out is None:
        out = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    _check(lib().hadamard_block_rotate(_ptr(x), _dtype_code(x), x.shape[0], x.shape[1], n,
                                       _ptr(out), _stream(x.device)))
    return out


_HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hip_runtime_api.h


def _hip_runtime():
    """The HIP runtime torch has loaded (for fence-free timing events)."""
    global _HIP
    if _HIP is None:
        h = ctypes.CDLL("libamdhip64.so")
        h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _HIP = h
    return _HIP


_HIP = None


class LaunchTimer:
    """Times the library's kernel launches with HIP events (fp4q_profile_events).

    Inside ``with LaunchTimer(n) as t:``, each kernel the library launches from
    this thread (up to ``n``) is bracketed by a pair of events on its stream;
    afterwards ``t.durations_us()`` (which synchronises) gives their durations
    in launch order.  A quantize call launches the amax pass (dynamic scale
    only), the quantize kernel and the stats reduction (stats only).

    The events are created without the system-scope fence a default HIP event
    performs when it is recorded (hipEventDisableSystemFence): that fence
    writes back and invalidates the caches after every kernel, which adds
    several microseconds to each timed launch and to the next one's start."""

    def __init__(self, n: int, device=None):
        dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        hip = _hip_runtime()
        with torch.cuda.device(dev):
            evs = []
            for _ in range(2 * n):
                e = ctypes.c_void_p()
                rc = hip.hipEventCreateWithFlags(ctypes.byref(e), _HIP_EVENT_DISABLE_SYSTEM_FENCE)
                if rc != 0:
                    for x in evs:
                        hip.hipEventDestroy(x)
                    raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
                evs.append(e.value)
        self._handles = (ctypes.c_void_p * (2 * n))(*evs)
        self.n = n
        self.count = 0

    def __enter__(self):
        _check(lib().fp4q_profile_events(self._handles, self.n))
        return self

    def __exit__(self, *exc):
        self.count = int(lib().fp4q_profile_count())
        lib().fp4q_profile_events(None, 0)
        return False

    def durations_us(self):
        torch.cuda.synchronize(self.device)
        hip = _hip_runtime()
        out, ms = [], ctypes.c_float()
        for i in range(self.count):
            rc = hip.hipEventElapsedTime(ctypes.byref(ms), self._handles[2 * i], self._handles[2 * i + 1])
            if rc != 0:
                raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
            out.append(ms.value * 1e3)
        return out

    def __del__(self):
        hip = _HIP
        if hip is not None and getattr(self, "_handles", None) is not None:
            for h in self._handles:
                if h:
                    hip.hipEventDestroy(h)
