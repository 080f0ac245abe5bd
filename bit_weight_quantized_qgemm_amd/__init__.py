"""Thin Python binding of the gfx950 quantized-weight GEMM library (libqgemm.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of ``include/qgemm.h``. PyTorch provides device memory
and the current HIP stream. Importing this package does not need a GPU; calling
anything that launches work needs an MI355X (gfx950) and the built library,
and raises if either is missing -- there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "FMT_W4A16", "FMT_W4A8", "FMT_W2W4", "QgemmError", "lib", "lib_path", "packed_bytes",
    "workspace_bytes", "plan", "set_plan_override", "repack", "repack_w4a16", "repack_w4a8",
    "repack_w2w4", "w4a16", "w4a8", "w2w4_mixed", "Workspace", "EXPORTED_SYMBOLS", "quantize_a8",
    "w4a8_fp16", "FMT_W4G", "DT_F16", "DT_BF16", "packed_bytes_w4g", "workspace_bytes_w4g",
    "repack_w4g", "w4g", "FMT_W4A16_SP24", "repack_sp24", "w4a16_sp24", "FMT_BITPLANE",
    "packed_bytes_bitplane", "workspace_bytes_bitplane", "repack_bitplane", "bitplane_a8", "plan_info",
    "w4a16_noalloc",
]

FMT_W4A16 = 1
FMT_W4A8 = 2
FMT_W2W4 = 3
FMT_W4G = 4
FMT_W4A16_SP24 = 5
FMT_BITPLANE = 6
DT_F16 = 1
DT_BF16 = 2

_HERE = os.path.dirname(os.path.abspath(__file__))
# QGEMM_LIB selects another build of the same library (the host-sanitized
# build of the CPU test tier); by default the in-tree libqgemm.so
_LIB_PATH = os.environ.get("QGEMM_LIB") or os.path.join(_HERE, "libqgemm.so")
_lib = None

EXPORTED_SYMBOLS = (
    "qgemm_status_str", "qgemm_last_error", "qgemm_version", "qgemm_packed_bytes",
    "qgemm_workspace_bytes", "qgemm_repack", "qgemm_w4a16", "qgemm_w4a8", "qgemm_w2w4_mixed",
    "qgemm_plan", "qgemm_set_plan_override", "qgemm_quantize_a8", "qgemm_w4g_packed_bytes",
    "qgemm_w4g_workspace_bytes", "qgemm_w4g_repack", "qgemm_w4g", "qgemm_w4a16_sp24",
    "qgemm_bitplane_packed_bytes", "qgemm_bitplane_workspace_bytes", "qgemm_bitplane_repack",
    "qgemm_bitplane_a8", "qgemm_bitplane_plan", "qgemm_w4g_plan", "qgemm_plan_info", "qgemm_w4a16_noalloc",
)


class QgemmError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        super().__init__(f"{where}: {_status_name(status)} ({status}){': ' + detail if detail else ''}")


def lib_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load libqgemm.so (built in-tree by ``build.py``); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: run `python -m bit_weight_quantized_qgemm_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        i64, u64p, vp = ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t), ctypes.c_void_p
        L.qgemm_status_str.restype = ctypes.c_char_p
        L.qgemm_status_str.argtypes = [ctypes.c_int]
        L.qgemm_last_error.restype = ctypes.c_char_p
        L.qgemm_last_error.argtypes = []
        L.qgemm_version.restype = ctypes.c_int
        L.qgemm_packed_bytes.argtypes = [ctypes.c_int, i64, i64, vp, u64p]
        L.qgemm_workspace_bytes.argtypes = [ctypes.c_int, i64, i64, i64, u64p]
        L.qgemm_repack.argtypes = [ctypes.c_int, i64, i64, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.qgemm_w4a16.argtypes = [vp, i64, vp, vp, i64, i64, i64, i64, vp, ctypes.c_size_t, vp]
        L.qgemm_w4a8.argtypes = [vp, i64, vp, vp, vp, i64, vp, i64, i64, i64, vp, ctypes.c_size_t, vp]
        L.qgemm_w2w4_mixed.argtypes = [vp, i64, vp, vp, i64, i64, i64, i64, vp, ctypes.c_size_t, vp]
        L.qgemm_w4a16_sp24.argtypes = [vp, i64, vp, vp, i64, i64, i64, i64, vp, ctypes.c_size_t, vp]
        L.qgemm_plan.argtypes = [ctypes.c_int, i64, i64, i64, ctypes.POINTER(ctypes.c_int64)]
        L.qgemm_set_plan_override.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        L.qgemm_quantize_a8.argtypes = [vp, i64, i64, i64, vp, i64, vp, vp]
        i32 = ctypes.c_int32
        L.qgemm_w4g_packed_bytes.argtypes = [i64, i64, i32, i32, u64p]
        L.qgemm_w4g_workspace_bytes.argtypes = [i64, i64, i64, u64p]
        L.qgemm_w4g_repack.argtypes = [i64, i64, i32, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.qgemm_w4g.argtypes = [vp, i64, vp, vp, i64, i64, i64, i64, i32, i32, i32, vp, ctypes.c_size_t, vp]
        L.qgemm_bitplane_packed_bytes.argtypes = [i64, i64, i32, u64p]
        L.qgemm_bitplane_workspace_bytes.argtypes = [i64, i64, i64, i32, u64p]
        L.qgemm_bitplane_repack.argtypes = [i64, i64, i32, vp, vp, vp, ctypes.c_size_t, vp]
        L.qgemm_bitplane_a8.argtypes = [vp, i64, vp, vp, vp, i64, vp, i64, i64, i64, i32, vp, ctypes.c_size_t, vp]
        L.qgemm_bitplane_plan.argtypes = [i64, i64, i64, i32, ctypes.POINTER(ctypes.c_int64)]
        L.qgemm_w4g_plan.argtypes = [i64, i64, i64, i32, i32, i32, ctypes.POINTER(ctypes.c_int64)]
        L.qgemm_plan_info.argtypes = [ctypes.c_int, i64, i64, i64, i32, i32, i32, i32,
                                      ctypes.POINTER(ctypes.c_int64)]
        L.qgemm_w4a16_noalloc.argtypes = [vp, i64, vp, vp, i64, i64, i64, i64, vp]
        for name in ("qgemm_packed_bytes", "qgemm_workspace_bytes", "qgemm_repack", "qgemm_w4a16",
                     "qgemm_w4a8", "qgemm_w2w4_mixed", "qgemm_plan", "qgemm_set_plan_override",
                     "qgemm_quantize_a8", "qgemm_w4g_packed_bytes", "qgemm_w4g_workspace_bytes",
                     "qgemm_w4g_repack", "qgemm_w4g", "qgemm_w4a16_sp24", "qgemm_bitplane_packed_bytes",
                     "qgemm_bitplane_workspace_bytes", "qgemm_bitplane_repack", "qgemm_bitplane_a8",
                     "qgemm_bitplane_plan", "qgemm_w4g_plan", "qgemm_plan_info", "qgemm_w4a16_noalloc"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _status_name(status: int) -> str:
    try:
        return lib().qgemm_status_str(status).decode()
    except ImportError:
        return "QGEMM_STATUS"


def _check(status: int, where: str):
    if status != 0:
        detail = lib().qgemm_last_error().decode()
        raise QgemmError(status, where, detail)


# ----------------------------------------------------------------------------- host-only queries
def _bitmap_ptr(bitmap):
    if bitmap is None:
        return None, None
    import numpy as np
    arr = np.ascontiguousarray(np.asarray(bitmap, dtype=np.uint32))
    return arr, arr.ctypes.data_as(ctypes.c_void_p)


def packed_bytes(fmt: int, K: int, N: int, bitmap=None) -> int:
    keep, ptr = _bitmap_ptr(bitmap)
    out = ctypes.c_size_t(0)
    _check(lib().qgemm_packed_bytes(fmt, K, N, ptr, ctypes.byref(out)), "qgemm_packed_bytes")
    del keep
    return out.value


def workspace_bytes(fmt: int, M: int, K: int, N: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().qgemm_workspace_bytes(fmt, M, K, N, ctypes.byref(out)), "qgemm_workspace_bytes")
    return out.value


_PLAN_KEYS = ("kernel", "mb", "nb", "wpt", "splits", "gps", "mt", "nt", "workgroups", "waves")


def plan(fmt: int, M: int, K: int, N: int, bits: int = 4, group_size: int = 128, zeros: bool = True,
         act_dtype: int = 1) -> dict:
    """Work decomposition of a call of this shape (bits: bit-plane width, used
    only for FMT_BITPLANE; group_size / zeros / act_dtype (DT_F16 or DT_BF16):
    the grid and activation type, used only for FMT_W4G)."""
    arr = (ctypes.c_int64 * 10)()
    if fmt == FMT_BITPLANE:
        _check(lib().qgemm_bitplane_plan(M, K, N, bits, arr), "qgemm_bitplane_plan")
    elif fmt == FMT_W4G:
        _check(lib().qgemm_w4g_plan(M, K, N, group_size, int(zeros), act_dtype, arr), "qgemm_w4g_plan")
    else:
        _check(lib().qgemm_plan(fmt, M, K, N, arr), "qgemm_plan")
    return dict(zip(_PLAN_KEYS, list(arr)))


def plan_info(fmt: int, M: int, K: int, N: int, bits: int = 4, group_size: int = 128,
              zeros: bool = True, act_dtype: int = 1) -> dict:
    """The plan of ``plan()`` plus the call's workspace bytes and the dynamic LDS
    bytes per workgroup its launch requests."""
    arr = (ctypes.c_int64 * 12)()
    _check(lib().qgemm_plan_info(fmt, M, K, N, bits, group_size, int(zeros), act_dtype, arr), "qgemm_plan_info")
    return dict(zip(_PLAN_KEYS + ("ws_bytes", "lds_bytes"), list(arr)))


def set_plan_override(nb_per_tile: int = 0, waves_per_tile: int = 0, k_splits: int = 0,
                      kernel: int = 0):
    """Force parts of the work decomposition (0 = automatic); see include/qgemm.h."""
    _check(lib().qgemm_set_plan_override(kernel, nb_per_tile, waves_per_tile, k_splits),
           "qgemm_set_plan_override")


# ----------------------------------------------------------------------------- device helpers
def _torch():
    import torch
    return torch


def _stream_ptr(device=None):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _require_cuda(*tensors):
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("tensor must live on the GPU")
        if t is not None and not t.is_contiguous():
            raise ValueError("tensor must be contiguous")


class Workspace:
    """Zero-initialised split-K workspace, grown on demand, one buffer per
    (device, stream).

    The kernels leave the counter region zero after each completed call, so the
    buffer is cleared only when it is (re)allocated. Calls that share one
    workspace buffer must run in order, so each stream gets its own buffer
    (allocated while that stream is current: the caching allocator then reuses
    a grown-out buffer's memory only in that stream's order).
    """

    def __init__(self):
        self._bufs = {}

    def get(self, nbytes: int, device):
        torch = _torch()
        idx = torch.device(device).index if torch.device(device).index is not None else torch.cuda.current_device()
        key = (idx, torch.cuda.current_stream(idx).cuda_stream)
        buf = self._bufs.get(key)
        if nbytes == 0:
            return None, 0
        if buf is None or buf.numel() < nbytes:
            buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
            self._bufs[key] = buf
        return buf, buf.numel()


_default_ws = Workspace()


# ----------------------------------------------------------------------------- repack
def repack(fmt: int, K: int, N: int, codes, group_scales, chan_scales=None, bitmap=None):
    """Repack canonical weights (device tensors) into a new uint8 blob tensor."""
    torch = _torch()
    _require_cuda(codes, group_scales, chan_scales)
    nbytes = packed_bytes(fmt, K, N, bitmap)
    out = torch.empty(nbytes, dtype=torch.uint8, device=codes.device)
    keep, bptr = _bitmap_ptr(bitmap)
    _check(lib().qgemm_repack(fmt, K, N, _ptr(codes), _ptr(group_scales), _ptr(chan_scales), bptr,
                              _ptr(out), nbytes, _stream_ptr(codes.device)), "qgemm_repack")
    del keep
    return out


def repack_w4a16(codes, scales):
    """codes: int32 [K/8][N] (canonical nibbles), scales: fp16 [K/128][N]."""
    K, N = codes.shape[0] * 8, codes.shape[1]
    return repack(FMT_W4A16, K, N, codes, scales)


def repack_w4a8(codes, group_scales, chan_scales):
    K, N = codes.shape[0] * 8, codes.shape[1]
    return repack(FMT_W4A8, K, N, codes, group_scales, chan_scales)


def repack_w2w4(codes_u8, scales, bitmap):
    K, N = codes_u8.shape
    return repack(FMT_W2W4, K, N, codes_u8, scales, bitmap=bitmap)


# ----------------------------------------------------------------------------- GEMMs
def _gemm_out(M, N, device, out):
    torch = _torch()
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=device)
    return out


def w4a16(A, blob, K: int, N: int, out=None, workspace: Workspace | None = None):
    """C = A @ dequant(W) with a W4A16 blob; A fp16 [M][K] on the GPU."""
    _require_cuda(A, blob)
    M = A.shape[0]
    out = _gemm_out(M, N, A.device, out)
    ws, wsb = (workspace or _default_ws).get(workspace_bytes(FMT_W4A16, M, K, N), A.device)
    _check(lib().qgemm_w4a16(_ptr(A), A.stride(0), _ptr(blob), _ptr(out), out.stride(0), M, K, N,
                             _ptr(ws), wsb, _stream_ptr(A.device)), "qgemm_w4a16")
    return out


def w4a16_noalloc(A, blob, K: int, N: int, out=None):
    """qgemm_w4a16 without a workspace argument: the library's own fixed
    split-K scratch array serves the call (nothing is allocated except `out`
    when it is not given)."""
    _require_cuda(A, blob)
    M = A.shape[0]
    out = _gemm_out(M, N, A.device, out)
    _check(lib().qgemm_w4a16_noalloc(_ptr(A), A.stride(0), _ptr(blob), _ptr(out), out.stride(0), M, K, N,
                                     _stream_ptr(A.device)), "qgemm_w4a16_noalloc")
    return out


def w4a8(A_i8, a_scale, blob, K: int, N: int, out=None, acc_out=None,
         workspace: Workspace | None = None):
    """W4A8 GEMM; returns C (fp16) and fills acc_out (int32 [M][N]) when given."""
    _require_cuda(A_i8, a_scale, blob, acc_out)
    M = A_i8.shape[0]
    out = _gemm_out(M, N, A_i8.device, out)
    ws, wsb = (workspace or _default_ws).get(workspace_bytes(FMT_W4A8, M, K, N), A_i8.device)
    _check(lib().qgemm_w4a8(_ptr(A_i8), A_i8.stride(0), _ptr(a_scale), _ptr(blob), _ptr(out),
                            out.stride(0), _ptr(acc_out), M, K, N, _ptr(ws), wsb,
                            _stream_ptr(A_i8.device)), "qgemm_w4a8")
    return out


def repack_sp24(codes, scales):
    """codes: int32 [K/8][N] dense W4A16 codes with pruned weights = 8 (at most two
    other codes in every 4 consecutive k of a column), scales: fp16 [K/128][N]."""
    K, N = codes.shape[0] * 8, codes.shape[1]
    return repack(FMT_W4A16_SP24, K, N, codes, scales)


def w4a16_sp24(A, blob, K: int, N: int, out=None, workspace: Workspace | None = None):
    """C = A @ dequant(W) with a 2:4 sparse W4A16 blob; A fp16 [M][K] on the GPU."""
    _require_cuda(A, blob)
    M = A.shape[0]
    out = _gemm_out(M, N, A.device, out)
    ws, wsb = (workspace or _default_ws).get(workspace_bytes(FMT_W4A16_SP24, M, K, N), A.device)
    _check(lib().qgemm_w4a16_sp24(_ptr(A), A.stride(0), _ptr(blob), _ptr(out), out.stride(0), M, K, N,
                                  _ptr(ws), wsb, _stream_ptr(A.device)), "qgemm_w4a16_sp24")
    return out


def w2w4_mixed(A, blob, K: int, N: int, out=None, workspace: Workspace | None = None):
    _require_cuda(A, blob)
    M = A.shape[0]
    out = _gemm_out(M, N, A.device, out)
    ws, wsb = (workspace or _default_ws).get(workspace_bytes(FMT_W2W4, M, K, N), A.device)
    _check(lib().qgemm_w2w4_mixed(_ptr(A), A.stride(0), _ptr(blob), _ptr(out), out.stride(0), M, K,
                                  N, _ptr(ws), wsb, _stream_ptr(A.device)), "qgemm_w2w4_mixed")
    return out


def quantize_a8(A, out=None, scale_out=None):
    """Per-token int8 quantization of fp16 activations A [M][K]; returns
    (A_q int8 [M][K'] with K' = K rounded up to 16 for the row stride, viewed as
    [M][K], a_scale fp16 [M])."""
    torch = _torch()
    _require_cuda(A)
    M, K = A.shape
    ldq = (K + 15) // 16 * 16
    if out is None:
        out = torch.empty((M, ldq), dtype=torch.int8, device=A.device)
    if scale_out is None:
        scale_out = torch.empty((M,), dtype=torch.float16, device=A.device)
    _check(lib().qgemm_quantize_a8(_ptr(A), A.stride(0), M, K, _ptr(out), out.stride(0), _ptr(scale_out),
                                   _stream_ptr(A.device)), "qgemm_quantize_a8")
    return out[:, :K], scale_out


def w4a8_fp16(A, blob, K: int, N: int, out=None, acc_out=None, workspace: Workspace | None = None):
    """W4A8 GEMM from fp16 activations: per-token int8 quantization, then the
    int8 x int4 GEMM (two launches on the current stream)."""
    A_q, a_s = quantize_a8(A)
    return w4a8(A_q, a_s, blob, K, N, out=out, acc_out=acc_out, workspace=workspace)


# ----------------------------------------------------------------------------- general grid
def packed_bytes_w4g(K: int, N: int, group_size: int, has_zeros: bool) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().qgemm_w4g_packed_bytes(K, N, group_size, int(bool(has_zeros)), ctypes.byref(out)),
           "qgemm_w4g_packed_bytes")
    return out.value


def workspace_bytes_w4g(M: int, K: int, N: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().qgemm_w4g_workspace_bytes(M, K, N, ctypes.byref(out)), "qgemm_w4g_workspace_bytes")
    return out.value


def repack_w4g(codes, scales, zeros, group_size: int):
    """codes: int32 [K/8][N]; scales: fp16 or bf16 (any 16-bit dtype) [K/gs][N];
    zeros: uint8 [K/gs][N] or None (implicit zero point 8)."""
    torch = _torch()
    _require_cuda(codes, scales, zeros)
    K, N = codes.shape[0] * 8, codes.shape[1]
    nbytes = packed_bytes_w4g(K, N, group_size, zeros is not None)
    out = torch.empty(nbytes, dtype=torch.uint8, device=codes.device)
    _check(lib().qgemm_w4g_repack(K, N, group_size, _ptr(codes), _ptr(scales), _ptr(zeros), _ptr(out),
                                  nbytes, _stream_ptr(codes.device)), "qgemm_w4g_repack")
    return out


def w4g(A, blob, K: int, N: int, group_size: int, has_zeros: bool, out=None,
        workspace: Workspace | None = None):
    """General-grid 4-bit GEMM; A fp16 or bf16 [M][K] (sets the activation,
    scale and output type); returns C of A's dtype."""
    torch = _torch()
    _require_cuda(A, blob)
    if A.dtype == torch.float16:
        dt = DT_F16
    elif A.dtype == torch.bfloat16:
        dt = DT_BF16
    else:
        raise ValueError("A must be float16 or bfloat16")
    M = A.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=A.dtype, device=A.device)
    ws, wsb = (workspace or _default_ws).get(workspace_bytes_w4g(M, K, N), A.device)
    _check(lib().qgemm_w4g(_ptr(A), A.stride(0), _ptr(blob), _ptr(out), out.stride(0), M, K, N, group_size,
                           int(bool(has_zeros)), dt, _ptr(ws), wsb, _stream_ptr(A.device)), "qgemm_w4g")
    return out


# ----------------------------------------------------------------------------- bit planes
def packed_bytes_bitplane(K: int, N: int, bits: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().qgemm_bitplane_packed_bytes(K, N, bits, ctypes.byref(out)), "qgemm_bitplane_packed_bytes")
    return out.value


def workspace_bytes_bitplane(M: int, K: int, N: int, bits: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().qgemm_bitplane_workspace_bytes(M, K, N, bits, ctypes.byref(out)),
           "qgemm_bitplane_workspace_bytes")
    return out.value


def repack_bitplane(codes_u8, chan_scales, bits: int):
    """codes_u8: uint8 [K][N] holding U (low `bits` bits); chan_scales: fp16 [N]."""
    torch = _torch()
    _require_cuda(codes_u8, chan_scales)
    K, N = codes_u8.shape
    nbytes = packed_bytes_bitplane(K, N, bits)
    out = torch.empty(nbytes, dtype=torch.uint8, device=codes_u8.device)
    _check(lib().qgemm_bitplane_repack(K, N, bits, _ptr(codes_u8), _ptr(chan_scales), _ptr(out), nbytes,
                                       _stream_ptr(codes_u8.device)), "qgemm_bitplane_repack")
    return out


def bitplane_a8(A_i8, a_scale, blob, K: int, N: int, bits: int, out=None, acc_out=None,
                workspace: Workspace | None = None):
    """Bit-plane W_b A8 GEMM; returns C (fp16) and fills acc_out (int32 [M][N]) when given."""
    _require_cuda(A_i8, a_scale, blob, acc_out)
    M = A_i8.shape[0]
    out = _gemm_out(M, N, A_i8.device, out)
    ws, wsb = (workspace or _default_ws).get(workspace_bytes_bitplane(M, K, N, bits), A_i8.device)
    _check(lib().qgemm_bitplane_a8(_ptr(A_i8), A_i8.stride(0), _ptr(a_scale), _ptr(blob), _ptr(out),
                                   out.stride(0), _ptr(acc_out), M, K, N, bits, _ptr(ws), wsb,
                                   _stream_ptr(A_i8.device)), "qgemm_bitplane_a8")
    return out
