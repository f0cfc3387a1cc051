"""Python binding of libqsgemm.so, the gfx950 quantized skinny MUL_MAT library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of ``include/mm.h``.  PyTorch supplies device
memory and the current stream.  Importing this package fails loudly when the
library has not been built (``python quantized_skinny_gemm_amd/build.py``);
there is no CPU fallback.

    dst = mul_mat_q4_0_f32(w_q4, x)      # w_q4: uint8 [N, K/32*18], x: f32 [M, K]
    dst = mul_mat_f16_f32(w_f16, x)      # w_f16: float16 [N, K]
    dst = mul_mat_f32(w_f32, x)          # w_f32: float32 [N, K]
    w_q4 = quantize_q4_0(w_f32)          # Q4_0 blocks of 18 bytes
    a_q8 = quantize_q8_0(x)              # Q8_0 blocks of 34 bytes (the wdata content)
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "LIB_PATH", "lib", "MM_TYPE_F32", "MM_TYPE_F16", "MM_TYPE_Q4_0", "MM_TYPE_Q8_0", "MM_TYPE_Q4_0R",
    "repacked_bytes", "repack_q4_0", "unpack_q4_0", "mul_mat_q4_0r_f32",
    "MMError", "quantize_q4_0", "quantize_q8_0", "mul_mat_q4_0_f32", "mul_mat_q8_0_f32",
    "mul_mat_f16_f32",
    "mul_mat_f32", "workspace_size", "debug_workspace_size", "row_bytes", "dispatch",
    "debug_mul_mat", "status_string", "q4_0_init", "q4_0_compute", "mul_mat_q4_0_f32_group",
    "group_workspace_size",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqsgemm.so")

MM_TYPE_F32, MM_TYPE_F16, MM_TYPE_Q4_0, MM_TYPE_Q8_0, MM_TYPE_Q4_0R = 0, 1, 2, 3, 4

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python quantized_skinny_gemm_amd/build.py` "
        "(the library has no CPU fallback)")

lib = ctypes.CDLL(LIB_PATH)

_i64, _sz, _vp, _int = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int
for _name, _args, _res in [
    ("mm_quantize_q4_0", [_vp, _vp, _i64, _i64, _vp], _int),
    ("mm_quantize_q8_0", [_vp, _vp, _i64, _i64, _vp], _int),
    ("mm_mul_mat_q4_0_f32", [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _vp], _int),
    ("mm_mul_mat_q4_0_f32_noalloc", [_vp, _vp, _vp, _i64, _i64, _i64, _vp], _int),
    ("mm_mul_mat_q4_0r_f32", [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _vp], _int),
    ("mm_mul_mat_q8_0_f32", [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _vp], _int),
    ("mm_repack_q4_0", [_vp, _vp, _i64, _i64, _vp], _int),
    ("mm_unpack_q4_0", [_vp, _vp, _i64, _i64, _vp], _int),
    ("mm_repacked_q4_0_bytes", [_i64, _i64], _i64),
    ("mm_mul_mat_f16_f32", [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _vp], _int),
    ("mm_mul_mat_f32", [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _vp], _int),
    ("mm_q4_0_init", [_vp, _vp, _i64, _i64, _i64, _sz, _vp], _int),
    ("mm_q4_0_compute", [_vp, _vp, _i64, _i64, _i64, _vp, _sz, _vp], _int),
    ("mm_mul_mat_q4_0_f32_group", [_int, ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                   ctypes.POINTER(_i64), _vp, _i64, _i64, _vp, _sz, _vp], _int),
    ("mm_mul_mat_q4_0_group_workspace_size", [_int, ctypes.POINTER(_i64), _i64, _i64], _sz),
    ("mm_mul_mat_workspace_size", [_int, _i64, _i64, _i64], _sz),
    ("mm_debug_workspace_size", [_int, _i64, _i64, _i64, _int], _sz),
    ("mm_row_bytes", [_int, _i64], _i64),
    ("mm_status_string", [_int], ctypes.c_char_p),
    ("mm_dispatch", [_int, _i64, _i64, _i64, ctypes.POINTER(_int)], _int),
    ("mm_debug_mul_mat", [_int, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _vp,
                          _sz, _vp], _int),
]:
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res


class MMError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


def status_string(status: int) -> str:
    return lib.mm_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise MMError(status, what)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t: torch.Tensor, name: str, dtype=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def row_bytes(mm_type: int, k: int) -> int:
    return int(lib.mm_row_bytes(int(mm_type), int(k)))


def workspace_size(mm_type: int, m: int, n: int, k: int) -> int:
    return int(lib.mm_mul_mat_workspace_size(int(mm_type), int(m), int(n), int(k)))


def debug_workspace_size(mm_type: int, m: int, n: int, k: int, variant: int) -> int:
    return int(lib.mm_debug_workspace_size(int(mm_type), int(m), int(n), int(k), int(variant)))


def dispatch(mm_type: int, m: int, n: int, k: int):
    """(variant, split, rows, cols, launches): the kernel mm_mul_mat_* picks at this shape."""
    out = (_int * 5)()
    _check(lib.mm_dispatch(int(mm_type), int(m), int(n), int(k), out), "mm_dispatch")
    return tuple(out)


def _workspace(nbytes: int, device, ws):
    if nbytes == 0:
        return None
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws


def _ptr(t):
    return None if t is None else t.data_ptr()


def quantize_q4_0(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """float32 [rows, K] -> uint8 [rows, K/32*18] Q4_0 blocks."""
    x = _dev(x, "x", torch.float32)
    rows, k = x.shape
    if out is None:
        out = torch.empty((rows, max(row_bytes(MM_TYPE_Q4_0, k), 0)), dtype=torch.uint8, device=x.device)
    _check(lib.mm_quantize_q4_0(_ptr(x), _ptr(out), rows, k, _stream(x)), "mm_quantize_q4_0")
    return out


def quantize_q8_0(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """float32 [rows, K] -> uint8 [rows, K/32*34] Q8_0 blocks."""
    x = _dev(x, "x", torch.float32)
    rows, k = x.shape
    if out is None:
        out = torch.empty((rows, max(row_bytes(MM_TYPE_Q8_0, k), 0)), dtype=torch.uint8, device=x.device)
    _check(lib.mm_quantize_q8_0(_ptr(x), _ptr(out), rows, k, _stream(x)), "mm_quantize_q8_0")
    return out


def _mul_mat(fn, mm_type, w, x, out, ws, what):
    m, k = x.shape
    n = w.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=x.device)
    else:
        _dev(out, "out", torch.float32)
    ws = _workspace(workspace_size(mm_type, m, n, k), x.device, ws)
    nbytes = 0 if ws is None else ws.numel()
    _check(fn(_ptr(w), _ptr(x), _ptr(out), m, n, k, _ptr(ws), nbytes, _stream(x)), what)
    return out


def mul_mat_q4_0_f32(w: torch.Tensor, x: torch.Tensor, out=None, ws=None) -> torch.Tensor:
    """dst[M, N] = Q8_0(x)[M, K] . Q4_0(w)[N, K]^T; w uint8 [N, K/32*18], x float32 [M, K]."""
    w = _dev(w, "w", torch.uint8)
    x = _dev(x, "x", torch.float32)
    if w.shape[1] != row_bytes(MM_TYPE_Q4_0, x.shape[1]):
        raise ValueError("w row bytes do not match K")
    return _mul_mat(lib.mm_mul_mat_q4_0_f32, MM_TYPE_Q4_0, w, x, out, ws, "mm_mul_mat_q4_0_f32")


def mul_mat_q8_0_f32(w: torch.Tensor, x: torch.Tensor, out=None, ws=None) -> torch.Tensor:
    """dst[M, N] = Q8_0(x)[M, K] . Q8_0(w)[N, K]^T; w uint8 [N, K/32*34], x float32 [M, K]."""
    w = _dev(w, "w", torch.uint8)
    x = _dev(x, "x", torch.float32)
    if w.shape[1] != row_bytes(MM_TYPE_Q8_0, x.shape[1]):
        raise ValueError("w row bytes do not match K")
    return _mul_mat(lib.mm_mul_mat_q8_0_f32, MM_TYPE_Q8_0, w, x, out, ws, "mm_mul_mat_q8_0_f32")


def repacked_bytes(n: int, k: int) -> int:
    return int(lib.mm_repacked_q4_0_bytes(int(n), int(k)))


def repack_q4_0(w: torch.Tensor, k: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """uint8 [N, K/32*18] Q4_0 -> uint8 [repacked_bytes(N, K)] repacked weights."""
    w = _dev(w, "w", torch.uint8)
    n = w.shape[0]
    if out is None:
        out = torch.empty(max(repacked_bytes(n, k), 0), dtype=torch.uint8, device=w.device)
    _check(lib.mm_repack_q4_0(_ptr(w), _ptr(out), n, k, _stream(w)), "mm_repack_q4_0")
    return out


def unpack_q4_0(wr: torch.Tensor, n: int, k: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Repacked weights -> uint8 [N, K/32*18] Q4_0."""
    wr = _dev(wr, "wr", torch.uint8)
    if out is None:
        out = torch.empty((n, max(row_bytes(MM_TYPE_Q4_0, k), 0)), dtype=torch.uint8, device=wr.device)
    _check(lib.mm_unpack_q4_0(_ptr(wr), _ptr(out), n, k, _stream(wr)), "mm_unpack_q4_0")
    return out


def mul_mat_q4_0r_f32(wr: torch.Tensor, n: int, x: torch.Tensor, out=None, ws=None) -> torch.Tensor:
    """dst[M, N] = Q8_0(x) . W^T with W (N x K) given in the repacked layout."""
    wr = _dev(wr, "wr", torch.uint8)
    x = _dev(x, "x", torch.float32)
    m, k = x.shape
    if wr.numel() < repacked_bytes(n, k):
        raise ValueError("repacked weights smaller than repacked_bytes(N, K)")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=x.device)
    else:
        _dev(out, "out", torch.float32)
    ws = _workspace(workspace_size(MM_TYPE_Q4_0R, m, n, k), x.device, ws)
    nbytes = 0 if ws is None else ws.numel()
    _check(lib.mm_mul_mat_q4_0r_f32(_ptr(wr), _ptr(x), _ptr(out), m, n, k, _ptr(ws), nbytes,
                                    _stream(x)), "mm_mul_mat_q4_0r_f32")
    return out


def group_workspace_size(ns, m: int, k: int) -> int:
    arr = (_i64 * len(ns))(*ns)
    return int(lib.mm_mul_mat_q4_0_group_workspace_size(len(ns), arr, int(m), int(k)))


def mul_mat_q4_0_f32_group(ws_list, x: torch.Tensor, outs=None, ws=None):
    """[Q8_0(x) . Q4_0(w)^T for w in ws_list] as one grouped call (shared x); returns the outputs."""
    x = _dev(x, "x", torch.float32)
    m, k = x.shape
    ws_list = [_dev(w, f"w[{i}]", torch.uint8) for i, w in enumerate(ws_list)]
    for w in ws_list:
        if w.shape[1] != row_bytes(MM_TYPE_Q4_0, k):
            raise ValueError("w row bytes do not match K")
    ns = [w.shape[0] for w in ws_list]
    if outs is None:
        outs = [torch.empty((m, n), dtype=torch.float32, device=x.device) for n in ns]
    count = len(ws_list)
    src = (_vp * count)(*[w.data_ptr() for w in ws_list])
    dst = (_vp * count)(*[o.data_ptr() for o in outs])
    narr = (_i64 * count)(*ns)
    ws = _workspace(group_workspace_size(ns, m, k), x.device, ws)
    nbytes = 0 if ws is None else ws.numel()
    _check(lib.mm_mul_mat_q4_0_f32_group(count, src, dst, narr, _ptr(x), m, k, _ptr(ws), nbytes,
                                         _stream(x)), "mm_mul_mat_q4_0_f32_group")
    return outs


def mul_mat_f16_f32(w: torch.Tensor, x: torch.Tensor, out=None, ws=None) -> torch.Tensor:
    """dst[M, N] = x[M, K] . w[N, K]^T; w float16, x float32."""
    w = _dev(w, "w", torch.float16)
    x = _dev(x, "x", torch.float32)
    if w.shape[1] != x.shape[1]:
        raise ValueError("K mismatch")
    return _mul_mat(lib.mm_mul_mat_f16_f32, MM_TYPE_F16, w, x, out, ws, "mm_mul_mat_f16_f32")


def mul_mat_f32(w: torch.Tensor, x: torch.Tensor, out=None, ws=None) -> torch.Tensor:
    """dst[M, N] = x[M, K] . w[N, K]^T; all float32."""
    w = _dev(w, "w", torch.float32)
    x = _dev(x, "x", torch.float32)
    if w.shape[1] != x.shape[1]:
        raise ValueError("K mismatch")
    return _mul_mat(lib.mm_mul_mat_f32, MM_TYPE_F32, w, x, out, ws, "mm_mul_mat_f32")


def q4_0_init(x: torch.Tensor, n: int, ws: torch.Tensor | None = None) -> torch.Tensor:
    """INIT stage: quantize x (float32 [M, K]) to Q8_0 into a workspace sized for
    (M, n, K); returns the workspace for q4_0_compute."""
    x = _dev(x, "x", torch.float32)
    m, k = x.shape
    need = workspace_size(MM_TYPE_Q4_0, m, n, k)
    ws = _workspace(need, x.device, ws)
    nbytes = 0 if ws is None else ws.numel()
    _check(lib.mm_q4_0_init(_ptr(x), _ptr(ws), m, n, k, nbytes, _stream(x)), "mm_q4_0_init")
    return ws


def q4_0_compute(w: torch.Tensor, ws: torch.Tensor, m: int, k: int, out=None) -> torch.Tensor:
    """COMPUTE stage: dst[M, N] from the Q8_0 wdata a q4_0_init with the same (M, N, K) left in ws."""
    w = _dev(w, "w", torch.uint8)
    n = w.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=w.device)
    nbytes = 0 if ws is None else ws.numel()
    _check(lib.mm_q4_0_compute(_ptr(w), _ptr(out), m, n, k, _ptr(ws), nbytes, _stream(w)),
           "mm_q4_0_compute")
    return out


_W_DTYPE = {MM_TYPE_Q4_0: torch.uint8, MM_TYPE_F16: torch.float16, MM_TYPE_F32: torch.float32}


def debug_mul_mat(mm_type: int, w: torch.Tensor, x: torch.Tensor, variant: int = 0,
                  n0: int = 0, n1: int = 0):
    """Product with the kernel forced (0 auto, 1 narrow, 2 wide, 3 skinny MFMA); for Q4_0
    also the int32 block dots [M, n1-n0, K/32] of columns n0..n1-1 as written by the
    production kernel."""
    w = _dev(w, "w", _W_DTYPE[mm_type])
    x = _dev(x, "x", torch.float32)
    m, k = x.shape
    n = w.shape[0]
    out = torch.empty((m, n), dtype=torch.float32, device=x.device)
    dots = None
    if mm_type == MM_TYPE_Q4_0 and n1 > n0:
        dots = torch.empty((m, n1 - n0, k // 32), dtype=torch.int32, device=x.device)
    ws = _workspace(debug_workspace_size(mm_type, m, n, k, variant), x.device, None)
    nbytes = 0 if ws is None else ws.numel()
    _check(lib.mm_debug_mul_mat(mm_type, _ptr(w), _ptr(x), _ptr(out), _ptr(dots), m, n, k, n0,
                                n1, variant, _ptr(ws), nbytes, _stream(x)), "mm_debug_mul_mat")
    return out, dots
