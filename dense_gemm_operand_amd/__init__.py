"""Python binding of libdgemm (include/dgemm.h, include/dattn.h): argument marshalling only.

Every function has the name of the C entry point it wraps. Device buffers are passed as
torch tensors (or raw integer device pointers); every step of the GEMM and of the attention
forward runs in the HIP kernels of libdgemm.so. There is no fallback: if the library is
missing, loading fails with an error that says how to build it. Tensor arguments are
checked to be contiguous device tensors at least as large as the operation needs (the C
ABI takes raw pointers and cannot check them); raw integer pointers are passed on as is.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdgemm.so")

GEMM_ROW_MAJOR, GEMM_COL_MAJOR, GEMM_U4_TILED = 0, 1, 2
GEMM_F32, GEMM_F16, GEMM_BF16, GEMM_U4, GEMM_F8 = 0, 1, 2, 3, 4
GEMM_OK = 0
GEMM_ERR_INVALID_ARG = -1
GEMM_ERR_UNSUPPORTED = -2
GEMM_ERR_MISALIGNED = -3
GEMM_ERR_WORKSPACE_TOO_SMALL = -4
GEMM_ERR_NO_DEVICE = -5
GEMM_ERR_HIP = -6

# Per-GPU workspace of gemm_run_noalloc (include/dgemm.h GEMM_NOALLOC_WORKSPACE_BYTES).
NOALLOC_WORKSPACE_BYTES = 32 << 20

LAYOUT = {"row": GEMM_ROW_MAJOR, "col": GEMM_COL_MAJOR, "u4_tiled": GEMM_U4_TILED}
DTYPE = {"f32": GEMM_F32, "f16": GEMM_F16, "bf16": GEMM_BF16, "u4": GEMM_U4, "f8": GEMM_F8}

# Bytes at the start of every workspace that hold arrival counters (must be zero before
# a workspace is first used; every completed run leaves them zero).
COUNTER_BYTES = 64 * 1024


class GemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {gemm_status_string(status)} ({status})")
        self.status = status


class gemm_quant_t(ctypes.Structure):
    _fields_ = [("group_size", ctypes.c_int32), ("zero_point", ctypes.c_int32),
                ("scale_dtype", ctypes.c_int32), ("scale_layout", ctypes.c_int32)]


class gemm_plan_info_t(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("layout_a", ctypes.c_int32), ("layout_b", ctypes.c_int32),
                ("dtype_a", ctypes.c_int32), ("dtype_b", ctypes.c_int32),
                ("dtype_c", ctypes.c_int32), ("kernel", ctypes.c_int32),
                ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("tile_k", ctypes.c_int32), ("waves", ctypes.c_int32),
                ("lds_pad_bytes", ctypes.c_int32), ("perm_block", ctypes.c_int32),
                ("perm_stride", ctypes.c_int32), ("split_k", ctypes.c_int32),
                ("wave_split_k", ctypes.c_int32), ("grid_x", ctypes.c_int64),
                ("grid_y", ctypes.c_int64), ("grid_z", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_int64), ("lds_bytes", ctypes.c_int32),
                ("cu_count", ctypes.c_int32), ("slots_per_cu", ctypes.c_int32),
                ("direct_lds", ctypes.c_int32), ("schedule", ctypes.c_int32),
                ("mfma_m", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libdgemm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m dense_gemm_operand_amd.build`"
                " (there is no fallback path)")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.gemm_plan.argtypes = [ctypes.POINTER(vp), i64, i64, i64, i32, i32, i32, i32, i32, i32,
                                ctypes.POINTER(gemm_quant_t)]
        L.gemm_plan.restype = i32
        L.gemm_workspace_size.argtypes = [vp, ctypes.POINTER(ctypes.c_size_t)]
        L.gemm_workspace_size.restype = i32
        L.gemm_run.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.gemm_run.restype = i32
        L.gemm_run_noalloc.argtypes = [vp, vp, vp, vp, vp, vp]
        L.gemm_run_noalloc.restype = i32
        L.gemm_plan_query.argtypes = [vp, ctypes.POINTER(gemm_plan_info_t)]
        L.gemm_plan_query.restype = i32
        L.gemm_plan_destroy.argtypes = [vp]
        L.gemm_plan_destroy.restype = None
        L.gemm_status_string.argtypes = [i32]
        L.gemm_status_string.restype = ctypes.c_char_p
        L.gemm_lds_row_perm.argtypes = [i32, i32, i32, i32]
        L.gemm_lds_row_perm.restype = i32
        L.gemm_pack_u4_tiled.argtypes = [vp, vp, i64, i64]
        L.gemm_pack_u4_tiled.restype = i32
        L.attn_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i32, ctypes.c_float, vp]
        L.attn_fwd.restype = i32
        _lib = L
    return _lib


def _code(v, table):
    return table[v] if isinstance(v, str) else int(v)


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


# Bytes that the operands of a plan made through gemm_plan occupy (A, B, scales, C), so that
# gemm_run refuses host tensors and tensors too small for the plan before a kernel would
# access memory outside them (the C ABI takes raw pointers and cannot check this).
_plan_bytes: dict = {}


def _check_buffer(x, need: int, what: str) -> None:
    """A tensor argument must be a contiguous device tensor of at least `need` bytes; raw
    integer pointers are passed on unchecked."""
    if x is None or isinstance(x, int):
        return
    if not getattr(x, "is_cuda", False):
        raise ValueError(f"{what}: a device tensor is needed")
    if not x.is_contiguous():
        raise ValueError(f"{what}: the tensor must be contiguous")
    have = x.numel() * x.element_size()
    if have < need:
        raise ValueError(f"{what}: {have} bytes, {need} needed")


def _nbytes(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        raise TypeError("pass the workspace as a tensor (its size is needed)")
    return x.numel() * x.element_size()


def gemm_plan(M: int, N: int, K: int, layout_a, layout_b, dtype_a, dtype_b, dtype_c,
              split_k: int = 0, quant: gemm_quant_t | None = None) -> int:
    """Make a plan; returns the opaque handle (an int). Layouts: "row"/"col" or codes;
    dtypes: "f32"/"f16"/"bf16"/"u4"/"f8" or codes."""
    h = ctypes.c_void_p()
    q = ctypes.byref(quant) if quant is not None else None
    st = lib().gemm_plan(ctypes.byref(h), M, N, K, _code(layout_a, LAYOUT), _code(layout_b, LAYOUT),
                         _code(dtype_a, DTYPE), _code(dtype_b, DTYPE), _code(dtype_c, DTYPE),
                         split_k, q)
    if st != GEMM_OK:
        raise GemmError(st, "gemm_plan")
    da, db, dc = _code(dtype_a, DTYPE), _code(dtype_b, DTYPE), _code(dtype_c, DTYPE)
    eb = 1 if da == GEMM_F8 else 2
    u4 = db == GEMM_U4
    _plan_bytes[h.value] = (M * K * eb, N * K // 2 if u4 else N * K * eb,
                            (K // quant.group_size) * N * 2 if u4 else 0,
                            M * N * (4 if dc == GEMM_F32 else 2))
    return h.value


def int4_quant(group_size: int = 128, zero_point: int = 8) -> gemm_quant_t:
    return gemm_quant_t(group_size, zero_point, GEMM_F16, 0)


def gemm_workspace_size(plan: int) -> int:
    n = ctypes.c_size_t()
    st = lib().gemm_workspace_size(plan, ctypes.byref(n))
    if st != GEMM_OK:
        raise GemmError(st, "gemm_workspace_size")
    return n.value


def gemm_run(plan: int, A, B, scales, C, workspace=None, stream=None) -> None:
    """Enqueue C = A*B. Tensors (or raw device pointers) for A, B, scales, C; workspace a
    tensor of at least gemm_workspace_size bytes (first 64 KiB zero before first use);
    stream a torch stream, a raw hipStream_t int, or None for torch's current stream."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    need = _plan_bytes.get(plan)
    if need is not None:
        for x, n, what in ((A, need[0], "A"), (B, need[1], "B"), (scales, need[2], "scales"),
                           (C, need[3], "C")):
            _check_buffer(x, n, what)
    _check_buffer(workspace, 0, "workspace")
    st = lib().gemm_run(plan, _ptr(A), _ptr(B), _ptr(scales), _ptr(C), _ptr(workspace),
                        _nbytes(workspace), stream)
    if st != GEMM_OK:
        raise GemmError(st, "gemm_run")


def gemm_run_noalloc(plan: int, A, B, scales, C, stream=None) -> None:
    """Enqueue C = A*B like gemm_run, with the library's own per-GPU split-K workspace
    (GEMM_NOALLOC_WORKSPACE_BYTES) instead of a caller buffer: nothing is allocated. Calls
    that overlap in time on one GPU share that workspace and must be serialised."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    need = _plan_bytes.get(plan)
    if need is not None:
        for x, n, what in ((A, need[0], "A"), (B, need[1], "B"), (scales, need[2], "scales"),
                           (C, need[3], "C")):
            _check_buffer(x, n, what)
    st = lib().gemm_run_noalloc(plan, _ptr(A), _ptr(B), _ptr(scales), _ptr(C), stream)
    if st != GEMM_OK:
        raise GemmError(st, "gemm_run_noalloc")


def attn_fwd(Q, K, V, O, BH: int, Sq: int, Sk: int, D: int, dtype, scale: float,
             stream=None) -> None:
    """Enqueue O = softmax(scale * Q K^T) V (include/dattn.h). Q, O: BH x Sq x D, K, V:
    BH x Sk x D device tensors (or raw pointers), head dim contiguous; dtype "f16"/"bf16"."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    if min(BH, Sq, Sk, D) > 0:
        for x, rows, what in ((Q, Sq, "Q"), (K, Sk, "K"), (V, Sk, "V"), (O, Sq, "O")):
            _check_buffer(x, BH * rows * D * 2, what)
    st = lib().attn_fwd(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), BH, Sq, Sk, D, _code(dtype, DTYPE),
                        float(scale), stream)
    if st != GEMM_OK:
        raise GemmError(st, "attn_fwd")


def gemm_plan_query(plan: int) -> dict:
    info = gemm_plan_info_t()
    st = lib().gemm_plan_query(plan, ctypes.byref(info))
    if st != GEMM_OK:
        raise GemmError(st, "gemm_plan_query")
    return {name: getattr(info, name) for name, _ in gemm_plan_info_t._fields_}


def gemm_plan_destroy(plan: int | None) -> None:
    _plan_bytes.pop(plan, None)
    lib().gemm_plan_destroy(plan)


def gemm_status_string(status: int) -> str:
    return lib().gemm_status_string(status).decode()


def gemm_lds_row_perm(block: int, stride: int, index: int, inverse: bool = False) -> int:
    return lib().gemm_lds_row_perm(block, stride, index, 1 if inverse else 0)


def gemm_pack_u4_tiled(codes, N: int, K: int):
    """Host repack of int4 codes (numpy uint8, N*K/2 bytes, column-major packing) into the
    pre-tiled layout; returns a new numpy uint8 array."""
    import numpy as np
    src = np.ascontiguousarray(codes, dtype=np.uint8)
    if N > 0 and K > 0 and src.size != N * K // 2:
        raise ValueError(f"codes: {src.size} bytes, N*K/2 = {N * K // 2} expected")
    dst = np.empty_like(src)
    st = lib().gemm_pack_u4_tiled(src.ctypes.data, dst.ctypes.data, N, K)
    if st != GEMM_OK:
        raise GemmError(st, "gemm_pack_u4_tiled")
    return dst
