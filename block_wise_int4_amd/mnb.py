"""Thin Python binding of libmnb (include/mnb.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  The functions keep the C names; device buffers are
torch CUDA tensors (or raw integer device addresses), and the stream is the
current torch stream unless one is passed.  A non-OK status raises MnbError
with the library's reason.  There is no fallback: if the library is missing
the import fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Union

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "lib", "libmnb.so")

MNB_OK = 0
MNB_ERR_INVALID_ARGUMENT = 1
MNB_ERR_UNSUPPORTED = 2
MNB_ERR_DEVICE = 3
MNB_F32 = 0
MNB_F16 = 1
MNB_BIAS_FUSED = 0
MNB_BIAS_AFTER_ROUND = 1

EXPORTS = ("mnb_repacked_bytes", "mnb_repacked_layout", "mnb_repack", "mnb_gemv",
           "mnb_gemv_gate_up_swiglu", "mnb_gemm_workspace_bytes", "mnb_gemm_workspace_bytes_for", "mnb_gemm",
           "mnb_gemm_bias",
           "mnb_act_order_permutation", "mnb_repack_act_order", "mnb_gemm_act_order_workspace_bytes",
           "mnb_gemm_act_order", "mnb_gemm_group_indices", "mnb_gemm_accuracy4_workspace_bytes", "mnb_gemm_accuracy4",
           "mnb_gemm_accuracy4_noalloc",
           "mnb_unpack_debug", "mnb_debug_prefill_rows", "mnb_status_string", "mnb_last_error", "mnb_last_variant")


class MnbError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (_status_name(status), message))
        self.status = status


class mnb_weight_desc(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("k", ctypes.c_int64), ("group_size", ctypes.c_int32),
                ("has_zero_points", ctypes.c_int32), ("scale_dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class mnb_layout(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int64) for name in (
        "tiles", "chunks", "groups_per_chunk", "codes_offset", "codes_bytes", "scales_offset",
        "scales_bytes", "zero_points_offset", "zero_points_bytes", "range_flags_offset",
        "range_flags_bytes", "total_bytes")]


def _hip_runtimes_mapped():
    """Paths of the HIP runtime libraries mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            return sorted({line.split()[-1] for line in f if "libamdhip64" in line})
    except OSError:
        return []


def _load():
    # torch brings its own HIP runtime.  It must be the one libmnb binds to:
    # device pointers and streams are only meaningful inside one runtime, so
    # torch is loaded first and libmnb's libamdhip64.so.7 dependency resolves
    # to the copy already in the process.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError("libmnb.so is not built (%s); run `python -m block_wise_int4_amd.build`"
                          % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    D = ctypes.POINTER(mnb_weight_desc)
    i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "mnb_repacked_bytes": (sz, [D]),
        "mnb_repacked_layout": (ctypes.c_int, [D, ctypes.POINTER(mnb_layout)]),
        "mnb_repack": (ctypes.c_int, [D, P, P, P, P, P]),
        "mnb_gemv": (ctypes.c_int, [D, P, P, i32, P, P]),
        "mnb_gemv_gate_up_swiglu": (ctypes.c_int, [D, P, P, P, i32, P, P]),
        "mnb_gemm_workspace_bytes": (sz, [D, i64]),
        "mnb_gemm_workspace_bytes_for": (sz, [D, i64, i32]),
        "mnb_gemm": (ctypes.c_int, [D, P, P, i64, i32, P, P, sz, P]),
        "mnb_gemm_bias": (ctypes.c_int, [D, P, P, i64, i32, P, i64, i32, P, P, sz, P]),
        "mnb_act_order_permutation": (ctypes.c_int, [D, P, P]),
        "mnb_repack_act_order": (ctypes.c_int, [D, P, P, P, P, P, P]),
        "mnb_gemm_act_order_workspace_bytes": (sz, [D, i64, i32]),
        "mnb_gemm_act_order": (ctypes.c_int, [D, P, P, i64, i32, P, P, P, sz, P]),
        "mnb_gemm_group_indices": (ctypes.c_int, [D, P, P, i64, i32, P, P, i64, i32, P, P]),
        "mnb_gemm_accuracy4_workspace_bytes": (sz, [D, i64]),
        "mnb_gemm_accuracy4": (ctypes.c_int, [D, P, P, i64, P, P, P, sz, P]),
        "mnb_gemm_accuracy4_noalloc": (ctypes.c_int, [D, P, P, i64, P, P, P]),
        "mnb_unpack_debug": (ctypes.c_int, [D, P, P, P, P]),
        "mnb_debug_prefill_rows": (ctypes.c_int32, [ctypes.c_int32]),
        "mnb_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "mnb_last_error": (ctypes.c_char_p, []),
        "mnb_last_variant": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise ImportError("two HIP runtimes are loaded (%s); import torch before loading libmnb"
                          % ", ".join(runtimes))
    return lib


lib = _load()


def _status_name(s: int) -> str:
    return lib.mnb_status_string(s).decode()


def _check(status: int) -> None:
    if status != MNB_OK:
        raise MnbError(status, lib.mnb_last_error().decode())


Ptr = Union[int, None, "torch.Tensor"]


def _ptr(x: Ptr):
    if x is None:
        return None
    if isinstance(x, int):
        return ctypes.c_void_p(x)
    if not x.is_cuda:
        raise ValueError("device tensor expected")
    if not x.is_contiguous():
        raise ValueError("contiguous tensor expected")
    return ctypes.c_void_p(x.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return MNB_F16
    if t.dtype == torch.float32:
        return MNB_F32
    raise ValueError("fp16 or fp32 tensor expected, got %s" % t.dtype)


def desc(n: int, k: int, group_size: int, has_zero_points: bool, scale_dtype: int) -> mnb_weight_desc:
    return mnb_weight_desc(n, k, group_size, int(bool(has_zero_points)), scale_dtype, 0)


# ---- the C entry points -----------------------------------------------------

def mnb_repacked_bytes(w: mnb_weight_desc) -> int:
    size = lib.mnb_repacked_bytes(ctypes.byref(w))
    if size == 0:
        raise MnbError(MNB_ERR_INVALID_ARGUMENT, lib.mnb_last_error().decode())
    return int(size)


def mnb_repacked_layout(w: mnb_weight_desc) -> dict:
    out = mnb_layout()
    _check(lib.mnb_repacked_layout(ctypes.byref(w), ctypes.byref(out)))
    return {name: getattr(out, name) for name, _ in mnb_layout._fields_}


def mnb_repack(w: mnb_weight_desc, packed: Ptr, scales: Ptr, zero_points: Ptr, repacked: Ptr,
               stream=None) -> None:
    _check(lib.mnb_repack(ctypes.byref(w), _ptr(packed), _ptr(scales), _ptr(zero_points),
                          _ptr(repacked), _stream(stream)))


def mnb_gemv(w: mnb_weight_desc, repacked: Ptr, a, y, a_dtype: Optional[int] = None,
             stream=None) -> None:
    dt = _dtype_code(a) if a_dtype is None else a_dtype
    _check(lib.mnb_gemv(ctypes.byref(w), _ptr(repacked), _ptr(a), dt, _ptr(y), _stream(stream)))


def mnb_gemv_gate_up_swiglu(w: mnb_weight_desc, gate_repacked: Ptr, up_repacked: Ptr, a, y,
                            a_dtype: Optional[int] = None, stream=None) -> None:
    dt = _dtype_code(a) if a_dtype is None else a_dtype
    _check(lib.mnb_gemv_gate_up_swiglu(ctypes.byref(w), _ptr(gate_repacked), _ptr(up_repacked),
                                       _ptr(a), dt, _ptr(y), _stream(stream)))


def mnb_gemm_workspace_bytes(w: mnb_weight_desc, m: int) -> int:
    return int(lib.mnb_gemm_workspace_bytes(ctypes.byref(w), m))


def mnb_gemm_workspace_bytes_for(w: mnb_weight_desc, m: int, a_dtype: int) -> int:
    return int(lib.mnb_gemm_workspace_bytes_for(ctypes.byref(w), m, a_dtype))


def mnb_gemm(w: mnb_weight_desc, repacked: Ptr, a, m: int, y, workspace: Ptr = None,
             workspace_bytes: Optional[int] = None, a_dtype: Optional[int] = None,
             stream=None) -> None:
    dt = _dtype_code(a) if a_dtype is None else a_dtype
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None or isinstance(workspace, int) else \
            workspace.numel() * workspace.element_size()
    _check(lib.mnb_gemm(ctypes.byref(w), _ptr(repacked), _ptr(a), m, dt, _ptr(y),
                        _ptr(workspace), workspace_bytes, _stream(stream)))


def mnb_gemm_bias(w: mnb_weight_desc, repacked: Ptr, a, m: int, bias, bias_row_stride: int,
                  bias_mode: int, y, workspace: Ptr = None, workspace_bytes: Optional[int] = None,
                  a_dtype: Optional[int] = None, stream=None) -> None:
    dt = _dtype_code(a) if a_dtype is None else a_dtype
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None or isinstance(workspace, int) else \
            workspace.numel() * workspace.element_size()
    _check(lib.mnb_gemm_bias(ctypes.byref(w), _ptr(repacked), _ptr(a), m, dt, _ptr(bias),
                             bias_row_stride, bias_mode, _ptr(y), _ptr(workspace), workspace_bytes,
                             _stream(stream)))


def mnb_act_order_permutation(w: mnb_weight_desc, g_idx):
    """Host: the act-order permutation of k for a g_idx (numpy int32 [K])."""
    import numpy as np
    g = np.ascontiguousarray(g_idx, np.int32)
    perm = np.empty(g.size, dtype=np.int32)
    _check(lib.mnb_act_order_permutation(ctypes.byref(w), g.ctypes.data_as(ctypes.c_void_p),
                                         perm.ctypes.data_as(ctypes.c_void_p)))
    return perm


def mnb_repack_act_order(w: mnb_weight_desc, packed: Ptr, scales: Ptr, zero_points: Ptr, perm: Ptr,
                         repacked: Ptr, stream=None) -> None:
    _check(lib.mnb_repack_act_order(ctypes.byref(w), _ptr(packed), _ptr(scales), _ptr(zero_points),
                                    _ptr(perm), _ptr(repacked), _stream(stream)))


def mnb_gemm_act_order_workspace_bytes(w: mnb_weight_desc, m: int, a_dtype: int = MNB_F16) -> int:
    return int(lib.mnb_gemm_act_order_workspace_bytes(ctypes.byref(w), m, a_dtype))


def mnb_gemm_act_order(w: mnb_weight_desc, repacked: Ptr, a, m: int, perm: Ptr, y, workspace: Ptr,
                       workspace_bytes: Optional[int] = None, a_dtype: Optional[int] = None,
                       stream=None) -> None:
    dt = _dtype_code(a) if a_dtype is None else a_dtype
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None or isinstance(workspace, int) else \
            workspace.numel() * workspace.element_size()
    _check(lib.mnb_gemm_act_order(ctypes.byref(w), _ptr(repacked), _ptr(a), m, dt, _ptr(perm), _ptr(y),
                                  _ptr(workspace), workspace_bytes, _stream(stream)))


def mnb_gemm_group_indices(w: mnb_weight_desc, repacked: Ptr, a, m: int, g_idx: Ptr, y, bias=None,
                           bias_row_stride: int = 0, bias_mode: int = MNB_BIAS_FUSED,
                           a_dtype: Optional[int] = None, stream=None) -> None:
    dt = _dtype_code(a) if a_dtype is None else a_dtype
    _check(lib.mnb_gemm_group_indices(ctypes.byref(w), _ptr(repacked), _ptr(a), m, dt, _ptr(g_idx), _ptr(bias),
                                      bias_row_stride, bias_mode, _ptr(y), _stream(stream)))


def mnb_gemm_accuracy4_workspace_bytes(w: mnb_weight_desc, m: int) -> int:
    return int(lib.mnb_gemm_accuracy4_workspace_bytes(ctypes.byref(w), m))


def mnb_gemm_accuracy4(w: mnb_weight_desc, repacked: Ptr, a, m: int, bias, y, workspace: Ptr = None,
                       workspace_bytes: Optional[int] = None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None or isinstance(workspace, int) else \
            workspace.numel() * workspace.element_size()
    _check(lib.mnb_gemm_accuracy4(ctypes.byref(w), _ptr(repacked), _ptr(a), m, _ptr(bias), _ptr(y),
                                  _ptr(workspace), workspace_bytes, _stream(stream)))


MNB_NOALLOC_SCRATCH_BYTES = 32 << 20


def mnb_gemm_accuracy4_noalloc(w: mnb_weight_desc, repacked: Ptr, a, m: int, bias, y, stream=None) -> None:
    _check(lib.mnb_gemm_accuracy4_noalloc(ctypes.byref(w), _ptr(repacked), _ptr(a), m, _ptr(bias), _ptr(y),
                                          _stream(stream)))


def mnb_unpack_debug(w: mnb_weight_desc, repacked: Ptr, codes: Ptr, w_f32: Ptr, stream=None) -> None:
    _check(lib.mnb_unpack_debug(ctypes.byref(w), _ptr(repacked), _ptr(codes), _ptr(w_f32),
                                _stream(stream)))


def mnb_debug_prefill_rows(rows: int) -> int:
    return lib.mnb_debug_prefill_rows(rows)


def mnb_status_string(s: int) -> str:
    return _status_name(s)


def mnb_last_error() -> str:
    return lib.mnb_last_error().decode()


def mnb_last_variant() -> str:
    return lib.mnb_last_variant().decode()


# ---- convenience over torch tensors (allocation only) -----------------------

class QuantWeight:
    """A repacked weight resident on the device, plus its descriptor."""

    def __init__(self, desc_: mnb_weight_desc, repacked):
        self.desc = desc_
        self.repacked = repacked

    @property
    def n(self) -> int:
        return self.desc.n

    @property
    def k(self) -> int:
        return self.desc.k


def repack(packed, scales, zero_points, n: int, k: int, group_size: int, stream=None) -> QuantWeight:
    """Allocate the repacked buffer (torch) and run mnb_repack into it."""
    import torch
    d = desc(n, k, group_size, zero_points is not None, _dtype_code(scales))
    out = torch.empty(mnb_repacked_bytes(d), dtype=torch.uint8, device=packed.device)
    mnb_repack(d, packed, scales, zero_points, out, stream)
    return QuantWeight(d, out)
