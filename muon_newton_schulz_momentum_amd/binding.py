"""ctypes binding of libmuon.so (include/muon.h): the same names, argument marshalling only.

Importing this module loads the in-tree libmuon.so and raises if it is missing; there is
no fallback path of any kind.  Build it with `python -m muon_newton_schulz_momentum_amd.build`.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmuon.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libmuon.so is not built ({LIB_PATH} missing); run "
                      "`python -m muon_newton_schulz_momentum_amd.build` first")

# torch ships its own HIP runtime, loaded under the file name libamdhip64.so.  libmuon.so
# asks for libamdhip64.so.7; if it is loaded first, the process ends up with two HIP
# runtimes and the second finds no device.  Importing torch first makes libmuon bind to
# torch's already-loaded runtime (same soname), so both share one device context.
import torch  # noqa: E402,F401

_lib = C.CDLL(LIB_PATH)

# ---- constants (include/muon.h) ----------------------------------------------------------
MUON_OK = 0
MUON_ERR_INVALID_ARG = 1
MUON_ERR_SHAPE = 2
MUON_ERR_ALIGNMENT = 3
MUON_ERR_WORKSPACE_TOO_SMALL = 4
MUON_ERR_NOT_BOUND = 5
MUON_ERR_STALE_PLAN = 6
MUON_ERR_HIP = 7

MUON_DTYPE_F32 = 0
MUON_DTYPE_BF16 = 1

MUON_KERNEL_MOMENTUM = 0
MUON_KERNEL_NORM_FINALIZE = 1
MUON_KERNEL_NORMALIZE = 2
MUON_KERNEL_SYRK = 3
MUON_KERNEL_SYRK_POLY = 4
MUON_KERNEL_GEMM_AXPY = 5
MUON_KERNEL_APPLY = 6
MUON_KERNEL_NS_SMALL = 7
MUON_KERNEL_ADAMW = 8
MUON_KERNEL_MOMENTUM_SIDE = 9
MUON_KERNEL_NORMALIZE_SIDE = 10
MUON_KERNEL_APPLY_SIDE = 11
MUON_KERNEL_NS_GROUPED = 12
MUON_KERNEL_PREP_GROUPED = 13
MUON_KERNEL_COUNT = 14

MUON_OPT_DEFAULT = 0
MUON_OPT_ADAMW = 1
MUON_OPT_NONE = 2

MUON_PLAN_TILED_SMALL = 1
MUON_PLAN_PIPELINE = 2
MUON_PLAN_UNFUSED_NORMALIZE = 4
MUON_PLAN_UNGROUPED = 8

MUON_SCALE_NONE = 0
MUON_SCALE_ASPECT = 1
MUON_SCALE_RMS_MATCH = 2


class muon_param_desc(C.Structure):
    _fields_ = [("ndim", C.c_int32), ("grad_dtype", C.c_int32), ("rows", C.c_int64),
                ("cols", C.c_int64), ("weight", C.c_void_p), ("momentum", C.c_void_p),
                ("grad", C.c_void_p), ("exp_avg_sq", C.c_void_p), ("optimizer", C.c_int32),
                ("reserved", C.c_int32)]


class muon_adamw_config(C.Structure):
    _fields_ = [("lr", C.c_float), ("beta1", C.c_float), ("beta2", C.c_float), ("eps", C.c_float),
                ("wd", C.c_float), ("reserved", C.c_int32), ("step", C.c_int64), ("dev_scalars", C.c_void_p)]


class muon_plan_opts(C.Structure):
    _fields_ = [("max_workspace_bytes", C.c_uint64), ("scale", C.POINTER(C.c_float)), ("flags", C.c_uint32),
                ("scale_mode", C.c_int32)]


class muon_chunk_info(C.Structure):
    _fields_ = [("m", C.c_int64), ("n", C.c_int64), ("m_pad", C.c_int64), ("n_pad", C.c_int64),
                ("count", C.c_int64), ("bucket", C.c_int32), ("tile", C.c_int32),
                ("grad_dtype", C.c_int32), ("shared_region", C.c_int32),
                ("fused_small", C.c_int32), ("grouped_small", C.c_int32),
                ("flops_conventional", C.c_double), ("flops_algorithmic", C.c_double),
                ("bytes_momentum", C.c_double), ("bytes_apply", C.c_double),
                ("region_offset", C.c_uint64), ("region_bytes", C.c_uint64)]


class muon_step_config(C.Structure):
    _fields_ = [("beta", C.c_float), ("lr", C.c_float), ("wd", C.c_float), ("eps", C.c_float),
                ("steps", C.c_int32), ("a", C.c_float), ("b", C.c_float), ("c", C.c_float),
                ("coeffs", C.POINTER(C.c_float)), ("nesterov", C.c_int32), ("dev_scalars", C.c_void_p),
                ("adamw", C.POINTER(muon_adamw_config)), ("pipeline", C.c_int32)]


class muon_param_info(C.Structure):
    _fields_ = [("included", C.c_int32), ("chunk", C.c_int32), ("slot", C.c_int64),
                ("transposed", C.c_int32), ("scale", C.c_float),
                ("output_offset", C.c_uint64), ("ld", C.c_int64)]


_P = C.c_void_p  # muon_plan*


def _fn(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


muon_plan_buckets = _fn("muon_plan_buckets", C.c_int32,
                        [C.POINTER(muon_param_desc), C.c_int64, C.POINTER(muon_plan_opts), C.POINTER(_P)])
muon_plan_workspace_bytes = _fn("muon_plan_workspace_bytes", C.c_int32, [_P, C.POINTER(C.c_uint64)])
muon_plan_counts = _fn("muon_plan_counts", C.c_int32,
                       [_P, C.POINTER(C.c_int32), C.POINTER(C.c_int32), C.POINTER(C.c_int64),
                        C.POINTER(C.c_int64)])
muon_plan_info = _fn("muon_plan_info", C.c_int32, [_P, C.c_int32, C.POINTER(muon_chunk_info)])
muon_plan_param_info = _fn("muon_plan_param_info", C.c_int32, [_P, C.c_int64, C.POINTER(muon_param_info)])
muon_plan_validate = _fn("muon_plan_validate", C.c_int32, [_P, C.POINTER(muon_param_desc), C.c_int64])
muon_plan_bind = _fn("muon_plan_bind", C.c_int32, [_P, C.c_void_p, C.c_uint64, C.c_void_p])
muon_momentum_update = _fn("muon_momentum_update", C.c_int32, [_P, C.c_int32, C.c_float, C.c_void_p])
muon_ns_batched = _fn("muon_ns_batched", C.c_int32,
                      [_P, C.c_int32, C.c_float, C.c_float, C.c_float, C.c_int32, C.c_float, C.c_void_p])
muon_apply = _fn("muon_apply", C.c_int32, [_P, C.c_int32, C.c_float, C.c_float, C.c_void_p])
muon_ns_batched_schedule = _fn("muon_ns_batched_schedule", C.c_int32,
                               [_P, C.c_int32, C.POINTER(C.c_float), C.c_int32, C.c_float, C.c_void_p])
muon_adamw_step = _fn("muon_adamw_step", C.c_int32, [_P, C.POINTER(muon_adamw_config), C.c_void_p])
muon_plan_adamw_counts = _fn("muon_plan_adamw_counts", C.c_int32, [_P, C.POINTER(C.c_int64), C.POINTER(C.c_int64)])
muon_step_ex = _fn("muon_step_ex", C.c_int32, [_P, C.c_int32, C.POINTER(muon_step_config), C.c_void_p])
muon_step_noalloc = _fn("muon_step_noalloc", C.c_int32, [_P, C.POINTER(muon_step_config), C.c_void_p])
MUON_NOALLOC_MAX_BYTES = 64 << 20
muon_step = _fn("muon_step", C.c_int32,
                [_P, C.c_int32, C.c_float, C.c_float, C.c_float, C.c_float, C.c_int32, C.c_float,
                 C.c_float, C.c_float, C.c_void_p])
_G = C.c_void_p  # muon_graph*
muon_graph_capture = _fn("muon_graph_capture", C.c_int32,
                         [_P, C.c_float, C.c_float, C.c_float, C.c_float, C.c_int32, C.c_float, C.c_float,
                          C.c_float, C.POINTER(_G)])
muon_graph_capture_ex = _fn("muon_graph_capture_ex", C.c_int32, [_P, C.POINTER(muon_step_config), C.POINTER(_G)])
muon_graph_launch = _fn("muon_graph_launch", C.c_int32, [_G, C.c_void_p])
muon_graph_node_count = _fn("muon_graph_node_count", C.c_int32, [_G, C.POINTER(C.c_int64)])
muon_graph_destroy = _fn("muon_graph_destroy", None, [_G])
muon_timing_enable = _fn("muon_timing_enable", C.c_int32, [_P, C.c_int32])
muon_timing_read = _fn("muon_timing_read", C.c_int32,
                       [_P, C.c_int32, C.POINTER(C.c_double), C.POINTER(C.c_int64), C.POINTER(C.c_double)])
muon_timing_reset = _fn("muon_timing_reset", C.c_int32, [_P])
muon_kernel_name = _fn("muon_kernel_name", C.c_char_p, [C.c_int32])
muon_plan_destroy = _fn("muon_plan_destroy", None, [_P])
muon_status_string = _fn("muon_status_string", C.c_char_p, [C.c_int32])
muon_last_error = _fn("muon_last_error", C.c_char_p, [])

EXPORTED = [
    "muon_plan_buckets", "muon_plan_workspace_bytes", "muon_plan_counts", "muon_plan_info",
    "muon_plan_param_info", "muon_plan_validate", "muon_plan_bind", "muon_momentum_update",
    "muon_ns_batched", "muon_ns_batched_schedule", "muon_apply", "muon_adamw_step", "muon_plan_adamw_counts",
    "muon_step", "muon_step_ex", "muon_step_noalloc",
    "muon_graph_capture", "muon_graph_capture_ex", "muon_graph_launch",
    "muon_graph_node_count", "muon_graph_destroy", "muon_timing_enable", "muon_timing_read",
    "muon_timing_reset", "muon_kernel_name", "muon_plan_destroy", "muon_status_string",
    "muon_last_error",
]


class MuonError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = muon_last_error().decode(errors="replace")
        super().__init__(f"{where}: {muon_status_string(status).decode()} ({status}): {msg}")


def check(status: int, where: str) -> None:
    if status != MUON_OK:
        raise MuonError(status, where)
