"""ctypes binding of librp.so (the C ABI in include/ragged_prefill.h).

Argument marshalling only: every step of the computation runs in the
library's kernels.  Loading fails loudly when the library has not been built.
"""

from __future__ import annotations

import ctypes
import os
import threading

from . import build as _build

_lib = None
_lock = threading.Lock()

RP_OK = 0
RP_EINVAL = -1
RP_EUNSUPPORTED = -2
RP_ENOMEM = -3
RP_EDEVICE = -4

RP_SPLIT_AUTO = 0
RP_SPLIT_NEVER = 1
RP_SPLIT_ALWAYS = 2

RP_ITEM_INTS = 16

# exported symbols declared in include/ragged_prefill.h
EXPORTS = [
    "rp_status_string",
    "rp_last_error",
    "rp_abi_version",
    "rp_available",
    "ragged_prefill_bf16",
    "rp_plan_create",
    "rp_plan_get_info",
    "rp_plan_workspace_bytes",
    "rp_plan_copy_items",
    "rp_run",
    "rp_run_noalloc",
    "rp_run_paged",
    "rp_run_fp8kv",
    "rp_run_paged_fp8kv",
    "rp_plan_destroy",
    "rp_merge_state",
    "rp_merge_state_in_place",
    "rp_merge_states",
    "rp_plan_create_shared_prefix",
    "rp_run_shared_prefix",
    "rp_run_shared_prefix_paged",
]


class RpPlanOpts(ctypes.Structure):
    _fields_ = [("kv_chunk", ctypes.c_int), ("split_mode", ctypes.c_int),
                ("host_only", ctypes.c_int), ("num_xcds", ctypes.c_int)]


class RpPlanInfo(ctypes.Structure):
    _fields_ = [("num_items", ctypes.c_int64), ("num_partial_items", ctypes.c_int64),
                ("num_merge_items", ctypes.c_int64), ("total_q", ctypes.c_int64),
                ("total_kv", ctypes.c_int64), ("tile_rows", ctypes.c_int32),
                ("tile_tokens", ctypes.c_int32), ("key_block", ctypes.c_int32),
                ("kv_chunk", ctypes.c_int32), ("flops", ctypes.c_double),
                ("bytes", ctypes.c_double), ("workspace_bytes", ctypes.c_size_t),
                ("num_fold_items", ctypes.c_int64)]


class RaggedPrefillError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def lib_path() -> str:
    return _build.LIB


def load():
    """Load librp.so; raise ImportError if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = lib_path()
        if not os.path.exists(path):
            raise ImportError(
                f"{path} is missing: build the gfx950 library first "
                "(python -m varlen_prefill_amd.build, or __graft_entry__.build())")
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.rp_status_string.argtypes = [I]
        lib.rp_status_string.restype = ctypes.c_char_p
        lib.rp_last_error.argtypes = []
        lib.rp_last_error.restype = ctypes.c_char_p
        lib.rp_abi_version.argtypes = []
        lib.rp_abi_version.restype = I
        lib.rp_available.argtypes = []
        lib.rp_available.restype = I
        lib.ragged_prefill_bf16.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, ctypes.c_float, P]
        lib.ragged_prefill_bf16.restype = I
        lib.rp_plan_create.argtypes = [P, P, I, I, I, I, I, ctypes.POINTER(RpPlanOpts),
                                       ctypes.POINTER(P)]
        lib.rp_plan_create.restype = I
        lib.rp_plan_get_info.argtypes = [P, ctypes.POINTER(RpPlanInfo)]
        lib.rp_plan_get_info.restype = I
        lib.rp_plan_workspace_bytes.argtypes = [P]
        lib.rp_plan_workspace_bytes.restype = ctypes.c_size_t
        lib.rp_plan_copy_items.argtypes = [P, P, ctypes.c_int64]
        lib.rp_plan_copy_items.restype = ctypes.c_int64
        lib.rp_run.argtypes = [P, P, P, P, P, P, ctypes.c_float, P, ctypes.c_size_t, P]
        lib.rp_run.restype = I
        lib.rp_run_noalloc.argtypes = [P, P, P, P, P, P, ctypes.c_float, P]
        lib.rp_run_noalloc.restype = I
        lib.rp_run_paged.argtypes = [P, P, P, P, P, I, I, P, P, ctypes.c_float, P, ctypes.c_size_t, P]
        lib.rp_run_paged.restype = I
        F = ctypes.c_float
        lib.rp_run_fp8kv.argtypes = [P, P, P, P, F, F, P, P, F, P, ctypes.c_size_t, P]
        lib.rp_run_fp8kv.restype = I
        lib.rp_run_paged_fp8kv.argtypes = [P, P, P, P, P, I, I, F, F, P, P, F, P, ctypes.c_size_t, P]
        lib.rp_run_paged_fp8kv.restype = I
        lib.rp_plan_destroy.argtypes = [P]
        lib.rp_plan_destroy.restype = None
        I64 = ctypes.c_int64
        lib.rp_merge_state.argtypes = [P, P, P, P, P, P, I64, I, I, P]
        lib.rp_merge_state.restype = I
        lib.rp_merge_state_in_place.argtypes = [P, P, P, P, I64, I, I, P]
        lib.rp_merge_state_in_place.restype = I
        lib.rp_merge_states.argtypes = [P, P, P, P, I64, I, I, I, P]
        lib.rp_merge_states.restype = I
        lib.rp_plan_create_shared_prefix.argtypes = [P, P, I, I, I, I, I, I,
                                                     ctypes.POINTER(RpPlanOpts), ctypes.POINTER(P)]
        lib.rp_plan_create_shared_prefix.restype = I
        lib.rp_run_shared_prefix.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_float, P,
                                             ctypes.c_size_t, P]
        lib.rp_run_shared_prefix.restype = I
        lib.rp_run_shared_prefix_paged.argtypes = [P, P, P, P, P, P, P, I, I, P, P, ctypes.c_float,
                                                   P, ctypes.c_size_t, P]
        lib.rp_run_shared_prefix_paged.restype = I
        _lib = lib
        return lib


def check(status: int, what: str) -> None:
    if status != RP_OK:
        lib = load()
        detail = lib.rp_last_error().decode(errors="replace")
        raise RaggedPrefillError(status, f"{what}: {detail}")
