"""ctypes declarations of libpmk.so (the C ABI of include/pmk.h), one Python name per C name.

Argument marshalling only: every step of the decode path runs in the library's kernels.
Loading fails loudly when the library is missing; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpmk.so")

PMK_OK = 0
PMK_ERR_INVALID_ARG = 1
PMK_ERR_UNSUPPORTED = 2
PMK_ERR_SCHEDULE_INVALID = 3
PMK_ERR_CAPACITY = 4
PMK_ERR_NOT_BOUND = 5
PMK_ERR_HIP = 6
PMK_ERR_TIMEOUT = 7
PMK_ERR_NAN = 8
PMK_ERR_DEVICE = 9

PMK_DT_F16, PMK_DT_BF16, PMK_DT_FP8_E4M3, PMK_DT_INT8, PMK_DT_INT4 = 0, 1, 2, 3, 4
PMK_MODE_MEGAKERNEL, PMK_MODE_GRAPH, PMK_MODE_PER_OP = 0, 1, 2
PMK_SYNC_FLAGS, PMK_SYNC_COUNTERS = 0, 1
PMK_OP_QKV, PMK_OP_ATTN, PMK_OP_OPROJ, PMK_OP_GATEUP, PMK_OP_DOWN, PMK_OP_LMHEAD, PMK_OP_TOKEN = range(1, 8)
PMK_OP_COMBINE = 8

i32, i64, u64, f32, vp, sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float, ctypes.c_void_p,
                              ctypes.c_size_t)


class pmk_model_config(ctypes.Structure):
    _fields_ = [("n_layers", i32), ("hidden", i32), ("n_q_heads", i32), ("n_kv_heads", i32), ("head_dim", i32),
                ("ffn", i32), ("vocab", i32), ("max_seq", i32), ("rms_eps", f32), ("rope_theta", f32),
                ("weight_dtype", i32), ("kv_dtype", i32), ("has_bias", i32), ("tie_embeddings", i32)]


class pmk_schedule_config(ctypes.Structure):
    _fields_ = [("n_cus", i32), ("sync_mode", i32), ("attn_splits", i32), ("prefetch", i32), ("trace_steps", i32),
                ("spin_limit", i64), ("combine_parts", i32), ("combine_o_share", i32), ("prefill_chunk", i32), ("prefill_ksplit", i32), ("combine_o_copy", i32),
                ("reserved", i32 * 3)]


class pmk_sizes(ctypes.Structure):
    _fields_ = [("arena_bytes", u64), ("kv_bytes", u64), ("workspace_bytes", u64)]


class pmk_weight_ptrs(ctypes.Structure):
    _fields_ = [("embed", vp), ("final_norm", vp), ("lm_head", vp), ("lm_head_scale", vp),
                ("layers", ctypes.POINTER(vp)), ("layer_scales", ctypes.POINTER(vp))]


class pmk_device_error(ctypes.Structure):
    _fields_ = [("code", i32), ("cu", i32), ("task", i32), ("counter", i32), ("expected", ctypes.c_uint32),
                ("seen", ctypes.c_uint32)]


class pmk_schedule_info(ctypes.Structure):
    _fields_ = [("n_tasks", i32), ("n_counters", i32), ("n_cus", i32), ("attn_splits", i32),
                ("max_tasks_per_cu", i32), ("sync_mode", i32), ("hash", u64)]


class pmk_tune_result(ctypes.Structure):
    _fields_ = [("tried", i32), ("kept", i32), ("gate_rejected", i32), ("invalid", i32), ("us_before", ctypes.c_double),
                ("us_after", ctypes.c_double), ("chosen", pmk_schedule_config), ("desc", ctypes.c_char * 232)]


class pmk_task(ctypes.Structure):
    _fields_ = [("op", i32), ("layer", i32), ("a0", i32), ("a1", i32), ("wait_ctr", i32), ("wait_count", i32),
                ("wait_lag", i32), ("signal_ctr", i32), ("signal_slot", i32)]


# name -> (restype, argtypes)
SIGNATURES = {
    "pmk_abi_version": (ctypes.c_int, []),
    "pmk_status_str": (ctypes.c_char_p, [i32]),
    "pmk_last_error": (ctypes.c_char_p, [vp]),
    "pmk_last_global_error": (ctypes.c_char_p, []),
    "pmk_create": (i32, [ctypes.POINTER(pmk_model_config), ctypes.POINTER(pmk_schedule_config), ctypes.c_int,
                         ctypes.POINTER(vp)]),
    "pmk_destroy": (None, [vp]),
    "pmk_buffer_sizes": (i32, [vp, ctypes.POINTER(pmk_sizes)]),
    "pmk_bind": (i32, [vp, vp, vp, vp]),
    "pmk_bind_static_workspace": (i32, [vp, vp, vp]),
    "pmk_load_weights": (i32, [vp, ctypes.POINTER(pmk_weight_ptrs), vp]),
    "pmk_prefill_kv": (i32, [vp, vp, i32, vp, vp, vp]),
    "pmk_get_kv_scales": (i32, [vp, vp, vp]),
    "pmk_read_kv": (i32, [vp, vp, vp, i32, vp]),
    "pmk_load_kv": (i32, [vp, vp, vp, i32, i32, vp, vp]),
    "pmk_rewind": (i32, [vp, i32, vp, vp]),
    "pmk_decode_n_tokens": (i32, [vp, i32, vp, vp, i32, vp, vp]),
    "pmk_set_mode": (i32, [vp, i32]),
    "pmk_get_position": (i32, [vp, ctypes.POINTER(i32)]),
    "pmk_poll_error": (i32, [vp, ctypes.POINTER(pmk_device_error)]),
    "pmk_set_trace": (i32, [vp, i32]),
    "pmk_tune": (i32, [vp, i32, ctypes.POINTER(pmk_tune_result), vp]),
    "pmk_trace_export": (i32, [vp, ctypes.c_char_p]),
    "pmk_trace_stats": (i32, [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]),
    "pmk_schedule_get_info": (i32, [vp, ctypes.POINTER(pmk_schedule_info)]),
    "pmk_schedule_build": (i32, [ctypes.POINTER(pmk_model_config), ctypes.POINTER(pmk_schedule_config), i32,
                                 ctypes.POINTER(vp)]),
    "pmk_schedule_build_weighted": (i32, [ctypes.POINTER(pmk_model_config), ctypes.POINTER(pmk_schedule_config), i32,
                                          ctypes.POINTER(f32), ctypes.POINTER(vp)]),
    "pmk_schedule_free": (None, [vp]),
    "pmk_schedule_num_tasks": (i32, [vp]),
    "pmk_schedule_num_counters": (i32, [vp]),
    "pmk_schedule_num_queues": (i32, [vp]),
    "pmk_schedule_get_task": (i32, [vp, i32, ctypes.POINTER(pmk_task)]),
    "pmk_schedule_set_task": (i32, [vp, i32, ctypes.POINTER(pmk_task)]),
    "pmk_schedule_queue": (ctypes.POINTER(i32), [vp, i32, ctypes.POINTER(i32)]),
    "pmk_schedule_set_queue": (i32, [vp, i32, ctypes.POINTER(i32), i32]),
    "pmk_schedule_counter_producers": (i32, [vp, i32]),
    "pmk_schedule_set_counter_producers": (i32, [vp, i32, i32]),
    "pmk_schedule_validate": (i32, [vp, ctypes.c_char_p, sz]),
    "pmk_schedule_simulate": (i32, [vp, i32, u64, ctypes.c_char_p, sz]),
    "pmk_schedule_hash": (u64, [vp]),
}

_lib = None


class PmkError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"pmk status {status}: {msg}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libpmk.so (built in-tree by build()); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with persistent_megakernel_02_amd.build.build()")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(status: int, ctx=None) -> None:
    if status != PMK_OK:
        lib = load()
        msg = (lib.pmk_last_error(ctx) if ctx else lib.pmk_last_global_error()) or b""
        raise PmkError(status, f"{lib.pmk_status_str(status).decode()}: {msg.decode()}")
