"""ctypes mirror of include/kda_recoverssm.h and the loader of the in-tree
`libkda_recoverssm.so`.  Marshalling only: no computation happens here."""
from __future__ import annotations

import ctypes
import os
from ctypes import (POINTER, Structure, c_char_p, c_float, c_int, c_int32,
                    c_int64, c_void_p)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "libkda_recoverssm.so")

KDA_OK = 0
KDA_E_SHAPE = 1
KDA_E_DTYPE = 2
KDA_E_LAYOUT = 3
KDA_E_UNALIGNED = 4
KDA_E_UNSUPPORTED = 5
KDA_E_CAPACITY = 6
KDA_E_DEVICE = 7
KDA_E_ARG = 8

KDA_SCHEDULE_DEFAULT = 0
KDA_SCHEDULE_PER_ITEM = 1
KDA_SCHEDULE_TICKETS = 2
KDA_SCHEDULE_V_TILES = 3

KDA_F32 = 0
KDA_BF16 = 1

EXPORTED = (
    "kda_abi_version", "kda_last_error", "kda_status_string",
    "kda_check_verify", "kda_conv_update_verify",
    "kda_conv_update_verify_noalloc", "kda_check_verify_qkv",
    "kda_recoverssm_verify_qkv", "kda_check_commit",
    "kda_recoverssm_commit", "kda_check_commit_plan", "kda_commit_plan",
    "kda_check_compact_conv", "kda_compact_conv_state",
    "kda_check_commit_step", "kda_recoverssm_commit_step",
    "kda_reset_counter", "kda_set_launch_events",
)


class KdaTensor(Structure):
    _fields_ = [("data", c_void_p), ("dtype", c_int32), ("ndim", c_int32),
                ("shape", c_int64 * 4), ("stride", c_int64 * 4)]


class KdaVerifyArgs(Structure):
    _fields_ = [
        ("mixed_qkv", KdaTensor), ("raw_gate", KdaTensor),
        ("raw_beta", KdaTensor), ("A_log", KdaTensor),
        ("dt_bias", KdaTensor), ("state", KdaTensor),
        ("correction", KdaTensor), ("key_gate", KdaTensor),
        ("out", KdaTensor), ("conv_state", KdaTensor),
        ("conv_weight", KdaTensor),
        ("query_start_loc", c_void_p), ("state_indices", c_void_p),
        ("num_accepted_tokens", c_void_p), ("record_rows", c_void_p),
        ("work_counter", c_void_p),
        ("batch", c_int32), ("spec_query_len", c_int32),
        ("null_block_id", c_int32), ("conv_dim_first", c_int32),
        ("use_lower_bound", c_int32), ("lower_bound", c_float),
        ("max_workgroups", c_int32), ("items_per_ticket", c_int32),
        ("schedule", c_int32),
        ("pending_lens", c_void_p),
        ("work_counter_len", c_int32), ("v_tiles", c_int32),
    ]


class KdaCommitArgs(Structure):
    _fields_ = [
        ("num_layers", c_int32), ("batch", c_int32), ("num_heads", c_int32),
        ("head_dim", c_int32), ("spec_query_len", c_int32),
        ("null_block_id", c_int32),
        ("num_slots", c_int64), ("num_record_rows", c_int64),
        ("state_base_addrs", c_void_p), ("state_block_strides", c_void_p),
        ("correction_base_addrs", c_void_p),
        ("correction_block_strides", c_void_p),
        ("key_gate_base_addrs", c_void_p),
        ("key_gate_block_strides", c_void_p),
        ("state_strides", c_int64 * 2), ("correction_strides", c_int64 * 2),
        ("key_gate_strides", c_int64 * 2),
        ("key_gate_dtype", c_int32), ("max_workgroups", c_int32),
        ("A_log", c_void_p), ("A_log_strides", c_int64 * 2),
        ("dt_bias", c_void_p), ("dt_bias_strides", c_int64 * 3),
        ("use_lower_bound", c_void_p), ("lower_bound", c_void_p),
        ("state_indices", c_void_p), ("commit_lens", c_void_p),
        ("final_state_indices", c_void_p), ("record_rows", c_void_p),
        ("host_tables", POINTER(c_int64)),
        ("boundary_state_indices", c_void_p),
        ("boundary_recovery_lens", c_void_p),
    ]


class KdaPlanArgs(Structure):
    _fields_ = [
        ("batch", c_int32), ("spec_query_len", c_int32),
        ("null_block_id", c_int32), ("mamba_block_size", c_int32),
        ("num_request_rows", c_int32), ("block_table_width", c_int32),
        ("block_table_strides", c_int64 * 2),
        ("num_accepted_tokens", c_void_p), ("request_indices", c_void_p),
        ("state_indices", c_void_p), ("query_start_loc", c_void_p),
        ("block_table", c_void_p), ("num_computed_tokens", c_void_p),
        ("commit_lens", c_void_p), ("final_state_indices", c_void_p),
        ("boundary_state_indices", c_void_p),
        ("boundary_recovery_lens", c_void_p),
    ]


class KdaCompactArgs(Structure):
    _fields_ = [
        ("num_layers", c_int32), ("batch", c_int32),
        ("spec_query_len", c_int32), ("null_block_id", c_int32),
        ("num_slots", c_int64), ("conv_dim", c_int64),
        ("conv_dtype", c_int32), ("pad_", c_int32),
        ("conv_tables", c_void_p), ("host_conv_tables", POINTER(c_int64)),
        ("state_indices", c_void_p), ("commit_lens", c_void_p),
        ("final_state_indices", c_void_p),
        ("boundary_state_indices", c_void_p),
        ("boundary_recovery_lens", c_void_p),
    ]


_LIB = None


def load() -> ctypes.CDLL:
    """Load the in-tree library; fails loudly when it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m linear_attention_speculative_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.kda_abi_version.restype = c_int
    lib.kda_abi_version.argtypes = []
    lib.kda_last_error.restype = c_char_p
    lib.kda_last_error.argtypes = []
    lib.kda_status_string.restype = c_char_p
    lib.kda_status_string.argtypes = [c_int]
    lib.kda_check_verify.restype = c_int
    lib.kda_check_verify.argtypes = [POINTER(KdaVerifyArgs)]
    lib.kda_conv_update_verify.restype = c_int
    lib.kda_conv_update_verify.argtypes = [POINTER(KdaVerifyArgs), c_void_p]
    lib.kda_conv_update_verify_noalloc.restype = c_int
    lib.kda_conv_update_verify_noalloc.argtypes = [POINTER(KdaVerifyArgs),
                                                   c_void_p]
    lib.kda_check_verify_qkv.restype = c_int
    lib.kda_check_verify_qkv.argtypes = [POINTER(KdaVerifyArgs)]
    lib.kda_recoverssm_verify_qkv.restype = c_int
    lib.kda_recoverssm_verify_qkv.argtypes = [POINTER(KdaVerifyArgs),
                                              c_void_p]
    lib.kda_check_commit.restype = c_int
    lib.kda_check_commit.argtypes = [POINTER(KdaCommitArgs)]
    lib.kda_recoverssm_commit.restype = c_int
    lib.kda_recoverssm_commit.argtypes = [POINTER(KdaCommitArgs), c_void_p]
    lib.kda_check_commit_plan.restype = c_int
    lib.kda_check_commit_plan.argtypes = [POINTER(KdaPlanArgs)]
    lib.kda_commit_plan.restype = c_int
    lib.kda_commit_plan.argtypes = [POINTER(KdaPlanArgs), c_void_p]
    lib.kda_check_compact_conv.restype = c_int
    lib.kda_check_compact_conv.argtypes = [POINTER(KdaCompactArgs)]
    lib.kda_compact_conv_state.restype = c_int
    lib.kda_compact_conv_state.argtypes = [POINTER(KdaCompactArgs), c_void_p]
    lib.kda_check_commit_step.restype = c_int
    lib.kda_check_commit_step.argtypes = [POINTER(KdaCommitArgs),
                                          POINTER(KdaPlanArgs),
                                          POINTER(KdaCompactArgs)]
    lib.kda_recoverssm_commit_step.restype = c_int
    lib.kda_recoverssm_commit_step.argtypes = [POINTER(KdaCommitArgs),
                                               POINTER(KdaPlanArgs),
                                               POINTER(KdaCompactArgs),
                                               c_void_p]
    lib.kda_reset_counter.restype = c_int
    lib.kda_reset_counter.argtypes = [c_void_p, c_int32, c_void_p]
    lib.kda_set_launch_events.restype = c_int
    lib.kda_set_launch_events.argtypes = [c_void_p, c_void_p, c_int32,
                                          POINTER(c_int32)]
    _LIB = lib
    return lib
