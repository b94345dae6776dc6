"""ctypes view of include/kda.h (libkda_mi355x.so).

Argument marshalling only: the structs mirror the C declarations field for
field, and every entry point returns the C status, turned into an exception
by the facade.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkda_mi355x.so")

KDA_OK = 0
STATUS = {
    0: "KDA_OK", -1: "KDA_ERR_NULLPTR", -2: "KDA_ERR_SHAPE", -3: "KDA_ERR_DTYPE",
    -4: "KDA_ERR_STRIDE", -5: "KDA_ERR_ALIGN", -6: "KDA_ERR_ALIAS", -7: "KDA_ERR_UNSUPPORTED",
    -8: "KDA_ERR_DEVICE", -9: "KDA_ERR_LAUNCH", -10: "KDA_ERR_ABI",
}
DTYPE_F32, DTYPE_BF16 = 0, 1
GATE_SOFTPLUS, GATE_LOWER_BOUND, GATE_PRECOMPUTED = 0, 1, 2
FLAG_NO_STATE_UPDATE = 1

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_U32 = ctypes.c_uint32
_I64 = ctypes.c_int64
_F32 = ctypes.c_float


class LaunchPlan(ctypes.Structure):
    _fields_ = [("struct_size", _U32), ("kernel", _I32), ("grid_x", _I32), ("block", _I32),
                ("rows_per_block", _I32), ("vsplit", _I32), ("items", _I64)]


class RecurrentArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", _U32), ("n_seqs", _I32), ("n_tokens", _I32), ("H", _I32), ("HV", _I32),
        ("K", _I32), ("V", _I32),
        ("q", _P), ("k", _P), ("v", _P), ("g", _P), ("beta", _P),
        ("q_stride", _I64), ("k_stride", _I64), ("v_stride", _I64), ("g_stride", _I64),
        ("beta_stride", _I64),
        ("A_log", _P), ("dt_bias", _P), ("scale", _F32), ("l2_eps", _F32),
        ("gate_mode", _I32), ("lower_bound", _F32),
        ("state", _P), ("state_dtype", _I32), ("ckpt_dtype", _I32), ("num_slots", _I64),
        ("slot_stride", _I64), ("state_indices", _P), ("cu_seqlens", _P), ("checkpoints", _P),
        ("out", _P), ("g_dtype", _I32), ("beta_dtype", _I32), ("tokens_per_seq", _I32),
        ("flags", _U32), ("correction_cache", _P), ("kg_cache", _P), ("kg_dtype", _I32),
        ("cache_t_max", _I32),
    ]


class PackedArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", _U32), ("B", _I32), ("H", _I32),
        ("mixed_qkv", _P), ("qkv_stride", _I64), ("raw_gate", _P), ("gate_stride", _I64),
        ("raw_beta", _P), ("beta_stride", _I64), ("A_log", _P), ("dt_bias", _P),
        ("gate_mode", _I32), ("lower_bound", _F32),
        ("state", _P), ("state_dtype", _I32), ("num_slots", _I64), ("slot_stride", _I64),
        ("state_indices", _P), ("out", _P),
    ]


class FusedArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", _U32), ("rows", _I32), ("H", _I32),
        ("x", _P), ("x_stride", _I64), ("weight", _P), ("conv_state", _P),
        ("conv_slot_stride", _I64), ("raw_gate", _P), ("gate_stride", _I64), ("raw_beta", _P),
        ("beta_stride", _I64), ("A_log", _P), ("dt_bias", _P), ("gate_mode", _I32),
        ("lower_bound", _F32), ("state_indices", _P), ("state", _P), ("state_dtype", _I32),
        ("num_slots", _I64), ("slot_stride", _I64), ("output_gate", _P), ("ogate_stride", _I64),
        ("norm_weight", _P), ("norm_eps", _F32), ("out", _P),
    ]


class PackedFusedArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", _U32), ("n_rows", _I32), ("n_seqs", _I32), ("H", _I32), ("max_tokens", _I32),
        ("x", _P), ("x_stride", _I64), ("weight", _P), ("conv_state", _P),
        ("conv_slot_stride", _I64), ("raw_gate", _P), ("gate_stride", _I64), ("raw_beta", _P),
        ("beta_stride", _I64), ("A_log", _P), ("dt_bias", _P), ("gate_mode", _I32),
        ("lower_bound", _F32), ("state_indices", _P), ("indices_stride", _I64),
        ("query_start_loc", _P), ("num_accepted_tokens", _P), ("state", _P), ("state_dtype", _I32),
        ("num_slots", _I64), ("slot_stride", _I64), ("output_gate", _P), ("ogate_stride", _I64),
        ("norm_weight", _P), ("norm_eps", _F32), ("out", _P), ("split_counters", _P),
        ("split_partials", _P),
    ]


EXPORTS = ["kda_recurrent", "kda_packed_decode", "kda_fused_decode", "kda_packed_fused_decode",
           "kda_packed_fused_decode_noalloc", "kda_packed_fused_workspace",
           "kda_recurrent_plan", "kda_packed_plan", "kda_fused_plan", "kda_packed_fused_plan",
           "kda_status_string", "kda_last_error", "kda_version", "kda_check_device"]

_lib = None


def load(path: str = LIB_PATH):
    """Load the built library (never builds; build with __graft_entry__.build()
    or ``python -m gated_delta_rule_decode_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: the KDA decode library has not been built "
            "(run __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(path)
    for name, argt in (("kda_recurrent", [ctypes.POINTER(RecurrentArgs), _P]),
                       ("kda_packed_decode", [ctypes.POINTER(PackedArgs), _P]),
                       ("kda_fused_decode", [ctypes.POINTER(FusedArgs), _P]),
                       ("kda_recurrent_plan", [ctypes.POINTER(RecurrentArgs), ctypes.POINTER(LaunchPlan)]),
                       ("kda_packed_plan", [ctypes.POINTER(PackedArgs), ctypes.POINTER(LaunchPlan)]),
                       ("kda_fused_plan", [ctypes.POINTER(FusedArgs), ctypes.POINTER(LaunchPlan)]),
                       ("kda_packed_fused_decode", [ctypes.POINTER(PackedFusedArgs), _P]),
                       ("kda_packed_fused_decode_noalloc", [ctypes.POINTER(PackedFusedArgs), _P]),
                       ("kda_packed_fused_plan", [ctypes.POINTER(PackedFusedArgs), ctypes.POINTER(LaunchPlan)]),
                       ("kda_check_device", [ctypes.c_int])):
        fn = getattr(lib, name)
        fn.argtypes = argt
        fn.restype = ctypes.c_int
    lib.kda_packed_fused_workspace.argtypes = [ctypes.POINTER(PackedFusedArgs), ctypes.POINTER(_I64),
                                               ctypes.POINTER(_I64)]
    lib.kda_packed_fused_workspace.restype = ctypes.c_int
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_last_error.argtypes = []
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_version.argtypes = []
    lib.kda_version.restype = ctypes.c_int
    _lib = lib
    return lib


class KDAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.code = STATUS.get(status, str(status))
        super().__init__(f"{self.code}: {detail}")


def check(status: int):
    if status != KDA_OK:
        lib = load()
        raise KDAError(status, lib.kda_last_error().decode(errors="replace"))
