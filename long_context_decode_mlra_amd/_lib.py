"""ctypes view of libmlra.so (include/mlra.h). Loading fails loudly if the library is missing."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmlra.so")

MLRA_BF16 = 0
MLRA_F32 = 1
MLRA_TILE_TOKENS = 32
MLRA_MAX_HEADS = 64
MLRA_NOALLOC_SCRATCH_BYTES = 64 << 20
ABI_VERSION = 1

ERRORS = {0: "MLRA_OK", -1: "MLRA_ERR_NULL", -2: "MLRA_ERR_SHAPE", -3: "MLRA_ERR_UNSUPPORTED",
          -4: "MLRA_ERR_ALIGN", -5: "MLRA_ERR_WORKSPACE", -6: "MLRA_ERR_HIP"}

# Every symbol include/mlra.h declares.
EXPORTS = ("mlra_abi_version", "mlra_last_error", "mlra_check_params", "mlra_decode_num_splits",
           "mlra_decode_workspace_size", "mlra_decode", "mlra_decode_noalloc", "mlra_decode_splitkv",
           "mlra_decode_combine",
           "mlra_decode_plan", "mlra_copy_bandwidth_probe", "mlra_read_bandwidth_probe", "mlra_absorb_query",
           "mlra_gqa_check_params", "mlra_gqa_num_splits", "mlra_gqa_workspace_size", "mlra_gqa_decode")


class DecodeParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("num_branches", ctypes.c_int32),
        ("d_latent", ctypes.c_int32), ("d_rope", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("page_size", ctypes.c_int32), ("max_seqlen", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32), ("num_splits", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("q_stride_b", ctypes.c_int64), ("q_stride_h", ctypes.c_int64),
        ("qr_stride_b", ctypes.c_int64), ("qr_stride_h", ctypes.c_int64),
        ("lat_stride_tok", ctypes.c_int64), ("rope_stride_tok", ctypes.c_int64),
        ("sm_scale", ctypes.c_float), ("out_scale", ctypes.c_float),
    ]


class GqaParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("max_seqlen", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32), ("num_splits", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("q_stride_b", ctypes.c_int64), ("q_stride_h", ctypes.c_int64),
        ("k_stride_tok", ctypes.c_int64), ("k_stride_head", ctypes.c_int64),
        ("v_stride_tok", ctypes.c_int64), ("v_stride_head", ctypes.c_int64),
        ("sm_scale", ctypes.c_float), ("reserved_f", ctypes.c_float),
    ]


class MlraError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{ERRORS.get(code, code)}: {message}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first with "
                          f"`python -m long_context_decode_mlra_amd.build` (needs ROCm hipcc)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    P = ctypes.POINTER(DecodeParams)
    L.mlra_abi_version.restype = ctypes.c_int
    L.mlra_last_error.restype = ctypes.c_char_p
    L.mlra_check_params.argtypes = [P]
    L.mlra_decode_num_splits.argtypes = [P, ctypes.POINTER(i32)]
    L.mlra_decode_workspace_size.argtypes = [P, ctypes.POINTER(sz)]
    L.mlra_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, P, vp, sz, vp]
    L.mlra_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, P, vp]
    L.mlra_decode_splitkv.argtypes = [vp, vp, vp, vp, vp, vp, P, vp, sz, vp]
    L.mlra_decode_combine.argtypes = [vp, vp, vp, P, vp, sz, vp]
    L.mlra_decode_plan.argtypes = [vp, i32, i32, i32, vp, vp]
    L.mlra_copy_bandwidth_probe.argtypes = [vp, vp, sz, vp]
    L.mlra_read_bandwidth_probe.argtypes = [vp, sz, vp, vp]
    i64 = ctypes.c_int64
    L.mlra_absorb_query.argtypes = [vp, vp, vp, P, i32, i64, i64, i64, vp]
    GP = ctypes.POINTER(GqaParams)
    L.mlra_gqa_check_params.argtypes = [GP]
    L.mlra_gqa_num_splits.argtypes = [GP, ctypes.POINTER(i32)]
    L.mlra_gqa_workspace_size.argtypes = [GP, ctypes.POINTER(sz)]
    L.mlra_gqa_decode.argtypes = [vp, vp, vp, vp, vp, vp, GP, vp, sz, vp]
    for name in EXPORTS:
        if name not in ("mlra_last_error", "mlra_abi_version"):
            getattr(L, name).restype = ctypes.c_int
    if L.mlra_abi_version() != ABI_VERSION:
        raise ImportError(f"libmlra.so ABI {L.mlra_abi_version()} != binding ABI {ABI_VERSION}")
    _lib = L
    return L


def check(code: int) -> None:
    if code != 0:
        raise MlraError(code, lib().mlra_last_error().decode(errors="replace"))
