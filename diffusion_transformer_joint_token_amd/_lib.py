"""ctypes view of libdit_attn.so (the C ABI declared in include/dit_attn.h).

The library is loaded from this package directory only.  There is no fallback:
if it has not been built, importing the binding raises, so nothing can silently
run another implementation.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdit_attn.so")

# Status codes (dit_attn_status).
OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ALIGN, ERR_DATA, ERR_HIP = range(7)
BF16, F32 = 0, 1
MASK_FULL, MASK_BLOCK_CAUSAL = 0, 1
POS_CENTERED_FHW, POS_GRID_HW = 0, 1
MAX_IMAGES = 64

NORM_RMS_PER_HEAD, NORM_LAYER_ACROSS_HEADS = 0, 1

EXPORTED = ("dit_attn_build_token_metadata", "dit_attn_build_key_valid", "dit_attn_qknorm_rope",
            "dit_attn_qknorm_rope_ex", "dit_attn_time_aware_rope_factors", "dit_attn_forward",
            "dit_attn_forward_cached", "dit_attn_forward_padded", "dit_attn_forward_cached_padded",
            "dit_attn_forward_cached_qnorm", "dit_attn_cfg_norm_rescale", "dit_attn_prescaled_q_factor",
            "dit_attn_status_string")


class TokenMetaStruct(ctypes.Structure):
    _fields_ = [("image_ids", ctypes.c_void_p), ("target_mask", ctypes.c_void_p),
                ("pos_ids", ctypes.c_void_p), ("kv_limit", ctypes.c_void_p), ("seq_len", ctypes.c_int32)]


class NormRopeParams(ctypes.Structure):
    _fields_ = [("norm", ctypes.c_int32), ("q_weight", ctypes.c_void_p), ("k_weight", ctypes.c_void_p),
                ("q_bias", ctypes.c_void_p), ("k_bias", ctypes.c_void_p), ("eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float), ("rope_linear_factor", ctypes.c_float),
                ("rope_ntk_factor", ctypes.c_float), ("q_scale", ctypes.c_float)]


Strides3 = ctypes.c_int64 * 3
i32, i64, vp, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError("libdit_attn.so is not built (%s); run __graft_entry__.build() or "
                          "python diffusion_transformer_joint_token_amd/build.py" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    lib.dit_attn_build_token_metadata.argtypes = [vp, i32, ctypes.POINTER(i32), i32, i32,
                                                  ctypes.POINTER(TokenMetaStruct), vp, vp]
    lib.dit_attn_build_key_valid.argtypes = [vp, i32, vp, i32, i32, i64, vp, i64, vp, vp]
    lib.dit_attn_qknorm_rope.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                         Strides3, Strides3, Strides3, Strides3, vp, i32,
                                         ctypes.POINTER(i32), f32, f32, f32, i32, vp]
    lib.dit_attn_qknorm_rope_ex.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, Strides3, Strides3, Strides3,
                                            Strides3, vp, i32, ctypes.POINTER(i32), ctypes.POINTER(NormRopeParams),
                                            i32, vp]
    lib.dit_attn_time_aware_rope_factors.argtypes = [f32, f32, f32, ctypes.POINTER(f32), ctypes.POINTER(f32)]
    lib.dit_attn_forward.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, Strides3 * 4, i32,
                                     ctypes.POINTER(TokenMetaStruct), f32, i32, vp]
    lib.dit_attn_forward_cached.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                            Strides3 * 6, i32, ctypes.POINTER(TokenMetaStruct), f32, i32, vp]
    lib.dit_attn_forward_padded.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, Strides3 * 4, i32,
                                            ctypes.POINTER(TokenMetaStruct), vp, i64, f32, i32, vp]
    lib.dit_attn_forward_cached_padded.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                                   Strides3 * 6, i32, ctypes.POINTER(TokenMetaStruct), vp, i64,
                                                   f32, i32, vp]
    lib.dit_attn_forward_cached_qnorm.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                                  Strides3 * 6, i32, ctypes.POINTER(TokenMetaStruct), vp, i64, vp,
                                                  i32, ctypes.POINTER(i32), ctypes.POINTER(NormRopeParams), f32, i32,
                                                  vp]
    lib.dit_attn_cfg_norm_rescale.argtypes = [vp, vp, vp, i64, i32, i64, i64, i64, f32, i32, vp]
    lib.dit_attn_prescaled_q_factor.argtypes = [i32, f32, ctypes.POINTER(f32)]
    for name in EXPORTED[:-1]:
        getattr(lib, name).restype = ctypes.c_int
    lib.dit_attn_status_string.argtypes = [i32]
    lib.dit_attn_status_string.restype = ctypes.c_char_p
    return lib


lib = _load()


class DitAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.dit_attn_status_string(status).decode()
        super().__init__("%s: %s (status %d)" % (where, msg, status))


def check(status: int, where: str) -> None:
    if status != OK:
        raise DitAttnError(status, where)
