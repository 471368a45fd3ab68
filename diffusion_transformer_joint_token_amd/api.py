"""Python binding of the C ABI: the same entry points on torch tensors.

Argument marshalling only: every step of the computation runs in the gfx950
kernels of libdit_attn.so.  torch provides device memory and the current HIP
stream; outputs the caller does not pass are allocated with torch.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple, Union

import torch

from . import _lib
from ._lib import DitAttnError, check, lib

__all__ = ["TokenMeta", "KeyValid", "DitAttnError", "LN2", "LOG2E", "prescaled_q_factor",
           "dit_attn_build_token_metadata", "dit_attn_build_key_valid", "dit_attn_qknorm_rope",
           "dit_attn_qknorm_rope_ex", "dit_attn_time_aware_rope_factors", "dit_attn_forward",
           "dit_attn_forward_cached", "dit_attn_forward_padded", "dit_attn_forward_cached_padded",
           "dit_attn_forward_cached_qnorm", "dit_attn_cfg_norm_rescale", "dit_attn_prescaled_q_factor",
           "build_token_metadata", "build_key_valid", "qknorm_rope",
           "time_aware_rope_factors", "forward", "forward_cached", "forward_cached_qnorm", "cfg_norm_rescale"]

_POS = {"centered_fhw": _lib.POS_CENTERED_FHW, "grid_hw": _lib.POS_GRID_HW}

LOG2E = 1.4426950408889634
LN2 = 0.6931471805599453


def prescaled_q_factor(head_dim: int, softmax_scale: Optional[float] = None) -> float:
    """q_scale for dit_attn_qknorm_rope that folds the softmax scale (default
    1/sqrt(head_dim)) and log2(e) into Q; then call the attention with
    softmax_scale=LN2 (dit_attn_prescaled_q_factor)."""
    out = ctypes.c_float()
    check(lib.dit_attn_prescaled_q_factor(int(head_dim), float(softmax_scale or 0.0), ctypes.byref(out)),
          "dit_attn_prescaled_q_factor")
    return out.value


_MASK = {"full": _lib.MASK_FULL, "block_causal": _lib.MASK_BLOCK_CAUSAL}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _lib.BF16
    if t.dtype == torch.float32:
        return _lib.F32
    raise DitAttnError(_lib.ERR_UNSUPPORTED, "dtype %s" % t.dtype)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _bshd_strides(t: torch.Tensor, name: str):
    if t.dim() != 4 or t.stride(3) != 1:
        raise DitAttnError(_lib.ERR_SHAPE, "%s must be [B, S, heads, head_dim] with head_dim contiguous" % name)
    return _lib.Strides3(t.stride(0), t.stride(1), t.stride(2))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


@dataclass
class TokenMeta:
    """Device buffers of the token metadata (one layout for the whole batch)."""
    image_ids: torch.Tensor    # int32 [S]
    target_mask: torch.Tensor  # uint8 [S]
    pos_ids: torch.Tensor      # int32 [S, 3]
    kv_limit: torch.Tensor     # int32 [S]
    status: torch.Tensor       # int32 [1]

    @property
    def seq_len(self) -> int:
        return self.image_ids.numel()

    def struct(self) -> _lib.TokenMetaStruct:
        return _lib.TokenMetaStruct(self.image_ids.data_ptr(), self.target_mask.data_ptr(),
                                    self.pos_ids.data_ptr(), self.kv_limit.data_ptr(), self.seq_len)

    def check(self) -> None:
        """Synchronise with the producing stream and raise on a data error."""
        code = int(self.status.item())
        check(code, "dit_attn_build_token_metadata (device status)")

    @staticmethod
    def empty(seq_len: int, device) -> "TokenMeta":
        return TokenMeta(torch.empty(seq_len, dtype=torch.int32, device=device),
                         torch.empty(seq_len, dtype=torch.uint8, device=device),
                         torch.empty(seq_len, 3, dtype=torch.int32, device=device),
                         torch.empty(seq_len, dtype=torch.int32, device=device),
                         torch.empty(1, dtype=torch.int32, device=device))


def dit_attn_build_token_metadata(image_pad_mask: torch.Tensor, img_shapes: Sequence[Sequence[int]],
                                  pos_mode: Union[str, int] = "centered_fhw", out: Optional[TokenMeta] = None,
                                  stream=None) -> TokenMeta:
    mask = image_pad_mask
    if mask.dtype == torch.bool:
        mask = mask.view(torch.uint8)
    if mask.dtype != torch.uint8 or mask.dim() != 1 or not mask.is_contiguous():
        raise DitAttnError(_lib.ERR_SHAPE, "image_pad_mask must be a contiguous 1-D uint8/bool tensor")
    S = mask.numel()
    meta = out if out is not None else TokenMeta.empty(S, mask.device)
    flat = [int(v) for shp in img_shapes for v in shp]
    if len(flat) != 3 * len(img_shapes):
        raise DitAttnError(_lib.ERR_SHAPE, "img_shapes entries must be (frames, height, width)")
    shapes = (ctypes.c_int32 * max(1, len(flat)))(*flat)
    mode = _POS[pos_mode] if isinstance(pos_mode, str) else int(pos_mode)
    ms = meta.struct()
    st = lib.dit_attn_build_token_metadata(mask.data_ptr(), S, shapes, len(img_shapes), mode, ctypes.byref(ms),
                                           meta.status.data_ptr(), _stream(stream))
    check(st, "dit_attn_build_token_metadata")
    return meta


@dataclass
class KeyValid:
    """Per-sample key validity bits (bit j of word t of row b: key 64 t + j of
    sample b may be attended), stored as int64 words, and the builder's status."""
    bits: torch.Tensor    # int64 [B, words]
    status: torch.Tensor  # int32 [1]

    def check(self) -> None:
        """Synchronise with the producing stream and raise on a data error."""
        check(int(self.status.item()), "dit_attn_build_key_valid (device status)")


def dit_attn_build_key_valid(image_pad_mask: torch.Tensor, text_valid: torch.Tensor,
                             out: Optional[KeyValid] = None, stream=None) -> KeyValid:
    """Key validity of the joint sequence from the text mask (text_valid:
    bool/uint8 [B, n_text], n_text = number of text tokens in the layout)."""
    mask = image_pad_mask.view(torch.uint8) if image_pad_mask.dtype == torch.bool else image_pad_mask
    if mask.dtype != torch.uint8 or mask.dim() != 1 or not mask.is_contiguous():
        raise DitAttnError(_lib.ERR_SHAPE, "image_pad_mask must be a contiguous 1-D uint8/bool tensor")
    tv = text_valid.view(torch.uint8) if text_valid.dtype == torch.bool else text_valid
    if tv.dtype != torch.uint8 or tv.dim() != 2 or (tv.shape[1] > 1 and tv.stride(1) != 1):
        raise DitAttnError(_lib.ERR_SHAPE, "text_valid must be [B, n_text] uint8/bool with unit inner stride")
    S = mask.numel()
    B, n_text = tv.shape
    words = (S + 63) // 64
    kv = out if out is not None else KeyValid(torch.empty(B, max(1, words), dtype=torch.int64, device=mask.device),
                                              torch.empty(1, dtype=torch.int32, device=mask.device))
    if kv.bits.dtype != torch.int64 or kv.bits.dim() != 2 or kv.bits.shape[0] != B or kv.bits.stride(1) != 1:
        raise DitAttnError(_lib.ERR_SHAPE, "key_valid bits must be int64 [B, words] with unit inner stride")
    st = lib.dit_attn_build_key_valid(mask.data_ptr(), S, tv.data_ptr() if n_text else None, B, n_text,
                                      tv.stride(0) if B > 1 else n_text, kv.bits.data_ptr(), kv.bits.stride(0)
                                      if B > 1 else kv.bits.shape[1], kv.status.data_ptr(), _stream(stream))
    check(st, "dit_attn_build_key_valid")
    return kv


def _key_bits(key_valid, B: int, n_keys: int) -> Tuple[int, int]:
    """Pointer and row stride of the key-validity words: one row per sample
    and at least one word per 64 keys of the logical sequence."""
    bits = key_valid.bits if isinstance(key_valid, KeyValid) else key_valid
    if bits.dtype != torch.int64 or bits.dim() != 2 or bits.stride(1) != 1:
        raise DitAttnError(_lib.ERR_SHAPE, "key_valid bits must be int64 [B, words] with unit inner stride")
    if bits.shape[0] != B or bits.shape[1] < (n_keys + 63) // 64:
        raise DitAttnError(_lib.ERR_SHAPE, "key_valid bits must be [%d, >= %d] (one row per sample, one word per "
                           "64 keys)" % (B, (n_keys + 63) // 64))
    if bits.device.type != "cuda":
        raise DitAttnError(_lib.ERR_UNSUPPORTED, "key_valid bits must be in device memory")
    return bits.data_ptr(), bits.stride(0) if bits.shape[0] > 1 else bits.shape[1]


def _out_buffer(out: Optional[torch.Tensor], like: torch.Tensor, name: str) -> torch.Tensor:
    """The caller's output buffer, checked to be exactly the shape and dtype of
    `like` (the C ABI cannot see allocation sizes), or a new one."""
    if out is None:
        return torch.empty_like(like, memory_format=torch.contiguous_format)
    if out.shape != like.shape or out.dtype != like.dtype or out.device != like.device:
        raise DitAttnError(_lib.ERR_SHAPE, "%s must be %s %s on %s like the queries" % (
            name, tuple(like.shape), like.dtype, like.device))
    return out


_NORM = {"rms_per_head": _lib.NORM_RMS_PER_HEAD, "layer_across_heads": _lib.NORM_LAYER_ACROSS_HEADS}


def dit_attn_time_aware_rope_factors(t: float, watershed: float, scaling_factor: float) -> Tuple[float, float]:
    """(linear_factor, ntk_factor) of a denoising step at reversed timestep t."""
    lin, ntk = ctypes.c_float(), ctypes.c_float()
    check(lib.dit_attn_time_aware_rope_factors(float(t), float(watershed), float(scaling_factor), ctypes.byref(lin),
                                               ctypes.byref(ntk)), "dit_attn_time_aware_rope_factors")
    return lin.value, ntk.value


def dit_attn_qknorm_rope(q: torch.Tensor, k: torch.Tensor, pos_ids: torch.Tensor, axes_dims: Sequence[int],
                         eps: float, q_weight: Optional[torch.Tensor] = None,
                         k_weight: Optional[torch.Tensor] = None, rope_theta: float = 10000.0,
                         q_out: Optional[torch.Tensor] = None, k_out: Optional[torch.Tensor] = None,
                         inplace: bool = False, q_scale: float = 1.0,
                         stream=None, norm: str = "rms_per_head", q_bias: Optional[torch.Tensor] = None,
                         k_bias: Optional[torch.Tensor] = None, rope_linear_factor: float = 1.0,
                         rope_ntk_factor: float = 1.0) -> Tuple[torch.Tensor, torch.Tensor]:
    """Q/K norm + rotary embedding.  The defaults call dit_attn_qknorm_rope;
    another norm, a bias or a rotary factor calls dit_attn_qknorm_rope_ex."""
    if inplace:
        q_out, k_out = q, k
    if q_out is None:
        q_out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if k_out is None:
        k_out = torch.empty_like(k, memory_format=torch.contiguous_format)
    B, S, H, D = q.shape
    Hk = k.shape[2]
    if k.shape[0] != B or k.shape[1] != S or k.shape[3] != D or q_out.shape != q.shape or k_out.shape != k.shape:
        raise DitAttnError(_lib.ERR_SHAPE, "q/k/out shapes disagree")
    if pos_ids.dtype != torch.int32 or not pos_ids.is_contiguous() or pos_ids.numel() < 3 * S:
        raise DitAttnError(_lib.ERR_SHAPE, "pos_ids must be contiguous int32 [S, 3]")
    if norm not in _NORM:
        raise DitAttnError(_lib.ERR_UNSUPPORTED, "norm %r" % (norm,))
    across = norm == "layer_across_heads"
    for w, n_ch in ((q_weight, H * D if across else D), (k_weight, Hk * D if across else D),
                    (q_bias, H * D), (k_bias, Hk * D)):
        if w is not None and (w.dtype != q.dtype or w.numel() != n_ch or not w.is_contiguous()):
            raise DitAttnError(_lib.ERR_SHAPE, "norm weight/bias must be contiguous [%d] in the input dtype" % n_ch)
    if not across and (q_bias is not None or k_bias is not None):
        raise DitAttnError(_lib.ERR_UNSUPPORTED, "a bias needs norm='layer_across_heads'")
    dt = _dtype_code(q)
    if k.dtype != q.dtype or q_out.dtype != q.dtype or k_out.dtype != q.dtype:
        raise DitAttnError(_lib.ERR_UNSUPPORTED, "mixed dtypes")
    axes = (ctypes.c_int32 * len(axes_dims))(*[int(a) for a in axes_dims])
    strides = (_bshd_strides(q, "q"), _bshd_strides(k, "k"), _bshd_strides(q_out, "q_out"),
               _bshd_strides(k_out, "k_out"))
    if not across and rope_linear_factor == 1.0 and rope_ntk_factor == 1.0:
        st = lib.dit_attn_qknorm_rope(q.data_ptr(), k.data_ptr(), q_out.data_ptr(), k_out.data_ptr(), _ptr(q_weight),
                                      _ptr(k_weight), B, S, H, Hk, D, *strides, pos_ids.data_ptr(), len(axes_dims),
                                      axes, float(rope_theta), float(eps), float(q_scale), dt, _stream(stream))
        check(st, "dit_attn_qknorm_rope")
        return q_out, k_out
    p = _lib.NormRopeParams(_NORM[norm], _ptr(q_weight), _ptr(k_weight), _ptr(q_bias), _ptr(k_bias), float(eps),
                            float(rope_theta), float(rope_linear_factor), float(rope_ntk_factor), float(q_scale))
    st = lib.dit_attn_qknorm_rope_ex(q.data_ptr(), k.data_ptr(), q_out.data_ptr(), k_out.data_ptr(), B, S, H, Hk, D,
                                     *strides, pos_ids.data_ptr(), len(axes_dims), axes, ctypes.byref(p), dt,
                                     _stream(stream))
    check(st, "dit_attn_qknorm_rope_ex")
    return q_out, k_out


def dit_attn_qknorm_rope_ex(q, k, pos_ids, axes_dims, eps, norm="rms_per_head", q_weight=None, k_weight=None,
                            q_bias=None, k_bias=None, rope_theta=10000.0, rope_linear_factor=1.0, rope_ntk_factor=1.0,
                            q_scale=1.0, q_out=None, k_out=None, inplace=False, stream=None):
    """Always through dit_attn_qknorm_rope_ex (even for the plain options).
    q=None norms K alone and returns (None, k_out): the form that goes with
    dit_attn_forward_cached_qnorm, which norms Q itself."""
    if inplace:
        q_out, k_out = q, k
    if q is not None and q_out is None:
        q_out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if k_out is None:
        k_out = torch.empty_like(k, memory_format=torch.contiguous_format)
    B, S, Hk, D = k.shape
    H = 0 if q is None else q.shape[2]
    if q is not None and (q.shape[0] != B or q.shape[1] != S or q.shape[3] != D or q_out.shape != q.shape):
        raise DitAttnError(_lib.ERR_SHAPE, "q/k/out shapes disagree")
    if k_out.shape != k.shape:
        raise DitAttnError(_lib.ERR_SHAPE, "k_out must match k")
    if pos_ids.dtype != torch.int32 or not pos_ids.is_contiguous() or pos_ids.numel() < 3 * S:
        raise DitAttnError(_lib.ERR_SHAPE, "pos_ids must be contiguous int32 [S, 3]")
    dt = _dtype_code(k)
    axes = (ctypes.c_int32 * len(axes_dims))(*[int(a) for a in axes_dims])
    p = _lib.NormRopeParams(_NORM[norm], _ptr(q_weight), _ptr(k_weight), _ptr(q_bias), _ptr(k_bias), float(eps),
                            float(rope_theta), float(rope_linear_factor), float(rope_ntk_factor), float(q_scale))
    zero = _lib.Strides3(0, 0, 0)
    st = lib.dit_attn_qknorm_rope_ex(_ptr(q), k.data_ptr(), _ptr(q_out), k_out.data_ptr(), B, S, H, Hk, D,
                                     _bshd_strides(q, "q") if q is not None else zero, _bshd_strides(k, "k"),
                                     _bshd_strides(q_out, "q_out") if q is not None else zero,
                                     _bshd_strides(k_out, "k_out"), pos_ids.data_ptr(), len(axes_dims), axes,
                                     ctypes.byref(p), dt, _stream(stream))
    check(st, "dit_attn_qknorm_rope_ex")
    return q_out, k_out


def _lse_buffer(return_lse: bool, lse_out: Optional[torch.Tensor], B: int, H: int, S: int,
                device) -> Optional[torch.Tensor]:
    """The lse output: the caller's fp32 [B, H, S] buffer (contiguous), a new
    one when only return_lse is set, or None."""
    if lse_out is not None:
        if (lse_out.shape != (B, H, S) or lse_out.dtype != torch.float32 or not lse_out.is_contiguous()
                or lse_out.device != torch.device(device)):
            raise DitAttnError(_lib.ERR_SHAPE, "lse_out must be contiguous float32 [%d, %d, %d]" % (B, H, S))
        return lse_out
    return torch.empty(B, H, S, dtype=torch.float32, device=device) if return_lse else None


def dit_attn_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask_mode: Union[str, int] = "full",
                     meta: Optional[TokenMeta] = None, softmax_scale: Optional[float] = None,
                     out: Optional[torch.Tensor] = None, return_lse: bool = False, stream=None,
                     key_valid=None, lse_out: Optional[torch.Tensor] = None):
    """Attention over the joint sequence; with key_valid (a KeyValid or its
    int64 bits [B, words]) padded keys are left out (dit_attn_forward_padded).
    out / lse_out: caller buffers for O ([B, S, H, D]) and the lse (fp32
    [B, H, S]); lse_out implies return_lse."""
    B, S, H, D = q.shape
    Hk = k.shape[2]
    if k.shape != (B, S, Hk, D) or v.shape != (B, S, Hk, D):
        raise DitAttnError(_lib.ERR_SHAPE, "k/v must be [B, S, H_kv, D] matching q")
    o = _out_buffer(out, q, "out")
    return_lse = return_lse or lse_out is not None
    lse = _lse_buffer(return_lse, lse_out, B, H, S, q.device)
    strides = (_lib.Strides3 * 4)(_bshd_strides(q, "q"), _bshd_strides(k, "k"), _bshd_strides(v, "v"),
                                  _bshd_strides(o, "out"))
    dt = _dtype_code(q)
    if any(t.dtype != q.dtype for t in (k, v, o)):
        raise DitAttnError(_lib.ERR_UNSUPPORTED, "mixed dtypes")
    mode = _MASK[mask_mode] if isinstance(mask_mode, str) else int(mask_mode)
    ms = meta.struct() if meta is not None else None
    scale = 0.0 if softmax_scale is None else float(softmax_scale)
    msp = ctypes.byref(ms) if ms is not None else None
    if key_valid is None:
        st = lib.dit_attn_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), _ptr(lse), B, S, H, Hk, D,
                                  strides, mode, msp, scale, dt, _stream(stream))
        check(st, "dit_attn_forward")
    else:
        kb, kbs = _key_bits(key_valid, B, S)
        st = lib.dit_attn_forward_padded(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), _ptr(lse), B, S, H,
                                         Hk, D, strides, mode, msp, kb, kbs, scale, dt, _stream(stream))
        check(st, "dit_attn_forward_padded")
    return (o, lse) if return_lse else o


def dit_attn_forward_cached(q_new: torch.Tensor, k_cache: Optional[torch.Tensor], v_cache: Optional[torch.Tensor],
                            k_new: torch.Tensor, v_new: torch.Tensor, mask_mode: Union[str, int] = "block_causal",
                            meta: Optional[TokenMeta] = None, softmax_scale: Optional[float] = None,
                            out: Optional[torch.Tensor] = None, return_lse: bool = False, stream=None,
                            key_valid=None, lse_out: Optional[torch.Tensor] = None):
    """Attention of the new tokens against cache + new keys; with key_valid
    (bits over the logical sequence) padded keys are left out
    (dit_attn_forward_cached_padded).  out / lse_out as for forward."""
    B, S_new, H, D = q_new.shape
    Hk = k_new.shape[2]
    P = 0 if k_cache is None else k_cache.shape[1]
    if k_new.shape != (B, S_new, Hk, D) or v_new.shape != (B, S_new, Hk, D):
        raise DitAttnError(_lib.ERR_SHAPE, "k_new/v_new must be [B, S_new, H_kv, D]")
    if P > 0 and (k_cache.shape != (B, P, Hk, D) or v_cache is None or v_cache.shape != (B, P, Hk, D)):
        raise DitAttnError(_lib.ERR_SHAPE, "k_cache/v_cache must be [B, P, H_kv, D]")
    o = _out_buffer(out, q_new, "out")
    return_lse = return_lse or lse_out is not None
    lse = _lse_buffer(return_lse, lse_out, B, H, S_new, q_new.device)
    zero = _lib.Strides3(0, 0, 0)
    strides = (_lib.Strides3 * 6)(_bshd_strides(q_new, "q_new"),
                                  _bshd_strides(k_cache, "k_cache") if P > 0 else zero,
                                  _bshd_strides(v_cache, "v_cache") if P > 0 else zero,
                                  _bshd_strides(k_new, "k_new"), _bshd_strides(v_new, "v_new"),
                                  _bshd_strides(o, "out"))
    dt = _dtype_code(q_new)
    mode = _MASK[mask_mode] if isinstance(mask_mode, str) else int(mask_mode)
    ms = meta.struct() if meta is not None else None
    scale = 0.0 if softmax_scale is None else float(softmax_scale)
    msp = ctypes.byref(ms) if ms is not None else None
    kc, vc = (_ptr(k_cache), _ptr(v_cache)) if P > 0 else (None, None)
    if key_valid is None:
        st = lib.dit_attn_forward_cached(q_new.data_ptr(), kc, vc, k_new.data_ptr(), v_new.data_ptr(), o.data_ptr(),
                                         _ptr(lse), B, P, S_new, H, Hk, D, strides, mode, msp, scale, dt,
                                         _stream(stream))
        check(st, "dit_attn_forward_cached")
    else:
        kb, kbs = _key_bits(key_valid, B, P + S_new)
        st = lib.dit_attn_forward_cached_padded(q_new.data_ptr(), kc, vc, k_new.data_ptr(), v_new.data_ptr(),
                                                o.data_ptr(), _ptr(lse), B, P, S_new, H, Hk, D, strides, mode, msp,
                                                kb, kbs, scale, dt, _stream(stream))
        check(st, "dit_attn_forward_cached_padded")
    return (o, lse) if return_lse else o


def dit_attn_forward_padded(q, k, v, key_valid, mask_mode="full", meta=None, softmax_scale=None, out=None,
                            return_lse=False, stream=None, lse_out=None):
    return dit_attn_forward(q, k, v, mask_mode, meta, softmax_scale, out, return_lse, stream, key_valid=key_valid,
                            lse_out=lse_out)


def dit_attn_forward_cached_padded(q_new, k_cache, v_cache, k_new, v_new, key_valid, mask_mode="block_causal",
                                   meta=None, softmax_scale=None, out=None, return_lse=False, stream=None,
                                   lse_out=None):
    return dit_attn_forward_cached(q_new, k_cache, v_cache, k_new, v_new, mask_mode, meta, softmax_scale, out,
                                   return_lse, stream, key_valid=key_valid, lse_out=lse_out)


def dit_attn_forward_cached_qnorm(q_raw: torch.Tensor, k_cache: Optional[torch.Tensor],
                                  v_cache: Optional[torch.Tensor], k_new: torch.Tensor, v_new: torch.Tensor,
                                  pos_ids: torch.Tensor, axes_dims: Sequence[int], eps: float,
                                  q_weight: Optional[torch.Tensor] = None, rope_theta: float = 10000.0,
                                  rope_linear_factor: float = 1.0, rope_ntk_factor: float = 1.0,
                                  q_scale: float = 1.0, mask_mode: Union[str, int] = "block_causal",
                                  meta: Optional[TokenMeta] = None, softmax_scale: Optional[float] = None,
                                  out: Optional[torch.Tensor] = None, return_lse: bool = False, stream=None,
                                  key_valid=None, lse_out: Optional[torch.Tensor] = None):
    """Attention on raw Q: the kernel applies Q's per-head RMSNorm (weight
    q_weight), its rotary embedding (positions pos_ids [S_new, 3] of the query
    tokens, i.e. meta.pos_ids[P:]) and the softmax scale as it loads Q.  K
    must be normed and rotated already (dit_attn_qknorm_rope_ex with q=None).
    k_cache=None is the plain (uncached) form; key_valid as forward_cached."""
    B, S_new, H, D = q_raw.shape
    Hk = k_new.shape[2]
    P = 0 if k_cache is None else k_cache.shape[1]
    if k_new.shape != (B, S_new, Hk, D) or v_new.shape != (B, S_new, Hk, D):
        raise DitAttnError(_lib.ERR_SHAPE, "k_new/v_new must be [B, S_new, H_kv, D]")
    if P > 0 and (k_cache.shape != (B, P, Hk, D) or v_cache is None or v_cache.shape != (B, P, Hk, D)):
        raise DitAttnError(_lib.ERR_SHAPE, "k_cache/v_cache must be [B, P, H_kv, D]")
    if pos_ids.dtype != torch.int32 or not pos_ids.is_contiguous() or pos_ids.numel() < 3 * S_new:
        raise DitAttnError(_lib.ERR_SHAPE, "pos_ids must be contiguous int32 [S_new, 3]")
    if q_weight is not None and (q_weight.dtype != q_raw.dtype or q_weight.numel() != D
                                 or not q_weight.is_contiguous()):
        raise DitAttnError(_lib.ERR_SHAPE, "q_weight must be contiguous [%d] in the input dtype" % D)
    o = _out_buffer(out, q_raw, "out")
    return_lse = return_lse or lse_out is not None
    lse = _lse_buffer(return_lse, lse_out, B, H, S_new, q_raw.device)
    zero = _lib.Strides3(0, 0, 0)
    strides = (_lib.Strides3 * 6)(_bshd_strides(q_raw, "q_raw"),
                                  _bshd_strides(k_cache, "k_cache") if P > 0 else zero,
                                  _bshd_strides(v_cache, "v_cache") if P > 0 else zero,
                                  _bshd_strides(k_new, "k_new"), _bshd_strides(v_new, "v_new"),
                                  _bshd_strides(o, "out"))
    dt = _dtype_code(q_raw)
    if any(t.dtype != q_raw.dtype for t in (k_new, v_new, o)):
        raise DitAttnError(_lib.ERR_UNSUPPORTED, "mixed dtypes")
    mode = _MASK[mask_mode] if isinstance(mask_mode, str) else int(mask_mode)
    ms = meta.struct() if meta is not None else None
    msp = ctypes.byref(ms) if ms is not None else None
    scale = 0.0 if softmax_scale is None else float(softmax_scale)
    kc, vc = (_ptr(k_cache), _ptr(v_cache)) if P > 0 else (None, None)
    kb, kbs = _key_bits(key_valid, B, P + S_new) if key_valid is not None else (None, 0)
    axes = (ctypes.c_int32 * len(axes_dims))(*[int(a) for a in axes_dims])
    p = _lib.NormRopeParams(_lib.NORM_RMS_PER_HEAD, _ptr(q_weight), None, None, None, float(eps), float(rope_theta),
                            float(rope_linear_factor), float(rope_ntk_factor), float(q_scale))
    st = lib.dit_attn_forward_cached_qnorm(q_raw.data_ptr(), kc, vc, k_new.data_ptr(), v_new.data_ptr(),
                                           o.data_ptr(), _ptr(lse), B, P, S_new, H, Hk, D, strides, mode, msp, kb,
                                           kbs, pos_ids.data_ptr(), len(axes_dims), axes, ctypes.byref(p), scale,
                                           dt, _stream(stream))
    check(st, "dit_attn_forward_cached_qnorm")
    return (o, lse) if return_lse else o


def _rows(t: torch.Tensor, name: str) -> Tuple[torch.Tensor, int]:
    """t as [rows, C] with a single row stride (a view), and that stride."""
    if t.dim() < 1 or t.stride(-1) != 1 and t.shape[-1] > 1:
        raise DitAttnError(_lib.ERR_SHAPE, "%s: channels must be contiguous" % name)
    try:
        v = t.view(-1, t.shape[-1])
    except RuntimeError:
        raise DitAttnError(_lib.ERR_SHAPE, "%s: rows must share one stride" % name) from None
    return v, (v.stride(0) if v.shape[0] > 1 else v.shape[1])


def dit_attn_cfg_norm_rescale(cond: torch.Tensor, uncond: torch.Tensor, guidance_scale: float,
                              out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Norm-rescaled classifier-free guidance over the last axis (one row per
    token); out may be cond or uncond (in place)."""
    if uncond.shape != cond.shape:
        raise DitAttnError(_lib.ERR_SHAPE, "cond and uncond shapes differ")
    if out is None:
        out = torch.empty_like(cond, memory_format=torch.contiguous_format)
    if out.shape != cond.shape or any(t.dtype != cond.dtype for t in (uncond, out)):
        raise DitAttnError(_lib.ERR_SHAPE, "out must match cond in shape and dtype")
    c2, cs = _rows(cond, "cond")
    u2, us = _rows(uncond, "uncond")
    o2, os_ = _rows(out, "out")
    st = lib.dit_attn_cfg_norm_rescale(c2.data_ptr(), u2.data_ptr(), o2.data_ptr(), c2.shape[0], c2.shape[1], cs, us,
                                       os_, float(guidance_scale), _dtype_code(cond), _stream(stream))
    check(st, "dit_attn_cfg_norm_rescale")
    return out


dit_attn_prescaled_q_factor = prescaled_q_factor
build_token_metadata = dit_attn_build_token_metadata
cfg_norm_rescale = dit_attn_cfg_norm_rescale
build_key_valid = dit_attn_build_key_valid
time_aware_rope_factors = dit_attn_time_aware_rope_factors
qknorm_rope = dit_attn_qknorm_rope
forward = dit_attn_forward
forward_cached = dit_attn_forward_cached
forward_cached_qnorm = dit_attn_forward_cached_qnorm
