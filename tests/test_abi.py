"""The C-ABI library loads, exports what include/dit_attn.h declares, and
rejects bad arguments on the host before touching a device (CPU only: every
call here fails validation, so nothing is enqueued)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dit_attn.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char \*)\s*(dit_attn_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    from diffusion_transformer_joint_token_amd import _lib
    names = declared_functions()
    assert names == sorted(_lib.EXPORTED)
    for name in names:
        assert hasattr(_lib.lib, name), name
    out = os.popen("nm -D --defined-only %s" % _lib.LIB_PATH).read()
    for name in names:
        assert re.search(r"\bT %s$" % name, out, re.M), name


def test_status_strings():
    from diffusion_transformer_joint_token_amd import _lib
    for code in range(7):
        assert _lib.lib.dit_attn_status_string(code)
    assert _lib.lib.dit_attn_status_string(99) == b"unknown status"


FAKE = 0x100000  # 16-byte aligned, never dereferenced: validation fails first
FAKE2 = 0x200000


def _meta(seq_len, ptr=FAKE):
    from diffusion_transformer_joint_token_amd import _lib
    return _lib.TokenMetaStruct(ptr, ptr, ptr, ptr, seq_len)


def test_metadata_argument_errors():
    from diffusion_transformer_joint_token_amd import _lib
    lib = _lib.lib
    m = _meta(16)
    shapes = (ctypes.c_int32 * 3)(1, 4, 4)
    f = lib.dit_attn_build_token_metadata
    assert f(None, 16, shapes, 1, 0, ctypes.byref(m), FAKE, None) == _lib.ERR_NULL
    assert f(FAKE, 16, shapes, 1, 0, None, FAKE, None) == _lib.ERR_NULL
    assert f(FAKE, 16, shapes, 1, 0, ctypes.byref(m), None, None) == _lib.ERR_NULL
    assert f(FAKE, 17, shapes, 1, 0, ctypes.byref(m), FAKE, None) == _lib.ERR_SHAPE       # seq_len mismatch
    assert f(FAKE, 16, shapes, 65, 0, ctypes.byref(m), FAKE, None) == _lib.ERR_SHAPE      # too many images
    assert f(FAKE, 16, shapes, 1, 7, ctypes.byref(m), FAKE, None) == _lib.ERR_UNSUPPORTED  # pos mode
    odd = (ctypes.c_int32 * 3)(1, 3, 4)
    assert f(FAKE, 16, odd, 1, 0, ctypes.byref(m), FAKE, None) == _lib.ERR_SHAPE          # odd H, centred
    frames = (ctypes.c_int32 * 3)(2, 2, 2)
    assert f(FAKE, 16, frames, 1, 1, ctypes.byref(m), FAKE, None) == _lib.ERR_SHAPE       # 2 frames, 2D grid
    big = (ctypes.c_int32 * 6)(1, 4, 4, 1, 2, 2)
    assert f(FAKE, 16, big, 2, 0, ctypes.byref(m), FAKE, None) == _lib.ERR_SHAPE          # 20 image tokens > 16
    zero = (ctypes.c_int32 * 3)(1, 0, 4)
    assert f(FAKE, 16, zero, 1, 0, ctypes.byref(m), FAKE, None) == _lib.ERR_SHAPE


def _s3(*v):
    from diffusion_transformer_joint_token_amd import _lib
    return _lib.Strides3(*v)


def test_qknorm_rope_argument_errors():
    from diffusion_transformer_joint_token_amd import _lib
    f = _lib.lib.dit_attn_qknorm_rope
    st = _s3(5120 * 4096, 4096, 128)
    axes = (ctypes.c_int32 * 3)(16, 56, 56)

    def call(q=FAKE, D=128, axes_arr=axes, n_axes=3, dtype=0, strides=st, theta=1e4, eps=1e-6, H=32, Hk=32,
             q_scale=1.0):
        return f(q, FAKE, FAKE2, FAKE2, None, None, 2, 5120, H, Hk, D, strides, strides, strides, strides, FAKE,
                 n_axes, axes_arr, theta, eps, q_scale, dtype, None)
    assert call(q=None) == _lib.ERR_NULL
    assert call(dtype=5) == _lib.ERR_UNSUPPORTED
    assert call(D=136) == _lib.ERR_UNSUPPORTED
    assert call(D=100) == _lib.ERR_UNSUPPORTED           # not a multiple of 8 (bf16)
    assert call(axes_arr=(ctypes.c_int32 * 3)(16, 56, 54)) == _lib.ERR_SHAPE   # sums to 126
    assert call(axes_arr=(ctypes.c_int32 * 3)(15, 57, 56)) == _lib.ERR_SHAPE   # odd axis
    assert call(n_axes=4) == _lib.ERR_SHAPE
    assert call(theta=0.0) == _lib.ERR_SHAPE
    assert call(eps=-1.0) == _lib.ERR_SHAPE
    assert call(q_scale=0.0) == _lib.ERR_SHAPE
    assert call(q_scale=float("inf")) == _lib.ERR_SHAPE
    assert call(H=0) == _lib.ERR_SHAPE
    assert call(q=FAKE + 2) == _lib.ERR_ALIGN
    assert call(strides=_s3(5120 * 4096, 4096, 132)) == _lib.ERR_ALIGN   # head stride 264 B


def test_attention_argument_errors():
    from diffusion_transformer_joint_token_amd import _lib
    f = _lib.lib.dit_attn_forward
    st4 = (_lib.Strides3 * 4)(*[_s3(5120 * 4096, 4096, 128)] * 4)
    m = _meta(5120)

    def call(q=FAKE, S=5120, H=32, Hk=32, D=128, mask=1, meta=m, dtype=0, strides=st4):
        return f(q, FAKE, FAKE, FAKE2, None, 2, S, H, Hk, D, strides, mask,
                 ctypes.byref(meta) if meta is not None else None, 0.0, dtype, None)
    assert call(q=None) == _lib.ERR_NULL
    assert call(meta=None) == _lib.ERR_NULL                 # block-causal needs kv_limit
    assert call(S=5000) == _lib.ERR_SHAPE                   # metadata length mismatch
    assert call(Hk=5) == _lib.ERR_SHAPE                     # 32 % 5
    assert call(D=256) == _lib.ERR_UNSUPPORTED
    assert call(mask=3) == _lib.ERR_UNSUPPORTED
    assert call(dtype=2) == _lib.ERR_UNSUPPORTED
    assert call(q=FAKE + 8) == _lib.ERR_ALIGN
    fc = _lib.lib.dit_attn_forward_cached
    st6 = (_lib.Strides3 * 6)(*[_s3(5120 * 4096, 4096, 128)] * 6)
    assert fc(FAKE, None, None, FAKE, FAKE, FAKE2, None, 1, 16, 100, 32, 32, 128, st6, 1, ctypes.byref(_meta(116)),
              0.0, 0, None) == _lib.ERR_NULL            # P > 0 needs the cache
    assert fc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE2, None, 1, 16, 100, 32, 32, 128, st6, 1,
              ctypes.byref(_meta(100)), 0.0, 0, None) == _lib.ERR_SHAPE   # seq_len must be P + S_new


def test_empty_inputs_are_noops():
    """B == 0 or S == 0 returns OK without launching anything."""
    from diffusion_transformer_joint_token_amd import _lib
    st4 = (_lib.Strides3 * 4)(*[_s3(0, 4096, 128)] * 4)
    assert _lib.lib.dit_attn_forward(FAKE, FAKE, FAKE, FAKE2, None, 0, 16, 32, 32, 128, st4, 0, None, 0.0, 0,
                                     None) == _lib.OK
    assert _lib.lib.dit_attn_forward(FAKE, FAKE, FAKE, FAKE2, None, 2, 0, 32, 32, 128, st4, 0, None, 0.0, 0,
                                     None) == _lib.OK


def test_key_valid_argument_errors():
    from diffusion_transformer_joint_token_amd import _lib
    f = _lib.lib.dit_attn_build_key_valid

    def call(mask=FAKE, S=5120, tv=FAKE, B=2, n_text=1024, tv_stride=1024, bits=FAKE2, words=80, status=FAKE):
        return f(mask, S, tv, B, n_text, tv_stride, bits, words, status, None)
    assert call(mask=None) == _lib.ERR_NULL
    assert call(tv=None) == _lib.ERR_NULL
    assert call(bits=None) == _lib.ERR_NULL
    assert call(status=None) == _lib.ERR_NULL
    assert call(n_text=5121) == _lib.ERR_SHAPE          # more text tokens than the sequence
    assert call(tv_stride=1000) == _lib.ERR_SHAPE       # rows overlap
    assert call(words=79) == _lib.ERR_SHAPE             # 5120 keys need 80 words
    assert call(n_text=-1) == _lib.ERR_SHAPE
    assert call(bits=FAKE2 + 4) == _lib.ERR_ALIGN
    assert call(B=70000) == _lib.ERR_UNSUPPORTED
    assert call(B=0, mask=None) == _lib.OK              # empty: nothing read
    assert call(S=0, mask=None) == _lib.OK


def test_padded_attention_argument_errors():
    from diffusion_transformer_joint_token_amd import _lib
    f = _lib.lib.dit_attn_forward_padded
    st4 = (_lib.Strides3 * 4)(*[_s3(5120 * 4096, 4096, 128)] * 4)
    m = _meta(5120)

    def call(q=FAKE, kb=FAKE2, words=80, S=5120, B=2):
        return f(q, FAKE, FAKE, FAKE2, None, B, S, 32, 32, 128, st4, 1, ctypes.byref(m), kb, words, 0.0, 0, None)
    assert call(kb=None) == _lib.ERR_NULL
    assert call(q=None) == _lib.ERR_NULL
    assert call(words=79) == _lib.ERR_SHAPE
    assert call(kb=FAKE2 + 4) == _lib.ERR_ALIGN
    assert call(S=5000, words=80) == _lib.ERR_SHAPE     # metadata length mismatch
    assert call(B=0, q=None) == _lib.OK
    fc = _lib.lib.dit_attn_forward_cached_padded
    st6 = (_lib.Strides3 * 6)(*[_s3(5120 * 4096, 4096, 128)] * 6)

    def callc(kb=FAKE2, words=2, kc=FAKE):
        return fc(FAKE, kc, FAKE, FAKE, FAKE, FAKE2, None, 1, 16, 100, 32, 32, 128, st6, 1,
                  ctypes.byref(_meta(116)), kb, words, 0.0, 0, None)
    assert callc(kb=None) == _lib.ERR_NULL
    assert callc(kc=None) == _lib.ERR_NULL
    assert callc(words=1) == _lib.ERR_SHAPE             # 116 logical keys need 2 words


def test_qknorm_rope_ex_argument_errors():
    from diffusion_transformer_joint_token_amd import _lib
    f = _lib.lib.dit_attn_qknorm_rope_ex
    st = _s3(4096 * 40 * 72, 40 * 72, 72)
    axes = (ctypes.c_int32 * 2)(36, 36)

    def call(params, H=32, Hk=8, D=72, q=FAKE, B=2):
        return f(q, FAKE, FAKE2, FAKE2, B, 4096, H, Hk, D, st, st, st, st, FAKE, 2, axes,
                 ctypes.byref(params) if params is not None else None, 0, None)

    def prm(**kw):
        p = _lib.NormRopeParams(1, None, None, None, None, 1e-5, 1e4, 1.0, 1.0, 1.0)
        for k, v in kw.items():
            setattr(p, k, v)
        return p
    assert call(None) == _lib.ERR_NULL
    assert call(prm(), q=None) == _lib.ERR_NULL
    assert call(prm(norm=2)) == _lib.ERR_UNSUPPORTED
    assert call(prm(rope_linear_factor=0.0)) == _lib.ERR_SHAPE
    assert call(prm(rope_ntk_factor=-1.0)) == _lib.ERR_SHAPE
    assert call(prm(rope_ntk_factor=float("inf"))) == _lib.ERR_SHAPE
    assert call(prm(eps=-1.0)) == _lib.ERR_SHAPE
    assert call(prm(q_bias=FAKE + 4)) == _lib.ERR_ALIGN
    assert call(prm(), H=256, Hk=256, D=128) == _lib.ERR_UNSUPPORTED   # (256 + 256) * 16 chunks > 2048
    assert call(prm(), B=0, q=None) == _lib.OK


def test_fused_qnorm_attention_argument_errors():
    """dit_attn_forward_cached_qnorm: bf16 and the per-head RMSNorm only, needs
    the positions and the options, checks the rotary axes and factors, eps and
    the alignment of the weight, then the checks of the cached / padded forms."""
    from diffusion_transformer_joint_token_amd import _lib
    f = _lib.lib.dit_attn_forward_cached_qnorm
    st6 = (_lib.Strides3 * 6)(*[_s3(4096 * 4096, 4096, 128)] * 6)

    def prm(**kw):
        p = _lib.NormRopeParams(0, None, None, None, None, 1e-6, 1e4, 1.0, 1.0, 1.0)
        for k, v in kw.items():
            setattr(p, k, v)
        return p

    def call(q=FAKE, kc=FAKE, P=16, kb=None, words=0, pos=FAKE2, axes=(16, 56, 56), params=None, dtype=0, B=1,
             S=100, D=128):
        ax = (ctypes.c_int32 * len(axes))(*axes)
        p = prm() if params is None else params
        return f(q, kc, FAKE, FAKE, FAKE, FAKE2, None, B, P, S, 32, 32, D, st6, 1, ctypes.byref(_meta(P + S)), kb,
                 words, pos, len(axes), ax, ctypes.byref(p) if params != "null" else None, 0.0, dtype, None)
    assert call(pos=None) == _lib.ERR_NULL
    assert call(params="null") == _lib.ERR_NULL
    assert call(q=None) == _lib.ERR_NULL
    assert call(kc=None) == _lib.ERR_NULL               # P > 0 needs the cache
    assert call(dtype=1) == _lib.ERR_UNSUPPORTED        # fused form is bf16 only
    assert call(params=prm(norm=1)) == _lib.ERR_UNSUPPORTED  # per-head RMSNorm only
    assert call(D=136, axes=(16, 56, 64)) == _lib.ERR_UNSUPPORTED
    assert call(axes=(16, 56, 58)) == _lib.ERR_SHAPE    # axes must sum to D
    assert call(axes=(17, 55, 56)) == _lib.ERR_SHAPE    # and be even
    assert call(params=prm(rope_ntk_factor=0.0)) == _lib.ERR_SHAPE
    assert call(params=prm(rope_linear_factor=float("inf"))) == _lib.ERR_SHAPE
    assert call(params=prm(rope_theta=-1.0)) == _lib.ERR_SHAPE
    assert call(params=prm(eps=-1.0)) == _lib.ERR_SHAPE
    assert call(params=prm(eps=float("nan"))) == _lib.ERR_SHAPE
    assert call(params=prm(q_scale=0.0)) == _lib.ERR_SHAPE
    assert call(params=prm(q_weight=FAKE + 2)) == _lib.ERR_ALIGN
    assert call(pos=FAKE2 + 2) == _lib.ERR_ALIGN
    assert call(kb=FAKE2, words=1) == _lib.ERR_SHAPE    # 116 logical keys need 2 words
    assert call(B=0, q=None, pos=None) == _lib.OK       # empty: nothing read
    assert call(S=0, q=None) == _lib.OK


def test_qknorm_rope_k_only_argument_errors():
    """q and q_out both NULL is the K-only form (H ignored); one of them alone
    is an error."""
    from diffusion_transformer_joint_token_amd import _lib
    f = _lib.lib.dit_attn_qknorm_rope_ex
    st = _s3(4096 * 8 * 128, 8 * 128, 128)
    axes = (ctypes.c_int32 * 3)(32, 48, 48)

    def call(q=None, qo=None, H=0, Hk=8, D=128, norm=0):
        p = _lib.NormRopeParams(norm, None, None, None, None, 1e-6, 1e4, 1.0, 1.0, 1.0)
        return f(q, FAKE, qo, FAKE2, 1, 4096, H, Hk, D, st, st, st, st, FAKE, 3, axes, ctypes.byref(p), 0, None)
    assert call(qo=FAKE2, H=32) == _lib.ERR_NULL        # q_out without q
    assert call(q=FAKE, H=32) == _lib.ERR_NULL          # q without q_out
    assert call(q=FAKE, qo=FAKE2, H=0) == _lib.ERR_SHAPE  # with Q, H must be >= 1
    assert call(Hk=0) == _lib.ERR_SHAPE
    assert call(D=136) == _lib.ERR_UNSUPPORTED
    # the LayerNorm item limit counts Q's heads only when Q is there
    assert call(q=FAKE, qo=FAKE2, H=256, Hk=8, norm=1) == _lib.ERR_UNSUPPORTED  # (256 + 8) * 16 > 2048


def test_time_aware_factors_host_helper():
    """The C helper against the oracle's switch (the product's only host-side
    arithmetic of the method), and its argument errors."""
    import oracle.qknorm_rope as oqr
    from diffusion_transformer_joint_token_amd import _lib
    lin, ntk = ctypes.c_float(), ctypes.c_float()
    for t in (0.0, 0.1, 0.29999, 0.3, 0.31, 0.7, 1.0):
        for sf in (1.0, 2.0, 4.0):
            assert _lib.lib.dit_attn_time_aware_rope_factors(t, 0.3, sf, ctypes.byref(lin), ctypes.byref(ntk)) == 0
            ref = oqr.time_aware_rope_factors(float(ctypes.c_float(t).value), float(ctypes.c_float(0.3).value), sf)
            assert (lin.value, ntk.value) == ref, (t, sf)
    f = _lib.lib.dit_attn_time_aware_rope_factors
    assert f(0.1, 0.3, 2.0, None, ctypes.byref(ntk)) == _lib.ERR_NULL
    assert f(float("nan"), 0.3, 2.0, ctypes.byref(lin), ctypes.byref(ntk)) == _lib.ERR_SHAPE
    assert f(0.1, 0.3, 0.0, ctypes.byref(lin), ctypes.byref(ntk)) == _lib.ERR_SHAPE


def test_cfg_argument_errors():
    from diffusion_transformer_joint_token_amd import _lib
    f = _lib.lib.dit_attn_cfg_norm_rescale

    def call(c=FAKE, u=FAKE2, o=FAKE2, rows=4096, C=64, cs=64, us=64, os_=64, g=4.0, dtype=0):
        return f(c, u, o, rows, C, cs, us, os_, g, dtype, None)
    assert call(c=None) == _lib.ERR_NULL
    assert call(C=60) == _lib.ERR_UNSUPPORTED          # not a multiple of 8 (bf16)
    assert call(C=8 * 513) == _lib.ERR_UNSUPPORTED     # more than 4096 bf16 channels
    assert call(cs=32) == _lib.ERR_SHAPE               # rows overlap
    assert call(g=float("nan")) == _lib.ERR_SHAPE
    assert call(C=0) == _lib.ERR_SHAPE
    assert call(dtype=3) == _lib.ERR_UNSUPPORTED
    assert call(u=FAKE2 + 8) == _lib.ERR_ALIGN
    assert call(cs=68) == _lib.ERR_ALIGN               # 136-byte row stride
    assert call(rows=0, c=None) == _lib.OK


def test_binding_checks_output_buffers_and_key_bits():
    """The binding compares caller buffers with the call before it reaches the
    C ABI (which cannot see allocation sizes): O must have the queries' shape
    and dtype, lse_out must be fp32 [B, H, S], and the key-validity words must
    have one row per sample and a word per 64 keys.  (CPU tensors: every case
    raises before anything is launched.)"""
    import torch
    import diffusion_transformer_joint_token_amd as dit
    bf = torch.bfloat16
    q = torch.zeros(2, 70, 8, 128, dtype=bf)
    k = v = torch.zeros(2, 70, 2, 128, dtype=bf)
    bad_outs = [torch.zeros(2, 70, 2, 128, dtype=bf),      # GQA-shaped: the kernel would write past its end
                torch.zeros(2, 70, 8, 128, dtype=torch.float32),
                torch.zeros(1, 70, 8, 128, dtype=bf)]
    for out in bad_outs:
        with pytest.raises(dit.DitAttnError):
            dit.forward(q, k, v, "full", out=out)
        with pytest.raises(dit.DitAttnError):
            dit.forward_cached(q, None, None, k, v, "full", out=out)
        with pytest.raises(dit.DitAttnError):
            dit.forward_cached_qnorm(q, None, None, k, v, torch.zeros(70, 3, dtype=torch.int32), (32, 48, 48),
                                     1e-6, mask_mode="full", out=out)
    for lse in (torch.zeros(2, 2, 70), torch.zeros(2, 8, 70, dtype=bf), torch.zeros(2, 70, 8)):
        with pytest.raises(dit.DitAttnError):
            dit.forward(q, k, v, "full", lse_out=lse)
    for bits in (torch.zeros(1, 2, dtype=torch.int64),     # one row for two samples
                 torch.zeros(2, 1, dtype=torch.int64),     # 70 keys need 2 words
                 torch.zeros(2, 2, dtype=torch.int32)):
        with pytest.raises(dit.DitAttnError):
            dit.forward(q, k, v, "full", key_valid=bits)
        with pytest.raises(dit.DitAttnError):
            dit.forward_cached(q, None, None, k, v, "full", key_valid=bits)
    # cached: the words cover the logical sequence P + S_new
    kc = vc = torch.zeros(2, 64, 2, 128, dtype=bf)
    with pytest.raises(dit.DitAttnError):
        dit.forward_cached(q, kc, vc, k, v, "full", key_valid=torch.zeros(2, 2, dtype=torch.int64))


def test_prescaled_factor_helper():
    """dit_attn_prescaled_q_factor: (scale or 1/sqrt(D)) * log2(e), in double,
    rounded once; the binding's prescaled_q_factor is that call."""
    import math
    from diffusion_transformer_joint_token_amd import _lib, api
    out = ctypes.c_float()
    for D, s in ((128, 0.0), (72, 0.0), (32, 0.0), (128, 0.3)):
        assert _lib.lib.dit_attn_prescaled_q_factor(D, s, ctypes.byref(out)) == _lib.OK
        want = ctypes.c_float((s if s > 0 else 1.0 / math.sqrt(D)) * 1.4426950408889634).value
        assert out.value == want
        assert api.prescaled_q_factor(D, s or None) == want
    assert _lib.lib.dit_attn_prescaled_q_factor(128, 0.0, None) == _lib.ERR_NULL
    assert _lib.lib.dit_attn_prescaled_q_factor(0, 0.0, ctypes.byref(out)) == _lib.ERR_SHAPE
    assert _lib.lib.dit_attn_prescaled_q_factor(128, float("nan"), ctypes.byref(out)) == _lib.ERR_SHAPE
