/*
 * dit_attn.h -- C ABI of the joint text+image DiT attention step on MI355X (gfx950).
 *
 * The step is the single-stream attention of a diffusion transformer whose
 * sequence holds text tokens and image-latent tokens together:
 *   1. token metadata: per-token image-block ids, target mask, rotary positions
 *      and the exclusive key bound of each query
 *      (QwenImage21Transformer2DModel API page, build_token_metadata);
 *   2. per-head RMSNorm of Q and K, then multi-axis rotary embedding
 *      (NucleusMoE-Image pipeline article, section 6.3; Lumina-Next DiT article,
 *      configuration table and section 4);
 *   3. softmax attention under the full mask or the block-causal rule
 *      "q_idx >= kv_idx or same image block", with grouped-query heads
 *      (QwenImage21Transformer2DModel API page, block-causal attention;
 *      NucleusMoE-Image article, section 6.3);
 *   4. the same attention with the keys/values of the timestep-independent
 *      prefix (text and condition images) taken from a cache
 *      (QwenImage21Transformer2DModel API page, causal_condition and
 *      forward's kv_cache / kv_cache_mode);
 *   5. either attention with padded text keys left out, per sample
 *      (QwenImage21Transformer2DModel API page, forward's
 *      encoder_hidden_states_mask);
 *   6. the Lumina-Next forms of step 2: LayerNorm across heads instead of the
 *      per-head RMSNorm, and the time-aware rotary scaling (Lumina-Next DiT
 *      article, sections 3 and 4);
 *   7. outside the attention: the norm-rescaled classifier-free guidance that
 *      combines the conditional and unconditional predictions of a step
 *      (NucleusMoE-Image pipeline article, section 4.3).
 *
 * Conventions shared by every entry point
 *   - Memory: every pointer marked "device" is device memory owned by the
 *     caller; "host" pointers are read before the call returns.  The library
 *     allocates nothing, frees nothing, keeps no state between calls and is
 *     thread-safe.
 *   - Layout: activations are [batch, seq, heads, head_dim] ("BSHD") with the
 *     head_dim axis contiguous; the other three strides are passed in elements
 *     as {batch, seq, head}.  Base pointers and strides must keep every row
 *     16-byte aligned.
 *   - Streams: `stream` is a hipStream_t (NULL = the default stream).  All work
 *     is enqueued asynchronously; no call synchronises.
 *   - Empty work: a qknorm/attention call with B == 0 or S == 0 (S_new == 0)
 *     returns DIT_ATTN_OK at once and reads none of its pointers.
 *   - Errors: argument errors are found on the host before anything is
 *     enqueued and returned as a dit_attn_status; a failed launch returns
 *     DIT_ATTN_ERR_HIP.  Errors that depend on device data (see
 *     dit_attn_build_token_metadata) are written to a device status word.
 *     Nothing aborts and no exception crosses the ABI.
 */
#ifndef DIT_ATTN_H
#define DIT_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DIT_ATTN_OK = 0,
  DIT_ATTN_ERR_NULL = 1,        /* a required pointer is NULL */
  DIT_ATTN_ERR_SHAPE = 2,       /* sizes inconsistent or out of range */
  DIT_ATTN_ERR_UNSUPPORTED = 3, /* valid request this build does not implement */
  DIT_ATTN_ERR_ALIGN = 4,       /* pointer or stride breaks 16-byte row alignment */
  DIT_ATTN_ERR_DATA = 5,        /* device data break the layout contract (status word) */
  DIT_ATTN_ERR_HIP = 6          /* a HIP runtime call or launch failed */
} dit_attn_status;

typedef enum { DIT_ATTN_BF16 = 0, DIT_ATTN_F32 = 1 } dit_attn_dtype;

typedef enum {
  DIT_ATTN_MASK_FULL = 0,        /* every query sees every key */
  DIT_ATTN_MASK_BLOCK_CAUSAL = 1 /* q sees k iff k <= q or both in one image block */
} dit_attn_mask_mode;

typedef enum {
  /* 3 axes (frame, height, width).  Image token (f, h, w) of a block of shape
   * (F, H, W) sits at (frame offset of the block + f, h - H/2, w - W/2); the
   * frame offset is the sum of F over earlier blocks.  Text token number t
   * (counting text tokens in sequence order) sits at max_vid_index + t on all
   * three axes, max_vid_index being one past the largest image coordinate
   * (0 with no image).  H and W must be even. */
  DIT_ATTN_POS_CENTERED_FHW = 0,
  /* 2 axes (height, width) from 0 inside each single-frame block; third
   * column 0.  Image tokens only (a text token is a data error). */
  DIT_ATTN_POS_GRID_HW = 1
} dit_attn_pos_mode;

/* Largest number of image blocks per sequence. */
#define DIT_ATTN_MAX_IMAGES 64

/* Token metadata of one joint sequence (shared by every batch element: all
 * samples share the layout, QwenImage21Transformer2DModel API page, forward's
 * img_shapes).  The struct is a host object; its pointers are device buffers
 * the caller owns, each with seq_len entries (pos_ids: seq_len * 3). */
typedef struct {
  int32_t *image_ids;   /* [seq_len] text = -1, image block b = b (0-based)       */
  uint8_t *target_mask; /* [seq_len] 1 on tokens of the last (target) image block */
  int32_t *pos_ids;     /* [seq_len][3] rotary positions (see dit_attn_pos_mode)  */
  int32_t *kv_limit;    /* [seq_len] exclusive bound of the keys token s may see
                           under the block-causal rule: s + 1 for text, one past
                           the last token of its block for image tokens          */
  int32_t seq_len;
} dit_attn_token_meta;

/* Token metadata (QwenImage21Transformer2DModel API page, build_token_metadata).
 *   image_pad_mask  device uint8 [seq_len], nonzero on image tokens.
 *   img_shapes      host int32 [n_img][3] = (frames, height, width) of each image
 *                   block in sequence order, condition images first, the target
 *                   last.  Block boundaries follow these token counts, not runs of
 *                   nonzero mask entries: adjacent images stay separate blocks.
 *   n_img           0..DIT_ATTN_MAX_IMAGES (0 = text only; nothing is target).
 *   pos_mode        dit_attn_pos_mode.
 *   meta            host struct of caller-owned device output buffers;
 *                   meta->seq_len must equal seq_len.
 *   status_dev      device int32 [1]; receives DIT_ATTN_OK or DIT_ATTN_ERR_DATA when
 *                   the mask marks a different number of tokens than img_shapes
 *                   describe, a block's tokens are not contiguous, or (GRID_HW) a
 *                   text token is present.  On a data error the outputs are
 *                   unspecified.  Read it after the stream has run the call.
 * Host-side errors: NULL pointers, seq_len < 1, n_img out of range, an extent < 1,
 * odd H/W (CENTERED_FHW), frames != 1 (GRID_HW), unknown pos_mode. */
int dit_attn_build_token_metadata(const uint8_t *image_pad_mask, int32_t seq_len,
                                  const int32_t *img_shapes, int32_t n_img, int32_t pos_mode,
                                  const dit_attn_token_meta *meta, int32_t *status_dev,
                                  void *stream);

/* Key validity of the joint sequence, per sample, from the text mask
 * (QwenImage21Transformer2DModel API page, forward's encoder_hidden_states_mask:
 * a [batch, text length] mask of the valid text tokens; padded ones take no part
 * in attention).  The j-th text token of the sequence (counting, in sequence
 * order, the tokens where image_pad_mask is 0) takes entry j of its sample's
 * text mask; image tokens are always valid.
 *   image_pad_mask     device uint8 [seq_len], nonzero on image tokens (the
 *                      metadata's input; shared by the batch).
 *   text_valid         device uint8 [B][n_text] (row stride text_valid_stride
 *                      bytes, >= n_text), nonzero = valid.  May be NULL when
 *                      n_text == 0.
 *   key_valid          device uint64 [B][key_valid_stride], 8-byte aligned,
 *                      key_valid_stride >= ceil(seq_len / 64): bit j of word t of
 *                      sample b is 1 iff key 64 t + j may be attended.  Words
 *                      0 .. ceil(seq_len / 64) - 1 are written, bits past seq_len
 *                      as 0; later words are left untouched.
 *   status_dev         device int32 [1]; receives DIT_ATTN_OK, or DIT_ATTN_ERR_DATA
 *                      when the mask has a number of text tokens other than
 *                      n_text (the bits are then unspecified).
 * B == 0 or seq_len == 0 returns DIT_ATTN_OK at once.  Host-side errors: NULL
 * pointers, negative sizes, n_text > seq_len, a short stride, B > 65535. */
int dit_attn_build_key_valid(const uint8_t *image_pad_mask, int32_t seq_len, const uint8_t *text_valid,
                             int32_t B, int32_t n_text, int64_t text_valid_stride, uint64_t *key_valid,
                             int64_t key_valid_stride, int32_t *status_dev, void *stream);

/* Fused per-head RMSNorm + multi-axis rotary embedding of Q and K
 * (NucleusMoE-Image pipeline article, section 6.3: qk_norm then rotary;
 *  Lumina-Next DiT article: 2D rotary needs head_dim % 4 == 0).
 * For every (b, s, head) of Q (H heads) and K (H_kv heads):
 *   y = x / sqrt(mean_d x_d^2 + eps) * w            (w: q_weight or k_weight)
 *   then for axis a owning channels [o_a, o_a + d_a), pair j turns
 *   (y[o_a+2j], y[o_a+2j+1]) by pos[s][a] * rope_theta^(-2j/d_a).
 * Q outputs are then multiplied by q_scale (1 = plain); passing
 * q_scale = log2(e) * softmax_scale folds the attention's softmax scale into Q
 * with a single rounding (then call the attention with softmax_scale = ln 2).
 * V is not touched.  Arithmetic in fp32; outputs rounded to the dtype (RNE).
 * Angles: pos * rope_theta^(-2j/d_a) / (2 pi) turns formed in double, whole
 * turns removed exactly, the fraction rounded to fp32 and its sin and cos
 * taken by the hardware instructions (absolute error <= 1.3e-7, measured).
 *   q, k           device [B, S, H | H_kv, D] in dtype, strides q_strides/k_strides.
 *   q_out, k_out   device outputs (may alias q, k exactly), strides qo_/ko_strides.
 *   q_weight, k_weight  device [D] in dtype, or NULL for unit weights.
 *   pos_ids        device int32 [S][3] (the metadata's pos_ids; for the new
 *                  tokens of a cached step pass meta.pos_ids + 3 * prefix_len).
 *   n_axes         2 or 3; axes_dims host int32 [n_axes], each even, summing to D.
 *   rope_theta     rotary base (> 0).  eps >= 0.  q_scale finite, != 0.
 * Requirements: D % 8 == 0 (bf16) or D % 4 == 0 (f32), 8 <= D <= 128. */
int dit_attn_qknorm_rope(const void *q, const void *k, void *q_out, void *k_out,
                         const void *q_weight, const void *k_weight,
                         int32_t B, int32_t S, int32_t H, int32_t H_kv, int32_t D,
                         const int64_t q_strides[3], const int64_t k_strides[3],
                         const int64_t qo_strides[3], const int64_t ko_strides[3],
                         const int32_t *pos_ids, int32_t n_axes, const int32_t *axes_dims,
                         float rope_theta, float eps, float q_scale, int32_t dtype, void *stream);

/* Normalisation applied to Q and K before the rotary embedding. */
typedef enum {
  DIT_ATTN_NORM_RMS_PER_HEAD = 0,      /* y = x / sqrt(mean_D x^2 + eps) * w, w: [D] shared by the heads */
  DIT_ATTN_NORM_LAYER_ACROSS_HEADS = 1 /* per token, over all heads' channels together:
                                          y = (x - mean) / sqrt(var + eps) * w + b, biased variance,
                                          w and b: [heads * D] (Lumina-Next DiT article, section 3) */
} dit_attn_qk_norm;

/* Options of dit_attn_qknorm_rope_ex (a host struct; its pointers are device
 * buffers in the data dtype, 16-byte aligned, or NULL). */
typedef struct {
  int32_t norm;             /* dit_attn_qk_norm */
  const void *q_weight;     /* RMS: [D]; LayerNorm: [H * D]; NULL = 1 */
  const void *k_weight;     /* RMS: [D]; LayerNorm: [H_kv * D]; NULL = 1 */
  const void *q_bias;       /* LayerNorm only: [H * D]; NULL = 0 (ignored for RMS) */
  const void *k_bias;       /* LayerNorm only: [H_kv * D]; NULL = 0 */
  float eps;                /* >= 0 */
  float rope_theta;         /* rotary base, > 0 */
  float rope_linear_factor; /* > 0: positions are divided by it (1 = none) */
  float rope_ntk_factor;    /* > 0: the rotary base is multiplied by it (1 = none) */
  float q_scale;            /* finite, != 0: multiplies the Q outputs (see dit_attn_qknorm_rope) */
} dit_attn_norm_rope_params;

/* dit_attn_qknorm_rope with a choice of norm and scaled rotary frequencies
 * (Lumina-Next DiT article, section 3: qk_norm as a LayerNorm across heads;
 * section 4: the rotary table rebuilt at every denoising step with a linear
 * and an NTK factor).  Pair j of axis a turns by
 * (pos / rope_linear_factor) * (rope_theta * rope_ntk_factor)^(-2j/d_a).
 * With norm = RMS_PER_HEAD, both factors 1 and no bias the result is
 * bit-identical to dit_attn_qknorm_rope.  The LayerNorm keeps separate
 * statistics for Q (over H * D channels) and K (over H_kv * D channels), in
 * fp32, reduced in a fixed order.  Limits: (H + H_kv) * D / 8 (bf16) or / 4
 * (f32) <= 2048 for the LayerNorm; otherwise as dit_attn_qknorm_rope.
 * q and q_out may both be NULL (with their strides): K only, H ignored -- the
 * form that goes with dit_attn_forward_cached_qnorm, which norms Q itself.
 * params is a host pointer (NULL -> DIT_ATTN_ERR_NULL). */
int dit_attn_qknorm_rope_ex(const void *q, const void *k, void *q_out, void *k_out,
                            int32_t B, int32_t S, int32_t H, int32_t H_kv, int32_t D,
                            const int64_t q_strides[3], const int64_t k_strides[3],
                            const int64_t qo_strides[3], const int64_t ko_strides[3],
                            const int32_t *pos_ids, int32_t n_axes, const int32_t *axes_dims,
                            const dit_attn_norm_rope_params *params, int32_t dtype, void *stream);

/* Host helper: the rotary factors of one denoising step (Lumina-Next DiT
 * article, section 4).  t is the pipeline's reversed timestep (0 = noise,
 * 1 = image).  Before the watershed (t < watershed) the linear factor is
 * scaling_factor and the NTK factor 1; from it on the reverse.  (The page's
 * comparison operator is lost from its text; this is the reading.)  Writes
 * both outputs; errors: NULL outputs, non-finite inputs, scaling_factor <= 0. */
int dit_attn_time_aware_rope_factors(float t, float watershed, float scaling_factor,
                                     float *linear_factor, float *ntk_factor);

/* Host helper: the q_scale that folds the attention's softmax scale into Q'
 * (the scale of the pages' attention is 1/sqrt(head_dim) when none is given,
 * as in scaled dot-product attention) together with log2(e), so that the
 * attention can run with softmax_scale = ln 2 and exponentiate its logits in
 * base 2: *q_scale_out = (softmax_scale > 0 ? softmax_scale : 1/sqrt(head_dim))
 * * log2(e), evaluated in double and rounded once to float.  Errors: NULL
 * output, head_dim < 1, a non-finite softmax_scale. */
int dit_attn_prescaled_q_factor(int32_t head_dim, float softmax_scale, float *q_scale_out);

/* Masked softmax attention (QwenImage21Transformer2DModel API page, block-causal
 * attention; NucleusMoE-Image article section 6.3 for GQA):
 *   O[b,q,h] = sum_k softmax_k(scale * <Q[b,q,h], K[b,k,g]>) V[b,k,g],  g = h / (H/H_kv)
 * over the keys k allowed for q: all keys (FULL) or k < meta->kv_limit[q]
 * (BLOCK_CAUSAL; this prefix is exactly "k <= q or same image block" for
 * contiguous blocks).
 *   q, k, v, o   device [B, S, H|H_kv|H_kv|H, D]; strides[0..3] = q, k, v, o.
 *   lse          device float [B, H, S] natural-log sum-exp of the scaled logits,
 *                or NULL.
 *   meta         host struct; only kv_limit is read (may be NULL for FULL);
 *                meta->seq_len must equal S.
 *   softmax_scale  <= 0 selects 1/sqrt(D).  With Q pre-multiplied by
 *                  log2(e) * scale (dit_attn_qknorm_rope's q_scale), pass ln 2: the
 *                  kernel then exponentiates the MFMA output directly.
 * bf16: QK^T and PV on bf16 MFMA with fp32 accumulation, P rounded to bf16 for
 * PV, O rounded once.  f32: fp32 throughout.  D <= 128, D % 8 == 0. */
int dit_attn_forward(const void *q, const void *k, const void *v, void *o, float *lse,
                     int32_t B, int32_t S, int32_t H, int32_t H_kv, int32_t D,
                     const int64_t strides[4][3], int32_t mask_mode,
                     const dit_attn_token_meta *meta, float softmax_scale, int32_t dtype,
                     void *stream);

/* Attention of the new tokens of a cached step (QwenImage21Transformer2DModel API
 * page, kv_cache_mode "cached"): the logical sequence has P prefix tokens whose
 * keys/values come from the cache, followed by S_new new tokens.  Query row i is
 * logical token P + i; keys 0..P-1 are read from k_cache/v_cache (post-norm,
 * post-rotary K; raw V) and keys P..P+S_new-1 from k_new/v_new.  The mask and
 * everything else are those of dit_attn_forward on the logical sequence, so the
 * rows equal rows P.. of a full forward over cache+new.
 *   strides[0..5] = q_new, k_cache, v_cache, k_new, v_new, o.
 *   meta->seq_len must equal P + S_new; P >= 0 (P == 0 is a plain forward). */
int dit_attn_forward_cached(const void *q_new, const void *k_cache, const void *v_cache,
                            const void *k_new, const void *v_new, void *o, float *lse,
                            int32_t B, int32_t P, int32_t S_new, int32_t H, int32_t H_kv,
                            int32_t D, const int64_t strides[6][3], int32_t mask_mode,
                            const dit_attn_token_meta *meta, float softmax_scale,
                            int32_t dtype, void *stream);

/* dit_attn_forward with padded keys left out (QwenImage21Transformer2DModel API
 * page, forward's encoder_hidden_states_mask): query q of sample b attends the
 * keys that the mask mode allows AND whose bit in key_valid is 1.
 *   key_valid         device uint64 [B][key_valid_stride] as written by
 *                     dit_attn_build_key_valid (any bits may be passed), 8-byte
 *                     aligned, key_valid_stride >= ceil(S / 64) words.
 * A query with no allowed valid key gets O = 0 and lse = -inf.  K and V must be
 * finite at padded keys too (they enter as probability 0 times the value).
 * With every bit of keys 0 .. S-1 set, the result is bit-identical to
 * dit_attn_forward.  Other arguments and errors as dit_attn_forward. */
int dit_attn_forward_padded(const void *q, const void *k, const void *v, void *o, float *lse,
                            int32_t B, int32_t S, int32_t H, int32_t H_kv, int32_t D,
                            const int64_t strides[4][3], int32_t mask_mode,
                            const dit_attn_token_meta *meta, const uint64_t *key_valid,
                            int64_t key_valid_stride, float softmax_scale, int32_t dtype,
                            void *stream);

/* dit_attn_forward_cached with padded keys left out: bits index the logical
 * sequence (cache keys 0 .. P-1, then the new keys), key_valid_stride >=
 * ceil((P + S_new) / 64).  Otherwise as dit_attn_forward_padded. */
int dit_attn_forward_cached_padded(const void *q_new, const void *k_cache, const void *v_cache,
                                   const void *k_new, const void *v_new, void *o, float *lse,
                                   int32_t B, int32_t P, int32_t S_new, int32_t H, int32_t H_kv,
                                   int32_t D, const int64_t strides[6][3], int32_t mask_mode,
                                   const dit_attn_token_meta *meta, const uint64_t *key_valid,
                                   int64_t key_valid_stride, float softmax_scale, int32_t dtype,
                                   void *stream);

/* Attention (plain, cached or padded) on raw Q: the per-head RMSNorm of Q,
 * its rotary embedding and the softmax scale are applied inside the attention
 * kernel as each work-group loads its query rows, so the normed Q never goes
 * through memory (NucleusMoE-Image pipeline article, section 6.3: qk_norm,
 * then the rotary embedding, then attention).  K must already be normed and
 * rotated: dit_attn_qknorm_rope_ex with q = q_out = NULL does K alone.
 * Per query row x of token i:
 *   y = x / sqrt(mean_D x^2 + eps) * q_weight, rotated as dit_attn_qknorm_rope_ex
 *   rotates (pair j of axis a by pos_ids[i][a] / rope_linear_factor *
 *   (rope_theta * rope_ntk_factor)^(-2j/d_a), the same angles bit for bit),
 *   times q_scale * softmax_scale * log2(e), rounded once to bf16
 * -- the Q' that dit_attn_qknorm_rope_ex with that q_scale produces, up to
 * the summation order of mean_D x^2 -- then the attention of
 * dit_attn_forward_cached_padded with scale ln 2.
 *   q_new_raw  device [B, S_new, H, D] raw Q (stride strides[0]).
 *   pos_ids    device int32 [S_new][3], 4-byte aligned: positions of the query
 *              tokens (the metadata's pos_ids + 3 * P).
 *   n_axes, axes_dims  as dit_attn_qknorm_rope.
 *   params     host: norm must be DIT_ATTN_NORM_RMS_PER_HEAD
 *              (DIT_ATTN_ERR_UNSUPPORTED otherwise); q_weight (device bf16
 *              [D] or NULL), eps, rope_theta, the two rotary factors and
 *              q_scale are used; the k_ and bias fields are ignored.
 *   key_valid  as dit_attn_forward_cached_padded, or NULL (no padding).
 *   P == 0 is the plain forward; other arguments as dit_attn_forward_cached.
 * bf16 only (DIT_ATTN_ERR_UNSUPPORTED otherwise). */
int dit_attn_forward_cached_qnorm(const void *q_new_raw, const void *k_cache, const void *v_cache,
                                  const void *k_new, const void *v_new, void *o, float *lse,
                                  int32_t B, int32_t P, int32_t S_new, int32_t H, int32_t H_kv,
                                  int32_t D, const int64_t strides[6][3], int32_t mask_mode,
                                  const dit_attn_token_meta *meta, const uint64_t *key_valid,
                                  int64_t key_valid_stride, const int32_t *pos_ids, int32_t n_axes,
                                  const int32_t *axes_dims, const dit_attn_norm_rope_params *params,
                                  float softmax_scale, int32_t dtype, void *stream);

/* Classifier-free guidance with norm rescaling (NucleusMoE-Image pipeline
 * article, section 4.3), row by row (a row = one token's C channels):
 *   mix = uncond + guidance_scale * (cond - uncond)
 *   out = mix * ||cond|| / ||mix||        (norms over the row's channels)
 * A row whose mix is exactly zero is written as zero.  Arithmetic in fp32,
 * one rounding on the store.
 *   cond, uncond, out  device [rows][channels] in dtype; row r starts at
 *                      ptr + r * stride (strides in elements, >= channels);
 *                      channels contiguous.  out may alias cond or uncond
 *                      exactly (same pointer and stride).
 *   channels           a multiple of 8 (bf16) or 4 (f32), at most 4096 (bf16)
 *                      or 2048 (f32).  guidance_scale finite.
 * rows == 0 returns DIT_ATTN_OK at once.  Base pointers and strides keep rows
 * 16-byte aligned. */
int dit_attn_cfg_norm_rescale(const void *cond, const void *uncond, void *out, int64_t rows,
                              int32_t channels, int64_t cond_stride, int64_t uncond_stride,
                              int64_t out_stride, float guidance_scale, int32_t dtype, void *stream);

/* Static description of a status code (never NULL). */
const char *dit_attn_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* DIT_ATTN_H */
