// C-ABI entry points: argument validation on the host, then one kernel launch
// on the caller's stream.  Nothing here allocates, frees or synchronises.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "../../include/dit_attn.h"
#include "kernels.h"

namespace {

constexpr int64_t kMaxDim = 128;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Every row start must stay 16-byte aligned: base pointer and each stride.
bool rows_aligned(const void* p, const int64_t st[3], int elem) {
  if (!aligned16(p)) return false;
  for (int i = 0; i < 3; ++i)
    if ((st[i] * elem) % 16 != 0) return false;
  return true;
}

bool strides_ok(const int64_t st[3]) {
  for (int i = 0; i < 3; ++i)
    if (st[i] < 0) return false;
  return true;
}

int elem_size(int32_t dtype) { return dtype == DIT_ATTN_BF16 ? 2 : 4; }

}  // namespace

extern "C" {

const char* dit_attn_status_string(int32_t status) {
  switch (status) {
    case DIT_ATTN_OK: return "ok";
    case DIT_ATTN_ERR_NULL: return "a required pointer is NULL";
    case DIT_ATTN_ERR_SHAPE: return "sizes are inconsistent or out of range";
    case DIT_ATTN_ERR_UNSUPPORTED: return "request not supported by this build";
    case DIT_ATTN_ERR_ALIGN: return "pointer or stride breaks 16-byte row alignment";
    case DIT_ATTN_ERR_DATA: return "device data break the layout contract";
    case DIT_ATTN_ERR_HIP: return "HIP runtime or launch failure";
    default: return "unknown status";
  }
}

int dit_attn_build_token_metadata(const uint8_t* image_pad_mask, int32_t seq_len, const int32_t* img_shapes,
                                  int32_t n_img, int32_t pos_mode, const dit_attn_token_meta* meta,
                                  int32_t* status_dev, void* stream) {
  if (!image_pad_mask || !meta || !status_dev || (n_img > 0 && !img_shapes)) return DIT_ATTN_ERR_NULL;
  if (!meta->image_ids || !meta->target_mask || !meta->pos_ids || !meta->kv_limit) return DIT_ATTN_ERR_NULL;
  if (seq_len < 1 || meta->seq_len != seq_len) return DIT_ATTN_ERR_SHAPE;
  if (n_img < 0 || n_img > DIT_ATTN_MAX_IMAGES) return DIT_ATTN_ERR_SHAPE;
  if (pos_mode != DIT_ATTN_POS_CENTERED_FHW && pos_mode != DIT_ATTN_POS_GRID_HW) return DIT_ATTN_ERR_UNSUPPORTED;

  dit::TokenMetaArgs a{};
  a.seq_len = seq_len;
  a.n_img = n_img;
  a.pos_mode = pos_mode;
  int64_t total = 0, frames = 0;
  int32_t max_coord = -1;
  a.cum[0] = 0;
  for (int b = 0; b < n_img; ++b) {
    const int64_t f = img_shapes[3 * b], h = img_shapes[3 * b + 1], w = img_shapes[3 * b + 2];
    if (f < 1 || h < 1 || w < 1) return DIT_ATTN_ERR_SHAPE;
    if (f * h * w > seq_len) return DIT_ATTN_ERR_SHAPE;
    if (pos_mode == DIT_ATTN_POS_CENTERED_FHW && ((h & 1) || (w & 1))) return DIT_ATTN_ERR_SHAPE;
    if (pos_mode == DIT_ATTN_POS_GRID_HW && f != 1) return DIT_ATTN_ERR_SHAPE;
    a.shape[b][0] = (int32_t)f;
    a.shape[b][1] = (int32_t)h;
    a.shape[b][2] = (int32_t)w;
    a.frame_off[b] = (int32_t)frames;
    total += f * h * w;
    if (total > seq_len) return DIT_ATTN_ERR_SHAPE;
    a.cum[b + 1] = (int32_t)total;
    frames += f;
    const int64_t mc = std::max<int64_t>(frames - 1, std::max<int64_t>(h / 2 - 1, w / 2 - 1));
    if (mc > max_coord) max_coord = (int32_t)mc;
  }
  a.max_vid = n_img > 0 ? max_coord + 1 : 0;
  hipError_t e = dit::launch_token_meta(image_pad_mask, a, meta->image_ids, meta->target_mask, meta->pos_ids,
                                        meta->kv_limit, status_dev, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? DIT_ATTN_OK : DIT_ATTN_ERR_HIP;
}

int dit_attn_build_key_valid(const uint8_t* image_pad_mask, int32_t seq_len, const uint8_t* text_valid,
                             int32_t B, int32_t n_text, int64_t text_valid_stride, uint64_t* key_valid,
                             int64_t key_valid_stride, int32_t* status_dev, void* stream) {
  if (B < 0 || seq_len < 0 || n_text < 0) return DIT_ATTN_ERR_SHAPE;
  if (B == 0 || seq_len == 0) return DIT_ATTN_OK;  // nothing to do; no pointer is read
  if (!image_pad_mask || !key_valid || !status_dev || (n_text > 0 && !text_valid)) return DIT_ATTN_ERR_NULL;
  if (n_text > seq_len || text_valid_stride < n_text) return DIT_ATTN_ERR_SHAPE;
  if (key_valid_stride < ((int64_t)seq_len + 63) / 64) return DIT_ATTN_ERR_SHAPE;
  if (B > 65535) return DIT_ATTN_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(key_valid) & 7u) != 0) return DIT_ATTN_ERR_ALIGN;
  dit::KeyValidArgs a{};
  a.mask = image_pad_mask;
  a.text_valid = text_valid;
  a.bits = key_valid;
  a.status = status_dev;
  a.tv_stride = text_valid_stride;
  a.bits_stride = key_valid_stride;
  a.S = seq_len;
  a.B = B;
  a.n_text = n_text;
  hipError_t e = dit::launch_key_valid(a, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? DIT_ATTN_OK : DIT_ATTN_ERR_HIP;
}

// Rotary frequencies: pair j of axis a turns by (pos / linear) *
// (theta * ntk)^(-2j/d_a) radians; both factors fold into the pair's
// frequency, stored in turns (divided by 2 pi) for the kernels' reduction.
// Validates the axes (each even, summing to D) and the factors.
static int rope_frequencies(int32_t D, int32_t n_axes, const int32_t* axes_dims, float theta, float linear,
                            float ntk, double* omega, int32_t* pair_axis) {
  if (!axes_dims) return DIT_ATTN_ERR_NULL;
  if (n_axes < 1 || n_axes > 3) return DIT_ATTN_ERR_SHAPE;
  int sum = 0;
  for (int i = 0; i < n_axes; ++i) {
    if (axes_dims[i] < 0 || (axes_dims[i] & 1)) return DIT_ATTN_ERR_SHAPE;
    sum += axes_dims[i];
  }
  if (sum != D) return DIT_ATTN_ERR_SHAPE;
  if (!(theta > 0.f) || !std::isfinite(theta) || !(linear > 0.f) || !std::isfinite(linear) || !(ntk > 0.f) ||
      !std::isfinite(ntk))
    return DIT_ATTN_ERR_SHAPE;
  const double base = (double)theta * (double)ntk;
  int pr = 0;
  for (int ax = 0; ax < n_axes; ++ax) {
    const int da = axes_dims[ax];
    for (int j = 0; j < da / 2; ++j, ++pr) {
      omega[pr] = std::pow(base, -2.0 * j / da) / (double)linear / 6.283185307179586476925;
      pair_axis[pr] = ax;
    }
  }
  return DIT_ATTN_OK;
}

static int qknorm_rope_common(const void* q, const void* k, void* q_out, void* k_out, int32_t B, int32_t S,
                              int32_t H, int32_t H_kv, int32_t D, const int64_t q_strides[3],
                              const int64_t k_strides[3], const int64_t qo_strides[3], const int64_t ko_strides[3],
                              const int32_t* pos_ids, int32_t n_axes, const int32_t* axes_dims,
                              const dit_attn_norm_rope_params& p, int32_t dtype, void* stream) {
  if (B < 0 || S < 0) return DIT_ATTN_ERR_SHAPE;
  if (B == 0 || S == 0) return DIT_ATTN_OK;  // nothing to do; no pointer is read
  // Q may be left out (both q and q_out NULL): K only.
  const bool has_q = q != nullptr || q_out != nullptr;
  if ((has_q && (!q || !q_out || !q_strides || !qo_strides)) || !k || !k_out || !pos_ids || !axes_dims ||
      !k_strides || !ko_strides)
    return DIT_ATTN_ERR_NULL;
  if (dtype != DIT_ATTN_BF16 && dtype != DIT_ATTN_F32) return DIT_ATTN_ERR_UNSUPPORTED;
  if (p.norm != DIT_ATTN_NORM_RMS_PER_HEAD && p.norm != DIT_ATTN_NORM_LAYER_ACROSS_HEADS)
    return DIT_ATTN_ERR_UNSUPPORTED;
  if ((has_q && H < 1) || H_kv < 1) return DIT_ATTN_ERR_SHAPE;
  const int32_t Hq = has_q ? H : 0;
  if (B > 65535) return DIT_ATTN_ERR_UNSUPPORTED;
  const int chunk = dtype == DIT_ATTN_BF16 ? 8 : 4;
  if (D < 8 || D > kMaxDim || D % chunk != 0) return DIT_ATTN_ERR_UNSUPPORTED;
  if (p.norm == DIT_ATTN_NORM_LAYER_ACROSS_HEADS && (int64_t)(Hq + H_kv) * (D / chunk) > dit::kLayerNormMaxItems)
    return DIT_ATTN_ERR_UNSUPPORTED;
  dit::QkNormRopeArgs a{};
  const int rs = rope_frequencies(D, n_axes, axes_dims, p.rope_theta, p.rope_linear_factor, p.rope_ntk_factor,
                                  a.omega, a.pair_axis);
  if (rs != DIT_ATTN_OK) return rs;
  if (!(p.eps >= 0.f) || !std::isfinite(p.eps) || !std::isfinite(p.q_scale) || p.q_scale == 0.f)
    return DIT_ATTN_ERR_SHAPE;
  if ((has_q && (!strides_ok(q_strides) || !strides_ok(qo_strides))) || !strides_ok(k_strides) ||
      !strides_ok(ko_strides))
    return DIT_ATTN_ERR_SHAPE;
  const int es = elem_size(dtype);
  if ((has_q && (!rows_aligned(q, q_strides, es) || !rows_aligned(q_out, qo_strides, es))) ||
      !rows_aligned(k, k_strides, es) || !rows_aligned(k_out, ko_strides, es) ||
      (p.q_weight && !aligned16(p.q_weight)) || (p.k_weight && !aligned16(p.k_weight)) ||
      (p.q_bias && !aligned16(p.q_bias)) || (p.k_bias && !aligned16(p.k_bias)))
    return DIT_ATTN_ERR_ALIGN;

  a.q = q;
  a.k = k;
  a.qo = q_out;
  a.ko = k_out;
  a.wq = p.q_weight;
  a.wk = p.k_weight;
  a.norm = p.norm;
  if (p.norm == DIT_ATTN_NORM_LAYER_ACROSS_HEADS) {
    a.bq = p.q_bias;
    a.bk = p.k_bias;
  }
  a.pos = pos_ids;
  for (int i = 0; i < 3; ++i) {
    a.qs[i] = has_q ? q_strides[i] : 0;
    a.ks[i] = k_strides[i];
    a.qos[i] = has_q ? qo_strides[i] : 0;
    a.kos[i] = ko_strides[i];
  }
  a.B = B;
  a.S = S;
  a.H = Hq;
  a.Hk = H_kv;
  a.D = D;
  a.eps = p.eps;
  a.q_scale = p.q_scale;
  hipError_t e = dit::launch_qknorm_rope(a, dtype, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? DIT_ATTN_OK : DIT_ATTN_ERR_HIP;
}

int dit_attn_qknorm_rope(const void* q, const void* k, void* q_out, void* k_out, const void* q_weight,
                         const void* k_weight, int32_t B, int32_t S, int32_t H, int32_t H_kv, int32_t D,
                         const int64_t q_strides[3], const int64_t k_strides[3], const int64_t qo_strides[3],
                         const int64_t ko_strides[3], const int32_t* pos_ids, int32_t n_axes,
                         const int32_t* axes_dims, float rope_theta, float eps, float q_scale, int32_t dtype,
                         void* stream) {
  dit_attn_norm_rope_params p{};
  p.norm = DIT_ATTN_NORM_RMS_PER_HEAD;
  p.q_weight = q_weight;
  p.k_weight = k_weight;
  p.eps = eps;
  p.rope_theta = rope_theta;
  p.rope_linear_factor = 1.0f;
  p.rope_ntk_factor = 1.0f;
  p.q_scale = q_scale;
  return qknorm_rope_common(q, k, q_out, k_out, B, S, H, H_kv, D, q_strides, k_strides, qo_strides, ko_strides,
                            pos_ids, n_axes, axes_dims, p, dtype, stream);
}

int dit_attn_qknorm_rope_ex(const void* q, const void* k, void* q_out, void* k_out, int32_t B, int32_t S,
                            int32_t H, int32_t H_kv, int32_t D, const int64_t q_strides[3],
                            const int64_t k_strides[3], const int64_t qo_strides[3], const int64_t ko_strides[3],
                            const int32_t* pos_ids, int32_t n_axes, const int32_t* axes_dims,
                            const dit_attn_norm_rope_params* params, int32_t dtype, void* stream) {
  if (B < 0 || S < 0) return DIT_ATTN_ERR_SHAPE;
  if (B == 0 || S == 0) return DIT_ATTN_OK;
  if (!params) return DIT_ATTN_ERR_NULL;
  return qknorm_rope_common(q, k, q_out, k_out, B, S, H, H_kv, D, q_strides, k_strides, qo_strides, ko_strides,
                            pos_ids, n_axes, axes_dims, *params, dtype, stream);
}

int dit_attn_time_aware_rope_factors(float t, float watershed, float scaling_factor, float* linear_factor,
                                     float* ntk_factor) {
  if (!linear_factor || !ntk_factor) return DIT_ATTN_ERR_NULL;
  if (!(scaling_factor > 0.f) || !std::isfinite(scaling_factor) || !std::isfinite(t) || !std::isfinite(watershed))
    return DIT_ATTN_ERR_SHAPE;
  if (t < watershed) {
    *linear_factor = scaling_factor;
    *ntk_factor = 1.0f;
  } else {
    *linear_factor = 1.0f;
    *ntk_factor = scaling_factor;
  }
  return DIT_ATTN_OK;
}

int dit_attn_prescaled_q_factor(int32_t head_dim, float softmax_scale, float* q_scale_out) {
  if (!q_scale_out) return DIT_ATTN_ERR_NULL;
  if (head_dim < 1 || !std::isfinite(softmax_scale)) return DIT_ATTN_ERR_SHAPE;
  const double scale = softmax_scale > 0.f ? (double)softmax_scale : 1.0 / std::sqrt((double)head_dim);
  *q_scale_out = (float)(scale * 1.4426950408889634);
  return DIT_ATTN_OK;
}

// Fused Q norm for attention_common (NULL: Q is already normed and rotated).
struct QNormArgs {
  const void* q_weight;
  const int32_t* pos;  // [S_new][3]
  float eps, q_scale;
  const double* omega;       // [kMaxPairs], turns per position
  const int32_t* pair_axis;  // [kMaxPairs]
};

static int attention_common(const void* q, const void* kc, const void* vc, const void* kn, const void* vn, void* o,
                            float* lse, int32_t B, int32_t P, int32_t S_new, int32_t H, int32_t H_kv, int32_t D,
                            const int64_t* const st[6], int32_t mask_mode, const dit_attn_token_meta* meta,
                            const uint64_t* key_valid, int64_t key_valid_stride, float softmax_scale,
                            int32_t dtype, void* stream, const QNormArgs* qn = nullptr) {
  if (dtype != DIT_ATTN_BF16 && dtype != DIT_ATTN_F32) return DIT_ATTN_ERR_UNSUPPORTED;
  if (mask_mode != DIT_ATTN_MASK_FULL && mask_mode != DIT_ATTN_MASK_BLOCK_CAUSAL) return DIT_ATTN_ERR_UNSUPPORTED;
  if (B < 0 || P < 0 || S_new < 0 || H < 1 || H_kv < 1 || H % H_kv != 0) return DIT_ATTN_ERR_SHAPE;
  const int chunk = dtype == DIT_ATTN_BF16 ? 8 : 4;
  if (D < 8 || D > kMaxDim || D % chunk != 0) return DIT_ATTN_ERR_UNSUPPORTED;
  if ((int64_t)P + S_new > INT32_MAX) return DIT_ATTN_ERR_SHAPE;
  for (int i = 0; i < 6; ++i)
    if (!strides_ok(st[i])) return DIT_ATTN_ERR_SHAPE;
  const int32_t* kv_limit = nullptr;
  if (mask_mode == DIT_ATTN_MASK_BLOCK_CAUSAL) {
    if (!meta || !meta->kv_limit) return DIT_ATTN_ERR_NULL;
    if (meta->seq_len != P + S_new) return DIT_ATTN_ERR_SHAPE;
    kv_limit = meta->kv_limit;
  } else if (meta && meta->seq_len != P + S_new) {
    return DIT_ATTN_ERR_SHAPE;
  }
  const int es = elem_size(dtype);
  if (!rows_aligned(q, st[0], es) || !rows_aligned(kn, st[3], es) || !rows_aligned(vn, st[4], es) ||
      !rows_aligned(o, st[5], es))
    return DIT_ATTN_ERR_ALIGN;
  if (P > 0 && (!rows_aligned(kc, st[1], es) || !rows_aligned(vc, st[2], es))) return DIT_ATTN_ERR_ALIGN;
  if (key_valid && key_valid_stride < ((int64_t)P + S_new + 63) / 64) return DIT_ATTN_ERR_SHAPE;
  if (key_valid && (reinterpret_cast<uintptr_t>(key_valid) & 7u) != 0) return DIT_ATTN_ERR_ALIGN;
  if (B == 0 || S_new == 0) return DIT_ATTN_OK;
  // Keys are addressed with 32-bit byte offsets inside one (batch, kv-head) slice.
  const int64_t span_new = (int64_t)S_new * std::max(st[3][1], st[4][1]) * es;
  const int64_t span_cache = (int64_t)P * std::max(st[1][1], st[2][1]) * es;
  if (span_new >= INT32_MAX || span_cache >= INT32_MAX) return DIT_ATTN_ERR_UNSUPPORTED;
  const int64_t blocks = ((int64_t)S_new + 127) / 128 * B * H;
  if (blocks > INT32_MAX || ((int64_t)S_new + 63) / 64 * B * H > INT32_MAX) return DIT_ATTN_ERR_UNSUPPORTED;

  dit::AttnArgs a{};
  a.q = q;
  a.kc = P > 0 ? kc : kn;
  a.vc = P > 0 ? vc : vn;
  a.kn = kn;
  a.vn = vn;
  a.o = o;
  a.lse = lse;
  a.kv_limit = kv_limit;
  a.key_bits = key_valid;
  a.kb_stride = key_valid ? key_valid_stride : 0;
  for (int i = 0; i < 3; ++i) {
    a.qs[i] = st[0][i];
    a.kcs[i] = P > 0 ? st[1][i] : st[3][i];
    a.vcs[i] = P > 0 ? st[2][i] : st[4][i];
    a.kns[i] = st[3][i];
    a.vns[i] = st[4][i];
    a.os[i] = st[5][i];
  }
  a.B = B;
  a.H = H;
  a.Hk = H_kv;
  a.D = D;
  a.P = P;
  a.Snew = S_new;
  a.Sk = P + S_new;
  a.scale = (softmax_scale > 0.f && std::isfinite(softmax_scale)) ? softmax_scale : (float)(1.0 / std::sqrt((double)D));
  if (qn != nullptr) {
    // The scale (and log2 e) go into Q with its norm; the kernel then
    // exponentiates its MFMA output directly (scale argument ln 2).
    a.wq = qn->q_weight;
    a.qpos = qn->pos;
    a.eps = qn->eps;
    a.q_scale = (float)((double)a.scale * 1.4426950408889634 * (double)qn->q_scale);
    // Each pair's frequency under its own axis, 0 under the others.
    for (int i = 0; i < dit::kMaxPairs; ++i)
      for (int ax = 0; ax < 3; ++ax) a.omega_axis[ax][i] = qn->pair_axis[i] == ax ? qn->omega[i] : 0.0;
    a.scale = 0.6931471805599453f;
  }
  hipError_t e = dit::launch_attention(a, dtype, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? DIT_ATTN_OK : DIT_ATTN_ERR_HIP;
}

int dit_attn_forward(const void* q, const void* k, const void* v, void* o, float* lse, int32_t B, int32_t S,
                     int32_t H, int32_t H_kv, int32_t D, const int64_t strides[4][3], int32_t mask_mode,
                     const dit_attn_token_meta* meta, float softmax_scale, int32_t dtype, void* stream) {
  if (B < 0 || S < 0) return DIT_ATTN_ERR_SHAPE;
  if (B == 0 || S == 0) return DIT_ATTN_OK;  // nothing to do; no pointer is read
  if (!q || !k || !v || !o || !strides) return DIT_ATTN_ERR_NULL;
  const int64_t* st[6] = {strides[0], strides[1], strides[2], strides[1], strides[2], strides[3]};
  return attention_common(q, k, v, k, v, o, lse, B, 0, S, H, H_kv, D, st, mask_mode, meta, nullptr, 0,
                          softmax_scale, dtype, stream);
}

int dit_attn_forward_padded(const void* q, const void* k, const void* v, void* o, float* lse, int32_t B,
                            int32_t S, int32_t H, int32_t H_kv, int32_t D, const int64_t strides[4][3],
                            int32_t mask_mode, const dit_attn_token_meta* meta, const uint64_t* key_valid,
                            int64_t key_valid_stride, float softmax_scale, int32_t dtype, void* stream) {
  if (B < 0 || S < 0) return DIT_ATTN_ERR_SHAPE;
  if (B == 0 || S == 0) return DIT_ATTN_OK;  // nothing to do; no pointer is read
  if (!q || !k || !v || !o || !strides || !key_valid) return DIT_ATTN_ERR_NULL;
  const int64_t* st[6] = {strides[0], strides[1], strides[2], strides[1], strides[2], strides[3]};
  return attention_common(q, k, v, k, v, o, lse, B, 0, S, H, H_kv, D, st, mask_mode, meta, key_valid,
                          key_valid_stride, softmax_scale, dtype, stream);
}

int dit_attn_forward_cached(const void* q_new, const void* k_cache, const void* v_cache, const void* k_new,
                            const void* v_new, void* o, float* lse, int32_t B, int32_t P, int32_t S_new, int32_t H,
                            int32_t H_kv, int32_t D, const int64_t strides[6][3], int32_t mask_mode,
                            const dit_attn_token_meta* meta, float softmax_scale, int32_t dtype, void* stream) {
  if (B < 0 || P < 0 || S_new < 0) return DIT_ATTN_ERR_SHAPE;
  if (B == 0 || S_new == 0) return DIT_ATTN_OK;  // nothing to do; no pointer is read
  if (!q_new || !k_new || !v_new || !o || !strides) return DIT_ATTN_ERR_NULL;
  if (P > 0 && (!k_cache || !v_cache)) return DIT_ATTN_ERR_NULL;
  const int64_t* st[6] = {strides[0], strides[1], strides[2], strides[3], strides[4], strides[5]};
  return attention_common(q_new, k_cache, v_cache, k_new, v_new, o, lse, B, P, S_new, H, H_kv, D, st, mask_mode,
                          meta, nullptr, 0, softmax_scale, dtype, stream);
}

int dit_attn_forward_cached_padded(const void* q_new, const void* k_cache, const void* v_cache, const void* k_new,
                                   const void* v_new, void* o, float* lse, int32_t B, int32_t P, int32_t S_new,
                                   int32_t H, int32_t H_kv, int32_t D, const int64_t strides[6][3],
                                   int32_t mask_mode, const dit_attn_token_meta* meta, const uint64_t* key_valid,
                                   int64_t key_valid_stride, float softmax_scale, int32_t dtype, void* stream) {
  if (B < 0 || P < 0 || S_new < 0) return DIT_ATTN_ERR_SHAPE;
  if (B == 0 || S_new == 0) return DIT_ATTN_OK;  // nothing to do; no pointer is read
  if (!q_new || !k_new || !v_new || !o || !strides || !key_valid) return DIT_ATTN_ERR_NULL;
  if (P > 0 && (!k_cache || !v_cache)) return DIT_ATTN_ERR_NULL;
  const int64_t* st[6] = {strides[0], strides[1], strides[2], strides[3], strides[4], strides[5]};
  return attention_common(q_new, k_cache, v_cache, k_new, v_new, o, lse, B, P, S_new, H, H_kv, D, st, mask_mode,
                          meta, key_valid, key_valid_stride, softmax_scale, dtype, stream);
}

int dit_attn_forward_cached_qnorm(const void* q_new_raw, const void* k_cache, const void* v_cache, const void* k_new,
                                  const void* v_new, void* o, float* lse, int32_t B, int32_t P, int32_t S_new,
                                  int32_t H, int32_t H_kv, int32_t D, const int64_t strides[6][3], int32_t mask_mode,
                                  const dit_attn_token_meta* meta, const uint64_t* key_valid,
                                  int64_t key_valid_stride, const int32_t* pos_ids, int32_t n_axes,
                                  const int32_t* axes_dims, const dit_attn_norm_rope_params* params,
                                  float softmax_scale, int32_t dtype, void* stream) {
  if (B < 0 || P < 0 || S_new < 0) return DIT_ATTN_ERR_SHAPE;
  if (B == 0 || S_new == 0) return DIT_ATTN_OK;  // nothing to do; no pointer is read
  if (!q_new_raw || !k_new || !v_new || !o || !strides || !pos_ids || !params) return DIT_ATTN_ERR_NULL;
  if (P > 0 && (!k_cache || !v_cache)) return DIT_ATTN_ERR_NULL;
  if (dtype != DIT_ATTN_BF16) return DIT_ATTN_ERR_UNSUPPORTED;  // the fused form is bf16 only
  if (params->norm != DIT_ATTN_NORM_RMS_PER_HEAD) return DIT_ATTN_ERR_UNSUPPORTED;
  if (D < 8 || D > kMaxDim) return DIT_ATTN_ERR_UNSUPPORTED;
  double omega[dit::kMaxPairs] = {};
  int32_t pair_axis[dit::kMaxPairs] = {};
  const int rs = rope_frequencies(D, n_axes, axes_dims, params->rope_theta, params->rope_linear_factor,
                                  params->rope_ntk_factor, omega, pair_axis);
  if (rs != DIT_ATTN_OK) return rs;
  if (!(params->eps >= 0.f) || !std::isfinite(params->eps) || !std::isfinite(params->q_scale) ||
      params->q_scale == 0.f)
    return DIT_ATTN_ERR_SHAPE;
  if (params->q_weight && !aligned16(params->q_weight)) return DIT_ATTN_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(pos_ids) & 3u) return DIT_ATTN_ERR_ALIGN;
  const int64_t* st[6] = {strides[0], strides[1], strides[2], strides[3], strides[4], strides[5]};
  QNormArgs qn{params->q_weight, pos_ids, params->eps, params->q_scale, omega, pair_axis};
  return attention_common(q_new_raw, k_cache, v_cache, k_new, v_new, o, lse, B, P, S_new, H, H_kv, D, st, mask_mode,
                          meta, key_valid, key_valid_stride, softmax_scale, dtype, stream, &qn);
}

int dit_attn_cfg_norm_rescale(const void* cond, const void* uncond, void* out, int64_t rows, int32_t channels,
                              int64_t cond_stride, int64_t uncond_stride, int64_t out_stride, float guidance_scale,
                              int32_t dtype, void* stream) {
  if (rows < 0 || channels < 1) return DIT_ATTN_ERR_SHAPE;
  if (rows == 0) return DIT_ATTN_OK;  // nothing to do; no pointer is read
  if (!cond || !uncond || !out) return DIT_ATTN_ERR_NULL;
  if (dtype != DIT_ATTN_BF16 && dtype != DIT_ATTN_F32) return DIT_ATTN_ERR_UNSUPPORTED;
  const int chunk = dtype == DIT_ATTN_BF16 ? 8 : 4;
  if (channels % chunk != 0) return DIT_ATTN_ERR_UNSUPPORTED;
  if (channels / chunk > 64 * 8) return DIT_ATTN_ERR_UNSUPPORTED;
  if (!std::isfinite(guidance_scale)) return DIT_ATTN_ERR_SHAPE;
  if (cond_stride < channels || uncond_stride < channels || out_stride < channels) return DIT_ATTN_ERR_SHAPE;
  if (rows > (int64_t)INT32_MAX * 8) return DIT_ATTN_ERR_UNSUPPORTED;
  const int es = elem_size(dtype);
  if (!aligned16(cond) || !aligned16(uncond) || !aligned16(out) || (cond_stride * es) % 16 ||
      (uncond_stride * es) % 16 || (out_stride * es) % 16)
    return DIT_ATTN_ERR_ALIGN;
  dit::CfgArgs a{};
  a.cond = cond;
  a.uncond = uncond;
  a.out = out;
  a.rows = rows;
  a.cs = cond_stride;
  a.us = uncond_stride;
  a.os = out_stride;
  a.C = channels;
  a.g = guidance_scale;
  hipError_t e = dit::launch_cfg_norm_rescale(a, dtype, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? DIT_ATTN_OK : DIT_ATTN_ERR_HIP;
}

}  // extern "C"
