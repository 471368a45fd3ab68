// Launch interface between the C-ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

constexpr int kMaxImages = 64;

// Token metadata: host-validated image-block shapes and derived constants.
struct TokenMetaArgs {
  int32_t seq_len;
  int32_t n_img;
  int32_t pos_mode;               // 0 centred (f, h, w); 1 grid (h, w)
  int32_t max_vid;                // first text position (centred mode)
  int32_t shape[kMaxImages][3];   // (frames, height, width)
  int32_t cum[kMaxImages + 1];    // cumulative token counts, cum[0] = 0
  int32_t frame_off[kMaxImages];  // sum of frames of the earlier blocks
};

hipError_t launch_token_meta(const uint8_t* mask, const TokenMetaArgs& a, int32_t* image_ids, uint8_t* target,
                             int32_t* pos, int32_t* kv_limit, int32_t* status, hipStream_t stream);

// Per-sample key validity bits of the joint sequence from a text mask.
struct KeyValidArgs {
  const uint8_t* mask;        // [S] nonzero on image tokens
  const uint8_t* text_valid;  // [B][n_text], row stride tv_stride bytes
  uint64_t* bits;             // [B][bits_stride] words; bit j of word t: key 64 t + j
  int32_t* status;
  int64_t tv_stride, bits_stride;
  int32_t S, B, n_text;
};

hipError_t launch_key_valid(const KeyValidArgs& a, hipStream_t stream);

// Fused QK-RMSNorm + rotary embedding.
constexpr int kMaxPairs = 64;  // head_dim <= 128

struct QkNormRopeArgs {
  const void* q;
  const void* k;
  void* qo;
  void* ko;
  const void* wq;  // nullable: unit weight ([D] per head, or [H*D] / [Hk*D] across heads)
  const void* wk;
  const void* bq;  // nullable: zero bias (LayerNorm across heads only)
  const void* bk;
  int32_t norm;    // 0: RMSNorm per head; 1: LayerNorm across heads
  const int32_t* pos;  // [S][3]
  int64_t qs[3], ks[3], qos[3], kos[3];
  int32_t B, S, H, Hk, D;
  float eps;
  float q_scale;                 // extra factor on Q outputs
  double omega[kMaxPairs];       // frequency of channel pair p, in turns per position
  int32_t pair_axis[kMaxPairs];  // axis that owns pair p
};

hipError_t launch_qknorm_rope(const QkNormRopeArgs& a, int dtype, hipStream_t stream);

// Most (head, chunk) items per token of the LayerNorm-across-heads kernel.
constexpr int kLayerNormMaxItems = 2048;

// Attention over a (possibly cached) key sequence.  Keys 0..P-1 come from the
// cache pointers, keys P..P+Snew-1 from the new-token pointers; query row i is
// logical token P + i.
struct AttnArgs {
  const void* q;
  const void* kc;
  const void* vc;
  const void* kn;
  const void* vn;
  void* o;
  float* lse;                // nullable
  const int32_t* kv_limit;   // logical-sequence bound per token; null for the full mask
  const uint64_t* key_bits;  // nullable: per-sample key validity, bit j of word t = key 64 t + j
  int64_t kb_stride;         // words per sample of key_bits
  int64_t qs[3], kcs[3], vcs[3], kns[3], vns[3], os[3];
  int32_t B, H, Hk, D, P, Snew, Sk;
  float scale;               // softmax scale
  // Fused Q norm, active when qpos is set (q then holds raw Q): per-head
  // RMSNorm with weight wq (nullable: unit) and eps, the rotary embedding of
  // each query's token and the factor q_scale, rounded once to bf16.  Pair p
  // turns by sum_a qpos[3 i + a] * omega_axis[a][p] turns: omega_axis holds
  // the pair's frequency under the axis that owns it and 0 under the others,
  // so the sum is exactly the norm kernel's pos * omega.
  const void* wq;
  const int32_t* qpos;       // [Snew][3] positions of the query tokens
  float eps, q_scale;
  double omega_axis[3][kMaxPairs];
};

hipError_t launch_attention(const AttnArgs& a, int dtype, hipStream_t stream);

// Norm-rescaled classifier-free guidance over rows of C channels.
struct CfgArgs {
  const void* cond;
  const void* uncond;
  void* out;
  int64_t rows, cs, us, os;  // row count; row strides in elements
  int32_t C;
  float g;                   // guidance scale
};

hipError_t launch_cfg_norm_rescale(const CfgArgs& a, int dtype, hipStream_t stream);

}  // namespace dit
