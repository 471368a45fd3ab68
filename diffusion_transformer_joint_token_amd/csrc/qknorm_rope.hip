// Fused per-head RMSNorm + multi-axis rotary embedding of Q and K (gfx950).
//
// NucleusMoE-Image pipeline article, section 6.3: Q and K are RMS-normalised
// per head (qk_norm = rms_norm) and then rotated by the rotary embedding built
// over the (frame, height, width) axes (axes_dims_rope (16, 56, 56)).  The
// Lumina-Next DiT article (configuration table, section 4) gives the 2D split
// (head_dim / 2 channels per axis, hence head_dim % 4 == 0) and a complex
// rotary table, i.e. adjacent channel pairs turned by a phase.
//
// HBM-bound: each element is read once and written once.  One work-group
// handles one token (b, s) for all H query heads and H_kv key heads, so the
// token's rotary phases (one cos/sin per channel pair) are computed once
// (whole turns removed in double precision, then sin/cos in fp32: see
// sincos_turns) and shared by every head.
// A group of LPH lanes owns one head; each lane holds a 16-byte chunk of it
// (8 bf16 or 4 fp32), so loads and stores are full 16-byte vectors and a
// head's sum of squares is a butterfly over LPH lanes.  When a head's chunk
// count is not a power of two (head_dim 72 in bf16: 9 chunks) a flat mapping
// of (head, chunk) items over 1-4 tokens per work-group is used instead.
//
// Lumina-Next DiT article, section 3: with qk_norm its self-attention uses a
// LayerNorm across heads instead -- one mean and variance over all of a
// token's Q channels (and separately its K channels), then a per-channel
// weight and bias.  qk_layernorm_rope_kernel handles that: one work-group per
// token, (head, chunk) items dealt to the threads, mean and then centred
// variance each reduced by wave butterflies and a fixed-order sum over the
// waves (so results do not depend on timing).  The article's time-aware
// rotary scaling (section 4) needs no kernel change: the host folds the
// linear and NTK factors into each pair's frequency.

#include "device_common.h"
#include "kernels.h"

namespace dit {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxIter = 4;  // heads per lane-group kept in flight

template <typename T>
struct Elem;
template <>
struct Elem<__bf16> {
  static constexpr int kPerChunk = 8;
  __device__ static void unpack(const u32x4& w, float* x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_lo(w[i]);
      x[2 * i + 1] = bf16_hi(w[i]);
    }
  }
  __device__ static u32x4 pack(const float* y) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(y[2 * i], y[2 * i + 1]);
    return w;
  }
};
template <>
struct Elem<float> {
  static constexpr int kPerChunk = 4;
  __device__ static void unpack(const u32x4& w, float* x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __builtin_bit_cast(float, static_cast<uint32_t>(w[i]));
  }
  __device__ static u32x4 pack(const float* y) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __builtin_bit_cast(uint32_t, y[i]);
    return w;
  }
};

template <typename T, int LPH>
__global__ __launch_bounds__(kThreads) void qknorm_rope_kernel(QkNormRopeArgs a) {
  constexpr int EPC = Elem<T>::kPerChunk;  // elements per 16-byte chunk
  constexpr int SLOTS = kThreads / LPH;    // heads processed side by side
  __shared__ float2 s_cs[kMaxPairs];

  const int tid = threadIdx.x;
  const int slot = tid / LPH;
  const int sub = tid % LPH;
  const int s = blockIdx.x;
  const int b = blockIdx.y;
  const int D = a.D;
  const int nvh = a.H + a.Hk;
  const bool lane_active = sub * EPC < D;  // D is a multiple of EPC

  // Per-channel weights for this lane's chunk.
  float wq[EPC], wk[EPC];
  {
    u32x4 raw;
    if (a.wq != nullptr && lane_active) {
      raw = *reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(a.wq) + sub * EPC);
      Elem<T>::unpack(raw, wq);
    } else {
#pragma unroll
      for (int i = 0; i < EPC; ++i) wq[i] = 1.0f;
    }
    if (a.wk != nullptr && lane_active) {
      raw = *reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(a.wk) + sub * EPC);
      Elem<T>::unpack(raw, wk);
    } else {
#pragma unroll
      for (int i = 0; i < EPC; ++i) wk[i] = 1.0f;
    }
  }

  bool first = true;
  for (int vh0 = 0; vh0 < nvh; vh0 += SLOTS * kMaxIter) {
    // Issue the loads of up to kMaxIter heads before any arithmetic.
    u32x4 raw[kMaxIter];
#pragma unroll
    for (int it = 0; it < kMaxIter; ++it) {
      const int vh = vh0 + it * SLOTS + slot;
      raw[it] = u32x4{0, 0, 0, 0};
      if (vh < nvh && lane_active) {
        const T* src;
        if (vh < a.H)
          src = reinterpret_cast<const T*>(a.q) + b * a.qs[0] + (int64_t)s * a.qs[1] + vh * a.qs[2];
        else
          src = reinterpret_cast<const T*>(a.k) + b * a.ks[0] + (int64_t)s * a.ks[1] + (vh - a.H) * a.ks[2];
        raw[it] = *reinterpret_cast<const u32x4*>(src + sub * EPC);
      }
    }
    if (first) {
      // Rotary phases of this token, one per channel pair: pos * omega turns,
      // formed in double.
      if (tid < D / 2) {
        const int ax = a.pair_axis[tid];
        float sn, cs;
        sincos_turns((double)a.pos[3 * s + ax] * a.omega[tid], sn, cs);
        s_cs[tid] = make_float2(cs, sn);
      }
      __syncthreads();
      first = false;
    }
#pragma unroll
    for (int it = 0; it < kMaxIter; ++it) {
      const int vh = vh0 + it * SLOTS + slot;
      const bool is_q = vh < a.H;
      float x[EPC];
      Elem<T>::unpack(raw[it], x);
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < EPC; ++i) ss = fmaf(x[i], x[i], ss);
#pragma unroll
      for (int m = LPH / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
      const float inv = 1.0f / sqrtf(ss / (float)D + a.eps) * (is_q ? a.q_scale : 1.0f);
      float y[EPC];
#pragma unroll
      for (int i = 0; i < EPC; ++i) y[i] = x[i] * inv * (is_q ? wq[i] : wk[i]);
#pragma unroll
      for (int i = 0; i < EPC / 2; ++i) {
        const float2 cs = s_cs[(sub * EPC) / 2 + i < kMaxPairs ? (sub * EPC) / 2 + i : 0];
        const float y0 = y[2 * i], y1 = y[2 * i + 1];
        y[2 * i] = y0 * cs.x - y1 * cs.y;
        y[2 * i + 1] = y0 * cs.y + y1 * cs.x;
      }
      if (vh < nvh && lane_active) {
        T* dst;
        if (is_q)
          dst = reinterpret_cast<T*>(a.qo) + b * a.qos[0] + (int64_t)s * a.qos[1] + vh * a.qos[2];
        else
          dst = reinterpret_cast<T*>(a.ko) + b * a.kos[0] + (int64_t)s * a.kos[1] + (vh - a.H) * a.kos[2];
        *reinterpret_cast<u32x4*>(dst + sub * EPC) = Elem<T>::pack(y);
      }
    }
  }
}

// Flat mapping for any number of 16-byte chunks per head (CPH = D / EPC):
// the TPW tokens of a work-group hold TPW * (H + H_kv) * CPH (head, chunk)
// items, dealt to the threads in order, so a head of 9 chunks (head_dim 72 in
// bf16) does not leave 7 of 16 lanes idle.  A head's sum of squares is formed
// through LDS: each item stores its partial, and after a barrier each item
// adds the CPH partials of its head.
constexpr int kFlatItems = 4;  // items per thread kept in flight
constexpr int kFlatTokens = 16; // most tokens per work-group

template <typename T>
__global__ __launch_bounds__(kThreads) void qknorm_rope_flat_kernel(QkNormRopeArgs a, int tpw) {
  constexpr int EPC = Elem<T>::kPerChunk;
  __shared__ float2 s_cs[kFlatTokens][kMaxPairs];
  __shared__ float s_ss[kThreads * kFlatItems];

  const int tid = threadIdx.x;
  const int b = blockIdx.y;
  const int D = a.D;
  const int cph = D / EPC;
  const int nvh = a.H + a.Hk;
  const int per_tok = nvh * cph;
  const int s0 = blockIdx.x * tpw;
  const int n_items = min(tpw, a.S - s0) * per_tok;

  // Decode and load this thread's items: item = tt * per_tok + vh * cph + c.
  int it_vh[kFlatItems], it_c[kFlatItems], it_t[kFlatItems];
  u32x4 raw[kFlatItems];
#pragma unroll
  for (int k = 0; k < kFlatItems; ++k) {
    const int item = tid + k * kThreads;
    const int tt = item / per_tok;
    const int rem = item - tt * per_tok;
    const int vh = rem / cph;
    it_t[k] = tt;
    it_vh[k] = vh;
    it_c[k] = rem - vh * cph;
    raw[k] = u32x4{0, 0, 0, 0};
    if (item < n_items) {
      const int s = s0 + tt;
      const T* src;
      if (vh < a.H)
        src = reinterpret_cast<const T*>(a.q) + b * a.qs[0] + (int64_t)s * a.qs[1] + vh * a.qs[2];
      else
        src = reinterpret_cast<const T*>(a.k) + b * a.ks[0] + (int64_t)s * a.ks[1] + (vh - a.H) * a.ks[2];
      raw[k] = *reinterpret_cast<const u32x4*>(src + it_c[k] * EPC);
    }
  }
  // Rotary phases of the work-group's tokens (as in the per-head kernel).
  for (int p = tid; p < tpw * (D / 2); p += kThreads) {
    const int tt = p / (D / 2), j = p - tt * (D / 2);
    const int s = min(s0 + tt, a.S - 1);
    float sn, cs;
    sincos_turns((double)a.pos[3 * s + a.pair_axis[j]] * a.omega[j], sn, cs);
    s_cs[tt][j] = make_float2(cs, sn);
  }
  // Partial sums of squares.
  float x[kFlatItems][EPC];
#pragma unroll
  for (int k = 0; k < kFlatItems; ++k) {
    Elem<T>::unpack(raw[k], x[k]);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < EPC; ++i) ss = fmaf(x[k][i], x[k][i], ss);
    s_ss[tid + k * kThreads] = ss;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kFlatItems; ++k) {
    const int item = tid + k * kThreads;
    if (item >= n_items) continue;
    const int head0 = item - it_c[k];  // first item of this head
    float ss = 0.f;
    for (int c = 0; c < cph; ++c) ss += s_ss[head0 + c];
    const bool is_q = it_vh[k] < a.H;
    const float inv = 1.0f / sqrtf(ss / (float)D + a.eps) * (is_q ? a.q_scale : 1.0f);
    float wv[EPC];
    {
      const T* wp = reinterpret_cast<const T*>(is_q ? a.wq : a.wk);
      if (wp != nullptr) {
        Elem<T>::unpack(*reinterpret_cast<const u32x4*>(wp + it_c[k] * EPC), wv);
      } else {
#pragma unroll
        for (int i = 0; i < EPC; ++i) wv[i] = 1.0f;
      }
    }
    float y[EPC];
#pragma unroll
    for (int i = 0; i < EPC; ++i) y[i] = x[k][i] * inv * wv[i];
#pragma unroll
    for (int i = 0; i < EPC / 2; ++i) {
      const float2 cs = s_cs[it_t[k]][(it_c[k] * EPC) / 2 + i];
      const float y0 = y[2 * i], y1 = y[2 * i + 1];
      y[2 * i] = y0 * cs.x - y1 * cs.y;
      y[2 * i + 1] = y0 * cs.y + y1 * cs.x;
    }
    const int s = s0 + it_t[k];
    T* dst;
    if (is_q)
      dst = reinterpret_cast<T*>(a.qo) + b * a.qos[0] + (int64_t)s * a.qos[1] + it_vh[k] * a.qos[2];
    else
      dst = reinterpret_cast<T*>(a.ko) + b * a.kos[0] + (int64_t)s * a.kos[1] + (it_vh[k] - a.H) * a.kos[2];
    *reinterpret_cast<u32x4*>(dst + it_c[k] * EPC) = Elem<T>::pack(y);
  }
}

// LayerNorm across heads: TOK tokens per work-group; item k of thread t is
// (head, chunk) number t + 256 k of each token, Q heads first, so a thread
// loads each channel's weight and bias once for all its tokens.
constexpr int kLnMaxItems = 8;

// Per token, the sum of a Q partial and of a K partial over the work-group,
// in a fixed order (the same tree for any TOK).
template <int TOK>
__device__ __forceinline__ void block_sums(float (&vq)[TOK], float (&vk)[TOK], float2 (*red)[TOK][kThreads / 64]) {
#pragma unroll
  for (int t = 0; t < TOK; ++t)
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      vq[t] += __shfl_xor(vq[t], m, 64);
      vk[t] += __shfl_xor(vk[t], m, 64);
    }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0)
#pragma unroll
    for (int t = 0; t < TOK; ++t) (*red)[t][wave] = make_float2(vq[t], vk[t]);
  __syncthreads();
#pragma unroll
  for (int t = 0; t < TOK; ++t) {
    float2 u = (*red)[t][0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) {
      u.x += (*red)[t][w].x;
      u.y += (*red)[t][w].y;
    }
    vq[t] = u.x;
    vk[t] = u.y;
  }
}

template <typename T, int ITEMS, int TOK>
__global__ __launch_bounds__(kThreads) void qk_layernorm_rope_kernel(QkNormRopeArgs a) {
  constexpr int EPC = Elem<T>::kPerChunk;
  __shared__ float2 s_cs[TOK][kMaxPairs];
  __shared__ float2 s_red[2][TOK][kThreads / 64];

  const int tid = threadIdx.x;
  const int s0 = blockIdx.x * TOK;
  const int b = blockIdx.y;
  const int D = a.D;
  const int cph = D / EPC;
  const int nq = a.H * cph;
  const int n = (a.H + a.Hk) * cph;

  u32x4 raw[TOK][ITEMS];
#pragma unroll
  for (int t = 0; t < TOK; ++t)
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      const int item = tid + k * kThreads;
      const int s = s0 + t;
      raw[t][k] = u32x4{0, 0, 0, 0};
      if (item < n && s < a.S) {
        const int vh = item / cph, c = item - vh * cph;
        const T* src;
        if (vh < a.H)
          src = reinterpret_cast<const T*>(a.q) + b * a.qs[0] + (int64_t)s * a.qs[1] + vh * a.qs[2];
        else
          src = reinterpret_cast<const T*>(a.k) + b * a.ks[0] + (int64_t)s * a.ks[1] + (vh - a.H) * a.ks[2];
        raw[t][k] = *reinterpret_cast<const u32x4*>(src + c * EPC);
      }
    }
  if (tid < TOK * (D / 2)) {  // rotary phases of these tokens, as in the per-head kernel
    const int t = tid / (D / 2), j = tid - t * (D / 2);
    const int s = min(s0 + t, a.S - 1);
    float sn, cs;
    sincos_turns((double)a.pos[3 * s + a.pair_axis[j]] * a.omega[j], sn, cs);
    s_cs[t][j] = make_float2(cs, sn);
  }

  // Mean of each token's Q channels and of its K channels.
  float x[TOK][ITEMS][EPC];
  float sq[TOK], sk[TOK];
#pragma unroll
  for (int t = 0; t < TOK; ++t) {
    sq[t] = 0.f;
    sk[t] = 0.f;
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      Elem<T>::unpack(raw[t][k], x[t][k]);
      float u = 0.f;
#pragma unroll
      for (int i = 0; i < EPC; ++i) u += x[t][k][i];
      if (tid + k * kThreads < nq) sq[t] += u; else sk[t] += u;  // items past n hold zeros
    }
  }
  block_sums<TOK>(sq, sk, &s_red[0]);
  float mq[TOK], mk[TOK];
#pragma unroll
  for (int t = 0; t < TOK; ++t) {
    mq[t] = sq[t] / (float)(a.H * D);
    mk[t] = sk[t] / (float)(a.Hk * D);
  }
  // Centred variance.
  float vq[TOK], vk[TOK];
#pragma unroll
  for (int t = 0; t < TOK; ++t) {
    vq[t] = 0.f;
    vk[t] = 0.f;
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      const int item = tid + k * kThreads;
      if (item >= n) continue;
      const float m = item < nq ? mq[t] : mk[t];
      float u = 0.f;
#pragma unroll
      for (int i = 0; i < EPC; ++i) {
        const float d = x[t][k][i] - m;
        u = fmaf(d, d, u);
      }
      if (item < nq) vq[t] += u; else vk[t] += u;
    }
  }
  block_sums<TOK>(vq, vk, &s_red[1]);
  float rq[TOK], rk[TOK];
#pragma unroll
  for (int t = 0; t < TOK; ++t) {
    rq[t] = 1.0f / sqrtf(vq[t] / (float)(a.H * D) + a.eps);
    rk[t] = 1.0f / sqrtf(vk[t] / (float)(a.Hk * D) + a.eps);
  }

#pragma unroll
  for (int k = 0; k < ITEMS; ++k) {
    const int item = tid + k * kThreads;
    if (item >= n) continue;
    const int vh = item / cph, c = item - vh * cph;
    const bool is_q = vh < a.H;
    const int ch0 = (is_q ? vh : vh - a.H) * D + c * EPC;  // channel within the heads' span
    float wv[EPC], bv[EPC];
    {
      const T* wp = reinterpret_cast<const T*>(is_q ? a.wq : a.wk);
      const T* bp = reinterpret_cast<const T*>(is_q ? a.bq : a.bk);
      if (wp != nullptr) {
        Elem<T>::unpack(*reinterpret_cast<const u32x4*>(wp + ch0), wv);
      } else {
#pragma unroll
        for (int i = 0; i < EPC; ++i) wv[i] = 1.0f;
      }
      if (bp != nullptr) {
        Elem<T>::unpack(*reinterpret_cast<const u32x4*>(bp + ch0), bv);
      } else {
#pragma unroll
        for (int i = 0; i < EPC; ++i) bv[i] = 0.0f;
      }
    }
    const float sc = is_q ? a.q_scale : 1.0f;
#pragma unroll
    for (int t = 0; t < TOK; ++t) {
      const int s = s0 + t;
      if (s >= a.S) continue;
      const float m = is_q ? mq[t] : mk[t], r = is_q ? rq[t] : rk[t];
      float y[EPC];
#pragma unroll
      for (int i = 0; i < EPC; ++i) y[i] = fmaf((x[t][k][i] - m) * r, wv[i], bv[i]) * sc;
#pragma unroll
      for (int i = 0; i < EPC / 2; ++i) {
        const float2 cs = s_cs[t][(c * EPC) / 2 + i];
        const float y0 = y[2 * i], y1 = y[2 * i + 1];
        y[2 * i] = y0 * cs.x - y1 * cs.y;
        y[2 * i + 1] = y0 * cs.y + y1 * cs.x;
      }
      T* dst;
      if (is_q)
        dst = reinterpret_cast<T*>(a.qo) + b * a.qos[0] + (int64_t)s * a.qos[1] + vh * a.qos[2];
      else
        dst = reinterpret_cast<T*>(a.ko) + b * a.kos[0] + (int64_t)s * a.kos[1] + (vh - a.H) * a.kos[2];
      *reinterpret_cast<u32x4*>(dst + c * EPC) = Elem<T>::pack(y);
    }
  }
}

template <typename T>
hipError_t launch_layernorm(const QkNormRopeArgs& a, hipStream_t stream) {
  constexpr int EPC = Elem<T>::kPerChunk;
  const int n = (a.H + a.Hk) * (a.D / EPC);
  // Two tokens per work-group while a thread holds at most two items of each,
  // so each thread keeps up to four loads in flight.
  const dim3 grid1(a.S, a.B), grid2((a.S + 1) / 2, a.B);
  if (n <= kThreads)
    hipLaunchKernelGGL((qk_layernorm_rope_kernel<T, 1, 2>), grid2, dim3(kThreads), 0, stream, a);
  else if (n <= 2 * kThreads)
    hipLaunchKernelGGL((qk_layernorm_rope_kernel<T, 2, 2>), grid2, dim3(kThreads), 0, stream, a);
  else if (n <= 4 * kThreads)
    hipLaunchKernelGGL((qk_layernorm_rope_kernel<T, 4, 1>), grid1, dim3(kThreads), 0, stream, a);
  else if (n <= kLnMaxItems * kThreads)
    hipLaunchKernelGGL((qk_layernorm_rope_kernel<T, kLnMaxItems, 1>), grid1, dim3(kThreads), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename T>
hipError_t launch_typed(const QkNormRopeArgs& a, hipStream_t stream) {
  if (a.norm == 1) return launch_layernorm<T>(a, stream);
  constexpr int EPC = Elem<T>::kPerChunk;
  const int chunks = a.D / EPC;
  const int per_tok = (a.H + a.Hk) * chunks;
  // Tokens per work-group: the count (1..16) that leaves the fewest idle item
  // slots per token, within the items a work-group keeps in flight.  A small
  // token (8 KV heads x 9 chunks) thus shares its work-group with 13 others
  // instead of leaving most of the slots idle.
  // A power-of-two chunk count fills whole lane groups: one head per group
  // with a butterfly sum is faster there.
  int tpw = 0;
  long best_idle = 0;
  const bool pow2 = (chunks & (chunks - 1)) == 0;
  for (int t = 1; !pow2 && t <= kFlatTokens; ++t) {
    const long items = (long)t * per_tok;
    if (items > (long)kThreads * kFlatItems) break;
    const long idle = (items + kThreads - 1) / kThreads * kThreads - items;
    if (tpw == 0 || idle * tpw < best_idle * t) { best_idle = idle; tpw = t; }  // idle / t < best_idle / tpw
  }
  if (tpw > 0) {
    dim3 grid((a.S + tpw - 1) / tpw, a.B);
    hipLaunchKernelGGL((qknorm_rope_flat_kernel<T>), grid, dim3(kThreads), 0, stream, a, tpw);
    return hipGetLastError();
  }
  // One head per lane group, looping over the heads.
  int lph = 1;
  while (lph < chunks) lph <<= 1;
  dim3 grid(a.S, a.B);
  switch (lph) {
    case 1: hipLaunchKernelGGL((qknorm_rope_kernel<T, 1>), grid, dim3(kThreads), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((qknorm_rope_kernel<T, 2>), grid, dim3(kThreads), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((qknorm_rope_kernel<T, 4>), grid, dim3(kThreads), 0, stream, a); break;
    case 8: hipLaunchKernelGGL((qknorm_rope_kernel<T, 8>), grid, dim3(kThreads), 0, stream, a); break;
    case 16: hipLaunchKernelGGL((qknorm_rope_kernel<T, 16>), grid, dim3(kThreads), 0, stream, a); break;
    case 32: hipLaunchKernelGGL((qknorm_rope_kernel<T, 32>), grid, dim3(kThreads), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qknorm_rope(const QkNormRopeArgs& a, int dtype, hipStream_t stream) {
  return dtype == 0 ? launch_typed<__bf16>(a, stream) : launch_typed<float>(a, stream);
}

}  // namespace dit
