// Classifier-free guidance with norm rescaling (gfx950).
//
// NucleusMoE-Image pipeline article, section 4.3: the conditional and the
// unconditional predictions are mixed as uncond + s * (cond - uncond), and
// each token's mix is rescaled to the norm of its conditional prediction
// (norms over the token's channels).  A token whose mix is exactly zero has
// no direction; it is written as zero.
//
// HBM-bound: two reads and one write per element, nothing reused.  A row
// (token) of C channels is spread over LPR lanes of one wave, each holding NCH
// 16-byte chunks (chunk sub + LPR * i), so loads and stores are full 16-byte
// vectors and the two squared norms are butterflies over LPR lanes; a wave
// handles 64 / LPR rows.  (Four rows per lane group, all loads issued first,
// measured slower than one: at 131072 x 64 the 4x larger grid of the one-row
// form hides the memory latency better.)  Arithmetic in fp32, one rounding on
// the store.

#include "device_common.h"
#include "kernels.h"

namespace dit {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void unpack8(const u32x4& w, float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_lo(w[i]);
    x[2 * i + 1] = bf16_hi(w[i]);
  }
}

template <typename T>
struct Chunk;
template <>
struct Chunk<__bf16> {
  static constexpr int N = 8;
  __device__ static void load(const void* p, float* x) { unpack8(*reinterpret_cast<const u32x4*>(p), x); }
  __device__ static void store(void* p, const float* y) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(y[2 * i], y[2 * i + 1]);
    *reinterpret_cast<u32x4*>(p) = w;
  }
};
template <>
struct Chunk<float> {
  static constexpr int N = 4;
  __device__ static void load(const void* p, float* x) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = v[i];
  }
  __device__ static void store(void* p, const float* y) {
    *reinterpret_cast<f32x4*>(p) = f32x4{y[0], y[1], y[2], y[3]};
  }
};

template <typename T, int LPR, int NCH>
__global__ __launch_bounds__(kThreads) void cfg_norm_rescale_kernel(CfgArgs a) {
  constexpr int EPC = Chunk<T>::N;
  constexpr int RPB = kThreads / LPR;  // rows per work-group
  const int tid = threadIdx.x;
  const int sub = tid % LPR;
  const int cpr = a.C / EPC;  // chunks per row
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / LPR;
  const bool row_ok = row < a.rows;
  const T* cp = reinterpret_cast<const T*>(a.cond) + (row_ok ? row : 0) * a.cs;
  const T* up = reinterpret_cast<const T*>(a.uncond) + (row_ok ? row : 0) * a.us;

  float c[NCH][EPC], m[NCH][EPC];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int ch = sub + LPR * i;
    if (row_ok && ch < cpr) {
      Chunk<T>::load(cp + ch * EPC, c[i]);
      Chunk<T>::load(up + ch * EPC, m[i]);
    } else {
#pragma unroll
      for (int e = 0; e < EPC; ++e) c[i][e] = m[i][e] = 0.f;
    }
  }
  float cn = 0.f, mn = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i)
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      const float mix = fmaf(a.g, c[i][e] - m[i][e], m[i][e]);  // uncond + s (cond - uncond)
      m[i][e] = mix;
      cn = fmaf(c[i][e], c[i][e], cn);
      mn = fmaf(mix, mix, mn);
    }
#pragma unroll
  for (int k = LPR / 2; k >= 1; k >>= 1) {
    cn += __shfl_xor(cn, k, 64);
    mn += __shfl_xor(mn, k, 64);
  }
  const float scale = mn > 0.f ? sqrtf(cn) / sqrtf(mn) : 0.f;
  if (!row_ok) return;
  T* op = reinterpret_cast<T*>(a.out) + row * a.os;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int ch = sub + LPR * i;
    if (ch < cpr) {
      float y[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) y[e] = m[i][e] * scale;
      Chunk<T>::store(op + ch * EPC, y);
    }
  }
}

template <typename T, int LPR>
hipError_t launch_lpr(const CfgArgs& a, int nch, hipStream_t stream) {
  const dim3 grid((unsigned)((a.rows + kThreads / LPR - 1) / (kThreads / LPR)));
  switch (nch) {
    case 1: hipLaunchKernelGGL((cfg_norm_rescale_kernel<T, LPR, 1>), grid, dim3(kThreads), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((cfg_norm_rescale_kernel<T, LPR, 2>), grid, dim3(kThreads), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((cfg_norm_rescale_kernel<T, LPR, 4>), grid, dim3(kThreads), 0, stream, a); break;
    case 8: hipLaunchKernelGGL((cfg_norm_rescale_kernel<T, LPR, 8>), grid, dim3(kThreads), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_typed(const CfgArgs& a, hipStream_t stream) {
  const int cpr = a.C / Chunk<T>::N;
  // Lanes per row: the chunk count rounded up to a power of two, at most a wave;
  // wider rows give each lane 2, 4 or 8 chunks.
  int lpr = 1;
  while (lpr < cpr && lpr < 64) lpr <<= 1;
  int nch = 1;
  while (nch * lpr < cpr) nch <<= 1;
  switch (lpr) {
    case 1: return launch_lpr<T, 1>(a, nch, stream);
    case 2: return launch_lpr<T, 2>(a, nch, stream);
    case 4: return launch_lpr<T, 4>(a, nch, stream);
    case 8: return launch_lpr<T, 8>(a, nch, stream);
    case 16: return launch_lpr<T, 16>(a, nch, stream);
    case 32: return launch_lpr<T, 32>(a, nch, stream);
    case 64: return launch_lpr<T, 64>(a, nch, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_cfg_norm_rescale(const CfgArgs& a, int dtype, hipStream_t stream) {
  return dtype == 0 ? launch_typed<__bf16>(a, stream) : launch_typed<float>(a, stream);
}

}  // namespace dit
