// Token metadata of the joint text+image sequence (gfx950).
//
// QwenImage21Transformer2DModel API page, build_token_metadata: every token of
// the joint sequence gets an image-block id (text = -1) and a flag for the
// target (last) image; block boundaries follow the token counts of img_shapes,
// not runs of image tokens, so adjacent condition images stay two blocks.
// From the ids this kernel also derives, for the later steps:
//   kv_limit[s]  exclusive bound of the keys token s may see under the
//                block-causal rule of the same page (s + 1 for text, one past
//                the block's last token for image tokens);
//   pos_ids[s]   rotary positions, centred (frame, height, width) or the
//                Lumina 2D grid (NucleusMoE-Image article section 6.3;
//                Lumina-Next DiT article sections 1 and 4).
//
// One work-group of 1024 threads walks the sequence in chunks, ranking image
// tokens with a block-wide prefix sum; the work is a few integer operations
// per token, so the launch itself dominates.  Data errors (count mismatch,
// split block, text under 2D positions) go to a device status word.

#include "device_common.h"
#include "kernels.h"

namespace dit {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ int wave_inclusive_scan(int x) {
  const int lane = __lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

__global__ __launch_bounds__(kThreads) void token_meta_kernel(const uint8_t* __restrict__ mask,
                                                              TokenMetaArgs a, int32_t* __restrict__ image_ids,
                                                              uint8_t* __restrict__ target,
                                                              int32_t* __restrict__ pos,
                                                              int32_t* __restrict__ kv_limit,
                                                              int32_t* __restrict__ status) {
  __shared__ int s_first[kMaxImages];
  __shared__ int s_last[kMaxImages];
  __shared__ int s_cum[kMaxImages + 1];
  __shared__ int s_wave_tot[kWaves];
  __shared__ int s_carry;
  __shared__ int s_bad;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n_img = a.n_img;
  const int S = a.seq_len;

  if (tid < kMaxImages) {
    s_first[tid] = 0x7fffffff;
    s_last[tid] = -1;
  }
  if (tid <= n_img) s_cum[tid] = a.cum[tid];
  if (tid == 0) {
    s_carry = 0;
    s_bad = 0;
  }
  __syncthreads();
  const int total_expected = s_cum[n_img];

  for (int base = 0; base < S; base += kThreads) {
    const int s = base + tid;
    const int m = (s < S && mask[s] != 0) ? 1 : 0;
    int incl = wave_inclusive_scan(m);
    if (lane == 63) s_wave_tot[wave] = incl;
    __syncthreads();
    int wave_off = 0;
    for (int w = 0; w < wave; ++w) wave_off += s_wave_tot[w];
    const int carry = s_carry;
    incl += wave_off + carry;  // image tokens in [0, s]
    if (s < S) {
      int id = -1;
      int p0 = 0, p1 = 0, p2 = 0;
      if (m) {
        const int r = incl - 1;  // rank of this image token
        if (r >= total_expected) {
          s_bad = 1;
        } else {
          // block b with cum[b] <= r < cum[b + 1]
          int lo = 0, hi = n_img - 1;
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_cum[mid] <= r) lo = mid; else hi = mid - 1;
          }
          id = lo;
          const int local = r - s_cum[id];
          atomicMin(&s_first[id], s);
          atomicMax(&s_last[id], s);
          const int F = a.shape[id][0], Hh = a.shape[id][1], W = a.shape[id][2];
          (void)F;
          const int f = local / (Hh * W);
          const int h = (local / W) % Hh;
          const int w = local % W;
          if (a.pos_mode == 0) {
            p0 = a.frame_off[id] + f;
            p1 = h - Hh / 2;
            p2 = w - W / 2;
          } else {
            p0 = h;
            p1 = w;
            p2 = 0;
          }
        }
      } else {
        if (a.pos_mode == 0) {
          const int t = s - incl;  // text tokens before s (s itself is text)
          p0 = p1 = p2 = a.max_vid + t;
        } else {
          s_bad = 1;
        }
      }
      image_ids[s] = id;
      pos[3 * s + 0] = p0;
      pos[3 * s + 1] = p1;
      pos[3 * s + 2] = p2;
    }
    __syncthreads();
    if (tid == kThreads - 1) s_carry = incl;
    __syncthreads();
  }

  if (tid == 0 && s_carry != total_expected) s_bad = 1;
  if (tid < n_img) {
    const long long span = (long long)s_last[tid] - (long long)s_first[tid] + 1;
    if (span != (long long)(s_cum[tid + 1] - s_cum[tid])) s_bad = 1;
  }
  __syncthreads();

  for (int s = tid; s < S; s += kThreads) {
    const int id = image_ids[s];  // written by this same thread above
    kv_limit[s] = (id < 0) ? s + 1 : s_last[id] + 1;
    target[s] = (id >= 0 && id == n_img - 1) ? 1 : 0;
  }
  if (tid == 0) status[0] = s_bad ? 5 : 0;
}

}  // namespace

hipError_t launch_token_meta(const uint8_t* mask, const TokenMetaArgs& a, int32_t* image_ids, uint8_t* target,
                             int32_t* pos, int32_t* kv_limit, int32_t* status, hipStream_t stream) {
  hipLaunchKernelGGL(token_meta_kernel, dim3(1), dim3(kThreads), 0, stream, mask, a, image_ids, target, pos,
                     kv_limit, status);
  return hipGetLastError();
}

}  // namespace dit
