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
// One work-group of 1024 threads.  Per pass each wave owns a contiguous
// segment of 64 * TPT tokens: it counts its image tokens, a block-wide scan
// over the 16 wave counts gives each segment its starting rank, and the wave
// then walks its segment 64 tokens at a time with lane = token, ranking image
// tokens with a ballot and mbcnt, so every load and store is coalesced.  A
// block's first and last tokens are the unique tokens holding its first and
// last ranks, so they are recorded without atomics; an image token's key bound
// is its position minus its rank in the block plus the block size, exact
// whenever the block is contiguous, which the first/last check verifies.
// Data errors (count mismatch, split block, text under 2D positions) go to a
// device status word.

#include "device_common.h"
#include "kernels.h"

namespace dit {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int TPT = 8;                  // 64-token groups per wave and pass
constexpr int kSeg = 64 * TPT;          // tokens per wave and pass
constexpr int kPass = kWaves * kSeg;    // tokens per pass

// Number of set bits of `bits` in the lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t bits) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(bits >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bits, 0));
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
  __shared__ int s_shape[kMaxImages][4];  // height, width, height * width, frame offset
  __shared__ int s_wave_cnt[kWaves];
  __shared__ int s_carry;
  __shared__ int s_bad;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n_img = a.n_img;
  const int S = a.seq_len;

  if (tid < kMaxImages) {
    s_first[tid] = -1;
    s_last[tid] = -1;
  }
  if (tid <= n_img) s_cum[tid] = a.cum[tid];
  if (tid < n_img) {  // per-block constants, read from LDS in the token loop
    s_shape[tid][0] = a.shape[tid][1];
    s_shape[tid][1] = a.shape[tid][2];
    s_shape[tid][2] = a.shape[tid][1] * a.shape[tid][2];
    s_shape[tid][3] = a.frame_off[tid];
  }
  if (tid == 0) {
    s_carry = 0;
    s_bad = 0;
  }
  __syncthreads();
  const int total_expected = s_cum[n_img];
  int bad = 0;

  for (int base = 0; base < S; base += kPass) {
    const int seg = base + wave * kSeg;
    // Image tokens of this wave's segment.
    int cnt = 0;
#pragma unroll
    for (int it = 0; it < TPT; ++it) {
      const int s = seg + it * 64 + lane;
      cnt += (s < S && mask[s] != 0) ? 1 : 0;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
    if (lane == 0) s_wave_cnt[wave] = cnt;
    __syncthreads();
    int r0 = s_carry;  // rank of the first image token of this segment
    for (int w = 0; w < wave; ++w) r0 += s_wave_cnt[w];
    int blk = 0;
    {
      int lo = 0, hi = n_img > 0 ? n_img - 1 : 0;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_cum[mid] <= r0) lo = mid; else hi = mid - 1;
      }
      blk = lo;
    }
    bool m[TPT];
#pragma unroll
    for (int it = 0; it < TPT; ++it) {
      const int s = seg + it * 64 + lane;
      m[it] = s < S && mask[s] != 0;
    }
#pragma unroll
    for (int it = 0; it < TPT; ++it) {
      const int s = seg + it * 64 + lane;
      const uint64_t bits = __ballot(m[it]);
      const int r = r0 + lanes_below(bits);  // image tokens before s
      if (s < S) {
        int id = -1, p0 = 0, p1 = 0, p2 = 0, lim = s + 1;
        if (m[it]) {
          if (r >= total_expected) {
            bad = 1;
          } else {
            int b = blk;
            while (s_cum[b + 1] <= r) ++b;
            id = b;
            const int count = s_cum[b + 1] - s_cum[b];
            const int local = r - s_cum[b];
            if (local == 0) s_first[b] = s;
            if (local == count - 1) s_last[b] = s;
            // One past the block's last token, if the block is contiguous
            // (checked below through its first and last tokens).
            lim = s - local + count;
            const int Hh = s_shape[b][0], W = s_shape[b][1];
            const int f = local / s_shape[b][2];
            const int h = (local / W) % Hh;
            const int w = local % W;
            if (a.pos_mode == 0) {
              p0 = s_shape[b][3] + f;
              p1 = h - Hh / 2;
              p2 = w - W / 2;
            } else {
              p0 = h;
              p1 = w;
            }
          }
        } else if (a.pos_mode == 0) {
          p0 = p1 = p2 = a.max_vid + (s - r);  // s - r = text tokens before s
        } else {
          bad = 1;
        }
        image_ids[s] = id;
        pos[3 * s + 0] = p0;
        pos[3 * s + 1] = p1;
        pos[3 * s + 2] = p2;
        kv_limit[s] = lim;
        target[s] = (id >= 0 && id == n_img - 1) ? 1 : 0;
      }
      r0 += __builtin_popcountll(bits);
      while (n_img > 0 && blk < n_img - 1 && s_cum[blk + 1] <= r0) ++blk;
    }
    __syncthreads();
    if (tid == kThreads - 1) s_carry = r0;
    __syncthreads();
  }
  if (bad) s_bad = 1;
  __syncthreads();
  if (tid == 0 && s_carry != total_expected) s_bad = 1;
  if (tid < n_img) {
    const int first = s_first[tid], last = s_last[tid];
    if (first < 0 || last < 0 || last - first + 1 != s_cum[tid + 1] - s_cum[tid]) s_bad = 1;
  }
  __syncthreads();
  if (tid == 0) status[0] = s_bad ? 5 : 0;
}

// Key validity of the joint sequence for one sample per work-group
// (QwenImage21Transformer2DModel API page, forward's encoder_hidden_states_mask:
// padded text tokens take no part in attention).  Text token s is the
// (s - r)-th text token, r being the image tokens before it, and takes that
// entry of the sample's text mask; image tokens are always valid.  Same
// segment scan as the metadata kernel; each 64-token group becomes one ballot
// word, stored by its first lane.  Bits past the sequence end are 0.
__global__ __launch_bounds__(kThreads) void key_valid_kernel(KeyValidArgs a) {
  __shared__ int s_wave_cnt[kWaves];
  __shared__ int s_carry;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int S = a.S;
  const uint8_t* __restrict__ mask = a.mask;
  const uint8_t* __restrict__ tv = a.text_valid + (int64_t)blockIdx.x * a.tv_stride;
  uint64_t* __restrict__ out = a.bits + (int64_t)blockIdx.x * a.bits_stride;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int base = 0; base < S; base += kPass) {
    const int seg = base + wave * kSeg;
    bool m[TPT];
    int cnt = 0;
#pragma unroll
    for (int it = 0; it < TPT; ++it) {
      const int s = seg + it * 64 + lane;
      m[it] = s < S && mask[s] != 0;
      cnt += m[it] ? 1 : 0;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
    if (lane == 0) s_wave_cnt[wave] = cnt;
    __syncthreads();
    int r0 = s_carry;  // image tokens before this segment
    for (int w = 0; w < wave; ++w) r0 += s_wave_cnt[w];
#pragma unroll
    for (int it = 0; it < TPT; ++it) {
      const int s = seg + it * 64 + lane;
      const uint64_t img = __ballot(m[it]);
      const int j = s - (r0 + lanes_below(img));  // text ordinal of a text token
      bool valid = m[it];
      if (s < S && !m[it] && j < a.n_text) valid = tv[j] != 0;
      const uint64_t word = __ballot(valid);
      if (lane == 0 && seg + it * 64 < S) out[(seg + it * 64) >> 6] = word;
      r0 += __builtin_popcountll(img);
    }
    __syncthreads();
    if (tid == kThreads - 1) s_carry = r0;
    __syncthreads();
  }
  // Every work-group sees the same layout; the first reports it.
  if (blockIdx.x == 0 && tid == 0) a.status[0] = (S - s_carry == a.n_text) ? 0 : 5;
}

}  // namespace

hipError_t launch_key_valid(const KeyValidArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(key_valid_kernel, dim3((unsigned)a.B), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_token_meta(const uint8_t* mask, const TokenMetaArgs& a, int32_t* image_ids, uint8_t* target,
                             int32_t* pos, int32_t* kv_limit, int32_t* status, hipStream_t stream) {
  hipLaunchKernelGGL(token_meta_kernel, dim3(1), dim3(kThreads), 0, stream, mask, a, image_ids, target, pos,
                     kv_limit, status);
  return hipGetLastError();
}

}  // namespace dit
