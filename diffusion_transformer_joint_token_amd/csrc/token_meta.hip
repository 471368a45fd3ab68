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
// One 1024-thread work-group per 1024-token chunk, plus one that checks the
// layout.  A chunk work-group counts the image tokens before its chunk (a
// reduction over the mask, 16-byte loads), then ranks its own image tokens
// with a ballot and mbcnt per wave and a scan over the 16 wave counts, so every
// load and store is coalesced.  An image token's rank places it in its block;
// its key bound is its position minus its rank in the block plus the block
// size, exact whenever the block is contiguous.  The checker scans the whole
// mask (segments of 64 * TPT tokens per wave) and writes the device status
// word: count mismatch, text under 2D positions, or a run of image tokens that
// does not start at a block's first rank (a split block).  Earlier versions
// ran everything in one work-group on one CU, instruction-bound at ~2200
// instructions per wave.
//
// The key-validity kernel further down keeps the single-work-group scan (one
// work-group per sample).

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

// Image tokens among mask[0, n), counted by the whole work-group (every
// thread gets the total).  16-byte loads when the mask is 16-byte aligned: a
// byte is zero iff its high bit survives ~((w & 0x7f..) + 0x7f.. | w | 0x7f..).
__device__ int count_image_tokens(const uint8_t* __restrict__ mask, int n, int* s_part) {
  const int tid = threadIdx.x;
  int cnt = 0;
  int done = 0;
  if ((reinterpret_cast<uintptr_t>(mask) & 15) == 0) {
    const int n16 = n >> 4;
    for (int i = tid; i < n16; i += kThreads) {
      const u32x4 w = reinterpret_cast<const u32x4*>(mask)[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t x = w[j];
        const uint32_t zero = ~(((x & 0x7f7f7f7fu) + 0x7f7f7f7fu) | x | 0x7f7f7f7fu);
        cnt += 4 - __builtin_popcount(zero);
      }
    }
    done = n16 << 4;
  }
  for (int i = done + tid; i < n; i += kThreads) cnt += mask[i] != 0 ? 1 : 0;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
  __syncthreads();  // s_part may still be read by an earlier call
  if ((tid & 63) == 0) s_part[tid >> 6] = cnt;
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) total += s_part[w];
  return total;
}

// Work-group c < n_chunks writes the outputs of tokens [c * kThreads,
// (c + 1) * kThreads): it counts the image tokens before its chunk, ranks its
// own with one ballot scan (a token's rank among image tokens places it in its
// block, the block's first token and size give its key bound, the rank within
// the block its positions).  The last work-group checks the layout of the
// whole sequence and alone writes the status word: the image-token count must
// match img_shapes, a 2D grid admits no text, and every run of consecutive
// image tokens must start at a block's first rank (so no block is split; two
// adjacent blocks may share a run).
__global__ __launch_bounds__(kThreads) void token_meta_kernel(const uint8_t* __restrict__ mask,
                                                              TokenMetaArgs a, int32_t* __restrict__ image_ids,
                                                              uint8_t* __restrict__ target,
                                                              int32_t* __restrict__ pos,
                                                              int32_t* __restrict__ kv_limit,
                                                              int32_t* __restrict__ status) {
  __shared__ int s_cum[kMaxImages + 1];
  __shared__ int s_shape[kMaxImages][4];  // height, width, height * width, frame offset
  __shared__ int s_part[kWaves];
  __shared__ int s_wave_cnt[kWaves];
  __shared__ int s_carry;
  __shared__ int s_bad;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n_img = a.n_img;
  const int S = a.seq_len;
  const int n_chunks = (S + kThreads - 1) / kThreads;

  if (tid <= n_img) s_cum[tid] = a.cum[tid];
  if (tid < n_img) {
    s_shape[tid][0] = a.shape[tid][1];
    s_shape[tid][1] = a.shape[tid][2];
    s_shape[tid][2] = a.shape[tid][1] * a.shape[tid][2];
    s_shape[tid][3] = a.frame_off[tid];
  }
  if (tid == 0) {
    s_carry = 0;
    s_bad = 0;
  }
  // (the first barrier inside count_image_tokens publishes these)

  if ((int)blockIdx.x == n_chunks) {
    // ---- layout check over the whole sequence
    const int total = count_image_tokens(mask, S, s_part);
    const int total_expected = s_cum[n_img];
    int bad = (total != total_expected || (a.pos_mode != 0 && total != S)) ? 1 : 0;
    for (int base = 0; base < S && !bad; base += kPass) {
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
      int r0 = s_carry;
      for (int w = 0; w < wave; ++w) r0 += s_wave_cnt[w];
#pragma unroll
      for (int it = 0; it < TPT; ++it) {
        const int s = seg + it * 64 + lane;
        const uint64_t bits = __ballot(m[it]);
        if (m[it]) {
          const bool prev = s > 0 && mask[s - 1] != 0;
          if (!prev) {  // a run starts here: its rank must open a block
            const int r = r0 + lanes_below(bits);
            int lo = 0, hi = n_img;  // first b with s_cum[b] >= r
            while (lo < hi) {
              const int mid = (lo + hi) >> 1;
              if (s_cum[mid] < r) lo = mid + 1; else hi = mid;
            }
            if (lo >= n_img || s_cum[lo] != r) bad = 1;
          }
        }
        r0 += __builtin_popcountll(bits);
      }
      __syncthreads();
      if (tid == kThreads - 1) s_carry = r0;
      if (bad) s_bad = 1;
      __syncthreads();
      bad = s_bad;
    }
    if (bad) s_bad = 1;
    __syncthreads();
    if (tid == 0) status[0] = s_bad ? 5 : 0;
    return;
  }

  // ---- outputs of this work-group's chunk
  const int s0 = (int)blockIdx.x * kThreads;
  const int r_base = count_image_tokens(mask, s0, s_part);  // image tokens before the chunk
  const int s = s0 + tid;
  const bool m = s < S && mask[s] != 0;
  const uint64_t bits = __ballot(m);
  if (lane == 0) s_wave_cnt[wave] = __builtin_popcountll(bits);
  __syncthreads();
  int r = r_base + lanes_below(bits);  // image tokens before s
  for (int w = 0; w < wave; ++w) r += s_wave_cnt[w];
  if (s >= S) return;
  int id = -1, p0 = 0, p1 = 0, p2 = 0, lim = s + 1;
  if (m) {
    if (n_img > 0) {
      int lo = 0, hi = n_img - 1;  // last block with s_cum[b] <= r (clamped: a count error is the checker's)
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_cum[mid] <= r) lo = mid; else hi = mid - 1;
      }
      const int bk = lo;
      id = bk;
      const int count = s_cum[bk + 1] - s_cum[bk];
      const int local = r - s_cum[bk];
      // One past the block's last token (exact when the block is contiguous,
      // which the checker verifies).
      lim = s - local + count;
      const int Hh = s_shape[bk][0], W = s_shape[bk][1];
      const int hw = s_shape[bk][2];
      const int f = local / hw;
      const int rem = local - f * hw;
      const int h = rem / W;
      const int w = rem - h * W;
      if (a.pos_mode == 0) {
        p0 = s_shape[bk][3] + f;
        p1 = h - Hh / 2;
        p2 = w - W / 2;
      } else {
        p0 = h;
        p1 = w;
      }
    }
  } else if (a.pos_mode == 0) {
    p0 = p1 = p2 = a.max_vid + (s - r);  // s - r = text tokens before s
  }
  image_ids[s] = id;
  pos[3 * s + 0] = p0;
  pos[3 * s + 1] = p1;
  pos[3 * s + 2] = p2;
  kv_limit[s] = lim;
  target[s] = (id >= 0 && id == n_img - 1) ? 1 : 0;
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
  const int n_chunks = (a.seq_len + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(token_meta_kernel, dim3(n_chunks + 1), dim3(kThreads), 0, stream, mask, a, image_ids, target,
                     pos, kv_limit, status);
  return hipGetLastError();
}

}  // namespace dit
