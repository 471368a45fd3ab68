// Masked softmax attention over the joint text+image sequence (gfx950).
//
// QwenImage21Transformer2DModel API page: a query attends a key when
// q_idx >= kv_idx or both lie in the same image block (block-causal), or every
// key (full).  For contiguous blocks the allowed keys of query q are exactly
// the prefix [0, kv_limit[q]) with kv_limit non-decreasing along the
// sequence, so a tile of queries x keys is either fully allowed, fully masked
// or needs a per-element test only near its diagonal; masked tiles are never
// loaded or computed.  The same page's cached mode ("kv_cache" of the
// timestep-independent prefix) is the same loop with keys [0, P) read from the
// cache and keys [P, P + S_new) from the new tokens.  GQA: query head h reads
// KV head h / (H / H_kv) (NucleusMoE-Image article, section 6.3).
//
// bf16 kernel layout (one work-group = NW waves = 32*NW query rows of one
// (batch, head); key tiles of 64):
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: A = K rows from LDS, B = Q^T kept
//    in registers for the whole kernel.  The accumulator then gives every lane
//    one query column and 16 keys, so the online-softmax max/sum are in-lane
//    reductions plus one exchange with the lane 32 apart (v_permlane32_swap).
//  * O^T += V^T P^T on the same MFMA: B = P^T straight from the S^T accumulator
//    (rounded to bf16), A = V^T read from the row-major V tile with
//    ds_read_b64_tr_b16, whose 16-lane transpose delivers 4 consecutive keys of
//    one head channel per lane in exactly the key order of the accumulator.
//  * K and V tiles move global -> LDS with direct 16-byte LDS loads (no VGPR
//    staging) into two K and two V stages; each stage is refilled right after
//    the barrier that ends its last read, so a tile has 1.5 iterations to land
//    (two barriers per iteration, waits counted in vector-memory instructions).
//    16-byte chunks are XOR-swizzled per row so both the K reads (16 rows, same
//    chunk) and the transposed V reads (4 rows x 4 chunks) hit distinct banks.
//  * Softmax in the exp2 domain; the running max is only moved when a row's
//    new maximum exceeds it by more than 8 (log2 units), so O is rarely
//    rescaled and probabilities stay <= 2^8.  Every S tile's accumulator
//    starts from one register tile holding -offset, rebuilt only when the
//    offset moves (the first QK^T MFMA reads it as its C operand).
//  * All query tiles of one (batch, head) run on one XCD (and its L2); the
//    light low query tiles of each XCD go out last.
//  * Padded text keys (same page, forward's encoder_hidden_states_mask): one
//    validity word per key tile and sample, read through the scalar cache; a
//    tile whose word is not all ones takes the per-element mask path.  A row
//    keeps no offset until its first finite logit, and a row with no valid key
//    at all ends with O = 0 and lse = -inf.

#include <cmath>

#include "device_common.h"
#include "kernels.h"

namespace dit {

namespace {

constexpr int kTileN = 64;        // keys per tile
constexpr int kRowBytes = 256;    // LDS bytes per key row (16 chunks of 16 B)
constexpr int kTileBytes = kTileN * kRowBytes;
constexpr float kLazyRescale = 8.0f;  // log2 units
constexpr int PF_K = 3;  // K operands read this many MFMAs ahead
// V^T operands read this many MFMAs ahead: 2, or 3 in the 80-channel variant
// (12 PV MFMAs per tile; one more read in flight measured 0.6 % faster there,
// while at 128 channels 3 is no better and the cached-prefix workload slows).
constexpr int pf_v(int dp) { return dp == 80 ? 3 : 2; }

__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// Work-group index -> (batch*head, query tile).  Work-groups are dealt to the
// 8 XCDs round-robin; each XCD gets whole (batch, head) units, so the query
// tiles of one unit share that XCD's L2.  Under the block-causal mask a query
// tile's work (its rows' key bounds) never decreases along the sequence, so
// the lowest fifth of the query tiles (the causal text rows of a joint
// sequence) are the light ones: each XCD first runs its units one after
// another, last query tile first, over the upper tiles, then the low tiles
// the same way, so light tiles fill the tail instead of delaying heavy ones
// and each unit's keys are re-read at most once.  Under the full mask every
// tile does the same work and the order is unit by unit.
// Units are dealt head-major, (head, sample), so each XCD holds the same
// heads of every sample: samples whose padded text leaves them fewer keys
// then do not all land on the same XCDs, which would finish early while the
// others set the launch time.  Query heads that share a KV head stay on one
// XCD.
__device__ __forceinline__ void map_block(int id, int nblocks, int n_qtiles, bool causal, int B, int H, int& bh,
                                          int& qtile) {
  const int per = nblocks >> 3;
  int unit;
  if (id < per * 8 && per % n_qtiles == 0) {
    const int x = id & 7, j = id >> 3;  // XCD, position in its queue
    const int units = per / n_qtiles;
    const int low = causal ? n_qtiles / 5 : 0;
    const int hi = n_qtiles - low;
    if (j < units * hi) {
      unit = x * units + j / hi;
      qtile = n_qtiles - 1 - j % hi;
    } else {
      const int k = j - units * hi;
      unit = x * units + k / low;
      qtile = low - 1 - k % low;
    }
  } else {
    int logical = id;
    if (id < per * 8) logical = (id & 7) * per + (id >> 3);
    unit = logical / n_qtiles;
    qtile = n_qtiles - 1 - (logical - unit * n_qtiles);
  }
  bh = (unit % B) * H + unit / B;  // unit = head * B + sample
}

// Buffer resource word 3 for untyped 32-bit accesses on gfx9-class parts.
constexpr int kRsrcWord3 = 0x00020000;

// s_waitcnt immediate (gfx9 layout): vmcnt in bits [3:0] and [15:14], expcnt
// in [6:4] (7: no wait), lgkmcnt in [11:8].  Issued through the builtin so the
// compiler's own wait insertion knows what has already been waited for.
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8); }

// acc + lo + hi of a packed bf16 pair, in one v_dot2 against (1, 1).
__device__ __forceinline__ float add_bf16_pair(uint32_t pair, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
}

// Value selects: a conditional between two captured variables would select
// their addresses, which keeps a lambda's captures in private memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t pick(bool c, __amdgpu_buffer_rsrc_t x, __amdgpu_buffer_rsrc_t y) {
  return c ? x : y;
}
__device__ __forceinline__ int pick(bool c, int x, int y) { return c ? x : y; }
__device__ __forceinline__ uint32_t pick(bool c, uint32_t x, uint32_t y) { return c ? x : y; }

// 16 bytes per lane from a buffer resource straight into LDS (lane i lands at
// dst + 16 i); an offset past the resource's extent reads as zeros.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, char* dst, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)dst, 16, voffset, 0, 0, 0);
}

// UNIT: Q already carries softmax_scale * log2(e) (scale argument ln 2), so the
// MFMA output is the exponent itself.
// ALIGNED: the cache length P is a multiple of the key tile, so no tile mixes
// cached and new keys and every tile load comes from one source.
// PADDED: a.key_bits marks the valid keys of each sample.
// QNORM: a.q holds raw Q; the prologue applies the per-head RMSNorm, the
// weight, the rotary embedding (phases from a.qpos and a.omega) and a.q_scale,
// and rounds once, as the norm kernel would have, so Q' never goes through
// memory.
template <int DP, int NW, bool UNIT, bool ALIGNED, bool PADDED, bool QNORM>
__global__ __launch_bounds__(NW * 64, 2) void attn_fwd_bf16_kernel(AttnArgs a) {
  // DP: head dim padded to a multiple of 16 for QK^T (80 for head dim 72: five
  // contraction steps, not six); O^T runs in 32-channel blocks, so its last
  // block may reach past DP, where the tiles hold zeros.
  static_assert(DP % 16 == 0 && DP >= 32 && DP <= 128, "padded head dim");
  constexpr int PF_V = pf_v(DP);
  constexpr int KSTEPS = DP / 16;         // QK^T contraction steps
  constexpr int MBLK = (DP + 31) / 32;    // 32-channel blocks of O^T
  constexpr int CHUNKS = DP / 8;          // 16-byte chunks per key row actually used
  // When the O^T blocks reach past DP, V's logical chunk CHUNKS is set to
  // (1, 0, ..., 0) in every V tile once it has landed (ones_col below), so
  // O^T channel 8 * CHUNKS accumulates sum_k P[q, k]: the row sum comes out of
  // the PV MFMAs, rescaled with O, instead of one dot product per pair of
  // probabilities.
  constexpr bool ONES_COL = 32 * MBLK > DP;
  constexpr int LOADS = (kTileN * 16) / (NW * 64);  // LDS-load instructions per wave per tile

  // Two K stages and two V stages, each a distinct LDS object, so the compiler
  // can tell the stage being filled from the stage being read.  K runs one
  // tile ahead of V: iteration t reads K(t+1) (for S(t+1)) and V(t) (for PV(t)).
  __shared__ __attribute__((aligned(1024))) char sK0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sK1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sV0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sV1[kTileBytes];
  __shared__ int s_lim[NW];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 5;  // k-group of the MFMA operands
  const int n_qtiles = (a.Snew + 32 * NW - 1) / (32 * NW);
  int bh, qtile;
  map_block(blockIdx.x, gridDim.x, n_qtiles, a.kv_limit != nullptr, a.B, a.H, bh, qtile);
  const int h = bh % a.H;
  const int b = bh / a.H;
  const int kvh = h / (a.H / a.Hk);
  const int Sk = a.Sk;
  const int P = a.P;

  // Validity word of key tile t for this sample (all ones without padding).
  // The constant address space lets the uniform load go through the scalar
  // cache, outside the vector-memory counts the tile waits rely on; volatile
  // keeps it where it is written (before a tile barrier, whose wait then
  // covers its latency) instead of next to its use.
  // The index goes in as a 32-bit byte offset, which the scalar load takes
  // in a register as it is (no 64-bit address arithmetic per tile).
  using const_u64 = const volatile __attribute__((address_space(4))) uint64_t;
  using const_u8 = const __attribute__((address_space(4))) char;
  const_u8* kbits = nullptr;
  if constexpr (PADDED) kbits = (const_u8*)(a.key_bits + (int64_t)b * a.kb_stride);
  auto tile_word = [&](int t) __attribute__((always_inline)) -> uint64_t {
    if constexpr (PADDED) return *(const_u64*)(kbits + ((uint32_t)t << 3));
    return ~0ull;
  };
  // The first three tiles' words, read together while Q loads.
  const int last_tile = (Sk - 1) / kTileN;
  const uint64_t pw0 = tile_word(0), pw1 = tile_word(min(1, last_tile)), pw2 = tile_word(min(2, last_tile));

  // This lane's query row and its key bound.
  const int qrow = qtile * 32 * NW + wave * 32 + (lane & 31);
  const bool row_ok = qrow < a.Snew;
  const int qclamp = row_ok ? qrow : a.Snew - 1;
  const int lim = a.kv_limit ? a.kv_limit[P + qclamp] : Sk;
  int wlim_max = lim, wlim_min = lim;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    wlim_max = max(wlim_max, __shfl_xor(wlim_max, m, 64));
    wlim_min = min(wlim_min, __shfl_xor(wlim_min, m, 64));
  }
  if (lane == 0) s_lim[wave] = wlim_max;

  // Q^T operand: lane holds query (lane & 31), channels 16*ks + 8*g .. +7.
  bf16x8 qreg[KSTEPS];
  constexpr int QN = QNORM ? KSTEPS : 1;
  u32x4 qn_w[QN];                 // fused Q norm: weight chunk per Q chunk
  int qn_p0 = 0, qn_p1 = 0, qn_p2 = 0;  // fused Q norm: the row's positions
  {
    const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + b * a.qs[0] + (int64_t)qclamp * a.qs[1] + h * a.qs[2];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const int d0 = 16 * ks + 8 * g;
      if (d0 < a.D && row_ok)
        qreg[ks] = *reinterpret_cast<const bf16x8*>(qp + d0);
      else
        qreg[ks] = bf16x8{};
    }
    if constexpr (QNORM) {
      // The weight chunks of this lane's channels and the row's positions,
      // read with Q; the norm itself runs once the first key/value tiles are
      // in flight (qnorm_apply), so these loads overlap theirs.
      const __bf16* wp = reinterpret_cast<const __bf16*>(a.wq);
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const int d0 = 16 * ks + 8 * g;
        qn_w[ks] = u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};  // bf16 pairs of 1.0
        if (wp != nullptr && d0 < a.D && row_ok) qn_w[ks] = *reinterpret_cast<const u32x4*>(wp + d0);
      }
      const int32_t* pp = a.qpos + 3 * (int64_t)qclamp;
      qn_p0 = pp[0];
      qn_p1 = pp[1];
      qn_p2 = pp[2];
    }
  }
  // Q's RMSNorm over the D channels (the row is split between this lane and
  // the lane 32 apart, the other k-group: one exchange completes the sum of
  // squares), the weight, the rotation and q_scale, rounded once to bf16.
  // Pair p = 8 ks + 4 g + i of the row turns by pos[axis_p] * omega_p turns,
  // formed in double (as a sum over the three axes with the other axes'
  // frequencies 0, so without a per-pair choice of axis) and evaluated as the
  // norm kernel evaluates it, so Q and K turn by the same angles.
  auto qnorm_apply = [&]() __attribute__((always_inline)) {
    if constexpr (QNORM) {
      // Nothing moves above this point: the first tiles' loads are issued
      // before the wait for Q, which then counts only the older loads.
      __builtin_amdgcn_sched_barrier(0);
      float ss = 0.f;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const u32x4 w = __builtin_bit_cast(u32x4, qreg[ks]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x0 = bf16_lo(w[i]), x1 = bf16_hi(w[i]);
          ss = fmaf(x0, x0, ss);
          ss = fmaf(x1, x1, ss);
        }
      }
      ss += __shfl_xor(ss, 32, 64);
      const float inv = 1.0f / sqrtf(ss / (float)a.D + a.eps) * a.q_scale;
      const double pd0 = qn_p0, pd1 = qn_p1, pd2 = qn_p2;
      // The frequencies are read through the kernel-argument segment (the
      // argument struct sits at its start) where they are used, so that one
      // chunk's worth is live at a time instead of all of them from entry.
      using const_f64 = const __attribute__((address_space(4))) double;
      const_f64* om = (const_f64*)((const_u8*)__builtin_amdgcn_kernarg_segment_ptr() + offsetof(AttnArgs, omega_axis));
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const int d0 = 16 * ks + 8 * g;
        const u32x4 w = __builtin_bit_cast(u32x4, qreg[ks]);
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // This chunk's pair i is pair j0 in k-group 0 and j0 + 4 in k-group
          // 1.  Both phases are formed from wave-uniform frequencies (scalar
          // loads) and the lane keeps its own: selecting a frequency per lane
          // would turn its load into a per-lane one.
          const int j0 = 8 * ks + i;
          constexpr int M = kMaxPairs;
          const double t0 = fma(pd2, om[2 * M + j0], fma(pd1, om[M + j0], pd0 * om[j0]));
          const double t1 = fma(pd2, om[2 * M + j0 + 4], fma(pd1, om[M + j0 + 4], pd0 * om[j0 + 4]));
          float sn, cs;
          sincos_turns(g ? t1 : t0, sn, cs);
          const float y0 = bf16_lo(w[i]) * inv * bf16_lo(qn_w[ks][i]);
          const float y1 = bf16_hi(w[i]) * inv * bf16_hi(qn_w[ks][i]);
          o[i] = pack_bf16x2(y0 * cs - y1 * sn, y0 * sn + y1 * cs);
        }
        // Channels past D and rows past the end keep their zeros.
        const bool keep = d0 < a.D && row_ok;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = keep ? o[i] : w[i];
        qreg[ks] = __builtin_bit_cast(bf16x8, o);
        // One chunk's frequencies live at a time: hoisting every scalar load
        // to the top would hold 384 SGPRs and spill.
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Key tiles this work-group visits (the largest bound of its waves).  Bare
  // barrier: only the s_lim stores must have landed, not the Q loads.
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
  __builtin_amdgcn_s_barrier();
  int wg_lim = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) wg_lim = max(wg_lim, s_lim[w]);
  const int n_tiles = (wg_lim + kTileN - 1) / kTileN;

  // Global -> LDS loader on buffer resources (one per K/V source), so a
  // tile costs one address add per load.  Position p = 64*(i*NW + wave) + lane
  // of a tile is row p/16, physical chunk p%16, holding logical chunk
  // (p%16) ^ swz(row).  Rows past the end of a source read as zeros.
  const int ke = 2;  // bytes per element
  const __bf16* kc = reinterpret_cast<const __bf16*>(a.kc) + b * a.kcs[0] + kvh * a.kcs[2];
  const __bf16* vc = reinterpret_cast<const __bf16*>(a.vc) + b * a.vcs[0] + kvh * a.vcs[2];
  const __bf16* kn = reinterpret_cast<const __bf16*>(a.kn) + b * a.kns[0] + kvh * a.kns[2];
  const __bf16* vn = reinterpret_cast<const __bf16*>(a.vn) + b * a.vns[0] + kvh * a.vns[2];
  const int rkc = (int)a.kcs[1] * ke, rvc = (int)a.vcs[1] * ke;  // row strides in bytes
  const int rkn = (int)a.kns[1] * ke, rvn = (int)a.vns[1] * ke;
  const int rowbytes = a.D * ke;
  const __amdgpu_buffer_rsrc_t rs_kc = __builtin_amdgcn_make_buffer_rsrc((void*)kc, 0, P > 0 ? (P - 1) * rkc + rowbytes : 0, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs_vc = __builtin_amdgcn_make_buffer_rsrc((void*)vc, 0, P > 0 ? (P - 1) * rvc + rowbytes : 0, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs_kn = __builtin_amdgcn_make_buffer_rsrc((void*)kn, 0, (a.Snew - 1) * rkn + rowbytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs_vn = __builtin_amdgcn_make_buffer_rsrc((void*)vn, 0, (a.Snew - 1) * rvn + rowbytes, kRsrcWord3);
  // Load i of a tile covers rows lr + 4*NW*i (lr = 4*wave + lane/16), 16
  // lanes per row.  With NW a multiple of 4 the row swizzle of lr + 4*NW*i
  // equals that of lr, so one per-lane byte offset per source serves all
  // loads; the wave index is read as a scalar so the LDS destinations stay in
  // scalar registers.  Lanes whose chunk lies beyond the padded head dim get
  // an offset past every extent (bit 31 set; the host keeps extents below
  // 2^31), so they read zeros without fetching and every load instruction
  // runs unmasked.
  static_assert(NW % 4 == 0, "loader assumes whole swizzle periods per load");
  const int dchunks = a.D / 8;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int lr = 4 * wv + (lane >> 4);
  const int lc = (lane & 15) ^ swz(lr);
  const uint32_t lcol = 16 * (lc < dchunks ? lc : 0);  // padding channels: any finite data (Q is zero there)
  const uint32_t loob = lc < CHUNKS ? 0u : 0x80000000u;
  const uint32_t vo_kc = (uint32_t)(lr * rkc) + lcol + loob, vo_vc = (uint32_t)(lr * rvc) + lcol + loob;
  const uint32_t vo_kn = (uint32_t)(lr * rkn) + lcol + loob, vo_vn = (uint32_t)(lr * rvn) + lcol + loob;
  constexpr int kSlab = 4 * NW;  // rows per load instruction and work-group
  // Byte offsets are formed in unsigned 32-bit arithmetic: a row just past the
  // end of a slice whose span is close to 2^31 bytes has an offset above 2^31,
  // which reads as zeros (past the extent) and must not be a signed overflow.
  // A tile past the work-group's last one is still issued, through a resource
  // of extent zero (every lane reads zeros, nothing is fetched), so that each
  // issue is exactly LOADS unmasked instructions per wave and the waits below
  // can count them.  A tile holds keys of one source (all cached, k0 + 64 <= P,
  // or all new, k0 >= P; always so when P is a multiple of 64) or, only when
  // P is not, is the one tile holding key P, where each lane picks its source.
  const __amdgpu_buffer_rsrc_t rs_null = __builtin_amdgcn_make_buffer_rsrc((void*)kn, 0, 0, kRsrcWord3);
  auto issue = [&](int t, char* dst, bool is_k) __attribute__((always_inline)) {
    const bool live = t < n_tiles;
    const int k0 = live ? t * kTileN : 0;
    // The wave's LDS offset goes through an opaque copy at every issue, so
    // the load destinations (M0 values) are formed where they are used
    // instead of being hoisted, sixteen of them, into scalar registers that
    // stay live across the loop.
    int wofs = 1024 * wv;
    asm volatile("" : "+s"(wofs));
    char* d0 = dst + wofs;
    if (ALIGNED || k0 + kTileN <= P || k0 >= P) {
      const bool cached = k0 < P;
      const __amdgpu_buffer_rsrc_t r =
          pick(live, pick(cached, pick(is_k, rs_kc, rs_vc), pick(is_k, rs_kn, rs_vn)), rs_null);
      const int st = pick(cached, pick(is_k, rkc, rvc), pick(is_k, rkn, rvn));
      const uint32_t o = pick(cached, pick(is_k, vo_kc, vo_vc), pick(is_k, vo_kn, vo_vn));
      const int r0 = cached ? k0 : k0 - P;
#pragma unroll
      for (int i = 0; i < LOADS; ++i) dma16(r, d0 + 1024 * NW * i, (int)(o + (uint32_t)(r0 + kSlab * i) * (uint32_t)st));
    } else {
      const __amdgpu_buffer_rsrc_t rc = pick(is_k, rs_kc, rs_vc);
      const __amdgpu_buffer_rsrc_t rn = pick(is_k, rs_kn, rs_vn);
      const int sc = pick(is_k, rkc, rvc), sn = pick(is_k, rkn, rvn);
      const uint32_t oc = pick(is_k, vo_kc, vo_vc), on = pick(is_k, vo_kn, vo_vn);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int key = k0 + kSlab * i + lr;
        if (key < P) dma16(rc, d0 + 1024 * NW * i, (int)(oc + (uint32_t)(k0 + kSlab * i) * (uint32_t)sc));
        if (key >= P) dma16(rn, d0 + 1024 * NW * i, (int)(on + (uint32_t)(k0 - P + kSlab * i) * (uint32_t)sn));
      }
    }
  };

  // Per-lane LDS byte offsets that do not depend on the tile.
  int k_off[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    const int row = lane & 31;  // +32 rows (8192 bytes) for the second key block
    k_off[ks] = row * kRowBytes + (((2 * ks + g) ^ swz(row)) << 4);
  }
  const int G = lane >> 4;
  const int il = lane & 15;
  int v_off[MBLK][2];
#pragma unroll
  for (int mb = 0; mb < MBLK; ++mb) {
    const int d = 32 * mb + 16 * (G & 1) + 4 * (il & 3);
    const int c = d >> 3;
    const int hb = ((d >> 2) & 1) * 8;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int key = 4 * (G >> 1) + (il >> 2) + 8 * hi;  // +16 (half) and +32 (kb) keep swz
      v_off[mb][hi] = key * kRowBytes + ((c ^ swz(key)) << 4) + hb;
    }
  }

  // Softmax bookkeeping.  m_off (log2 units) is this row's offset; every S
  // tile's accumulator starts at -m_off (in logit units), so the MFMA yields
  // logits minus the offset in effect when the tile was computed.  The offset
  // only moves when a tile's max exceeds it by more than the lazy threshold,
  // so probabilities stay <= 2^8 and O is rarely rescaled; only the rows that
  // grew move, so a row's result never depends on the other rows of its wave.
  f32x16 oacc[MBLK];
#pragma unroll
  for (int mb = 0; mb < MBLK; ++mb) oacc[mb] = f32x16{};
  const float c2 = UNIT ? 1.0f : a.scale * 1.4426950408889634f;  // scale * log2(e)
  const float ic2 = UNIT ? 1.0f : 1.0f / c2;
  float m_off = 0.f;   // running offset (log2 units)
  // Every S tile's accumulator starts here: -m_off in logit units, rebuilt only
  // when the offset moves.
  f32x16 s_init;
#pragma unroll
  for (int i = 0; i < 16; ++i) s_init[i] = -m_off * ic2;
  bool fresh = true;   // no finite logit seen yet: the first one sets the offset
  float l_part = 0.f;  // this lane's share of the row sum

  // S^T (logits minus the offset, logit units) for the 64 keys of a K stage.
  auto qk = [&](const char* kt, f32x16 (&sacc)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kop = *reinterpret_cast<const bf16x8*>(kt + k_off[ks] + kb * 32 * kRowBytes);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[ks], ks == 0 ? s_init : sacc[kb], 0, 0, 0);
      }
    }
  };
  // Mask keys >= this row's bound and keys whose validity bit is 0 (only
  // tiles that reach past a wave's smallest bound or hold a padded key).
  auto mask = [&](int t, f32x16 (&sacc)[2], uint64_t word) __attribute__((always_inline)) {
    const int k0 = t * kTileN;
    const uint64_t wl = word >> (4 * g);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = 32 * kb + 8 * (i >> 2) + (i & 3);  // key within the tile, less 4g
        bool off = k0 + j + 4 * g >= lim;
        if constexpr (PADDED) off = off || ((wl >> j) & 1) == 0;
        if (off) sacc[kb][i] = -INFINITY;
      }
  };
  auto rowmax = [&](const f32x16 (&sacc)[2]) __attribute__((always_inline)) {
    float mx = sacc[0][0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[0][i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[1][i]);
    return max_with_partner32(mx);
  };
  // mx: max of the tile's shifted logits (logit units).  Rows that grew past
  // the threshold (or see their first tile) move the offset to the tile max,
  // rescale O and l, and shift the tile's logits to the new offset.
  // Without padding every row's first tile holds key 0, which it may see: the
  // prologue moves the offset for S(0) (update_first) and the loop's test is
  // the threshold alone.
  auto update = [&](float mx, f32x16 (&sacc)[2]) __attribute__((always_inline)) {
    const bool grow = PADDED ? mx > -INFINITY && (fresh || mx * c2 > kLazyRescale) : mx * c2 > kLazyRescale;
    if (__any(grow)) {
      const float d = grow ? mx : 0.f;
      const float alpha = fresh ? 0.f : __builtin_amdgcn_exp2f(-d * c2);
      l_part *= alpha;
#pragma unroll
      for (int mb = 0; mb < MBLK; ++mb) oacc[mb] *= alpha;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sacc[kb] -= d;
      m_off += d * c2;
      const float ni = -m_off * ic2;
#pragma unroll
      for (int i = 0; i < 16; ++i) s_init[i] = ni;
    }
    if constexpr (PADDED) fresh = fresh && !(mx > -INFINITY);
  };
  auto update_first = [&](float mx, f32x16 (&sacc)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sacc[kb] -= mx;
    m_off = mx * c2;
    const float ni = -m_off * ic2;
#pragma unroll
    for (int i = 0; i < 16; ++i) s_init[i] = ni;
  };
  // P = exp2(c2 * S) as bf16 B operands; row sums from the same bf16 values.
  auto softmax = [&](const f32x16 (&sacc)[2], bf16x8 (&pop)[2][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x0 = sacc[kb][8 * half + 2 * j], x1 = sacc[kb][8 * half + 2 * j + 1];
          w[j] = pack_bf16x2(__builtin_amdgcn_exp2f(UNIT ? x0 : x0 * c2), __builtin_amdgcn_exp2f(UNIT ? x1 : x1 * c2));
          if constexpr (!ONES_COL) l_part = add_bf16_pair(w[j], l_part);
        }
        pop[kb][half] = __builtin_bit_cast(bf16x8, w);
      }
    }
  };
  // One iteration: S(t) (masked, its row max mx) is in registers, K(t+1) and
  // V(t) are in LDS.  Softmax of tile t runs interleaved with the QK^T MFMAs of
  // tile t+1, then PV of tile t interleaved with the row max of tile t+1.
  // O^T += V^T P^T for the 64 keys of a V stage.
  auto pv = [&](const char* vt, const bf16x8 (&pop)[2][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int shift = (32 * kb + 16 * half) * kRowBytes;
#pragma unroll
        for (int mb = 0; mb < MBLK; ++mb) {
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(lds_void*)(vt + v_off[mb][0] + shift));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(lds_void*)(vt + v_off[mb][1] + shift));
          const u32x4 vw = {__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                            __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]};
          oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vw), pop[kb][half],
                                                            oacc[mb], 0, 0, 0);
        }
      }
    }
  };

  // Iteration t, phase 1: S(t) (masked, its max mx_cur) is in s_cur and K(t+1)
  // is in LDS; the softmax of tile t runs interleaved with the QK^T MFMAs of
  // tile t+1.  Phase 2: V(t) is in LDS; PV of tile t runs interleaved with the
  // mask and row max of tile t+1.
  // Two S buffers alternate roles across the unrolled iteration pair (tile t
  // even: S(t) in sA, S(t+1) into sB; odd: the reverse), so no copies.
  f32x16 sA[2], sB[2];
  bf16x8 pop[2][2];
  float mx_cur = -INFINITY;
  // t: the tile whose S is in s_cur; tn: the tile after it (t + 1, or without
  // padding the next tile that holds a valid key); wn: tn's validity word.
  auto phase1 = [&](int t, int tn, const char* k_next, f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2])
                    __attribute__((always_inline)) {
    const int k0 = t * kTileN;
    if (k0 >= wlim_max) return;  // wave-uniform: nothing allowed from here on
    update(mx_cur, s_cur);
    const int k1 = PADDED ? tn * kTileN : k0 + kTileN;
    const bool has_next = k1 < wlim_max && k1 < Sk;
    softmax(s_cur, pop);
    if (has_next) {
      qk(k_next, s_nxt);
      __builtin_amdgcn_sched_group_barrier(0x100, PF_K, 0);  // DS read (K operand) ahead
#pragma unroll
      for (int i = 0; i < 2 * KSTEPS - PF_K; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
      }
#pragma unroll
      for (int i = 0; i < PF_K; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
    }
  };
  auto phase2 = [&](int t, int tn, const char* v_cur, f32x16 (&s_nxt)[2], uint64_t wn)
                    __attribute__((always_inline)) {
    const int k0 = t * kTileN;
    if (k0 >= wlim_max) return;
    const int k1 = PADDED ? tn * kTileN : k0 + kTileN;
    const bool has_next = k1 < wlim_max && k1 < Sk;
    if (has_next) {
      if (k1 + kTileN > wlim_min || wn != ~0ull) {
        pv(v_cur, pop);
        mask(PADDED ? tn : t + 1, s_nxt, wn);
        mx_cur = rowmax(s_nxt);
      } else {
        pv(v_cur, pop);
        mx_cur = rowmax(s_nxt);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF_V, 0);  // V^T reads ahead
#pragma unroll
        for (int i = 0; i < 4 * MBLK - PF_V; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read (transposed)
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
        }
#pragma unroll
        for (int i = 0; i < PF_V; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        }
      }
    } else {
      pv(v_cur, pop);
    }
  };


  // Load schedule (two K and two V stages).  A stage is refilled right after
  // the barrier that ends its last read: K(t+3) at the middle of iteration t
  // (after QK^T(t+1) read K(t+1)), V(t+2) at the top of iteration t+1 (after
  // PV(t) read V(t)).  Each tile thus has 1.5 iterations to land.  Every issue
  // is exactly LOADS vector-memory instructions per wave (at least LOADS on a
  // tile that mixes cached and new keys) and loads complete in order, so at
  // each wait "at most 2*LOADS outstanding" means the tile issued two issues
  // earlier has landed:
  //   top of t:  K(t+1) | V(t), K(t+2)     -> K(t+1) in LDS
  //   mid of t:  V(t)   | K(t+2), V(t+1)   -> V(t) in LDS
  // Each wave waits for its own loads and its own LDS reads, then a bare
  // barrier (a workgroup fence would drain every load in flight) makes the
  // tile whole and the stage about to be refilled unread.
  auto wait_tile = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * LOADS, 0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // The ones column of a landed V tile.  Each wave writes it into the 16 rows
  // its own loads filled (rows 4 wave + j + 16 i), after its wait for those
  // loads and before the barrier that hands the tile to every wave: no other
  // wave's loads touch those rows, and the load issues stay unconditional.
  auto ones_col = [&](char* vt) __attribute__((always_inline)) {
    if constexpr (ONES_COL) {
      if ((lane & 15) < 4) {
        const int row = 4 * wv + (lane >> 4) + kSlab * (lane & 3);
        *reinterpret_cast<u32x4*>(vt + row * kRowBytes + ((CHUNKS ^ swz(row)) << 4)) =
            u32x4{0x3f80u, 0u, 0u, 0u};  // bf16 1.0 in channel 8 * CHUNKS
      }
    }
  };
  // As wait_tile, for the barrier after which the V tile in vt is read.
  auto wait_tile_v = [&](char* vt) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * LOADS, 0));
    if constexpr (ONES_COL) {
      ones_col(vt);
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  if constexpr (!PADDED) {
    // Prologue: K(0), K(1), V(0); S(0) once they land; then K(2).
    issue(0, sK0, true);
    issue(1, sK1, true);
    issue(0, sV0, false);
    qnorm_apply();
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    if constexpr (ONES_COL) {
      ones_col(sV0);
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    qk(sK0, sA);
    if (kTileN > wlim_min) mask(0, sA, ~0ull);
    update_first(rowmax(sA), sA);
    fresh = false;
    mx_cur = -INFINITY;  // S(0) is shifted already: nothing to move in phase 1
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    __builtin_amdgcn_s_barrier();  // every wave is done with K(0)
    asm volatile("" ::: "memory");
    issue(2, sK0, true);

    // Stages are named statically, two iterations per trip.
    for (int t = 0; t < n_tiles; t += 2) {
      wait_tile();  // K(t+1) in sK1; sV1 (V(t-1)) read by every wave
      issue(t + 1, sV1, false);
      phase1(t, t + 1, sK1, sA, sB);
      wait_tile_v(sV0);  // V(t) in sV0; sK1 (K(t+1)) read by every wave
      issue(t + 3, sK1, true);
      phase2(t, t + 1, sV0, sB, ~0ull);
      if (t + 1 >= n_tiles) break;
      wait_tile();  // K(t+2) in sK0; sV0 (V(t)) read by every wave
      issue(t + 2, sV0, false);
      phase1(t + 1, t + 2, sK0, sB, sA);
      wait_tile_v(sV1);  // V(t+1) in sV1; sK0 (K(t+2)) read by every wave
      issue(t + 4, sK0, true);
      phase2(t + 1, t + 2, sV1, sA, ~0ull);
    }
  } else {
    // Padded keys: the same schedule over the tiles that hold a valid key.
    // Iteration i runs tile T(i); tiles whose validity word is 0 are never
    // loaded or computed (they would add probability 0 to every row).  T(i+3)
    // is needed at the middle of iteration i: its first candidate's word is
    // read before the barrier there (whose wait covers the load) and only a
    // run of empty tiles costs further, serial reads.  Indices at or past
    // n_tiles are dead tiles (zero loads, phases return at once).
    auto skip_empty = [&](int x, uint64_t& w) __attribute__((always_inline)) {
      if (w == 0) {  // rare: a run of empty tiles (or a dead index)
        while (x < n_tiles && w == 0) {
          ++x;
          w = tile_word(min(x, last_tile));
        }
      }
      return x;
    };
    uint64_t w0 = pw0;
    const int t0 = skip_empty(0, w0);
    uint64_t w1 = t0 == 0 ? pw1 : tile_word(min(t0 + 1, last_tile));
    int ta = t0, tb = skip_empty(t0 + 1, w1);  // T(i), T(i+1)
    uint64_t w2 = tb == 1 ? pw2 : tile_word(min(tb + 1, last_tile));
    int tc = skip_empty(tb + 1, w2);  // T(i+2)
    uint64_t wb = w1, wc = w2;        // words of T(i+1), T(i+2)

    issue(t0, sK0, true);
    issue(tb, sK1, true);
    issue(t0, sV0, false);
    qnorm_apply();
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    if constexpr (ONES_COL) {
      ones_col(sV0);
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    qk(sK0, sA);
    if ((t0 + 1) * kTileN > wlim_min || w0 != ~0ull) mask(t0, sA, w0);
    mx_cur = rowmax(sA);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    __builtin_amdgcn_s_barrier();  // every wave is done with K(T(0))
    asm volatile("" ::: "memory");
    issue(tc, sK0, true);

    while (ta < n_tiles) {
      wait_tile();  // K(T(i+1)) in sK1
      issue(tb, sV1, false);
      phase1(ta, tb, sK1, sA, sB);
      uint64_t wd = tile_word(min(tc + 1, last_tile));
      wait_tile_v(sV0);  // V(T(i)) in sV0
      int td = skip_empty(tc + 1, wd);  // T(i+3)
      issue(td, sK1, true);
      phase2(ta, tb, sV0, sB, wb);
      ta = tb, tb = tc, tc = td;
      wb = wc, wc = wd;
      if (ta >= n_tiles) break;
      wait_tile();  // K(T(i+2)) in sK0
      issue(tb, sV0, false);
      phase1(ta, tb, sK0, sB, sA);
      wd = tile_word(min(tc + 1, last_tile));
      wait_tile_v(sV1);  // V(T(i+1)) in sV1
      td = skip_empty(tc + 1, wd);
      issue(td, sK0, true);
      phase2(ta, tb, sV1, sA, wb);
      ta = tb, tb = tc, tc = td;
      wb = wc, wc = wd;
    }
  }
  // Tiles past the last one were issued too: drain before the work-group's
  // LDS can be handed to another.
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));

  // Normalise and store: lane holds query (lane & 31), channels
  // 32*mb + 8*(i/4) + 4*g + (i%4).
  float l_own = l_part;
  if constexpr (ONES_COL) {
    // Channel 8 * CHUNKS is element (c0 / 8) * 4 of the last O^T block in
    // the k-group-0 lanes; the partner lane 32 apart holds channel
    // 8 * CHUNKS + 4 there, which is zero, so the pair sum is the row sum.
    constexpr int c0 = 8 * CHUNKS - 32 * (MBLK - 1);
    static_assert(c0 % 8 == 0, "ones column on a chunk boundary");
    l_own = oacc[MBLK - 1][(c0 / 8) * 4];
  }
  const float l_tot = sum_with_partner32(l_own);
  const bool empty = PADDED && !(l_tot > 0.f);  // no valid key: O = 0, lse = -inf
  const float inv = empty ? 0.f : 1.0f / l_tot;
  // The output arguments are read here, through an opaque copy of the
  // kernel-argument pointer, so that they are not loaded at entry and held in
  // scalar registers (or spilled) across the tile loop.
  using const_args = const __attribute__((address_space(4))) AttnArgs;
  const_args* ka = (const_args*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(ka));
  if (row_ok) {
    __bf16* op = reinterpret_cast<__bf16*>(ka->o) + b * ka->os[0] + (int64_t)qrow * ka->os[1] + h * ka->os[2];
#pragma unroll
    for (int mb = 0; mb < MBLK; ++mb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = 32 * mb + 8 * r + 4 * g;
        if (d < a.D) {
          u32x2 w;
          w[0] = pack_bf16x2(oacc[mb][4 * r + 0] * inv, oacc[mb][4 * r + 1] * inv);
          w[1] = pack_bf16x2(oacc[mb][4 * r + 2] * inv, oacc[mb][4 * r + 3] * inv);
          *reinterpret_cast<u32x2*>(op + d) = w;
        }
      }
    }
    float* lse = ka->lse;
    if (lse != nullptr && g == 0)
      lse[((int64_t)b * ka->H + h) * ka->Snew + qrow] = empty ? -INFINITY : (m_off + __log2f(l_tot)) * 0.6931471805599453f;
  }
}

// fp32 path: one thread per query row, K/V tiles of 32 keys in LDS, exact
// online softmax per tile.  Used for fp32 inputs (parity-grade small shapes).
// fp32 path: one work-group of 256 threads per 64 query rows of one
// (batch, head); each row is split over 4 neighbouring lanes that hold DP/4
// channels of q and O each (so no head dim needs private memory), and a score
// is the sum of the 4 partial dot products (two exchanges within the group).
// Keys go through LDS in tiles of 32 with an exact online softmax per tile.
template <int DP>
__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(AttnArgs a) {
  constexpr int TK = 32;
  constexpr int CH = DP / 4;  // channels per lane
  __shared__ float sk[TK][DP];
  __shared__ float sv[TK][DP];
  __shared__ int s_lim[4];
  const int tid = threadIdx.x;
  const int c = tid & 3;  // lane within the row's group: channels c*CH .. c*CH + CH-1
  const int n_qtiles = (a.Snew + 63) / 64;
  const int bh = blockIdx.x / n_qtiles;
  const int qt = blockIdx.x % n_qtiles;
  const int h = bh % a.H;
  const int b = bh / a.H;
  const int kvh = h / (a.H / a.Hk);
  const int qrow = qt * 64 + (tid >> 2);
  const bool row_ok = qrow < a.Snew;
  const int qclamp = row_ok ? qrow : a.Snew - 1;
  const int lim = a.kv_limit ? a.kv_limit[a.P + qclamp] : a.Sk;
  const uint64_t* kbits = a.key_bits ? a.key_bits + (int64_t)b * a.kb_stride : nullptr;
  int wlim = lim;
  for (int m = 32; m >= 1; m >>= 1) wlim = max(wlim, __shfl_xor(wlim, m, 64));
  if ((tid & 63) == 0) s_lim[tid >> 6] = wlim;
  __syncthreads();
  wlim = max(max(s_lim[0], s_lim[1]), max(s_lim[2], s_lim[3]));

  float q[CH], o[CH];
  const float* qp = reinterpret_cast<const float*>(a.q) + b * a.qs[0] + (int64_t)qclamp * a.qs[1] + h * a.qs[2];
#pragma unroll
  for (int d = 0; d < CH; ++d) {
    const int dd = c * CH + d;
    q[d] = dd < a.D ? qp[dd] : 0.f;
    o[d] = 0.f;
  }
  float m_cur = -INFINITY, l = 0.f;
  for (int k0 = 0; k0 < wlim; k0 += TK) {
    __syncthreads();
    for (int e = tid; e < TK * DP; e += 256) {
      const int r = e / DP, d = e % DP;
      int key = k0 + r;
      key = key < a.Sk ? key : a.Sk - 1;
      float kvv = 0.f, vvv = 0.f;
      if (d < a.D) {
        if (key < a.P) {
          kvv = reinterpret_cast<const float*>(a.kc)[b * a.kcs[0] + (int64_t)key * a.kcs[1] + kvh * a.kcs[2] + d];
          vvv = reinterpret_cast<const float*>(a.vc)[b * a.vcs[0] + (int64_t)key * a.vcs[1] + kvh * a.vcs[2] + d];
        } else {
          const int kk = key - a.P;
          kvv = reinterpret_cast<const float*>(a.kn)[b * a.kns[0] + (int64_t)kk * a.kns[1] + kvh * a.kns[2] + d];
          vvv = reinterpret_cast<const float*>(a.vn)[b * a.vns[0] + (int64_t)kk * a.vns[1] + kvh * a.vns[2] + d];
        }
      }
      sk[r][d] = kvv;
      sv[r][d] = vvv;
    }
    __syncthreads();
    float s[TK];
    float mx = -INFINITY;
    // Validity of keys k0 .. k0 + 31 (one half of a 64-key word).
    const uint32_t vbits = kbits ? (uint32_t)(kbits[k0 >> 6] >> (k0 & 63)) : 0xffffffffu;
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < CH; ++d) acc = fmaf(q[d], sk[j][c * CH + d], acc);
      acc += __shfl_xor(acc, 1, 64);
      acc += __shfl_xor(acc, 2, 64);
      s[j] = (k0 + j < lim && ((vbits >> j) & 1u)) ? acc * a.scale : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_cur, mx);
    if (m_new > -INFINITY) {
      const float alpha = expf(m_cur - m_new);
      l *= alpha;
#pragma unroll
      for (int d = 0; d < CH; ++d) o[d] *= alpha;
#pragma unroll
      for (int j = 0; j < TK; ++j) {
        const float p = expf(s[j] - m_new);
        l += p;
#pragma unroll
        for (int d = 0; d < CH; ++d) o[d] = fmaf(p, sv[j][c * CH + d], o[d]);
      }
      m_cur = m_new;
    }
  }
  if (row_ok) {
    float* op = reinterpret_cast<float*>(a.o) + b * a.os[0] + (int64_t)qrow * a.os[1] + h * a.os[2];
    // A row with no valid key (padding) has l = 0: O = 0, lse = -inf.
    const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
    for (int d = 0; d < CH; ++d)
      if (c * CH + d < a.D) op[c * CH + d] = o[d] * inv;
    if (a.lse != nullptr && c == 0)
      a.lse[((int64_t)b * a.H + h) * a.Snew + qrow] = l > 0.f ? m_cur + logf(l) : -INFINITY;
  }
}

constexpr int kWaves = 4;

template <int DP, bool UNIT, bool ALIGNED>
void launch_bf16_variant(const AttnArgs& a, dim3 grid, hipStream_t stream) {
  const dim3 block(kWaves * 64);
  if constexpr (UNIT) {  // the fused Q norm always folds the scale into Q
    if (a.qpos != nullptr) {
      if (a.key_bits != nullptr)
        hipLaunchKernelGGL((attn_fwd_bf16_kernel<DP, kWaves, true, ALIGNED, true, true>), grid, block, 0, stream,
                           a);
      else
        hipLaunchKernelGGL((attn_fwd_bf16_kernel<DP, kWaves, true, ALIGNED, false, true>), grid, block, 0, stream,
                           a);
      return;
    }
  }
  if (a.key_bits != nullptr)
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<DP, kWaves, UNIT, ALIGNED, true, false>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<DP, kWaves, UNIT, ALIGNED, false, false>), grid, block, 0, stream, a);
}

template <int DP>
hipError_t launch_bf16(const AttnArgs& a, hipStream_t stream) {
  const int n_qtiles = (a.Snew + 32 * kWaves - 1) / (32 * kWaves);
  const long long nblocks = (long long)n_qtiles * a.B * a.H;
  // Q pre-scaled by scale * log2(e): the scale argument is ln 2 (to rounding).
  const bool unit = std::fabs((double)a.scale * 1.4426950408889634 - 1.0) < 1e-6;
  const bool aligned = a.P % 64 == 0;
  const dim3 grid((unsigned)nblocks);
  if (unit && aligned)
    launch_bf16_variant<DP, true, true>(a, grid, stream);
  else if (unit)
    launch_bf16_variant<DP, true, false>(a, grid, stream);
  else if (aligned)
    launch_bf16_variant<DP, false, true>(a, grid, stream);
  else
    launch_bf16_variant<DP, false, false>(a, grid, stream);
  return hipGetLastError();
}

template <int DP>
hipError_t launch_f32(const AttnArgs& a, hipStream_t stream) {
  const int n_qtiles = (a.Snew + 63) / 64;
  const long long nblocks = (long long)n_qtiles * a.B * a.H;
  hipLaunchKernelGGL((attn_fwd_f32_kernel<DP>), dim3((unsigned)nblocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, int dtype, hipStream_t stream) {
  const int dp = (a.D + 31) / 32 * 32;
  if (dtype == 0) {
    // Head dims 65..80 (Lumina-Next's 72) take five QK^T steps instead of six.
    if (a.D > 64 && a.D <= 80) return launch_bf16<80>(a, stream);
    switch (dp) {
      case 32: return launch_bf16<32>(a, stream);
      case 64: return launch_bf16<64>(a, stream);
      case 96: return launch_bf16<96>(a, stream);
      case 128: return launch_bf16<128>(a, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (dp) {
    case 32: return launch_f32<32>(a, stream);
    case 64: return launch_f32<64>(a, stream);
    case 96: return launch_f32<96>(a, stream);
    case 128: return launch_f32<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dit
