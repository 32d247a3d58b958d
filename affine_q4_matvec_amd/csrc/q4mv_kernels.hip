// HIP kernels for gfx950 (CDNA4, wave64): the affine 4-bit matvec (q4mv).
//
// y[r] = sum_g s[r,g] * (q[r,g] . x_g) + b[r,g] * xs[g] over 64-column
// groups ("Array.q4mv on Metal: one kernel thread per row for products of
// 4M weights or more, bit-identical" (#1435), Change), with every row summed
// in a fixed tree order ("Metal: queued rmsq, swq, gdn and atq kernels and a
// 4-row q4mv ..." (#1440), Change, q4mv bullet).  Fixed mode, per row:
//   p_i = q_i * x_i;  d_g = T(p over the group);  t_g = (s*d_g) + (b*xs_g);
//   y = T(t over the groups)
// with T the canonical tree described in q4mv_device.h.
//
// Three kernel shapes, all reading each code byte from HBM once:
//   row64  rows of exactly 2048 columns (32 groups): one wave per row,
//          lane l owns columns [32l, 32l+32) and keeps their activations in
//          registers across all rows it visits (the pages' 4-row sharing of
//          one activation group by several rows, taken to every row of the
//          wave); one 16-byte buffer load per lane and row.
//   seg    rows of at most 31 groups: 64/LPR row segments of LPR lanes.
//   split  rows of more than 32 groups: one wave per 2048-column pass, pass
//          sums combined through LDS with the tree over passes.
//
// Fused stages (one kernel instead of two or three; same bits as the
// separate kernels, because the same code computes them):
//   prologue kProXsum    the group sums of x are formed in the kernel (each
//                        lane pair: T over its 32 + 32 activations)
//   prologue kProNorm    x = rmsq(h, wn): the workgroup forms rho, each lane
//                        its own 32 normalised activations and group sum
//   epilogue kEpiSwiglu  rows come in (gate, up) pairs; the pair's outputs
//                        go through swq's SwiGLU into m[r/2]
//   epilogue kEpiArgmax  greedy argmax of y: each workgroup writes the key
//                        of its best row; a one-workgroup kernel picks the
//                        largest key
#include <string.h>

#include <atomic>

#include "ops_device.h"
#include "q4mv_device.h"

#ifndef Q4_ROW64_MAX_WG
#define Q4_ROW64_MAX_WG 2048  // cap when the occupancy query is unavailable
#endif
#ifndef Q4_ROW64_OCC_PCT
#define Q4_ROW64_OCC_PCT 100  // share of the resident workgroups launched
#endif
// A row64 launch whose waves loop over several blocks runs one workgroup of
// 16 waves per compute unit (4 per SIMD).
constexpr int kLoopThreads = 1024;
constexpr int kLoopWaves = kLoopThreads / 64;
#ifndef Q4_SPLIT_R
#define Q4_SPLIT_R 4  // a multiple of 4
#endif
#ifndef Q4_SPLIT_MAX_WG
#define Q4_SPLIT_MAX_WG 2048
#endif
#ifndef Q4_SEG_MAX_WG
#define Q4_SEG_MAX_WG 1024
#endif

namespace q4 {
namespace {

using namespace dev;

constexpr int kSegR = 4;
constexpr int kThreads = 256;
// Rows per block of the row64 kernel: four rows share each lane's
// activations and are reduced together (quad_row_sums).  The measurement
// variants (q4mv_variant) instantiate it for 1, 2 and 8 rows as well.
constexpr int kRow64R = 4;
static_assert(kRow64R % 2 == 0, "the SwiGLU epilogue takes (gate, up) row pairs of a block");

// Activations of `chunk` and its group sum for prologues kProX / kProXsum.
template <int PRO>
__device__ __forceinline__ void chunk_inputs(const Prod &P, int chunk, bool active, float *xv,
                                             float &xsv) {
  load_x_values(P.x + 32 * chunk, active, xv);
  if constexpr (PRO == kProXsum)
    xsv = pair_group_sum(xv);
  else
    xsv = active ? P.xs[chunk >> 1] : 0.0f;
}

// ---------------------------------------------------------------------------
// row64
// ---------------------------------------------------------------------------
template <int R>
struct Row64Block {
  u32x4 cw[R];
  float sv[R], bv[R];
};

// Issues the loads of rows [r0, r0 + nrows) (codes, scales, biases).
template <int R>
__device__ __forceinline__ void row64_load(const Prod &P, int r0, int nrows, uint32_t voff_q,
                                           uint32_t voff_g, Row64Block<R> &blk) {
  constexpr uint32_t kRowBytes = 1024;   // 2048 codes
  constexpr uint32_t kGroupBytes = 128;  // 32 groups of 4 bytes
  const auto qr = buffer(P.q + (size_t)r0 * 256, nrows * kRowBytes);
  const auto sr = buffer(P.s + (size_t)r0 * 32, nrows * kGroupBytes);
  const auto br = buffer(P.b + (size_t)r0 * 32, nrows * kGroupBytes);
#pragma unroll
  for (int j = 0; j < R; ++j) {
    blk.cw[j] = load_codes(qr, voff_q, j * kRowBytes);
    blk.sv[j] = load_f32(sr, voff_g, j * kGroupBytes);
    blk.bv[j] = load_f32(br, voff_g, j * kGroupBytes);
  }
}

// Greedy pick over the rows a wave has summed.
struct RunningMax {
  float value = 0.0f;
  int index = -1;  // -1: no row yet
  bool nan = false;
  __device__ unsigned long long key() const {
    if (nan) return ops::kNanKey;
    return index < 0 ? 0ull : ops::argmax_key(value, index);
  }
};

// One block of rows [r, r + nrows) held in `a`: group terms, row sums in the
// tree T, then the epilogue.  R a multiple of 4: four rows reduced at once,
// row j of a quad ending in lane 16 j + 15; otherwise each row on its own,
// ending in lane 63.
template <int R, bool FAST, int EPI, class Store>
__device__ __forceinline__ void row64_block(const Prod &P, const float *xv, float xsv, int lane,
                                            int negz, int r, int nrows, const Row64Block<R> &a,
                                            RunningMax &best, SwigluBatch &batch,
                                            const Store &store_m) {
  const bool odd = lane & 1;
  constexpr bool kQuad = R % 4 == 0;
  constexpr int kSums = kQuad ? R / 4 : R;
  const int jq = kQuad ? lane >> 4 : 0;
  const bool holder = kQuad ? (lane & 15) == 15 : lane == kWave - 1;
  float tq[kSums];
  if constexpr (kQuad) {
#pragma unroll
    for (int q = 0; q < R / 4; ++q) {
      float gt[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        gt[j] = group_term<FAST>(a.cw[4 * q + j], xv, a.sv[4 * q + j], a.bv[4 * q + j], xsv,
                                 true, odd);
      tq[q] = quad_row_sums(gt[0], gt[1], gt[2], gt[3]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < R; ++j)
      tq[j] = wave_sum_lane63(
          group_term<FAST>(a.cw[j], xv, a.sv[j], a.bv[j], xsv, true, odd), negz);
  }
  if constexpr (EPI == kEpiSwiglu) {
    // (gate, up) = rows (2i, 2i + 1) of the block
#pragma unroll
    for (int i = 0; 2 * i + 1 < R; ++i) {
      if (2 * i + 1 < nrows) {
        const int jg = 2 * i, ju = 2 * i + 1;
        const int bg = __float_as_int(tq[kQuad ? jg / 4 : jg]);
        const int bu = __float_as_int(tq[kQuad ? ju / 4 : ju]);
        const float g = __int_as_float(__builtin_amdgcn_readlane(bg, kQuad ? 16 * (jg % 4) + 15 : 63));
        const float u = __int_as_float(__builtin_amdgcn_readlane(bu, kQuad ? 16 * (ju % 4) + 15 : 63));
        swiglu_push<FAST>(store_m, batch, lane, g, u, (r + jg) >> 1);
      }
    }
  } else if (holder) {
#pragma unroll
    for (int k = 0; k < kSums; ++k) {
      const int j = kQuad ? 4 * k + jq : k;
      if (j < nrows) {
        float v = tq[k];
        if (P.res) v = P.res[r + j] + v;
        P.y[r + j] = v;
        if constexpr (EPI == kEpiArgmax) {
          // a lane's rows arrive in increasing order: strictly greater
          // keeps the lowest index of equal values (and -0 == +0)
          const bool gt = (v > best.value) || best.index < 0;
          best.value = gt ? v : best.value;
          best.index = gt ? r + j : best.index;
          best.nan |= v != v;
        }
      }
    }
  }
}

// x = rmsq(h, wn) over the workgroup into LDS (4 floats of padding after
// every 32, so that the lanes' 16-byte reads of their 32 values hit
// distinct banks); the lane's 32 values and its group's sum.  Every wave of
// the workgroup must call it (two barriers).  The first workgroup also
// publishes u and its group sums when asked.
__device__ __forceinline__ void norm_prologue(const Extra &ex, int lw, int lane, float *xv,
                                              float &xsv) {
  __shared__ float red[17];
  __shared__ float su[2048 + 2048 / 8];
  __shared__ float sus[32];
  float hv[8], wv[8];
  const float rho = ops::rmsq_rho(ex.h, ex.wn, 2048, ex.eps, red, hv, wv);
  ops::rmsq_u<4>(2048, rho, hv, wv, su, sus);
  __syncthreads();
  if (lw == 0 && ex.u_out) {
    for (int i = threadIdx.x; i < 2048; i += kThreads) ex.u_out[i] = su[i + (i >> 5) * 4];
    if (threadIdx.x < 32) ex.us_out[threadIdx.x] = sus[threadIdx.x];
  }
  load_x_values(su + 36 * lane, true, xv);
  xsv = sus[lane >> 1];
}

// x = rmsq(h, wn) by each wave for itself, without LDS or barriers: lane l
// holds values [32 l, 32 l + 32).  The same trees as norm_prologue (the
// balanced tree over the 2048 squares; per group, the lane's 32 values and
// then its partner's), so the same bits.  Wave 0 of the first workgroup
// also publishes u and its group sums when asked.
__device__ __forceinline__ void norm_prologue_wave(const Extra &ex, int lw, int lane, float *xv,
                                                   float &xsv) {
  float wv[32];
  load_x_values(ex.h + 32 * lane, true, xv);
  load_x_values(ex.wn + 32 * lane, true, wv);
  const float rho = ops::rmsq_rho_wave2048(xv, ex.eps);
#pragma unroll
  for (int k = 0; k < 32; ++k) xv[k] = ops::rmsq_value(xv[k], rho, wv[k]);
  xsv = pair_group_sum(xv);
  if (lw == 0 && wave_index() == 0 && ex.u_out) {
    float4 *up = reinterpret_cast<float4 *>(ex.u_out + 32 * lane);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      up[k] = make_float4(xv[4 * k], xv[4 * k + 1], xv[4 * k + 2], xv[4 * k + 3]);
    if ((lane & 1) == 0) ex.us_out[lane >> 1] = xsv;
  }
}

// The activations of the lane: the prologue's.  `l` is the lane index.
// WAVE_NORM: rmsq by each wave (the looping launches, where the workgroup's
// barriers would hold back every wave's first block); otherwise over the
// workgroup.
template <int PRO, bool WAVE_NORM>
__device__ __forceinline__ void row64_inputs(const Prod &P, const Extra &ex, int lw, int l,
                                             float *xv, float &xsv) {
  if constexpr (PRO == kProNorm && WAVE_NORM)
    norm_prologue_wave(ex, lw, l, xv, xsv);
  else if constexpr (PRO == kProNorm)
    norm_prologue(ex, lw, l, xv, xsv);
  else
    chunk_inputs<PRO>(P, l, true, xv, xsv);
}

// PRELOAD (every wave has at most one block): the block's loads were issued
// before the prologue and `a` holds them.
template <int R, bool FAST, int EPI>
__device__ __forceinline__ void row64_single(const Prod &P, const Extra &ex, const float *xv,
                                             float xsv, int lane, int r, Row64Block<R> &a,
                                             RunningMax &best) {
  if (r >= P.rows) return;
  SwigluBatch batch;
  float *m_out = ex.m_out;
  const auto store_m = [m_out](int i, float v) { m_out[i] = v; };
  const int negz = R % 4 == 0 ? 0 : neg_zero_reg();  // only the one-row sums use it
  row64_block<R, FAST, EPI>(P, xv, xsv, lane, negz, r, min(R, P.rows - r), a, best, batch,
                                   store_m);
  if constexpr (EPI == kEpiSwiglu) swiglu_flush<FAST>(store_m, batch);
}

// Items [begin, end) of part `k` when `rows` items are split into `parts` balanced
// contiguous ranges.
__device__ __forceinline__ void balanced_range(int rows, int k, int parts, int &begin, int &end) {
  begin = (int)(((long long)rows * k) / parts);
  end = (int)(((long long)rows * (k + 1)) / parts);
}

// The blocks of workgroup lw of nwg: a contiguous, balanced range of the
// product's blocks of R rows (so that each 128-byte line of y is written
// from one XCD's L2), taken by its 16 waves as they become free.  Ticket t
// names the range's block t; waves take tickets 0..15 first and then
// one at a time from a counter in LDS, fetched while the current block is
// summed.  (Dealt statically, one block in four per wave, the first waves a
// SIMD received finished several microseconds before its last: a SIMD
// favours its oldest waves.  Here the waves that are served more take more
// blocks, and a workgroup's waves finish within about one block of each
// other; dealing a workgroup's last blocks one row per ticket, to finish
// closer together, was slower: 50.9 us on the head with whole blocks, 53.0
// with the last 4 blocks by rows, 54.5 with 8.)  A wave's tickets, and so its rows, increase.  Each block is
// loaded at the top of its iteration (issuing the next block's loads while
// summing the current one keeps two blocks of registers live and measured
// no faster).  The activations are formed in the first iteration, after
// its block's loads have gone out, so that those HBM loads are in flight
// while the prologue runs; every wave runs that first iteration, also one
// without a block.
template <int R, bool FAST, int PRO, int EPI>
__device__ __forceinline__ void row64_loop_rows(const Prod &P, const Extra &ex, int lw, int nwg,
                                                int lane, int wave, uint32_t *ticket,
                                                RunningMax &best) {
  const uint32_t voff_q = 16u * lane;
  const uint32_t voff_g = 4u * (lane >> 1);
  int b0, b1;  // this workgroup's blocks
  balanced_range((P.rows + R - 1) / R, lw, nwg, b0, b1);
  const int nblk = b1 - b0;
  const int negz = R % 4 == 0 ? 0 : neg_zero_reg();  // only the one-row sums use it
  SwigluBatch batch;
  float *m_out = ex.m_out;
  const auto store_m = [m_out](int i, float v) { m_out[i] = v; };
  // defined before the loop: a value first set inside it would be an
  // undefined loop-carried value, which costs registers
  float xv[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) xv[i] = 0.0f;
  float xsv = 0.0f;
  Row64Block<R> a;
  int t = wave;
  for (bool first = true; first || t < nblk; first = false) {
    const int r = (b0 + t) * R;
    // a wave without a block loads from a buffer of zero bytes: nothing
    const int nrows = t < nblk ? min(R, P.rows - r) : 0;
    row64_load<R>(P, nrows > 0 ? r : 0, nrows, voff_q, voff_g, a);
    if (first) {
      // the lane index hidden from the optimiser, so that the activations'
      // addresses are formed here and not held through the loop
      int l = lane;
      asm volatile("" : "+v"(l));
      row64_inputs<PRO, true>(P, ex, lw, l, xv, xsv);
    }
    if (nrows == 0) break;
    uint32_t tn = 0;
    if (lane == 0) tn = atomicAdd(ticket, 1u);
    tn = __builtin_amdgcn_readfirstlane(tn);
    row64_block<R, FAST, EPI>(P, xv, xsv, lane, negz, r, nrows, a, best, batch, store_m);
    t = (int)tn;
  }
  if constexpr (EPI == kEpiSwiglu) swiglu_flush<FAST>(store_m, batch);
}

// One workgroup of 16 waves per compute unit, looping over its blocks.
template <int R, bool FAST, int PRO, int EPI>
__global__ __launch_bounds__(kLoopThreads) void q4mv_row64_loop_kernel(ProdGroup grp, Extra ex) {
  __shared__ uint32_t ticket;
  Prod P;
  int lw = 0, nwg = 1;
  select_product(grp, P, lw, nwg);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = wave_index();
  if (threadIdx.x == 0) ticket = kLoopWaves;
  __syncthreads();
  RunningMax best;
  row64_loop_rows<R, FAST, PRO, EPI>(P, ex, lw, nwg, lane, wave, &ticket, best);
  if constexpr (EPI == kEpiArgmax) {
    // one key per workgroup; a second kernel reduces them
    __shared__ unsigned long long wbest[kLoopWaves];
    const unsigned long long k = ops::key_max_rows(best.key());
    if (lane == kWave - 1) wbest[wave] = k;
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned long long k = wbest[0];
#pragma unroll
      for (int i = 1; i < kLoopWaves; ++i) k = wbest[i] > k ? wbest[i] : k;
      ex.amax[lw] = k;
    }
  }
}

// Launches where every wave has one block at most: the block's loads go out
// before the activations are formed.
template <int R, bool FAST, int PRO, int EPI>
__global__ __launch_bounds__(kThreads) void q4mv_row64_kernel(ProdGroup grp, Extra ex) {
  Prod P;
  int lw = 0, nwg = 1;
  select_product(grp, P, lw, nwg);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = wave_index();
  const int wpg = kThreads / kWave;
  const int first = (lw * wpg + wave) * R;

  RunningMax best;
  {
    Row64Block<R> a;
    if (first < P.rows)
      row64_load<R>(P, first, min(R, P.rows - first), 16u * lane, 4u * (lane >> 1), a);
    float xv[32];
    float xsv;
    row64_inputs<PRO, false>(P, ex, lw, lane, xv, xsv);
    row64_single<R, FAST, EPI>(P, ex, xv, xsv, lane, first, a, best);
  }

  if constexpr (EPI == kEpiArgmax) {
    // one key per workgroup; a second kernel reduces them (a single counter
    // or maximum shared by every workgroup would serialise their atomics)
    __shared__ unsigned long long wbest[kThreads / kWave];
    // the best of the four holder lanes (other lanes hold key 0)
    const unsigned long long k = ops::key_max_rows(best.key());
    if (lane == kWave - 1) wbest[wave] = k;
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned long long k = wbest[0];
#pragma unroll
      for (int i = 1; i < kThreads / kWave; ++i) k = wbest[i] > k ? wbest[i] : k;
      ex.amax[lw] = k;
    }
  }
}

// ---------------------------------------------------------------------------
// seg: rows of at most 31 groups.  A wave holds 64/LPR row segments of LPR
// lanes; lane `chunk` of a segment owns columns [32 chunk, 32 chunk + 32).
// ---------------------------------------------------------------------------
template <int LPR, int R, bool FAST, int PRO>
__global__ __launch_bounds__(kThreads) void q4mv_seg_kernel(ProdGroup grp) {
  Prod P;
  int lw = 0, nwg = 1;
  select_product(grp, P, lw, nwg);

  constexpr int RPW = kWave / LPR;
  constexpr int RB = R * RPW;
  const int G = P.cols >> 6;
  const int wpr = P.cols >> 3;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = wave_index();
  const int wpg = kThreads / kWave;
  const int seg = lane / LPR;
  const int chunk = lane % LPR;
  const bool active = chunk < 2 * G;
  const int g = chunk >> 1;

  float xv[32];
  float xsv;
  chunk_inputs<PRO>(P, chunk, active, xv, xsv);

  const int waves_total = nwg * wpg;
  for (int rb = lw * wpg + wave; rb * RB < P.rows; rb += waves_total) {
    u32x4 cw[R];
    float sv[R], bv[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int r = rb * RB + j * RPW + seg;
      cw[j] = u32x4{0u, 0u, 0u, 0u};
      sv[j] = 0.0f;
      bv[j] = 0.0f;
      if (active && r < P.rows) {
        cw[j] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4 *>(P.q + (size_t)r * wpr) + chunk);
        sv[j] = P.s[(size_t)r * G + g];
        bv[j] = P.b[(size_t)r * G + g];
      }
    }
    float tot[R];
#pragma unroll
    for (int j = 0; j < R; ++j)
      tot[j] = segment_sum<LPR>(
          group_term<FAST>(cw[j], xv, sv[j], bv[j], xsv, active, chunk & 1));
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int r = rb * RB + j * RPW + seg;
      if (chunk == 0 && r < P.rows) {
        float v = tot[j];
        if (P.res) v = P.res[r] + v;
        P.y[r] = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// split: rows of more than 32 groups.  Workgroup = `passes` waves; wave p
// owns pass p (columns [2048 p, 2048 p + 2048)) of every row it visits.
// Each pass sum (T over its 32 group slots, -0 padded) goes to LDS and the
// first wave combines a row's pass sums with a -0-padded balanced tree over
// PP = next power of two >= passes, which is T over the passes.
// ---------------------------------------------------------------------------
template <int R>
struct SplitBlock {
  u32x4 cw[R];
  float sv[R], bv[R];
};

template <int R>
__device__ __forceinline__ void split_load(const Prod &P, int r0, int nrows, uint32_t voff_q,
                                           uint32_t voff_g, SplitBlock<R> &blk) {
  const int G = P.cols >> 6;
  const uint32_t row_bytes = (uint32_t)P.cols / 2;
  const uint32_t group_bytes = 4u * G;
  const auto qr = buffer(P.q + (size_t)r0 * (P.cols >> 3), nrows * row_bytes);
  const auto sr = buffer(P.s + (size_t)r0 * G, nrows * group_bytes);
  const auto br = buffer(P.b + (size_t)r0 * G, nrows * group_bytes);
#pragma unroll
  for (int j = 0; j < R; ++j) {
    blk.cw[j] = load_codes(qr, voff_q, j * row_bytes);
    blk.sv[j] = load_f32(sr, voff_g, j * group_bytes);
    blk.bv[j] = load_f32(br, voff_g, j * group_bytes);
  }
}

template <int PP, int R, bool FAST>
__device__ __forceinline__ void split_rows(const Prod &P, const float *xv, float xsv, int lane,
                                           int wave, int passes, int begin, int end,
                                           SplitBlock<R> &a, float (*part)[16]) {
  const int G = P.cols >> 6;
  const int chunk = wave * kWave + lane;
  const bool active = chunk < 2 * G;
  const bool odd = lane & 1;
  const uint32_t voff_q = 16u * chunk;
  const uint32_t voff_g = 4u * (chunk >> 1);
  // `a` holds the loads of the first block on entry
  for (int r0 = begin; r0 < end; r0 += R) {
    const int nrows = min(R, end - r0);
#pragma unroll
    for (int q = 0; q < R / 4; ++q) {
      float gt[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        gt[j] = group_term<FAST>(a.cw[4 * q + j], xv, a.sv[4 * q + j], a.bv[4 * q + j], xsv,
                                 active, odd);
      // row 4 q + j's pass sum in lanes [16 j, 16 j + 16)
      const float tq = quad_row_sums(gt[0], gt[1], gt[2], gt[3]);
      if ((lane & 15) == 15) part[4 * q + (lane >> 4)][wave] = tq;
    }
    const int r1 = r0 + R;
    if (r1 < end) split_load<R>(P, r1, min(R, end - r1), voff_q, voff_g, a);
    __syncthreads();
    if (wave == 0 && lane < R) {
      float v[PP];
#pragma unroll
      for (int k = 0; k < PP; ++k) v[k] = k < passes ? part[lane][k] : kNegZero;
#pragma unroll
      for (int w = 1; w < PP; w *= 2)
#pragma unroll
        for (int i = 0; i < PP; i += 2 * w) v[i] = v[i] + v[i + w];
      if (lane < nrows) {
        float o = v[0];
        if (P.res) o = P.res[r0 + lane] + o;
        P.y[r0 + lane] = o;
      }
    }
    __syncthreads();
  }
}

template <int PP, int R, bool FAST, int PRO>
__global__ __launch_bounds__(1024) void q4mv_split_kernel(ProdGroup grp) {
  Prod P;
  int lw = 0, nwg = 1;
  select_product(grp, P, lw, nwg);
  const int G = P.cols >> 6;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = wave_index();
  const int passes = blockDim.x / kWave;
  const int chunk = wave * kWave + lane;
  const bool active = chunk < 2 * G;
  int begin, end;  // one contiguous, balanced range of rows per workgroup
  balanced_range(P.rows, lw, nwg, begin, end);

  // the first block's loads go out before the activations are ready
  SplitBlock<R> a;
  if (begin < end)
    split_load<R>(P, begin, min(R, end - begin), 16u * chunk, 4u * (chunk >> 1), a);

  float xv[32];
  float xsv;
  chunk_inputs<PRO>(P, chunk, active, xv, xsv);
  __shared__ float part[R][16];
  split_rows<PP, R, FAST>(P, xv, xsv, lane, wave, passes, begin, end, a, part);
}

int next_pow2(int v) {
  int p = 1;
  while (p < v) p *= 2;
  return p;
}

template <bool FAST, int PRO>
hipError_t launch_seg(const ProdGroup &g, int lpr, hipStream_t st) {
  const dim3 grid(g.wg_begin[g.n]), block(kThreads);
  switch (lpr) {
    case 2: hipLaunchKernelGGL((q4mv_seg_kernel<2, kSegR, FAST, PRO>), grid, block, 0, st, g); break;
    case 4: hipLaunchKernelGGL((q4mv_seg_kernel<4, kSegR, FAST, PRO>), grid, block, 0, st, g); break;
    case 8: hipLaunchKernelGGL((q4mv_seg_kernel<8, kSegR, FAST, PRO>), grid, block, 0, st, g); break;
    case 16: hipLaunchKernelGGL((q4mv_seg_kernel<16, kSegR, FAST, PRO>), grid, block, 0, st, g); break;
    case 32: hipLaunchKernelGGL((q4mv_seg_kernel<32, kSegR, FAST, PRO>), grid, block, 0, st, g); break;
    case 64: hipLaunchKernelGGL((q4mv_seg_kernel<64, kSegR, FAST, PRO>), grid, block, 0, st, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool FAST, int PRO>
hipError_t launch_split(const ProdGroup &g, int passes, hipStream_t st) {
  const dim3 grid(g.wg_begin[g.n]), block(kWave * passes);
  switch (next_pow2(passes)) {
    case 2: hipLaunchKernelGGL((q4mv_split_kernel<2, Q4_SPLIT_R, FAST, PRO>), grid, block, 0, st, g); break;
    case 4: hipLaunchKernelGGL((q4mv_split_kernel<4, Q4_SPLIT_R, FAST, PRO>), grid, block, 0, st, g); break;
    case 8: hipLaunchKernelGGL((q4mv_split_kernel<8, Q4_SPLIT_R, FAST, PRO>), grid, block, 0, st, g); break;
    case 16: hipLaunchKernelGGL((q4mv_split_kernel<16, Q4_SPLIT_R, FAST, PRO>), grid, block, 0, st, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool FAST, int PRO, int EPI>
hipError_t launch_row64(const ProdGroup &g, bool preload, const Extra &ex, hipStream_t st) {
  if (preload)
    hipLaunchKernelGGL((q4mv_row64_kernel<kRow64R, FAST, PRO, EPI>), dim3(g.wg_begin[g.n]),
                       dim3(kThreads), 0, st, g, ex);
  else
    hipLaunchKernelGGL((q4mv_row64_loop_kernel<kRow64R, FAST, PRO, EPI>), dim3(g.wg_begin[g.n]),
                       dim3(kLoopThreads), 0, st, g, ex);
  return hipGetLastError();
}

// The row64 variants: prologue x epilogue pairs that exist.
#define Q4_ROW64_VARIANTS(X) \
  X(kProX, kEpiStore)        \
  X(kProXsum, kEpiStore)     \
  X(kProNorm, kEpiStore)     \
  X(kProNorm, kEpiSwiglu)    \
  X(kProNorm, kEpiArgmax)

template <bool FAST, bool PRELOAD>
const void *row64_ptr(int pro, int epi) {
#define Q4_PTR_CASE(P_, E_) \
  if (pro == P_ && epi == E_)   \
    return PRELOAD ? reinterpret_cast<const void *>(&q4mv_row64_kernel<kRow64R, FAST, P_, E_>)  \
                   : reinterpret_cast<const void *>(&q4mv_row64_loop_kernel<kRow64R, FAST, P_, E_>);
  Q4_ROW64_VARIANTS(Q4_PTR_CASE)
#undef Q4_PTR_CASE
  return nullptr;
}

// One block per wave or fewer: preload.
bool row64_single_pass(const ProdGroup &g) {
  for (int i = 0; i < g.n; ++i) {
    const long long waves = (long long)(g.wg_begin[i + 1] - g.wg_begin[i]) * (kThreads / kWave);
    if ((long long)g.p[i].rows > waves * kRow64R) return false;
  }
  return true;
}

template <bool FAST>
hipError_t dispatch_row64(const ProdGroup &g, const Shape &sh, const Extra &ex, hipStream_t st) {
  const bool preload = row64_single_pass(g);
#define Q4_LAUNCH_CASE(P_, E_) \
  if (sh.pro == P_ && sh.epi == E_) return launch_row64<FAST, P_, E_>(g, preload, ex, st);
  Q4_ROW64_VARIANTS(Q4_LAUNCH_CASE)
#undef Q4_LAUNCH_CASE
  return hipErrorInvalidValue;
}

// Workgroups of a row64 kernel variant that fit on the current device at
// once: its occupancy per compute unit (at most limit_per_cu if that is
// positive) times the compute units, queried once per device and variant.
constexpr int kMaxDevices = 64;
constexpr int kVariantSlots = 2 * 2 * 3 * 3;  // mode x preload x prologue x epilogue
std::atomic<int> g_resident[kMaxDevices][kVariantSlots];

int resident_workgroups(const void *kernel, int threads, int slot, int limit_per_cu) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev < 0 || dev >= kMaxDevices || slot < 0 || slot >= kVariantSlots) return 0;
  const int cached = g_resident[dev][slot].load(std::memory_order_relaxed);
  if (cached > 0) return cached;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (limit_per_cu > 0 && per_cu > limit_per_cu) per_cu = limit_per_cu;
  int v = (per_cu < 1 ? 1 : per_cu) * (cus < 1 ? 1 : cus);
  v = v * Q4_ROW64_OCC_PCT / 100;
  if (v < 1) v = 1;
  g_resident[dev][slot].store(v, std::memory_order_relaxed);
  return v;
}

int32_t clamp_wg(long long need, long long cap) {
  if (need < 1) need = 1;
  return (int32_t)(need < cap ? need : cap);
}

// ---------------------------------------------------------------------------
// Measurement variants of the 2048-column product (q4mv_variant).
//
// lane_row: one lane per row, the first Metal kernel of "Array.q4mv on
// Metal: one kernel thread per row for products of 4M weights or more,
// bit-identical" (#1435), Change.  Each lane walks its row's 32 groups in
// order, 32 bytes of codes per group (two 16-byte loads 1 KiB from the next
// lane's), with x and its group sums in LDS (every lane reads the same
// address: a broadcast).  The sums keep the fixed tree: per group the
// balanced tree over its 64 products (8-product word trees, then words,
// then the two halves), and over the groups the balanced tree of 32, formed
// as the groups arrive (a binary counter of partial sums: a left subtree is
// always added before the right one, which is T).
// ---------------------------------------------------------------------------
constexpr int kLaneRowThreads = 256;

// The term of group g of row r (fixed: T over its 64 products, then the
// unfused affine step; fast: fused multiply-adds).
template <bool FAST>
__device__ __forceinline__ float lane_row_group(const u32x4 *qr, const float *sr, const float *br,
                                                int g, const float *sx, const float *sxs) {
  const u32x4 c0 = __builtin_nontemporal_load(qr + 2 * g);
  const u32x4 c1 = __builtin_nontemporal_load(qr + 2 * g + 1);
  const float sv = sr[g], bv = br[g];
  float xv[64];
#pragma unroll
  for (int k = 0; k < 64; k += 4) {
    const float4 v = *reinterpret_cast<const float4 *>(sx + 64 * g + k);
    xv[k] = v.x;
    xv[k + 1] = v.y;
    xv[k + 2] = v.z;
    xv[k + 3] = v.w;
  }
  if constexpr (!FAST) {
    const float d = chunk_tree(c0, xv) + chunk_tree(c1, xv + 32);
    const float sd = sv * d;
    const float bx = bv * sxs[g];
    return sd + bx;
  } else {
    const float dot = chunk_dot_fast(c0, xv) + chunk_dot_fast(c1, xv + 32);
    return fmaf(sv, dot, bv * sxs[g]);
  }
}

// Row r: the groups in 8 blocks of 4.  Fixed order: each block's balanced
// tree, then the blocks' balanced tree formed as they arrive (a binary
// counter: lv[k] holds the last complete run of 2^k blocks, always added as
// the left operand), which is the balanced tree over the 32 groups, T.
template <bool FAST>
__device__ __forceinline__ float lane_row_sum(const Prod &P, int r, const float *sx,
                                              const float *sxs) {
  const u32x4 *qr = reinterpret_cast<const u32x4 *>(P.q) + (size_t)r * 64;  // 1 KiB per row
  const float *sr = P.s + (size_t)r * 32;
  const float *br = P.b + (size_t)r * 32;
  float lv0 = 0.0f, lv1 = 0.0f, lv2 = 0.0f, acc = 0.0f;
#pragma unroll 1
  for (int j = 0; j < 8; ++j) {
    float t[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) t[k] = lane_row_group<FAST>(qr, sr, br, 4 * j + k, sx, sxs);
    if constexpr (FAST) {
      acc = ((acc + t[0]) + t[1]) + (t[2] + t[3]);
    } else {
      float b = (t[0] + t[1]) + (t[2] + t[3]);
      if (j & 1) {
        b = lv0 + b;
        if (j & 2) {
          b = lv1 + b;
          if (j & 4)
            b = lv2 + b;
          else
            lv2 = b;
        } else {
          lv1 = b;
        }
      } else {
        lv0 = b;
      }
      acc = b;  // after the last block (j = 7): the sum of all 32 groups
    }
  }
  return acc;
}

template <bool FAST>
__global__ __launch_bounds__(kLaneRowThreads) void q4mv_lane_row_kernel(Prod P) {
  __shared__ float sx[2048];
  __shared__ float sxs[32];
  // x and its group sums
  for (int i = threadIdx.x; i < 2048; i += kLaneRowThreads) sx[i] = P.x[i];
  if (threadIdx.x < 32) sxs[threadIdx.x] = P.xs[threadIdx.x];
  __syncthreads();
  for (int r = blockIdx.x * kLaneRowThreads + threadIdx.x; r < P.rows;
       r += gridDim.x * kLaneRowThreads) {
    P.y[r] = lane_row_sum<FAST>(P, r, sx, sxs);
  }
}

// wave_R: the row64 kernel with R rows per block (R = 1, 2, 4, 8): the rows
// of a block share the lane's activations in registers; [P1] (#1440), Change
// and Verification, q4mv bullet, names the sharing of one activation group by
// 4 rows of a SIMD group and found 2 and 8 rows no better.
template <int R, bool FAST>
hipError_t launch_wave_variant(const Prod &p, hipStream_t st) {
  ProdGroup g;
  memset(&g, 0, sizeof(g));
  g.n = 1;
  g.p[0] = p;
  const int wpg = kThreads / kWave;
  const long long need = (p.rows + (long long)wpg * R - 1) / ((long long)wpg * R);
  int dev = 0, per_cu = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return hipErrorInvalidValue;
  const void *kpre = reinterpret_cast<const void *>(&q4mv_row64_kernel<R, FAST, kProX, kEpiStore>);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kpre, kThreads, 0) != hipSuccess)
    return hipErrorInvalidValue;
  const Extra ex{};
  if (need <= (long long)per_cu * cus) {
    for (int i = 1; i <= kMaxGroup; ++i) g.wg_begin[i] = (int32_t)need;
    hipLaunchKernelGGL((q4mv_row64_kernel<R, FAST, kProX, kEpiStore>), dim3((int)need),
                       dim3(kThreads), 0, st, g, ex);
    return hipGetLastError();
  }
  // the looping kernel: one workgroup per compute unit
  const int nwg = cus < 1 ? 1 : cus;
  for (int i = 1; i <= kMaxGroup; ++i) g.wg_begin[i] = nwg;
  hipLaunchKernelGGL((q4mv_row64_loop_kernel<R, FAST, kProX, kEpiStore>), dim3(nwg),
                     dim3(kLoopThreads), 0, st, g, ex);
  return hipGetLastError();
}

template <bool FAST>
hipError_t launch_variant(const Prod &p, int variant, hipStream_t st) {
  switch (variant) {
    case 0: {
      // one lane per row: as many workgroups as the rows need (the pages'
      // grid), at most 8 per compute unit's worth, looping beyond
      int dev = 0, cus = 0;
      if (hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return hipErrorInvalidValue;
      const long long need = (p.rows + kLaneRowThreads - 1) / kLaneRowThreads;
      const long long cap = 8LL * (cus < 1 ? 1 : cus);
      hipLaunchKernelGGL(q4mv_lane_row_kernel<FAST>, dim3((int)(need < cap ? need : cap)),
                         dim3(kLaneRowThreads), 0, st, p);
      return hipGetLastError();
    }
    case 1: return launch_wave_variant<1, FAST>(p, st);
    case 2: return launch_wave_variant<2, FAST>(p, st);
    case 4: return launch_wave_variant<4, FAST>(p, st);
    case 8: return launch_wave_variant<8, FAST>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_q4mv_variant(const Prod &p, int variant, int mode, hipStream_t st) {
  return mode != 0 ? launch_variant<true>(p, variant, st) : launch_variant<false>(p, variant, st);
}

Shape shape_of(int32_t cols, int pro, int epi) {
  const int G = cols / 64;
  if (G == 32) return Shape{Shape::kRow64, 64, 0, pro, epi};
  if (G < 32) {
    int lpr = next_pow2(2 * G);
    return Shape{Shape::kSeg, lpr < 2 ? 2 : lpr, 0, pro, epi};
  }
  return Shape{Shape::kSplit, 0, (G + 31) / 32, pro, epi};
}

bool shape_supported(const Shape &sh) {
  if (sh.kind == Shape::kRow64) return true;
  return sh.epi == kEpiStore && sh.pro != kProNorm;
}

// Resident workgroups of the row64 variant for this shape and mode.
int32_t row64_capacity(const Shape &sh, int mode, bool preload) {
  const bool fast = mode != 0;
  const void *k = fast ? (preload ? row64_ptr<true, true>(sh.pro, sh.epi)
                                  : row64_ptr<true, false>(sh.pro, sh.epi))
                       : (preload ? row64_ptr<false, true>(sh.pro, sh.epi)
                                  : row64_ptr<false, false>(sh.pro, sh.epi));
  if (!k) return 0;
  // the looping kernel: one workgroup of kLoopThreads per compute unit
  return resident_workgroups(k, preload ? kThreads : kLoopThreads,
                             18 * (fast ? 1 : 0) + 9 * (preload ? 1 : 0) + 3 * sh.pro + sh.epi,
                             preload ? 0 : 1);
}

void plan_group(const Shape &sh, int mode, const int32_t *rows, int n, int32_t *want) {
  long long total = 0;
  for (int i = 0; i < n; ++i) {
    want[i] = workgroups_for(sh, rows[i], mode);
    total += want[i];
  }
  if (sh.kind != Shape::kRow64) return;  // no cap from occupancy
  // every product one block per wave, all resident at once: the preloading
  // kernel; otherwise the looping kernel for all of them, its workgroups
  // (one per compute unit) shared in proportion to the wants
  const int wpg = kThreads / kWave;
  long long need_pre = 0;
  for (int i = 0; i < n; ++i) need_pre += (rows[i] + wpg * kRow64R - 1) / (wpg * kRow64R);
  const int cap_pre = row64_capacity(sh, mode, true);
  if (cap_pre > 0 && need_pre <= cap_pre) {
    for (int i = 0; i < n; ++i) want[i] = (rows[i] + wpg * kRow64R - 1) / (wpg * kRow64R);
    return;
  }
  total = 0;
  for (int i = 0; i < n; ++i) {
    want[i] = clamp_wg((rows[i] + kLoopWaves * kRow64R - 1) / (kLoopWaves * kRow64R),
                       Q4_ROW64_MAX_WG);
    total += want[i];
  }
  const int cap = row64_capacity(sh, mode, false);
  if (cap > 0 && total > cap)
    for (int i = 0; i < n; ++i) {
      const long long w = (long long)want[i] * cap / total;
      want[i] = (int32_t)(w < 1 ? 1 : w);
    }
}

int32_t workgroups_for(const Shape &sh, int32_t rows, int mode) {
  const int wpg = kThreads / kWave;
  switch (sh.kind) {
    case Shape::kRow64: {
      // one block of R rows per wave if that fits on the device at once
      // (the preloading kernel then runs, workgroups of kThreads);
      // otherwise the looping kernel, one workgroup of kLoopThreads per
      // compute unit
      const long long need = (rows + wpg * kRow64R - 1) / (wpg * kRow64R);
      const int cap_pre = row64_capacity(sh, mode, true);
      if (cap_pre > 0 && need <= cap_pre) return clamp_wg(need, cap_pre);
      const long long need_loop = (rows + kLoopWaves * kRow64R - 1) / (kLoopWaves * kRow64R);
      const int cap = row64_capacity(sh, mode, false);
      return clamp_wg(need_loop, cap > 0 ? cap : Q4_ROW64_MAX_WG);
    }
    case Shape::kSeg: {
      const long long per_wg = (long long)wpg * kSegR * (kWave / sh.lpr);
      return clamp_wg((rows + per_wg - 1) / per_wg, Q4_SEG_MAX_WG);
    }
    default:
      return clamp_wg((rows + Q4_SPLIT_R - 1) / Q4_SPLIT_R, Q4_SPLIT_MAX_WG);
  }
}

hipError_t launch_q4mv_group(const ProdGroup &g, const Shape &sh, int mode, const Extra &ex,
                             hipStream_t st) {
  if (!shape_supported(sh)) return hipErrorInvalidValue;
  const bool fast = mode != 0;
  switch (sh.kind) {
    case Shape::kRow64:
      return fast ? dispatch_row64<true>(g, sh, ex, st) : dispatch_row64<false>(g, sh, ex, st);
    case Shape::kSeg:
      if (sh.pro == kProXsum)
        return fast ? launch_seg<true, kProXsum>(g, sh.lpr, st)
                    : launch_seg<false, kProXsum>(g, sh.lpr, st);
      return fast ? launch_seg<true, kProX>(g, sh.lpr, st) : launch_seg<false, kProX>(g, sh.lpr, st);
    default:
      if (sh.pro == kProXsum)
        return fast ? launch_split<true, kProXsum>(g, sh.passes, st)
                    : launch_split<false, kProXsum>(g, sh.passes, st);
      return fast ? launch_split<true, kProX>(g, sh.passes, st)
                  : launch_split<false, kProX>(g, sh.passes, st);
  }
}

}  // namespace q4
