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
//          registers across all rows it visits (the pages' "4-row" sharing of
//          one activation group by several rows, taken to every row of the
//          wave); one 16-byte buffer load per lane and row.
//   seg    rows of at most 31 groups: 64/LPR row segments of LPR lanes.
//   split  rows of more than 32 groups: one wave per 2048-column pass, pass
//          sums combined through LDS with the tree over passes.
#include <atomic>

#include "q4mv_device.h"

#ifndef Q4_ROW64_R
#define Q4_ROW64_R 4  // rows per wave iteration (loads in flight per lane)
#endif
#ifndef Q4_ROW64_MAX_WG
#define Q4_ROW64_MAX_WG 2048  // workgroups of 4 waves (grid-stride beyond)
#endif
#ifndef Q4_ROW64_PREFETCH
#define Q4_ROW64_PREFETCH 0  // issue the next block's loads before summing
#endif
#ifndef Q4_ROW64_INTERLEAVE
#define Q4_ROW64_INTERLEAVE 1  // round-robin row blocks instead of ranges
#endif
#ifndef Q4_ROW64_OCC_PCT
#define Q4_ROW64_OCC_PCT 100  // share of the resident workgroups launched
#endif
#ifndef Q4_SPLIT_R
#define Q4_SPLIT_R 4
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

// Sums the rows of a loaded block and stores them (lane 63 holds the sums).
template <int R, bool FAST, bool PAIRS>
__device__ __forceinline__ void row64_finish(const Prod &P, int r0, int nrows, const float *xv,
                                             float xsv, int lane, const Row64Block<R> &blk) {
  const bool odd = lane & 1;
  const int negz = neg_zero_reg();
  float tot[R];
#pragma unroll
  for (int j = 0; j < R; ++j)
    tot[j] = wave_sum_lane63(
        group_term<FAST, PAIRS>(blk.cw[j], xv, blk.sv[j], blk.bv[j], xsv, true, odd), negz);
  if (lane == kWave - 1) {
#pragma unroll
    for (int j = 0; j < R; ++j) {
      if (j < nrows) {
        float v = tot[j];
        if (P.res) v = P.res[r0 + j] + v;
        P.y[r0 + j] = v;
      }
    }
  }
}

// Rows [begin, end) in blocks of R, or (interleaved) blocks first,
// first + step, ... of R rows.  With PREFETCH the loads of the next block
// are issued before the current block is summed (two register sets used in
// turn, so no copies).
template <int R, bool FAST, bool PAIRS>
__device__ __forceinline__ void row64_rows(const Prod &P, const float *xv, float xsv, int lane,
                                           int begin, int end, int stride) {
  const uint32_t voff_q = 16u * lane;
  const uint32_t voff_g = 4u * (lane >> 1);
  auto count = [&](int r0) { return min(R, end - r0); };
#if Q4_ROW64_PREFETCH
  Row64Block<R> a, b;
  int r0 = begin;
  if (r0 >= end) return;
  row64_load<R>(P, r0, count(r0), voff_q, voff_g, a);
  while (true) {
    const int r1 = r0 + stride;
    if (r1 < end) row64_load<R>(P, r1, count(r1), voff_q, voff_g, b);
    row64_finish<R, FAST, PAIRS>(P, r0, count(r0), xv, xsv, lane, a);
    if (r1 >= end) break;
    const int r2 = r1 + stride;
    if (r2 < end) row64_load<R>(P, r2, count(r2), voff_q, voff_g, a);
    row64_finish<R, FAST, PAIRS>(P, r1, count(r1), xv, xsv, lane, b);
    if (r2 >= end) break;
    r0 = r2;
  }
#else
  for (int r0 = begin; r0 < end; r0 += stride) {
    Row64Block<R> a;
    row64_load<R>(P, r0, count(r0), voff_q, voff_g, a);
    row64_finish<R, FAST, PAIRS>(P, r0, count(r0), xv, xsv, lane, a);
  }
#endif
}

// Rows [begin, end) of part `k` when `rows` are split into `parts` balanced
// contiguous ranges.
__device__ __forceinline__ void balanced_range(int rows, int k, int parts, int &begin, int &end) {
  begin = (int)(((long long)rows * k) / parts);
  end = (int)(((long long)rows * (k + 1)) / parts);
}

template <int R, bool FAST>
__global__ __launch_bounds__(kThreads) void q4mv_row64_kernel(ProdGroup grp) {
  Prod P;
  int lw = 0, nwg = 1;
  select_product(grp, P, lw, nwg);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = wave_index();
  const int wpg = kThreads / kWave;
  float xv[32];
  float xsv;
  load_x_chunk(P, lane, true, xv, xsv);
#if Q4_ROW64_INTERLEAVE
  // blocks of R rows dealt round-robin to the waves
  const int begin = (lw * wpg + wave) * R, end = P.rows, stride = nwg * wpg * R;
#else
  // each wave streams one contiguous, balanced range of rows
  int begin, end;
  balanced_range(P.rows, lw * wpg + wave, nwg * wpg, begin, end);
  const int stride = R;
#endif
  if (prescale_for_pairs(xv))
    row64_rows<R, FAST, true>(P, xv, xsv, lane, begin, end, stride);
  else
    row64_rows<R, FAST, false>(P, xv, xsv, lane, begin, end, stride);
}

// ---------------------------------------------------------------------------
// seg: rows of at most 31 groups.  A wave holds 64/LPR row segments of LPR
// lanes; lane `chunk` of a segment owns columns [32 chunk, 32 chunk + 32).
// ---------------------------------------------------------------------------
template <int LPR, int R, bool FAST>
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
  load_x_chunk(P, chunk, active, xv, xsv);

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
          group_term<FAST, false>(cw[j], xv, sv[j], bv[j], xsv, active, chunk & 1));
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
template <int PP, int R, bool FAST, bool PAIRS>
__device__ __forceinline__ void split_rows(const Prod &P, const float *xv, float xsv, int lane,
                                           int wave, int passes, int lw, int nwg,
                                           float (*part)[16]) {
  const int G = P.cols >> 6;
  const uint32_t row_bytes = (uint32_t)P.cols / 2;
  const uint32_t group_bytes = 4u * G;
  const int chunk = wave * kWave + lane;
  const bool active = chunk < 2 * G;
  const bool odd = lane & 1;
  const uint32_t voff_q = 16u * chunk;
  const uint32_t voff_g = 4u * (chunk >> 1);
  int begin, end;  // one contiguous, balanced range of rows per workgroup
  balanced_range(P.rows, lw, nwg, begin, end);
  for (int r0 = begin; r0 < end; r0 += R) {
    const int nrows = min(R, end - r0);
    const auto qr = buffer(P.q + (size_t)r0 * (P.cols >> 3), nrows * row_bytes);
    const auto sr = buffer(P.s + (size_t)r0 * G, nrows * group_bytes);
    const auto br = buffer(P.b + (size_t)r0 * G, nrows * group_bytes);
    u32x4 cw[R];
    float sv[R], bv[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      cw[j] = load_codes(qr, voff_q, j * row_bytes);
      sv[j] = load_f32(sr, voff_g, j * group_bytes);
      bv[j] = load_f32(br, voff_g, j * group_bytes);
    }
    const int negz = neg_zero_reg();
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const float tot = wave_sum_lane63(
          group_term<FAST, PAIRS>(cw[j], xv, sv[j], bv[j], xsv, active, odd), negz);
      if (lane == kWave - 1) part[j][wave] = tot;
    }
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

template <int PP, int R, bool FAST>
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
  float xv[32];
  float xsv;
  load_x_chunk(P, chunk, active, xv, xsv);
  // one decode choice for the whole workgroup (the loop has barriers)
  bool large = false;
#pragma unroll
  for (int k = 0; k < 32; ++k) large |= !(__builtin_fabsf(xv[k]) < 0x1p118f);
  __shared__ float part[R][16];
  if (!__syncthreads_or(large)) {
    const float scale = 1.0f / fp8_unit();
#pragma unroll
    for (int k = 0; k < 32; ++k) xv[k] = xv[k] * scale;
    split_rows<PP, R, FAST, true>(P, xv, xsv, lane, wave, passes, lw, nwg, part);
  } else {
    split_rows<PP, R, FAST, false>(P, xv, xsv, lane, wave, passes, lw, nwg, part);
  }
}

int next_pow2(int v) {
  int p = 1;
  while (p < v) p *= 2;
  return p;
}

template <bool FAST>
hipError_t launch_seg(const ProdGroup &g, int lpr, hipStream_t st) {
  const dim3 grid(g.wg_begin[g.n]), block(kThreads);
  switch (lpr) {
    case 2: hipLaunchKernelGGL((q4mv_seg_kernel<2, kSegR, FAST>), grid, block, 0, st, g); break;
    case 4: hipLaunchKernelGGL((q4mv_seg_kernel<4, kSegR, FAST>), grid, block, 0, st, g); break;
    case 8: hipLaunchKernelGGL((q4mv_seg_kernel<8, kSegR, FAST>), grid, block, 0, st, g); break;
    case 16: hipLaunchKernelGGL((q4mv_seg_kernel<16, kSegR, FAST>), grid, block, 0, st, g); break;
    case 32: hipLaunchKernelGGL((q4mv_seg_kernel<32, kSegR, FAST>), grid, block, 0, st, g); break;
    case 64: hipLaunchKernelGGL((q4mv_seg_kernel<64, kSegR, FAST>), grid, block, 0, st, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool FAST>
hipError_t launch_split(const ProdGroup &g, int passes, hipStream_t st) {
  const dim3 grid(g.wg_begin[g.n]), block(kWave * passes);
  switch (next_pow2(passes)) {
    case 2: hipLaunchKernelGGL((q4mv_split_kernel<2, Q4_SPLIT_R, FAST>), grid, block, 0, st, g); break;
    case 4: hipLaunchKernelGGL((q4mv_split_kernel<4, Q4_SPLIT_R, FAST>), grid, block, 0, st, g); break;
    case 8: hipLaunchKernelGGL((q4mv_split_kernel<8, Q4_SPLIT_R, FAST>), grid, block, 0, st, g); break;
    case 16: hipLaunchKernelGGL((q4mv_split_kernel<16, Q4_SPLIT_R, FAST>), grid, block, 0, st, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool FAST>
hipError_t launch_row64(const ProdGroup &g, hipStream_t st) {
  hipLaunchKernelGGL((q4mv_row64_kernel<Q4_ROW64_R, FAST>), dim3(g.wg_begin[g.n]), dim3(kThreads),
                     0, st, g);
  return hipGetLastError();
}

// Workgroups of a kernel (with `block` threads) that fit on the current
// device at once: its occupancy per compute unit times the compute units.
// Queried once per device and kernel slot, then cached.
constexpr int kMaxDevices = 64;
constexpr int kKernelSlots = 2;  // row64 fixed, row64 fast
std::atomic<int> g_resident[kMaxDevices][kKernelSlots];

int resident_workgroups(const void *kernel, int slot, int block) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev < 0 || dev >= kMaxDevices) return 0;
  const int cached = g_resident[dev][slot].load(std::memory_order_relaxed);
  if (cached > 0) return cached;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
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

}  // namespace

Shape shape_of(int32_t cols) {
  const int G = cols / 64;
  if (G == 32) return Shape{Shape::kRow64, 64, 0};
  if (G < 32) {
    int lpr = next_pow2(2 * G);
    return Shape{Shape::kSeg, lpr < 2 ? 2 : lpr, 0};
  }
  return Shape{Shape::kSplit, 0, (G + 31) / 32};
}

int32_t resident_capacity(const Shape &sh, int mode) {
  const bool fast = mode != 0;
  if (sh.kind != Shape::kRow64) return 0;  // no cap from occupancy
  const void *k = fast ? reinterpret_cast<const void *>(&q4mv_row64_kernel<Q4_ROW64_R, true>)
                       : reinterpret_cast<const void *>(&q4mv_row64_kernel<Q4_ROW64_R, false>);
  return resident_workgroups(k, fast ? 1 : 0, kThreads);
}

int32_t workgroups_for(const Shape &sh, int32_t rows, int mode) {
  const int wpg = kThreads / kWave;
  switch (sh.kind) {
    case Shape::kRow64: {
      // at most what fits on the device at once (no second round of
      // workgroups), at least R rows per wave
      const int cap = resident_capacity(sh, mode);
      return clamp_wg((rows + wpg * Q4_ROW64_R - 1) / (wpg * Q4_ROW64_R),
                      cap > 0 ? cap : Q4_ROW64_MAX_WG);
    }
    case Shape::kSeg: {
      const long long per_wg = (long long)wpg * kSegR * (kWave / sh.lpr);
      return clamp_wg((rows + per_wg - 1) / per_wg, Q4_SEG_MAX_WG);
    }
    default:
      return clamp_wg((rows + Q4_SPLIT_R - 1) / Q4_SPLIT_R, Q4_SPLIT_MAX_WG);
  }
}

hipError_t launch_q4mv_group(const ProdGroup &g, const Shape &sh, int mode, hipStream_t st) {
  const bool fast = mode != 0;
  switch (sh.kind) {
    case Shape::kRow64: return fast ? launch_row64<true>(g, st) : launch_row64<false>(g, st);
    case Shape::kSeg: return fast ? launch_seg<true>(g, sh.lpr, st) : launch_seg<false>(g, sh.lpr, st);
    default: return fast ? launch_split<true>(g, sh.passes, st) : launch_split<false>(g, sh.passes, st);
  }
}

}  // namespace q4
