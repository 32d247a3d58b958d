// HIP kernels for gfx950 (CDNA4, wave64): the affine 4-bit matvec (q4mv)
// and its producers.  Compiled with -ffp-contract=off: every float
// expression below is the exact sequence of IEEE binary32 / binary64
// operations it spells; fused multiply-adds appear only where written out
// (fma / fmaf), i.e. only in the Q4_FAST kernels and the fixed binary64 exp.
//
// Operations (bendlang/bend pull-request pages):
//  - q4mv: "Array.q4mv on Metal: one kernel thread per row ..." (#1435),
//    Change; rows of packed 4-bit codes with a scale and bias per
//    64-column group, summed in a fixed tree order ("Metal: queued rmsq,
//    swq, gdn and atq kernels and a 4-row q4mv ..." (#1440), Change, q4mv
//    bullet).
//  - rmsq, swq: #1440, Change (rmsq and swq bullets).
//
// The fixed summation tree T(v[0..n)) splits at the largest power of two
// below n.  It equals a balanced pairwise tree over the next power of two
// >= n in which the missing leaves are -0.0 (x + -0.0 == x for every x,
// including +-0), so a lane butterfly with -0.0 padding reproduces it for
// any n, and T over n leaves equals T over the sums of aligned blocks of any
// power-of-two size.  IEEE addition is commutative, so which lane of a
// butterfly pair adds which operand does not change a bit.
#include <math.h>

#include "q4mv_internal.h"

#pragma clang fp contract(off)

namespace q4 {
namespace {

constexpr int kWave = 64;
constexpr float kNegZero = -0.0f;

// Four packed code words (one 16-byte load).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// DPP controls of the gfx9 family.
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <- 7-i within 8 lanes
constexpr int kDppRowMirror = 0x140;      // lane i <- 15-i within 16 lanes

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum of the group terms of one row segment of LPR lanes, where each group
// term is held (identically) by a lane pair.  Requires every lane of the
// segment to run it (no divergence).  After step k every aligned block of
// 2^k lanes holds one value, so a mirror within 8 (16) lanes pairs block
// 4 (8) lanes apart, exactly like xor 4 (8).
template <int LPR>
__device__ __forceinline__ float segment_sum(float t) {
  if constexpr (LPR >= 4) t = t + dpp<kDppQuadXor2>(t);
  if constexpr (LPR >= 8) t = t + dpp<kDppRowHalfMirror>(t);
  if constexpr (LPR >= 16) t = t + dpp<kDppRowMirror>(t);
  if constexpr (LPR >= 32) t = t + __shfl_xor(t, 16);
  if constexpr (LPR >= 64) t = t + __shfl_xor(t, 32);
  return t;
}

// Balanced tree of the eight products of one packed word:
// word bits 4k..4k+3 hold code k; p_k = code_k * x_k.
__device__ __forceinline__ float word_tree(uint32_t w, const float *xk) {
  const uint32_t lo = w & 0x0F0F0F0Fu;         // codes 0, 2, 4, 6
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;  // codes 1, 3, 5, 7
  const float p0 = (float)(lo & 0xFFu) * xk[0];
  const float p1 = (float)(hi & 0xFFu) * xk[1];
  const float p2 = (float)((lo >> 8) & 0xFFu) * xk[2];
  const float p3 = (float)((hi >> 8) & 0xFFu) * xk[3];
  const float p4 = (float)((lo >> 16) & 0xFFu) * xk[4];
  const float p5 = (float)((hi >> 16) & 0xFFu) * xk[5];
  const float p6 = (float)(lo >> 24) * xk[6];
  const float p7 = (float)(hi >> 24) * xk[7];
  return ((p0 + p1) + (p2 + p3)) + ((p4 + p5) + (p6 + p7));
}

// Tree of one lane's 32-code chunk (four words, contiguous columns).
__device__ __forceinline__ float chunk_tree(u32x4 c, const float *xv) {
  return (word_tree(c.x, xv) + word_tree(c.y, xv + 8)) +
         (word_tree(c.z, xv + 16) + word_tree(c.w, xv + 24));
}

// Q4_FAST: the same dot product accumulated with fused multiply-adds.
__device__ __forceinline__ float chunk_dot_fast(u32x4 c, const float *xv) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  float acc = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t lo = w[k] & 0x0F0F0F0Fu;
    const uint32_t hi = (w[k] >> 4) & 0x0F0F0F0Fu;
    acc = fmaf((float)(lo & 0xFFu), xv[8 * k + 0], acc);
    acc = fmaf((float)(hi & 0xFFu), xv[8 * k + 1], acc);
    acc = fmaf((float)((lo >> 8) & 0xFFu), xv[8 * k + 2], acc);
    acc = fmaf((float)((hi >> 8) & 0xFFu), xv[8 * k + 3], acc);
    acc = fmaf((float)((lo >> 16) & 0xFFu), xv[8 * k + 4], acc);
    acc = fmaf((float)((hi >> 16) & 0xFFu), xv[8 * k + 5], acc);
    acc = fmaf((float)(lo >> 24), xv[8 * k + 6], acc);
    acc = fmaf((float)(hi >> 24), xv[8 * k + 7], acc);
  }
  return acc;
}

// Group term of a lane (the lane pair 2g, 2g+1 holds group g):
//   fixed: d = T(pair's chunk trees); t = (s*d) + (b*xs)
//   fast : each lane adds s*dot (+ b*xs on the even lane); the row sum then
//          runs over lanes instead of lane pairs.
template <bool FAST>
__device__ __forceinline__ float group_term(u32x4 c, const float *xv, float sv, float bv,
                                            float xsv, bool active, bool odd) {
  if constexpr (!FAST) {
    float L = chunk_tree(c, xv);
    L = active ? L : kNegZero;
    const float d = L + dpp<kDppQuadXor1>(L);
    const float sd = sv * d;
    const float bx = bv * xsv;
    const float t = sd + bx;
    return active ? t : kNegZero;
  } else {
    const float acc = chunk_dot_fast(c, xv);
    float t = fmaf(sv, acc, odd ? 0.0f : bv * xsv);
    t = active ? t : 0.0f;
    return t + dpp<kDppQuadXor1>(t);
  }
}

// Picks product i of a group with constant indices only (a dynamic index
// into the kernel-argument struct would spill it to scratch).
__device__ __forceinline__ void select_product(const ProdGroup &grp, Prod &P, int &lw,
                                               int &nwg) {
  const int bid = blockIdx.x;
  int pi = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroup; ++i)
    if (i < grp.n && bid >= grp.wg_begin[i]) pi = i;
#pragma unroll
  for (int i = 0; i < kMaxGroup; ++i) {
    if (i == pi) {
      P = grp.p[i];
      lw = bid - grp.wg_begin[i];
      nwg = grp.wg_begin[i + 1] - grp.wg_begin[i];
    }
  }
}

__device__ __forceinline__ void load_x_chunk(const Prod &P, int chunk, bool active, float *xv,
                                             float &xsv) {
  if (active) {
    const float4 *xp = reinterpret_cast<const float4 *>(P.x + 32 * chunk);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float4 v = xp[k];
      xv[4 * k + 0] = v.x;
      xv[4 * k + 1] = v.y;
      xv[4 * k + 2] = v.z;
      xv[4 * k + 3] = v.w;
    }
    xsv = P.xs[chunk >> 1];
  } else {
#pragma unroll
    for (int k = 0; k < 32; ++k) xv[k] = 0.0f;
    xsv = 0.0f;
  }
}

// Rows of at most 32 groups.  A wave holds 64/LPR row segments of LPR lanes;
// lane `chunk` of a segment owns columns [32 chunk, 32 chunk + 32) and keeps
// their activations in registers for every row it visits.  Each wave
// iteration covers R row slots (R x 64/LPR rows) whose codes are loaded with
// one 16-byte load per lane and slot before any arithmetic.
template <int LPR, int R, bool FAST>
__global__ __launch_bounds__(256) void q4mv_seg_kernel(ProdGroup grp) {
  Prod P;
  int lw = 0, nwg = 1;
  select_product(grp, P, lw, nwg);

  constexpr int RPW = kWave / LPR;
  constexpr int RB = R * RPW;
  const int G = P.cols >> 6;
  const int wpr = P.cols >> 3;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int waves_per_wg = blockDim.x / kWave;
  const int seg = lane / LPR;
  const int chunk = lane % LPR;
  const bool active = chunk < 2 * G;
  const int g = chunk >> 1;

  float xv[32];
  float xsv;
  load_x_chunk(P, chunk, active, xv, xsv);

  const int waves_total = nwg * waves_per_wg;
  for (int rb = lw * waves_per_wg + wave; rb * RB < P.rows; rb += waves_total) {
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
      tot[j] = segment_sum<LPR>(group_term<FAST>(cw[j], xv, sv[j], bv[j], xsv, active, chunk & 1));
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

// Rows wider than 32 groups: a workgroup of `passes` waves; wave p owns the
// 2048-column pass p of every row it visits (activations in registers).
// Each pass sum (a T over its 32 group slots) goes to LDS, and the first
// wave combines the pass sums of a row with a -0-padded balanced tree over
// PP = next power of two >= passes, which is T over the passes.
template <int PP, int R, bool FAST>
__global__ __launch_bounds__(1024) void q4mv_split_kernel(ProdGroup grp) {
  Prod P;
  int lw = 0, nwg = 1;
  select_product(grp, P, lw, nwg);

  const int G = P.cols >> 6;
  const int wpr = P.cols >> 3;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int passes = blockDim.x / kWave;
  const int chunk = wave * kWave + lane;
  const bool active = chunk < 2 * G;
  const int g = chunk >> 1;

  float xv[32];
  float xsv;
  load_x_chunk(P, chunk, active, xv, xsv);

  __shared__ float part[R][16];
  for (int rb = lw; rb * R < P.rows; rb += nwg) {
    u32x4 cw[R];
    float sv[R], bv[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int r = rb * R + j;
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
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const float tot =
          segment_sum<kWave>(group_term<FAST>(cw[j], xv, sv[j], bv[j], xsv, active, chunk & 1));
      if (lane == 0) part[j][wave] = tot;
    }
    __syncthreads();
    if (wave == 0 && lane < R) {
      const int r = rb * R + lane;
      float v[PP];
#pragma unroll
      for (int k = 0; k < PP; ++k) v[k] = k < passes ? part[lane][k] : kNegZero;
#pragma unroll
      for (int w = 1; w < PP; w *= 2)
#pragma unroll
        for (int i = 0; i < PP; i += 2 * w) v[i] = v[i] + v[i + w];
      if (r < P.rows) {
        float o = v[0];
        if (P.res) o = P.res[r] + o;
        P.y[r] = o;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// rmsq: one workgroup of NT = max(64, P/8) threads, P = next power of two
// >= n.  Thread t owns the contiguous slots [8t, 8t+8); slots >= n hold -0.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float tree8(const float *v) {
  return ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
}

__global__ __launch_bounds__(1024) void rmsq_kernel(const float *__restrict__ h,
                                                    const float *__restrict__ w, int n,
                                                    float eps, float *__restrict__ u,
                                                    float *__restrict__ us) {
  __shared__ float wave_sums[16];
  __shared__ float total;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = t / kWave;
  const int nw = blockDim.x / kWave;

  float hv[8], v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int i = 8 * t + k;
    hv[k] = i < n ? h[i] : 0.0f;
    v[k] = i < n ? hv[k] * hv[k] : kNegZero;
  }
  float s = tree8(v);
#pragma unroll
  for (int m = 1; m < kWave; m *= 2) s = s + __shfl_xor(s, m);
  if (lane == 0) wave_sums[wave] = s;
  __syncthreads();
  if (t == 0) {
    // balanced tree over the (power-of-two many) wave sums
    for (int m = 1; m < nw; m *= 2)
      for (int i = 0; i < nw; i += 2 * m) wave_sums[i] = wave_sums[i] + wave_sums[i + m];
    total = wave_sums[0];
  }
  __syncthreads();
  const float ms = total / (float)n;
  const float rho = 1.0f / sqrtf(ms + eps);

  float uv[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int i = 8 * t + k;
    const float hr = hv[k] * rho;
    uv[k] = i < n ? hr * w[i] : kNegZero;
    if (i < n) u[i] = uv[k];
  }
  // group sums: 8 threads per 64-value group
  float gsum = tree8(uv);
  gsum = gsum + __shfl_xor(gsum, 1);
  gsum = gsum + __shfl_xor(gsum, 2);
  gsum = gsum + __shfl_xor(gsum, 4);
  if ((t & 7) == 0 && 8 * t < n) us[t >> 3] = gsum;
}

// ---------------------------------------------------------------------------
// swq.  Fixed mode evaluates exp by the fixed binary64 method:
//   k = rint(t/ln2) (as t*INV_LN2), r = (t - k*LN2_HI) - k*LN2_LO,
//   p = sum_{j<=13} r^j/j! by fused Horner, E = ldexp(p, k);
//   E = +inf for t >= 710, +0 for t <= -746.
// INV_LN2 = RN64(1/ln 2); LN2_HI = ln 2 truncated to 32 significant bits;
// LN2_LO = RN64(ln 2 - LN2_HI); 1/j! correctly rounded.
// ---------------------------------------------------------------------------
__device__ double fixed_exp(double t) {
  if (t != t) return t;
  if (t >= 710.0) return __builtin_inf();
  if (t <= -746.0) return 0.0;
  const double inv_ln2 = 0x1.71547652b82fep+0;
  const double ln2_hi = 0x1.62e42fee00000p-1;
  const double ln2_lo = 0x1.a39ef35793c76p-33;
  const double k = rint(t * inv_ln2);
  const double hi = t - k * ln2_hi;
  const double lo = k * ln2_lo;
  const double r = hi - lo;
  double p = 1.0 / 6227020800.0;  // 1/13!
  p = fma(p, r, 1.0 / 479001600.0);
  p = fma(p, r, 1.0 / 39916800.0);
  p = fma(p, r, 1.0 / 3628800.0);
  p = fma(p, r, 1.0 / 362880.0);
  p = fma(p, r, 1.0 / 40320.0);
  p = fma(p, r, 1.0 / 5040.0);
  p = fma(p, r, 1.0 / 720.0);
  p = fma(p, r, 1.0 / 120.0);
  p = fma(p, r, 1.0 / 24.0);
  p = fma(p, r, 1.0 / 6.0);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  return ldexp(p, (int)k);
}

// One wave per 64-value group: lane i computes o[64g+i], then a butterfly
// gives the group's balanced tree.
template <bool FAST>
__global__ __launch_bounds__(256) void swq_kernel(const float *__restrict__ a, int n,
                                                  float *__restrict__ o,
                                                  float *__restrict__ os) {
  const int g = (blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (g >= n / 64) return;  // uniform per wave
  const int i = 64 * g + lane;
  float ov;
  if constexpr (!FAST) {
    const double gate = (double)a[i];
    const double up = (double)a[n + i];
    const double sig = gate / (1.0 + fixed_exp(-gate));
    ov = (float)(sig * up);
  } else {
    const float gate = a[i];
    ov = gate / (1.0f + __expf(-gate)) * a[n + i];
  }
  o[i] = ov;
  float s = ov;
#pragma unroll
  for (int m = 1; m < kWave; m *= 2) s = s + __shfl_xor(s, m);
  if (lane == 0) os[g] = s;
}

// ---------------------------------------------------------------------------
// argmax: 64-bit keys ordered by (value, -index); NaN maps to the largest
// key.  Phase 1: one key per workgroup slice; phase 2: one workgroup.
// ---------------------------------------------------------------------------
constexpr int kArgmaxMaxBlocks = 1024;
constexpr unsigned long long kNanKey = ~0ull;

__device__ __forceinline__ unsigned long long argmax_key(float v, int i) {
  if (v != v) return kNanKey;
  uint32_t u = __float_as_uint(v);
  if (v == 0.0f) u = 0u;  // -0 and +0 compare equal
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (unsigned long long)(~(uint32_t)i);
}

__device__ __forceinline__ unsigned long long block_max_key(unsigned long long k) {
  __shared__ unsigned long long wk[16];
#pragma unroll
  for (int m = 1; m < kWave; m *= 2) {
    const unsigned long long o = __shfl_xor(k, m);
    k = o > k ? o : k;
  }
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) wk[wave] = k;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < (int)(blockDim.x / kWave); ++i) k = wk[i] > k ? wk[i] : k;
  }
  return k;  // valid in thread 0
}

__global__ __launch_bounds__(256) void argmax_partial_kernel(const float *__restrict__ v, int n,
                                                             int per_block,
                                                             unsigned long long *__restrict__ ws) {
  const int lo = blockIdx.x * per_block;
  const int hi = min(n, lo + per_block);
  unsigned long long k = 0ull;
  for (int i = lo + threadIdx.x; i < hi; i += blockDim.x) {
    const unsigned long long c = argmax_key(v[i], i);
    k = c > k ? c : k;
  }
  k = block_max_key(k);
  if (threadIdx.x == 0) ws[blockIdx.x] = k;
}

__global__ __launch_bounds__(256) void argmax_final_kernel(const unsigned long long *__restrict__ ws,
                                                           int nb, int32_t *__restrict__ idx) {
  unsigned long long k = 0ull;
  for (int i = threadIdx.x; i < nb; i += blockDim.x) k = ws[i] > k ? ws[i] : k;
  k = block_max_key(k);
  if (threadIdx.x == 0) *idx = (k == kNanKey) ? -1 : (int32_t)(~(uint32_t)(k & 0xFFFFFFFFull));
}

// ---------------------------------------------------------------------------
// embed: e[c] = (s[t, c/64] * q(t, c)) + b[t, c/64], t read on the device.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void embed_kernel(Prod w, const int32_t *__restrict__ tok,
                                                    float *__restrict__ e) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= w.cols) return;
  const int t = *tok;
  if (t < 0 || t >= w.rows) {
    e[c] = __builtin_nanf("");
    return;
  }
  const int G = w.cols >> 6;
  const uint32_t word = w.q[(size_t)t * (w.cols >> 3) + (c >> 3)];
  const float code = (float)((word >> (4 * (c & 7))) & 15u);
  const float sq = w.s[(size_t)t * G + (c >> 6)] * code;
  e[c] = sq + w.b[(size_t)t * G + (c >> 6)];
}

int next_pow2(int v) {
  int p = 1;
  while (p < v) p *= 2;
  return p;
}

constexpr int kSegR = 4;
constexpr int kSplitR = 4;
constexpr int kSegThreads = 256;
constexpr int kMaxWorkgroups = 1024;

template <bool FAST>
hipError_t launch_seg(const ProdGroup &g, int lpr, hipStream_t st) {
  const dim3 grid(g.wg_begin[g.n]), block(kSegThreads);
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
    case 2: hipLaunchKernelGGL((q4mv_split_kernel<2, kSplitR, FAST>), grid, block, 0, st, g); break;
    case 4: hipLaunchKernelGGL((q4mv_split_kernel<4, kSplitR, FAST>), grid, block, 0, st, g); break;
    case 8: hipLaunchKernelGGL((q4mv_split_kernel<8, kSplitR, FAST>), grid, block, 0, st, g); break;
    case 16: hipLaunchKernelGGL((q4mv_split_kernel<16, kSplitR, FAST>), grid, block, 0, st, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

Shape shape_of(int32_t cols) {
  const int G = cols / 64;
  if (G <= 32) {
    int lpr = next_pow2(2 * G);
    return Shape{lpr < 2 ? 2 : lpr, 0};
  }
  return Shape{0, (G + 31) / 32};
}

int32_t workgroups_for(const Shape &sh, int32_t rows) {
  long long need;
  if (sh.lpr) {
    const long long rows_per_wg = (long long)(kSegThreads / kWave) * kSegR * (kWave / sh.lpr);
    need = (rows + rows_per_wg - 1) / rows_per_wg;
  } else {
    need = (rows + kSplitR - 1) / kSplitR;
  }
  if (need < 1) need = 1;
  return (int32_t)(need < kMaxWorkgroups ? need : kMaxWorkgroups);
}

hipError_t launch_q4mv_group(const ProdGroup &g, const Shape &sh, int mode, hipStream_t st) {
  const bool fast = mode != 0;
  if (sh.lpr) return fast ? launch_seg<true>(g, sh.lpr, st) : launch_seg<false>(g, sh.lpr, st);
  return fast ? launch_split<true>(g, sh.passes, st) : launch_split<false>(g, sh.passes, st);
}

hipError_t launch_rmsq(const float *h, const float *w, int32_t n, float eps, float *u, float *us,
                       hipStream_t st) {
  int threads = next_pow2(n) / 8;
  if (threads < kWave) threads = kWave;
  hipLaunchKernelGGL(rmsq_kernel, dim3(1), dim3(threads), 0, st, h, w, n, eps, u, us);
  return hipGetLastError();
}

hipError_t launch_swq(const float *a, int32_t n, float *o, float *os, int mode, hipStream_t st) {
  const int groups = n / 64;
  const int blocks = (groups * kWave + 255) / 256;
  if (mode)
    hipLaunchKernelGGL(swq_kernel<true>, dim3(blocks), dim3(256), 0, st, a, n, o, os);
  else
    hipLaunchKernelGGL(swq_kernel<false>, dim3(blocks), dim3(256), 0, st, a, n, o, os);
  return hipGetLastError();
}

static int argmax_blocks(int32_t n) {
  int nb = (n + 2047) / 2048;
  if (nb < 1) nb = 1;
  return nb < kArgmaxMaxBlocks ? nb : kArgmaxMaxBlocks;
}

size_t argmax_ws_bytes(int32_t n) { return sizeof(unsigned long long) * (size_t)argmax_blocks(n); }

hipError_t launch_argmax(const float *v, int32_t n, int32_t *idx, void *ws, hipStream_t st) {
  const int nb = argmax_blocks(n);
  const int per_block = (n + nb - 1) / nb;
  auto *keys = static_cast<unsigned long long *>(ws);
  hipLaunchKernelGGL(argmax_partial_kernel, dim3(nb), dim3(256), 0, st, v, n, per_block, keys);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(argmax_final_kernel, dim3(1), dim3(256), 0, st, keys, nb, idx);
  return hipGetLastError();
}

hipError_t launch_embed(const Prod &w, const int32_t *tok, float *e, hipStream_t st) {
  hipLaunchKernelGGL(embed_kernel, dim3((w.cols + 255) / 256), dim3(256), 0, st, w, tok, e);
  return hipGetLastError();
}

}  // namespace q4
