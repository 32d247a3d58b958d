// HIP kernels for gfx950 (CDNA4, wave64): the producers of q4mv's inputs
// (rmsq, swq) and the greedy-decode glue (argmax, embed).  Compiled with
// -ffp-contract=off: every float expression is the exact sequence of IEEE
// binary32 / binary64 operations it spells; fused multiply-adds appear only
// where written out (fma / fmaf): the fixed binary64 exp and the Q4_FAST swq.
//
// rmsq and swq: "Metal: queued rmsq, swq, gdn and atq kernels and a 4-row
// q4mv, so a decode token is one command buffer with one wait" (#1440),
// Change (rmsq and swq bullets).  Group sums use the canonical tree (see
// q4mv_device.h).
#include <math.h>

#include "q4mv_internal.h"

#pragma clang fp contract(off)

namespace q4 {
namespace {

constexpr int kWave = 64;
constexpr float kNegZero = -0.0f;

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

}  // namespace

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
