// Device building blocks shared by the standalone producer kernels and the
// fused q4mv prologues/epilogues: the same code runs in both, so a fused
// stage produces the bits of the separate one.
//
// rmsq and swq follow "Metal: queued rmsq, swq, gdn and atq kernels and a
// 4-row q4mv, so a decode token is one command buffer with one wait"
// (#1440), Change (rmsq and swq bullets); greedy argmax its Verification
// (greedy token ids).  Compiled with -ffp-contract=off.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#pragma clang fp contract(off)

namespace q4 {
namespace ops {

constexpr int kWave = 64;
constexpr float kNegZero = -0.0f;

__device__ __forceinline__ float tree8(const float *v) {
  return ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
}

// Lane butterflies with DPP and the gfx950 lane swaps instead of shuffles
// routed through LDS (a ds_bpermute each, whose latency sits on the
// critical path of every reduction).  Steps: xor 1 and xor 2 within quads;
// then, once every aligned block of 4 (8) lanes holds one value, the mirror
// within 8 (16) lanes pairs the same blocks as xor 4 (8); then the 16- and
// 32-lane swaps pair 16-lane rows 0/1, 2/3 and then halves 0/1, as xor 16
// and xor 32 do.  Each step adds the same two operands as the xor
// butterfly (in the other order in half the lanes, which IEEE addition does
// not see), so the result is the balanced tree over the lanes, in every
// lane.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned block of 8 lanes.
__device__ __forceinline__ float lane_sum8(float s) {
  s = s + dpp_move<0xB1>(s);   // quad_perm [1,0,3,2]: xor 1
  s = s + dpp_move<0x4E>(s);   // quad_perm [2,3,0,1]: xor 2
  return s + dpp_move<0x141>(s);  // row_half_mirror: xor 4 here
}

// Sum of the two 32-lane halves (xor 32), in every lane.
__device__ __forceinline__ float half_sum32(float s) {
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false,
                                                  false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Largest of the 64 lanes (fmaxf: any order gives the same value).
__device__ __forceinline__ float lane_max64(float s) {
  s = fmaxf(s, dpp_move<0xB1>(s));
  s = fmaxf(s, dpp_move<0x4E>(s));
  s = fmaxf(s, dpp_move<0x141>(s));
  s = fmaxf(s, dpp_move<0x140>(s));
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false,
                                                  false);
  s = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false,
                                                  false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// 64-bit (value, index) keys: the largest over lanes, by the same steps on
// the two 32-bit halves (a maximum, so the order of the steps does not
// matter).
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_move_key(unsigned long long v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((unsigned long long)hi << 32) | lo;
}

__device__ __forceinline__ unsigned long long key_max(unsigned long long a, unsigned long long b) {
  return a > b ? a : b;
}

// The larger key of lanes i and i ^ 16, then of i and i ^ 32, in every lane.
__device__ __forceinline__ unsigned long long key_max_rows(unsigned long long k) {
  auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)k, (uint32_t)k, false, false);
  auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(k >> 32), (uint32_t)(k >> 32), false, false);
  k = key_max(((unsigned long long)hi[0] << 32) | lo[0], ((unsigned long long)hi[1] << 32) | lo[1]);
  lo = __builtin_amdgcn_permlane32_swap((uint32_t)k, (uint32_t)k, false, false);
  hi = __builtin_amdgcn_permlane32_swap((uint32_t)(k >> 32), (uint32_t)(k >> 32), false, false);
  return key_max(((unsigned long long)hi[0] << 32) | lo[0], ((unsigned long long)hi[1] << 32) | lo[1]);
}

// The largest key of the 64 lanes, in every lane.
__device__ __forceinline__ unsigned long long lane_key_max64(unsigned long long k) {
  k = key_max(k, dpp_move_key<0xB1>(k));
  k = key_max(k, dpp_move_key<0x4E>(k));
  k = key_max(k, dpp_move_key<0x141>(k));
  k = key_max(k, dpp_move_key<0x140>(k));
  return key_max_rows(k);
}

// Sum over the 64 lanes of the wave.
__device__ __forceinline__ float lane_sum64(float s) {
  s = lane_sum8(s);
  s = s + dpp_move<0x140>(s);  // row_mirror: xor 8 here
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false,
                                                  false);
  s = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false,
                                                  false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// RMS norm of n values with weights, plus group sums, by one workgroup of
// blockDim.x = max(64, P/8) threads (P = next power of two >= n, n % 64 ==
// 0, at most 1024 threads).  Thread t owns the contiguous slots [8t, 8t+8);
// slots >= n hold -0.0, so the lane and wave butterflies give the canonical
// tree over the n squares:
//   ss = T(h*h); ms = ss / n; rho = 1 / sqrt(ms + eps)  (correctly rounded);
//   u_i = (h_i * rho) * w_i; us_g = T(u[64g .. 64g+63]).

// rho from the sum of squares ss of the n values.
__device__ __forceinline__ float rmsq_rho_from_ss(float ss, int n, float eps) {
  const float ms = ss / (float)n;
  return 1.0f / sqrtf(ms + eps);
}

// The first half: rho, in every thread, from the thread's 8 slots of h
// already in registers (hv; slots >= n must hold 0).  red is LDS scratch of
// 17 floats; every thread of the workgroup must call it (two barriers).
__device__ __forceinline__ float rmsq_rho_regs(const float *hv, int n, float eps, float *red) {
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = t / kWave;
  const int nw = blockDim.x / kWave;
  float v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = 8 * t + k < n ? hv[k] * hv[k] : kNegZero;
  const float s = lane_sum64(tree8(v));
  if (lane == 0) red[wave] = s;
  __syncthreads();
  if (t == 0) {
    // balanced tree over the (power-of-two many) wave sums
    for (int m = 1; m < nw; m *= 2)
      for (int i = 0; i < nw; i += 2 * m) red[i] = red[i] + red[i + m];
    red[16] = red[0];
  }
  __syncthreads();
  return rmsq_rho_from_ss(red[16], n, eps);
}

// The same, loading the thread's 8 slots of h and of w together up front
// (hv, wv) so that their latencies overlap.
__device__ __forceinline__ float rmsq_rho(const float *__restrict__ h,
                                          const float *__restrict__ w, int n, float eps,
                                          float *red, float *hv, float *wv) {
  const int t = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int i = 8 * t + k;
    hv[k] = i < n ? h[i] : 0.0f;
    wv[k] = i < n ? w[i] : 0.0f;
  }
  return rmsq_rho_regs(hv, n, eps, red);
}

// rho of 2048 values by one wave without LDS: lane l holds values
// [32 l, 32 l + 32) in hv.  The same tree as rmsq_rho_regs (the balanced
// tree over the 2048 squares in index order), so the same bits.
__device__ __forceinline__ float rmsq_rho_wave2048(const float *hv, float eps) {
  float sq[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) sq[k] = hv[k] * hv[k];
  const float s = lane_sum64((tree8(sq) + tree8(sq + 8)) + (tree8(sq + 16) + tree8(sq + 24)));
  return rmsq_rho_from_ss(s, 2048, eps);
}

// One normalised value: (h * rho) * w.
__device__ __forceinline__ float rmsq_value(float h, float rho, float w) {
  const float hr = h * rho;
  return hr * w;
}

// The second half: u for the thread's 8 slots and the group sums (8
// threads per group), stored at u[i + PAD * (i / 32)] (PAD = 0: plain; 4:
// the padded LDS layout whose 32-value runs start on distinct banks).  u and
// us may point to global or LDS memory.
template <int PAD>
__device__ __forceinline__ void rmsq_u(int n, float rho, const float *hv, const float *wv,
                                       float *u, float *us) {
  const int t = threadIdx.x;
  float uv[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int i = 8 * t + k;
    uv[k] = i < n ? rmsq_value(hv[k], rho, wv[k]) : kNegZero;
    if (i < n) u[i + (i >> 5) * PAD] = uv[k];
  }
  const float gsum = lane_sum8(tree8(uv));
  if ((t & 7) == 0 && 8 * t < n) us[t >> 3] = gsum;
}

__device__ __forceinline__ void rmsq_block(const float *__restrict__ h,
                                           const float *__restrict__ w, int n, float eps,
                                           float *u, float *us, float *red) {
  float hv[8], wv[8];
  const float rho = rmsq_rho(h, w, n, eps, red, hv, wv);
  rmsq_u<0>(n, rho, hv, wv, u, us);
}

// exp in binary64 by a fixed method (every implementation that follows the
// same steps gets the same bits):
//   k = rint(t * INV_LN2); r = (t - k*LN2_HI) - k*LN2_LO;
//   p = sum_{j<=13} r^j / j! by fused Horner; E = ldexp(p, k);
//   E = +inf for t >= 710, +0 for t <= -746, NaN for NaN.
// INV_LN2 = RN64(1/ln 2); LN2_HI = ln 2 truncated to 32 significant bits;
// LN2_LO = RN64(ln 2 - LN2_HI); 1/j! correctly rounded.
__device__ __forceinline__ double fixed_exp(double t) {
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

// One SwiGLU output.  Fixed: silu in binary64, a / (1 + E(-a)), times up in
// binary64, rounded once to binary32.  Fast: binary32 with the hardware exp.
template <bool FAST>
__device__ __forceinline__ float swiglu_value(float gate, float up) {
  if constexpr (!FAST) {
    const double g = (double)gate;
    const double sig = g / (1.0 + fixed_exp(-g));
    return (float)(sig * (double)up);
  } else {
    return gate / (1.0f + __expf(-gate)) * up;
  }
}

// 64-bit key ordered by (value, -index): the largest key is the lowest index
// of the largest value; -0 and +0 compare equal; NaN maps to the largest key.
constexpr unsigned long long kNanKey = ~0ull;

__device__ __forceinline__ unsigned long long argmax_key(float v, int i) {
  if (v != v) return kNanKey;
  uint32_t u = __float_as_uint(v);
  if (v == 0.0f) u = 0u;
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (unsigned long long)(~(uint32_t)i);
}

__device__ __forceinline__ int32_t argmax_index(unsigned long long key) {
  return key == kNanKey ? -1 : (int32_t)(~(uint32_t)(key & 0xFFFFFFFFull));
}

}  // namespace ops
}  // namespace q4
