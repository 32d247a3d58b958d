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

#include "ops_device.h"
#include "q4mv_internal.h"

#pragma clang fp contract(off)

namespace q4 {
namespace {

using namespace ops;

// rmsq: one workgroup of NT = max(64, P/8) threads, P = next power of two
// >= n (the body is ops::rmsq_block).
__global__ __launch_bounds__(1024) void rmsq_kernel(const float *__restrict__ h,
                                                    const float *__restrict__ w, int n,
                                                    float eps, float *__restrict__ u,
                                                    float *__restrict__ us) {
  __shared__ float red[17];
  rmsq_block(h, w, n, eps, u, us, red);
}

// rmsq for n = 2048 by one wave, without LDS or barriers: lane l holds
// values [32 l, 32 l + 32) of h and w.  The same trees as rmsq_block (the
// balanced tree over the 2048 squares; per group, the balanced tree over
// its 64 values: the lane's 32, then its partner's), so the same bits.
__global__ __launch_bounds__(64) void rmsq2048_wave_kernel(const float *__restrict__ h,
                                                           const float *__restrict__ w, float eps,
                                                           float *__restrict__ u,
                                                           float *__restrict__ us) {
  const int lane = threadIdx.x;
  const float4 *hp = reinterpret_cast<const float4 *>(h) + 8 * lane;
  const float4 *wp = reinterpret_cast<const float4 *>(w) + 8 * lane;
  float hv[32], wv[32];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float4 a = hp[k], c = wp[k];
    hv[4 * k] = a.x, hv[4 * k + 1] = a.y, hv[4 * k + 2] = a.z, hv[4 * k + 3] = a.w;
    wv[4 * k] = c.x, wv[4 * k + 1] = c.y, wv[4 * k + 2] = c.z, wv[4 * k + 3] = c.w;
  }
  const float rho = rmsq_rho_wave2048(hv, eps);
  float uv[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) uv[k] = rmsq_value(hv[k], rho, wv[k]);
  float4 *up = reinterpret_cast<float4 *>(u) + 8 * lane;
#pragma unroll
  for (int k = 0; k < 8; ++k) up[k] = make_float4(uv[4 * k], uv[4 * k + 1], uv[4 * k + 2], uv[4 * k + 3]);
  const float half = (tree8(uv) + tree8(uv + 8)) + (tree8(uv + 16) + tree8(uv + 24));
  const float g = half + ops::dpp_move<0xB1>(half);  // xor 1
  if ((lane & 1) == 0) us[lane >> 1] = g;
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
  const float ov = swiglu_value<FAST>(a[i], a[n + i]);
  o[i] = ov;
  const float s = ops::lane_sum64(ov);
  if (lane == 0) os[g] = s;
}

// ---------------------------------------------------------------------------
// argmax: one key per workgroup slice, then one workgroup over the keys.
// ---------------------------------------------------------------------------
constexpr int kArgmaxMaxBlocks = 1024;

__device__ __forceinline__ unsigned long long block_max_key(unsigned long long k) {
  __shared__ unsigned long long wk[16];
  k = lane_key_max64(k);
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
  if (threadIdx.x == 0) *idx = argmax_index(k);
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

// ---------------------------------------------------------------------------
// mailbox: copies n int32 values into pinned host memory, then publishes the
// next sequence number there (one thread; system-scope release, so a host
// that reads the new number also reads the values).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void mailbox_kernel(const int32_t *__restrict__ vals, int n,
                                                     int32_t *host_vals, uint32_t *host_seq,
                                                     uint32_t *dev_count) {
  if (threadIdx.x != 0) return;
  for (int i = 0; i < n; ++i)
    __hip_atomic_store(host_vals + i, vals[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  const uint32_t seq = *dev_count + 1u;
  *dev_count = seq;
  __hip_atomic_store(host_seq, seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

// One thread: *pos += 1 (a decode chain's position, advanced inside its
// captured graph after the token's last attention step).
__global__ __launch_bounds__(64) void pos_advance_kernel(int32_t *pos) {
  if (threadIdx.x == 0) *pos = *pos + 1;
}

int next_pow2(int v) {
  int p = 1;
  while (p < v) p *= 2;
  return p;
}

}  // namespace

hipError_t launch_rmsq(const float *h, const float *w, int32_t n, float eps, float *u, float *us,
                       hipStream_t st) {
  // the one-wave kernel reads and writes 16 bytes at a time
  const bool aligned16 = ((reinterpret_cast<uintptr_t>(h) | reinterpret_cast<uintptr_t>(w) |
                           reinterpret_cast<uintptr_t>(u)) & 15u) == 0;
  if (n == 2048 && aligned16) {
    hipLaunchKernelGGL(rmsq2048_wave_kernel, dim3(1), dim3(kWave), 0, st, h, w, eps, u, us);
    return hipGetLastError();
  }
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

hipError_t launch_argmax_final(const unsigned long long *keys, int32_t nkeys, int32_t *idx,
                               hipStream_t st) {
  hipLaunchKernelGGL(argmax_final_kernel, dim3(1), dim3(256), 0, st, keys, nkeys, idx);
  return hipGetLastError();
}

hipError_t launch_mailbox(const int32_t *vals, int32_t n, int32_t *host_vals, uint32_t *host_seq,
                          uint32_t *dev_count, hipStream_t st) {
  hipLaunchKernelGGL(mailbox_kernel, dim3(1), dim3(64), 0, st, vals, n, host_vals, host_seq,
                     dev_count);
  return hipGetLastError();
}

hipError_t launch_pos_advance(int32_t *pos, hipStream_t st) {
  hipLaunchKernelGGL(pos_advance_kernel, dim3(1), dim3(64), 0, st, pos);
  return hipGetLastError();
}

hipError_t launch_embed(const Prod &w, const int32_t *tok, float *e, hipStream_t st) {
  hipLaunchKernelGGL(embed_kernel, dim3((w.cols + 255) / 256), dim3(256), 0, st, w, tok, e);
  return hipGetLastError();
}

}  // namespace q4
