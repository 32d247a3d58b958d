// Gated attention of one decode token over key/value caches (atq), for
// gfx950: "Metal: queued rmsq, swq, gdn and atq kernels and a 4-row q4mv, so
// a decode token is one command buffer with one wait" (#1440), Change (atq
// bullet: q/k RMS norm and rotation, the new key and value into the caches,
// scores, softmax, weighted values, sigmoid gate, group sums; a group of
// query heads shares one key/value head).  The pages give no formulas; the
// arithmetic read from them, operation by operation (D = 128, G = hq / hkv
// query heads per key/value head j, n = pos + 1 positions):
//   qn = rmsq(q_h, wq), kn = rmsq(k_j, wk) over D values
//   rotation of x by the position's table (c_i, s_i), i < D/2, pairing i
//   with i + D/2:  r_i = (x_i c_i) - (x_{i+64} s_i),
//                  r_{i+64} = (x_i s_i) + (x_{i+64} c_i)
//   K[j][pos] = rotated kn, V[j][pos] = v_j
//   s_t = T(qr_i K[j][t]_i over i) * RN32(1/sqrt(D))
//   e_t = RN32(E(s_t - max s)), the difference in binary32, E the fixed
//         binary64 exp
//   o_i = (T(e_t V[j][t]_i over t) / T(e over t)) * RN32(1 / (1 + E(-g_i)))
//   osum = T over each 64 values of o
// with T the canonical tree (the balanced tree over the next power of two
// with -0 in the empty slots).  Compiled with -ffp-contract=off.
//
// The position is read from device memory (a captured graph replays the
// same launches token after token), with the rotation table's row of that
// position.
//
// Layout of the work (MI355X-first rather than one workgroup per query
// head): the positions are cut into aligned chunks of 64, and a grid of
// (chunks of the whole cache x key/value heads) workgroups runs twice; the
// workgroups past the position leave at once.
//   scores kernel:  each workgroup normalises and rotates the G queries of
//     its head group (and, in the chunk holding pos, the new key, which it
//     writes to the caches with the new value), reads each key row of its
//     chunk once for all G queries, and writes the scores and each query's
//     chunk maximum.
//   weights kernel: each workgroup takes the largest score from the chunk
//     maxima, forms its chunk's weights, the chunk's sum of weights and of
//     weighted value rows (each value row read once for all G queries), and
//     writes them; the last workgroup of the head group to arrive (a device
//     counter, no waiting) adds up the chunks and applies the gate.
// A chunk of 64 aligned positions is a subtree of the canonical tree over
// the n positions, and the chunks' tree (64 slots, -0 in the unused ones)
// is the rest of it: every sum has the bits of T over the n terms.
#include <math.h>

#include "ops_device.h"
#include "q4mv_internal.h"

#pragma clang fp contract(off)

namespace q4 {
namespace {

using namespace ops;

constexpr int kD = kAtqD;
constexpr int kC = kAtqChunk;
constexpr int kMaxG = kAtqMaxGroup;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr float kScale = 0x1.6a09e6p-4f;  // RN32(1 / sqrt(128))

// Sum over the 16 lanes of an aligned 16-lane group, as the balanced tree
// over the lanes' values in lane order (every lane gets it).
__device__ __forceinline__ float sum16(float s) {
#pragma unroll
  for (int m = 1; m < 16; m *= 2) s = s + __shfl_xor(s, m);
  return s;
}

__device__ __forceinline__ float sum64(float s) {
#pragma unroll
  for (int m = 1; m < kWave; m *= 2) s = s + __shfl_xor(s, m);
  return s;
}

__device__ __forceinline__ float max64(float s) {
#pragma unroll
  for (int m = 1; m < kWave; m *= 2) s = fmaxf(s, __shfl_xor(s, m));
  return s;
}

__device__ __forceinline__ void load8(const float *p, float *v) {
  const float4 a = reinterpret_cast<const float4 *>(p)[0];
  const float4 b = reinterpret_cast<const float4 *>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__global__ __launch_bounds__(kThreads) void atq_scores_kernel(AtqArgs a) {
  __shared__ float un[kMaxG + 1][kD];   // normed rows (queries, then the new key)
  __shared__ float rot[kMaxG + 1][kD];  // rotated rows
  __shared__ float wmax[kWaves][kMaxG];
  const int t = threadIdx.x;
  const int c = blockIdx.x;  // chunk of positions
  const int j = blockIdx.y;  // key/value head
  const int G = a.hq / a.hkv;
  // the weights kernel's arrival counter of this head group starts at zero
  if (c == 0 && t == 0) a.cnt[j] = 0u;
  const int pos = *a.pos;
  // outside the cache (the weights kernel then writes NaN) or past the
  // position: nothing to do
  if (pos < 0 || pos >= a.max_pos || c > pos / kC) return;
  const int n = pos + 1;
  const bool owns_pos = c == pos / kC;
  const float *cs = a.cs + (size_t)pos * (kD / 2);
  const float *sn = a.sn + (size_t)pos * (kD / 2);

  // 16 lanes per row, 8 values per lane: rows r < G are the queries of
  // heads j*G + r; row G is the new key, in the workgroup owning pos only
  const int r = t >> 4, l = t & 15;
  const bool active = r < G || (r == G && owns_pos);
  // every global load up front, so that their latencies overlap: this
  // lane's slice of its row and norm weights, of the rotation table, and
  // of the key rows of its four positions (16 positions per pass)
  float xv[8], wv[8], ct[8], st[8];
  float kv[kC / 16][8];
  if (active) {
    const float *x = r < G ? a.q + (size_t)(j * G + r) * kD : a.k + (size_t)j * kD;
    const float *w = r < G ? a.wq : a.wk;
    load8(x + 8 * l, xv);
    load8(w + 8 * l, wv);
    const int i0 = 8 * (l & 7);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      ct[k] = cs[i0 + k];
      st[k] = sn[i0 + k];
    }
  }
#pragma unroll
  for (int pass = 0; pass < kC / 16; ++pass) {
    const int tp = c * kC + 16 * pass + r;
    if (tp < n && tp != pos) load8(a.kc + ((size_t)j * a.max_pos + tp) * kD + 8 * l, kv[pass]);
  }
  if (active) {
    float sq[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) sq[k] = xv[k] * xv[k];
    const float rho = rmsq_rho_from_ss(sum16(tree8(sq)), kD, a.eps);
#pragma unroll
    for (int k = 0; k < 8; ++k) un[r][8 * l + k] = rmsq_value(xv[k], rho, wv[k]);
  }
  __syncthreads();
  if (active) {
    float rv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = 8 * l + k;
      if (l < 8) {  // i < 64: the first of the pair
        const float A = un[r][i], B = un[r][i + kD / 2];
        const float ac = A * ct[k], bs = B * st[k];
        rv[k] = ac - bs;
      } else {
        const int i2 = i - kD / 2;
        const float A = un[r][i2], B = un[r][i];
        const float as = A * st[k], bc = B * ct[k];
        rv[k] = as + bc;
      }
      rot[r][i] = rv[k];
    }
    if (r == G) {
      float *kd = a.kc + ((size_t)j * a.max_pos + pos) * kD + 8 * l;
      float *vd = a.vc + ((size_t)j * a.max_pos + pos) * kD + 8 * l;
      const float *vs = a.v + (size_t)j * kD + 8 * l;
      reinterpret_cast<float4 *>(kd)[0] = make_float4(rv[0], rv[1], rv[2], rv[3]);
      reinterpret_cast<float4 *>(kd)[1] = make_float4(rv[4], rv[5], rv[6], rv[7]);
      reinterpret_cast<float4 *>(vd)[0] = reinterpret_cast<const float4 *>(vs)[0];
      reinterpret_cast<float4 *>(vd)[1] = reinterpret_cast<const float4 *>(vs)[1];
    }
  }
  __syncthreads();

  // scores: 16 lanes per position, 16 positions per pass, 4 passes
  float qv[kMaxG][8];
  float mx[kMaxG];
#pragma unroll
  for (int gi = 0; gi < kMaxG; ++gi) {
    mx[gi] = -INFINITY;
    if (gi < G) {
#pragma unroll
      for (int k = 0; k < 8; ++k) qv[gi][k] = rot[gi][8 * l + k];
    }
  }
#pragma unroll
  for (int pass = 0; pass < kC / 16; ++pass) {
    const int tp = c * kC + 16 * pass + r;
    if (tp < n) {  // uniform over the 16 lanes of the position
      if (tp == pos) {
#pragma unroll
        for (int k = 0; k < 8; ++k) kv[pass][k] = rot[G][8 * l + k];
      }
#pragma unroll
      for (int gi = 0; gi < kMaxG; ++gi) {
        if (gi < G) {
          float pr[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) pr[k] = qv[gi][k] * kv[pass][k];
          const float s = sum16(tree8(pr)) * kScale;
          if (l == gi) a.sc[(size_t)(j * G + gi) * kAtqMaxPos + tp] = s;
          mx[gi] = fmaxf(mx[gi], s);
        }
      }
    }
  }
  const int lane = t & (kWave - 1), wave = t / kWave;
#pragma unroll
  for (int gi = 0; gi < kMaxG; ++gi) {
    if (gi < G) {
      float m = fmaxf(mx[gi], __shfl_xor(mx[gi], 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      if (lane == 0) wmax[wave][gi] = m;
    }
  }
  __syncthreads();
  if (t < G) {
    float m = wmax[0][t];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = fmaxf(m, wmax[w][t]);
    a.cmax[(size_t)(j * G + t) * kAtqMaxChunks + c] = m;
  }
}

__global__ __launch_bounds__(kThreads) void atq_weights_kernel(AtqArgs a) {
  __shared__ float eS[kMaxG][kC];
  __shared__ float part[kMaxG][kD];
  __shared__ float zS[kMaxG];
  __shared__ int last;
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int c = blockIdx.x, j = blockIdx.y;
  const int G = a.hq / a.hkv;
  const int pos = *a.pos;
  if (pos < 0 || pos >= a.max_pos) {  // no such cache row: o and osum are NaN
    if (c == 0) {
      for (int idx = t; idx < G * kD; idx += kThreads) a.o[(size_t)j * G * kD + idx] = NAN;
      if (t < 2 * G) a.os[(size_t)j * G * 2 + t] = NAN;
    }
    return;
  }
  if (c > pos / kC) return;
  const int n = pos + 1;
  const int nchunk = pos / kC + 1;
  const int i = t & (kD - 1), half = t / kD;
  const int p0 = c * kC + 32 * half;
  const int tp = c * kC + lane;

  // every global load up front: this thread's column of 32 value rows
  // (thread = column i, half of the chunk), and per query of this wave
  // the chunk maxima and the score of position tp
  float vv[32];
#pragma unroll
  for (int k = 0; k < 32; ++k)
    vv[k] = p0 + k < n ? a.vc[((size_t)j * a.max_pos + p0 + k) * kD + i] : 0.0f;
  constexpr int kPerWave = kMaxG / kWaves;
  float cm[kPerWave], sv[kPerWave];
#pragma unroll
  for (int u = 0; u < kPerWave; ++u) {
    const int gi = wave + kWaves * u;
    cm[u] = -INFINITY;
    sv[u] = 0.0f;
    if (gi < G) {
      if (lane < nchunk) cm[u] = a.cmax[(size_t)(j * G + gi) * kAtqMaxChunks + lane];
      if (tp < n) sv[u] = a.sc[(size_t)(j * G + gi) * kAtqMaxPos + tp];
    }
  }
  // the chunk's weights e (lane = position) from the largest score, and
  // their sum
#pragma unroll
  for (int u = 0; u < kPerWave; ++u) {
    const int gi = wave + kWaves * u;
    if (gi < G) {  // uniform per wave
      const float m = max64(cm[u]);
      float e = kNegZero;
      if (tp < n) {
        const float d = sv[u] - m;
        e = (float)fixed_exp((double)d);
      }
      eS[gi][lane] = e;
      const float z = sum64(e);
      if (lane == 0) a.zp[(size_t)(j * G + gi) * kAtqMaxChunks + c] = z;
    }
  }
  __syncthreads();
  // the chunk's weighted value sums
  float own[kMaxG];
#pragma unroll
  for (int gi = 0; gi < kMaxG; ++gi) {
    own[gi] = 0.0f;
    if (gi < G) {
      float pr[32];
#pragma unroll
      for (int k = 0; k < 32; ++k) pr[k] = p0 + k < n ? eS[gi][32 * half + k] * vv[k] : kNegZero;
      own[gi] = (tree8(pr) + tree8(pr + 8)) + (tree8(pr + 16) + tree8(pr + 24));
      if (half == 1) part[gi][i] = own[gi];
    }
  }
  __syncthreads();
  if (half == 0) {
#pragma unroll
    for (int gi = 0; gi < kMaxG; ++gi)
      if (gi < G)
        a.wp[((size_t)(j * G + gi) * kAtqMaxChunks + c) * kD + i] = own[gi] + part[gi][i];
  }

  // the last workgroup of the head group to arrive adds up the chunks
  __threadfence();
  __syncthreads();
  if (t == 0)
    last = __hip_atomic_fetch_add(a.cnt + j, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
           (uint32_t)(nchunk - 1);
  __syncthreads();
  if (!last) return;
  __threadfence();
  for (int gi = wave; gi < G; gi += kWaves) {
    const float z = lane < nchunk ? a.zp[(size_t)(j * G + gi) * kAtqMaxChunks + lane] : kNegZero;
    const float zz = sum64(z);
    if (lane == 0) zS[gi] = zz;
  }
  __syncthreads();
  for (int idx = t; idx < G * kD; idx += kThreads) {  // uniform per wave
    const int gi = idx / kD, ii = idx & (kD - 1);
    const size_t hrow = (size_t)(j * G + gi);
    const float *wp = a.wp + hrow * kAtqMaxChunks * kD + ii;
    float blk[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      float v8[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int cc = 8 * b + k;
        v8[k] = cc < nchunk ? wp[(size_t)cc * kD] : kNegZero;
      }
      blk[b] = tree8(v8);
    }
    const float w = tree8(blk) / zS[gi];
    const double gv = (double)a.g[hrow * kD + ii];
    const float sig = (float)(1.0 / (1.0 + fixed_exp(-gv)));
    const float ov = w * sig;
    a.o[hrow * kD + ii] = ov;
    const float s = sum64(ov);
    if (lane == 0) a.os[hrow * 2 + ii / 64] = s;
  }
}

}  // namespace

void atq_ws_layout(int32_t hq, int32_t hkv, AtqWs *out) {
  size_t at = 0;
  auto take = [&at](size_t bytes) {
    const size_t p = at;
    at += (bytes + 255) & ~(size_t)255;
    return p;
  };
  out->sc = take(sizeof(float) * (size_t)hq * kAtqMaxPos);
  out->cmax = take(sizeof(float) * (size_t)hq * kAtqMaxChunks);
  out->zp = take(sizeof(float) * (size_t)hq * kAtqMaxChunks);
  out->wp = take(sizeof(float) * (size_t)hq * kAtqMaxChunks * kAtqD);
  out->cnt = take(sizeof(uint32_t) * (size_t)hkv);
  out->bytes = at;
}

hipError_t launch_atq(const AtqArgs &a, hipStream_t st) {
  // one workgroup per chunk of the whole cache: the position is read on the
  // device, and the workgroups past it leave at once
  const dim3 grid((a.max_pos + kAtqChunk - 1) / kAtqChunk, a.hkv);
  hipLaunchKernelGGL(atq_scores_kernel, grid, dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(atq_weights_kernel, grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace q4
