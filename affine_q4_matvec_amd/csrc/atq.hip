// Gated attention of one decode token over key/value caches (atq), for
// gfx950: "Metal: queued rmsq, swq, gdn and atq kernels and a 4-row q4mv, so
// a decode token is one command buffer with one wait" (#1440), Change, atq
// bullet: the step normalises and rotates the query and the new key, appends
// the key and value to caches that stay on the GPU, weighs every cached
// position by a softmax of its score, gates the weighted sum with a sigmoid
// and emits the 64-value sums the next product needs; several query heads
// read one key/value head.  The pages give no formulas; the
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
// One launch of (spans of 256 positions of the whole cache) x (query
// heads) workgroups of 1024 threads; the position is read from device
// memory (a captured graph replays the same launch token after token), and
// the workgroups past it leave at once.  Workgroup (c, h) works on query
// head h over positions [256 c, 256 c + 256) (one workgroup per query head
// rather than per head group: a group's work on one compute unit made the
// arithmetic, not the loads, the bound; the G queries of a group read the
// same key and value rows, the later ones from the caches):
//   - every global load is issued first: its query, the new key and the
//     norm weights, the position's table row, and the key and value rows of
//     its span;
//   - norms and rotations into LDS; in the workgroup holding pos the new
//     key is formed (its own loads take the new rows from the inputs) and
//     the group's first query head writes the new cache rows;
//   - scores (16 lanes per position, DPP row sums), the span's largest
//     score;
//   - with more than one span, the span maxima are exchanged through tagged
//     device-scope words and each workgroup takes the largest;
//   - weights e and the span's sums T(e) and T(e V) (256 aligned positions:
//     a subtree of the canonical tree; each thread sums 8 positions of 4
//     value columns, the lanes 32 apart add neighbouring blocks, LDS the
//     16 blocks of 16);
//   - one span: the workgroup finishes o itself; more: the span sums are
//     published as tagged words and workgroup (0, h) polls them all at
//     once, adds them up in a 16-slot balanced tree (-0 in the unused
//     slots, the rest of the canonical tree) and applies the gate.
// At position 204 of a 4096 cache this is one busy workgroup per query
// head and no exchange at all; at 4095, 16 per head.  The exchanges follow
// the tagged-word protocol of tagged_device.h (no fences, no grid barrier):
// every workgroup publishes its maximum before it waits for any, so the
// waits of a head end once its (at most 16) workgroups are resident.
// Each workgroup counts its calls in a word of its own, which gives the
// call's tag.
#include <math.h>

#include "ops_device.h"
#include "q4mv_device.h"
#include "q4mv_internal.h"
#include "tagged_device.h"

#pragma clang fp contract(off)

namespace q4 {
namespace {

using ops::fixed_exp;
using ops::rmsq_rho_from_ss;
using ops::rmsq_value;
using ops::tree8;
using dev::dpp;
using dev::kDppQuadXor1;
using dev::kNegZero;
using dev::kWave;
using dev::segment_sum;

constexpr int kD = kAtqD;
constexpr int kSpan = kAtqSpan;
constexpr int kMaxSpans = kAtqMaxSpans;
constexpr int kThreads = 1024;
constexpr float kScale = 0x1.6a09e6p-4f;  // RN32(1 / sqrt(128))
static_assert(kMaxSpans == 16, "two tree8 levels over the spans");
static_assert(kSpan == 256, "4 passes of 64 positions; 32 blocks of 8");

// The balanced tree over the 16 lanes of an aligned 16-lane row, in lane
// order, in every lane of the row (xor 1 by quad permutation, then xor 2
// and the two mirrors).
__device__ __forceinline__ float sum16(float s) {
  s = s + dpp<kDppQuadXor1>(s);
  return segment_sum<16>(s);
}

__device__ __forceinline__ float sum64(float s) {
  s = s + dpp<kDppQuadXor1>(s);
  return segment_sum<64>(s);
}

__device__ __forceinline__ float max64(float s) { return ops::lane_max64(s); }

__device__ __forceinline__ void load8(const float *p, float *v) {
  const float4 a = reinterpret_cast<const float4 *>(p)[0];
  const float4 b = reinterpret_cast<const float4 *>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ float gate_value(float g) {
  return (float)(1.0 / (1.0 + fixed_exp(-(double)g)));
}


struct Lds {
  float un[2][kD];     // normed rows: the query, then the new key
  float rot[2][kD];    // rotated rows
  float s[kSpan];      // scores of the span
  float e[kSpan];      // weights of the span
  float part[16][kD];  // value sums over 16 positions
  float sw[kMaxSpans][kD];  // the spans' value sums (workgroup 0 of a head)
  float sz[kMaxSpans];      // the spans' weight sums
  float wsum[4];       // weight sums over 64 positions
  float m;             // largest score
  float z;             // the span's weight sum
};

__global__ __launch_bounds__(kThreads) void atq_kernel(AtqArgs a) {
  __shared__ Lds S;
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = dev::wave_index();
  const int c = blockIdx.x, h = blockIdx.y;
  const int G = a.hq / a.hkv, j = h / G;
  uint32_t *err = a.ctl + kAtqErrorWord;
  uint32_t *mine = a.ctl + h * kMaxSpans + c;
  // the control words and the position, loaded together
  const uint32_t e0 = load_word(err);
  const uint32_t tag = load_word(mine) + 1;
  const int pos = *a.pos;
  if (__syncthreads_or(e0 != 0)) return;
  const bool valid = pos >= 0 && pos < a.max_pos;
  const int nspan = valid ? pos / kSpan + 1 : 0;
  if (c >= nspan) {
    if (!valid && c == 0) {  // no such cache row: o and osum are NaN
      if (t < kD) a.o[(size_t)h * kD + t] = NAN;
      if (t < 2) a.os[(size_t)h * 2 + t] = NAN;
    }
    __syncthreads();
    if (t == 0) store_word(mine, tag);
    return;
  }
  const int n = pos + 1;
  const int base = c * kSpan;
  const bool owns_pos = pos / kSpan == c;
  // the new cache rows are written by the first query head of the group
  const bool writes_rows = owns_pos && h % G == 0;

  // ---- every global load first -------------------------------------------
  // row 0: the query of head h; row 1: the new key and value (workgroup
  // holding pos only); 16 lanes per row, 8 values per lane
  const int r = t >> 4, l = t & 15;
  const bool nrow = r == 0 || (r == 1 && owns_pos);
  float xv[8], wv[8], ct[8], st[8], nv[8];
  if (nrow) {
    const float *x = r == 0 ? a.q + (size_t)h * kD : a.k + (size_t)j * kD;
    load8(x + 8 * l, xv);
    load8((r == 0 ? a.wq : a.wk) + 8 * l, wv);
    load8(a.cs + (size_t)pos * (kD / 2) + 8 * (l & 7), ct);
    load8(a.sn + (size_t)pos * (kD / 2) + 8 * (l & 7), st);
    if (r == 1 && writes_rows) load8(a.v + (size_t)j * kD + 8 * l, nv);
  }
  // key rows: position base + 64 pass + r (r < 64), dims [8 l, 8 l + 8)
  float kv[kSpan / 64][8];
#pragma unroll
  for (int pass = 0; pass < kSpan / 64; ++pass) {
    const int tp = base + 64 * pass + r;
    if (tp < n && tp != pos) load8(a.kc + ((size_t)j * a.max_pos + tp) * kD + 8 * l, kv[pass]);
  }
  // value columns [4 cq, 4 cq + 4) of positions pb .. pb + 7 (the new row
  // from v)
  const int cq = t & 31, pg = t >> 5;
  const int pb = base + 8 * pg;
  float4 vv[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int p = pb + k;
    vv[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (p < n)
      vv[k] = reinterpret_cast<const float4 *>(
          p == pos ? a.v + (size_t)j * kD : a.vc + ((size_t)j * a.max_pos + p) * kD)[cq];
  }
  // the gate of output t (t < 128), needed by workgroup 0
  const bool out_t = t < kD;
  const float gv = c == 0 && out_t ? a.g[(size_t)h * kD + t] : 0.0f;

  // ---- norms and rotations -------------------------------------------------
  if (nrow) {
    float sq[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) sq[k] = xv[k] * xv[k];
    const float rho = rmsq_rho_from_ss(sum16(tree8(sq)), kD, a.eps);
#pragma unroll
    for (int k = 0; k < 8; ++k) S.un[r][8 * l + k] = rmsq_value(xv[k], rho, wv[k]);
  }
  // the same threads of wave 0 read S.un back: the wave's LDS accesses are
  // done in order, so a compiler barrier is enough
  asm volatile("" ::: "memory");
  if (nrow) {
    // value d < 64: A c - B s with A = un[d], B = un[d + 64]; value d >= 64:
    // A s + B c with A = un[d - 64], B = un[d]; as one expression, own c +
    // (-/+ partner s): the same products and sum, no branch
    const float *own = S.un[r] + 8 * l, *partner = S.un[r] + 8 * (l ^ 8);
    const bool first_half = l < 8;
    float rv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float pc = own[k] * ct[k], ps = partner[k] * st[k];
      rv[k] = pc + (first_half ? -ps : ps);
      S.rot[r][8 * l + k] = rv[k];
    }
    if (r == 1 && writes_rows) {  // the new cache rows
      float4 *kd = reinterpret_cast<float4 *>(a.kc + ((size_t)j * a.max_pos + pos) * kD + 8 * l);
      float4 *vd = reinterpret_cast<float4 *>(a.vc + ((size_t)j * a.max_pos + pos) * kD + 8 * l);
      kd[0] = make_float4(rv[0], rv[1], rv[2], rv[3]);
      kd[1] = make_float4(rv[4], rv[5], rv[6], rv[7]);
      vd[0] = make_float4(nv[0], nv[1], nv[2], nv[3]);
      vd[1] = make_float4(nv[4], nv[5], nv[6], nv[7]);
    }
  }
  __syncthreads();

  // ---- scores ---------------------------------------------------------------
  // (the rotated q and new k read once; the new k is chosen by a select,
  // not a branch around an LDS read)
  float qv[8], nk[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    qv[k] = S.rot[0][8 * l + k];
    nk[k] = S.rot[1][8 * l + k];
  }
#pragma unroll
  for (int pass = 0; pass < kSpan / 64; ++pass) {
    const int tp = base + 64 * pass + r;
    if (tp < n) {  // uniform over the 16 lanes of the position
      const bool at_pos = tp == pos;
#pragma unroll
      for (int k = 0; k < 8; ++k) kv[pass][k] = at_pos ? nk[k] : kv[pass][k];
      float pr[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) pr[k] = qv[k] * kv[pass][k];
      const float sc = sum16(tree8(pr)) * kScale;
      if (l == 0) S.s[64 * pass + r] = sc;
    }
  }
  __syncthreads();

  // ---- the largest score (wave 0) -------------------------------------------
  bool ok = true;
  if (wave == 0) {
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < kSpan / 64; ++k)
      if (base + 64 * k + lane < n) m = fmaxf(m, S.s[64 * k + lane]);
    m = max64(m);
    if (nspan > 1) {
      uint64_t *mx = a.mx + (size_t)h * kMaxSpans;
      if (lane == 0) store_tagged(mx + c, m, tag);
      float o = -INFINITY;
      if (lane < nspan) ok = poll_tagged<1>(mx + lane, tag, &o, err, a.spin_ticks);
      m = max64(o);
    }
    if (lane == 0) S.m = m;
  }
  if (__syncthreads_or(!ok)) return;

  // ---- weights e and their sums over 64 positions (waves 0..3) --------------
  if (t < kSpan) {
    float e = kNegZero;
    if (base + t < n) {
      const float d = S.s[t] - S.m;
      e = (float)fixed_exp((double)d);
    }
    S.e[t] = e;
    const float z = sum64(e);
    if (lane == 0) S.wsum[wave] = z;
  }
  __syncthreads();
  // the span's weighted value sums: 8 positions of 4 columns per thread, then
  // the lanes 32 apart (blocks 2w and 2w + 1 of wave w) give 16 positions
  {
    float w4[4];
#pragma unroll
    for (int col = 0; col < 4; ++col) {
      float pr[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float vk = col == 0 ? vv[k].x : col == 1 ? vv[k].y : col == 2 ? vv[k].z : vv[k].w;
        pr[k] = pb + k < n ? S.e[8 * pg + k] * vk : kNegZero;
      }
      const float b8 = tree8(pr);
      w4[col] = ops::half_sum32(b8);
    }
    if (lane < 32)
      *reinterpret_cast<float4 *>(&S.part[wave][4 * cq]) = make_float4(w4[0], w4[1], w4[2], w4[3]);
  }
  if (t == 0) S.z = (S.wsum[0] + S.wsum[1]) + (S.wsum[2] + S.wsum[3]);
  __syncthreads();

  // ---- the span's sums; o (workgroup 0) --------------------------------------
  float w = 0.0f, z = 0.0f;  // output column t's value sum and the weight sum
  if (out_t) {
    float pq[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) pq[k] = S.part[k][t];
    w = tree8(pq) + tree8(pq + 8);
    z = S.z;
  }
  if (nspan > 1) {
    uint64_t *wp = a.wp + (size_t)h * kMaxSpans * kD;
    uint64_t *zp = a.zp + (size_t)h * kMaxSpans;
    if (c > 0) {
      if (out_t) store_tagged(wp + (size_t)c * kD + t, w, tag);
      if (t == 0) store_tagged(zp + c, z, tag);
    } else {
      // every thread polls: column t % 128 of the spans 1 + 2 q, 2 + 2 q
      // (q = t / 128), and the weight sum of span t (t < 16), into LDS
      const int i = t % kD, sp0 = 1 + 2 * (t / kD);
      float v2[2];
      ok = poll_tagged_groups<1, 2>(wp + (size_t)sp0 * kD + i, kD, min(2, nspan - sp0), tag, v2,
                                  err, a.spin_ticks);
#pragma unroll
      for (int k = 0; k < 2; ++k)
        if (sp0 + k < kMaxSpans) S.sw[sp0 + k][i] = v2[k];
      if (t > 0 && t < kMaxSpans) {
        float zv = kNegZero;
        if (t < nspan) ok &= poll_tagged<1>(zp + t, tag, &zv, err, a.spin_ticks);
        S.sz[t] = zv;
      }
      if (out_t) S.sw[0][t] = w;
      if (t == 0) S.sz[0] = z;
    }
  }
  if (__syncthreads_or(!ok)) return;
  if (out_t) {
    const int i = t;
    if (nspan > 1 && c == 0) {
      // T over the positions: the balanced tree over 16 span slots (-0 past
      // the last span) of the spans' trees
      float ws[kMaxSpans], zs[kMaxSpans];
#pragma unroll
      for (int sp = 0; sp < kMaxSpans; ++sp) {
        ws[sp] = S.sw[sp][i];
        zs[sp] = S.sz[sp];
      }
      w = tree8(ws) + tree8(ws + 8);
      z = tree8(zs) + tree8(zs + 8);
    }
    if (c == 0) {
      const float ov = (w / z) * gate_value(gv);
      a.o[(size_t)h * kD + i] = ov;
      const float s = sum64(ov);  // the wave holds 64 consecutive values
      if (lane == 0) a.os[(size_t)h * 2 + i / 64] = s;
    }
  }
  if (__syncthreads_or(!ok)) return;
  if (t == 0) store_word(mine, tag);
}

}  // namespace

void atq_ws_layout(int32_t hq, int32_t hkv, AtqWs *out) {
  (void)hkv;
  size_t at = 0;
  auto take = [&at](size_t bytes) {
    const size_t p = at;
    at += (bytes + 255) & ~(size_t)255;
    return p;
  };
  out->mx = take(sizeof(uint64_t) * (size_t)hq * kAtqMaxSpans);
  out->zp = take(sizeof(uint64_t) * (size_t)hq * kAtqMaxSpans);
  out->wp = take(sizeof(uint64_t) * (size_t)hq * kAtqMaxSpans * kAtqD);
  out->ctl = take(sizeof(uint32_t) * (size_t)(kAtqErrorWord + 32));
  out->bytes = at;
}

hipError_t launch_atq(const AtqArgs &a, hipStream_t st) {
  const dim3 grid((a.max_pos + kAtqSpan - 1) / kAtqSpan, a.hq);
  hipLaunchKernelGGL(atq_kernel, grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace q4
