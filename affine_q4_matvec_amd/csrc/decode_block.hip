// Decoder layers of a decode token, attention block and MLP block, in one
// persistent launch (gfx950): "Metal: queued rmsq, swq, gdn and atq
// kernels and a 4-row q4mv, so a decode token is one command buffer with
// one wait" (#1440), Change (the rmsq, q4mv, atq and swq stages queued for
// a whole token) and Verification (one command buffer, one wait).  Each
// layer is the same as the separate calls
//   y = q4mv_norm(qgkv, h, wa)            [q; gate; k; v] = y
//   o = q4_atq(q, gate, k, v, ...)        (16 query heads of 128)
//   h = q4mv_add(O, o, osum, h)
//   m = q4mv_norm_swiglu(gate_up, h, wn); h = q4mv_add(down, m, NULL, h)
// with their bits, in one grid of one workgroup per compute unit whose
// stages hand their outputs to each other through tagged words (the
// protocol of tagged_device.h, as in the persistent MLP layers):
//   stage Q    every wave: rmsq(h, wa) for itself, its 2..4 rows of
//              [Q; gate; K; V]                    -> tagged q, gate, k, v
//   stage ATQ  one workgroup per query head and 256-position span up to
//              the position (16 to 256 workgroups): the attention step of
//              atq_kernel (scores, the span maxima exchanged as tagged
//              words, weights, the span sums gathered by span 0 of the
//              head, which forms o); the head's new key and value rows are
//              written by the span holding the position, if the head is
//              its group's first; the span's cache rows are loaded before
//              the wait                             -> tagged o, osum
//   stage O    every wave: one O row + the residual -> tagged h
//   stage A    rmsq(h, wn) once per workgroup (workgroup_rmsq); every
//              wave: its (gate, up) pairs, SwiGLU   -> tagged m
//   stage B    every wave: one down row + the residual -> tagged h for the
//              next layer's stage Q, or h (plain store) after the last
// The weights of a wave's next rows are loaded before the wait that
// precedes them (the next layer's Q rows before the wait for its h).  The
// tags name the call (a counter per workgroup), the layer and the stage.
// Every wait is bounded; one that runs out sets the error word and every
// workgroup leaves at its next wait.  Compiled with -ffp-contract=off, and
// with machine-level loop-invariant code motion off (build.py).
#include <math.h>

#include "decode_device.h"
#include "tagged_device.h"

#pragma clang fp contract(off)

namespace q4 {
namespace {

using namespace dev;
using namespace decode;

constexpr int kD = kAtqD;
constexpr int kHeads = kBlockHeads;
constexpr float kScale = 0x1.6a09e6p-4f;  // RN32(1 / sqrt(128))
constexpr int kQRowsPerWave = kBlockQRows / kCols;  // rows of [Q; gate; K; V] per wave, at most
static_assert(kThreads == 512, "the attention stage's thread layout");
static_assert(kBlockSpan == 256, "8 passes of 32 positions; 16 blocks of 16");

struct QBlock {
  u32x4 cw[kQRowsPerWave];
  float sv[kQRowsPerWave], bv[kQRowsPerWave];
};

struct Row {
  u32x4 cw;
  float sv, bv;
};

__device__ __forceinline__ void load_qrows(const BlockLayer &Y, int r0, int nrows, int lane,
                                           QBlock &a) {
  const auto qr = buffer_uniform(Y.qq + (size_t)r0 * 256, nrows * 1024);
  const auto sr = buffer_uniform(Y.qs + (size_t)r0 * 32, nrows * 128);
  const auto br = buffer_uniform(Y.qb + (size_t)r0 * 32, nrows * 128);
#pragma unroll
  for (int j = 0; j < kQRowsPerWave; ++j) {
    a.cw[j] = load_codes(qr, 16u * lane, j * 1024);
    a.sv[j] = load_f32(sr, 4u * (lane >> 1), j * 128);
    a.bv[j] = load_f32(br, 4u * (lane >> 1), j * 128);
  }
}

__device__ __forceinline__ void load_orow(const BlockLayer &Y, int r, int lane, Row &d) {
  const auto qr = buffer_uniform(Y.oq + (size_t)r * 256, 1024);
  const auto sr = buffer_uniform(Y.os + (size_t)r * 32, 128);
  const auto br = buffer_uniform(Y.ob + (size_t)r * 32, 128);
  d.cw = load_codes(qr, 16u * lane, 0);
  d.sv = load_f32(sr, 4u * (lane >> 1), 0);
  d.bv = load_f32(br, 4u * (lane >> 1), 0);
}

__device__ __forceinline__ void load8(const float *p, float *v) {
  const float4 a = reinterpret_cast<const float4 *>(p)[0];
  const float4 b = reinterpret_cast<const float4 *>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// The balanced tree over the 16 lanes of an aligned 16-lane row, in every
// lane of the row.
__device__ __forceinline__ float sum16(float s) {
  s = s + dpp<kDppQuadXor1>(s);
  return segment_sum<16>(s);
}

__device__ __forceinline__ float sum64(float s) {
  s = s + dpp<kDppQuadXor1>(s);
  return segment_sum<64>(s);
}

__device__ __forceinline__ float max64(float s) { return ops::lane_max64(s); }

struct AttnLds {
  float in[4][kD];          // q, gate, k, v of the head
  float tab[3 * kD];        // q and k norm weights, then the rotation's cos and sin
  float un[2][kD];          // normed q, k
  float rot[2][kD];         // rotated q, k
  float s[kBlockSpan];      // scores of the span
  float e[kBlockSpan];      // weights of the span
  alignas(16) float part[16][kD];  // value sums over 16 positions (stage B: m as polled)
  float sw[kBlockMaxSpans][kD];  // the spans' value sums (span 0 of a head)
  float sz[kBlockMaxSpans];      // the spans' weight sums
  float wsum[4];            // weight sums over 64 positions
  float m;                  // largest score
};

// Stages o into LDS for the O rows (the padded layout; the group sums are
// written by the caller): v[k] is value t + 512 k of thread t.
__device__ __forceinline__ void stage_o_input(Lds<1> &L, const float *v) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = threadIdx.x + kThreads * k;
    L.x[c + 4 * (c >> 5)] = v[k];
  }
}

// v, through an empty asm the optimiser cannot see through.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// The tags of layer l in call `call`: + 1 .. + 7 name the stage (and the
// attention stage's two exchanges between spans).
__device__ __forceinline__ uint32_t stage_tag(uint32_t call, int l) {
  return (call << 8) | ((uint32_t)l << 3);
}

// The layer table as the kernel reads it: the same layout as BlockLayer,
// with pointers typed as global ones, so that loads through them are
// global (or buffer) loads rather than flat loads of the generic address
// space.
#define Q4_GLOBAL __attribute__((address_space(1)))
struct GlobalLayer {
  const uint32_t Q4_GLOBAL *qq;
  const float Q4_GLOBAL *qs, *qb;
  const uint32_t Q4_GLOBAL *oq;
  const float Q4_GLOBAL *os, *ob;
  const float Q4_GLOBAL *wa, *wq, *wk;
  float Q4_GLOBAL *kc, *vc;
  const uint32_t Q4_GLOBAL *gq;
  const float Q4_GLOBAL *gs, *gb, *wn;
  const uint32_t Q4_GLOBAL *dq;
  const float Q4_GLOBAL *ds, *db;
};
static_assert(sizeof(GlobalLayer) == sizeof(BlockLayer), "one layout");

// Layer l: from the device layer table, else the one layer of the arguments.
__device__ __forceinline__ BlockLayer layer_at(const DecodeBlockArgs &A, int l) {
  GlobalLayer g;
  if (A.layers) {
    g = reinterpret_cast<const GlobalLayer *>(A.layers)[l];
  } else {
    const BlockLayer &o = A.one;
    g = GlobalLayer{(const uint32_t Q4_GLOBAL *)o.qq, (const float Q4_GLOBAL *)o.qs,
                    (const float Q4_GLOBAL *)o.qb, (const uint32_t Q4_GLOBAL *)o.oq,
                    (const float Q4_GLOBAL *)o.os, (const float Q4_GLOBAL *)o.ob,
                    (const float Q4_GLOBAL *)o.wa, (const float Q4_GLOBAL *)o.wq,
                    (const float Q4_GLOBAL *)o.wk, (float Q4_GLOBAL *)o.kc,
                    (float Q4_GLOBAL *)o.vc, (const uint32_t Q4_GLOBAL *)o.mlp.gq,
                    (const float Q4_GLOBAL *)o.mlp.gs, (const float Q4_GLOBAL *)o.mlp.gb,
                    (const float Q4_GLOBAL *)o.mlp.wn, (const uint32_t Q4_GLOBAL *)o.mlp.dq,
                    (const float Q4_GLOBAL *)o.mlp.ds, (const float Q4_GLOBAL *)o.mlp.db};
  }
  BlockLayer y;
  y.qq = (const uint32_t *)g.qq; y.qs = (const float *)g.qs; y.qb = (const float *)g.qb;
  y.oq = (const uint32_t *)g.oq; y.os = (const float *)g.os; y.ob = (const float *)g.ob;
  y.wa = (const float *)g.wa; y.wq = (const float *)g.wq; y.wk = (const float *)g.wk;
  y.kc = (float *)g.kc; y.vc = (float *)g.vc;
  y.mlp = DecodeLayer{(const uint32_t *)g.gq, (const float *)g.gs, (const float *)g.gb,
                      (const float *)g.wn, (const uint32_t *)g.dq, (const float *)g.ds,
                      (const float *)g.db};
  return y;
}

template <bool FAST, int NP>
__global__ __launch_bounds__(kThreads) void decode_block_kernel(DecodeBlockArgs A) {
  __shared__ Lds<NP> S;  // x = rmsq(h) (stage A) or m (stage B)
  __shared__ Lds<1> SO;  // h between layers (stage Q) or o (stage O)
  __shared__ AttnLds T;
  const int nwg = gridDim.x;
  const int wg = blockIdx.x;
  const int wave = wave_index();
  uint32_t *err = A.ctl + kBlockErrorWord;
  if (__syncthreads_or(load_word(err) != 0)) return;
  const uint32_t call = load_word(A.ctl + wg);
  const int gw = wave * nwg + wg;
  const int stride = kWaves * nwg;
  const int row = gw;
  const bool has_row = row < kCols;
  const int copy = wg % kDecodeCopies;
  const int G = kHeads / A.hkv;
  const int nq = 2 * kCols + 2 * A.hkv * kD;
  const int qb = (int)(((long long)nq * gw) / stride);
  const int qe = (int)(((long long)nq * (gw + 1)) / stride);
  const int pb = (int)(((long long)A.inter * gw) / stride);
  const int pe = (int)(((long long)A.inter * (gw + 1)) / stride);
  const int pos = *A.pos;
  const bool pos_ok = pos >= 0 && pos < A.max_pos;
  const int n = pos_ok ? pos + 1 : 0;
  const int negz = neg_zero_reg();
  // the residual of the wave's row (lane 63): h before the first layer,
  // carried from layer to layer
  const int lane0 = threadIdx.x & (kWave - 1);
  float res = has_row && lane0 == kWave - 1 ? A.h[row] : 0.0f;
  QBlock qa;
  if (qb < qe) load_qrows(layer_at(A, 0), qb, qe - qb, lane0, qa);

  for (int l = 0; l < A.nlayers; ++l) {
    // the thread index, opaque to the optimiser: the addresses and table
    // loads derived from it stay in the layer instead of being hoisted out
    // of the loop and held in registers through every stage
    const int t = opaque(threadIdx.x);
    const int lane = t & (kWave - 1);
    const bool mine = 8 * t < kCols;
    const bool odd = lane & 1;
    const BlockLayer Y = layer_at(A, l);
    // + 1 q/gate/k/v, + 2 o, + 3 h after attention, + 4 m, + 5 h after the
    // layer, + 6 span maxima, + 7 span sums
    const uint32_t tag = stage_tag(call, l);

    // ---- stage Q --------------------------------------------------------------
    // x = rmsq(h, wa) over the workgroup, as in stage A (threads 0..255
    // take 8 columns): h is the layer's input, or the previous layer's
    // tagged output, polled as words t + 512 k (each wave's load: 64
    // consecutive words) into SO.x; after a barrier threads 0..255 take
    // their 8 values
    {
      bool ok = true;
      float h8[8] = {}, w8[8] = {};
      if (mine) load8(Y.wa + 8 * t, w8);
      if (l == 0) {
        if (mine) load8(A.h + 8 * t, h8);
      } else {
        static_assert(kCols == 4 * kThreads, "4 words of h per thread");
        float h4[4];
        ok = poll_tagged<4, kThreads>(A.hb + (size_t)copy * kCols + t, stage_tag(call, l - 1) + 5,
                                      h4, err, A.spin_ticks);
#pragma unroll
        for (int k = 0; k < 4; ++k) SO.x[t + kThreads * k] = h4[k];
        __syncthreads();
        if (mine) {
          const float4 *src = reinterpret_cast<const float4 *>(SO.x + 8 * t);
          const float4 a0 = src[0], a1 = src[1];
          h8[0] = a0.x; h8[1] = a0.y; h8[2] = a0.z; h8[3] = a0.w;
          h8[4] = a1.x; h8[5] = a1.y; h8[6] = a1.z; h8[7] = a1.w;
        }
      }
      if (!workgroup_rmsq(SO, h8, w8, A.eps, ok)) return;
      float xv[32];
      const float xsv = load_rmsq_x(SO, lane, xv);
#pragma unroll
      for (int i = 0; i < kQRowsPerWave; ++i) {
        if (qb + i < qe) {  // uniform per wave
          const float tv = group_term<FAST>(qa.cw[i], xv, qa.sv[i], qa.bv[i], xsv, true, odd);
          const float v = wave_sum_lane63(tv, negz);
          if (lane == kWave - 1)
#pragma unroll
            for (int c = 0; c < kDecodeCopies; ++c)
              store_tagged(A.qv + (size_t)c * kBlockQRows + qb + i, v, tag + 1);
        }
      }
    }
    // (zero-initialised: a value loaded under a condition would otherwise
    // be carried from the previous layer and held through every stage)
    Row od{};
    if (has_row) load_orow(Y, row, lane, od);
    issue_order();

    // ---- stage ATQ (one workgroup per query head and 256-position span) ------
    // Task i = ((c hkv + j) G + g): head j G + g of key/value head j over
    // positions [256 c, 256 c + 256), for the spans up to pos; span 0 of
    // each head gathers the others' sums and forms o.  Workgroup w runs on
    // XCD w % 8 and takes task (w % 8) (nwg / 8) + w / 8, so that the G
    // heads that read the same cache rows share an XCD and its L2.
    const int nspan = pos_ok ? pos / kBlockSpan + 1 : 1;
    const int per_xcd = nwg / kXcds;
    const int task = wg < kXcds * per_xcd ? (wg % kXcds) * per_xcd + wg / kXcds : nwg;
    if (task < kHeads * nspan) {
      const int g = task % G, jc = task / G;
      const int j = jc % A.hkv, c = jc / A.hkv, hd = j * G + g;
      const int p0 = kBlockSpan * c;           // the span's first position
      const int pn = min(n - p0, kBlockSpan);  // its positions below n (none for a bad pos)
      const bool owns_pos = pos_ok && pos / kBlockSpan == c;
      const int r = t >> 4, lq = t & 15;  // scores: 32 positions per pass
      // the norm weights and the rotation table's row, for LDS below
      float tv = 0.0f;
      if (t < 2 * kD) {
        tv = (t < kD ? Y.wq : Y.wk)[t % kD];
      } else if (t < 3 * kD) {
        const int pr = pos_ok ? pos : 0;
        tv = (t < 5 * kD / 2 ? A.cs : A.sn)[(size_t)pr * (kD / 2) + t % (kD / 2)];
      }
      // the span's cache rows below n, loaded before the wait (bounded
      // buffer loads: zeros from n on; row pos is stale here and not used)
      const size_t hb = ((size_t)j * A.max_pos + p0) * kD;
      const uint32_t span_bytes = (uint32_t)max(pn, 0) * kD * 4u;
      const auto kr = buffer_uniform(Y.kc + hb, span_bytes);
      const auto vr = buffer_uniform(Y.vc + hb, span_bytes);
      float kv[8][8];
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const uint32_t off = 4u * (uint32_t)((32 * p + r) * kD + 8 * lq);
        const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, 0);
        const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(kr, off + 16u, 0, 0);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          kv[p][k] = __uint_as_float(a[k]);
          kv[p][k + 4] = __uint_as_float(b[k]);
        }
      }
      const int cq = t & 31, pg = t >> 5;  // values: 4 columns x 16 positions
      float v0[16], v1[16], v2[16], v3[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const uint32_t off = 4u * (uint32_t)((16 * pg + k) * kD + 4 * cq);
        const u32x4 f = __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, 0);
        v0[k] = __uint_as_float(f[0]);
        v1[k] = __uint_as_float(f[1]);
        v2[k] = __uint_as_float(f[2]);
        v3[k] = __uint_as_float(f[3]);
      }
      if (t < 3 * kD) T.tab[t] = tv;  // waits for these loads only, not the cache rows
      // q, gate (rows of this head), k, v (rows of its key/value head)
      {
        const int part = t / kD, i = t % kD;
        const int src = part == 0   ? kD * hd + i
                        : part == 1 ? kCols + kD * hd + i
                        : part == 2 ? 2 * kCols + kD * j + i
                                    : 2 * kCols + kD * A.hkv + kD * j + i;
        float v = 0.0f;
        const bool ok =
            poll_tagged<1>(A.qv + (size_t)copy * kBlockQRows + src, tag + 1, &v, err, A.spin_ticks);
        T.in[part][i] = v;
        if (!__syncthreads_and(ok)) return;
      }
      // rmsq of q (row 0) and k (row 1), then the rotation
      if (t < 32) {
        float x[8], sq[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          x[k] = T.in[r == 0 ? 0 : 2][8 * lq + k];
          sq[k] = x[k] * x[k];
        }
        const float rho = ops::rmsq_rho_from_ss(sum16(ops::tree8(sq)), kD, A.eps);
#pragma unroll
        for (int k = 0; k < 8; ++k)
          T.un[r][8 * lq + k] = ops::rmsq_value(x[k], rho, T.tab[kD * r + 8 * lq + k]);
      }
      // the same 32 threads of wave 0 read T.un back: the wave's LDS
      // accesses are done in order, so no barrier
      issue_order();
      if (t < 32) {
        // value d < 64: a c - b s with a = un[d], b = un[d + 64]; value
        // d >= 64: a s + b c with a = un[d - 64], b = un[d]; as one
        // expression, own c + (-/+ partner s): the same sums, no branch
        const float *ct = T.tab + 2 * kD + 8 * (lq & 7), *st = ct + kD / 2;
        const float *own = T.un[r] + 8 * lq, *partner = T.un[r] + 8 * (lq ^ 8);
        const bool first_half = lq < 8;
        float rv[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float pc = own[k] * ct[k], ps = partner[k] * st[k];
          rv[k] = pc + (first_half ? -ps : ps);
          T.rot[r][8 * lq + k] = rv[k];
        }
        if (r == 1 && hd % G == 0 && owns_pos) {  // the new cache rows
          const size_t at = ((size_t)j * A.max_pos + pos) * kD + 8 * lq;
          float4 *kd = reinterpret_cast<float4 *>(Y.kc + at);
          float4 *vd = reinterpret_cast<float4 *>(Y.vc + at);
          kd[0] = make_float4(rv[0], rv[1], rv[2], rv[3]);
          kd[1] = make_float4(rv[4], rv[5], rv[6], rv[7]);
          const float *nv = T.in[3] + 8 * lq;
          vd[0] = make_float4(nv[0], nv[1], nv[2], nv[3]);
          vd[1] = make_float4(nv[4], nv[5], nv[6], nv[7]);
        }
      }
      __syncthreads();
      // scores (the rotated q and new k read once: a select between the new
      // k and a cache row, not a branch around an LDS read)
      float rq[8], rk[8];
      {
        const float4 *q4p = reinterpret_cast<const float4 *>(&T.rot[0][8 * lq]);
        const float4 *k4p = reinterpret_cast<const float4 *>(&T.rot[1][8 * lq]);
        const float4 a0 = q4p[0], a1 = q4p[1], b0 = k4p[0], b1 = k4p[1];
        rq[0] = a0.x; rq[1] = a0.y; rq[2] = a0.z; rq[3] = a0.w;
        rq[4] = a1.x; rq[5] = a1.y; rq[6] = a1.z; rq[7] = a1.w;
        rk[0] = b0.x; rk[1] = b0.y; rk[2] = b0.z; rk[3] = b0.w;
        rk[4] = b1.x; rk[5] = b1.y; rk[6] = b1.z; rk[7] = b1.w;
      }
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const int tp = 32 * p + r;
        if (tp < pn) {  // uniform over the 16 lanes of the position
          const bool at_pos = p0 + tp == pos;
          float pr[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) pr[k] = rq[k] * (at_pos ? rk[k] : kv[p][k]);
          const float sc = sum16(ops::tree8(pr)) * kScale;
          if (lq == 0) T.s[tp] = sc;
        }
      }
      __syncthreads();
      // the largest score: of the span, then over the head's spans
      bool ok = true;
      if (wave == 0) {
        float m = -INFINITY;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (64 * k + lane < pn) m = fmaxf(m, T.s[64 * k + lane]);
        m = max64(m);
        if (nspan > 1) {
          uint64_t *mx = A.mx + (size_t)hd * kBlockMaxSpans;
          if (lane == 0) store_tagged(mx + c, m, tag + 6);
          float o = -INFINITY;
          if (lane < nspan) ok = poll_tagged<1>(mx + lane, tag + 6, &o, err, A.spin_ticks);
          m = max64(o);
        }
        if (lane == 0) T.m = m;
      }
      if (__syncthreads_or(!ok)) return;
      if (t < kBlockSpan) {
        float e = kNegZero;
        if (t < pn) {
          const float d = T.s[t] - T.m;
          e = (float)ops::fixed_exp((double)d);
        }
        T.e[t] = e;
        const float z = sum64(e);
        if (lane == 0) T.wsum[wave] = z;
      }
      __syncthreads();
      // the weighted value sums over 16 positions of 4 columns (the new row,
      // at pos, from the inputs)
      {
        const int kp = pos - p0 - 16 * pg;  // the new row's slot in this thread's block, if any
        if (kp >= 0 && kp < 16) {
          const float4 nv = *reinterpret_cast<const float4 *>(&T.in[3][4 * cq]);
#pragma unroll
          for (int k = 0; k < 16; ++k) {  // selects, not branches
            const bool at = k == kp;
            v0[k] = at ? nv.x : v0[k];
            v1[k] = at ? nv.y : v1[k];
            v2[k] = at ? nv.z : v2[k];
            v3[k] = at ? nv.w : v3[k];
          }
        }
        float ek[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) ek[k] = T.e[16 * pg + k];
        const auto block16 = [&](const float *vc) {
          float pr[16];
#pragma unroll
          for (int k = 0; k < 16; ++k) pr[k] = 16 * pg + k < pn ? ek[k] * vc[k] : kNegZero;
          return ops::tree8(pr) + ops::tree8(pr + 8);
        };
        *reinterpret_cast<float4 *>(&T.part[pg][4 * cq]) =
            make_float4(block16(v0), block16(v1), block16(v2), block16(v3));
      }
      __syncthreads();
      float w = 0.0f, z = 0.0f;  // output column t's value sum and the weight sum
      if (t < kD) {
        float pq[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) pq[k] = T.part[k][t];
        w = ops::tree8(pq) + ops::tree8(pq + 8);
        z = (T.wsum[0] + T.wsum[1]) + (T.wsum[2] + T.wsum[3]);
      }
      if (nspan > 1) {
        // the spans' sums: T over the positions is the balanced tree over
        // 16 span slots (-0 past the last span) of the spans' trees
        uint64_t *wp = A.wp + (size_t)hd * kBlockMaxSpans * kD;
        uint64_t *zp = A.zp + (size_t)hd * kBlockMaxSpans;
        if (c > 0) {
          if (t < kD) store_tagged(wp + (size_t)c * kD + t, w, tag + 7);
          if (t == 0) store_tagged(zp + c, z, tag + 7);
        } else {
          // span 0 gathers them with every thread: column t % 128 of the
          // spans 1 + 4 q .. 4 + 4 q (q = t / 128), and the weight sum of
          // span t (t < 16), into LDS
          const int i = t % kD, sp0 = 1 + 4 * (t / kD);
          float v4[4];
          ok = poll_tagged_groups<1, 4>(wp + (size_t)sp0 * kD + i, kD, min(4, nspan - sp0),
                                      tag + 7, v4, err, A.spin_ticks);
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if (sp0 + k < kBlockMaxSpans) T.sw[sp0 + k][i] = v4[k];
          if (t > 0 && t < kBlockMaxSpans) {
            float zv = kNegZero;
            if (t < nspan) ok &= poll_tagged<1>(zp + t, tag + 7, &zv, err, A.spin_ticks);
            T.sz[t] = zv;
          }
          if (t < kD) T.sw[0][t] = w;
          if (t == 0) T.sz[0] = z;
        }
      }
      if (__syncthreads_or(!ok)) return;
      if (nspan > 1 && c == 0 && t < kD) {
        float ws[kBlockMaxSpans], zs[kBlockMaxSpans];
#pragma unroll
        for (int sp = 0; sp < kBlockMaxSpans; ++sp) {
          ws[sp] = T.sw[sp][t];
          zs[sp] = T.sz[sp];
        }
        w = ops::tree8(ws) + ops::tree8(ws + 8);
        z = ops::tree8(zs) + ops::tree8(zs + 8);
      }
      if (c == 0 && t < kD) {
        const double gd = (double)T.in[1][t];
        const float sig = (float)(1.0 / (1.0 + ops::fixed_exp(-gd)));
        const float ov = pos_ok ? (w / z) * sig : __builtin_nanf("");
        const float gsum = sum64(ov);  // waves 0 and 1: the head's two groups
#pragma unroll
        for (int cp = 0; cp < kDecodeCopies; ++cp) {
          uint64_t *o = A.ov + (size_t)cp * kBlockORows;
          store_tagged(o + kD * hd + t, ov, tag + 2);
          if (lane == 0) store_tagged(o + kCols + 2 * hd + wave, gsum, tag + 2);
        }
      }
    }

    // ---- stage O: h = h + O o ---------------------------------------------------
    GuBlock a{};
    if (pb < pe) load_gu(Y.mlp, pb, min(kGuPairs, pe - pb), lane, a);
    issue_order();
    {
      // the wait for the attention stage is long: wave 0 alone polls (the
      // group sums of every head) until it ends, then every thread takes its
      // words
      bool ok = wave != 0 || await_words(A.ov + (size_t)copy * kBlockORows + kCols, 2 * kHeads,
                                         tag + 2, err, A.spin_ticks);
      if (!__syncthreads_and(ok)) return;
      // every thread polls words t + 512 k of o (lane-contiguous loads);
      // threads t < 32 also the group sum t (the others poll word t again
      // in its place)
      float o5[5];
      {
        const int off[5] = {t, t + kThreads, t + 2 * kThreads, t + 3 * kThreads,
                            t < 2 * kHeads ? kCols + t : t};
        ok = poll_tagged_at<5>(A.ov + (size_t)copy * kBlockORows, off, tag + 2, o5, err,
                               A.spin_ticks);
      }
      if (!__syncthreads_and(ok)) return;
      if (t < 2 * kHeads) SO.xs[t] = o5[4];
      stage_o_input(SO, o5);
      __syncthreads();
      if (has_row) {
        Lds<1> &L = SO;
        float xv[32];
        load_x_values(L.x + lane * kChunkStride, true, xv);
        const float xsv = L.xs[lane >> 1];
        const float tv = group_term<FAST>(od.cw, xv, od.sv, od.bv, xsv, true, odd);
        const float v = wave_sum_lane63(tv, negz);
        if (lane == kWave - 1) {
          res = res + v;
#pragma unroll
          for (int c = 0; c < kDecodeCopies; ++c)
            store_tagged(A.hv + (size_t)c * kCols + row, res, tag + 3);
        }
      }
    }

    // ---- stage A: m = SwiGLU([gate; up] rmsq(h, wn)) --------------------------
    {
      // x = rmsq(h, wn) over the workgroup: threads 0..255 take 8 columns
      bool ok = true;
      float h8[8] = {}, w8[8] = {};
      // every thread polls words t + 512 k of h into S.x (free: its last
      // readers, the previous layer's down rows, are past several
      // barriers); after a barrier threads 0..255 take their 8 values
      if (mine) load8(Y.mlp.wn + 8 * t, w8);
      {
        float h4[4];
        ok = poll_tagged<4, kThreads>(A.hv + (size_t)copy * kCols + t, tag + 3, h4, err,
                                      A.spin_ticks);
#pragma unroll
        for (int k = 0; k < 4; ++k) S.x[t + kThreads * k] = h4[k];
      }
      issue_order();
      DownRow<NP> d{};
      if (has_row) load_down<NP>(Y.mlp, row, lane, d);
      __syncthreads();
      if (mine) {
        const float4 *src = reinterpret_cast<const float4 *>(S.x + 8 * t);
        const float4 a0 = src[0], a1 = src[1];
        h8[0] = a0.x; h8[1] = a0.y; h8[2] = a0.z; h8[3] = a0.w;
        h8[4] = a1.x; h8[5] = a1.y; h8[6] = a1.z; h8[7] = a1.w;
      }
      if (!workgroup_rmsq(S, h8, w8, A.eps, ok)) return;
      {
        float xv[32];
        const float xsv = load_rmsq_x(S, lane, xv);
        uint64_t *mq = A.mq;
        const uint32_t tm = tag + 4;
        const auto store_m = [mq, tm](int i, float v) {
#pragma unroll
          for (int c = 0; c < kDecodeCopies; ++c) store_tagged(mq + c * kDecodeMaxInter + i, v, tm);
        };
        if (pb < pe) gu_stage<FAST>(Y.mlp, xv, xsv, lane, pb, pe, a, store_m);
      }

      // ---- stage B: h = h + down m ---------------------------------------------
      // chunk c = 8 consecutive values of m; the last four waves poll them
      // (poller p: chunks p, p + 256, ...) and write them to LDS.  A wave's
      // loads complete in issue order for its
      // wait counter, so a poll behind a fresh prefetch would wait for it:
      // the first four waves (which poll h in the next stage Q) load their
      // next Q rows now, the pollers once their polls are done.
      constexpr int kChunks = NP * kCols / 8;
      constexpr int kPollThreads = 256;
      constexpr int kPerPoller = kChunks / kPollThreads;
      static_assert(kChunks % kPollThreads == 0, "whole rounds of chunks");
      const bool poller = t >= kThreads - kPollThreads;
      if (!poller && l + 1 < A.nlayers && qb < qe)
        load_qrows(layer_at(A, l + 1), qb, qe - qb, lane, qa);
      issue_order();
      if (t == 0) S.flag = 0u;
      __syncthreads();  // every wave of the workgroup is done with stage A
      const uint64_t *mcopy = A.mq + (size_t)copy * kDecodeMaxInter;
      if (poller) {
        const int p = t - (kThreads - kPollThreads);
        // the poller wave's 64 chunks of a round (512 consecutive words)
        // polled lane-contiguous (words lane + 64 k: 4 cache lines per
        // load), then through the wave's slice of T.part (free in this
        // stage; one wave writes and reads it, and its LDS accesses are done
        // in order) to chunk c = 8 consecutive values per lane
        float *stg = &T.part[0][0] + 512 * (p / kWave);
        static_assert(sizeof(T.part) >= 4 * 512 * sizeof(float), "4 poller waves");
        // one chunk at a time: polling several in the same rounds multiplies
        // the polled traffic while the wait lasts
#pragma unroll 1
        for (int r = 0; r < kPerPoller; ++r) {
          const int c = p + r * kPollThreads;
          float xm[8];
          if (!poll_tagged<8, kWave>(mcopy + 2048 * r + 512 * (p / kWave) + lane, tag + 4, xm,
                                     err, A.spin_ticks)) {
            S.flag = 1u;
            break;
          }
#pragma unroll
          for (int k = 0; k < 8; ++k) stg[lane + kWave * k] = xm[k];
          issue_order();
          {
            const float4 *src = reinterpret_cast<const float4 *>(stg + 8 * lane);
            const float4 a0 = src[0], a1 = src[1];
            xm[0] = a0.x; xm[1] = a0.y; xm[2] = a0.z; xm[3] = a0.w;
            xm[4] = a1.x; xm[5] = a1.y; xm[6] = a1.z; xm[7] = a1.w;
          }
          // group sums: T over each chunk, then over 8 chunks by a butterfly
          const float gs = ops::lane_sum8(ops::tree8(xm));
          if ((c & 7) == 0) S.xs[c >> 3] = gs;
          float4 *dst = reinterpret_cast<float4 *>(S.x + 8 * c + 4 * (c >> 2));
          dst[0] = make_float4(xm[0], xm[1], xm[2], xm[3]);
          dst[1] = make_float4(xm[4], xm[5], xm[6], xm[7]);
        }
        if (l + 1 < A.nlayers && qb < qe) load_qrows(layer_at(A, l + 1), qb, qe - qb, lane, qa);
        issue_order();
      }
      __syncthreads();
      if (S.flag != 0u) return;
      if (has_row) {
        const float v = down_row<NP, FAST>(S, lane, d);
        if (lane == kWave - 1) {
          res = res + v;
          if (l + 1 < A.nlayers) {
#pragma unroll
            for (int c = 0; c < kDecodeCopies; ++c)
              store_tagged(A.hb + (size_t)c * kCols + row, res, tag + 5);
          } else {
            A.h[row] = res;
          }
        }
      }
    }
  }  // layers
  __syncthreads();
  if (threadIdx.x == 0) store_word(A.ctl + wg, call + 1);
}

template <bool FAST, int NP>
const void *kernel_ptr() {
  return reinterpret_cast<const void *>(&decode_block_kernel<FAST, NP>);
}

const void *block_kernel(int mode, int np) {
  const bool fast = mode != 0;
  switch (np) {
    case 1: return fast ? kernel_ptr<true, 1>() : kernel_ptr<false, 1>();
    case 2: return fast ? kernel_ptr<true, 2>() : kernel_ptr<false, 2>();
    case 3: return fast ? kernel_ptr<true, 3>() : kernel_ptr<false, 3>();
    case 4: return fast ? kernel_ptr<true, 4>() : kernel_ptr<false, 4>();
    default: return nullptr;
  }
}

}  // namespace

int32_t decode_block_grid(int mode, int32_t inter) {
  const void *k = block_kernel(mode, inter / kCols);
  if (!k || inter % kCols) return 0;
  int dev = 0, per_cu = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kThreads, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  // one workgroup per compute unit, a wave for every O and down row, a
  // workgroup for every head and span of the attention stage
  if (per_cu < 1 || cus * kWaves < kCols || cus < kBlockHeads * kBlockMaxSpans ||
      cus > kDecodeMaxGroups)
    return 0;
  return cus;
}

hipError_t launch_decode_block(const DecodeBlockArgs &a, int mode, hipStream_t st) {
  const int32_t grid = decode_block_grid(mode, a.inter);
  const void *k = block_kernel(mode, a.inter / kCols);
  if (grid < 1 || !k) return hipErrorInvalidValue;
  void *args[] = {const_cast<DecodeBlockArgs *>(&a)};
  return hipLaunchKernel(k, dim3(grid), dim3(kThreads), args, 0, st);
}

}  // namespace q4
