// Building blocks of the persistent decode kernels (decode_layers.hip,
// decode_block.hip): one workgroup of 512 threads per compute unit, rows
// of 2048 columns summed by one wave each with the q4mv kernels' group
// terms and row trees (q4mv_device.h), so every value has the bits of the
// separate kernels.
#pragma once

#include "ops_device.h"
#include "q4mv_device.h"
#include "q4mv_internal.h"

#pragma clang fp contract(off)

namespace q4 {
namespace decode {

using namespace dev;

constexpr int kThreads = 512;   // 8 waves: two per SIMD, up to 256 registers each
constexpr int kWaves = kThreads / kWave;
constexpr int kCols = 2048;     // width of h: the gate/up rows and the down output
constexpr int kGuPairs = 3;     // (gate, up) row pairs per block
constexpr int kGuR = 2 * kGuPairs;
constexpr int kChunkStride = 36;  // LDS floats per 32-value chunk (4 of padding)
constexpr int kXcds = 8;          // MI355X: workgroup w is dispatched to XCD w % 8

template <int NP>
struct alignas(16) Lds {
  float x[NP * 64 * kChunkStride];  // x = rmsq(h) (stage A) or m (stage B)
  float xs[NP * 32];                // their group sums
  float red[kWaves];                // the waves' sums of squares
  uint32_t flag;                    // stage B: a wait gave up
  alignas(16) uint32_t wflag[kWaves];     // workgroup_rmsq: per wave, a wait gave up
  float own[8 * 4];                 // stage B: the owned rows' pass sums
  float ownw[8 * 8 * 4];            // stage B: the owned rows' node sums
};

// Whether `p` holds in any thread of the workgroup, with one barrier: each
// wave's vote goes to slot[wave], then every thread reads all of them.
// (HIP's __syncthreads_or takes three barriers and an LDS atomic.)  The
// caller must not use the same slots again before a further barrier.
__device__ __forceinline__ bool workgroup_any(uint32_t *slot, bool p) {
  static_assert(kWaves == 8, "two 16-byte reads of the slots");
  const bool w = __any(p);
  if ((threadIdx.x & (kWave - 1)) == 0) slot[threadIdx.x / kWave] = w ? 1u : 0u;
  __syncthreads();
  const uint4 a = reinterpret_cast<const uint4 *>(slot)[0];
  const uint4 b = reinterpret_cast<const uint4 *>(slot)[1];
  return ((a.x | a.y | a.z | a.w) | (b.x | b.y | b.z | b.w)) != 0u;
}

// rmsq of h over the workgroup, with the arithmetic and tree of the rmsq
// kernel (ops_device.h), so the bits of every wave forming it alone:
// threads 0..255 (waves 0..3) hold h and the weights of columns [8t, 8t+8)
// (h8, w8); the sum of squares goes over the 64 lanes of each wave, then
// the 4 wave sums in a balanced tree: the balanced tree over the 2048
// squares in index order.  Waves 4..7 only vote: each shares a SIMD with
// one of waves 0..3, and when they formed the same sums (over -0 in place
// of h: four -0 wave sums more in the tree, which change nothing) their
// copy of the arithmetic delayed both at the barriers.  x goes to L.x in
// the row stages' padded layout, its group sums to L.xs.  Returns false
// when `ok` is false in any thread (a wait gave up).  Two workgroup
// barriers; L must be free (every earlier reader past a barrier).
template <int NP>
__device__ __forceinline__ bool workgroup_rmsq(Lds<NP> &L, const float *h8, const float *w8,
                                              float eps, bool ok) {
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1), wave = t / kWave;
  constexpr int kHWaves = kCols / (8 * kWave);
  static_assert(kHWaves == 4, "the tree over the wave sums");
  const bool hw = wave < kHWaves;  // wave-uniform: the 8 t < kCols threads
  if (hw) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = h8[k] * h8[k];
    const float s = ops::lane_sum64(ops::tree8(v));
    if (lane == 0) L.red[wave] = s;
  }
  if (workgroup_any(L.wflag, !ok)) return false;
  if (hw) {
    const float *r = L.red;
    const float ss = (r[0] + r[1]) + (r[2] + r[3]);
    const float rho = ops::rmsq_rho_from_ss(ss, kCols, eps);
    float u[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) u[k] = ops::rmsq_value(h8[k], rho, w8[k]);
    float4 *dst = reinterpret_cast<float4 *>(L.x + 8 * t + 4 * (t >> 2));
    dst[0] = make_float4(u[0], u[1], u[2], u[3]);
    dst[1] = make_float4(u[4], u[5], u[6], u[7]);
    const float g = ops::lane_sum8(ops::tree8(u));
    if ((t & 7) == 0) L.xs[t >> 3] = g;
  }
  __syncthreads();
  return true;
}

// A wave's 32 values of x from L (lane l: columns [32 l, 32 l + 32)) and
// the group sum of its lane pair.
template <int NP>
__device__ __forceinline__ float load_rmsq_x(const Lds<NP> &L, int lane, float *xv) {
  load_x_values(L.x + kChunkStride * lane, true, xv);
  return L.xs[lane >> 1];
}

// A buffer descriptor from a base and size that are the same in every
// lane of the wave (a wave's rows, a task's cache span), taken from the
// first lane: the compiler then keeps the descriptor in scalar registers.
// Built from values it cannot prove uniform (pointers read from the layer
// table), a descriptor would cost a waterfall loop around every load.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_uniform(const void *base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return buffer(reinterpret_cast<const void *>(((uint64_t)hi << 32) | lo),
                __builtin_amdgcn_readfirstlane(bytes));
}

struct GuBlock {
  u32x4 cw[kGuR];
  float sv[kGuR], bv[kGuR];
};

template <int NP>
struct DownRow {
  u32x4 cw[NP];
  float sv[NP], bv[NP];
};

// Rows 2 p0 .. 2 p0 + 2 np - 1 (np <= kGuPairs pairs); the buffer's size
// makes the loads of the rows past them return zero without a memory access.
__device__ __forceinline__ void load_gu(const DecodeLayer &L, int p0, int np, int lane,
                                        GuBlock &a) {
  const size_t r0 = 2 * (size_t)p0;
  const auto qr = buffer_uniform(L.gq + r0 * 256, 2 * np * 1024);
  const auto sr = buffer_uniform(L.gs + r0 * 32, 2 * np * 128);
  const auto br = buffer_uniform(L.gb + r0 * 32, 2 * np * 128);
#pragma unroll
  for (int j = 0; j < kGuR; ++j) {
    a.cw[j] = load_codes(qr, 16u * lane, j * 1024);
    a.sv[j] = load_f32(sr, 4u * (lane >> 1), j * 128);
    a.bv[j] = load_f32(br, 4u * (lane >> 1), j * 128);
  }
}

// Row r of the down matrix: pass p covers columns [2048 p, 2048 p + 2048).
template <int NP>
__device__ __forceinline__ void load_down(const DecodeLayer &L, int r, int lane, DownRow<NP> &d) {
  const auto qr = buffer_uniform(L.dq + (size_t)r * (NP * 256), NP * 1024);
  const auto sr = buffer_uniform(L.ds + (size_t)r * (NP * 32), NP * 128);
  const auto br = buffer_uniform(L.db + (size_t)r * (NP * 32), NP * 128);
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    d.cw[p] = load_codes(qr, 16u * lane, p * 1024);
    d.sv[p] = load_f32(sr, 4u * (lane >> 1), p * 128);
    d.bv[p] = load_f32(br, 4u * (lane >> 1), p * 128);
  }
}

// Keeps the compiler from moving memory accesses across this point (the
// weight loads of the next stage stay behind the loads of the current wait).
__device__ __forceinline__ void issue_order() { asm volatile("" ::: "memory"); }

// Appends the pair (gate, up) for m[out], the same in every lane, to the
// wave's SwiGLU batch (swiglu_push of q4mv_device.h for values already
// read from their lane).
template <bool FAST, class Store>
__device__ __forceinline__ void swiglu_push_uniform(const Store &store, SwigluBatch &b, int lane,
                                                    float g, float u, int out) {
  const bool mine = lane == b.count;
  b.gate = mine ? g : b.gate;
  b.up = mine ? u : b.up;
  b.out = mine ? out : b.out;
  b.count = b.count + 1;
  if (b.count == kWave) swiglu_flush<FAST>(store, b);
}

// One gate/up block of np pairs: the group terms of all its rows, then the
// row sums (rows 0..3 together by quad_row_sums, row j ending in lanes
// [16 j, 16 j + 16); rows 4 and 5 in lane 63: the same tree as
// wave_sum_lane63), then each (gate, up) pair goes into the wave's SwiGLU
// batch (m[p0 + i]).
template <bool FAST, class Store>
__device__ __forceinline__ void gu_block(const GuBlock &a, const float *xv, float xsv, int lane,
                                         int p0, int np, const Store &store, SwigluBatch &batch,
                                         int negz) {
  static_assert(kGuR == 6, "four rows by quad_row_sums, two by wave_sum_lane63");
  const bool odd = lane & 1;
  float t[kGuR];
#pragma unroll
  for (int j = 0; j < kGuR; ++j)
    t[j] = j < 2 * np ? group_term<FAST>(a.cw[j], xv, a.sv[j], a.bv[j], xsv, true, odd)
                      : kNegZero;
  const float q = quad_row_sums(t[0], t[1], t[2], t[3]);
  const float r4 = wave_sum_lane63(t[4], negz);
  const float r5 = wave_sum_lane63(t[5], negz);
  const auto at = [](float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
  };
  const float g[kGuPairs] = {at(q, 15), at(q, 47), at(r4, kWave - 1)};
  const float u[kGuPairs] = {at(q, 31), at(q, kWave - 1), at(r5, kWave - 1)};
#pragma unroll
  for (int i = 0; i < kGuPairs; ++i)
    if (i < np) swiglu_push_uniform<FAST>(store, batch, lane, g[i], u[i], p0 + i);
}

// Stage A over the wave's pairs [pb, pe) in blocks of kGuPairs; `a` holds
// the first block's loads.
template <bool FAST, class Store>
__device__ __forceinline__ void gu_stage(const DecodeLayer &L, const float *xv, float xsv, int lane,
                                         int pb, int pe, GuBlock &a, const Store &store) {
  const int negz = neg_zero_reg();
  SwigluBatch batch;
  for (int p = pb; p < pe; p += kGuPairs) {
    const int np = min(kGuPairs, pe - p);
    if (p != pb) load_gu(L, p, np, lane, a);
    gu_block<FAST>(a, xv, xsv, lane, p, np, store, batch, negz);
  }
  swiglu_flush<FAST>(store, batch);
}

// Stage B's slice of the down product: lane l of a wave covers row `row`
// (8 rows per wave, 8 lanes per row) and, in local pass j < NP, half l % 2
// of group 4 (NP x + j) + (l / 2) % 4: the 8 lanes of a row read the 128
// contiguous bytes of its 4 groups, and the XCD's NP passes are contiguous.
template <int NP>
__device__ __forceinline__ void load_down_slice(const DecodeLayer &L, int row, int x, int lane,
                                                DownRow<NP> &d) {
  const auto qr = buffer(L.dq, 2048u * NP * 1024u);
  const auto sr = buffer(L.ds, 2048u * NP * 128u);
  const auto br = buffer(L.db, 2048u * NP * 128u);
  const uint32_t vq = (uint32_t)row * (NP * 1024u) + 16u * (uint32_t)(lane & 7);
  const uint32_t vs = (uint32_t)row * (NP * 128u) + 4u * (uint32_t)((lane >> 1) & 3);
  const uint32_t n0 = (uint32_t)(NP * x);
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    d.cw[j] = load_codes(qr, vq, 128u * (n0 + j));
    d.sv[j] = load_f32(sr, vs, 16u * (n0 + j));
    d.bv[j] = load_f32(br, vs, 16u * (n0 + j));
  }
}

// The slice's sums: for each local pass j, T over the row's 4 group terms
// (the lane pairs of the row's 8 lanes: xor 2 within quads, then the mirror
// within 8 lanes), a node of the balanced tree over the 32 groups of the
// pass holding them; every lane of the row ends with it.  m (local group 4 j + g: values
// [256 j + 64 g, +64)) and its group sums are in LDS.
template <int NP, bool FAST>
__device__ __forceinline__ void down_slice(const Lds<NP> &S, int lane, const DownRow<NP> &d,
                                           float *sj) {
  const bool odd = lane & 1;
  const int g = (lane >> 1) & 3;
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    float xv[32];
    load_x_values(S.x + (8 * j + (lane & 7)) * kChunkStride, true, xv);
    const float xsv = S.xs[4 * j + g];
    float t = group_term<FAST>(d.cw[j], xv, d.sv[j], d.bv[j], xsv, true, odd);
    t = t + dpp<kDppQuadXor2>(t);
    sj[j] = t + dpp<kDppRowHalfMirror>(t);
    issue_order();  // one pass's activations in registers at a time
  }
}

// A row's value from its pass sums v[0..NP): the -0-padded balanced tree
// over the passes (the canonical tree over the row's NP * 32 group terms).
template <int NP>
__device__ __forceinline__ float combine_passes(const float *p) {
  constexpr int PP = NP == 1 ? 1 : NP == 2 ? 2 : 4;
  float v[PP];
#pragma unroll
  for (int i = 0; i < PP; ++i) v[i] = i < NP ? p[i] : kNegZero;
#pragma unroll
  for (int w = 1; w < PP; w *= 2)
#pragma unroll
    for (int i = 0; i < PP; i += 2 * w) v[i] = v[i] + v[i + w];
  return v[0];
}

// Stage B: the wave's down row from `d` and the activations in LDS: T over
// each pass's 32 group terms, then the -0-padded balanced tree over the
// passes (T over all groups); valid in lane 63.
template <int NP, bool FAST>
__device__ __forceinline__ float down_row(const Lds<NP> &S, int lane, const DownRow<NP> &d) {
  constexpr int PP = NP == 1 ? 1 : NP == 2 ? 2 : 4;
  const int negz = neg_zero_reg();
  const bool odd = lane & 1;
  float v[PP];
#pragma unroll
  for (int p = 0; p < PP; ++p) {
    if (p < NP) {
      float xv[32];
      load_x_values(S.x + (p * 64 + lane) * kChunkStride, true, xv);
      const float xsv = S.xs[p * 32 + (lane >> 1)];
      v[p] = wave_sum_lane63(group_term<FAST>(d.cw[p], xv, d.sv[p], d.bv[p], xsv, true, odd),
                             negz);
      issue_order();  // one pass's activations in registers at a time
    } else {
      v[p] = kNegZero;
    }
  }
#pragma unroll
  for (int w = 1; w < PP; w *= 2)
#pragma unroll
    for (int i = 0; i < PP; i += 2 * w) v[i] = v[i] + v[i + w];
  return v[0];
}


// ---------------------------------------------------------------------------
// The head inside the persistent launch: blocks of 4 rows of the tied
// embedding matrix (2048 columns), summed with the head kernel's group
// terms and four-row tree (q4mv_device.h), so the same bits.
// ---------------------------------------------------------------------------
constexpr int kHeadR = 4;

struct HeadBlock {
  u32x4 cw[kHeadR];
  float sv[kHeadR], bv[kHeadR];
};

// Rows [4 blk, 4 blk + 4) of the head that exist; a block past the last row
// reads a zero-byte buffer (no memory access, zeros).
__device__ __forceinline__ void head_load(const DecodeArgs &A, int blk, int lane, HeadBlock &b) {
  const long long r0 = (long long)kHeadR * blk;
  const long long left = (long long)A.vocab - r0;
  const int nrows = left <= 0 ? 0 : (left < kHeadR ? (int)left : kHeadR);
  const size_t r = nrows > 0 ? (size_t)r0 : 0;
  const auto qr = buffer(A.eq + r * 256, nrows * 1024);
  const auto sr = buffer(A.es + r * 32, nrows * 128);
  const auto br = buffer(A.eb + r * 32, nrows * 128);
#pragma unroll
  for (int j = 0; j < kHeadR; ++j) {
    b.cw[j] = load_codes(qr, 16u * lane, j * 1024);
    b.sv[j] = load_f32(sr, 4u * (lane >> 1), j * 128);
    b.bv[j] = load_f32(br, 4u * (lane >> 1), j * 128);
  }
}

// The same rows into the first four rows of a gate/up block (whose
// registers are free after the last layer's gate/up products), and back.
__device__ __forceinline__ void head_load_into(const DecodeArgs &A, int blk, int lane,
                                               GuBlock &a) {
  HeadBlock b;
  head_load(A, blk, lane, b);
#pragma unroll
  for (int j = 0; j < kHeadR; ++j) {
    a.cw[j] = b.cw[j];
    a.sv[j] = b.sv[j];
    a.bv[j] = b.bv[j];
  }
}

__device__ __forceinline__ void head_from(const GuBlock &a, HeadBlock &b) {
  static_assert(kGuR >= kHeadR, "a head block fits in a gate/up block");
#pragma unroll
  for (int j = 0; j < kHeadR; ++j) {
    b.cw[j] = a.cw[j];
    b.sv[j] = a.sv[j];
    b.bv[j] = a.bv[j];
  }
}

// Greedy pick over the rows a lane has stored (rows in increasing order).
struct HeadMax {
  float value = 0.0f;
  int index = -1;  // -1: no row yet
  bool nan = false;
  __device__ unsigned long long key() const {
    if (nan) return ops::kNanKey;
    return index < 0 ? 0ull : ops::argmax_key(value, index);
  }
};

// Block blk held in b: the four rows' sums (row j in lanes [16 j, 16 j +
// 16), as in the head kernel), stored to logits and folded into the lane's
// running maximum (holder lanes 15, 31, 47, 63).
template <bool FAST>
__device__ __forceinline__ void head_block(const DecodeArgs &A, const float *xv, float xsv,
                                           int lane, int blk, const HeadBlock &b, HeadMax &best) {
  const long long r0 = (long long)kHeadR * blk;
  if (r0 >= A.vocab) return;  // wave-uniform
  const int nrows = A.vocab - r0 < kHeadR ? (int)(A.vocab - r0) : kHeadR;
  const bool odd = lane & 1;
  float gt[kHeadR];
#pragma unroll
  for (int j = 0; j < kHeadR; ++j)
    gt[j] = group_term<FAST>(b.cw[j], xv, b.sv[j], b.bv[j], xsv, true, odd);
  const float v = quad_row_sums(gt[0], gt[1], gt[2], gt[3]);
  const int j = lane >> 4;
  if ((lane & 15) == 15 && j < nrows) {
    const int r = (int)r0 + j;
    A.logits[r] = v;
    // strictly greater keeps the lowest index of equal values (-0 == +0)
    const bool gt_ = (v > best.value) || best.index < 0;
    best.value = gt_ ? v : best.value;
    best.index = gt_ ? r : best.index;
    best.nan |= v != v;
  }
}

// The wave's head blocks first, first + stride, ... (nblk of them), three
// in registers at a time: b0 and b1 hold the loads of the first two on
// entry; each block's loads go out two blocks ahead.  (Two blocks summed
// together for more independent work per wave measured slower: 0.3694
// against 0.3664 ms per token.)
template <bool FAST>
__device__ __forceinline__ void head_rows(const DecodeArgs &A, const float *xv, float xsv,
                                          int lane, int first, int stride, int nblk,
                                          HeadBlock &b0, HeadBlock &b1, HeadMax &best) {
  HeadBlock b2;
#pragma unroll 1
  for (int k = 0; k < nblk; k += 3) {
    head_load(A, first + (k + 2) * stride, lane, b2);
    head_block<FAST>(A, xv, xsv, lane, first + k * stride, b0, best);
    head_load(A, first + (k + 3) * stride, lane, b0);
    if (k + 1 < nblk) head_block<FAST>(A, xv, xsv, lane, first + (k + 1) * stride, b1, best);
    head_load(A, first + (k + 4) * stride, lane, b1);
    if (k + 2 < nblk) head_block<FAST>(A, xv, xsv, lane, first + (k + 2) * stride, b2, best);
  }
}

}  // namespace decode
}  // namespace q4
