// Device helpers shared by the q4mv kernels (gfx950, wave64).
//
// Compiled with -ffp-contract=off: every float expression is the exact
// sequence of IEEE binary32 operations it spells.
//
// The fixed summation tree T(v[0..n)) splits at the largest power of two
// below n: the reading taken of the fixed order the pages name for q4mv's
// sums ("Metal: queued rmsq, swq, gdn and atq kernels and a 4-row q4mv, so a
// decode token is one command buffer with one wait" (#1440), Change, q4mv
// bullet).  T equals a balanced pairwise tree
// over the next power of two >= n whose missing leaves are -0.0 (x + -0.0 ==
// x for every x, including +-0), so a lane butterfly with -0.0 padding
// reproduces it for any n, and T over n leaves equals T over the sums of
// aligned blocks of any power-of-two size.  IEEE addition is commutative, so
// which lane of a butterfly pair adds which operand does not change a bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ops_device.h"
#include "q4mv_internal.h"

#pragma clang fp contract(off)

namespace q4 {
namespace dev {

constexpr int kWave = 64;
constexpr float kNegZero = -0.0f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// DPP controls of the gfx9 family.
constexpr int kDppQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <- 7-i within 8 lanes
constexpr int kDppRowMirror = 0x140;      // lane i <- 15-i within 16 lanes
constexpr int kDppRowBcast15 = 0x142;     // lane 15 of row k -> row k+1
constexpr int kDppRowBcast31 = 0x143;     // lane 31 -> rows 2 and 3

// Buffer resource (gfx9 format): raw byte addressing, no stride; loads past
// num_records bytes return zero.
constexpr int kBufferFlags = 0x00020000;
// Cache policy of the streaming code loads: non-temporal.
constexpr int kAuxNonTemporal = 2;

// Index of the wave in its workgroup, as a wave-uniform (scalar) value: the
// compiler cannot prove threadIdx.x / 64 uniform by itself, and addresses
// built from a value it thinks divergent turn every buffer load into a loop.
__device__ __forceinline__ int wave_index() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// -0.0 in a register the compiler cannot rematerialise (it would rebuild
// the constant with one instruction at every use).
__device__ __forceinline__ int neg_zero_reg() {
  int v = __float_as_int(kNegZero);
  asm volatile("" : "+v"(v));
  return v;
}

// DPP move limited to the rows in ROW_MASK; lanes of the other rows read
// `old` (-0.0, the additive identity of the tree).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_rows(float v, int old) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(old, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}

// Sum of the group terms of one row segment of LPR lanes (every group term
// held identically by a lane pair).  All lanes of the segment must run it.
// After each step every aligned block of 2^k lanes holds one value, so a
// mirror within 8 (16) lanes pairs blocks 4 (8) lanes apart, like xor 4 (8).
template <int LPR>
__device__ __forceinline__ float segment_sum(float t) {
  if constexpr (LPR >= 4) t = t + dpp<kDppQuadXor2>(t);
  if constexpr (LPR >= 8) t = t + dpp<kDppRowHalfMirror>(t);
  if constexpr (LPR >= 16) t = t + dpp<kDppRowMirror>(t);
  if constexpr (LPR >= 32) {  // the 16-lane rows are uniform: rows 0/1, 2/3 (xor 16)
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t), false,
                                                    false);
    t = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
  if constexpr (LPR >= 64) {  // halves 0/1 (xor 32)
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false,
                                                    false);
    t = __uint_as_float(q[0]) + __uint_as_float(q[1]);
  }
  return t;
}

// Sum over the 32 lane pairs of a wave, valid in lane 63 only.  The first
// three steps leave each 16-lane row R_k uniform; row_bcast15 adds R0 into
// row 1 and R2 into row 3; row_bcast31 adds (R0+R1) into row 3:
// ((R0+R1)+(R2+R3)), the balanced tree over the four rows.
// `negz` holds -0.0 (neg_zero_reg()).
__device__ __forceinline__ float wave_sum_lane63(float t, int negz) {
  t = t + dpp<kDppQuadXor2>(t);
  t = t + dpp<kDppRowHalfMirror>(t);
  t = t + dpp<kDppRowMirror>(t);
  t = t + dpp_rows<kDppRowBcast15, 0xA>(t, negz);
  t = t + dpp_rows<kDppRowBcast31, 0xC>(t, negz);
  return t;
}

// The sums of four rows at once, each row's group terms held as for
// wave_sum_lane63 (lane pairs identical).  Within each 16-lane row the
// steps xor 2 and the two mirrors leave R_jk, the sum over row k's lanes,
// in every lane of row k of register j; the gfx950 lane swaps then combine
// the 16-lane rows across the four registers: v_permlane16_swap of
// registers (0, 1) gives [R00, R10, R02, R12] and [R01, R11, R03, R13],
// whose sum holds R_j0 + R_j1 and R_j2 + R_j3; v_permlane32_swap of the
// two sums gathers each row's two halves into one 16-lane row.  Row j's
// total, ((R_j0 + R_j1) + (R_j2 + R_j3)) as in wave_sum_lane63, ends in
// lanes [16 j, 16 j + 16).  Three swaps and three adds replace the eight
// broadcast instructions per row of wave_sum_lane63.
__device__ __forceinline__ float swap_sum16(float a, float b) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

__device__ __forceinline__ float quad_row_sums(float t0, float t1, float t2, float t3) {
  float t[4] = {t0, t1, t2, t3};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    t[j] = t[j] + dpp<kDppQuadXor2>(t[j]);
    t[j] = t[j] + dpp<kDppRowHalfMirror>(t[j]);
    t[j] = t[j] + dpp<kDppRowMirror>(t[j]);
  }
  const float x = swap_sum16(t[0], t[1]);
  const float y = swap_sum16(t[2], t[3]);
  const auto z = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false,
                                                  false);
  return __uint_as_float(z[0]) + __uint_as_float(z[1]);
}

// ---------------------------------------------------------------------------
// Codes -> products.  Word bits 4k..4k+3 hold code k; p_k = code_k * x_k.
// ---------------------------------------------------------------------------

// Byte k of v (0..255) as binary32, exactly: v_cvt_f32_ubyte0..3.  These
// conversions issue at the rate of a plain add and let two waves of a SIMD
// issue together, unlike v_cvt_pk_f32_fp8 (which holds the SIMD's VALU for
// about two issue cycles and issues alone), and unlike a bit-field extract
// followed by ubyte0 (two VOP3-class instructions per code).
template <int K>
__device__ __forceinline__ float byte_f32(uint32_t v) {
  float f;
  if constexpr (K == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(f) : "v"(v));
  if constexpr (K == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(f) : "v"(v));
  if constexpr (K == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(f) : "v"(v));
  if constexpr (K == 3) asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(f) : "v"(v));
  return f;
}

// Plain decode: every code converted to binary32 exactly.
__device__ __forceinline__ float word_tree(uint32_t w, const float *xk) {
  const uint32_t lo = w & 0x0F0F0F0Fu;         // codes 0, 2, 4, 6
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;  // codes 1, 3, 5, 7
  const float p0 = byte_f32<0>(lo) * xk[0];
  const float p1 = byte_f32<0>(hi) * xk[1];
  const float p2 = byte_f32<1>(lo) * xk[2];
  const float p3 = byte_f32<1>(hi) * xk[3];
  const float p4 = byte_f32<2>(lo) * xk[4];
  const float p5 = byte_f32<2>(hi) * xk[5];
  const float p6 = byte_f32<3>(lo) * xk[6];
  const float p7 = byte_f32<3>(hi) * xk[7];
  return ((p0 + p1) + (p2 + p3)) + ((p4 + p5) + (p6 + p7));
}

// Tree of one lane's 32-code chunk (four words, contiguous columns).
__device__ __forceinline__ float chunk_tree(u32x4 c, const float *xv) {
  return (word_tree(c.x, xv) + word_tree(c.y, xv + 8)) +
         (word_tree(c.z, xv + 16) + word_tree(c.w, xv + 24));
}

// Q4_FAST: the chunk's dot product accumulated with fused multiply-adds.
__device__ __forceinline__ float chunk_dot_fast(u32x4 c, const float *xv) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  float acc = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t lo = w[k] & 0x0F0F0F0Fu;
    const uint32_t hi = (w[k] >> 4) & 0x0F0F0F0Fu;
    const float *xk = xv + 8 * k;
    acc = fmaf(byte_f32<0>(lo), xk[0], acc);
    acc = fmaf(byte_f32<0>(hi), xk[1], acc);
    acc = fmaf(byte_f32<1>(lo), xk[2], acc);
    acc = fmaf(byte_f32<1>(hi), xk[3], acc);
    acc = fmaf(byte_f32<2>(lo), xk[4], acc);
    acc = fmaf(byte_f32<2>(hi), xk[5], acc);
    acc = fmaf(byte_f32<3>(lo), xk[6], acc);
    acc = fmaf(byte_f32<3>(hi), xk[7], acc);
  }
  return acc;
}

// Group term of a lane (the lane pair 2g, 2g+1 holds group g):
//   fixed: d = T(pair's chunk trees); t = (s*d) + (b*xs); both lanes of the
//          pair end with the same t
//   fast : each lane adds s*dot (+ b*xs on the even lane), then the pair is
//          summed, so both lanes again hold the group's term.
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
__device__ __forceinline__ void select_product(const ProdGroup &grp, Prod &P, int &lw, int &nwg) {
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

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           kBufferFlags);
}

__device__ __forceinline__ u32x4 load_codes(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                            uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kAuxNonTemporal);
}

__device__ __forceinline__ float load_f32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// Group sum of the lane pair's 64 activations: T over the lane's 32
// (balanced) plus the partner's 32.
__device__ __forceinline__ float pair_group_sum(const float *xv) {
  const float L =
      (ops::tree8(xv) + ops::tree8(xv + 8)) + (ops::tree8(xv + 16) + ops::tree8(xv + 24));
  return L + dpp<kDppQuadXor1>(L);
}

__device__ __forceinline__ void load_x_values(const float *x, bool active, float *xv) {
  if (active) {
    const float4 *xp = reinterpret_cast<const float4 *>(x);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float4 v = xp[k];
      xv[4 * k + 0] = v.x;
      xv[4 * k + 1] = v.y;
      xv[4 * k + 2] = v.z;
      xv[4 * k + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 32; ++k) xv[k] = 0.0f;
  }
}

// (gate, up) pairs waiting for their SwiGLU: lane k of a wave holds pair k
// of the current batch.  The pairs come out of the row sums one or two per
// block, but the SwiGLU costs the same instructions for 1 pair as for 64, so
// a wave evaluates them in batches of up to 64.
struct SwigluBatch {
  float gate = 0.0f, up = 0.0f;
  int out = -1;  // index into m, -1 for an empty slot
  int count = 0; // pairs held (wave-uniform)
};

// `store(i, v)` writes output i (plain or tagged stores, by the caller).
template <bool FAST, class Store>
__device__ __forceinline__ void swiglu_flush(const Store &store, SwigluBatch &b) {
  if (b.count == 0) return;
  if (b.out >= 0) store(b.out, ops::swiglu_value<FAST>(b.gate, b.up));
  b.out = -1;
  b.count = 0;
}

// Appends the pair (gate, up) for m[out], both held by lane 63, to slot
// b.count (lane b.count takes them).
template <bool FAST, class Store>
__device__ __forceinline__ void swiglu_push(const Store &store, SwigluBatch &b, int lane,
                                            float gate, float up, int out) {
  const float g = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gate), kWave - 1));
  const float u = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(up), kWave - 1));
  const bool mine = lane == b.count;
  b.gate = mine ? g : b.gate;
  b.up = mine ? u : b.up;
  b.out = mine ? out : b.out;
  b.count = b.count + 1;
  if (b.count == kWave) swiglu_flush<FAST>(store, b);
}

}  // namespace dev
}  // namespace q4
