// Device-scope words for handing values between the workgroups of one
// launch without fences: a 64-bit word holds a float's bits and a 32-bit
// tag naming the call and stage that produced it, stored and loaded with
// device-scope (agent) atomics, i.e. with the sc1 cache policy that writes
// through to the memory side where device-scope loads read it.  A consumer
// polls until the tag is the expected one: the wait and the data arrive in
// the same load, and no cache write-back or invalidation is needed.  Every
// wait is bounded by a number of wall-clock ticks; one that runs out sets an
// error word that the other waits also give up on.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

__device__ __forceinline__ uint32_t load_word(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_word(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_tagged(uint64_t *p, float v, uint32_t tag) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// Polls the N tagged words p[STRIDE k] (k < N) until each carries `tag`;
// their floats go to v.  False when the wait ran out (the error word is
// then set) or another wait did.  (With STRIDE the wave's width, a wave's
// load covers 64 consecutive words: a few cache lines per load instead of
// up to one per lane.)
template <int N, int STRIDE = 1>
__device__ __forceinline__ bool poll_tagged(const uint64_t *p, uint32_t tag, float *v,
                                            uint32_t *err, long long spin_ticks) {
  const long long t0 = wall_clock64();
  for (int it = 1;; ++it) {
    bool ready = true;
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const uint64_t w =
          __hip_atomic_load(p + STRIDE * k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      v[k] = __uint_as_float((uint32_t)w);
      ready &= (uint32_t)(w >> 32) == tag;
    }
    if (ready) return true;
    if ((it & 63) == 0 && load_word(err) != 0) return false;
    if (wall_clock64() - t0 > spin_ticks) {
      store_word(err, 1u);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Polls the N tagged words p[off[k]] until each carries `tag`, as
// poll_tagged does.
template <int N>
__device__ __forceinline__ bool poll_tagged_at(const uint64_t *p, const int (&off)[N],
                                               uint32_t tag, float *v, uint32_t *err,
                                               long long spin_ticks) {
  const long long t0 = wall_clock64();
  for (int it = 1;; ++it) {
    bool ready = true;
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const uint64_t w =
          __hip_atomic_load(p + off[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      v[k] = __uint_as_float((uint32_t)w);
      ready &= (uint32_t)(w >> 32) == tag;
    }
    if (ready) return true;
    if ((it & 63) == 0 && load_word(err) != 0) return false;
    if (wall_clock64() - t0 > spin_ticks) {
      store_word(err, 1u);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// A hand-off through the L2 of each XCD.  The producers' words (device
// scope) are read by one workgroup per XCD only, which stores them again
// into its XCD's copy; the other workgroups of that XCD poll that copy.
// Both use non-temporal loads and stores: these go past the compute unit's
// own cache to the L2 that the XCD's compute units share (a workgroup-scope
// load may be served by the unit's own cache, and a poll with it would not
// see another unit's store).  Measured between two workgroups of one XCD:
// a round trip of 0.55 us this way against 0.99 us at device scope (1.37
// us across XCDs); across XCDs these words are not seen at all, so each
// XCD has its copy.  The device-scope traffic of a hand-off that every
// workgroup reads falls from one read per workgroup to one per XCD.

// Index of the XCD the calling wave runs on.
__device__ __forceinline__ uint32_t xcd_id() {
  // HW_REG_XCC_ID (register 20), bits 0..3
  return __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11));
}

// Relays word i of the producers' copy `far` into this XCD's copy `near`
// once it carries `tag`.  False when the wait ran out or another did.
__device__ __forceinline__ bool relay_word(const uint64_t *far, uint64_t *near, int i, uint32_t tag,
                                           uint32_t *err, long long spin_ticks) {
  float v;
  if (!poll_tagged<1>(far + i, tag, &v, err, spin_ticks)) return false;
  __builtin_nontemporal_store(((uint64_t)tag << 32) | __float_as_uint(v), near + i);
  return true;
}

// Polls the N words near[STRIDE k] (this XCD's copy) until each carries
// `tag`, for at most near_ticks, then the same words at far (the
// producers' copy) as poll_tagged does; with use_near false (or once
// near_ticks has run out, which clears it), only far.  A relay that never
// comes (a workgroup not where the relay expects it) costs time, not
// correctness: both copies hold the same values under the same tag.
template <int N, int STRIDE = 1>
__device__ __forceinline__ bool poll_tagged_near(const uint64_t *near, const uint64_t *far,
                                                 uint32_t tag, float *v, uint32_t *err,
                                                 bool &use_near, long long near_ticks,
                                                 long long spin_ticks) {
  if (use_near) {
    const long long t0 = wall_clock64();
    for (int it = 1;; ++it) {
      bool ready = true;
#pragma unroll
      for (int k = 0; k < N; ++k) {
        const uint64_t w = __builtin_nontemporal_load(near + STRIDE * k);
        v[k] = __uint_as_float((uint32_t)w);
        ready &= (uint32_t)(w >> 32) == tag;
      }
      if (ready) return true;
      if ((it & 63) == 0 && load_word(err) != 0) return false;
      if (wall_clock64() - t0 > near_ticks) {
        use_near = false;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  return poll_tagged<N, STRIDE>(far, tag, v, err, spin_ticks);
}

// Polls `groups` (at most M) groups of N consecutive words, group g at
// p + g * stride, in one round each time, until every word carries `tag`;
// v[N g + k] gets word k of group g, and -0 for the groups from `groups`
// on.
template <int N, int M>
__device__ __forceinline__ bool poll_tagged_groups(const uint64_t *p, size_t stride, int groups,
                                                   uint32_t tag, float *v, uint32_t *err,
                                                   long long spin_ticks) {
  const long long t0 = wall_clock64();
  for (int it = 1;; ++it) {
    bool ready = true;
#pragma unroll
    for (int g = 0; g < M; ++g) {
#pragma unroll
      for (int k = 0; k < N; ++k) {
        v[N * g + k] = -0.0f;
        if (g < groups) {
          const uint64_t w = __hip_atomic_load(p + (size_t)g * stride + k, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
          v[N * g + k] = __uint_as_float((uint32_t)w);
          ready &= (uint32_t)(w >> 32) == tag;
        }
      }
    }
    if (ready) return true;
    if ((it & 63) == 0 && load_word(err) != 0) return false;
    if (wall_clock64() - t0 > spin_ticks) {
      store_word(err, 1u);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// The first half of a long wait: lanes [0, n) of the calling wave poll the
// n consecutive words at p until each carries `tag` (their values are not
// kept); the caller's workgroup barrier holds its other waves meanwhile.  A
// waiting workgroup then sends one narrow load per round instead of one
// per thread, which leaves the memory side to the workgroups still at
// work.  It proves nothing about other words: the caller still polls every
// word it takes, which by then has mostly arrived.
__device__ __forceinline__ bool await_words(const uint64_t *p, int n, uint32_t tag, uint32_t *err,
                                            long long spin_ticks) {
  const int lane = threadIdx.x & 63;
  float v;
  return lane >= n || poll_tagged<1>(p + lane, tag, &v, err, spin_ticks);
}

}  // namespace q4
