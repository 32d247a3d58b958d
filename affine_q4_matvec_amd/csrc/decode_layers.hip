// The MLP layers of one decode step as a single persistent launch (gfx950).
//
// A decode token runs rmsq, the gate/up product, swq and the down product
// of every layer in order ("Metal: queued rmsq, swq, gdn and atq kernels and
// a 4-row q4mv, so a decode token is one command buffer with one wait"
// (#1440), Change and Verification).  Launched one kernel per stage, each
// stage pays a launch and the cold start of its loads; here one grid of
// resident workgroups (one per compute unit) runs every stage:
//
//   h = embed(tok)                          (8 columns per thread, from the weights)
//   per layer:  u = rmsq(h, wn)              (once per workgroup, into LDS)
//               m = SwiGLU([gate; up] u)     (rows in (gate, up) pairs)
//               h = h + down m               (by slices, see below)
//
// Dataflow instead of grid barriers.  Every value one workgroup hands to
// another is stored as a 64-bit word: the float's bits and a 32-bit tag
// naming the call and the stage that produced it.  A consumer polls the
// words it needs until each carries the expected tag: the wait and the data
// arrive in the same load, and no cache write-back, invalidation or barrier
// is needed.  (On this device a grid barrier built on the memory model's
// agent-scope fences costs about 10 us, a fence-free one about 4 us.)  Two
// kinds of copies: a device-scope one (sc1 stores and loads: written
// through to the memory side, where device-scope loads read it), and one
// per XCD, written and polled with non-temporal stores and loads, which the
// XCD's shared L2 serves (a round trip between two workgroups of one XCD:
// 0.55 us, against 0.99 us at device scope; across XCDs these words are not
// seen).  A wait that its XCD's copy does not serve within a bounded time
// turns to the device-scope copy, so a workgroup not on the XCD the dealing
// assumes costs time, not correctness.
//
// The work is dealt by XCD.  The grid is 8 XCDs x 32 workgroups (the
// dispatcher deals them round robin: workgroups w = x, x + 8, ... share one
// XCD); for x = w mod 8, k = w / 8:
//   - stage A: wave 8 k + i of XCD x takes (gate, up) pairs [256 NP x +
//     NP (8 k + i), + NP), so XCD x produces m[256 NP x, + 256 NP): the
//     down product's column groups [4 NP x, 4 NP x + 4 NP);
//   - m of those groups goes through the XCD's copy to its workgroups;
//   - stage B: workgroup w sums rows [64 k, 64 k + 64) over each 4 of its
//     XCD's groups (node NP x + j of the row's 8 NP nodes: the balanced
//     tree over the 32 group terms of pass n / 8 has node n % 8 of that
//     pass as a subtree) and publishes those sums (device scope);
//   - the owner of row r (workgroup r / 8, threads 0..7) gathers the 8
//     node sums of each pass in order, forms the passes' tree, adds the
//     residual and publishes h[r] (device scope);
//   - on each XCD, each workgroup relays a 64-value slice of h into the
//     XCD's copy, which the XCD's workgroups read for the next rmsq.
// Every workgroup used to read all of m at device scope (12.6 MB across
// the GPU per poll round, 0.3452 ms per token); now the device-scope
// polls of a layer are the sums (0.4 MB) and h's slices (0.13 MB): 0.3389.
// Each XCD's groups are contiguous, so its share of a down row's codes is
// whole 128-byte lines and its scales and biases span 1 or 2 lines; with 4
// groups of every pass instead, every XCD read 16 bytes of every line of
// them, and the 8 L2s fetched 1.5x the weights' bytes.
//
// Tags: call c (each workgroup counts its calls in a word of its own in the
// workspace; the grid has the same size in every call, so after a
// completed call all counters agree) gives m of layer l and the down sums
// of layer l the tag 64 c + 2 l + 1 and h after layer l the tag 64 c +
// 2 l + 2 (at most 32 layers).  m and h alternate between two buffers each
// by layer; the sums need one.  No word is overwritten while a reader may
// still need it: writing the sums of layer l + 1 needs h after layer l
// complete, hence every owner done with the sums of layer l; writing m of
// layer l + 2 needs h after layer l + 1 complete, which needs every
// workgroup's sums of layer l + 1, which follow its reads of m of layer l
// + 1 and, before them, of layer l; likewise for h.
//
// Every wait is bounded by spin_ticks of the wall clock; a wait that runs
// out sets the error word, and every workgroup leaves at its next wait, so
// the grid always drains.  On an otherwise idle device every workgroup of
// the launch is resident.
//
// The weights of a stage do not depend on the previous one, so every wave
// loads its next stage's rows ahead: the down slice right after the wait
// for h, the next layer's gate/up rows as early as they can go.  A wave's
// loads complete in issue order for its wait counter, so a poll issued
// after a prefetch also waits for the prefetch (for the gate/up rows, about
// 16 MB across the GPU).  Hence two kinds of waves: waves 0-3 poll h (at a
// layer's start) and load their next gate/up rows right after their gate/up
// products; waves 4-7 poll m (in stage B) and load theirs only once those
// polls are done.  No poll then waits behind a fresh prefetch.
//
// Every value is computed by the same code as the per-stage kernels (rmsq
// and SwiGLU from ops_device.h, group terms and row trees from
// q4mv_device.h), in the same trees, so the result has the bits of the
// unfused chain.
#include "decode_device.h"
#include "tagged_device.h"

#pragma clang fp contract(off)

namespace q4 {
namespace {

using namespace dev;
using namespace decode;

// Threads of the workgroup that may poll m in stage B (the last four
// waves); 64 NP of them poll 4 values each (the XCD's 256 NP values).
constexpr int kPollThreads = 256;

// e[c] of the embedding row tk (the embed kernel's arithmetic; NaN for a
// token outside the vocabulary).
__device__ __forceinline__ float embed_value(const DecodeArgs &A, int tk, int c) {
  if (tk < 0 || tk >= A.vocab) return __builtin_nanf("");
  const uint32_t word = A.eq[(size_t)tk * 256 + (c >> 3)];
  const float code = (float)((word >> (4 * (c & 7))) & 15u);
  const float sq = A.es[(size_t)tk * 32 + (c >> 6)] * code;
  return sq + A.eb[(size_t)tk * 32 + (c >> 6)];
}

template <bool FAST, int NP>
__global__ __launch_bounds__(kThreads) void decode_layers_kernel(DecodeArgs A) {
  __shared__ Lds<NP> S;
  const int nwg = gridDim.x;
  const int wg = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = wave_index();
  uint32_t *err = A.ctl + kDecodeErrorWord;
  if (__syncthreads_or(load_word(err) != 0)) return;
  const uint32_t call = load_word(A.ctl + wg);
  const uint32_t tag0 = call << 6;

  // wave gw = wave * nwg + wg (consecutive gw on different compute units)
  // takes the head's blocks gw, gw + stride, ...
  const int gw = wave * nwg + wg;
  const int stride = kWaves * nwg;
  const bool mine = 8 * t < kCols;  // threads 0..255 own 8 values of h each
  // the (gate, up) pairs and the down groups by XCD (the grid has 8 x 32
  // workgroups): XCD x = wg mod 8, k = wg / 8; wave 8 k + wave of XCD x
  // takes pairs [pb, pb + NP); the workgroup's down slice is rows [64 k,
  // 64 k + 64) of groups [4 NP x, 4 NP x + 4 NP); it owns rows [8 wg, 8 wg
  // + 8) (threads 0..7: the residual, the pass sums' gather, h)
  const int x = wg % kDecodeXcds, k = wg / kDecodeXcds;
  const int pb = 256 * NP * x + NP * (8 * k + wave);
  const int drow = 64 * k + 8 * wave + lane / 8;
  const bool owner = t < 8;
  const int orow = 8 * wg + t;
  const int tk = *A.tok;
  // h goes through the L2 of each XCD: workgroup wg relays slice wg / 8 of
  // h from the device-scope copy (kDecodeXcds) into its XCD's copy and reads
  // that copy.  (The earlier dealing relayed m the same way, from producers
  // on every XCD: 0.381 against 0.366 ms per token without; forming h from
  // the sums on every XCD instead of the owners: 0.374 against 0.340.)
  const uint32_t xcd = xcd_id();
  const int nslot = nwg / kDecodeXcds;
  const bool relay = nwg % kDecodeXcds == 0 && xcd < (uint32_t)kDecodeXcds && kCols <= kWave * nslot;
  const int slot = wg / kDecodeXcds;
  const int near_copy = relay ? (int)xcd : 0;
  bool use_near = relay;
  // m through the XCD's L2.  The dispatcher deals the grid to the XCDs
  // round robin but not always from the first XCD (one launch in a long run
  // started at XCD 7: every workgroup on XCD (w + 7) mod 8), so the check
  // is not xcd == wg mod 8: the workgroups w = x, x + 8, ... still share one
  // XCD, which is all the producers and readers of copy x need.  If they do
  // not, the readers' waits turn to the device-scope copy after near_ticks.
  const bool local_m = relay;
  bool use_near_m = local_m;
  // h after layer l - 1 (tag 64 c + 2 l): the relay of this workgroup's
  // slice (wave 0); then every thread polls words t + 512 k (each wave's
  // load is 64 consecutive words, a few cache lines; polling 8 consecutive
  // words per thread made each load touch a line per lane) into S.x, and
  // after a barrier threads 0..255 take their 8 consecutive values into h8.
  // Every thread of the workgroup calls it; S.x must be free.
  const auto poll_h = [&](int l, float *h8) {
    const uint32_t th = tag0 + 2 * l;
    uint64_t *hb = A.hq + (size_t)((l - 1) & 1) * kDecodeSlots * kCols;
    const uint64_t *far = hb + kDecodeXcds * kCols;
    bool ok = true;
    if (relay && wave == 0) {
      const int i = slot * kCols / nslot + lane;
      if (i < (slot + 1) * kCols / nslot)
        ok = relay_word(far, hb + near_copy * kCols, i, th, err, A.spin_ticks);
    }
    static_assert(kCols == 4 * kThreads, "4 words of h per thread");
    float hv[4];
    ok = ok && poll_tagged_near<4, kThreads>(hb + near_copy * kCols + t, far + t, th, hv, err,
                                             use_near, A.near_ticks, A.spin_ticks);
#pragma unroll
    for (int k = 0; k < 4; ++k) S.x[t + kThreads * k] = hv[k];
    __syncthreads();
    if (mine) {
      const float4 *src = reinterpret_cast<const float4 *>(S.x + 8 * t);
      const float4 a0 = src[0], a1 = src[1];
      h8[0] = a0.x; h8[1] = a0.y; h8[2] = a0.z; h8[3] = a0.w;
      h8[4] = a1.x; h8[5] = a1.y; h8[6] = a1.z; h8[7] = a1.w;
    }
    return ok;
  };

  GuBlock a;
  DownRow<NP> d;
  load_gu(A.layer[0], pb, min(kGuPairs, NP), lane, a);
  // the head (q4_decode_token): blocks of 4 rows gw, gw + stride, ...; the
  // first is loaded during the last layer, into the registers of the gate/up
  // block (free by then: there is no next layer)
  const bool head = A.wf != nullptr;
  const int head_blocks = (A.vocab + kHeadR - 1) / kHeadR;
  const int head_nblk = gw < head_blocks ? (head_blocks - gw + stride - 1) / stride : 0;
  // the residual of an owned row: h before the layer
  float res = owner ? embed_value(A, tk, orow) : 0.0f;

  for (int l = 0; l < A.nlayers; ++l) {
    const DecodeLayer &L = A.layer[l];
    uint64_t *mq = A.mq + (size_t)(l & 1) * kDecodeSlots * kDecodeMaxInter;  // copy 0
    uint64_t *mfar = mq + (size_t)kDecodeXcds * kDecodeMaxInter;
    uint64_t *mnear = mq + (size_t)x * kDecodeMaxInter;

    // ---- stage A: x = rmsq(h, wn) over the workgroup (threads 0..255: 8
    // columns each); m = SwiGLU of the gate/up rows
    bool ok = true;
    float h8[8] = {}, w8[8] = {};  // (zero: not carried from layer to layer)
    if (mine) {
      const float4 *wp = reinterpret_cast<const float4 *>(L.wn + 8 * t);
      const float4 w0 = wp[0], w1 = wp[1];
      w8[0] = w0.x; w8[1] = w0.y; w8[2] = w0.z; w8[3] = w0.w;
      w8[4] = w1.x; w8[5] = w1.y; w8[6] = w1.z; w8[7] = w1.w;
    }
    if (l == 0) {
      // the embedding row of the token (the embed kernel's arithmetic)
      if (mine) {
        const bool valid = tk >= 0 && tk < A.vocab;
        const size_t er = valid ? (size_t)tk : 0;
        const float sg = valid ? A.es[er * 32 + (t >> 3)] : 0.0f;
        const float bg = valid ? A.eb[er * 32 + (t >> 3)] : 0.0f;
        const uint32_t word = valid ? A.eq[er * 256 + t] : 0u;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float sq = sg * (float)((word >> (4 * i)) & 15u);
          h8[i] = valid ? sq + bg : __builtin_nanf("");
        }
      }
    } else {
      // h after the previous layer, 8 values per thread
      ok = poll_h(l, h8);
    }
    issue_order();
    load_down_slice<NP>(L, drow, x, lane, d);
    {
      if (!workgroup_rmsq(S, h8, w8, A.eps, ok)) return;
      float xv[32];
      const float xsv = load_rmsq_x(S, lane, xv);
      const uint32_t tag = tag0 + 2 * l + 1;
      // m[i] to the XCD's copy (non-temporal: its L2) and the device-scope
      // one
      const auto store_m = [mfar, mnear, tag, local_m](int i, float v) {
        if (local_m)
          __builtin_nontemporal_store(((uint64_t)tag << 32) | __float_as_uint(v), mnear + i);
        store_tagged(mfar + i, v, tag);
      };
      gu_stage<FAST>(L, xv, xsv, lane, pb, pb + NP, a, store_m);
    }

    // the next layer's gate/up rows, for the waves that do not poll m (they
    // poll h at the next layer's start, long after these have landed)
    const bool poller = t >= kThreads - kPollThreads;
    if (!poller && l + 1 < A.nlayers)
      load_gu(A.layer[l + 1], pb, min(kGuPairs, NP), lane, a);
    if (!poller && l + 1 == A.nlayers && head) head_load_into(A, gw, lane, a);
    issue_order();
    const uint32_t tag_m = tag0 + 2 * l + 1;

    // ---- stage B: this XCD's m (its workgroup's 4 NP groups) and their
    // group sums into LDS; the slice's pass sums to the rows' owners; h =
    // h + down m for the owned rows.  Poller thread p < 64 NP takes local
    // values [4 p, 4 p + 4): m[256 NP x + 4 p ..], local group p / 16.  The
    // pollers are waves without fresh loads in
    // flight: a wave's loads complete in issue order for its wait counter,
    // so a poll behind a prefetch of the GPU's next gate/up rows would wait
    // for that prefetch to land.
    // the workgroup polls only once all its waves are done with stage A (the
    // values go to S.x, which stage A reads)
    if (t == 0) S.flag = 0u;
    __syncthreads();
    const int p = t - (kThreads - kPollThreads);
    const bool mpoll = poller && p < 64 * NP;  // wave-uniform
    if (poller) {
      if (mpoll) {
        const int lv = 4 * p;
        const int i = 256 * NP * x + lv;
        float v[4];
        if (!poll_tagged_near<4>(mnear + i, mfar + i, tag_m, v, err, use_near_m, A.near_ticks,
                                 A.spin_ticks))
          S.flag = 1u;
        // group sums: the balanced tree over the group's 64 values (4 per
        // lane, 16 lanes)
        float gs = (v[0] + v[1]) + (v[2] + v[3]);
        gs = ops::lane_sum8(gs);
        gs = gs + ops::dpp_move<0x140>(gs);  // row_mirror: xor 8 here
        if ((p & 15) == 0) S.xs[p >> 4] = gs;
        *reinterpret_cast<float4 *>(S.x + lv + 4 * (lv >> 5)) = make_float4(v[0], v[1], v[2], v[3]);
      }
      // this wave's gate/up rows of the next layer (or its first head
      // blocks after the last layer), now that its polls are done
      if (l + 1 < A.nlayers)
        load_gu(A.layer[l + 1], pb, min(kGuPairs, NP), lane, a);
      if (l + 1 == A.nlayers && head) head_load_into(A, gw, lane, a);
      issue_order();
    }
    __syncthreads();
    if (S.flag != 0u) return;
    {
      // the slice: the row's 4-group sums (nodes NP x + j of the row's 8 NP
      // nodes), to the row's owner
      float sj[NP];
      down_slice<NP, FAST>(S, lane, d, sj);
      if ((lane & 7) == 0)
#pragma unroll
        for (int j = 0; j < NP; ++j)
          store_tagged(A.pq + (size_t)drow * (8 * NP) + NP * x + j, sj[j], tag_m);
    }
    if (wave == 0) {
      // the owned rows' 64 NP node sums (rows [8 wg, 8 wg + 8) x 8 NP
      // nodes, contiguous): lane l polls words l + 64 i (coalesced) into
      // S.ownw; then thread t < 8 NP, for owned row 8 wg + t % 8 and pass
      // t / 8, reads the pass's 8 node sums in order (the balanced tree over
      // its 32 group terms).  One wave writes and reads S.ownw: its LDS
      // accesses are done in order.
      float pv[NP];
      const bool okp = poll_tagged<NP, kWave>(A.pq + (size_t)wg * (64 * NP) + lane, tag_m, pv,
                                               err, A.spin_ticks);
#pragma unroll
      for (int i = 0; i < NP; ++i) S.ownw[lane + kWave * i] = pv[i];
      issue_order();
      if (t < 8 * NP) {
        const float *q = S.ownw + (t & 7) * (8 * NP) + 8 * (t >> 3);
        float v8[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v8[k] = q[k];
        S.own[t] = ops::tree8(v8);
      }
      const bool all_ok = __all(okp);
      issue_order();  // the same wave reads them back below
      if (owner && all_ok) {
        float pj[NP];
#pragma unroll
        for (int jj = 0; jj < NP; ++jj) pj[jj] = S.own[t + 8 * jj];
        res = res + combine_passes<NP>(pj);
        // h to the producers' copy, from which each XCD relays it
        if (l + 1 < A.nlayers || head)
          store_tagged(A.hq + ((size_t)(l & 1) * kDecodeSlots + kDecodeXcds) * kCols + orow, res,
                       tag0 + 2 * l + 2);
        if (l + 1 == A.nlayers) A.h[orow] = res;
      }
    }
    // the next stage A writes S.x (all reads of it above are done)
    __syncthreads();
  }

  if (head) {
    // ---- the head: x = rmsq(h, wf) over the workgroup, as a layer's
    // stage A; logits = emb x, every wave over its blocks of 4 rows
    const int L = A.nlayers;
    bool ok = true;
    float h8[8] = {}, w8[8] = {};
    if (mine) {
      const float4 *wp = reinterpret_cast<const float4 *>(A.wf + 8 * t);
      const float4 w0 = wp[0], w1 = wp[1];
      w8[0] = w0.x; w8[1] = w0.y; w8[2] = w0.z; w8[3] = w0.w;
      w8[4] = w1.x; w8[5] = w1.y; w8[6] = w1.z; w8[7] = w1.w;
    }
    ok = poll_h(L, h8);
    // the second block's loads, after the wait for h (a poll issued behind
    // them would wait for them too)
    HeadBlock hb0, hb1;
    head_from(a, hb0);
    issue_order();
    head_load(A, gw + stride, lane, hb1);
    if (!workgroup_rmsq(S, h8, w8, A.eps, ok)) return;
    HeadMax best;
    {
      float xv[32];
      const float xsv = load_rmsq_x(S, lane, xv);
      head_rows<FAST>(A, xv, xsv, lane, gw, stride, head_nblk, hb0, hb1, best);
    }
    // the workgroup's best key (holder lanes 15, 31, 47, 63 of each wave;
    // other lanes hold key 0) to workgroup 0 as two tagged words
    __shared__ unsigned long long wkey[kWaves];
    unsigned long long k = ops::key_max_rows(best.key());
    if (lane == kWave - 1) wkey[wave] = k;
    __syncthreads();
    const uint32_t ktag = call + 1;  // never 0, the workspace's initial contents
    if (t == 0) {
      k = wkey[0];
#pragma unroll
      for (int i = 1; i < kWaves; ++i) k = wkey[i] > k ? wkey[i] : k;
      store_tagged(A.kq + 2 * wg, __uint_as_float((uint32_t)(k >> 32)), ktag);
      store_tagged(A.kq + 2 * wg + 1, __uint_as_float((uint32_t)k), ktag);
    }
    if (wg == 0) {
      // every workgroup's key; the largest names the token (the lowest
      // index of the largest logit, -1 if any logit is NaN)
      unsigned long long best_key = 0ull;
      ok = true;
      for (int i = t; i < nwg; i += kThreads) {
        float kv[2];
        ok &= poll_tagged<2>(A.kq + 2 * i, ktag, kv, err, A.spin_ticks);
        const unsigned long long c =
            ((unsigned long long)__float_as_uint(kv[0]) << 32) | __float_as_uint(kv[1]);
        best_key = c > best_key ? c : best_key;
      }
      best_key = ops::lane_key_max64(best_key);
      __syncthreads();  // wkey is free again (every reader is past it)
      if (lane == 0) wkey[wave] = best_key;
      if (!__syncthreads_and(ok)) return;
      if (t == 0) {
#pragma unroll
        for (int i = 1; i < kWaves; ++i) best_key = wkey[i] > best_key ? wkey[i] : best_key;
        *A.tok_out = ops::argmax_index(best_key);
      }
    }
  }
  if (t == 0) store_word(A.ctl + wg, call + 1);
}

template <bool FAST, int NP>
const void *kernel_ptr() {
  return reinterpret_cast<const void *>(&decode_layers_kernel<FAST, NP>);
}

const void *decode_kernel(int mode, int np) {
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

int32_t decode_layers_grid(int mode, int32_t inter) {
  const void *k = decode_kernel(mode, inter / kCols);
  if (!k || inter % kCols) return 0;
  int dev = 0, per_cu = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kThreads, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  // one workgroup per compute unit; the work is dealt to 8 XCDs of 32
  // workgroups (further compute units stay idle)
  if (per_cu < 1 || cus < kDecodeGroups) return 0;
  return kDecodeGroups;
}

hipError_t launch_decode_layers(const DecodeArgs &a, int mode, hipStream_t st) {
  const int np = a.inter / kCols;
  const int32_t grid = decode_layers_grid(mode, a.inter);
  if (grid < 1) return hipErrorInvalidValue;
  const dim3 g(grid), b(kThreads);
#define Q4_DECODE_CASE(NP_)                                                           \
  case NP_:                                                                           \
    if (mode != 0)                                                                    \
      hipLaunchKernelGGL((decode_layers_kernel<true, NP_>), g, b, 0, st, a);          \
    else                                                                              \
      hipLaunchKernelGGL((decode_layers_kernel<false, NP_>), g, b, 0, st, a);         \
    break;
  switch (np) {
    Q4_DECODE_CASE(1)
    Q4_DECODE_CASE(2)
    Q4_DECODE_CASE(3)
    Q4_DECODE_CASE(4)
    default: return hipErrorInvalidValue;
  }
#undef Q4_DECODE_CASE
  return hipGetLastError();
}

}  // namespace q4
