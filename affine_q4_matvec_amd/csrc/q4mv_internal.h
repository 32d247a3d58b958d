// Internal interface between the C ABI layer (q4mv_api.hip) and the kernels
// (q4mv_kernels.hip).  Not installed; the public interface is include/q4mv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

// One product as the kernels see it.  All pointers are device pointers.
struct Prod {
  const uint32_t *q;  // [rows][cols/8] packed codes
  const float *s;     // [rows][G] scales
  const float *b;     // [rows][G] biases
  const float *x;     // [cols] activations
  const float *xs;    // [G] group sums of x
  const float *res;   // [rows] residual added to the result, or nullptr
  float *y;           // [rows] output
  int32_t rows;
  int32_t cols;
};

// Up to kMaxGroup products of one kernel shape, launched as one grid: the
// workgroups [wg_begin[i], wg_begin[i+1]) work on product i.
constexpr int kMaxGroup = 8;
struct ProdGroup {
  Prod p[kMaxGroup];
  int32_t wg_begin[kMaxGroup + 1];
  int32_t n;
};

// Stages fused into a product's kernel.
constexpr int kProX = 0;      // x and its group sums are inputs
constexpr int kProXsum = 1;   // x is an input, its group sums formed in the kernel
constexpr int kProNorm = 2;   // x = rmsq(h, wn) formed in the kernel (2048 columns)
constexpr int kEpiStore = 0;  // y[r] = (res[r] +) row sum
constexpr int kEpiSwiglu = 1; // (gate, up) row pairs -> m[r/2] = SwiGLU
constexpr int kEpiArgmax = 2; // y stored, and one argmax key per workgroup

// Inputs and outputs of the fused stages (unused fields are ignored).
struct Extra {
  const float *h;            // kProNorm: [cols] values to normalise
  const float *wn;           // kProNorm: [cols] norm weights
  float eps;                 // kProNorm
  float *u_out;              // kProNorm, optional: [cols] normalised x
  float *us_out;             //   and its [cols/64] group sums
  float *m_out;              // kEpiSwiglu: [rows/2]
  unsigned long long *amax;  // kEpiArgmax: [workgroups] one key per workgroup
};

// Kernel shape of a product: rows of exactly 32 groups (2048 columns) take
// one wave each (row64); rows of fewer groups are covered by one segment of
// `lpr` lanes of a wave (lpr = 2..64); wider rows are split into `passes`
// 2048-column passes, one wave each, combined through LDS.  `pro` and `epi`
// name the fused stages (kProNorm and the epilogues other than kEpiStore
// exist for row64 only).
struct Shape {
  enum Kind : int32_t { kRow64 = 0, kSeg = 1, kSplit = 2 };
  int32_t kind;
  int32_t lpr;     // lanes per row segment (seg)
  int32_t passes;  // waves per row (split)
  int32_t pro;
  int32_t epi;
  bool operator==(const Shape &o) const {
    return kind == o.kind && lpr == o.lpr && passes == o.passes && pro == o.pro && epi == o.epi;
  }
};

Shape shape_of(int32_t cols, int pro = kProX, int epi = kEpiStore);
bool shape_supported(const Shape &sh);
// Workgroups a product of this shape gets when launched alone.
int32_t workgroups_for(const Shape &sh, int32_t rows, int mode);
// Workgroups of the products of one grouped launch (want[0..n)), in the
// units of the kernel that will run: for row64 shapes the preloading kernel
// when every product's blocks fit on the device at once, else the looping
// kernel with the device's workgroups shared in proportion.
void plan_group(const Shape &sh, int mode, const int32_t *rows, int n, int32_t *want);

// Launchers.  They assume validated arguments and return the HIP status of
// the launch.
hipError_t launch_q4mv_group(const ProdGroup &g, const Shape &sh, int mode, const Extra &ex,
                             hipStream_t st);
// Measurement variants of a 2048-column product (see q4mv_variant in
// q4mv.h): 0 = one lane per row, R = 1, 2, 4, 8 = one wave per row with R
// rows per block.
hipError_t launch_q4mv_variant(const Prod &p, int variant, int mode, hipStream_t st);
hipError_t launch_rmsq(const float *h, const float *w, int32_t n, float eps, float *u,
                       float *us, hipStream_t st);
hipError_t launch_swq(const float *a, int32_t n, float *o, float *os, int mode,
                      hipStream_t st);
size_t argmax_ws_bytes(int32_t n);
hipError_t launch_argmax(const float *v, int32_t n, int32_t *idx, void *ws, hipStream_t st);
// The last step of an argmax: the largest of `nkeys` keys -> *idx.
hipError_t launch_argmax_final(const unsigned long long *keys, int32_t nkeys, int32_t *idx,
                               hipStream_t st);
hipError_t launch_embed(const Prod &w, const int32_t *tok, float *e, hipStream_t st);
hipError_t launch_pos_advance(int32_t *pos, hipStream_t st);
// One thread: host_vals[0..n) = vals[0..n), then *host_seq = ++*dev_count.
hipError_t launch_mailbox(const int32_t *vals, int32_t n, int32_t *host_vals, uint32_t *host_seq,
                          uint32_t *dev_count, hipStream_t st);

// The MLP layers of a decode step in one persistent launch (decode_layers.hip).
constexpr int kMaxDecodeLayers = 32;
struct DecodeLayer {
  const uint32_t *gq;  // gate/up rows interleaved: [2*inter][256] codes
  const float *gs, *gb;
  const float *wn;     // [2048] norm weights
  const uint32_t *dq;  // down: [2048][inter/8] codes
  const float *ds, *db;
};
struct DecodeArgs {
  DecodeLayer layer[kMaxDecodeLayers];
  int32_t nlayers;
  int32_t inter;        // 2048, 4096, 6144 or 8192
  const uint32_t *eq;   // embedding rows: [vocab][256] codes
  const float *es, *eb;
  int32_t vocab;
  const int32_t *tok;   // [1] token read on the device
  float *h;             // [2048] hidden state after the last layer (output)
  uint64_t *hq;         // workspace: [2][slots][2048] tagged h between layers
  uint64_t *mq;         // workspace: [2][slots][max inter] tagged m
  uint64_t *pq;         // workspace: [2048][4][8] tagged down partial sums
  uint32_t *ctl;        // workspace: call counters and error word
  float eps;
  long long spin_ticks; // bound of one wait in wall-clock ticks
  long long near_ticks; // how long a wait reads its XCD's copy before the producers'
  // The head, when wf is not null (q4_decode_token): logits = emb
  // rmsq(h, wf), *tok_out = argmax(logits), with the workgroups' best keys
  // handed to workgroup 0 through tagged words in kq.
  const float *wf;      // [2048] final norm weights, or nullptr
  float *logits;        // [vocab]
  int32_t *tok_out;     // [1] the next token (may be tok)
  uint64_t *kq;         // workspace: [max groups][2] tagged argmax keys
};
// Workspace layout (bytes): tagged h and tagged m of the widest inter (each
// in kDecodeSlots copies, twice by layer parity); the down product's
// partial sums (per row, pass and XCD); two tagged words per workgroup for
// the head's argmax keys; then the control words: one call counter per
// workgroup (at most kDecodeMaxGroups) and the error word on a 128-byte
// line of its own (32 words before the end).
constexpr int kDecodeMaxInter = 8192;
constexpr int kDecodeMaxGroups = 1024;
// The decode-block kernels write each tagged value in kDecodeCopies copies;
// workgroup i reads copy i % kDecodeCopies, so that each cache line is
// polled by a fraction of the grid only.
constexpr int kDecodeCopies = 8;
// The decode-layers kernel hands h and m on through the L2 of each XCD:
// copy x of each is read by the workgroups of XCD x, copy kDecodeXcds (the
// device-scope one) by any workgroup that its XCD's copy does not serve.
// h's producers write copy kDecodeXcds and the workgroups of XCD x relay it
// into copy x; m's producers write both copies (each XCD produces the m
// values its own workgroups read).
constexpr int kDecodeXcds = 8;
constexpr int kDecodeSlots = kDecodeXcds + 1;
// The persistent grid: 8 XCDs of 32 workgroups.
constexpr int kDecodeGroups = 256;
constexpr size_t kDecodeHqOffset = 0;
constexpr size_t kDecodeMqOffset = 2 * kDecodeSlots * 8 * 2048;
constexpr size_t kDecodePqOffset =
    kDecodeMqOffset + 2 * kDecodeSlots * 8 * (size_t)kDecodeMaxInter;
constexpr size_t kDecodeKqOffset = kDecodePqOffset + 8 * (size_t)2048 * 4 * kDecodeXcds;
constexpr size_t kDecodeCtlOffset = kDecodeKqOffset + 2 * 8 * (size_t)kDecodeMaxGroups;
constexpr int kDecodeErrorWord = kDecodeMaxGroups + 32;
constexpr size_t kDecodeWsBytes = kDecodeCtlOffset + 4 * (kDecodeErrorWord + 32);
// Workgroups of the persistent launch for this mode and width (0: none fit).
int32_t decode_layers_grid(int mode, int32_t inter);
hipError_t launch_decode_layers(const DecodeArgs &a, int mode, hipStream_t st);

// Decoder layers (attention block and MLP block), one or several in one
// persistent launch (decode_block.hip): 16 query heads of 128 (hq * 128 =
// 2048), hkv key/value heads dividing 16, caches of up to 16 spans of 256
// positions (one workgroup per head and span).
constexpr int kBlockHeads = 16;
constexpr int kBlockSpan = 256;
constexpr int kBlockMaxSpans = 16;
constexpr int kBlockMaxPos = kBlockSpan * kBlockMaxSpans;
constexpr int kBlockQRows = 8192;         // rows of [Q; gate; K; V], at most (hkv = 16)
constexpr int kBlockORows = 2048 + 64;    // o and its 32 group sums (padded)
// One decoder layer's arrays.
struct BlockLayer {
  const uint32_t *qq;  // [Q; gate; K; V] codes: [(32 + 2 hkv) * 128][256]
  const float *qs, *qb;
  const uint32_t *oq;  // O: [2048][256] codes
  const float *os, *ob;
  const float *wa;     // [2048] attention norm weights
  const float *wq, *wk;  // [128] query and key norm weights
  float *kc, *vc;      // [hkv][max_pos][128] caches; row pos is written
  DecodeLayer mlp;     // gate/up rows interleaved, down, MLP norm weights
};
constexpr int kBlockMaxLayers = 32;
struct DecodeBlockArgs {
  BlockLayer one;             // the layer, when `layers` is null
  const BlockLayer *layers;   // device table [nlayers], or null
  int32_t nlayers;            // 1 .. kBlockMaxLayers
  const float *cs, *sn;  // [max_pos][64] rotation tables
  const int32_t *pos;  // [1] the token's position
  int32_t max_pos, hkv;
  int32_t inter;
  float *h;            // [2048] hidden state: read at the start, written at the end
  uint64_t *qv;        // workspace: [copies][kBlockQRows] tagged q, gate, k, v
  uint64_t *ov;        // workspace: [copies][kBlockORows] tagged o and its group sums
  uint64_t *hv;        // workspace: [copies][2048] tagged h after the attention block
  uint64_t *mq;        // workspace: [copies][kDecodeMaxInter] tagged m
  uint64_t *hb;        // workspace: [copies][2048] tagged h between layers
  uint64_t *mx;        // workspace: [heads][spans] tagged span maxima
  uint64_t *zp;        // workspace: [heads][spans] tagged span weight sums
  uint64_t *wp;        // workspace: [heads][spans][128] tagged span value sums
  uint32_t *ctl;       // workspace: call counters and the error word
  float eps;
  long long spin_ticks;
};
// Each hand-off buffer serves every layer of a launch: a workgroup writes
// layer l + 1's values of a buffer only after every workgroup has passed
// its read of layer l's (each stage waits on outputs of every workgroup's
// previous stage, around the whole layer).
constexpr size_t kBlockQvOffset = 0;
constexpr size_t kBlockOvOffset = kBlockQvOffset + 8 * (size_t)kDecodeCopies * kBlockQRows;
constexpr size_t kBlockHvOffset = kBlockOvOffset + 8 * (size_t)kDecodeCopies * kBlockORows;
constexpr size_t kBlockMqOffset = kBlockHvOffset + 8 * (size_t)kDecodeCopies * 2048;
constexpr size_t kBlockHbOffset = kBlockMqOffset + 8 * (size_t)kDecodeCopies * kDecodeMaxInter;
constexpr size_t kBlockMxOffset = kBlockHbOffset + 8 * (size_t)kDecodeCopies * 2048;
constexpr size_t kBlockZpOffset = kBlockMxOffset + 8 * (size_t)kBlockHeads * kBlockMaxSpans;
constexpr size_t kBlockWpOffset = kBlockZpOffset + 8 * (size_t)kBlockHeads * kBlockMaxSpans;
constexpr size_t kBlockCtlOffset =
    kBlockWpOffset + 8 * (size_t)kBlockHeads * kBlockMaxSpans * 128;
constexpr int kBlockErrorWord = kDecodeMaxGroups + 32;
constexpr size_t kBlockWsBytes = kBlockCtlOffset + 4 * (kBlockErrorWord + 32);
int32_t decode_block_grid(int mode, int32_t inter);
hipError_t launch_decode_block(const DecodeBlockArgs &a, int mode, hipStream_t st);

// Gated attention of one decode token (atq.hip).  Caches are float
// [hkv][max_pos][128]; positions are worked on in aligned spans of 256.
constexpr int kAtqD = 128;
constexpr int kAtqSpan = 256;
constexpr int kAtqMaxPos = 4096;
constexpr int kAtqMaxSpans = kAtqMaxPos / kAtqSpan;
constexpr int kAtqMaxGroup = 8;   // query heads per key/value head
constexpr int kAtqMaxHeads = 128; // query heads
// Control words: one call counter per workgroup ([hkv][kAtqMaxSpans]), then
// the error word on a 128-byte line of its own.
constexpr int kAtqErrorWord = kAtqMaxHeads * kAtqMaxSpans + 32;
struct AtqArgs {
  const float *q, *g;    // [hq][128]
  const float *k, *v;    // [hkv][128]
  const float *wq, *wk;  // [128] norm weights
  const float *cs, *sn;  // [max_pos][64] rotation tables, row pos used
  float *kc, *vc;        // [hkv][max_pos][128] caches; row pos is written
  float *o;              // [hq][128]
  float *os;             // [hq][2] group sums of o
  uint64_t *mx;          // workspace: [hq][kAtqMaxSpans] tagged span maxima
  uint64_t *zp;          // workspace: [hq][kAtqMaxSpans] tagged span weight sums
  uint64_t *wp;          // workspace: [hq][kAtqMaxSpans][128] tagged span value sums
  uint32_t *ctl;         // workspace: call counters and the error word
  const int32_t *pos;    // [1] the token's position, read on the device
  float eps;
  int32_t max_pos, hq, hkv;
  long long spin_ticks;  // bound of one wait in wall-clock ticks
};
// Byte offsets of the workspace arrays for hq query heads.
struct AtqWs {
  size_t mx, zp, wp, ctl, bytes;
};
void atq_ws_layout(int32_t hq, int32_t hkv, AtqWs *out);
hipError_t launch_atq(const AtqArgs &a, hipStream_t st);

}  // namespace q4
