// C ABI of libq4mv.so (declared in include/q4mv.h): argument checks, the
// stage queue, graph capture and status codes.  Every check runs before any
// HIP call, so a rejected call touches neither the device nor the runtime.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <chrono>
#include <mutex>
#include <new>
#include <vector>

// Only the C ABI is exported; everything else is hidden (-fvisibility=hidden).
#pragma GCC visibility push(default)
#include "../../include/q4mv.h"
#pragma GCC visibility pop
#include "q4mv_internal.h"

namespace {

using q4::Prod;
using q4::ProdGroup;
using q4::Shape;

constexpr int32_t kMaxRows = 1 << 30;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// [a, a+na) and [b, b+nb) (bytes) overlap?
bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

bool env_flag(const char *name) {
  const char *v = getenv(name);
  return v && *v && strcmp(v, "0") != 0;
}

int check_mat(const q4_mat *w) {
  if (!w || !w->q || !w->s || !w->b) return Q4_EINVAL;
  if (w->rows < 1 || w->rows > kMaxRows) return Q4_EINVAL;
  if (w->cols < 64 || w->cols % 64 != 0 || w->cols > Q4_MAX_COLS) return Q4_EINVAL;
  if (!aligned(w->q, 16) || !aligned(w->s, 4) || !aligned(w->b, 4)) return Q4_EINVAL;
  return Q4_OK;
}

// Does the output range [p, p + bytes) overlap the matrix arrays?
bool overlaps_mat(const void *p, size_t bytes, const q4_mat *w) {
  const size_t G = (size_t)w->cols / 64;
  return overlap(p, bytes, w->q, (size_t)w->rows * (size_t)w->cols / 2) ||
         overlap(p, bytes, w->s, sizeof(float) * G * (size_t)w->rows) ||
         overlap(p, bytes, w->b, sizeof(float) * G * (size_t)w->rows);
}

// Checks one product and fills the kernel's view of it.  xsum may be null
// (the kernel then forms the group sums of x).
int make_prod(const q4_mat *w, const float *x, const float *xsum, const float *resid, float *y,
              Prod *out) {
  int rc = check_mat(w);
  if (rc != Q4_OK) return rc;
  if (!x || !y) return Q4_EINVAL;
  if (!aligned(x, 16) || !aligned(y, 4) || (xsum && !aligned(xsum, 4))) return Q4_EINVAL;
  if (resid && !aligned(resid, 4)) return Q4_EINVAL;
  const size_t G = (size_t)w->cols / 64;
  const size_t ybytes = sizeof(float) * (size_t)w->rows;
  if (overlap(y, ybytes, x, sizeof(float) * (size_t)w->cols) ||
      (xsum && overlap(y, ybytes, xsum, sizeof(float) * G)) || overlaps_mat(y, ybytes, w))
    return Q4_EINVAL;
  if (resid && resid != y && overlap(y, ybytes, resid, ybytes)) return Q4_EINVAL;
  *out = Prod{w->q, w->s, w->b, x, xsum, resid, y, w->rows, w->cols};
  return Q4_OK;
}

// Checks the inputs of an rmsq prologue over n values.
int check_norm_inputs(const float *h, const float *wn) {
  if (!h || !wn || !aligned(h, 16) || !aligned(wn, 16)) return Q4_EINVAL;
  return Q4_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? Q4_OK : Q4_EHIP; }

// Bound of one device-side wait (the persistent layers kernel, the
// attention step's exchanges): Q4_DECODE_TIMEOUT_MS (default 2000, at most
// 60000) of the device's constant wall clock; a negative value makes every
// wait that does not find its data at the first look run out (a test of
// that path).
int wait_ticks(long long *ticks) {
  long long ms = 2000;
  if (const char *v = getenv("Q4_DECODE_TIMEOUT_MS")) ms = atoll(v);
  if (ms > 60000) ms = 60000;
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
    return Q4_EHIP;
  *ticks = ms < 0 ? -1 : ms * (long long)(khz > 0 ? khz : 100000);
  return Q4_OK;
}

// How long a wait for h reads its XCD's copy before it turns to the
// producers' copy: 50 us by default (every relay of a launch is done well
// within that; only a workgroup that no relay serves runs it out), or
// Q4_DECODE_NEAR_US microseconds (0: after one round), at most the whole
// bound.
long long near_ticks(long long spin_ticks) {
  long long us = 50;
  if (const char *v = getenv("Q4_DECODE_NEAR_US")) us = atoll(v);
  if (us < 0) us = 0;
  if (us > 60000000) us = 60000000;
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
    khz = 100000;
  const long long t = us * (khz > 0 ? khz : 100000) / 1000;
  return spin_ticks < t ? spin_ticks : t;
}

// Host wait on `stream`, then the error word at byte offset err_off of a
// workspace: Q4_OK, or Q4_ETIMEOUT after clearing the first `clear` bytes
// of the workspace (a wait ran out and left its words in an unknown state).
int ws_status(void *ws, size_t err_off, size_t clear, void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) return Q4_EHIP;
  if (cs != hipStreamCaptureStatusNone) return Q4_ESTATE;
  if (hipStreamSynchronize(st) != hipSuccess) return Q4_EHIP;
  uint32_t err = 0;
  if (hipMemcpy(&err, static_cast<const char *>(ws) + err_off, sizeof(err),
                hipMemcpyDeviceToHost) != hipSuccess)
    return Q4_EHIP;
  if (err == 0) return Q4_OK;
  if (hipMemsetAsync(ws, 0, clear, st) != hipSuccess || hipStreamSynchronize(st) != hipSuccess)
    return Q4_EHIP;
  return Q4_ETIMEOUT;
}

// Launches a list of products of one shape as grouped kernels (up to
// kMaxGroup products per launch), each launch's workgroups planned by
// plan_group.
int launch_products(const Prod *prods, int count, const Shape &sh, int mode, hipStream_t st,
                    const q4::Extra &ex = q4::Extra{}) {
  if (!q4::shape_supported(sh)) return Q4_EINVAL;
  for (int at = 0; at < count; at += q4::kMaxGroup) {
    ProdGroup g;
    memset(&g, 0, sizeof(g));
    g.n = count - at < q4::kMaxGroup ? count - at : q4::kMaxGroup;
    int32_t rows[q4::kMaxGroup], want[q4::kMaxGroup];
    for (int i = 0; i < g.n; ++i) rows[i] = prods[at + i].rows;
    q4::plan_group(sh, mode, rows, g.n, want);
    g.wg_begin[0] = 0;
    for (int i = 0; i < g.n; ++i) {
      g.p[i] = prods[at + i];
      g.wg_begin[i + 1] = g.wg_begin[i] + want[i];
    }
    for (int i = g.n; i < q4::kMaxGroup; ++i) g.wg_begin[i + 1] = g.wg_begin[g.n];
    const int rc = hip_status(q4::launch_q4mv_group(g, sh, mode, ex, st));
    if (rc != Q4_OK) return rc;
  }
  return Q4_OK;
}

}  // namespace

struct q4_mailbox {
  int32_t n = 0;
  int32_t *host_vals = nullptr;   // pinned, coherent host memory (mapped)
  uint32_t *host_seq = nullptr;
  int32_t *dev_vals_view = nullptr;  // device addresses of the same memory
  uint32_t *dev_seq_view = nullptr;
  uint32_t *dev_count = nullptr;  // device memory: posts executed
};

struct q4_queue {
  hipStream_t st = nullptr;
  int mode = Q4_FIXED;
  std::vector<Prod> stage;  // products of the open stage
  bool debug = false;
  bool trace = false;
  // trace state: events around the work since the last wait
  hipEvent_t ev_begin = nullptr, ev_end = nullptr;
  bool began = false;
  int products_since_wait = 0;
  std::chrono::steady_clock::time_point wall_begin;
  // Q4_WAIT_MAILBOX: the wait spins on this mailbox instead of the stream
  q4_mailbox *mailbox = nullptr;
  uint32_t posted = 0;
  int32_t timeout_ms = 0;
};

struct q4_graph {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

namespace {

Shape prod_shape(const Prod &p) {
  return q4::shape_of(p.cols, p.xs ? q4::kProX : q4::kProXsum);
}

// Launches the open stage: products grouped by kernel shape.
int flush_stage(q4_queue *q) {
  if (q->stage.empty()) return Q4_OK;
  if (q->trace && !q->began) {
    if (hipEventRecord(q->ev_begin, q->st) != hipSuccess) return Q4_EHIP;
    q->began = true;
    q->wall_begin = std::chrono::steady_clock::now();
  }
  std::vector<bool> done(q->stage.size(), false);
  std::vector<Prod> same;
  for (size_t i = 0; i < q->stage.size(); ++i) {
    if (done[i]) continue;
    const Shape sh = prod_shape(q->stage[i]);
    same.clear();
    for (size_t j = i; j < q->stage.size(); ++j) {
      if (!done[j] && prod_shape(q->stage[j]) == sh) {
        same.push_back(q->stage[j]);
        done[j] = true;
      }
    }
    const int rc = launch_products(same.data(), (int)same.size(), sh, q->mode, q->st);
    if (rc != Q4_OK) return rc;
  }
  q->products_since_wait += (int)q->stage.size();
  q->stage.clear();
  return Q4_OK;
}

}  // namespace

extern "C" {

int q4mv(const q4_mat *w, const float *x, const float *xsum, float *y, int mode, void *stream) {
  return q4mv_add(w, x, xsum, nullptr, y, mode, stream);
}

int q4mv_add(const q4_mat *w, const float *x, const float *xsum, const float *resid, float *y,
             int mode, void *stream) {
  if (mode != Q4_FIXED && mode != Q4_FAST) return Q4_EINVAL;
  Prod p;
  const int rc = make_prod(w, x, xsum, resid, y, &p);
  if (rc != Q4_OK) return rc;
  return launch_products(&p, 1, prod_shape(p), mode, static_cast<hipStream_t>(stream));
}

int q4mv_norm(const q4_mat *w, const float *h, const float *wn, float eps, float *y, float *u,
              float *usum, int mode, void *stream) {
  if (mode != Q4_FIXED && mode != Q4_FAST) return Q4_EINVAL;
  int rc = check_mat(w);
  if (rc != Q4_OK) return rc;
  if ((rc = check_norm_inputs(h, wn)) != Q4_OK) return rc;
  if (!y || !aligned(y, 4) || (!u) != (!usum)) return Q4_EINVAL;
  if (u && (!aligned(u, 16) || !aligned(usum, 4))) return Q4_EINVAL;
  const size_t n = (size_t)w->cols, ybytes = sizeof(float) * (size_t)w->rows;
  const size_t nb = sizeof(float) * n, gb = sizeof(float) * (n / 64);
  if (overlap(y, ybytes, h, nb) || overlap(y, ybytes, wn, nb) || overlaps_mat(y, ybytes, w))
    return Q4_EINVAL;
  if (u && (overlap(u, nb, h, nb) || overlap(u, nb, wn, nb) || overlap(u, nb, y, ybytes) ||
            overlap(usum, gb, h, nb) || overlap(usum, gb, wn, nb) || overlap(usum, gb, u, nb) ||
            overlap(usum, gb, y, ybytes) || overlaps_mat(u, nb, w) || overlaps_mat(usum, gb, w)))
    return Q4_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (w->cols != 2048) {
    // no fused kernel for this width: the norm, then the product
    if (!u) return Q4_EINVAL;
    if (w->cols > Q4_MAX_RMSQ_N) return Q4_EINVAL;
    rc = rmsq(h, wn, w->cols, eps, u, usum, stream);
    if (rc != Q4_OK) return rc;
    return q4mv(w, u, usum, y, mode, stream);
  }
  Prod p{w->q, w->s, w->b, nullptr, nullptr, nullptr, y, w->rows, w->cols};
  q4::Extra ex{};
  ex.h = h;
  ex.wn = wn;
  ex.eps = eps;
  ex.u_out = u;
  ex.us_out = usum;
  return launch_products(&p, 1, q4::shape_of(w->cols, q4::kProNorm, q4::kEpiStore), mode, st, ex);
}

int q4mv_norm_swiglu(const q4_mat *w, const float *h, const float *wn, float eps, float *m,
                     int mode, void *stream) {
  if (mode != Q4_FIXED && mode != Q4_FAST) return Q4_EINVAL;
  int rc = check_mat(w);
  if (rc != Q4_OK) return rc;
  if ((rc = check_norm_inputs(h, wn)) != Q4_OK) return rc;
  if (w->cols != 2048 || w->rows % 2 != 0) return Q4_EINVAL;
  if (!m || !aligned(m, 4)) return Q4_EINVAL;
  const size_t nb = sizeof(float) * 2048, mb = sizeof(float) * (size_t)(w->rows / 2);
  if (overlap(m, mb, h, nb) || overlap(m, mb, wn, nb) || overlaps_mat(m, mb, w)) return Q4_EINVAL;
  Prod p{w->q, w->s, w->b, nullptr, nullptr, nullptr, nullptr, w->rows, w->cols};
  q4::Extra ex{};
  ex.h = h;
  ex.wn = wn;
  ex.eps = eps;
  ex.m_out = m;
  return launch_products(&p, 1, q4::shape_of(2048, q4::kProNorm, q4::kEpiSwiglu), mode,
                         static_cast<hipStream_t>(stream), ex);
}

// One 8-byte key per workgroup of the fused argmax launch.
constexpr int32_t kArgmaxMaxWorkgroups = 4096;

namespace {

// The checks of q4mv_norm_argmax other than those of its workspace.
int check_norm_argmax(const q4_mat *w, const float *h, const float *wn, const float *y,
                      const int32_t *idx, int mode) {
  if (mode != Q4_FIXED && mode != Q4_FAST) return Q4_EINVAL;
  int rc = check_mat(w);
  if (rc != Q4_OK) return rc;
  if ((rc = check_norm_inputs(h, wn)) != Q4_OK) return rc;
  if (w->cols != 2048) return Q4_EINVAL;
  if (!y || !idx || !aligned(y, 4) || !aligned(idx, 4)) return Q4_EINVAL;
  const size_t nb = sizeof(float) * 2048, yb = sizeof(float) * (size_t)w->rows;
  if (overlap(y, yb, h, nb) || overlap(y, yb, wn, nb) || overlaps_mat(y, yb, w) ||
      overlap(idx, 4, y, yb) || overlap(idx, 4, h, nb) || overlap(idx, 4, wn, nb) ||
      overlaps_mat(idx, 4, w))
    return Q4_EINVAL;
  return Q4_OK;
}

// The product with its argmax epilogue, then the final pick over the
// workgroups' keys; at most `slots` workgroups (one key each at keys[i]).
int launch_norm_argmax(const q4_mat *w, const float *h, const float *wn, float eps, float *y,
                       int32_t *idx, unsigned long long *keys, long long slots, int mode,
                       hipStream_t st) {
  const Shape sh = q4::shape_of(2048, q4::kProNorm, q4::kEpiArgmax);
  long long nwg = q4::workgroups_for(sh, w->rows, mode);
  if (nwg > slots) nwg = slots;
  if (nwg > kArgmaxMaxWorkgroups) nwg = kArgmaxMaxWorkgroups;
  ProdGroup g;
  memset(&g, 0, sizeof(g));
  g.n = 1;
  g.p[0] = Prod{w->q, w->s, w->b, nullptr, nullptr, nullptr, y, w->rows, w->cols};
  for (int i = 1; i <= q4::kMaxGroup; ++i) g.wg_begin[i] = (int32_t)nwg;
  q4::Extra ex{};
  ex.h = h;
  ex.wn = wn;
  ex.eps = eps;
  ex.amax = keys;
  const int rc = hip_status(q4::launch_q4mv_group(g, sh, mode, ex, st));
  if (rc != Q4_OK) return rc;
  return hip_status(q4::launch_argmax_final(keys, (int32_t)nwg, idx, st));
}

// Device scratch of q4mv_norm_argmax_noalloc: the workgroups' argmax keys,
// one array per GPU for the life of the process.  Its name is a host-side
// stand-in: host code uses the device address that hipGetSymbolAddress
// returns for the current device, never the name itself.
static __device__ __align__(256) unsigned long long scratch[kArgmaxMaxWorkgroups];

constexpr int kScratchDevices = 64;
std::atomic<void *> g_scratch[kScratchDevices];
std::mutex g_scratch_mu;

// The address of `scratch` on the current device, looked up on the first
// call for each device and kept.
int scratch_address(unsigned long long **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return Q4_EHIP;
  if (dev < 0 || dev >= kScratchDevices) return Q4_EINVAL;
  void *p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return Q4_EHIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = static_cast<unsigned long long *>(p);
  return Q4_OK;
}

}  // namespace

size_t q4mv_argmax_ws_bytes(void) { return sizeof(unsigned long long) * kArgmaxMaxWorkgroups; }

int q4mv_norm_argmax(const q4_mat *w, const float *h, const float *wn, float eps, float *y,
                     int32_t *idx, void *ws, size_t ws_bytes, int mode, void *stream) {
  int rc = check_norm_argmax(w, h, wn, y, idx, mode);
  if (rc != Q4_OK) return rc;
  if (!ws || !aligned(ws, 8) || ws_bytes < sizeof(unsigned long long)) return Q4_EINVAL;
  const size_t nb = sizeof(float) * 2048, yb = sizeof(float) * (size_t)w->rows;
  if (overlap(ws, ws_bytes, y, yb) || overlap(ws, ws_bytes, idx, 4) ||
      overlap(ws, ws_bytes, h, nb) || overlap(ws, ws_bytes, wn, nb) ||
      overlaps_mat(ws, ws_bytes, w))
    return Q4_EINVAL;
  return launch_norm_argmax(w, h, wn, eps, y, idx, static_cast<unsigned long long *>(ws),
                            (long long)(ws_bytes / sizeof(unsigned long long)), mode,
                            static_cast<hipStream_t>(stream));
}

int q4mv_variant(const q4_mat *w, const float *x, const float *xsum, float *y, int variant,
                 int mode, void *stream) {
  if (mode != Q4_FIXED && mode != Q4_FAST) return Q4_EINVAL;
  if (variant != Q4_VARIANT_LANE_PER_ROW && variant != Q4_VARIANT_WAVE_R1 &&
      variant != Q4_VARIANT_WAVE_R2 && variant != Q4_VARIANT_WAVE_R4 &&
      variant != Q4_VARIANT_WAVE_R8)
    return Q4_EINVAL;
  if (!xsum) return Q4_EINVAL;
  Prod p;
  const int rc = make_prod(w, x, xsum, nullptr, y, &p);
  if (rc != Q4_OK) return rc;
  if (w->cols != 2048) return Q4_EINVAL;
  return hip_status(q4::launch_q4mv_variant(p, variant, mode, static_cast<hipStream_t>(stream)));
}

int q4mv_norm_argmax_noalloc(const q4_mat *w, const float *h, const float *wn, float eps,
                             float *y, int32_t *idx, int mode, void *stream) {
  int rc = check_norm_argmax(w, h, wn, y, idx, mode);
  if (rc != Q4_OK) return rc;
  unsigned long long *keys = nullptr;
  if ((rc = scratch_address(&keys)) != Q4_OK) return rc;
  return launch_norm_argmax(w, h, wn, eps, y, idx, keys, kArgmaxMaxWorkgroups, mode,
                            static_cast<hipStream_t>(stream));
}

int rmsq(const float *h, const float *w, int32_t n, float eps, float *u, float *usum,
         void *stream) {
  if (!h || !w || !u || !usum) return Q4_EINVAL;
  if (n < 64 || n % 64 != 0 || n > Q4_MAX_RMSQ_N) return Q4_EINVAL;
  if (!aligned(h, 4) || !aligned(w, 4) || !aligned(u, 4) || !aligned(usum, 4)) return Q4_EINVAL;
  const size_t nb = sizeof(float) * (size_t)n, gb = sizeof(float) * (size_t)(n / 64);
  if (overlap(u, nb, h, nb) || overlap(u, nb, w, nb) || overlap(usum, gb, h, nb) ||
      overlap(usum, gb, w, nb) || overlap(usum, gb, u, nb))
    return Q4_EINVAL;
  return hip_status(q4::launch_rmsq(h, w, n, eps, u, usum, static_cast<hipStream_t>(stream)));
}

int swq(const float *a, int32_t n, float *o, float *osum, int mode, void *stream) {
  if (mode != Q4_FIXED && mode != Q4_FAST) return Q4_EINVAL;
  if (!a || !o || !osum) return Q4_EINVAL;
  if (n < 64 || n % 64 != 0 || n > (1 << 28)) return Q4_EINVAL;
  if (!aligned(a, 4) || !aligned(o, 4) || !aligned(osum, 4)) return Q4_EINVAL;
  const size_t ab = sizeof(float) * 2 * (size_t)n, nb = sizeof(float) * (size_t)n,
               gb = sizeof(float) * (size_t)(n / 64);
  if (overlap(o, nb, a, ab) || overlap(osum, gb, a, ab) || overlap(osum, gb, o, nb))
    return Q4_EINVAL;
  return hip_status(q4::launch_swq(a, n, o, osum, mode, static_cast<hipStream_t>(stream)));
}

size_t q4_argmax_ws_bytes(int32_t n) { return n < 1 ? 0 : q4::argmax_ws_bytes(n); }

int q4_argmax(const float *v, int32_t n, int32_t *idx, void *ws, size_t ws_bytes, void *stream) {
  if (!v || !idx || !ws || n < 1) return Q4_EINVAL;
  if (!aligned(v, 4) || !aligned(idx, 4) || !aligned(ws, 8)) return Q4_EINVAL;
  if (ws_bytes < q4::argmax_ws_bytes(n)) return Q4_EINVAL;
  const size_t vb = sizeof(float) * (size_t)n;
  if (overlap(idx, 4, v, vb) || overlap(ws, ws_bytes, v, vb) || overlap(ws, ws_bytes, idx, 4))
    return Q4_EINVAL;
  return hip_status(q4::launch_argmax(v, n, idx, ws, static_cast<hipStream_t>(stream)));
}

int q4_embed(const q4_mat *w, const int32_t *tok, float *e, void *stream) {
  int rc = check_mat(w);
  if (rc != Q4_OK) return rc;
  if (!tok || !e || !aligned(tok, 4) || !aligned(e, 4)) return Q4_EINVAL;
  if (overlap(e, sizeof(float) * (size_t)w->cols, tok, 4)) return Q4_EINVAL;
  Prod p{w->q, w->s, w->b, nullptr, nullptr, nullptr, e, w->rows, w->cols};
  return hip_status(q4::launch_embed(p, tok, e, static_cast<hipStream_t>(stream)));
}

size_t q4_decode_layers_ws_bytes(void) { return q4::kDecodeWsBytes; }

}  // extern "C"

namespace {

// Checks of q4_decode_layers and q4_decode_token and the kernel's arguments;
// `outs` are the arrays the call writes (h, ws and, for the token, logits):
// none may overlap an input.
int decode_args(const q4_mat *emb, const int32_t *tok, const q4_mlp_layer *layers,
                int32_t nlayers, float eps, float *h, void *ws, size_t ws_bytes, int mode,
                const void *const *outs, const size_t *outb, int nouts, q4::DecodeArgs *a) {
  if (mode != Q4_FIXED && mode != Q4_FAST) return Q4_EINVAL;
  int rc = check_mat(emb);
  if (rc != Q4_OK) return rc;
  if (emb->cols != 2048) return Q4_EINVAL;
  if (!layers || nlayers < 1 || nlayers > Q4_MAX_DECODE_LAYERS) return Q4_EINVAL;
  if (!tok || !aligned(tok, 4) || !h || !aligned(h, 4)) return Q4_EINVAL;
  if (!ws || !aligned(ws, 16) || ws_bytes < q4::kDecodeWsBytes) return Q4_EINVAL;
  const int32_t inter = layers[0].down.cols;
  if (inter < 2048 || inter % 2048 != 0 || inter > q4::kDecodeMaxInter) return Q4_EINVAL;
  const size_t hb = sizeof(float) * 2048;
  for (int i = 0; i < nouts; ++i) {
    for (int k = i + 1; k < nouts; ++k)
      if (overlap(outs[i], outb[i], outs[k], outb[k])) return Q4_EINVAL;
    if (overlaps_mat(outs[i], outb[i], emb) || overlap(outs[i], outb[i], tok, 4)) return Q4_EINVAL;
  }
  memset(a, 0, sizeof(*a));
  for (int l = 0; l < nlayers; ++l) {
    const q4_mlp_layer &L = layers[l];
    if (check_mat(&L.gate_up) != Q4_OK || check_mat(&L.down) != Q4_OK) return Q4_EINVAL;
    if (L.gate_up.cols != 2048 || L.gate_up.rows != 2 * inter) return Q4_EINVAL;
    if (L.down.rows != 2048 || L.down.cols != inter) return Q4_EINVAL;
    if (!L.wn || !aligned(L.wn, 16)) return Q4_EINVAL;
    for (int i = 0; i < nouts; ++i)
      if (overlaps_mat(outs[i], outb[i], &L.gate_up) || overlaps_mat(outs[i], outb[i], &L.down) ||
          overlap(outs[i], outb[i], L.wn, hb))
        return Q4_EINVAL;
    a->layer[l] = q4::DecodeLayer{L.gate_up.q, L.gate_up.s, L.gate_up.b, L.wn,
                                  L.down.q,    L.down.s,    L.down.b};
  }
  a->nlayers = nlayers;
  a->inter = inter;
  a->eq = emb->q;
  a->es = emb->s;
  a->eb = emb->b;
  a->vocab = emb->rows;
  a->tok = tok;
  a->h = h;
  char *w = static_cast<char *>(ws);
  a->hq = reinterpret_cast<uint64_t *>(w + q4::kDecodeHqOffset);
  a->mq = reinterpret_cast<uint64_t *>(w + q4::kDecodeMqOffset);
  a->pq = reinterpret_cast<uint64_t *>(w + q4::kDecodePqOffset);
  a->ctl = reinterpret_cast<uint32_t *>(w + q4::kDecodeCtlOffset);
  a->kq = reinterpret_cast<uint64_t *>(w + q4::kDecodeKqOffset);
  a->eps = eps;
  if (wait_ticks(&a->spin_ticks) != Q4_OK) return Q4_EHIP;
  a->near_ticks = near_ticks(a->spin_ticks);
  if (q4::decode_layers_grid(mode, inter) < 1) return Q4_EINVAL;  // too few compute units
  return Q4_OK;
}

}  // namespace

extern "C" {

int q4_decode_layers(const q4_mat *emb, const int32_t *tok, const q4_mlp_layer *layers,
                     int32_t nlayers, float eps, float *h, void *ws, size_t ws_bytes, int mode,
                     void *stream) {
  const void *outs[2] = {h, ws};
  const size_t outb[2] = {sizeof(float) * 2048, q4::kDecodeWsBytes};
  q4::DecodeArgs a;
  const int rc = decode_args(emb, tok, layers, nlayers, eps, h, ws, ws_bytes, mode, outs, outb, 2,
                             &a);
  if (rc != Q4_OK) return rc;
  return hip_status(q4::launch_decode_layers(a, mode, static_cast<hipStream_t>(stream)));
}

int q4_decode_token(const q4_mat *emb, int32_t *tok, const q4_mlp_layer *layers, int32_t nlayers,
                    const float *wn_final, float eps, float *h, float *logits, void *ws,
                    size_t ws_bytes, int mode, void *stream) {
  if (!wn_final || !aligned(wn_final, 16) || !logits || !aligned(logits, 4)) return Q4_EINVAL;
  if (check_mat(emb) != Q4_OK) return Q4_EINVAL;
  const void *outs[3] = {h, ws, logits};
  const size_t outb[3] = {sizeof(float) * 2048, q4::kDecodeWsBytes,
                          sizeof(float) * (size_t)emb->rows};
  q4::DecodeArgs a;
  const int rc = decode_args(emb, tok, layers, nlayers, eps, h, ws, ws_bytes, mode, outs, outb, 3,
                             &a);
  if (rc != Q4_OK) return rc;
  // wn_final is read, the outputs must not overlap it
  for (int i = 0; i < 3; ++i)
    if (overlap(outs[i], outb[i], wn_final, sizeof(float) * 2048)) return Q4_EINVAL;
  a.wf = wn_final;
  a.logits = logits;
  a.tok_out = tok;
  return hip_status(q4::launch_decode_layers(a, mode, static_cast<hipStream_t>(stream)));
}

int q4_decode_layers_status(void *ws, void *stream) {
  if (!ws || !aligned(ws, 16)) return Q4_EINVAL;
  return ws_status(ws, q4::kDecodeCtlOffset + 4 * (size_t)q4::kDecodeErrorWord,
                   q4::kDecodeWsBytes, stream);
}

size_t q4_atq_ws_bytes(int32_t hq, int32_t hkv) {
  if (hq < 1 || hq > q4::kAtqMaxHeads || hkv < 1 || hq % hkv != 0 ||
      hq / hkv > q4::kAtqMaxGroup)
    return 0;
  q4::AtqWs L;
  q4::atq_ws_layout(hq, hkv, &L);
  return L.bytes;
}

int q4_atq(const float *q, const float *g, const float *k, const float *v, const float *wq,
           const float *wk, float eps, const float *rope_cos, const float *rope_sin,
           float *kcache, float *vcache, const int32_t *pos, int32_t max_pos, int32_t hq,
           int32_t hkv, float *o, float *osum, void *ws, size_t ws_bytes, void *stream) {
  const size_t need = q4_atq_ws_bytes(hq, hkv);
  if (need == 0) return Q4_EINVAL;
  if (max_pos < 1 || max_pos > q4::kAtqMaxPos || !pos || !aligned(pos, 4)) return Q4_EINVAL;
  const float *in16[5] = {q, k, v, wq, wk};
  for (int i = 0; i < 5; ++i)
    if (!in16[i] || !aligned(in16[i], 16)) return Q4_EINVAL;
  if (!g || !aligned(g, 4) || !rope_cos || !aligned(rope_cos, 4) || !rope_sin ||
      !aligned(rope_sin, 4))
    return Q4_EINVAL;
  if (!kcache || !vcache || !aligned(kcache, 16) || !aligned(vcache, 16)) return Q4_EINVAL;
  if (!o || !aligned(o, 4) || !osum || !aligned(osum, 4)) return Q4_EINVAL;
  if (!ws || !aligned(ws, 256) || ws_bytes < need) return Q4_EINVAL;
  const size_t D = q4::kAtqD;
  const size_t qb = sizeof(float) * (size_t)hq * D, kb = sizeof(float) * (size_t)hkv * D;
  const size_t cb = sizeof(float) * (size_t)hkv * (size_t)max_pos * D;
  const size_t wb = sizeof(float) * D, rb = sizeof(float) * (size_t)max_pos * D / 2;
  // written: the caches, o, osum and the workspace; they overlap nothing
  const void *outs[5] = {kcache, vcache, o, osum, ws};
  const size_t outb[5] = {cb, cb, qb, sizeof(float) * (size_t)hq * 2, need};
  const void *ins[9] = {q, g, k, v, wq, wk, rope_cos, rope_sin, pos};
  const size_t inb[9] = {qb, qb, kb, kb, wb, wb, rb, rb, sizeof(int32_t)};
  for (int i = 0; i < 5; ++i) {
    for (int m = i + 1; m < 5; ++m)
      if (overlap(outs[i], outb[i], outs[m], outb[m])) return Q4_EINVAL;
    for (int m = 0; m < 9; ++m)
      if (overlap(outs[i], outb[i], ins[m], inb[m])) return Q4_EINVAL;
  }
  q4::AtqWs L;
  q4::atq_ws_layout(hq, hkv, &L);
  char *w = static_cast<char *>(ws);
  q4::AtqArgs a;
  a.q = q; a.g = g; a.k = k; a.v = v; a.wq = wq; a.wk = wk;
  a.cs = rope_cos; a.sn = rope_sin;
  a.kc = kcache; a.vc = vcache; a.o = o; a.os = osum;
  a.mx = reinterpret_cast<uint64_t *>(w + L.mx);
  a.zp = reinterpret_cast<uint64_t *>(w + L.zp);
  a.wp = reinterpret_cast<uint64_t *>(w + L.wp);
  a.ctl = reinterpret_cast<uint32_t *>(w + L.ctl);
  if (wait_ticks(&a.spin_ticks) != Q4_OK) return Q4_EHIP;
  a.pos = pos;
  a.eps = eps;
  a.max_pos = max_pos; a.hq = hq; a.hkv = hkv;
  return hip_status(q4::launch_atq(a, static_cast<hipStream_t>(stream)));
}

size_t q4_decode_block_ws_bytes(void) { return q4::kBlockWsBytes; }

namespace {

size_t cache_bytes(const q4_attn_block &b, int32_t max_pos) {
  return sizeof(float) * (size_t)b.hkv * (size_t)max_pos * q4::kAtqD;
}

// The checks of one block that do not depend on the call: shapes,
// alignment, and its two caches apart.  Sets *inter.
int check_block(const q4_attn_block &b, int32_t max_pos, int32_t *inter) {
  const int32_t hkv = b.hkv;
  if (hkv < 1 || hkv > q4::kBlockHeads || q4::kBlockHeads % hkv != 0) return Q4_EINVAL;
  if (check_mat(&b.qgkv) != Q4_OK || check_mat(&b.o) != Q4_OK) return Q4_EINVAL;
  if (b.qgkv.cols != 2048 || b.qgkv.rows != (2 * q4::kBlockHeads + 2 * hkv) * q4::kAtqD)
    return Q4_EINVAL;
  if (b.o.rows != 2048 || b.o.cols != 2048) return Q4_EINVAL;
  const q4_mlp_layer &L = b.mlp;
  if (check_mat(&L.gate_up) != Q4_OK || check_mat(&L.down) != Q4_OK) return Q4_EINVAL;
  const int32_t in = L.down.cols;
  if (in < 2048 || in % 2048 != 0 || in > q4::kDecodeMaxInter) return Q4_EINVAL;
  if (L.gate_up.cols != 2048 || L.gate_up.rows != 2 * in || L.down.rows != 2048)
    return Q4_EINVAL;
  const float *w[4] = {b.wa, b.wq, b.wk, L.wn};
  for (int i = 0; i < 4; ++i)
    if (!w[i] || !aligned(w[i], 16)) return Q4_EINVAL;
  if (!b.kcache || !b.vcache || !aligned(b.kcache, 16) || !aligned(b.vcache, 16))
    return Q4_EINVAL;
  if (max_pos < 1 || max_pos > q4::kBlockMaxPos) return Q4_EINVAL;
  const size_t cb = cache_bytes(b, max_pos);
  if (overlap(b.kcache, cb, b.vcache, cb)) return Q4_EINVAL;
  *inter = in;
  return Q4_OK;
}

// Does [p, p + bytes) overlap an array that the block only reads?
bool overlaps_weights(const void *p, size_t bytes, const q4_attn_block &b) {
  const size_t hb = sizeof(float) * 2048, wb = sizeof(float) * q4::kAtqD;
  return overlap(p, bytes, b.wa, hb) || overlap(p, bytes, b.wq, wb) ||
         overlap(p, bytes, b.wk, wb) || overlap(p, bytes, b.mlp.wn, hb) ||
         overlaps_mat(p, bytes, &b.qgkv) || overlaps_mat(p, bytes, &b.o) ||
         overlaps_mat(p, bytes, &b.mlp.gate_up) || overlaps_mat(p, bytes, &b.mlp.down);
}

// Does [p, p + bytes) overlap any array of the block?
bool overlaps_block(const void *p, size_t bytes, const q4_attn_block &b, int32_t max_pos) {
  const size_t cb = cache_bytes(b, max_pos);
  return overlap(p, bytes, b.kcache, cb) || overlap(p, bytes, b.vcache, cb) ||
         overlaps_weights(p, bytes, b);
}

// Each block's caches (written) overlap no other array of any block.
int check_caches(const q4_attn_block *b, int32_t n, int32_t max_pos) {
  for (int32_t i = 0; i < n; ++i) {
    const size_t cb = cache_bytes(b[i], max_pos);
    for (int32_t j = 0; j < n; ++j) {
      if (overlaps_weights(b[i].kcache, cb, b[j]) || overlaps_weights(b[i].vcache, cb, b[j]))
        return Q4_EINVAL;
      if (j != i && (overlaps_block(b[i].kcache, cb, b[j], max_pos) ||
                     overlaps_block(b[i].vcache, cb, b[j], max_pos)))
        return Q4_EINVAL;
    }
  }
  return Q4_OK;
}

// The arguments of one call: h and the workspace (written) overlap nothing
// else; the caches overlap none of the call's inputs.
int check_block_call(const q4_attn_block *b, int32_t n, int32_t max_pos, const float *h,
                     const int32_t *pos, const float *cs, const float *sn, const void *ws,
                     size_t ws_bytes) {
  if (!h || !aligned(h, 16) || !pos || !aligned(pos, 4)) return Q4_EINVAL;
  if (!cs || !sn || !aligned(cs, 16) || !aligned(sn, 16)) return Q4_EINVAL;
  if (!ws || !aligned(ws, 16) || ws_bytes < q4::kBlockWsBytes) return Q4_EINVAL;
  const size_t hb = sizeof(float) * 2048, wsb = q4::kBlockWsBytes;
  const size_t rb = sizeof(float) * (size_t)max_pos * q4::kAtqD / 2;
  if (overlap(h, hb, ws, wsb)) return Q4_EINVAL;
  const void *ins[3] = {cs, sn, pos};
  const size_t inb[3] = {rb, rb, sizeof(int32_t)};
  for (int m = 0; m < 3; ++m)
    if (overlap(h, hb, ins[m], inb[m]) || overlap(ws, wsb, ins[m], inb[m])) return Q4_EINVAL;
  for (int32_t i = 0; i < n; ++i) {
    if (overlaps_block(h, hb, b[i], max_pos) || overlaps_block(ws, wsb, b[i], max_pos))
      return Q4_EINVAL;
    const size_t cb = cache_bytes(b[i], max_pos);
    for (int m = 0; m < 3; ++m)
      if (overlap(b[i].kcache, cb, ins[m], inb[m]) || overlap(b[i].vcache, cb, ins[m], inb[m]))
        return Q4_EINVAL;
  }
  return Q4_OK;
}

q4::BlockLayer block_layer(const q4_attn_block &b) {
  q4::BlockLayer y;
  y.qq = b.qgkv.q; y.qs = b.qgkv.s; y.qb = b.qgkv.b;
  y.oq = b.o.q; y.os = b.o.s; y.ob = b.o.b;
  y.wa = b.wa; y.wq = b.wq; y.wk = b.wk;
  y.kc = b.kcache; y.vc = b.vcache;
  const q4_mlp_layer &L = b.mlp;
  y.mlp = q4::DecodeLayer{L.gate_up.q, L.gate_up.s, L.gate_up.b, L.wn, L.down.q, L.down.s, L.down.b};
  return y;
}

int launch_blocks(const q4::BlockLayer &one, const q4::BlockLayer *table, int32_t n, int32_t hkv,
                  int32_t inter, int32_t max_pos, float eps, float *h, const int32_t *pos,
                  const float *cs, const float *sn, void *ws, int mode, void *stream) {
  q4::DecodeBlockArgs a;
  memset(&a, 0, sizeof(a));
  a.one = one;
  a.layers = table;
  a.nlayers = n;
  a.cs = cs; a.sn = sn; a.pos = pos;
  a.max_pos = max_pos; a.hkv = hkv; a.inter = inter;
  a.h = h;
  char *w = static_cast<char *>(ws);
  a.qv = reinterpret_cast<uint64_t *>(w + q4::kBlockQvOffset);
  a.ov = reinterpret_cast<uint64_t *>(w + q4::kBlockOvOffset);
  a.hv = reinterpret_cast<uint64_t *>(w + q4::kBlockHvOffset);
  a.mq = reinterpret_cast<uint64_t *>(w + q4::kBlockMqOffset);
  a.hb = reinterpret_cast<uint64_t *>(w + q4::kBlockHbOffset);
  a.mx = reinterpret_cast<uint64_t *>(w + q4::kBlockMxOffset);
  a.zp = reinterpret_cast<uint64_t *>(w + q4::kBlockZpOffset);
  a.wp = reinterpret_cast<uint64_t *>(w + q4::kBlockWpOffset);
  a.ctl = reinterpret_cast<uint32_t *>(w + q4::kBlockCtlOffset);
  a.eps = eps;
  if (wait_ticks(&a.spin_ticks) != Q4_OK) return Q4_EHIP;
  if (q4::decode_block_grid(mode, inter) < 1) return Q4_EINVAL;  // too few compute units
  return hip_status(q4::launch_decode_block(a, mode, static_cast<hipStream_t>(stream)));
}

}  // namespace

struct q4_block_stack {
  // host copy, for the checks of each call (a plain array: a template
  // instantiated on the public type would be exported)
  q4_attn_block *blocks = nullptr;
  int32_t n = 0;
  q4::BlockLayer *table = nullptr;  // device copy of the layers' arrays
  int32_t max_pos = 0, inter = 0;
  ~q4_block_stack() { delete[] blocks; }
};

int q4_decode_block(const q4_attn_block *blk, float eps, float *h, const int32_t *pos,
                    int32_t max_pos, const float *rope_cos, const float *rope_sin, void *ws,
                    size_t ws_bytes, int mode, void *stream) {
  if (mode != Q4_FIXED && mode != Q4_FAST) return Q4_EINVAL;
  if (!blk) return Q4_EINVAL;
  int32_t inter = 0;
  if (check_block(*blk, max_pos, &inter) != Q4_OK || check_caches(blk, 1, max_pos) != Q4_OK ||
      check_block_call(blk, 1, max_pos, h, pos, rope_cos, rope_sin, ws, ws_bytes) != Q4_OK)
    return Q4_EINVAL;
  return launch_blocks(block_layer(*blk), nullptr, 1, blk->hkv, inter, max_pos, eps, h, pos,
                       rope_cos, rope_sin, ws, mode, stream);
}

int q4_block_stack_create(const q4_attn_block *blocks, int32_t nlayers, int32_t max_pos,
                          q4_block_stack **out) {
  if (!out) return Q4_EINVAL;
  *out = nullptr;
  if (!blocks || nlayers < 1 || nlayers > q4::kBlockMaxLayers) return Q4_EINVAL;
  int32_t inter = 0;
  for (int32_t i = 0; i < nlayers; ++i) {
    int32_t in = 0;
    if (check_block(blocks[i], max_pos, &in) != Q4_OK) return Q4_EINVAL;
    if (i > 0 && (in != inter || blocks[i].hkv != blocks[0].hkv)) return Q4_EINVAL;
    inter = in;
  }
  if (check_caches(blocks, nlayers, max_pos) != Q4_OK) return Q4_EINVAL;
  q4_block_stack *s = new (std::nothrow) q4_block_stack();
  if (!s) return Q4_ENOMEM;
  std::vector<q4::BlockLayer> host;
  try {
    host.resize(nlayers);
  } catch (...) {
    delete s;
    return Q4_ENOMEM;
  }
  s->blocks = new (std::nothrow) q4_attn_block[nlayers];
  if (!s->blocks) {
    delete s;
    return Q4_ENOMEM;
  }
  s->n = nlayers;
  for (int32_t i = 0; i < nlayers; ++i) {
    s->blocks[i] = blocks[i];
    host[i] = block_layer(blocks[i]);
  }
  const size_t bytes = sizeof(q4::BlockLayer) * (size_t)nlayers;
  if (hipMalloc(&s->table, bytes) != hipSuccess) {
    delete s;
    return Q4_EHIP;
  }
  if (hipMemcpy(s->table, host.data(), bytes, hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(s->table);
    delete s;
    return Q4_EHIP;
  }
  s->max_pos = max_pos;
  s->inter = inter;
  *out = s;
  return Q4_OK;
}

int q4_block_stack_destroy(q4_block_stack *s) {
  if (!s) return Q4_EINVAL;
  const hipError_t e = hipFree(s->table);
  delete s;
  return hip_status(e);
}

int q4_decode_blocks(const q4_block_stack *s, float eps, float *h, const int32_t *pos,
                     const float *rope_cos, const float *rope_sin, void *ws, size_t ws_bytes,
                     int mode, void *stream) {
  if (mode != Q4_FIXED && mode != Q4_FAST) return Q4_EINVAL;
  if (!s) return Q4_EINVAL;
  const int32_t n = s->n;
  if (check_block_call(s->blocks, n, s->max_pos, h, pos, rope_cos, rope_sin, ws, ws_bytes) !=
      Q4_OK)
    return Q4_EINVAL;
  q4::BlockLayer none;
  memset(&none, 0, sizeof(none));
  return launch_blocks(none, s->table, n, s->blocks[0].hkv, s->inter, s->max_pos, eps, h, pos,
                       rope_cos, rope_sin, ws, mode, stream);
}

int q4_decode_block_status(void *ws, void *stream) {
  if (!ws || !aligned(ws, 16)) return Q4_EINVAL;
  return ws_status(ws, q4::kBlockCtlOffset + 4 * (size_t)q4::kBlockErrorWord, q4::kBlockWsBytes,
                   stream);
}

int q4_pos_advance(int32_t *pos, void *stream) {
  if (!pos || !aligned(pos, 4)) return Q4_EINVAL;
  return hip_status(q4::launch_pos_advance(pos, static_cast<hipStream_t>(stream)));
}

int q4_atq_status(void *ws, int32_t hq, int32_t hkv, void *stream) {
  const size_t need = q4_atq_ws_bytes(hq, hkv);
  if (need == 0 || !ws || !aligned(ws, 256)) return Q4_EINVAL;
  q4::AtqWs L;
  q4::atq_ws_layout(hq, hkv, &L);
  return ws_status(ws, L.ctl + 4 * (size_t)q4::kAtqErrorWord, need, stream);
}

int q4_queue_create(void *stream, int mode, q4_queue **out) {
  if (!out || (mode != Q4_FIXED && mode != Q4_FAST)) return Q4_EINVAL;
  *out = nullptr;
  q4_queue *q = new (std::nothrow) q4_queue();
  if (!q) return Q4_ENOMEM;
  q->st = static_cast<hipStream_t>(stream);
  q->mode = mode;
  q->debug = env_flag("Q4MV_DEBUG_CHECKS");
  q->trace = env_flag("Q4MV_TRACE");
  if (q->trace) {
    if (hipEventCreate(&q->ev_begin) != hipSuccess || hipEventCreate(&q->ev_end) != hipSuccess) {
      if (q->ev_begin) (void)hipEventDestroy(q->ev_begin);
      delete q;
      return Q4_EHIP;
    }
  }
  *out = q;
  return Q4_OK;
}

int q4_queue_destroy(q4_queue *q) {
  if (!q) return Q4_EINVAL;
  int rc = Q4_OK;
  if (q->mailbox && q4_mailbox_destroy(q->mailbox) != Q4_OK) rc = Q4_EHIP;
  if (q->ev_begin && hipEventDestroy(q->ev_begin) != hipSuccess) rc = Q4_EHIP;
  if (q->ev_end && hipEventDestroy(q->ev_end) != hipSuccess) rc = Q4_EHIP;
  delete q;
  return rc;
}

int q4_queue_set_wait(q4_queue *q, int how, int32_t timeout_ms) {
  if (!q || (how != Q4_WAIT_STREAM && how != Q4_WAIT_MAILBOX) || timeout_ms < 0) return Q4_EINVAL;
  if (how == Q4_WAIT_STREAM) {
    if (q->mailbox) {
      // posts still in flight write into the mailbox: let them land first
      if (hipStreamSynchronize(q->st) != hipSuccess) return Q4_EHIP;
      const int rc = q4_mailbox_destroy(q->mailbox);
      q->mailbox = nullptr;
      if (rc != Q4_OK) return rc;
    }
    return Q4_OK;
  }
  if (!q->mailbox) {
    const int rc = q4_mailbox_create(1, &q->mailbox);
    if (rc != Q4_OK) return rc;
    q->posted = 0;
  }
  q->timeout_ms = timeout_ms;
  return Q4_OK;
}

int q4mv_queue(q4_queue *q, const q4_mat *w, const float *x, const float *xsum, float *y) {
  if (!q) return Q4_EINVAL;
  Prod p;
  const int rc = make_prod(w, x, xsum, nullptr, y, &p);
  if (rc != Q4_OK) return rc;
  if (q->debug) {
    // products of one stage may run concurrently: none may read another's y
    const size_t yb = sizeof(float) * (size_t)p.rows;
    for (const Prod &o : q->stage) {
      const size_t ob = sizeof(float) * (size_t)o.rows;
      if (overlap(p.y, yb, o.x, sizeof(float) * (size_t)o.cols) ||
          (o.xs && overlap(p.y, yb, o.xs, sizeof(float) * (size_t)(o.cols / 64))) ||
          overlap(o.y, ob, p.x, sizeof(float) * (size_t)p.cols) ||
          (p.xs && overlap(o.y, ob, p.xs, sizeof(float) * (size_t)(p.cols / 64))) ||
          overlap(o.y, ob, p.y, yb))
        return Q4_EINVAL;
    }
  }
  try {
    q->stage.push_back(p);
  } catch (...) {
    return Q4_ENOMEM;
  }
  return Q4_OK;
}

int q4_stage(q4_queue *q) {
  if (!q) return Q4_EINVAL;
  return flush_stage(q);
}

int q4mv_wait(q4_queue *q) {
  if (!q) return Q4_EINVAL;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(q->st, &cs) != hipSuccess) return Q4_EHIP;
  if (cs != hipStreamCaptureStatusNone) return Q4_ESTATE;
  int rc = flush_stage(q);
  if (rc != Q4_OK) return rc;
  if (q->trace && q->began) {
    if (hipEventRecord(q->ev_end, q->st) != hipSuccess) return Q4_EHIP;
  }
  if (q->mailbox) {
    // a one-thread kernel after the last stage publishes the next number
    const int32_t *any = reinterpret_cast<const int32_t *>(q->mailbox->dev_count);
    rc = q4_mailbox_post(q->mailbox, any, q->st);
    if (rc != Q4_OK) return rc;
    rc = q4_mailbox_wait(q->mailbox, ++q->posted, nullptr, q->timeout_ms);
    if (rc != Q4_OK) return rc;
  } else if (hipStreamSynchronize(q->st) != hipSuccess) {
    return Q4_EHIP;
  }
  if (q->trace && q->began && q->mailbox && hipEventSynchronize(q->ev_end) != hipSuccess)
    return Q4_EHIP;
  if (q->trace && q->began) {
    float gpu_ms = 0.0f;
    if (hipEventElapsedTime(&gpu_ms, q->ev_begin, q->ev_end) != hipSuccess) return Q4_EHIP;
    const double wall_ms =
        std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - q->wall_begin)
            .count();
    fprintf(stderr, "q4mv_wait: %d products, gpu %.3f ms, wall %.3f ms\n",
            q->products_since_wait, gpu_ms, wall_ms);
  }
  q->began = false;
  q->products_since_wait = 0;
  return Q4_OK;
}

int q4_capture_begin(void *stream) {
  if (!stream) return Q4_EINVAL;  // the null stream cannot be captured
  return hip_status(
      hipStreamBeginCapture(static_cast<hipStream_t>(stream), hipStreamCaptureModeRelaxed));
}

int q4_capture_end(void *stream, q4_graph **out) {
  if (!stream || !out) return Q4_EINVAL;
  *out = nullptr;
  q4_graph *g = new (std::nothrow) q4_graph();
  if (!g) return Q4_ENOMEM;
  if (hipStreamEndCapture(static_cast<hipStream_t>(stream), &g->graph) != hipSuccess ||
      !g->graph) {
    delete g;
    return Q4_EHIP;
  }
  if (hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0) != hipSuccess) {
    (void)hipGraphDestroy(g->graph);
    delete g;
    return Q4_EHIP;
  }
  *out = g;
  return Q4_OK;
}

int q4_graph_launch(q4_graph *g, void *stream) {
  if (!g || !g->exec) return Q4_EINVAL;
  return hip_status(hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream)));
}

int q4_graph_destroy(q4_graph *g) {
  if (!g) return Q4_EINVAL;
  int rc = Q4_OK;
  if (g->exec && hipGraphExecDestroy(g->exec) != hipSuccess) rc = Q4_EHIP;
  if (g->graph && hipGraphDestroy(g->graph) != hipSuccess) rc = Q4_EHIP;
  delete g;
  return rc;
}

int q4_mailbox_create(int32_t nvals, q4_mailbox **out) {
  if (!out || nvals < 1 || nvals > Q4_MAILBOX_MAX_VALUES) return Q4_EINVAL;
  *out = nullptr;
  q4_mailbox *mb = new (std::nothrow) q4_mailbox();
  if (!mb) return Q4_ENOMEM;
  mb->n = nvals;
  void *host = nullptr;
  // 64 bytes for the sequence number, then the values
  const size_t bytes = 64 + sizeof(int32_t) * (size_t)nvals;
  if (hipHostMalloc(&host, bytes, hipHostMallocMapped | hipHostMallocCoherent) != hipSuccess) {
    delete mb;
    return Q4_EHIP;
  }
  memset(host, 0, bytes);
  mb->host_seq = static_cast<uint32_t *>(host);
  mb->host_vals = reinterpret_cast<int32_t *>(static_cast<char *>(host) + 64);
  void *dview = nullptr;
  if (hipHostGetDevicePointer(&dview, host, 0) != hipSuccess ||
      hipMalloc(&mb->dev_count, sizeof(uint32_t)) != hipSuccess ||
      hipMemset(mb->dev_count, 0, sizeof(uint32_t)) != hipSuccess) {
    if (mb->dev_count) (void)hipFree(mb->dev_count);
    (void)hipHostFree(host);
    delete mb;
    return Q4_EHIP;
  }
  mb->dev_seq_view = static_cast<uint32_t *>(dview);
  mb->dev_vals_view = reinterpret_cast<int32_t *>(static_cast<char *>(dview) + 64);
  *out = mb;
  return Q4_OK;
}

int q4_mailbox_destroy(q4_mailbox *mb) {
  if (!mb) return Q4_EINVAL;
  int rc = Q4_OK;
  if (hipFree(mb->dev_count) != hipSuccess) rc = Q4_EHIP;
  if (hipHostFree(mb->host_seq) != hipSuccess) rc = Q4_EHIP;
  delete mb;
  return rc;
}

int q4_mailbox_post(q4_mailbox *mb, const int32_t *vals, void *stream) {
  if (!mb || !vals || !aligned(vals, 4)) return Q4_EINVAL;
  return hip_status(q4::launch_mailbox(vals, mb->n, mb->dev_vals_view, mb->dev_seq_view,
                                       mb->dev_count, static_cast<hipStream_t>(stream)));
}

int q4_mailbox_wait(q4_mailbox *mb, uint32_t target, int32_t *vals, int32_t timeout_ms) {
  if (!mb || timeout_ms < 0) return Q4_EINVAL;
  const auto t0 = std::chrono::steady_clock::now();
  const auto limit = std::chrono::milliseconds(timeout_ms);
  for (uint64_t spin = 0;; ++spin) {
    const uint32_t seq = __atomic_load_n(mb->host_seq, __ATOMIC_ACQUIRE);
    if ((int32_t)(seq - target) >= 0) break;
    if ((spin & 1023) == 1023 && std::chrono::steady_clock::now() - t0 > limit) return Q4_ETIMEOUT;
  }
  if (vals)
    for (int32_t i = 0; i < mb->n; ++i) vals[i] = __atomic_load_n(mb->host_vals + i, __ATOMIC_RELAXED);
  return Q4_OK;
}

uint32_t q4_mailbox_seq(const q4_mailbox *mb) {
  return mb ? __atomic_load_n(mb->host_seq, __ATOMIC_ACQUIRE) : 0u;
}

int q4_sync(void *stream) {
  return hip_status(hipStreamSynchronize(static_cast<hipStream_t>(stream)));
}

const char *q4_strerror(int code) {
  switch (code) {
    case Q4_OK: return "ok";
    case Q4_EINVAL: return "invalid argument (nothing was launched)";
    case Q4_EHIP: return "HIP runtime error";
    case Q4_ETIMEOUT: return "a bounded wait timed out";
    case Q4_ESTATE: return "call not legal in the current state (e.g. host wait during capture)";
    case Q4_ENOMEM: return "host allocation failed";
    default: return "unknown status";
  }
}

}  // extern "C"
