/*
 * q4mv.h -- C ABI of libq4mv.so: the affine 4-bit matvec (q4mv), its
 * producers (rmsq, swq), the greedy-decode glue (argmax, embed), a
 * stage queue with a single host wait, and whole-token graph capture,
 * for AMD Instinct MI355X (gfx950).
 *
 * The operations come from three pull-request pages of the Bend language
 * repository (bendlang/bend):
 *   [P1] "Metal: queued rmsq, swq, gdn and atq kernels and a 4-row q4mv, so
 *        a decode token is one command buffer with one wait" (#1440)
 *   [P2] "Array.q4go / Array.q4wait queue Metal Q4 products in one command
 *        buffer and wait once on a flag" (#1437)
 *   [P3] "Array.q4mv on Metal: one kernel thread per row for products of 4M
 *        weights or more, bit-identical" (#1435)
 *
 * Conventions for every entry point
 *   - Pointers named "device" must point to GPU memory of the current HIP
 *     device; the caller allocates and owns every buffer, and must keep it
 *     alive until the work that uses it has completed (for the queue: until
 *     q4mv_wait returns -- the lifetime rule of [P2], Change).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls only
 *     enqueue work and return; they are legal inside stream capture, except
 *     q4mv_wait, which waits on the host.
 *   - Arguments are checked before anything is launched.  A bad argument
 *     returns Q4_EINVAL and launches nothing; a failed launch returns
 *     Q4_EHIP.  There is no CPU fallback and no size threshold.
 *   - Outputs must not overlap inputs unless stated.
 */
#ifndef Q4MV_H
#define Q4MV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define Q4_OK 0
#define Q4_EINVAL (-1)   /* bad argument; nothing was launched            */
#define Q4_EHIP (-2)     /* a HIP runtime call failed                     */
#define Q4_ETIMEOUT (-3) /* a bounded wait (host or device) ran out       */
#define Q4_ESTATE (-4)   /* call not legal now (e.g. host wait in capture) */
#define Q4_ENOMEM (-5)   /* host allocation failed                        */

/* Modes of q4mv and swq. */
#define Q4_FIXED 0 /* fixed operation order: bit-identical to the reference */
#define Q4_FAST 1  /* any order, fused multiply-add: relative error <= 1e-5 */

/* Size limits of this build. */
#define Q4_MAX_COLS 32768 /* q4mv: cols <= 32768 (512 groups)          */
#define Q4_MAX_RMSQ_N 8192 /* rmsq: n <= 8192                          */
#define Q4_MAX_DECODE_LAYERS 32 /* q4_decode_layers: layers per call    */

/*
 * One affine Q4 matrix ([P3] Why/Change: rows of 4-bit codes; [P1] Change:
 * 64-value groups).  Layout (all device, row-major):
 *   q : uint32[rows][cols/8]; column 8j+k is held in bits 4k..4k+3 of word
 *       j of its row (low nibble first).  16-byte aligned.
 *   s : float[rows][cols/64] scale of each 64-column group.  4-byte aligned.
 *   b : float[rows][cols/64] bias of each group.          4-byte aligned.
 * rows >= 1; cols a positive multiple of 64, at most Q4_MAX_COLS.
 * Dequantised weight: W[r][c] = s[r][c/64] * q(r,c) + b[r][c/64].
 */
typedef struct q4_mat {
  const uint32_t *q;
  const float *s;
  const float *b;
  int32_t rows;
  int32_t cols;
} q4_mat;

/*
 * q4mv: y[r] = sum_g s[r,g] * (q[r,g] . x_g) + b[r,g] * xsum[g]
 * ([P3] Change: the product itself; [P1] Change, rmsq bullet: the group
 * sums it reads; [P1] Change, q4mv bullet: each row keeps a fixed
 * summation tree).
 *   w    : host pointer to the matrix descriptor (read during the call).
 *   x    : device float[cols], 16-byte aligned.
 *   xsum : device float[cols/64]; xsum[g] is the sum of x[64g..64g+63]
 *          as emitted by rmsq/swq (an input: never recomputed).  NULL asks
 *          the kernel to form the group sums of x itself with the same
 *          tree rmsq and swq use (same bits as passing them).
 *   y    : device float[rows]; must not overlap w, x or xsum.
 *   mode : Q4_FIXED -- per row, p_i = q_i * x_i, d_g = T(p over the group),
 *          t_g = (s*d_g) + (b*xsum_g) unfused, y = T(t over groups), with T
 *          the canonical tree (split at the largest power of two below n);
 *          bit-identical to the reference.  Q4_FAST -- reordered, fused;
 *          |err| <= 1e-5*|y| + 1e-5*rms(y).
 */
int q4mv(const q4_mat *w, const float *x, const float *xsum, float *y, int mode,
         void *stream);

/*
 * q4mv_add: y[r] = resid[r] + (W x)[r], the product of q4mv followed by one
 * binary32 addition (a decode chain's residual, fused into the product's
 * store).  resid: device float[rows]; it may be the same array as y.
 */
int q4mv_add(const q4_mat *w, const float *x, const float *xsum,
             const float *resid, float *y, int mode, void *stream);

/*
 * Fused stages ([P1] Change: rmsq, swq and the 4-row q4mv as one queued
 * sequence; [P1] Verification: one command buffer per token).  Each gives
 * the bits of the separate calls it replaces; each needs cols == 2048.
 *
 * q4mv_norm: y = W rmsq(h, wn)  (rmsq's arithmetic in the product's
 *   prologue).  h, wn: device float[cols], 16-byte aligned.  u, usum:
 *   optional outputs (both or neither; float[cols] 16-byte aligned and
 *   float[cols/64]) receiving rmsq's u and group sums.  For cols != 2048 it
 *   runs rmsq into u, usum (then required) and q4mv: two launches.
 */
int q4mv_norm(const q4_mat *w, const float *h, const float *wn, float eps, float *y, float *u,
              float *usum, int mode, void *stream);

/*
 * q4mv_norm_swiglu: m = swq(W rmsq(h, wn)) for a matrix whose rows come in
 *   (gate, up) pairs: row 2i is gate row i, row 2i+1 up row i.  m: device
 *   float[rows/2]; rows even; cols == 2048.  The group sums of m are not
 *   written: pass xsum = NULL to the product that reads m.
 */
int q4mv_norm_swiglu(const q4_mat *w, const float *h, const float *wn, float eps, float *m,
                     int mode, void *stream);

/*
 * q4mv_norm_argmax: y = W rmsq(h, wn) and *idx = q4_argmax(y) (cols ==
 *   2048): the product kernel also leaves the key of each workgroup's best
 *   row in ws, and one small kernel picks the largest.  ws: device
 *   workspace, 8-byte aligned, of q4mv_argmax_ws_bytes() bytes (fewer bytes
 *   limit the product to one workgroup per 8 bytes); no initialisation
 *   needed.  Calls that overlap in time must not share it.
 */
size_t q4mv_argmax_ws_bytes(void);
int q4mv_norm_argmax(const q4_mat *w, const float *h, const float *wn, float eps, float *y,
                     int32_t *idx, void *ws, size_t ws_bytes, int mode, void *stream);

/*
 * q4mv_norm_argmax_noalloc: q4mv_norm_argmax without a caller workspace, for
 *   callers that cannot allocate device memory (code under stream capture,
 *   tight serving loops, harnesses that forbid allocation).  The
 *   workgroups' keys go to a static device array of the library (32 KiB per
 *   GPU, held until the process ends; its address is looked up on the first
 *   call on each device).  The call allocates nothing.  Same arguments,
 *   results and errors as q4mv_norm_argmax with a full workspace; any rows
 *   count is accepted (the product uses at most 4096 workgroups, one key
 *   each).  Every call on one GPU shares that array: calls that overlap in
 *   time on one GPU (other streams, other threads) race and must not be
 *   issued.  Nothing in it needs to start at zero: each call writes every
 *   key it reads.
 */
int q4mv_norm_argmax_noalloc(const q4_mat *w, const float *h, const float *wn, float eps,
                             float *y, int32_t *idx, int mode, void *stream);

/*
 * q4mv_variant: q4mv of a 2048-column matrix by one of the kernel designs
 * the pages compare, for measuring them side by side (same arguments as
 * q4mv; xsum required; same results: bit-identical in Q4_FIXED).
 *   Q4_VARIANT_LANE_PER_ROW  one lane per row, walking its row's groups in
 *                            order ([P3] Change: one kernel thread per row;
 *                            [P3] Limits: its strided reads stay below the
 *                            memory bandwidth).
 *   Q4_VARIANT_WAVE_R1 / R2 / R4 / R8
 *                            one wave per row, 1, 2, 4 or 8 rows per block
 *                            sharing each lane's activations ([P1] Change,
 *                            q4mv bullet: 4 rows of a SIMD group share each
 *                            activation group; Verification: 2 and 8 rows
 *                            were no better).  R4 is the kernel q4mv runs.
 */
#define Q4_VARIANT_LANE_PER_ROW 0
#define Q4_VARIANT_WAVE_R1 1
#define Q4_VARIANT_WAVE_R2 2
#define Q4_VARIANT_WAVE_R4 4
#define Q4_VARIANT_WAVE_R8 8
int q4mv_variant(const q4_mat *w, const float *x, const float *xsum, float *y, int variant,
                 int mode, void *stream);

/*
 * rmsq: the RMS norm of h scaled by float weights, and the sum of each 64
 * consecutive outputs, which is the xsum input of the next q4mv ([P1]
 * Change, rmsq bullet; bit-exact on the pages' GPU).
 *   ss = T(h_i*h_i); rho = 1 / sqrt(ss/n + eps)  (correctly rounded);
 *   u_i = (h_i*rho)*w_i;  usum[g] = T(u[64g..64g+63]).
 *   h, w : device float[n];  u : device float[n];  usum : device float[n/64].
 *   n a positive multiple of 64, at most Q4_MAX_RMSQ_N.  u may not overlap h.
 */
int rmsq(const float *h, const float *w, int32_t n, float eps, float *u,
         float *usum, void *stream);

/*
 * swq: SwiGLU, o[i] = silu(a[i]) times a[n+i], rounded, plus group sums
 * ([P1] Change, swq bullet).
 *   a    : device float[2n], gate in a[0..n), up in a[n..2n).
 *   o    : device float[n];  osum : device float[n/64].
 *   n a positive multiple of 64 (the n = 32 case the pages criticise is
 *   Q4_EINVAL here, not a silently untouched o).
 *   mode : Q4_FIXED -- binary64 silu a/(1+E(-a)) with E a fixed binary64
 *          exp (Cody-Waite reduction by ln 2, degree-13 Taylor polynomial by
 *          fused Horner, ldexp), one rounding of the binary64 product to
 *          binary32; bit-identical to the reference.  Q4_FAST -- binary32.
 */
int swq(const float *a, int32_t n, float *o, float *osum, int mode,
        void *stream);

/*
 * q4_argmax: greedy pick for a decode chain ([P1] Verification: greedy token
 * ids).  *idx = lowest index of the largest value of v[0..n); -1 when any
 * value is NaN.  -0 and +0 compare equal.
 *   v   : device float[n], n >= 1.   idx : device int32[1].
 *   ws  : device workspace of at least q4_argmax_ws_bytes(n) bytes, 8-byte
 *         aligned, owned by the caller; calls that overlap in time must not
 *         share it.
 */
size_t q4_argmax_ws_bytes(int32_t n);
int q4_argmax(const float *v, int32_t n, int32_t *idx, void *ws,
              size_t ws_bytes, void *stream);

/*
 * q4_embed: the input row of the next greedy step ([P1] Verification: the
 * greedy decode whose token ids are compared, one token feeding the next),
 * looked up in a tied Q4 matrix: e[c] = (s[t,c/64] *
 * q(t,c)) + b[t,c/64] with t = *tok read on the device (so a captured graph
 * can feed argmax's output straight back).  A token outside [0, rows) fills
 * e with quiet NaNs.  tok: device int32[1]; e: device float[cols].
 */
int q4_embed(const q4_mat *w, const int32_t *tok, float *e, void *stream);

/*
 * The MLP layers of a decode token as one persistent kernel ([P1] Change:
 * rmsq, swq and the 4-row q4mv queued for a whole decode token; [P1]
 * Verification: one command buffer and one wait per token).  Computes
 *   h = e_tok  (the q4_embed row of *tok)
 *   for each layer:  h = h + down * swq(gate_up * rmsq(h, wn))
 * with the bits of the separate calls: q4_embed, then per layer
 * q4mv_norm_swiglu(gate_up, h, wn, eps, m) and q4mv_add(down, m, NULL, h, h).
 * One launch of one workgroup per compute unit (the device needs at least
 * 256 of them); the stages hand their outputs to each other through tagged
 * words in the workspace that the consumers poll, with no grid barrier, and
 * each wave loads its next stage's weights before it waits.
 *
 *   emb     : host pointer to the embedding matrix (cols == 2048), the
 *             decode head's tied weights.  A token outside [0, rows) makes
 *             h NaN.
 *   tok     : device int32[1], read on the device.
 *   layers  : host array of nlayers (1..Q4_MAX_DECODE_LAYERS) descriptors,
 *             read during the call.  gate_up: rows 2*inter, cols 2048, gate
 *             row i at row 2i and up row i at row 2i+1.  down: rows 2048,
 *             cols inter; inter (taken from layers[0].down.cols) is 2048,
 *             4096, 6144 or 8192 and the same in every layer.  wn: device
 *             float[2048], 16-byte aligned.
 *   h       : device float[2048]: the output (its prior contents are not
 *             read).
 *   ws      : device workspace of q4_decode_layers_ws_bytes() bytes (about
 *             2.0 MB), 16-byte aligned, zero-filled before its first use;
 *             each call leaves it ready for the next.  Calls that overlap in
 *             time must not share it, and no other kernel should hold the
 *             device's compute units while this one runs.
 * h and ws must not overlap each other or any input.  Each wait for another
 * workgroup's output is bounded (env Q4_DECODE_TIMEOUT_MS, default 2000, at
 * most 60000; negative: no waiting at all, for tests of this path): when
 * one runs out, every workgroup leaves the kernel and h is undefined;
 * q4_decode_layers_status reports it.  A workspace whose error word is set
 * makes the kernel return at once until the status call clears it.
 * h between layers goes through the L2 of each XCD (the XCD's workgroups
 * relay slices of it); a wait for h that its XCD's copy has not served
 * within Q4_DECODE_NEAR_US microseconds (env, default 50) reads the
 * device-scope copy from then on in that call.
 * Q4_EINVAL also when the device has fewer than 256 compute units.
 */
typedef struct q4_mlp_layer {
  q4_mat gate_up;
  q4_mat down;
  const float *wn;
} q4_mlp_layer;
size_t q4_decode_layers_ws_bytes(void);
int q4_decode_layers(const q4_mat *emb, const int32_t *tok, const q4_mlp_layer *layers,
                     int32_t nlayers, float eps, float *h, void *ws, size_t ws_bytes, int mode,
                     void *stream);

/*
 * A whole greedy decode step in one persistent launch ([P1] Change and
 * Verification: a decode token as one command buffer with one wait, greedy
 * token ids): q4_decode_layers, then the final RMS norm, the head product
 * over the same tied matrix and its argmax, with the bits of
 *   q4_decode_layers(emb, tok, layers, nlayers, eps, h, ...);
 *   q4mv_norm_argmax(emb, h, wn_final, eps, logits, tok, ...)
 * The token is read at the start and the next one written over it at the
 * end, so a graph of this one call replays token after token.  After the
 * last layer h is handed to every workgroup as between layers; each forms
 * rmsq(h, wn_final) once and every wave sums its blocks of 4 head rows (the
 * first loaded during the last layer); workgroup 0 gathers the workgroups'
 * best (value, index) keys through tagged words and writes the token.
 *   emb     : as for q4_decode_layers; also the head (vocab = emb->rows).
 *   tok     : device int32[1], read, then overwritten with the next token
 *             (-1 when a logit is NaN).
 *   wn_final: device float[2048], 16-byte aligned.
 *   h       : device float[2048]: the hidden state after the last layer.
 *   logits  : device float[emb->rows].
 *   ws      : as for q4_decode_layers (the same size and status call).
 * h, logits and ws must overlap each other and no input.  Errors and
 * bounded waits as for q4_decode_layers; a wait that runs out leaves the
 * token unwritten.
 */
int q4_decode_token(const q4_mat *emb, int32_t *tok, const q4_mlp_layer *layers, int32_t nlayers,
                    const float *wn_final, float eps, float *h, float *logits, void *ws,
                    size_t ws_bytes, int mode, void *stream);

/*
 * Waits for `stream` on the host, then returns Q4_ETIMEOUT if a wait of a
 * q4_decode_layers call using `ws` ran out since the workspace was last
 * cleared (and clears the whole workspace), else Q4_OK.  Q4_ESTATE during
 * capture.
 */
int q4_decode_layers_status(void *ws, void *stream);

/*
 * Gated attention of one decode token over key/value caches ([P1] Change,
 * atq bullet, which lists the parts without formulas: normalise and rotate
 * the query and new key, append key and value to the caches, softmax-weight
 * the cached values by score, gate with a sigmoid, emit 64-value sums for
 * the next product; several query heads per key/value head).  The pages state no
 * formulas; the operations as read, D = 128, G = hq / hkv, query head h
 * using key/value head j = h / G, n = pos + 1:
 *   qn = rmsq(q_h, wq), kn = rmsq(k_j, wk)          (rmsq over 128 values)
 *   rotate(x)_i      = (x_i c_i) - (x_{i+64} s_i)      i < 64, with
 *   rotate(x)_{i+64} = (x_i s_i) + (x_{i+64} c_i)      c = rope_cos, s = rope_sin
 *   kcache[j][pos] = rotate(kn), vcache[j][pos] = v_j
 *   s_t = T(rotate(qn) * kcache[j][t]) * RN32(1/sqrt(128)),  t < n
 *   e_t = RN32(E(s_t - max_t s_t))   (E: the fixed binary64 exp of swq)
 *   o_h = (T(e_t * vcache[j][t] over t) / T(e)) * RN32(1 / (1 + E(-g_h)))
 *   osum[2h + b] = T(o_h[64b .. 64b+63])
 * with T the canonical tree of q4mv; bit-identical to the reference.
 *
 *   q, g    : device float[hq][128] query and gate; q 16-byte aligned.
 *   k, v    : device float[hkv][128] new key and value, 16-byte aligned.
 *   wq, wk  : device float[128] norm weights, 16-byte aligned.
 *   eps     : the epsilon of both norms (as rmsq's).
 *   rope_cos, rope_sin : device float[max_pos][64], the rotation tables
 *             of every position; row pos is read.
 *   kcache, vcache : device float[hkv][max_pos][128], 16-byte aligned; rows
 *             below pos are read, row pos is written, others untouched.
 *   pos     : device int32[1], the token's position, read on the device (so
 *             that a captured graph can be replayed token after token).  A
 *             position outside [0, max_pos) writes no cache row and fills o
 *             and osum with quiet NaNs.  max_pos <= Q4_ATQ_MAX_POS.
 *   hq, hkv : 1 <= hkv, hq % hkv == 0, hq / hkv <= 8, hq <= 128.
 *   o       : device float[hq][128]; osum: device float[hq][2].
 *   ws      : device workspace of q4_atq_ws_bytes(hq, hkv) bytes, 256-byte
 *             aligned, zero-filled before its first use; each call leaves
 *             it ready for the next call of the same hq, hkv and max_pos
 *             (zero-fill it again before a call of another shape).  Calls
 *             that overlap in time must not share it.
 * One launch on `stream` of (max_pos/256 rounded up) x hq workgroups; those
 * past the position leave at once.  Past 256 positions the workgroups of a
 * query head hand span maxima and sums to each other through tagged words
 * in the workspace; each such wait is bounded like q4_decode_layers' (env
 * Q4_DECODE_TIMEOUT_MS); when one runs out, o is undefined and
 * q4_atq_status reports it (and clears the workspace); until then, calls
 * with that workspace return at once without writing.  Every output and
 * the workspace must overlap no other argument.  Inputs are assumed finite
 * (a NaN score makes the position of the maximum, and so the output,
 * unspecified).  q4_atq_ws_bytes returns 0 for head counts outside the
 * limits above.
 */
#define Q4_ATQ_MAX_POS 4096
size_t q4_atq_ws_bytes(int32_t hq, int32_t hkv);
int q4_atq(const float *q, const float *g, const float *k, const float *v, const float *wq,
           const float *wk, float eps, const float *rope_cos, const float *rope_sin,
           float *kcache, float *vcache, const int32_t *pos, int32_t max_pos, int32_t hq,
           int32_t hkv, float *o, float *osum, void *ws, size_t ws_bytes, void *stream);
/* Host wait on `stream`; Q4_OK, or Q4_ETIMEOUT when a wait of q4_atq ran
 * out since the last status call (the workspace is then zero-filled). */
int q4_atq_status(void *ws, int32_t hq, int32_t hkv, void *stream);

/*
 * One decoder layer of a decode token, the attention block and the MLP
 * block, in one persistent launch ([P1] Change: rmsq, q4mv, atq and swq
 * queued for a whole token; Verification: one command buffer and one wait).
 * Computes, with the bits of the separate calls,
 *   y = q4mv_norm(qgkv, h, wa)           [q; gate; k; v] = y
 *   q4_atq(q, gate, k, v, wq, wk, eps, rope_cos, rope_sin, kcache, vcache,
 *          pos, max_pos, 16, hkv, o, osum)
 *   h = q4mv_add(o_mat, o, osum, h)
 *   m = q4mv_norm_swiglu(mlp.gate_up, h, mlp.wn); h = q4mv_add(mlp.down, m, NULL, h)
 * in one grid of one workgroup per compute unit (at least 256) whose stages
 * hand their outputs to each other through tagged words in the workspace,
 * with bounded waits (as q4_decode_layers).
 *
 *   blk->qgkv : rows (32 + 2 hkv) * 128, cols 2048: the 16 query heads'
 *               rows, the 16 gate heads' rows, hkv key heads', hkv value
 *               heads'.
 *   blk->o    : rows 2048, cols 2048 (16 heads of 128 in).
 *   blk->wa   : device float[2048] attention norm weights; wq, wk: float[128];
 *               all 16-byte aligned.
 *   blk->kcache, vcache : device float[hkv][max_pos][128], 16-byte aligned.
 *   blk->hkv  : 1, 2, 4, 8 or 16 key/value heads.
 *   blk->mlp  : as for q4_decode_layers (inter 2048..8192).
 *   h         : device float[2048], 16-byte aligned, read and written.
 *   pos       : device int32[1]; max_pos <= Q4_BLOCK_MAX_POS (16 spans of
 *               256 positions; one workgroup per query head and span);
 *               rope_cos, rope_sin: device float[max_pos][64], 16-byte
 *               aligned.  A position outside [0, max_pos) makes h NaN.
 *   ws        : q4_decode_block_ws_bytes() bytes (about 1.6 MB), 16-byte
 *               aligned, zero-filled before first use; one call at a time.
 * Errors: Q4_EINVAL for a shape, alignment or limit above, or when an
 * array that the call writes (h, the caches, ws) overlaps another of its
 * arrays; nothing is launched then.
 * q4_decode_block_status waits on the stream and reports a wait that ran
 * out (Q4_ETIMEOUT, after clearing the workspace).
 */
#define Q4_BLOCK_MAX_POS 4096
typedef struct q4_attn_block {
  q4_mat qgkv;
  q4_mat o;
  const float *wa;
  const float *wq;
  const float *wk;
  float *kcache;
  float *vcache;
  int32_t hkv;
  q4_mlp_layer mlp;
} q4_attn_block;
size_t q4_decode_block_ws_bytes(void);
int q4_decode_block(const q4_attn_block *blk, float eps, float *h, const int32_t *pos,
                    int32_t max_pos, const float *rope_cos, const float *rope_sin, void *ws,
                    size_t ws_bytes, int mode, void *stream);
int q4_decode_block_status(void *ws, void *stream);

/*
 * Several decoder layers of a decode token in one persistent launch
 * ([P1] Change and Verification, as q4_decode_block): layer l + 1 takes h
 * from layer l through tagged words, and each workgroup loads its rows of
 * the next layer before it waits for the values they multiply.  The result
 * has the bits of q4_decode_block called once per layer, in order.
 *
 * q4_block_stack_create checks the layers (each as q4_decode_block does;
 * all with the same hkv and inter; no cache overlapping another layer's
 * arrays) and copies their pointers to a table in device memory, with a
 * synchronous copy: not a call for stream capture.  The arrays stay owned
 * by the caller and must outlive the stack.  1 <= nlayers <=
 * Q4_BLOCK_MAX_LAYERS; every cache holds max_pos positions.
 * q4_decode_blocks runs every layer of the stack on h (read, then written
 * with the last layer's output); pos, rope tables and ws as for
 * q4_decode_block (the same workspace size and status call).  Errors as
 * for q4_decode_block, Q4_ENOMEM or Q4_EHIP from create.
 * q4_block_stack_destroy frees the table (after the device is idle).
 */
#define Q4_BLOCK_MAX_LAYERS 32
typedef struct q4_block_stack q4_block_stack;
int q4_block_stack_create(const q4_attn_block *blocks, int32_t nlayers, int32_t max_pos,
                          q4_block_stack **out);
int q4_block_stack_destroy(q4_block_stack *s);
int q4_decode_blocks(const q4_block_stack *s, float eps, float *h, const int32_t *pos,
                     const float *rope_cos, const float *rope_sin, void *ws, size_t ws_bytes,
                     int mode, void *stream);

/*
 * q4_pos_advance: *pos += 1 on the device (one thread), so that a decode
 * token captured once as a graph moves its attention steps to the next
 * position on every replay ([P1] Verification: one command buffer per
 * token, replayed token after token here).  pos: device int32[1].
 */
int q4_pos_advance(int32_t *pos, void *stream);

/*
 * Stage queue ([P2] Change: q4go encodes products into one open concurrent
 * command buffer and returns; q4wait commits and waits once).
 * q4mv_queue appends a product to the current stage.  Products of one stage
 * may run concurrently, so none may read another's y ([P2] Change).
 * q4_stage closes the stage: its products are launched as grouped kernels
 * (one launch per kernel shape) with no host wait; later stages are ordered
 * after it on the queue's stream.  q4mv_wait closes the open stage and waits
 * once on the host for all of it; every buffer the queue's products use
 * must stay alive until it returns.  With env Q4MV_DEBUG_CHECKS=1,
 * q4mv_queue rejects (Q4_EINVAL) a product whose y overlaps an input of
 * another product of the same stage.  With env Q4MV_TRACE=1, q4mv_wait
 * prints the product count, GPU time and wall time of each wait to stderr.
 * A queue is used by one host thread at a time.
 */
typedef struct q4_queue q4_queue;
int q4_queue_create(void *stream, int mode, q4_queue **out);
int q4_queue_destroy(q4_queue *q);

/*
 * How q4mv_wait waits ([P2] Change: q4wait waits on a flag).  Q4_WAIT_STREAM
 * (the default): hipStreamSynchronize.  Q4_WAIT_MAILBOX: q4mv_wait enqueues
 * a mailbox post (below) after the last stage and spins on the host until
 * it lands, at most timeout_ms milliseconds (then Q4_ETIMEOUT; errors of the
 * stream itself are reported by q4_sync).  Switching to Q4_WAIT_MAILBOX
 * allocates the queue's mailbox; switching back waits for the stream and
 * frees it.
 */
#define Q4_WAIT_STREAM 0
#define Q4_WAIT_MAILBOX 1
int q4_queue_set_wait(q4_queue *q, int how, int32_t timeout_ms);
int q4mv_queue(q4_queue *q, const q4_mat *w, const float *x, const float *xsum,
               float *y);
int q4_stage(q4_queue *q);
int q4mv_wait(q4_queue *q);

/*
 * Whole-token graph capture ([P1] Verification: a decode token encoded as
 * one command buffer of 194 kernels and one wait).  Between
 * q4_capture_begin and q4_capture_end every call on `stream` is recorded,
 * not run; q4_graph_launch replays the recording on a stream.  No host wait
 * may happen in between (q4mv_wait returns Q4_ESTATE).
 */
typedef struct q4_graph q4_graph;
int q4_capture_begin(void *stream);
int q4_capture_end(void *stream, q4_graph **out);
int q4_graph_launch(q4_graph *g, void *stream);
int q4_graph_destroy(q4_graph *g);

/*
 * Mailbox: a host wait on a flag instead of on the stream ([P2] Change: the
 * host waits once on a flag that the last queued work sets).  A mailbox is
 * pinned, coherent host memory holding n int32 values and a sequence
 * number, plus a device counter.
 *   q4_mailbox_create : n in 1..Q4_MAILBOX_MAX_VALUES; allocates (not for
 *                       use during capture).
 *   q4_mailbox_post   : enqueues on `stream` one single-thread kernel that
 *                       copies vals (device int32[n]) into the mailbox and
 *                       then publishes the next sequence number (the
 *                       number of posts executed so far).  Legal inside
 *                       stream capture: every replay posts once.
 *   q4_mailbox_wait   : spins on the host until the sequence number reaches
 *                       `target` (compared modulo 2^32), then copies the
 *                       values into vals (host int32[n], NULL to skip).
 *                       Q4_ETIMEOUT after timeout_ms milliseconds (a fault or
 *                       an error on the stream is reported by q4_sync, not
 *                       here).
 *   q4_mailbox_seq    : the sequence number now (0 before the first post).
 * Posts on one mailbox must be ordered (one stream).  The caller keeps vals
 * alive until the post has run.
 */
#define Q4_MAILBOX_MAX_VALUES 1024
typedef struct q4_mailbox q4_mailbox;
int q4_mailbox_create(int32_t nvals, q4_mailbox **out);
int q4_mailbox_destroy(q4_mailbox *mb);
int q4_mailbox_post(q4_mailbox *mb, const int32_t *vals, void *stream);
int q4_mailbox_wait(q4_mailbox *mb, uint32_t target, int32_t *vals, int32_t timeout_ms);
uint32_t q4_mailbox_seq(const q4_mailbox *mb);

/* Host wait for all work on `stream` (one hipStreamSynchronize). */
int q4_sync(void *stream);

/* Text of a status code. */
const char *q4_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif /* Q4MV_H */
