/*
 * kata.h - C ABI of libkata: the KATA (Kernelized Linear Attention Activations)
 * causal forward pass and recurrent decode step on AMD MI355X (gfx950).
 *
 * Method: "Kernelized Linear Attention: Breaking the Capacity Wall with
 * Symmetric Cones" (arXiv 2607.17419).  Citations below use
 *   [ABS]    the paper's abstract (fugumt.com entry for 2607.17419v1),
 *   [TS-x]   section x of the gist.science technical summary of the paper.
 *
 * What the library computes, per batch row b and head h, for tokens t = 0..T-1:
 *
 *   u_t = P_h q_t,  w_s = P_h k_s                      (P_h: p x d, [TS-2.2])
 *   phi(x) = vec((P_h x)(P_h x)^T)                       (rank-one PSD feature, [TS-2.2])
 *   S_t = S0 + sum_{s<=t} phi(k_s) v_s^T,  z_t = z0 + sum_{s<=t} phi(k_s)
 *   y_t = S_t^T phi(q_t) / (z_t . phi(q_t))              ([TS-1], [TS-2.1]; y_t = 0 if the
 *                                                        denominator is 0)
 *
 * i.e. normalised causal attention whose weights are ((P q_t).(P k_s))^2 >= 0.
 * kata_forward evaluates it in the exact chunked-state form ([TS-2.3], [ABS]):
 * per chunk of C tokens a state phi(K_c)^T [V_c | 1]; an associative prefix of
 * those states (log depth in the number of chunks); per chunk the masked squared
 * score tile times [V_c | 1] plus the prefix state read out through phi(Q_c);
 * then the output gate (the division).  kata_decode_step is the constant-time
 * recurrent step of the same attention ([TS-1], [ABS]).
 *
 * Conventions shared by every entry point:
 *  - Every data pointer is DEVICE memory owned by the caller.  The library never
 *    allocates, frees or synchronises; all work is enqueued on `stream`
 *    (a hipStream_t; NULL = the default stream) and is complete when the stream
 *    reaches it.  Outputs are undefined until then.
 *  - Tensors are dense, row-major (C-contiguous) in the shapes given.
 *  - Argument errors are detected on the host and returned before anything is
 *    enqueued; KATA_ERR_LAUNCH reports a failed kernel launch (hipGetLastError).
 *    No exception crosses the boundary.  The functions keep no state between
 *    calls and are safe to call from several host threads.
 *  - State layout ("canonical"): S [.., p*p, dv] and z [.., p*p] float32 with
 *    feature index i*p + j, i.e. S holds sum phi(k) v^T with phi = vec(w w^T).
 *    phi(k) = vec(w w^T) is symmetric, and so is every state built from it.  Every entry
 *    point reads a caller's state through its symmetric part: the mean of the mirror
 *    entries (i, j) and (j, i), which is the entry itself, bit for bit, for the states
 *    this library produces.  kata_forward, kata_forward_decay and kata_forward_factors
 *    export ST, zT as that symmetric part plus the tokens' contribution (for T = 0: the
 *    symmetric part of S0, z0).  The decode steps and the DeltaKATA entry points add
 *    their symmetric updates to the caller's state, so an antisymmetric part a caller
 *    puts in passes through them unchanged and never reaches y.
 *  - Supported in this version: p = 16; (d, dv) = (16, 16) or (64, 64);
 *    chunk in {32, 64, 128}; in_dtype F32 or BF16 (kata_forward also BF16_HILO);
 *    out_dtype F32 or BF16; any T >= 0 (a ragged last
 *    chunk is handled); B*H <= 65535.  Other values return KATA_ERR_UNSUPPORTED.
 */
#ifndef KATA_H
#define KATA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KATA_ABI_VERSION 1

typedef enum {
  KATA_OK = 0,
  KATA_ERR_NULL = 1,         /* a required pointer is NULL                      */
  KATA_ERR_SHAPE = 2,        /* a size is negative / inconsistent / too large   */
  KATA_ERR_UNSUPPORTED = 3,  /* valid but not implemented (p, d, dv, chunk, dtype) */
  KATA_ERR_WORKSPACE = 4,    /* workspace NULL or smaller than required         */
  KATA_ERR_LAUNCH = 5,       /* a kernel launch failed                          */
  KATA_ERR_SCRATCH = 6       /* kata_forward_noalloc: the problem needs more scratch
                                than its fixed device buffer holds                */
} kata_status;

/* Storage (and compute) type of tensors.
 *  KATA_F32, KATA_BF16: float32 / bfloat16 storage.  With float32 q, k, v every matrix-core
 *    operand is a hi/lo pair of bf16 (about 16 significant bits).  With bfloat16 q, k, v the
 *    projections u = Pq, w = Pk enter the score tiles as hi/lo pairs and the features
 *    phi(k), phi(q) and the published state H are single bf16 (8 significant bits).
 *  KATA_BF16_HILO (in_dtype of kata_forward and kata_forward_noalloc only): bfloat16
 *    storage like KATA_BF16, but phi(k), phi(q) and H also enter the matrix cores as hi/lo
 *    pairs.  For output gates that are far from well conditioned while keys are read
 *    through a state: where den_t = sum_s (u_t.w_s)^2 is a small fraction of
 *    sum_s |u_t|^2 |w_s|^2 (a query nearly orthogonal to keys of earlier chunks or of the
 *    initial state), the single-bf16 readout phi(q_t)^T H loses y_t to rounding, while
 *    this mode keeps it to the bf16 bar for fractions down to about 1e-3.  It takes about
 *    1.45x the time of KATA_BF16 on the long-context shape (twice the state LDS, so two
 *    workgroups per compute unit instead of three, and three matrix-core products per
 *    readout and two per state update instead of one).  Other entry points reject it. */
typedef enum { KATA_F32 = 0, KATA_BF16 = 1, KATA_BF16_HILO = 2 } kata_dtype;

/* How the inter-chunk state prefix is formed ([TS-2.3], [ABS]: an associative scan over
 * the chunk states replaces the chunk-after-chunk recurrence; the combine is +).
 *  KATA_SCAN_ASSOC: a reduce-then-scan.  The chunks are grouped into leaves of L =
 *    `scan_leaf` consecutive chunks (0: chosen by the library so the leaves fill the GPU
 *    in whole rounds, e.g. L = 43, 48 leaves per sequence, at T = 131072, C = 64).
 *    (1) Every leaf's chunk states are summed, all leaves in parallel.  (2) The leaf sums
 *    get an exclusive prefix: each thread keeps up to 16 consecutive leaf rows of one
 *    16-byte column quad in registers and sums them in order, the totals of up to 16
 *    such segments are combined through LDS, and sequences of more than 256 leaves take
 *    several such passes chained by a carry.  (3) Inside each leaf, the pass that forms
 *    the outputs completes every chunk's prefix with a running sum kept on chip, walking
 *    the leaf's chunks in order.  The sequential depth is therefore L chunk steps inside a
 *    leaf plus at most 16 + 16 combine steps per 256 leaves: O(L + n_leaf / 16), not a
 *    log-depth tree; with the library's choice of L it is about sqrt of the work per
 *    GPU round.  A log-depth combine of the leaf sums measured 1.5x slower at these leaf
 *    counts.  scan_leaf = 1 writes and scans every chunk state (the literal chunk-level
 *    scan, depth 16 per pass plus the segment combine).  When the library's own plan
 *    (scan_leaf = 0) has at most 8 leaves per sequence (many short sequences), step (2)
 *    is folded into step (3): the output pass's workgroup of leaf g adds the sums of
 *    leaves 0 .. g-1 itself (depth up to 7 leaf additions) and no separate scan runs.
 *  KATA_SCAN_SEQUENTIAL: one leaf per sequence - the chunk states are propagated
 *    strictly chunk after chunk (depth O(T/C)), the matched sequential baseline
 *    the pages compare the scan against ([ABS]). */
typedef enum { KATA_SCAN_ASSOC = 0, KATA_SCAN_SEQUENTIAL = 1 } kata_scan_mode;

typedef struct {
  int64_t B;              /* batch rows                                   */
  int64_t H;              /* heads                                        */
  int64_t T;              /* tokens per sequence (>= 0)                   */
  int d;                  /* query/key head dimension                     */
  int dv;                 /* value head dimension                         */
  int p;                  /* projection dimension (16)                    */
  int chunk;              /* chunk length C                               */
  kata_dtype in_dtype;    /* dtype of q, k, v                             */
  kata_dtype out_dtype;   /* dtype of y                                   */
  kata_scan_mode scan;    /* see kata_scan_mode                           */
  int scan_leaf;          /* chunks per leaf in KATA_SCAN_ASSOC; 0 = chosen by the library */
} kata_forward_desc;

/* ABI version of the loaded library (KATA_ABI_VERSION). */
int kata_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char* kata_status_string(kata_status s);

/* Bytes of device workspace kata_forward needs for `desc` (written to *bytes).
 * The workspace holds the per-leaf chunk states, B*H*n_leaf blocks of (ceil-packed)
 * state, float32, and after the call their exclusive prefixes; when the plan folds the
 * prefix into the output pass (see KATA_SCAN_ASSOC) it still holds the leaf sums. */
kata_status kata_forward_workspace_bytes(const kata_forward_desc* desc, size_t* bytes);

/* The leaf plan kata_forward (and kata_forward_noalloc) uses for `desc` (KATA_SCAN_ASSOC,
 * [TS-2.3]): *n_leaf leaves per sequence of *leaf_chunks chunks each (the last may be
 * shorter; 0 leaves when T == 0), and *scanned = 1 when a separate scan forms the leaf
 * prefixes, 0 when the output pass adds the earlier leaves itself.  Any output pointer
 * may be NULL.  Pure host computation from the descriptor; the same validation as
 * kata_forward_workspace_bytes. */
kata_status kata_forward_plan(const kata_forward_desc* desc, int64_t* n_leaf, int64_t* leaf_chunks, int* scanned);

/* Causal KATA forward over whole sequences in the exact chunked-state form
 * ([TS-2.3], [ABS]; definition in the header comment).
 *   q  [B,H,T,d], k [B,H,T,d], v [B,H,T,dv]   in_dtype
 *   P  [H,p,d]   float32 (one projection per head)
 *   S0 [B,H,p*p,dv], z0 [B,H,p*p] float32 initial state, or both NULL for zero
 *   y  [B,H,T,dv] out_dtype (written)
 *   ST [B,H,p*p,dv], zT [B,H,p*p] float32 final state (written), or NULL if unwanted
 *   workspace: device memory of at least kata_forward_workspace_bytes bytes,
 *   owned by the caller, contents on entry ignored.
 * Returns KATA_OK once everything is enqueued on `stream`. */
kata_status kata_forward(const kata_forward_desc* desc,
                         const void* q, const void* k, const void* v,
                         const float* P,
                         const float* S0, const float* z0,
                         void* y,
                         float* ST, float* zT,
                         void* workspace, size_t workspace_bytes,
                         void* stream);

/* kata_forward that also stamps four caller-created hipEvent_t (created with timing
 * enabled) from the kernel launches on `stream`: events[0] at the start of
 * kata_chunk_state, events[1] at the start of kata_state_scan (or, when the plan runs no
 * scan, at the end of kata_chunk_state), events[2] at the start of kata_chunk_intra and
 * events[3] at its end, so a caller can time each kernel of
 * the chunked forward on the stream it runs on.  The launches record the events
 * themselves (no extra commands enter the stream).  events == NULL behaves exactly
 * like kata_forward.  A NULL element is not stamped: every stamped launch costs a few
 * microseconds of dispatch gap, so a caller timing one kernel passes only its two.
 * When nothing is launched (B*H == 0 or T == 0) no event is recorded.  The same rule
 * holds for every *_timed entry point below. */
kata_status kata_forward_timed(const kata_forward_desc* desc,
                               const void* q, const void* k, const void* v,
                               const float* P,
                               const float* S0, const float* z0,
                               void* y,
                               float* ST, float* zT,
                               void* workspace, size_t workspace_bytes,
                               void* stream, void* const* events);

/* kata_forward for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops and harnesses that forbid hipMalloc.  It computes exactly
 * what kata_forward computes, with the same kernels, leaf plan and arguments (results are
 * bit for bit those of kata_forward), but takes no workspace: the leaf states live in a
 * device array inside the library, KATA_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, set up
 * when the library is first used on that GPU and held until the process ends.  The call
 * itself allocates nothing (no hipMalloc, no allocating library routine).
 *   Limit: kata_forward_workspace_bytes(desc) must be at most KATA_NOALLOC_SCRATCH_BYTES,
 *   else KATA_ERR_SCRATCH is returned before anything is enqueued (the long-context,
 *   mid-size and 340M-layer shapes need 27 to 29 MiB; B*H = 4096 sequences of 8192
 *   tokens need 465 MB and are rejected).
 *   Concurrency: every call on one GPU uses that GPU's one array, which keeps the last
 *   call's contents (nothing in it needs clearing: every leaf state is written before it
 *   is read).  Calls whose work overlaps on one GPU (different streams, or host threads
 *   enqueueing concurrently without ordering) race on it and give undefined results;
 *   calls ordered on one stream are safe.
 * Other arguments, layouts, ownership and errors as for kata_forward. */
#define KATA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
kata_status kata_forward_noalloc(const kata_forward_desc* desc,
                                 const void* q, const void* k, const void* v,
                                 const float* P,
                                 const float* S0, const float* z0,
                                 void* y,
                                 float* ST, float* zT,
                                 void* stream);

/* Flash-style O(T^2) forward (no state): the first operating point of the
 * hardware section of the gist.science summary of arXiv 2607.17419 (section 2.3),
 * the fused kernel behind the 1.6x-over-FlashAttention-2 figure of the paper's
 * abstract.  Computes the same y as kata_forward with no initial state,
 *   y_t = sum_{s<=t} (u_t . w_s)^2 v_s / sum_{s<=t} (u_t . w_s)^2   (0 if the sum is 0),
 * by accumulating masked squared score tiles over all earlier key blocks; no state is
 * formed or returned.  Supported: p = 16, d = dv = 64, in_dtype BF16, out_dtype F32 or
 * BF16; desc->chunk, scan and scan_leaf are ignored.  q, k [B,H,T,64], v [B,H,T,64]
 * bf16, P [H,16,64] f32, y [B,H,T,64] out_dtype, all device memory owned by the caller.
 * The workspace (kata_flash_workspace_bytes: 256 bytes per token and head, T rounded
 * up to 128) holds the projected u and w (each as a hi/lo pair of bf16, so the squared
 * scores keep about 16 significant bits) and V in MFMA operand order.
 * events: NULL, or three caller-created hipEvent_t (timing enabled) stamped with the
 * start of the projection kernel, the start of the attention kernel and its end.
 * Errors are returned before anything is enqueued; B*H == 0 or T == 0 is a no-op. */
kata_status kata_flash_workspace_bytes(const kata_forward_desc* desc, size_t* bytes);
kata_status kata_flash_forward(const kata_forward_desc* desc,
                               const void* q, const void* k, const void* v,
                               const float* P, void* y,
                               void* workspace, size_t workspace_bytes,
                               void* stream, void* const* events);

/* Backward of kata_forward: gradients of q, k, v, P and the initial state for a given
 * gradient gy of the output y and (optionally) gST, gzT of the final state.  The pages
 * give no backward pass; it is the derivative of the forward defined above (chain rule):
 * with num_t, den_t the numerator and denominator of y_t, g_t = gy_t / den_t and
 * h_t = -(g_t . num_t) / den_t = -(gy_t . y_t) / den_t (both 0 where den_t = 0, where y_t
 * is the constant 0), and B_ts = 2 (u_t . w_s) (g_t . v_s + h_t) for s <= t,
 *   du_t = sum_s B_ts w_s + 2 mat(S_t g_t + z_t h_t) u_t        dq = du P
 *   dw_s = sum_t B_ts u_t + 2 mat(R_s v_s + r_s) w_s            dk = dw P
 *   dv_s = sum_{t>=s} a_ts g_t + gST^T phi(k_s)                 dP = sum over b, t of du q^T + dw k^T
 *   dS0 = gST + sum_t phi(q_t) g_t^T,  dz0 = gzT + sum_t phi(q_t) h_t
 * where S_t, z_t is the forward's prefix state (exclusive of chunk-local tokens, which
 * enter through B_ts) and R_s, r_s = gST, gzT + sum_{t > chunk of s} phi(q_t) [g_t | h_t]
 * the backward's suffix state.  It runs in the chunked-state form: the forward's chunk
 * states and their associative prefix, a walk over the chunks that forms g, h and dq,
 * the backward's chunk states phi(Q_c)^T [G_c | h_c] and their associative SUFFIX (the
 * hardware section of the gist.science summary, section 2.3, applied to the reversed
 * sequence), and a reverse walk that forms dv and dk.
 *   desc: as for kata_forward; supported p = 16, d = dv = 64, chunk = 64, in_dtype BF16
 *         (q, k, v, dq, dk, dv), out_dtype F32 or BF16 (gy).  scan / scan_leaf as for
 *         kata_forward (the leaf plan is the backward's own).
 *   q, k [B,H,T,64], v [B,H,T,64] bf16; P [H,16,64] f32; S0 [B,H,256,64], z0 [B,H,256] f32
 *   or both NULL (those of the forward being differentiated);
 *   gy [B,H,T,64] out_dtype: the gradient of the loss w.r.t. the forward's output y.  y itself
 *   is not an input: g_t . num_t is formed from the state and score tiles of the walk, so
 *   the gradient does not inherit the rounding of a stored y;
 *   gST [B,H,256,64], gzT [B,H,256] f32 or both NULL (zero): gradient w.r.t. the final state;
 *   dq, dk, dv [B,H,T,64] bf16, dP [H,16,64] f32 (summed over the batch) - written;
 *   dS0 [B,H,256,64], dz0 [B,H,256] f32 or both NULL - written.  A state is symmetric in
 *   (i, j), so dS0 / dz0 are returned as the gradient within symmetric states: gST and gzT
 *   enter through the mean of their mirror entries, and dS0[i*16+j] = dS0[j*16+i].
 *   workspace: kata_backward_workspace_bytes bytes (device memory owned by the caller).
 * B*H == 0 or T == 0 writes dP = 0 and dS0, dz0 = gST, gzT (zero when NULL).  Errors are
 * returned before anything is enqueued.  kata_backward_timed stamps eight caller events
 * (NULL = none): the starts of the forward chunk-state kernel, the forward scan, the query
 * walk, the backward chunk-state kernel, the reverse scan, the key walk and the dP
 * reduction, and the end of the last. */
kata_status kata_backward_workspace_bytes(const kata_forward_desc* desc, size_t* bytes);
kata_status kata_backward(const kata_forward_desc* desc,
                          const void* q, const void* k, const void* v, const float* P,
                          const float* S0, const float* z0,
                          const void* gy,
                          const float* gST, const float* gzT,
                          void* dq, void* dk, void* dv, float* dP,
                          float* dS0, float* dz0,
                          void* workspace, size_t workspace_bytes, void* stream);
kata_status kata_backward_timed(const kata_forward_desc* desc,
                                const void* q, const void* k, const void* v, const float* P,
                                const float* S0, const float* z0,
                                const void* gy,
                                const float* gST, const float* gzT,
                                void* dq, void* dk, void* dv, float* dP,
                                float* dS0, float* dz0,
                                void* workspace, size_t workspace_bytes, void* stream,
                                void* const* events);

/* Decay-gated causal forward.  The paper's abstract names "decay gates" among the
 * mechanisms studied with KATA's features without defining them; the reading taken is
 * the scalar forget gate of gated linear attention applied to KATA's state [S | z]:
 *   S_t = gamma_t S_{t-1} + phi(k_t) v_t^T,  z_t = gamma_t z_{t-1} + phi(k_t),
 *   y_t = S_t^T phi(q_t) / (z_t . phi(q_t)),  gamma_t = exp(lam_t)
 * with one log-gate lam_t <= 0 per token and head (the current token is not decayed; an
 * initial state S0, z0 decays like the rest).  Numerator and denominator decay alike, so
 * the output gate stays convex.  Chunked form ([TS-2.3]): keys weighted by their decay
 * to the end of the chunk, the inter-chunk prefix by the affine recurrence
 * H <- exp(L_c) H + chunk state (an associative scan with combine (D_a, S_a) o (D_b, S_b)
 * = (D_a D_b, D_b S_a + S_b)), and inside the chunk weights (u_t.w_s)^2 exp(l_t - l_s).
 *   lam [B,H,T] float32 (device); other arguments as for kata_forward.
 * Supported: p = 16, d = dv = 64, chunk = 64, in_dtype BF16, out_dtype F32 or BF16.
 * The workspace (kata_forward_decay_workspace_bytes) is kata_forward's plus one float per
 * leaf.  kata_forward_decay_timed stamps the same four events as kata_forward_timed. */
kata_status kata_forward_decay_workspace_bytes(const kata_forward_desc* desc, size_t* bytes);
kata_status kata_forward_decay(const kata_forward_desc* desc,
                               const void* q, const void* k, const void* v,
                               const float* P, const float* lam,
                               const float* S0, const float* z0,
                               void* y, float* ST, float* zT,
                               void* workspace, size_t workspace_bytes, void* stream);
kata_status kata_forward_decay_timed(const kata_forward_desc* desc,
                                     const void* q, const void* k, const void* v,
                                     const float* P, const float* lam,
                                     const float* S0, const float* z0,
                                     void* y, float* ST, float* zT,
                                     void* workspace, size_t workspace_bytes, void* stream,
                                     void* const* events);

/* The packed symmetric state: phi(k) = vec(w w^T) is symmetric, so every state the
 * decode steps or kata_forward produce has equal mirror rows (a, b) and (b, a) of S and z,
 * and every read phi(q) . S sees only their sum.  The packed layout keeps one row per
 * pair {a, b}: KATA_PACKED_ROWS = 136 rows, row 16 delta + a (delta = 0..7, a = 0..15)
 * and row 128 + a (delta = 8, a = 0..7) for the pair {a, (a + delta) mod 16} (p = 16):
 * the slots of the packed feature layouts of kata_feature_map without their 8 zero slots.
 * Sp [n, 136, dv], zp [n, 136] float32 device memory owned by the caller.
 *   kata_state_pack:   Sp row of {a, b} = (S[16a+b] + S[16b+a]) / 2 (exact where the
 *                      mirror rows are equal; a read sees only their sum, which this
 *                      keeps); zp likewise.  n = number of (stream, head) states.
 *   kata_state_unpack: both S[16a+b] and S[16b+a] = Sp row of {a, b}; z likewise.
 * z and zp are both NULL (S only) or both given.  dv = 16 or 64.  The calls are enqueued
 * on `stream`; S and Sp must not overlap. */
#define KATA_PACKED_ROWS 136
kata_status kata_state_pack(int64_t n, int dv, const float* S, const float* z, float* Sp, float* zp,
                            void* stream);
kata_status kata_state_unpack(int64_t n, int dv, const float* Sp, const float* zp, float* S, float* z,
                              void* stream);

/* kata_decode_step on the packed state ([TS-1], [ABS]; packed as above):
 *   Sp += phi_p(k) v^T, zp += phi_p(k),  phi_p(k)[row of {a, b}] = w_a w_b
 *   y = sum_r c_r phi_p(q)[r] Sp[r] / sum_r c_r phi_p(q)[r] zp[r],  c_r = 1 on the
 *       diagonal (a = b), 2 off it (a pair stands for two mirror rows)
 * which equals kata_decode_step on the unpacked state, with 136 instead of 256 rows
 * read and written per head.  Sp [N,H,136,dv], zp [N,H,136] float32 in place; other
 * arguments, support and errors as for kata_decode_step. */
kata_status kata_decode_step_packed(int64_t N, int64_t H, int d, int dv, int p,
                                    kata_dtype in_dtype, kata_dtype out_dtype,
                                    float* Sp, float* zp,
                                    const void* q, const void* k, const void* v,
                                    const float* P, void* y, void* stream);

/* kata_decode_step_decay on the packed state: Sp <- gamma Sp + phi_p(k) v^T,
 * zp <- gamma zp + phi_p(k), gamma = exp(lam) (lam [N,H] float32), then the packed read.
 * Other arguments, support and errors as for kata_decode_step_decay. */
kata_status kata_decode_step_decay_packed(int64_t N, int64_t H, int d, int dv, int p,
                                          kata_dtype in_dtype, kata_dtype out_dtype,
                                          float* Sp, float* zp,
                                          const void* q, const void* k, const void* v,
                                          const float* P, const float* lam, void* y, void* stream);

/* One decay-gated recurrent decode step (same reading): S <- gamma S + phi(k) v^T,
 * z <- gamma z + phi(k), y = S^T phi(q) / (z . phi(q)), gamma = exp(lam), lam [N,H]
 * float32 (device).  Other arguments and support as for kata_decode_step. */
kata_status kata_decode_step_decay(int64_t N, int64_t H, int d, int dv, int p,
                                   kata_dtype in_dtype, kata_dtype out_dtype,
                                   float* S, float* z,
                                   const void* q, const void* k, const void* v,
                                   const float* P, const float* lam, void* y, void* stream);

/* One recurrent decode step for N independent streams ([TS-1], [ABS]):
 *   S += phi(k) v^T, z += phi(k)   (in place, canonical layout)
 *   y  = S^T phi(q) / (z . phi(q)) (after the update; 0 if the denominator is 0)
 *   S [N,H,p*p,dv], z [N,H,p*p] float32, read and written in place
 *   q [N,H,d], k [N,H,d], v [N,H,dv] in_dtype; P [H,p,d] float32; y [N,H,dv] out_dtype.
 * The state is updated in full (both mirror entries), so it stays canonical. */
kata_status kata_decode_step(int64_t N, int64_t H, int d, int dv, int p,
                             kata_dtype in_dtype, kata_dtype out_dtype,
                             float* S, float* z,
                             const void* q, const void* k, const void* v,
                             const float* P, void* y, void* stream);

/* KATA-Mg and KATA-Sigma-g: g PSD factors per head.  [TS-2.3] (item "Variantes") names
 * "several PSD factors" (Mg) and "summed PSD factors" (Sigma-g), trading state size
 * against packing efficiency, and [TS-4] quotes the chunked-state kernel of KATA-M2;
 * none defines how the factors combine.  Reading taken, with u_i = P_i x, w_i = P_i k:
 *   KATA_FACTORS_CONCAT (Mg): phi(x) = [vec(u_1 u_1^T); ...; vec(u_g u_g^T)],
 *       a_ts = sum_i (u_i,t . w_i,s)^2, state g*p*p x dv (the g one-factor states stacked)
 *   KATA_FACTORS_SUM (Sigma-g): phi(x) = vec(sum_i u_i u_i^T),
 *       a_ts = sum_i sum_j (u_i,t . w_j,s)^2, state p*p x dv
 * and y_t = sum_s a_ts v_s / sum_s a_ts as for KATA; g = 1 is KATA in both modes. */
typedef enum { KATA_FACTORS_CONCAT = 0, KATA_FACTORS_SUM = 1 } kata_factor_mode;

/* Bytes of workspace kata_forward_factors needs (g times the one-factor leaf states). */
kata_status kata_forward_factors_workspace_bytes(const kata_forward_desc* desc, int g,
                                                 kata_factor_mode mode, size_t* bytes);

/* The causal forward with g PSD factors in the chunked-state form.
 *   q, k [B,H,T,d], v [B,H,T,dv] in_dtype; P [H,g,p,d] float32 (factor-major per head);
 *   S0 [B,H,g*p*p,dv], z0 [B,H,g*p*p] float32 (CONCAT; factor i's rows i*p*p ..) or NULL;
 *   y [B,H,T,dv]; ST, zT in the layout of S0, z0, or NULL; workspace as returned above.
 * Supported: g = 1 with everything kata_forward supports (it runs kata_forward); g = 2 or 3
 * with KATA_FACTORS_CONCAT, d = dv = 64, chunk 64, in_dtype BF16, B*H*g <= 65535.  Other
 * values return KATA_ERR_UNSUPPORTED.  kata_forward_factors_timed stamps the events of
 * kata_forward_timed (state pass over the B*H*g factor states, scan, intra pass). */
kata_status kata_forward_factors(const kata_forward_desc* desc, int g, kata_factor_mode mode,
                                 const void* q, const void* k, const void* v, const float* P,
                                 const float* S0, const float* z0, void* y, float* ST, float* zT,
                                 void* workspace, size_t workspace_bytes, void* stream);
kata_status kata_forward_factors_timed(const kata_forward_desc* desc, int g, kata_factor_mode mode,
                                       const void* q, const void* k, const void* v, const float* P,
                                       const float* S0, const float* z0, void* y, float* ST, float* zT,
                                       void* workspace, size_t workspace_bytes, void* stream,
                                       void* const* events);

/* One decode step of KATA-Mg / KATA-Sigma-g (same reading as kata_forward_factors) for N
 * independent streams, in place: the token's feature (concatenated: one 256-row block per
 * factor; summed: one block) is folded into (S, z), then y = S^T phi(q) / (z . phi(q)).
 *   S [N,H,R,dv], z [N,H,R] float32 with R = g*p*p (CONCAT, factor-major) or p*p (SUM);
 *   q, k [N,H,d], v [N,H,dv] in_dtype; P [H,g,p,d] float32; y [N,H,dv] out_dtype.
 * Supported: g = 1 (runs kata_decode_step), g = 2 or 3; p = 16; (d, dv) = (16, 16) or
 * (64, 64); in/out dtype F32 or BF16. */
kata_status kata_decode_step_factors(int64_t N, int64_t H, int d, int dv, int p, int g,
                                     kata_factor_mode mode, kata_dtype in_dtype, kata_dtype out_dtype,
                                     float* S, float* z, const void* q, const void* k, const void* v,
                                     const float* P, void* y, void* stream);

/* kata_decode_step_factors on packed states (layout as for kata_decode_step_packed):
 * concat: Sp [N,H,g*136,dv], zp [N,H,g*136], factor-major (each block is the packed form
 * of that factor's canonical block; pack it with kata_state_pack over N*H*g states);
 * sum: Sp [N,H,136,dv], zp [N,H,136].  Same step, arguments, support and errors as
 * kata_decode_step_factors; g = 1 is kata_decode_step_packed. */
kata_status kata_decode_step_factors_packed(int64_t N, int64_t H, int d, int dv, int p, int g,
                                            kata_factor_mode mode, kata_dtype in_dtype, kata_dtype out_dtype,
                                            float* Sp, float* zp, const void* q, const void* k, const void* v,
                                            const float* P, void* y, void* stream);

/* DeltaKATA.  [TS-4] (repeated-key overwrite) credits the delta-rule variant of KATA with
 * correcting stale bindings when a key is written again, and [TS-1] / [ABS] name delta
 * rules among the mechanisms studied with KATA's features; none defines it.  The reading
 * taken is DeltaNet's delta rule with KATA's feature normalised to unit norm:
 *   phi^(x) = vec(u u^T) / |u|^2, u = P x     (|phi^(x)| = 1; phi^(x) = 0 where u = 0)
 *   S_t = S_{t-1} + beta_t phi^(k_t) (v_t - S_{t-1}^T phi^(k_t))^T
 *   y_t = S_t^T phi^(q_t)                      (no denominator, no z)
 * beta is taken as given (0 <= beta <= 1 keeps the update a contraction toward v; beta = 1
 * with a repeated key overwrites its value exactly).
 *
 * kata_forward_delta: the causal forward by the token recurrence, the state held on chip
 * by one workgroup per (batch row, head); it reads q, k, v once and the state once.
 *   q [B,H,T,d], k [B,H,T,d], v [B,H,T,dv] in_dtype; P [H,p,d] float32;
 *   beta [B,H,T] float32; S0 [B,H,p*p,dv] float32 initial state or NULL for zero;
 *   y [B,H,T,dv] out_dtype (written); ST [B,H,p*p,dv] float32 final state or NULL.
 * desc->chunk, scan and scan_leaf are not used.  No workspace.
 * Supported: p = 16, (d, dv) = (16, 16) or (64, 64), in/out dtype F32 or BF16,
 * B*H < 2^31, any T >= 0 (T = 0 writes ST = S0, or 0).  The state is carried in full
 * (both mirror entries of the symmetric feature are updated alike). */
kata_status kata_forward_delta(const kata_forward_desc* desc,
                               const void* q, const void* k, const void* v,
                               const float* P, const float* beta, const float* S0,
                               void* y, float* ST, void* stream);

/* DeltaKATA causal forward in the chunked (WY) form, for few long sequences: chunks of 64
 * tokens; per chunk T = (I + tril(diag(beta) K^K^^T, -1))^{-1} over the chunk's unit key
 * features K^ (formed for all chunks in parallel), then, walking the chunks in order,
 * E = T diag(beta)(V - K^ S), Y = Q^ S + (Q^K^^T o M) E (M: s <= t), S += K^^T E.  Same
 * definition and arguments as kata_forward_delta (exactly equal up to rounding), plus a
 * device workspace of kata_forward_delta_chunked_workspace_bytes bytes (normalised
 * projections and T per chunk: 9 KiB per 64 tokens and head; one int per walk workgroup
 * that keeps a sequence's workgroups within a few chunks of each other, so they share
 * their inputs in L2; and with segments, below, 256 x dv floats per segment and
 * 144 x (dv + 144) per segment but the last of each sequence), owned by the caller; calls
 * that overlap on one workspace race.
 * The walk of a sequence is split over dv/16 workgroups (value-column blocks of S) and
 * keeps the state's symmetric part packed (the antisymmetric part of S0, which no read
 * sees, reaches ST unchanged).  Segments: the chunk transition is affine in S, so with few
 * sequences the walk is cut into segments (kata_forward_delta_chunked_plan): each
 * segment's map S_end = M S_start + b is formed side by side (M from the packed unit
 * vectors; not for the last segment, whose walk exports ST, nor M for the first without
 * S0), the maps are chained into every segment's start state, and the segments' walks run
 * side by side.  desc->scan_leaf > 0 sets the chunks per segment and
 * KATA_SCAN_SEQUENTIAL one walk per sequence; 0 lets the library choose.  Either way the
 * plan keeps B*H*segments <= 65535 (longer segments where scan_leaf asks for more).  Supported: p = 16, (d, dv) = (16, 16) or (64, 64),
 * desc->chunk = 64, in/out dtype F32 or BF16, B*H <= 65535, and a sequence of q, k, v
 * or y under 2 GiB at 4 bytes per element (T * max(d, dv) * 4 < 2^31 - 4096, less 256
 * tokens; else KATA_ERR_SHAPE: the walk addresses a sequence with 32-bit offsets).
 * kata_forward_delta_chunked_timed stamps three caller-created events: start of the
 * per-chunk pass, start and end of the walk. */
kata_status kata_forward_delta_chunked_workspace_bytes(const kata_forward_desc* desc, size_t* bytes);
/* The walk plan kata_forward_delta_chunked uses for `desc`: each sequence's walk cut into
 * *segments segments of *segment_chunks chunks of 64 tokens (the last may be shorter; one
 * segment of all chunks when the walks already fill the GPU or under
 * KATA_SCAN_SEQUENTIAL).  Any output pointer may be NULL.  Pure host computation from the
 * descriptor; the same validation as kata_forward_delta_chunked_workspace_bytes. */
kata_status kata_forward_delta_chunked_plan(const kata_forward_desc* desc, int64_t* segments,
                                            int64_t* segment_chunks);
kata_status kata_forward_delta_chunked(const kata_forward_desc* desc,
                                       const void* q, const void* k, const void* v,
                                       const float* P, const float* beta, const float* S0,
                                       void* y, float* ST, void* workspace, size_t workspace_bytes,
                                       void* stream);
kata_status kata_forward_delta_chunked_timed(const kata_forward_desc* desc,
                                             const void* q, const void* k, const void* v,
                                             const float* P, const float* beta, const float* S0,
                                             void* y, float* ST, void* workspace,
                                             size_t workspace_bytes, void* stream,
                                             void* const* events);

/* One DeltaKATA decode step for N independent streams (same reading), in place:
 *   S <- S + beta phi^(k) (v - S^T phi^(k))^T,  y = S^T phi^(q)  (after the update)
 *   S [N,H,p*p,dv] float32; q, k [N,H,d], v [N,H,dv] in_dtype; P [H,p,d] float32;
 *   beta [N,H] float32; y [N,H,dv] out_dtype.  Support as for kata_forward_delta. */
kata_status kata_decode_step_delta(int64_t N, int64_t H, int d, int dv, int p,
                                   kata_dtype in_dtype, kata_dtype out_dtype,
                                   float* S, const void* q, const void* k, const void* v,
                                   const float* P, const float* beta, void* y, void* stream);

/* kata_decode_step_delta on the packed symmetric state (layout as for
 * kata_decode_step_packed; pack with kata_state_pack, z NULL): every update adds
 * beta phi^(k) e^T with phi^(k) symmetric, so the packed step writes a pair's row with
 * the unweighted feature and reads it with weight 2 off the diagonal.
 * Sp [N,H,136,dv] float32 in place; other arguments, support and errors as for
 * kata_decode_step_delta. */
kata_status kata_decode_step_delta_packed(int64_t N, int64_t H, int d, int dv, int p,
                                          kata_dtype in_dtype, kata_dtype out_dtype,
                                          float* Sp, const void* q, const void* k, const void* v,
                                          const float* P, const float* beta, void* y, void* stream);

/* Feature layouts for kata_feature_map. */
typedef enum {
  KATA_FEATURE_FULL = 0,         /* p*p entries, index i*p + j: phi = vec(u u^T)       */
  KATA_FEATURE_PACKED_KEY = 1,   /* 9*p slots (delta, a): u_a u_{(a+delta) mod p},      */
  KATA_FEATURE_PACKED_QUERY = 2  /*   delta = 0..8; query side weighted 2 off the        */
} kata_feature_layout;           /*   diagonal; slots (8, a>=8) are 0 (see below)        */

/* The feature map the chunk kernels build on chip, exposed for identity tests
 * ([TS-2.2]: phi(q).phi(k) = ((Pq).(Pk))^2).  The packed layouts hold the
 * p(p+1)/2 = 136 distinct entries of the symmetric u u^T in "circulant" order:
 * slot (delta, a) = 16*delta + a holds u_a u_b with b = (a + delta) mod 16,
 * delta = 0..8; for delta = 8 only a < 8 is distinct and slots a >= 8 hold 0.
 * The key side carries weight 1, the query side weight 2 off the diagonal, so
 * packed_query(q) . packed_key(k) = phi(q) . phi(k) exactly.
 *   x [n,H,d] in dtype; P [H,p,d] float32; phi [n,H,p*p] (FULL) or [n,H,9*p] float32. */
kata_status kata_feature_map(const void* x, const float* P, int64_t n, int64_t H, int d, int p,
                             kata_feature_layout layout, kata_dtype dtype, float* phi,
                             void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KATA_H */
