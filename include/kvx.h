/*
 * kvx: translation of a sender model's per-layer KV cache into a receiver
 * model's KV space without re-running the receiver's prefill, on MI355X
 * (gfx950).
 *
 * The operation is the translator of the interface KV_B(C) = T_{A->B}(KV_A(C))
 * ("A Universal Context-Reuse Layer for Cross-Model KV Sharing", section 2.2),
 * built from:
 *   - token alignment on shared character-end boundaries, forward fill, no
 *     averaging ("Prefill-Free Cross-Family KV Cache Transfer for
 *     Heterogeneous Multi-Agent LLMs", Key Contributions item 1 and
 *     Methodology step 1);
 *   - proportional layer matching with sender taps at -4, 0, +4 and
 *     flattened cross-head affine maps for K and V (same page, Methodology
 *     step 2), rank-16 corrections folded into one fixed affine map per layer
 *     and role (Methodology step 3);
 *   - RoPE stripping of cached keys, per-head d x d maps, the proportional
 *     layer formula and RoPE re-application at the receiver, and the closed
 *     form ridge fit W = (X^T X + lambda I)^-1 X^T Y ("Cross-Model KV Cache
 *     Transfer in Production: ... Closed-Form Ridge Projections ...",
 *     section "The Closed-Form Ridge Mapping Pipeline", stages 1-4).
 *
 * Conventions shared by every call:
 *   - Buffers are owned by the caller.  Pointers documented as "device" must
 *     point to memory of the device that is current on the calling thread;
 *     pointers documented as "host" are ordinary host memory.
 *   - Caches are dense [layers][tokens][kv_heads][head_dim] arrays, K and V
 *     separate, element type given by kvx_dtype.
 *   - Token offsets and maps are int32.
 *   - Streams are hipStream_t passed as void* (NULL = the default stream).
 *   - Argument and shape errors are reported before anything is launched.
 *     HIP runtime failures return KVX_ERR_HIP.  No C++ exception crosses
 *     this interface.
 *   - The library keeps no per-call state; calls on different streams with
 *     disjoint buffers may run concurrently.
 */
#ifndef KVX_H
#define KVX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVX_OK = 0,
  KVX_ERR_INVALID = 1,     /* bad argument value (null pointer, bad offsets, tap out of range) */
  KVX_ERR_SHAPE = 2,       /* inconsistent shapes between arguments */
  KVX_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the size query returns */
  KVX_ERR_NOT_SPD = 4,     /* regularised Gram matrix not positive definite */
  KVX_ERR_HIP = 5,         /* a HIP runtime call failed */
  KVX_ERR_UNSUPPORTED = 6, /* a valid combination the library does not implement */
  KVX_ERR_NOT_CONVERGED = 7 /* an iteration did not converge, or its result is not determined
                               (polar factor of a rank-deficient whitened cross-covariance) */
} kvx_status;

typedef enum { KVX_F32 = 0, KVX_BF16 = 1 } kvx_dtype;

/* Size limits checked by every entry point (larger values are refused with
 * KVX_ERR_INVALID or, for the fits, KVX_ERR_UNSUPPORTED; size queries return
 * 0): features of one cache row (kv_heads * head_dim), problems of one fit
 * call, and features on either side of a fitted map (a fit's fp64 matrices
 * of one problem then hold at most 2^28 elements, 2 GiB, which the fp64
 * products address with 32-bit byte offsets). */
#define KVX_MAX_ROW 65536
#define KVX_MAX_PROBLEMS 65535
#define KVX_MAX_FIT_FEATURES 16384

/* Shape of one role (K or V) of one model's cache. */
typedef struct {
  int32_t layers;     /* >= 1, <= 255 */
  int32_t tokens;     /* >= 0 */
  int32_t kv_heads;   /* >= 1; kv_heads * head_dim <= KVX_MAX_ROW */
  int32_t head_dim;   /* >= 1; even when rope_base > 0 */
  int32_t dtype;      /* kvx_dtype of the cache elements */
  double rope_base;   /* > 0: keys are stored rotated (RoPE, half-split pairs
                         (c, c + head_dim/2), angle pos * base^(-2j/head_dim));
                         0: keys are stored unrotated.  Values are never rotated. */
  const float* k_norm; /* receiver only ("Prefill-Free ...", Methodology 2: keys
                         are mapped before the receiver's own key normalisation
                         and RoPE): device fp32 [layers][head_dim] weights w of
                         an RMS normalisation of each translated key head vector,
                         y / sqrt(mean_c y_c^2 + k_norm_eps) * w, applied after
                         the bias and before the rotation; NULL: none.  Ignored
                         for the sender. */
  double k_norm_eps;  /* >= 0 */
} kvx_cache_desc;

/* Human-readable name of a status code (static string). */
const char* kvx_status_string(int status);

/* ------------------------------------------------------------------------
 * Token alignment ("Prefill-Free Cross-Family KV Cache Transfer ...",
 * Key Contributions 1, Methodology 1).
 *
 * send_end, recv_end: device int32 exclusive character-end offsets of the
 *   sender's n_send and the receiver's n_recv tokens over one shared string;
 *   each strictly increasing and > 0.
 * recv_to_send: device int32 [n_recv] output.  For receiver token i, let b be
 *   the largest offset that ends both a sender and a receiver token and is
 *   <= recv_end[i]; recv_to_send[i] is the sender token ending at b (so a
 *   receiver token whose end is shared takes the sender token ending at the
 *   same character, and an unshared one is forward-filled).  Receiver tokens
 *   before the first shared boundary map to sender token 0.  The result is
 *   non-decreasing.
 * workspace: device scratch of at least kvx_align_workspace_size(n_recv)
 *   bytes.
 * Synchronises `stream` once to read a device-side validity flag: offsets
 *   that are not strictly increasing and positive give KVX_ERR_INVALID (the
 *   output is then unspecified).  n_recv == 0 is a no-op; n_send == 0 with
 *   n_recv > 0 is KVX_ERR_SHAPE.
 * ---------------------------------------------------------------------- */
size_t kvx_align_workspace_size(int32_t n_recv);
int kvx_align_tokens(const int32_t* send_end, int32_t n_send,
                     const int32_t* recv_end, int32_t n_recv,
                     int32_t* recv_to_send, void* workspace, size_t ws_bytes,
                     void* stream);

/* ------------------------------------------------------------------------
 * Token alignment of n_seq sequences at once (several requests' caches
 * translated together).  Their tokens are concatenated: sequence q owns
 * sender tokens send_off[q] .. send_off[q+1]-1 and receiver tokens
 * recv_off[q] .. recv_off[q+1]-1 (send_off, recv_off: HOST int32 arrays of
 * n_seq + 1 non-decreasing entries starting at 0).  send_end / recv_end hold
 * each sequence's own character-end offsets (each sequence's string starts
 * at 0), with the rules of kvx_align_tokens per sequence.  recv_to_send
 * (device int32 [recv_off[n_seq]]) receives indices into the concatenated
 * sender tokens: the per-sequence alignment plus send_off[q].  A sequence
 * with receiver tokens and no sender tokens is KVX_ERR_SHAPE.
 * workspace: kvx_align_batched_workspace_size(recv_off, n_seq) bytes.
 * Synchronises `stream` once (KVX_ERR_INVALID if any sequence's offsets are
 * invalid).
 * ---------------------------------------------------------------------- */
size_t kvx_align_batched_workspace_size(const int32_t* recv_off, int32_t n_seq);
int kvx_align_tokens_batched(const int32_t* send_end, const int32_t* send_off,
                             const int32_t* recv_end, const int32_t* recv_off, int32_t n_seq,
                             int32_t* recv_to_send, void* workspace, size_t ws_bytes,
                             void* stream);

/* ------------------------------------------------------------------------
 * Layer matching ("Prefill-Free ...", Methodology 2: proportional depth and
 * taps at -4, 0, +4; "Cross-Model KV Cache Transfer in Production", stage 3).
 *
 * Host only.  taps_out: host int32 [recv_layers][n_taps].  Receiver layer l
 * matches m = round(l * (send_layers-1) / (recv_layers-1)) (halves rounded
 * up, exact integer arithmetic; m = 0 when recv_layers == 1) and reads sender
 * layers m + (t - (n_taps-1)/2) * tap_stride for t = 0..n_taps-1, clamped to
 * [0, send_layers-1], duplicates kept.  n_taps must be odd, 1..7.
 * ---------------------------------------------------------------------- */
int kvx_layer_map(int32_t send_layers, int32_t recv_layers, int32_t n_taps,
                  int32_t tap_stride, int32_t* taps_out);

/* ------------------------------------------------------------------------
 * Translation ("Cross-Model KV Cache Transfer in Production", pipeline
 * stages 1, 2 and 4; "Prefill-Free ...", Methodology 2).
 *
 * For every receiver layer l, receiver token i and role (K, V):
 *   j = recv_to_send[i];
 *   x = concat over t of the sender row cache[taps[l][t]][j][:][:]
 *       (feature f = t*H_S*d_S + h*d_S + c); keys of a sender with
 *       rope_base > 0 are first rotated back by position j;
 *   y = x W_l + b_l                  (flattened, per_head = 0), or
 *   y_h = x_h W_{l,h} + b_{l,h}      (per_head = 1: one tap, H and d equal on
 *                                     both sides, one d x d map per head);
 *   keys of a receiver with rope_base > 0 are then rotated to position i.
 *   The result is rounded to the receiver's dtype (nearest even).
 *
 * send, recv: host descriptors.  Layers, heads and head_dim must agree
 *   between K and V of one side; send->tokens is the sender token count,
 *   recv->tokens the receiver token count.
 * k_send, v_send: device caches of the sender (send->dtype).
 * k_recv, v_recv: device output caches of the receiver (recv->dtype; must
 *   equal send->dtype).  Either role may be NULL together with its maps to
 *   skip that role.
 * recv_to_send: device int32 [recv->tokens]; values must lie in
 *   [0, send->tokens) (values outside are clamped on the device, never read
 *   out of bounds).
 * taps: host int32 [recv->layers][n_taps], values in [0, send->layers).
 * w_dtype: element type of the maps (KVX_F32 or KVX_BF16).
 * wt_k, wt_v: device maps, row-major with y = x W:
 *   flattened: [L_R][n_taps*H_S*d_S][H_R*d_R], w[l][f][o] multiplies
 *              feature f into output o;
 *   per_head:  [L_R][H][d][d], w[l][h][c][o] multiplies channel c of head h
 *              into output channel o of head h.
 *   Each call first puts them into the kernels' layout inside the workspace
 *   (a transposition, and the conversions of kvx_prepare_maps); callers that
 *   translate repeatedly with the same maps prepare them once with
 *   kvx_prepare_maps and call kvx_translate_prepared.
 * b_k, b_v: device fp32 bias [L_R][H_R*d_R], or NULL for none.  The bias is
 *   added before the receiver rotation.
 * workspace: device scratch of kvx_translate_workspace_size(...) bytes.
 * Asynchronous on `stream`.
 *
 * Arithmetic: bf16 caches with bf16 maps use bf16 matrix cores; fp32 maps are
 * applied as a 16-bit high part plus a 16-bit low part; keys rotated back
 * from a rotated sender are fed as fp16 (the map converted to, or split
 * into, fp16), other bf16 rows as bf16; fp32 caches use fp32 arithmetic.
 * Accumulation is fp32 everywhere.
 * Range of the fp16 operands (rotated keys only): fp16 holds magnitudes up
 * to 65504 with 11 significant bits down to 2^-14 (about 6.1e-5).  Rotated-
 * back key values and key-map entries (bf16 maps converted to fp16, the high
 * part of a split fp32 map) beyond 65504 become infinities in the result;
 * nothing checks for them.  Smaller entries are kept as fp16 subnormals with
 * an absolute error of at most 2^-25 (bf16 maps) or below 2^-25 after the
 * low part (fp32 maps).  bf16 rows and maps (values, unrotated keys) have
 * bf16's range.
 * Supported: recv->dtype == send->dtype; bf16 caches need head_dim == 128
 * on both sides, and flattened bf16 translation needs H_R*d_R a multiple of
 * 256 (the kernel's output tile); fp32 caches take any head count and size
 * up to 8192 features on either side; recv->k_norm only on the flattened
 * bf16 path (KVX_ERR_UNSUPPORTED otherwise).
 * ---------------------------------------------------------------------- */
size_t kvx_translate_workspace_size(const kvx_cache_desc* send,
                                    const kvx_cache_desc* recv,
                                    int32_t n_taps, int32_t per_head);
int kvx_translate(const kvx_cache_desc* send, const void* k_send, const void* v_send,
                  const kvx_cache_desc* recv, void* k_recv, void* v_recv,
                  const int32_t* recv_to_send, const int32_t* taps, int32_t n_taps,
                  int32_t per_head, int32_t w_dtype, const void* wt_k, const void* wt_v,
                  const float* b_k, const float* b_v,
                  void* workspace, size_t ws_bytes, void* stream);

/* Same translation as kvx_translate, synchronous, reporting elapsed device
 * time of its two phases measured with HIP events on `stream`:
 * stage_ms[0] = preparation (run compaction, rotation tables, rotated-back
 * key rows), stage_ms[1] = the translation kernel itself.  stage_ms: host
 * float[2] (both 0 when nothing was launched).  For benchmarks and
 * profiling; the results are bit-identical to kvx_translate. */
int kvx_translate_timed(const kvx_cache_desc* send, const void* k_send, const void* v_send,
                        const kvx_cache_desc* recv, void* k_recv, void* v_recv,
                        const int32_t* recv_to_send, const int32_t* taps, int32_t n_taps,
                        int32_t per_head, int32_t w_dtype, const void* wt_k, const void* wt_v,
                        const float* b_k, const float* b_v,
                        void* workspace, size_t ws_bytes, void* stream, float* stage_ms);

/* ------------------------------------------------------------------------
 * Feature gather: the flattened sender features that the translation feeds
 * to the map, written out for a fit ("Prefill-Free ...", Methodology 2).
 *
 * send: host descriptor; kv_send: device cache of one role.
 * derotate: nonzero rotates keys back by the sender position (send->rope_base
 *   must be > 0).
 * recv_to_send: device int32 [n_rows]; taps_of_layer: host int32 [n_taps].
 * x_out: device [n_rows][n_taps*H*d] in send->dtype (rotated-back keys are
 *   rounded to that dtype).  Asynchronous.
 * ---------------------------------------------------------------------- */
int kvx_gather_features(const kvx_cache_desc* send, const void* kv_send, int32_t derotate,
                        const int32_t* recv_to_send, int32_t n_rows,
                        const int32_t* taps_of_layer, int32_t n_taps,
                        void* x_out, void* stream);

/* ------------------------------------------------------------------------
 * Translation placed into the receiver's paged KV cache, for one or several
 * sequences at once ("Cross-Model KV Cache Transfer in Production", stage 4:
 * the translated keys and values go straight into the receiver's
 * PagedAttention cache slots; "Prefill-Free ...", Main Findings: requests
 * translated in batches).
 *
 * Arguments as kvx_translate, plus `place` (host, may be NULL = plain
 * kvx_translate):
 *   slot: device int64 [recv->tokens] or NULL: the row of receiver token i in
 *     the output pool; k_recv / v_recv are then [recv->layers][pool_rows]
 *     [H_R][d_R] and layer l of token i is written at row l * pool_rows +
 *     slot[i] (a slot outside [0, pool_rows) writes nothing).  NULL: row i,
 *     pool_rows >= recv->tokens (0 means recv->tokens).
 *   recv_pos: device int32 [recv->tokens] or NULL: rotary position of
 *     receiver token i (NULL: i).  send_pos: device int32 [send->tokens] or
 *     NULL: rotary position of sender token j (NULL: j).  Positions are
 *     clamped to [0, pos_limit).
 *   pos_limit: > every position given; sizes the rotation tables.
 * Several sequences: concatenate their sender tokens and their receiver
 * tokens, take recv_to_send from kvx_align_tokens_batched (indices into the
 * concatenated sender tokens), positions relative to each sequence's start,
 * and slots from each sequence's block table (slot = block * block_size +
 * offset).  Runs of equal sender tokens never cross sequences, so each
 * sequence's rows are exactly its own translation.
 * workspace: kvx_translate_placed_workspace_size(send, recv, n_taps,
 *   per_head, pos_limit) bytes.
 * Supported on the bf16 paths (flattened and per head); fp32 caches with a
 * placement give KVX_ERR_UNSUPPORTED.
 * ---------------------------------------------------------------------- */
typedef struct {
  const int64_t* slot;
  int64_t pool_rows;
  const int32_t* recv_pos;
  const int32_t* send_pos;
  int32_t pos_limit;
} kvx_placement;

size_t kvx_translate_placed_workspace_size(const kvx_cache_desc* send,
                                           const kvx_cache_desc* recv, int32_t n_taps,
                                           int32_t per_head, int32_t pos_limit);
int kvx_translate_placed(const kvx_cache_desc* send, const void* k_send, const void* v_send,
                         const kvx_cache_desc* recv, void* k_recv, void* v_recv,
                         const int32_t* recv_to_send, const int32_t* taps, int32_t n_taps,
                         int32_t per_head, int32_t w_dtype, const void* wt_k,
                         const void* wt_v, const float* b_k, const float* b_v,
                         void* workspace, size_t ws_bytes, void* stream,
                         const kvx_placement* place);

/* ------------------------------------------------------------------------
 * Closed-form ridge fit ("Cross-Model KV Cache Transfer in Production",
 * stage 2: W = (X^T X + lambda I)^-1 X^T Y; section "Implementation
 * Guidelines": lambda in [1e-4, 1e-2]).
 *
 * x: device [n_rows][f_in] with row stride ldx elements; y: device
 *   [n_rows][f_out] with row stride ldy; both of in_dtype.  bf16 rows are
 *   read in 16-byte pieces: f_in, f_out, ldx and ldy must be multiples of 8
 *   and x, y 16-byte aligned (KVX_ERR_UNSUPPORTED otherwise).
 * lambda = lambda_abs + lambda_rel * trace(G) / f_in, where G = X^T X (or the
 *   centred Gram when fit_intercept != 0).
 * fit_intercept != 0: the bias is unpenalised; X and Y are centred by their
 *   column means, W solves the centred system and b = mean_y - mean_x W.
 * w_out: device fp32 [f_in][f_out], row-major (y = x W: the layout
 *   kvx_translate and kvx_prepare_maps take); b_out: device fp32 [f_out]
 *   (written only with fit_intercept; may be NULL otherwise).
 * workspace: device scratch of kvx_fit_ridge_workspace_size(f_in, f_out).
 * f_in, f_out <= KVX_MAX_FIT_FEATURES (KVX_ERR_UNSUPPORTED beyond).
 * G and X^T Y are accumulated in fp32 on matrix cores; the solve (Cholesky
 * factorisation and two triangular solves) runs in fp64.
 * Synchronises `stream` once to read the factorisation flag:
 *   KVX_ERR_NOT_SPD when G + lambda I is not positive definite.
 * ---------------------------------------------------------------------- */
size_t kvx_fit_ridge_workspace_size(int32_t f_in, int32_t f_out);
int kvx_fit_ridge(const void* x, int64_t ldx, const void* y, int64_t ldy, int32_t in_dtype,
                  int64_t n_rows, int32_t f_in, int32_t f_out,
                  double lambda_abs, double lambda_rel, int32_t fit_intercept,
                  float* w_out, float* b_out, void* workspace, size_t ws_bytes,
                  void* stream);

/* ------------------------------------------------------------------------
 * The same fit for `count` problems of one shape (the maps of every receiver
 * layer and role of one model pair, same source), with the results of
 * `count` calls of kvx_fit_ridge.  The serial chain of the fp64 solve (one
 * diagonal factor after another) then runs once for all problems, each of
 * its launches covering every problem.
 *
 * x, y, w_out, b_out: HOST arrays of `count` device pointers, each as in
 *   kvx_fit_ridge (b_out may be NULL without fit_intercept).
 * status: host int32 [count] or NULL; receives KVX_OK or KVX_ERR_NOT_SPD
 *   per problem.  count <= KVX_MAX_PROBLEMS (KVX_ERR_UNSUPPORTED beyond).
 * workspace: device scratch of kvx_fit_ridge_batched_workspace_size(count,
 *   f_in, f_out) bytes (the Gram partials, shared, plus about
 *   8 (f_in + 1)(f_in + f_out) bytes per problem).
 * Returns KVX_ERR_NOT_SPD when any problem is not positive definite (the
 * others are still solved), otherwise as kvx_fit_ridge.  Synchronises
 * `stream` once.
 * ---------------------------------------------------------------------- */
size_t kvx_fit_ridge_batched_workspace_size(int32_t count, int32_t f_in, int32_t f_out);
int kvx_fit_ridge_batched(int32_t count, const void* const* x, int64_t ldx, const void* const* y,
                          int64_t ldy, int32_t in_dtype, int64_t n_rows, int32_t f_in,
                          int32_t f_out, double lambda_abs, double lambda_rel,
                          int32_t fit_intercept, float* const* w_out, float* const* b_out,
                          int32_t* status, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * The ridge fits of every receiver layer and role of one model pair,
 * straight from the calibration caches ("Cross-Model KV Cache Transfer in
 * Production", stage 2: W = (X^T X + lambda I)^-1 X^T Y per layer pair, with
 * X the sender features of the matched layers (stage 3's layer map and the
 * taps) at each receiver token's aligned sender token, and Y the receiver's
 * own cache rows).  The result equals kvx_fit_ridge_batched on the features
 * kvx_gather_features builds (no rotation, no intercept), up to the rounding
 * of the sums, without materialising those features:
 *   - a receiver token's feature row is the row of its aligned sender token,
 *     so X^T X = sum over runs u of equal map values of c_u x_u x_u^T (c_u =
 *     the run's length): formed from the distinct rows, each run's count
 *     written in binary, the rows with bit j set accumulated as one group and
 *     the groups combined by exact doublings (every product stays exact in
 *     the fp32 sums, as in kvx_fit_ridge_batched);
 *   - X^T Y = sum over runs of x_u (sum of the run's target rows)^T, each
 *     run's target sum formed in fp32 in token order and taken to 16
 *     significant bits as a high and a low bf16 part (the error this adds is
 *     at most 2^-16 of the sum, below the fp32 accumulation error of the
 *     products).
 *
 * send, k_send, v_send: the sender's calibration caches [L_S][N_S][H_S][d_S]
 *   (bf16, 16-byte aligned).  With send->rope_base > 0 the keys are stored
 *   rotated: each key row is rotated back at its sender position (its token
 *   index; pairs (c, c + d/2), fp32 from an fp64-derived table) and rounded
 *   to bf16, as kvx_gather_features does (the fit then equals the fit on
 *   those rounded features; the rounding is a 2^-9 relative perturbation of
 *   the inputs that an ill-conditioned system amplifies); d_S must then be a
 *   multiple of 16.  Values are never rotated.
 * recv, k_recv, v_recv: the receiver's calibration caches [L_R][N][H_R][d_R]
 *   (bf16, 16-byte aligned), the targets of each receiver layer;
 *   N = recv->tokens.  With recv->rope_base > 0 the target keys are rotated
 *   back at the receiver position before they are summed (fp32); d_R must
 *   then be a multiple of 16.
 * recv_to_send: device int32 [N], the calibration alignment (values clamped
 *   into [0, N_S) as in kvx_translate).
 * taps: host int32 [L_R][n_taps] from kvx_layer_map; the features of
 *   receiver layer l are taps[l][0..n_taps) x H_S d_S (F_in = n_taps H_S d_S,
 *   F_out = H_R d_R).  H_S d_S must be a multiple of 256; F_out a multiple
 *   of 8; F_in, F_out <= KVX_MAX_FIT_FEATURES.
 * lambda = lambda_abs + lambda_rel * trace(X^T X) / F_in per problem.
 * w_k, w_v: device fp32 [L_R][F_in][F_out] (row-major, y = x W, the layout
 *   kvx_translate takes), or NULL to skip that role (at least one given).
 *   No intercept is fitted (use kvx_fit_ridge_batched for one).
 * status: host int32 [2][L_R] or NULL: per role and layer KVX_OK or
 *   KVX_ERR_NOT_SPD (a skipped role's entries are KVX_OK).
 * workspace: kvx_fit_ridge_caches_workspace_size(send, recv, n_taps) bytes
 *   (sized for the worst case of N runs of one token: the fp64 systems of
 *   2 L_R problems plus, for one role at a time, the distinct sender rows of
 *   every sender layer, twice, and the receiver's run sums; with rotated
 *   keys also the (cos, sin) tables of the positions).
 * Synchronises `stream` twice (the run lengths, the factorisation flags).
 * KVX_ERR_UNSUPPORTED for other dtypes or shapes; otherwise errors as
 * kvx_fit_ridge_batched.
 * ---------------------------------------------------------------------- */
size_t kvx_fit_ridge_caches_workspace_size(const kvx_cache_desc* send, const kvx_cache_desc* recv,
                                           int32_t n_taps);
int kvx_fit_ridge_caches(const kvx_cache_desc* send, const void* k_send, const void* v_send,
                         const kvx_cache_desc* recv, const void* k_recv, const void* v_recv,
                         const int32_t* recv_to_send, const int32_t* taps, int32_t n_taps,
                         double lambda_abs, double lambda_rel, float* w_k, float* w_v,
                         int32_t* status, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * kvx_align_tokens without synchronisation, for callers that chain the
 * alignment and the translation on one stream: the same map, and *invalid
 * (device int32) is set to 1 when an offset array is not positive and
 * strictly increasing, else 0, for the caller to read when it synchronises.
 * The map is unspecified when *invalid is 1.  Host-side argument errors are
 * returned as by kvx_align_tokens.  Asynchronous on `stream`.
 * ---------------------------------------------------------------------- */
int kvx_align_tokens_async(const int32_t* send_end, int32_t n_send, const int32_t* recv_end,
                           int32_t n_recv, int32_t* recv_to_send, int32_t* invalid,
                           void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * kvx_align_tokens_async for callers that cannot allocate (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): no
 * workspace argument, and the call allocates nothing.  Its scratch (the
 * scan's per-tile aggregates) is a static device array of the library,
 * 64 KiB per device, held until the process ends; its address on each device
 * is looked up once, on the first call there.
 *
 * Arguments, result and the device-side validity flag as
 * kvx_align_tokens_async.  n_recv > KVX_NOALLOC_MAX_RECV returns
 * KVX_ERR_WORKSPACE before anything is launched.  All calls on one device
 * share its scratch: calls that overlap on one device (different streams
 * without ordering) race and must not be issued; calls in stream order may
 * follow each other freely (nothing carries over between calls).
 * Asynchronous on `stream`.
 * ---------------------------------------------------------------------- */
#define KVX_NOALLOC_MAX_RECV (1 << 24)
int kvx_align_tokens_noalloc(const int32_t* send_end, int32_t n_send, const int32_t* recv_end,
                             int32_t n_recv, int32_t* recv_to_send, int32_t* invalid, void* stream);

/* ------------------------------------------------------------------------
 * kvx_translate recording three caller-created events (hipEvent_t, passed
 * as void*) on `stream`: events[0] before the preparation kernels,
 * events[1] before the translation kernel, events[2] after it; nothing is
 * synchronised, so a caller can time many calls and read the events once.
 * Nothing is recorded when the call has no work (empty problem).  Arguments
 * and errors otherwise as kvx_translate; NULL events return KVX_ERR_INVALID.
 * ---------------------------------------------------------------------- */
int kvx_translate_recorded(const kvx_cache_desc* send, const void* k_send, const void* v_send,
                           const kvx_cache_desc* recv, void* k_recv, void* v_recv,
                           const int32_t* recv_to_send, const int32_t* taps, int32_t n_taps,
                           int32_t per_head, int32_t w_dtype, const void* wt_k, const void* wt_v,
                           const float* b_k, const float* b_v, void* workspace, size_t ws_bytes,
                           void* stream, void* const* events);

/* ------------------------------------------------------------------------
 * Prepared maps: the maps of one role put once into the layout the
 * translation kernels read, so repeated translations with the same maps do
 * no per-call conversion ("Cross-Model KV Cache Transfer in Production",
 * stages 2 and 4: the projections are fixed once fitted and applied to every
 * new cache).
 *
 * kvx_prepare_maps: w: device maps of `role` (0 = K, 1 = V) in the layout
 *   kvx_translate takes (row-major [L_R][F_in][F_out], or [L_R][H][d][d] per
 *   head), element type w_dtype (KVX_F32 or KVX_BF16).  prepared: device
 *   buffer of kvx_prepared_maps_size(...) bytes that receives the kernel
 *   layout: the maps transposed to output-major, and for flattened bf16
 *   caches converted to the role's operand type: bf16, or fp16 for keys of a
 *   rotated sender (send->rope_base > 0); fp32 maps split into a 16-bit high
 *   and low part (each rounded to nearest even; the range limits of fp16
 *   operands under kvx_translate apply).  The layout depends on send->dtype,
 *   send->rope_base, per_head, role and w_dtype: a prepared buffer is valid
 *   only for translations with the same values (and shapes).
 *   Asynchronous on `stream`.  KVX_ERR_WORKSPACE when prepared_bytes is too
 *   small.
 *
 * kvx_translate_prepared: kvx_translate with prepared maps pk, pv (either
 *   NULL with its role skipped) of the given w_dtype, and optionally a
 *   placement (`place`, as kvx_translate_placed; NULL = none) and three
 *   events (`events`, as kvx_translate_recorded; NULL = none).  workspace:
 *   kvx_translate_prepared_workspace_size(send, recv, n_taps, per_head,
 *   pos_limit) bytes (pos_limit 0 without per-token positions), which holds
 *   no maps.  Results are bit-identical to kvx_translate with the maps the
 *   buffers were prepared from.  Asynchronous on `stream`.
 * ---------------------------------------------------------------------- */
size_t kvx_prepared_maps_size(const kvx_cache_desc* send, const kvx_cache_desc* recv,
                              int32_t n_taps, int32_t per_head, int32_t role, int32_t w_dtype);
int kvx_prepare_maps(const kvx_cache_desc* send, const kvx_cache_desc* recv, int32_t n_taps,
                     int32_t per_head, int32_t role, int32_t w_dtype, const void* w,
                     void* prepared, size_t prepared_bytes, void* stream);
size_t kvx_translate_prepared_workspace_size(const kvx_cache_desc* send,
                                             const kvx_cache_desc* recv, int32_t n_taps,
                                             int32_t per_head, int32_t pos_limit);
int kvx_translate_prepared(const kvx_cache_desc* send, const void* k_send, const void* v_send,
                           const kvx_cache_desc* recv, void* k_recv, void* v_recv,
                           const int32_t* recv_to_send, const int32_t* taps, int32_t n_taps,
                           int32_t per_head, int32_t w_dtype, const void* pk, const void* pv,
                           const float* b_k, const float* b_v, void* workspace, size_t ws_bytes,
                           void* stream, const kvx_placement* place, void* const* events);

/* ------------------------------------------------------------------------
 * FP8 map storage ("Cross-Model KV Cache Transfer in Production",
 * Implementation Guidelines: weight matrices may be stored quantised, e.g.
 * FP8, while the products keep 16-bit operands).
 *
 * kvx_quantize_fp8: w: device fp32 [count][f_in][f_out], row-major maps
 * (y = x W; e.g. every layer's map of one role, count = L_R).  Per map and
 * output o:
 *   scale = amax_f |w[f][o]| / 448 (fp32, correctly rounded; 1 when that is 0),
 *   q = the nearest OCP E4M3 code of w[f][o] / scale (fp32 quotient, correctly
 *       rounded; ties to the even code; beyond 448 saturated to +-448),
 * so w[f][o] is stored as scale[o] * e4m3(q[o][f]).  q_out: device uint8
 * [count][f_out][f_in] (output-major: the layout kvx_translate_fp8 reads);
 * scale_out: device fp32 [count][f_out].  Inputs must be finite.  count up
 * to 65535.  Asynchronous on `stream`.
 * ---------------------------------------------------------------------- */
int kvx_quantize_fp8(const float* w, int32_t count, int32_t f_in, int32_t f_out, uint8_t* q_out,
                     float* scale_out, void* stream);

/* ------------------------------------------------------------------------
 * kvx_translate with fp8 maps: the flattened path (per_head = 0) of
 * kvx_translate for bf16 caches, the maps given as E4M3 codes and scales as
 * kvx_quantize_fp8 writes them: wq_k / wq_v device uint8 [L_R][F_out][F_in]
 * (output-major), s_k / s_v device fp32 [L_R][F_out] (needed for each role
 * translated).  The map of output o is s[o] * e4m3(wq[o][:]): the codes are
 * widened exactly to the operand type of the role (bf16, or fp16 for
 * rotated-back keys), products accumulate in fp32 and the sum is scaled by
 * s[o] before the bias.  Every other argument, the workspace size
 * (kvx_translate_workspace_size with per_head = 0) and the error behaviour
 * are those of kvx_translate; per-head translation and fp32 caches return
 * KVX_ERR_UNSUPPORTED.
 * stage_ms: NULL (asynchronous) or host float[2]: as kvx_translate_timed
 * (synchronises `stream`).
 * ---------------------------------------------------------------------- */
int kvx_translate_fp8(const kvx_cache_desc* send, const void* k_send, const void* v_send,
                      const kvx_cache_desc* recv, void* k_recv, void* v_recv,
                      const int32_t* recv_to_send, const int32_t* taps, int32_t n_taps,
                      const uint8_t* wq_k, const uint8_t* wq_v, const float* s_k, const float* s_v,
                      const float* b_k, const float* b_v, void* workspace, size_t ws_bytes,
                      void* stream, float* stage_ms);

/* ------------------------------------------------------------------------
 * Moment-matched ("Recolor") fit of `count` affine maps of one shape
 * ("Prefill-Free Cross-Family KV Cache Transfer ...", Key Contributions 2 and
 * Methodology 3: both feature spaces are whitened, aligned by an orthogonal
 * Procrustes solution, and the receiver's means and covariances are put
 * back):
 *   S_xx, S_yy, S_xy = covariances of the centred calibration rows,
 *   S_xx += rho_x trace(S_xx) / f_in I,  S_yy += rho_y trace(S_yy) / f_out I,
 *   M = A_x^T S_xy A_y for whitenings with A^T S A = I,
 *   Q = the polar factor of M (orthonormal columns, Q = U V^T from M's SVD),
 *   W = A_x Q A_y^-1,  b = mean_y - mean_x W.
 * W does not depend on the choice of whitening.  The translated calibration
 * rows x W + b have the receiver's mean and (with rho_x = 0) covariance.
 *
 * x, y: HOST arrays of `count` device pointers to [n_rows][f_in] (row stride
 *   ldx) and [n_rows][f_out] (row stride ldy) matrices of in_dtype; bf16
 *   rows need f_in, f_out, ldx, ldy multiples of 8 and 16-byte aligned bases.
 * f_in >= f_out (Q with orthonormal columns); f_in < f_out returns
 *   KVX_ERR_UNSUPPORTED, as do count > KVX_MAX_PROBLEMS and f_in >
 *   KVX_MAX_FIT_FEATURES.
 * rho_x, rho_y >= 0: relative regularisers (rows that repeat a layer tap make
 *   S_xx singular; rho_x > 0 is then required).
 * w_out: HOST array of device fp32 [f_in][f_out] (row-major, y = x W + b,
 *   the layout kvx_translate takes); b_out: HOST array of device fp32
 *   [f_out]; neither may be NULL.
 * status: host int32 [count] or NULL; receives per problem KVX_OK,
 *   KVX_ERR_NOT_SPD (a regularised covariance is not positive definite) or
 *   KVX_ERR_NOT_CONVERGED (M numerically rank-deficient, so Q is not
 *   determined: the iteration did not converge, or ||(M^T M / c)^-1/2||_F >
 *   1e6 for the iteration's scale c (about 1.1 times the largest eigenvalue
 *   of M^T M); this happens when the calibration rows hold fewer distinct
 *   sender rows than f_out).
 * iters: host int32 or NULL; receives the number of polar iterations run.
 * workspace: device scratch of kvx_fit_recolor_workspace_size(count, f_in,
 *   f_out) bytes (the Gram partials, shared, plus about
 *   8 (f_in^2 + 2 f_in f_out + 7 f_out^2) bytes per problem).
 * Moments are accumulated as in kvx_fit_ridge (bf16: fp32 on matrix cores,
 * partials added in fp64); the factorisations, the polar iteration (coupled
 * third-order Newton-Schulz for (M^T M)^-1/2) and the products run in fp64.
 * Synchronises `stream` once per polar iteration.  Returns the first non-OK
 * problem status, else KVX_OK; argument errors as kvx_fit_ridge.
 * ---------------------------------------------------------------------- */
size_t kvx_fit_recolor_workspace_size(int32_t count, int32_t f_in, int32_t f_out);
int kvx_fit_recolor(int32_t count, const void* const* x, int64_t ldx, const void* const* y,
                    int64_t ldy, int32_t in_dtype, int64_t n_rows, int32_t f_in, int32_t f_out,
                    double rho_x, double rho_y, float* const* w_out, float* const* b_out,
                    int32_t* status, int32_t* iters, void* workspace, size_t ws_bytes,
                    void* stream);

/* ------------------------------------------------------------------------
 * The Recolor fits of every receiver layer and role of one model pair,
 * straight from the calibration caches: kvx_fit_recolor on the features
 * kvx_gather_features builds and each receiver layer's own rows, without
 * materialising the features (the moment-matched fit of "Prefill-Free
 * Cross-Family KV Cache Transfer ...", Methodology 3, on the calibration
 * alignment and stage 3's layer map of "Cross-Model KV Cache Transfer in
 * Production").  The feature moments come from the alignment's runs as in
 * kvx_fit_ridge_caches (X^T X, X^T Y); the feature column sums are the
 * distinct sender rows weighted by their run lengths, summed in fp64; Y^T Y
 * and the target column sums come from the receiver rows as in
 * kvx_fit_recolor.  The solve (whitening, polar factor, W, b) is
 * kvx_fit_recolor's, for all 2 L_R problems at once.
 *
 * send, k_send, v_send, recv, k_recv, v_recv, recv_to_send, taps, n_taps:
 *   as for kvx_fit_ridge_caches (same shape limits); F_in >= F_out besides
 *   (else KVX_ERR_UNSUPPORTED).
 * rho_x, rho_y >= 0: as for kvx_fit_recolor.
 * w_k, w_v: device fp32 [L_R][F_in][F_out], or NULL to skip that role (at
 *   least one given); b_k, b_v: device fp32 [L_R][F_out], required for each
 *   role fitted (the intercept is part of the map).
 * status: host int32 [2][L_R] or NULL: per role and layer KVX_OK,
 *   KVX_ERR_NOT_SPD or KVX_ERR_NOT_CONVERGED as in kvx_fit_recolor (a
 *   skipped role's entries are KVX_OK).  iters: host int32 or NULL: the
 *   polar iterations run.
 * workspace: kvx_fit_recolor_caches_workspace_size(send, recv, n_taps)
 *   bytes (worst case, as for kvx_fit_ridge_caches, plus the Recolor solve's
 *   per-problem matrices and, with rotated receiver keys, one layer of them
 *   rotated back for Y^T Y).
 * Synchronises `stream` once for the run lengths and once per polar
 * iteration.  Returns the first non-OK problem status, else KVX_OK; argument
 * errors as kvx_fit_ridge_caches.
 * ---------------------------------------------------------------------- */
size_t kvx_fit_recolor_caches_workspace_size(const kvx_cache_desc* send, const kvx_cache_desc* recv,
                                             int32_t n_taps);
int kvx_fit_recolor_caches(const kvx_cache_desc* send, const void* k_send, const void* v_send,
                           const kvx_cache_desc* recv, const void* k_recv, const void* v_recv,
                           const int32_t* recv_to_send, const int32_t* taps, int32_t n_taps,
                           double rho_x, double rho_y, float* w_k, float* w_v, float* b_k,
                           float* b_v, int32_t* status, int32_t* iters, void* workspace,
                           size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Rank-r fold ("Prefill-Free ...", Methodology 3: low-rank corrections folded
 * into one fixed affine map per layer and role).
 *
 * For each of `count` maps, all row-major (y = x W): w: device fp32
 * [f_in][f_out]; a: device fp32 [f_in][rank]; b: device fp32 [rank][f_out];
 * W_eff = W + A B:
 * w_out[f][o] = w[f][o] + sum_r a[f][r] * b[r][o], each product rounded to
 * fp32, the products summed in rank order r = 0, 1, ... in fp32 and the sum
 * added to w[f][o] in fp32 (no fused multiply-add anywhere), then stored as
 * out_dtype (bf16: nearest even).  The maps are consecutive in memory.
 * w_out: device, count*f_in*f_out elements; must not overlap the inputs.
 * The fold runs on the device (one pass over the maps), asynchronous on
 * `stream`.
 * ---------------------------------------------------------------------- */
int kvx_fold_lowrank(const float* w, const float* a, const float* b, int32_t count,
                     int32_t f_in, int32_t f_out, int32_t rank, void* w_out,
                     int32_t out_dtype, void* stream);

/* ------------------------------------------------------------------------
 * Measurement probes (not part of the translation): the rates this chip
 * sustains, the denominators of "fraction of achievable peak" beside the
 * published peaks.
 *
 * kvx_probe_hbm: mode 0 copies `bytes` from device buffer a to device buffer
 *   b (each byte read once and written once), mode 1 reads a (b: device
 *   uint32 sink of kvx_probe_scratch_words() words), mode 2 fills a.  bytes:
 *   a positive multiple of 16, far above the 256 MB last-level cache for an
 *   HBM figure.  16-byte vector accesses, eight per thread and pass with the
 *   loads issued before the stores.  One untimed
 *   launch, then `iters` launches between two events on `stream`;
 *   *ms_per_launch = their mean.  Synchronises `stream`.
 * kvx_probe_mfma: every wave of 8 per compute unit issues `reps` x 4
 *   independent v_mfma_f32_32x32x16_bf16 (bf16 dense products, fp32
 *   accumulation); out: device float scratch of kvx_probe_scratch_words()
 *   entries (receives the accumulator sums).  Timed like kvx_probe_hbm;
 *   *flops_per_launch = the products' flops (2 m n k each).
 * kvx_probe_scratch_words: scratch words either probe needs on the current
 *   device.
 * ---------------------------------------------------------------------- */
int kvx_probe_hbm(int32_t mode, void* a, void* b, int64_t bytes, int32_t iters, float* ms_per_launch,
                  void* stream);
int kvx_probe_mfma(float* out, int32_t reps, int32_t iters, float* ms_per_launch,
                   double* flops_per_launch, void* stream);
int32_t kvx_probe_scratch_words(void);

#ifdef __cplusplus
}
#endif

#endif /* KVX_H */
