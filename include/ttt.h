/*
 * ttt.h -- C ABI of the MI355X (gfx950) Test-Time-Training layer library.
 *
 * One call computes the forward pass of a TTT layer for every (batch, head)
 * pair: the key/value pairs of the pair are a small training set for a
 * fast-weight inner model F_W; the library instance-normalises the keys, runs
 * F_W on them, back-propagates the reconstruction loss by hand to dW, takes one
 * gradient step with learning rate eta and reads the result out on the queries:
 *
 *     V_hat = F_W(K_hat),   W* = W0 - eta * dL(V_hat, V)/dW,   O = F_W*(Q)
 *
 * (ViT3 summary page, section 02 "method essence", update equation; single
 * full-batch step: section 03 guideline 2.)  With chunk > 0 the sequence is cut
 * into causal chunks: each chunk first reads the weights left by the chunks
 * before it, then takes its own step on its keys and values, with per-token
 * learning rates and an optional L2 re-normalisation of the weights after each
 * step (LaCT analysis page, sections "Nonlinear memory complements local
 * attention" and "Order of operations excludes leaking the future").
 *
 * Conventions shared by every entry point
 *   - Every function returns a ttt_status; nothing throws across the ABI.
 *     ttt_last_error() returns a human-readable message for the last failure.
 *   - All tensor pointers are DEVICE pointers (memory of the current HIP
 *     device), owned by the caller.  The library allocates no device memory:
 *     scratch space is the caller's `workspace`.
 *   - ttt_forward only enqueues work on `stream` (a hipStream_t; NULL is the
 *     default stream) and returns without synchronising, unless the flag
 *     TTT_FLAG_CHECK_FINITE is set.  Arguments are validated on the host before
 *     anything is enqueued; an invalid call enqueues nothing.
 *   - A handle holds host state only.  One handle must not be used by two
 *     threads at the same time; calls on one handle are ordered by the caller.
 *   - Dense row-major layouts, no padding between rows:
 *       q, k, v, o     [B, H, N, d]       dtype of the config (fp32 or bf16),
 *                                         16-byte aligned (TTT_ERR_INVALID if not)
 *       weights        [in, out] per matrix, fp32 (see ttt_weights)
 *       per-token eta  [B, H, N]          fp32
 */
#ifndef TTT_H_
#define TTT_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TTT_ABI_VERSION 2

typedef enum {
  TTT_OK = 0,
  TTT_ERR_INVALID = 1,      /* bad argument: null pointer, bad size, unknown enum */
  TTT_ERR_UNSUPPORTED = 2,  /* valid request this library does not implement */
  TTT_ERR_HIP = 3,          /* a HIP runtime call failed; see ttt_last_error */
  TTT_ERR_NONFINITE = 4,    /* TTT_FLAG_CHECK_FINITE: O or the final weights hold NaN/Inf */
  TTT_ERR_WORKSPACE = 5     /* workspace pointer null or smaller than ttt_workspace_bytes */
} ttt_status;

typedef enum { TTT_F32 = 0, TTT_BF16 = 1 } ttt_dtype;

/* Reconstruction loss (ViT3 page, section 03 guideline 1; LaCT page):
 *   TTT_LOSS_MSE: L = sum_n eta_n/(n_b*d) * ||F(k_n) - v_n||^2   (mean over the
 *                 n_b*d entries of the update batch, token-weighted by eta_n)
 *   TTT_LOSS_DOT: L = -sum_n eta_n * <F(k_n), v_n>                (negative dot product) */
typedef enum { TTT_LOSS_MSE = 0, TTT_LOSS_DOT = 1 } ttt_loss;

/* Inner model F_W, row-vector convention, every matrix stored [in, out]:
 *   TTT_INNER_LINEAR  : F(x) = x W                     w[0] = W  [d, d]
 *   TTT_INNER_MLP_GELU: F(x) = gelu(x W1) W2           w[0] = W1 [d, h], w[1] = W2 [h, d]
 *   TTT_INNER_SWIGLU  : F(x) = (silu(x W1) * (x W3)) W2
 *                                  w[0] = W1 [d, h], w[1] = W2 [h, d], w[2] = W3 [d, h]
 *   TTT_INNER_GLU     : F(x) = (x W1) * silu(x W2)     w[0] = W1 [d, d], w[1] = W2 [d, d]
 *                       (the simplified gated linear unit; hidden is ignored)
 *   TTT_INNER_DWCONV  : F(x)[t, c] = sum_{a, b} w[c, a k + b] x[t(i + a - r, j + b - r), c]
 *                       a depthwise k x k cross-correlation over the token
 *                       raster (token t = i grid_w + j, r = (k - 1) / 2, zero
 *                       padding); the kernel is the fast weight, w[0] = [d, k*k]
 *   TTT_INNER_VIT3    : the ViT3 block: head 0 is a DWCONV head, heads 1..H-1
 *                       are GLU heads; w[0], w[1] = the GLU matrices [H, d, d],
 *                       w[2] = the convolution kernels [H, d, k*k] (each head
 *                       reads only the entries of its own model; W_out rows of
 *                       the other model are not written)
 * gelu is the exact erf form.  (ViT3 page, guideline 4: two-layer MLP of width
 * h = r*d; guideline 6, the inner-model table and section 04: simplified GLU,
 * depthwise convolution, one convolution head per block; LaCT page: SwiGLU
 * fast weights with three matrices.)  DWCONV and VIT3 are full-batch only
 * (chunk 0) and take neither TTT_RULE_MUON nor renorm, which are defined for
 * matrices; VIT3 needs W0.batch_stride == 0. */
typedef enum {
  TTT_INNER_LINEAR = 0, TTT_INNER_MLP_GELU = 1, TTT_INNER_SWIGLU = 2,
  TTT_INNER_GLU = 3, TTT_INNER_DWCONV = 4, TTT_INNER_VIT3 = 5
} ttt_inner;

/* Flags (ttt_config.flags). */
#define TTT_FLAG_CHECK_FINITE 0x1u   /* after the call, synchronise the stream and
                                        return TTT_ERR_NONFINITE if O or the final
                                        weights hold a NaN or Inf */
#define TTT_FLAG_FORCE_GENERIC 0x2u  /* use the generic fp32-arithmetic kernels even
                                        where an MFMA kernel exists.  The GELU-MLP
                                        MFMA kernels (bf16 tensors, d = 64) carry
                                        the activations, the loss gradient and dZ
                                        as f16, so they need |F(k) - v|, |v| and
                                        the pre-activations below ~4e4; larger
                                        values overflow to Inf (reported by
                                        TTT_FLAG_CHECK_FINITE).  This flag lifts
                                        that limit at fp32-kernel speed. */
#define TTT_FLAG_LOG 0x4u            /* print the chosen kernels and launch shapes to stderr */

typedef struct {
  int B, H, N;      /* batch, heads, tokens per sequence (N >= 1) */
  int d;            /* head dimension: 1..128 */
  int hidden;       /* inner width h (MLP, SwiGLU): 1..512; ignored for LINEAR */
  int dtype;        /* ttt_dtype of q, k, v, o */
  int key_norm;     /* 1: instance-normalise the keys per (b, h, channel) over
                       the N tokens, biased variance, no affine (Test-Time
                       Training vs Sleep page, section "Side one") */
  float eps;        /* added to the key variance inside the square root (>= 0) */
  int renorm;       /* 1: after each update rescale every column of every
                       matrix to the L2 norm that column has in W0 (LaCT page) */
  unsigned flags;   /* TTT_FLAG_* */
  int grid_h, grid_w; /* DWCONV / VIT3: the N tokens form a grid_h x grid_w
                         raster (grid_h * grid_w == N); otherwise ignored */
  int conv_k;       /* DWCONV / VIT3: odd kernel size 1, 3, 5 or 7 */
} ttt_config;

/* Initial fast weights W0, fp32 device memory.  w[i] points at matrix i of
 * the inner model (see ttt_inner; unused entries are ignored).  With
 * batch_stride == 0 each matrix is [H, in, out] and shared by every batch
 * element; otherwise matrix i of batch b starts at w[i] + b * batch_stride
 * elements, e.g. batch_stride = H*in*out when each matrix is its own
 * [B, H, in, out] buffer (all matrices of one model have in*out = d*h, or d*d
 * for LINEAR, so one stride serves them all).  batch_stride must be 0 or
 * >= H*in*out. */
typedef struct {
  const float* w[3];
  long long batch_stride;
} ttt_weights;

/* Optional output of the final fast weights (after the last update), fp32
 * [B, H, in, out] per matrix.  NULL entries (or a NULL struct) are skipped.
 * Passing them back as W0 with batch_stride = H*in*out continues a chunked
 * sequence: a split at a chunk boundary gives the same result as one call
 * (when the re-norm targets are the same, e.g. unit-norm W0 columns). */
typedef struct {
  float* w[3];
} ttt_weights_out;

/* Inner learning rate (ViT3 page, guideline 3; per-token rates: LaCT page):
 * eta_n = scale * (per_token ? per_token[b, h, n] : 1), per_token fp32
 * [B, H, N] device memory or NULL. */
typedef struct {
  float scale;
  const float* per_token;
} ttt_eta;

/* Update rule applied to the eta-weighted gradient G of every update batch
 * (LaCT page, "Nonlinear memory complements local attention": gradient
 * descent, momentum and Muon, the last turning the matrix gradient into an
 * orthogonalised matrix by Newton-Schulz iterations; L2 normalisation, when
 * renorm is on, follows every update):
 *   TTT_RULE_GD      : W <- W - G
 *   TTT_RULE_MOMENTUM: M <- beta M + G,  W <- W - M          (M starts at 0)
 *   TTT_RULE_MUON    : M <- beta M + G,  W <- W - muon_scale NS(M)
 * NS is the quintic Newton-Schulz iteration of the published Muon optimiser:
 * X = M / (||M||_F + 1e-7), then ns_steps times X <- a X + (b A + c A^2) X with
 * A = X X^T and (a, b, c) = (3.4445, -4.7750, 2.0315), on the wide orientation
 * of M (a tall matrix is transposed and back).  Computed in fp32.  The
 * momentum of one call starts at zero (it is not carried across calls). */
typedef enum { TTT_RULE_GD = 0, TTT_RULE_MOMENTUM = 1, TTT_RULE_MUON = 2 } ttt_rule;

/* Order of reads and writes with chunk > 0 (LaCT page, "Order of operations
 * excludes leaking the future"; ViT3 page, section 03 guideline 2):
 *   TTT_ORDER_CAUSAL          : each chunk reads the weights left by the chunks
 *                               before it, then updates them (language, video);
 *                               key_norm is rejected (it would read the future).
 *   TTT_ORDER_WRITE_THEN_QUERY: the chunks update in turn (sequential
 *                               mini-batches), then every query reads the final
 *                               weights (sets of images); key_norm allowed. */
typedef enum { TTT_ORDER_CAUSAL = 0, TTT_ORDER_WRITE_THEN_QUERY = 1 } ttt_order;

/* Per-call options of ttt_forward_ex.  A zero-initialised struct (or a NULL
 * pointer) gives the plain layer: one epoch, every matrix updated, causal
 * order, every chunk writes, gradient descent.
 *   epochs       gradient steps on each update batch (0 or 1: one step; ViT3
 *                page, section 03 guideline 2: several epochs)
 *   update_mask  bit i set: matrix i of the inner model is updated; the others
 *                keep W0 (0: every matrix).  0x1 adjusts only the first layer
 *                (Test-Time Training vs Sleep page, "Side one").
 *   order        ttt_order (used when chunk > 0)
 *   chunk_update HOST array of ceil(N / chunk) flags, or NULL: a chunk whose
 *                flag is 0 only reads (its keys and values are not trained on;
 *                video: clean chunks write, noisy chunks read, LaCT page)
 *   rule, beta, muon_scale, ns_steps: the update rule (ttt_rule); ns_steps 0
 *                means 5; muon_scale must be finite (TTT_RULE_MUON) */
typedef struct {
  int epochs;
  unsigned update_mask;
  int order;
  const unsigned char* chunk_update;
  int rule;
  float beta;
  float muon_scale;
  int ns_steps;
} ttt_options;

typedef struct ttt_handle ttt_handle;

/* Version of this ABI (TTT_ABI_VERSION). */
int ttt_version(void);

/* Validate a configuration and create a handle (host memory only; makes no HIP
 * call).  On error *out is set to NULL and the message is available from
 * ttt_last_error(NULL). */
int ttt_create(const ttt_config* cfg, ttt_handle** out);

/* Bytes of device workspace ttt_forward needs for this handle and this
 * (loss, inner, chunk) request; written to *bytes.  Host-only. */
int ttt_workspace_bytes(const ttt_handle* h, int loss, int inner, int chunk, size_t* bytes);

/* Enqueue the TTT-layer forward pass on `stream`.
 *   q, k, v   [B, H, N, d] inputs (dtype of the config); o [B, H, N, d] output
 *   W0        initial fast weights (fp32), eta learning rates
 *   loss      ttt_loss; inner: ttt_inner
 *   chunk     0: one full-batch step over all N tokens, then every query reads
 *                the updated weights (write-then-query).
 *             C > 0: causal chunks of C tokens (the last may be shorter); chunk c
 *                reads the weights left by chunks 0..c-1, then updates them.
 *                key_norm must be 0 (whole-sequence key statistics would leak
 *                future keys): TTT_ERR_UNSUPPORTED otherwise.
 *   W_out     optional final weights; workspace/ws_bytes: device scratch of at
 *             least ttt_workspace_bytes(...) bytes, 256-byte aligned.
 * q/k/v/o/W0 must not alias o or the workspace.  Returns TTT_OK once the work
 * is enqueued (or, with TTT_FLAG_CHECK_FINITE, once it has finished).
 * Range of the fast path: the GELU-MLP MFMA kernels (bf16 tensors, d = 64)
 * carry the activations, the loss gradient and dZ in f16.  If |V - F(K)|, |V|
 * or a pre-activation exceeds about 4e4, those values overflow and O and the
 * final weights can hold Inf or NaN while the call still returns TTT_OK.
 * Set TTT_FLAG_CHECK_FINITE to have such a result reported as
 * TTT_ERR_NONFINITE, or TTT_FLAG_FORCE_GENERIC to compute it in fp32.
 * Streams: the ViT3 block's head ranges (TTT_INNER_VIT3) are independent and
 * run concurrently, the smaller one on a second stream of the handle (default
 * priority), forked from `stream` by an event and joined back to it before the
 * call returns; that stream and its two events are created on the first such
 * request and released by ttt_destroy.  Every other request runs on `stream`
 * alone. */
int ttt_forward(ttt_handle* h, const void* q, const void* k, const void* v,
                const ttt_weights* W0, const ttt_eta* eta, int loss, int inner, int chunk,
                void* o, const ttt_weights_out* W_out, void* workspace, size_t ws_bytes,
                void* stream);

/* ttt_forward with per-call options (NULL: the plain layer; see ttt_options).
 * The workspace must hold ttt_workspace_bytes_ex(..., opt, ...) bytes. */
int ttt_forward_ex(ttt_handle* h, const void* q, const void* k, const void* v,
                   const ttt_weights* W0, const ttt_eta* eta, int loss, int inner, int chunk,
                   const ttt_options* opt, void* o, const ttt_weights_out* W_out,
                   void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes of a ttt_forward_ex request (opt NULL: the plain layer). */
int ttt_workspace_bytes_ex(const ttt_handle* h, int loss, int inner, int chunk, const ttt_options* opt,
                           size_t* bytes);

/* Kernel family ttt_forward_ex would use; NULL for an invalid request. */
const char* ttt_path_name_ex(const ttt_handle* h, int loss, int inner, int chunk, const ttt_options* opt);

/* Outer-loop backward: the gradients of an outer loss S through the layer,
 * given dO = dS/dO of its output (ViT3 page, section 02: the inner update is
 * differentiable and trained end to end with the outer network, a gradient of
 * a gradient; section 03 guideline 1: the value projection learns through the
 * mixed second derivative of the inner loss).  Full batch (chunk 0), one plain
 * gradient step, no re-norm; inner TTT_INNER_LINEAR or TTT_INNER_MLP_GELU;
 * both losses; key norm on or off.  Other requests: TTT_ERR_UNSUPPORTED.
 *   q, k, v, W0, eta, loss, inner: as for ttt_forward
 *   dO          [B, H, N, d] in the config's dtype
 *   dq, dk, dv  [B, H, N, d] fp32 outputs
 *               (q, k, v, dO, dq, dk, dv 16-byte aligned, else TTT_ERR_INVALID)
 *   dW0         fp32 outputs in W0's layout: [H, in, out] summed over the batch
 *               when W0.batch_stride == 0, else [B, H, in, out]; NULL entries
 *               (or a NULL struct) are skipped
 *   deta        [B, H, N] fp32 output or NULL: the gradient with respect to each
 *               token's effective rate eta_n = scale * per_token[b, h, n]
 *   workspace   at least ttt_backward_workspace_bytes bytes, 256-byte aligned
 * Asynchronous on `stream`, like ttt_forward; arithmetic in fp32. */
int ttt_backward_workspace_bytes(const ttt_handle* h, int loss, int inner, size_t* bytes);
int ttt_backward(ttt_handle* h, const void* q, const void* k, const void* v, const ttt_weights* W0,
                 const ttt_eta* eta, int loss, int inner, const void* dO, float* dq, float* dk, float* dv,
                 const ttt_weights_out* dW0, float* deta, void* workspace, size_t ws_bytes, void* stream);

/* ttt_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Arguments and results are those of ttt_forward, without the workspace: the
 * scratch memory is a fixed array of TTT_NOALLOC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on, from the first call on that GPU until
 * the process ends.  The call allocates and frees nothing.
 *   - A request whose ttt_workspace_bytes exceeds TTT_NOALLOC_SCRATCH_BYTES is
 *     rejected with TTT_ERR_WORKSPACE before anything is enqueued.
 *   - Every call on one GPU shares that GPU's array, and the array keeps the
 *     last call's contents (nothing in it needs to start at zero).  Calls that
 *     overlap on one GPU (two streams, two threads, or two handles without an
 *     ordering between them) race on it: order them on one stream or
 *     synchronise between them.
 *   - The first call on a GPU makes one runtime call to look the array up
 *     (hipGetSymbolAddress); TTT_ERR_HIP if that fails. */
#define TTT_NOALLOC_SCRATCH_BYTES ((size_t)192 << 20)
int ttt_forward_noalloc(ttt_handle* h, const void* q, const void* k, const void* v,
                        const ttt_weights* W0, const ttt_eta* eta, int loss, int inner, int chunk,
                        void* o, const ttt_weights_out* W_out, void* stream);

/* Name of the kernel family ttt_forward would use for this request; NULL for
 * an invalid request.  Host-only.  Names: "mfma" (GELU-MLP bf16 MFMA gradient
 * and readout kernels), "mfma_fused" (the same gradient kernel, every pair held
 * whole by one workgroup, which also applies the step and reads the pair out),
 * "mfma_swiglu" (LaCT SwiGLU kernels), "mfma_glu", "dwconv", "dwconv+mfma_glu"
 * and "dwconv+generic" (ViT3 block), "mfma_f32_grad" and
 * "mfma_f32_grad+mfma_query" (fp32 matrix-core step), "generic_grad+..." and
 * "generic". */
const char* ttt_path_name(const ttt_handle* h, int loss, int inner, int chunk);

/* Measurement hook: with n_events == 8 and events[] holding hipEvent_t
 * handles created by the caller, every later ttt_forward on this handle
 * records events[2k] on its stream right before and events[2k+1] right after
 * kernel family k: 0 key statistics, 1 gradient of the first update batch,
 * 2 weight update of the first batch, 3 readout.  A family that does not run
 * (no key norm) records both of its events back to back.  A NULL entry is
 * skipped (each recorded event adds a little time between kernels, so a
 * caller timing one family passes only its two events).  events == NULL or
 * n_events == 0 switches the hook off.  The events are not owned by the
 * library.  Host-only; returns TTT_ERR_INVALID for any other n_events. */
int ttt_set_timing_events(ttt_handle* h, void* const* events, int n_events);

/* Release a handle (NULL is a no-op). */
int ttt_destroy(ttt_handle* h);

/* Message of the last failure on this handle (or of the last ttt_create when h
 * is NULL); never NULL, "" when there was none. */
const char* ttt_last_error(const ttt_handle* h);

/* Static description of a status code. */
const char* ttt_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* TTT_H_ */
