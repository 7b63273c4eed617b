/*
 * gla.h -- C ABI of libgla, the MI355X (gfx950) Simple GLA mixer library.
 *
 * The method is the "GLA mixer" of the Laplace 3B post (AWS ML blog "Beyond the
 * KV cache: training and serving i14's Laplace 3B linear attention model on
 * AWS Trainium2 with native PyTorch"), section "i14 and the Laplace 3B
 * architecture", paragraph "GLA mixer".  Per head h, with a fixed decay
 * lambda_h shared by all sequences, a dk x dv matrix state evolves per token as
 *       S_t = lambda_h * S_{t-1} + k_t v_t^T          (rank-1 write)
 *       o_t = scale * S_t^T q_t                       (readout after the write)
 * `scale` multiplies the readout only; the state never depends on it.
 *
 * Conventions shared by every call
 * --------------------------------
 * - All tensor pointers are DEVICE pointers (HIP global memory on the current
 *   device); `stream` is a hipStream_t passed as void* (NULL = default stream).
 *   Sizes are host ints.  The library never allocates or frees device memory:
 *   the caller owns every buffer, including the workspace.
 * - Layouts are row-major, last index fastest:
 *     q, k  [B][T][H][dk]     v, o  [B][T][H][dv]      (token-major, as the fused
 *                                                        QKVG projection emits them)
 *     S0, S_final, dS_T, dS0   [B][H][dk][dv] fp32, dense
 *     lambda, dlambda          [H] fp32
 *   The token-major tensors of the chunked forward and backward may be strided
 *   views (gla_strides below): the paragraph "QKVG projection" of the same
 *   section has q, k, v and the output gate g come out of one fused projection
 *   of width H (2 dk + 2 dv) = 9,216, so they can be read in place from it.
 * - dtype selects the element type of q, k, v, o, do, dq, dk, dv: GLA_F32 (fp32)
 *   or GLA_BF16 (bfloat16).  States, lambda and every accumulation are fp32.
 *   bf16 outputs are rounded to nearest even.
 * - Supported shapes (instantiated kernels), (dk, dv, chunk):
 *     bf16: (96, 192, 256), (96, 192, 128), (96, 192, 64), (96, 192, 32);
 *     fp32: (96, 192, 64) forward only, (16, 32, 32);
 *     decode, either dtype: (dk, dv) = (96, 192) or (16, 32).
 *   Anything else returns GLA_ERR_UNSUPPORTED, and so does a chunked forward
 *   or backward with B*H above 65,535 (the units take one 16-bit grid
 *   dimension; a larger batch is split by the caller).  T need not be a
 *   multiple of chunk (the last chunk is partial).
 * - Validation is host-only and finishes before any HIP call: on any error
 *   nothing is enqueued and no output is touched.  Pointers must be 16-byte
 *   aligned.  Every computing entry point returns a gla_status.  lambda in
 *   [0, 1] is a precondition (device data is not read on the host).  Outputs
 *   must not alias inputs (decode's S is in/out by design).
 * - Calls are asynchronous: GLA_OK means "validated and enqueued on `stream`".
 *   GLA_ERR_DEVICE reports a launch failure; device faults surface at the
 *   caller's next synchronisation.  Results are deterministic (no float
 *   atomics): the same inputs and sizes give the same bits, and a sequence's
 *   bits do not depend on its position in the batch.  (The forward's launch
 *   plan depends on B*H and T, so changing B may change rounding, not results
 *   beyond it; decode is independent of N.)
 * - No exception or abort crosses this ABI.  Calls are thread-safe.
 */
#ifndef GLA_H
#define GLA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GLA_OK = 0,
    GLA_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, negative size, ... */
    GLA_ERR_UNSUPPORTED = 2,   /* no kernel instantiated for (dtype, dk, dv, chunk) */
    GLA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than *_workspace_bytes */
    GLA_ERR_DEVICE = 4         /* a HIP launch or query failed */
} gla_status;

typedef enum { GLA_F32 = 0, GLA_BF16 = 1 } gla_dtype;

/*
 * Element strides of one token-major tensor [B][T][H][d] whose head and
 * feature dimensions are packed (head h of token t of sequence b starts at
 * b * batch + t * token + h * d).  A zero field takes the packed value:
 * token = H * d, batch = T * token.  Rules (else GLA_ERR_INVALID_ARG):
 * strides >= 0 and multiples of 16 bytes; H * d <= token < 2^22; for an
 * output with B > 1, batch >= (T - 1) * token + H * d (its sequences do not
 * overlap).  Example, the fused projection output X [B][T][H (2dk + 2dv)]:
 * q = X, k = X + H dk, v = X + 2 H dk, g = X + 2 H dk + H dv, each with
 * token = H (2dk + 2dv) and batch = T * token.
 */
typedef struct {
    long long batch;
    long long token;
} gla_stride;

/* Strides of every token-major tensor of the chunked calls; a call reads only
 * the entries of the tensors it takes (o holds y for the epilogue forward).
 * A NULL gla_strides pointer means every tensor is packed. */
typedef struct {
    gla_stride q, k, v, o, d_o, dq, dk, dv, g;
} gla_strides;

/* Version of this ABI (bumped on any signature or semantic change). */
int gla_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* gla_status_str(gla_status status);

/*
 * Workspace needed by gla_fwd_chunked for these sizes, in bytes (0 if none).
 * The launch plan assumes the 256 compute units of gfx950 parts, so the size
 * depends only on the arguments (no device query).
 * Returns 0 as well for unsupported or invalid sizes; the call then reports it.
 */
size_t gla_fwd_workspace_bytes(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk);

/*
 * Chunked-parallel forward (Laplace 3B post, section "Challenge 1": per chunk
 * of `chunk` tokens, a decay-masked causal linear attention inside the chunk
 * plus the running state's contribution; the state then advances by the decay
 * compounded over the chunk).  Equal, up to rounding, to the per-token
 * recurrence above run from S0.
 *   q, k, v     inputs (dtype), layouts above
 *   lambda      [H] fp32 per-head decay
 *   S0          optional initial state (NULL = zero)
 *   scale       readout scale
 *   o           output [B][T][H][dv] (dtype)
 *   S_final     optional output: state after token T-1 (NULL = not written);
 *               with T == 0 it receives S0 (or zeros)
 *   st          optional strides of q, k, v, o (NULL = packed)
 *   ws, ws_bytes  caller-owned device workspace, at least
 *               gla_fwd_workspace_bytes(...) bytes (may be NULL when that is 0)
 */
gla_status gla_fwd_chunked(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk,
                           const void* q, const void* k, const void* v,
                           const float* lambda, const float* S0, float scale,
                           void* o, float* S_final, const gla_strides* st,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * gla_fwd_chunked for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  It
 * takes no workspace argument and calls no allocating routine: the workspace
 * is a fixed GLA_NOALLOC_WORKSPACE_MAX-byte device array inside the library,
 * one per GPU, held until the process ends.  Sizes whose
 * gla_fwd_workspace_bytes exceeds that limit return GLA_ERR_WORKSPACE (before
 * any HIP call); that admits, among others, the Laplace layer (B=1, T=2,048:
 * 9.4 MB), the training width (B=8, T=2,048: 28.3 MB) and the 64k-token
 * prefill (B=1, T=65,536: 26.5 MB).  All calls on one GPU share the array:
 * calls that overlap in time on one GPU (two streams, two threads) race and
 * give wrong results; calls ordered on one stream are safe.  The array keeps
 * the last call's contents; the forward writes every workspace byte it reads
 * before reading it, so nothing needs clearing.  Results equal
 * gla_fwd_chunked's bit for bit.  GLA_ERR_DEVICE if the array's address cannot
 * be found on the current device.
 */
#define GLA_NOALLOC_WORKSPACE_MAX (32u << 20)

gla_status gla_fwd_chunked_noalloc(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk,
                                   const void* q, const void* k, const void* v,
                                   const float* lambda, const float* S0, float scale,
                                   void* o, float* S_final, const gla_strides* st, void* stream);

/*
 * Workspace needed by gla_bwd_chunked (bytes; 0 for unsupported/invalid sizes).
 * Holds the per-chunk state snapshots (2 * B*H*ceil(T/chunk)*dk*dv elements of
 * the input dtype), segment states and the dlambda partials.
 */
size_t gla_bwd_workspace_bytes(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk);

/*
 * Chunked backward: gradients of a scalar loss L given do = dL/do and the
 * optional dS_final = dL/dS_final, through the forward defined above (Laplace
 * 3B post, section "Challenge 3": the backward differentiates through the
 * sequential chunk-to-chunk state chain, run here in reverse chunk order).
 * Supported shapes: bf16 (96, 192, 128), (96, 192, 64), (96, 192, 32); fp32 (16, 32, 32).
 *   q, k, v, lambda, S0, scale, chunk   as in gla_fwd_chunked (S0 nullable)
 *   d_o        [B][T][H][dv] (dtype) upstream gradient of o
 *   dS_final   [B][H][dk][dv] fp32 upstream gradient of S_final (NULL = 0)
 *   dq, dk_out [B][T][H][dk] (dtype) outputs;  dv_out [B][T][H][dv] (dtype) output
 *   dlambda    [H] fp32 output, summed over the batch (NULL = not computed)
 *   dS0        [B][H][dk][dv] fp32 output, gradient of the initial state (NULL = skip)
 *   st         optional strides of q, k, v, d_o, dq, dk, dv (NULL = packed)
 *   ws, ws_bytes  caller-owned workspace of at least gla_bwd_workspace_bytes(...)
 * With T == 0: dS0 = dS_final (or 0) and dlambda = 0.
 */
gla_status gla_bwd_chunked(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk,
                           const void* q, const void* k, const void* v,
                           const float* lambda, const float* S0, float scale,
                           const void* d_o, const float* dS_final,
                           void* dq, void* dk_out, void* dv_out,
                           float* dlambda, float* dS0, const gla_strides* st,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * Training pair: a forward that also saves the state entering every chunk, and
 * a backward that reads those states instead of re-running the forward state
 * chain (Laplace 3B post, section "Challenge 3": the backward walks the chunk
 * chain; its forward half is exactly what the forward already computed).
 *   states  [B][H][ceil(T/chunk)][dk][dv] in the dtype of q (bf16 or fp32):
 *           states[b][h][c] = the state before chunk c (S0 or 0 for c = 0),
 *           rounded to the dtype; gla_fwd_states_bytes gives its size.
 * gla_fwd_chunked_states: as gla_fwd_chunked, plus `states` (written).  Only for
 * shapes gla_bwd_chunked supports (else GLA_ERR_UNSUPPORTED); same workspace
 * (gla_fwd_workspace_bytes).
 * gla_bwd_chunked_states: as gla_bwd_chunked, plus `states` (read), which must
 * come from gla_fwd_chunked_states over the same q, k, v, lambda, S0 and sizes.
 * Its workspace, gla_bwd_states_workspace_bytes, holds no state snapshots
 * (about half of gla_bwd_workspace_bytes).  The gradients agree with
 * gla_bwd_chunked's within rounding (the saved states are rounded as the
 * backward's own are, from a differently ordered but equal fp32 recurrence).
 */
size_t gla_fwd_states_bytes(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk);

gla_status gla_fwd_chunked_states(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk,
                                  const void* q, const void* k, const void* v,
                                  const float* lambda, const float* S0, float scale,
                                  void* o, float* S_final, void* states, const gla_strides* st,
                                  void* ws, size_t ws_bytes, void* stream);

size_t gla_bwd_states_workspace_bytes(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk);

gla_status gla_bwd_chunked_states(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk,
                                  const void* q, const void* k, const void* v,
                                  const float* lambda, const float* S0, float scale,
                                  const void* d_o, const float* dS_final, const void* states,
                                  void* dq, void* dk_out, void* dv_out,
                                  float* dlambda, float* dS0, const gla_strides* st,
                                  void* ws, size_t ws_bytes, void* stream);

/*
 * Batched single-token decode step (Laplace 3B post, section "Optimizing
 * inference on Trainium2": one fixed state page per sequence, read and written
 * once per generated token).  For every sequence n and head h, in place:
 *       S[n,h] <- lambda_h S[n,h] + k[n,h] v[n,h]^T ;  o[n,h] = scale S[n,h]^T q[n,h]
 *   q, k   [N][H][dk] (dtype)      v, o  [N][H][dv] (dtype)
 *   S      [N][H][dk][dv] fp32, updated in place (the sequence's state page)
 * No workspace.  One kernel launch per call.
 */
gla_status gla_decode_step(gla_dtype dtype, int N, int H, int dk, int dv,
                           const void* q, const void* k, const void* v,
                           const float* lambda, float* S, float scale, void* o,
                           void* stream);

/*
 * The same decode step on a pool of state pages (Laplace 3B post, section
 * "Optimizing inference on Trainium2": the serving stack gives every sequence
 * one fixed state page, and decode batches are padded to fixed widths).
 *   pool   [P][H][dk][dv] fp32, one page per sequence slot, updated in place
 *   slots  [N] int32 (device): row n of q, k, v, o uses page slots[n].  A slot
 *          outside [0, P) -- use -1 for a padding row -- touches no page and
 *          gives a zero output row.  Two rows of one call must not share a
 *          page (they would race).
 *   q, k, v, o, lambda, scale   as in gla_decode_step
 * Each (row, head) is computed on its own: a sequence's outputs and page are
 * bit-identical whatever batch, position or padding it is decoded in.  A
 * prefill hands over by passing a page range of the pool as gla_fwd_chunked's
 * S_final (batch element b -> page first + b).
 * Errors: as gla_decode_step; P < 0 or a NULL slots pointer -> GLA_ERR_INVALID_ARG.
 * No workspace.  One kernel launch per call.
 */
gla_status gla_decode_step_pool(gla_dtype dtype, int N, int H, int dk, int dv,
                                const void* q, const void* k, const void* v,
                                const float* lambda, float* pool, int P, const int* slots,
                                float scale, void* o, void* stream);

/*
 * Mixer epilogue (Laplace 3B post, section "i14 and the Laplace 3B
 * architecture", paragraph "GLA mixer", the sentences after the readout): a
 * value copy gated by a self-augmentation sigmoid, a head RMSNorm shared by the
 * heads of one decay tier, and a SiLU output gate.  For every row m and head h:
 *       s = sigmoid( q[m,h] . (aug_a[h] (.) k[m,h]) )
 *       x = o[m,h] + s * v[m,h]
 *       y[m,h] = silu(g[m,h]) (.) x / sqrt(mean_j x_j^2 + eps) (.) norm_w[head_tier[h]]
 * q and k enter unscaled (the readout's scale is already inside o).  With
 * aug_a == NULL the gate is sigmoid(0) = 1/2: a half-strength value skip.
 * The head concatenation is the [..][H][dv] layout itself.
 */
#define GLA_EPI_MAX_HEADS 64

typedef struct {
    const float* aug_a;      /* [H][dk] fp32 device, self-augmentation vectors; NULL = 0 */
    const float* norm_w;     /* [n_tiers][dv] fp32 device, RMSNorm weight of each tier */
    const int* head_tier;    /* [H] int32 HOST array: the tier of head h, in [0, n_tiers);
                                read during the call only */
    int n_tiers;             /* 1 .. 64 */
    float eps;               /* >= 0, finite; added to the mean square */
} gla_epilogue_params;

/*
 *   q, k       [M][H][dk] (dtype)        the mixer inputs of the rows
 *   v, o, g    [M][H][dv] (dtype)        values, the readout, the output-gate logits
 *   y          [M][H][dv] (dtype)        output; may alias o (each element of o
 *                                         is read before y's element is written)
 * M = B * T for a prefill (token rows), N for a decode batch.  H <= 64.
 * Supported (dk, dv): (96, 192), (16, 32).  One kernel launch, no workspace.
 * Errors: NULL ep, a NULL/misaligned tensor, n_tiers outside [1, 64], a head_tier entry
 * out of range, a negative or non-finite eps, M < 0 -> GLA_ERR_INVALID_ARG;
 * H > 64 or another (dk, dv) -> GLA_ERR_UNSUPPORTED.  M == 0 enqueues nothing.
 */
gla_status gla_mixer_epilogue(gla_dtype dtype, int M, int H, int dk, int dv,
                              const void* q, const void* k, const void* v,
                              const void* o, const void* g,
                              const gla_epilogue_params* ep, void* y, void* stream);

/*
 * The forward (gla_fwd_chunked) followed by the epilogue above, with y in place
 * of o: y[b,t,h] = epilogue(q, k, v, o, g)[b,t,h] for the readout o the forward
 * defines (o itself is not stored).  For bf16 plans that run the tiled state
 * chain (128-token chunks, B*H <= 16 and at most 16 chunks, as at B = 1, H = 16,
 * T = 2,048) the epilogue is
 * applied in the output kernel's store, on the fp32 readout; other plans run the
 * forward into y and the epilogue pass over y in place.
 *   g      [B][T][H][dv] (dtype) output-gate logits;   y  [B][T][H][dv] (dtype) output
 *   st     optional strides of q, k, v, g and of y (the `o` entry); NULL = packed
 *   ws     as gla_fwd_chunked (gla_fwd_workspace_bytes of the same sizes)
 *   others as gla_fwd_chunked and gla_mixer_epilogue; the errors of both.
 */
gla_status gla_fwd_chunked_epilogue(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk,
                                    const void* q, const void* k, const void* v,
                                    const float* lambda, const float* S0, float scale,
                                    const void* g, const gla_epilogue_params* ep, void* y,
                                    float* S_final, const gla_strides* st,
                                    void* ws, size_t ws_bytes, void* stream);

/*
 * Decode step with the epilogue fused into it: the state update and readout of
 * gla_decode_step (slots == NULL, S holds N pages [N][H][dk][dv]) or of
 * gla_decode_step_pool (slots != NULL, S is a pool of P pages), then the
 * epilogue above on the readout; only y is written (the readout o is never
 * stored).  A padding row (slot outside [0, P)) gives a zero y row.
 *   g   [N][H][dv] (dtype) output-gate logits;  y  [N][H][dv] (dtype) output
 * Other arguments and errors: as gla_decode_step(_pool) and gla_mixer_epilogue
 * (P is ignored when slots == NULL).  One kernel launch, no workspace.
 */
gla_status gla_decode_step_epilogue(gla_dtype dtype, int N, int H, int dk, int dv,
                                    const void* q, const void* k, const void* v, const void* g,
                                    const float* lambda, float* S, int P, const int* slots,
                                    float scale, const gla_epilogue_params* ep, void* y,
                                    void* stream);

/*
 * Depth-wise causal convolution of width K = 4 with SiLU, the step before the
 * mixer (Laplace 3B post, section "i14 and the Laplace 3B architecture",
 * paragraph "Normalization and convolution"; the "Conv" row of the parameter
 * table).  Every channel d is filtered on its own:
 *       u_t[d] = bias[d] + sum_{j<K} w[d][j] * x_{t-(K-1)+j}[d],    y_t[d] = silu(u_t[d])
 * (w[d][K-1] weighs the current token), with inputs before the first token
 * taken from a per-sequence window of the K most recent earlier inputs.
 *   x, y      [B][T][D] (dtype)
 *   w         [D][K] fp32;   bias  [D] fp32 or NULL (no bias)
 *   win_in    [B][K][D] fp32: win_in[b][s] = x_{s-K} (oldest first); NULL = zeros
 *   win_out   [B][K][D] fp32 or NULL: the window after the last token,
 *             x_{T-K..T-1} (the decode carry); may alias win_in (in place)
 * Supported: K == 4, D a multiple of 8 (D <= 2^20).  T == 0 passes the window
 * through.  One kernel launch, no workspace.
 * Errors: a NULL/misaligned required pointer, negative sizes -> GLA_ERR_INVALID_ARG;
 * another K or D, B > 65,535 or T > 2,097,120 -> GLA_ERR_UNSUPPORTED.
 */
gla_status gla_conv1d_silu(gla_dtype dtype, int B, int T, int D, int K,
                           const void* x, const float* w, const float* bias,
                           const float* win_in, void* y, float* win_out, void* stream);

/*
 * One decode token per sequence through the same convolution: the window of
 * row n drops its oldest input and appends x[n], then y[n] = silu(bias + w . window).
 *   x, y   [N][D] (dtype)
 *   win    fp32, updated in place: [N][K][D] (slots == NULL), or a pool of P
 *          windows [P][K][D] with row n using window slots[n] (device int32 [N]);
 *          a slot outside [0, P) is a padding row: zero output, no window touched.
 * Each row is computed on its own (bit-identical whatever batch it is in).
 * Errors and support: as gla_conv1d_silu (N in place of B); P < 0 with slots ->
 * GLA_ERR_INVALID_ARG.
 */
gla_status gla_conv1d_silu_decode(gla_dtype dtype, int N, int D, int K,
                                  const void* x, const float* w, const float* bias,
                                  float* win, int P, const int* slots, void* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GLA_H */
