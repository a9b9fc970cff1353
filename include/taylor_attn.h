/*
 * taylor_attn.h -- C ABI of the Taylor-truncated causal attention library (gfx950 / MI355X).
 *
 * The method ("Expanding Attention: A Taylor-Series Route to Linear-Time
 * Transformers with a Fixed Number of Recurrent States", Z. Huang,
 * arXiv:2610.20637, Abstract): the attention kernel exp(s), s = scale * q.k,
 * is replaced by its Taylor polynomial of n terms,
 *
 *     K_n(s) = sum_{m=0}^{n-1} s^m / m!,
 *
 * each term is factorised as an inner product of symmetric tensor powers,
 * s^m/m! = <phi_m(scale*q), phi_m(k)>, with binom(d_k+m-1, m) monomial features
 * phi_m(x)_alpha = x^alpha / sqrt(alpha!), and the causal history collapses into
 * n fixed-size recurrent states
 *
 *     S_m = sum_j phi_m(k_j) v_j^T      (W_m x d_v)
 *     z_m = sum_j phi_m(k_j)            (W_m)
 *
 * read out as  o_i = sum_m phi_m(scale*q_i)^T S_m / sum_m phi_m(scale*q_i)^T z_m
 * (inclusive causality: token i sees keys 0..i).  Decoding updates the states
 * with one rank-one outer product per token; states add across chunks, so
 * prefill is a chunked computation plus a prefix scan of chunk states.
 *
 * Conventions for every entry point
 * ---------------------------------
 * - All tensors are dense row-major.  q, k: [B, H, N, d_k]; v: [B, H, N, d_v]
 *   (decode: N = 1 and the token axis is dropped); o: [B, H, N, d_v] float32.
 * - q, k, v have element type cfg->in_dtype (float32 or bfloat16); outputs,
 *   states and all accumulation are float32.
 * - Device pointers are owned by the caller.  The library never allocates,
 *   frees or synchronises; every call only enqueues kernels on `stream`
 *   (0 = the null stream) and returns at once.  Pointers must be 16-byte
 *   aligned device addresses.
 * - Every call returns a taylor_status (0 = TAYLOR_OK, negative = error).
 *   Arguments are validated before anything is enqueued; on an error return
 *   nothing has been enqueued (TAYLOR_ERR_HIP: a launch failed; earlier
 *   kernels of the same call may already be queued).  No C++ exception crosses
 *   this boundary.  Calls are re-entrant; the only global state is the
 *   address of taylor_attn_prefill_into_static's workspace on each device and
 *   a process-wide counter that tags the single-pass prefill's flags per call
 *   (so a workspace's prior contents never read as this call's).
 *
 * State layout (per head, float32): the "packed" block of
 * W*(d_v+1) values the Abstract counts (9,945 at n=3, d_k=16, d_v=64),
 * stored as
 *     S   : [W][d_v]  row-major, feature-major rows, rows ordered as the
 *                     monomial table below (orders ascending, lexicographic
 *                     coordinate tuples within an order);
 *     z   : [W]       the normaliser column (the "+1" column of [v | 1]);
 *     pad : zeros up to taylor_state_stride() floats (a multiple of 4, so every
 *           head block and every S row starts 16-byte aligned).
 * A state buffer is [B][H][stride] floats.
 */
#ifndef TAYLOR_ATTN_H
#define TAYLOR_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TAYLOR_OK = 0,
  TAYLOR_ERR_INVALID_ARG = -1, /* bad pointer, size, alignment or config value */
  TAYLOR_ERR_UNSUPPORTED = -2, /* valid config with no compiled kernel (see taylor_supported) */
  TAYLOR_ERR_HIP = -3          /* the HIP runtime reported an error on launch */
} taylor_status;

typedef enum { TAYLOR_F32 = 0, TAYLOR_BF16 = 1 } taylor_dtype;

/* How the states are read out.
 *   TAYLOR_READOUT_KERNEL   (0): the truncated exp kernel, normalised -- the
 *       method above (Abstract of "Expanding Attention").
 *   TAYLOR_READOUT_CENTERED (1): softmax expanded about the mean score (Su
 *       Jianlin, kexue.fm translation 11814, "Calculating the Gradient" and
 *       "Linear Attention"), truncated at order n_terms - 1 (1 or 2).  Token i
 *       weights key j <= i by, with x_j = scale * q_i.k_j, y_j = x_j - mean(x)
 *       over the i+1 keys, p_j = (1 + y_j)/(i+1) at order 1 and
 *       (1 + y_j + (y_j^2 - mean(y^2))/2)/(i+1) at order 2, and outputs
 *       o_i = sum_j p_j v_j (the weights sum to one and may be negative).  It
 *       reads the same states (S, z of n_terms terms: counts, sums of k, of
 *       phi_2(k) and their products with v), so a state written under one
 *       readout continues under the other.  Compiled for n_terms = 2, 3 at
 *       d_k = 16, d_v = 64. */
typedef enum { TAYLOR_READOUT_KERNEL = 0, TAYLOR_READOUT_CENTERED = 1 } taylor_readout;

typedef struct {
  int n_terms;  /* n: Taylor terms, orders 0..n-1 (1..5 compiled)                         */
  int d_k;      /* q/k head dimension (4, 8 or 16 compiled)                                */
  int d_v;      /* v head dimension (multiple of 4; 4, 16, 32, 64, 128 compiled)           */
  int chunk;    /* requested prefill chunk length C: 0 (default), 64 or 128.  Only the      *
                 * portable float32 kernels (d_k = 4, 8) walk C-token chunks; the matrix-  *
                 * core kernels (d_k = 16, d_v = 64) walk a fixed length whatever C is:   *
                 * 64 tokens (bfloat16 inputs at n <= 3), else 32 (float32 inputs,     *
                 * and n = 4, 5).                                                      *
                 * Outputs depend on the chunk length only through float32 rounding     *
                 * (states add across chunks).  taylor_prefill_chunk() reports it.       */
  float scale;  /* score scale sigma: s = scale * q.k                                      */
  int in_dtype; /* taylor_dtype of q, k, v                                                 */
  int readout;  /* taylor_readout (0 = the truncated kernel)                               */
} taylor_config;

/* Human-readable name of a taylor_status; never NULL. */
const char* taylor_status_string(int status);

/* Feature width W = sum_{m<n} binom(d_k+m-1, m) (Abstract: the m-th state is
 * binom(d+m-1, m) wide), e.g. 153 at n=3, d_k=16.  Host only.
 * Returns TAYLOR_ERR_INVALID_ARG if n_terms < 1, d_k < 1 or W would exceed 2^31-1. */
int taylor_feature_width(int n_terms, int d_k);

/* Logical state size per head, W*(d_v+1) floats (9,945 at n=3, d_k=16, d_v=64).
 * Host only.  Negative taylor_status if cfg is invalid. */
int64_t taylor_state_elems(const taylor_config* cfg);

/* Floats between consecutive head blocks of a state buffer: W*(d_v+1) rounded
 * up to a multiple of 4.  Host only.  Negative taylor_status if cfg is invalid. */
int64_t taylor_state_stride(const taylor_config* cfg);

/* Export the monomial table the kernels use (host only, bit-exact).  The
 * Abstract of "Expanding Attention" gives each Taylor term as an inner product
 * of tensor powers whose m-th state is binom(d+m-1, m) wide: the distinct
 * monomials of degree m in d coordinates, one per multiset of coordinates.  The
 * table lists them with the coefficient that splits the term's multiplicity
 * and 1/m! evenly between query and key:
 *   idx_out  [W][max(n-1,1)] int32: coordinates i_1 <= ... <= i_m of each
 *            feature, -1 padded (row 0, the constant feature, is all -1);
 *   coef_out [W] double: 1/sqrt(alpha!) with alpha the exponent vector, computed
 *            as 1.0/sqrt((double)prod_i alpha_i!).
 * Rows follow the feature order: orders m = 0..n-1 ascending, lexicographic
 * within an order.  Either output pointer may be NULL.  `cap_rows` is the
 * capacity of the outputs in rows.  Returns W, or TAYLOR_ERR_INVALID_ARG for a
 * bad (n, d_k) or cap_rows < W (nothing written then). */
int taylor_monomial_table(int n_terms, int d_k, int32_t* idx_out, double* coef_out, size_t cap_rows);

/* TAYLOR_OK if kernels are compiled for this config (n_terms, d_k, d_v, chunk,
 * in_dtype, readout); TAYLOR_ERR_UNSUPPORTED if valid but not compiled;
 * TAYLOR_ERR_INVALID_ARG if invalid.  Host only. */
int taylor_supported(const taylor_config* cfg);

/* The chunk length, in tokens, that the prefill kernels walk for this config
 * (64 or 32 on the matrix-core kernels whatever cfg->chunk says; cfg->chunk, or
 * 64 for 0, on the portable ones).  The Abstract of "Expanding Attention" fixes
 * no chunk length: the states add across chunks, so any length gives the same
 * result up to rounding.  Host only.  Negative taylor_status if cfg is invalid
 * or not compiled (taylor_supported). */
int taylor_prefill_chunk(const taylor_config* cfg);

/* Bytes of device workspace taylor_attn_prefill needs for these sizes (may be 0).
 * Host only.  Negative taylor_status if cfg or sizes are invalid. */
int64_t taylor_prefill_workspace_bytes(const taylor_config* cfg, int B, int H, int N);

/* Zero B*H state blocks (S, z and padding) -- an empty history (Abstract: the
 * states are sums over the causal history).  `state` is [B][H][stride] floats.
 * B*H == 0 is a no-op. */
int taylor_state_init(float* state, int B, int H, const taylor_config* cfg, hipStream_t stream);

/* Chunked causal prefill over N tokens (Abstract: states add across chunks,
 * so prefill is chunk-local work plus a prefix scan of chunk states).
 *   q, k, v   : [B,H,N,d_k], [B,H,N,d_k], [B,H,N,d_v] in cfg->in_dtype;
 *   o         : [B,H,N,d_v] float32 outputs, or NULL for a state-only pass;
 *   state     : [B,H,stride] float32, in/out.  On entry the state of the
 *               tokens before this call (zero = empty history); on return the
 *               state including these N tokens, so prefill(N1) followed by
 *               prefill(N2) equals prefill(N1+N2).  NULL: start from an empty
 *               history and discard the final state.  At least one of o and
 *               state must be non-NULL;
 *   workspace : device buffer of taylor_prefill_workspace_bytes(cfg, B, H, N)
 *               bytes (NULL allowed when that is 0); its contents on entry are
 *               ignored and on return undefined.
 * N == 0 or B*H == 0 is a no-op.  Calls sharing a workspace must not overlap. */
int taylor_attn_prefill(const void* q, const void* k, const void* v, float* o, float* state, void* workspace, int B,
                        int H, int N, const taylor_config* cfg, hipStream_t stream);

/* taylor_attn_prefill with the incoming and the final state in separate arrays
 * (Abstract: the state after the call is the state before it plus the sum over
 * the call's tokens, so where each lives is free).
 *   state_in  : [B,H,stride] float32, read only: the state of the tokens before
 *               this call; NULL = an empty history (no zeroed array needed);
 *   state_out : [B,H,stride] float32, written: the state including these N
 *               tokens; NULL = discarded.  At least one of o and state_out must
 *               be non-NULL.  state_out may be state_in (in place, as
 *               taylor_attn_prefill) or an array that does not overlap it
 *               (TAYLOR_ERR_INVALID_ARG otherwise); out of place it serves
 *               e.g. continuing a cached prefix state without overwriting it;
 *   q, k, v, o, workspace, B, H, N, cfg: as taylor_attn_prefill (the same
 *               workspace size).
 * N == 0 copies state_in to state_out (zero when state_in is NULL).  B*H == 0
 * is a no-op. */
int taylor_attn_prefill_into(const void* q, const void* k, const void* v, float* o, const float* state_in,
                             float* state_out, void* workspace, int B, int H, int N, const taylor_config* cfg,
                             hipStream_t stream);

/* Size of the static device workspace of taylor_attn_prefill_into_static, per GPU. */
#define TAYLOR_STATIC_WORKSPACE_BYTES (32u << 20)

/* taylor_attn_prefill_into with no workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace is a static device array of
 * TAYLOR_STATIC_WORKSPACE_BYTES (32 MiB) inside the library, one per GPU, held
 * from the first call on that GPU until the process ends; the call itself
 * allocates nothing.  The current device must be the stream's.  Sizes whose
 * workspace (taylor_prefill_workspace_bytes) exceeds that size return
 * TAYLOR_ERR_INVALID_ARG before anything is enqueued (at n = 3, d_k = 16,
 * d_v = 64 up to 843 (sequence, head) pairs of any length fit; float32 inputs at
 * n = 4, 5 need far more).  Every call on one GPU shares that GPU's array: calls that overlap in
 * time on one GPU (other streams, other host threads) race and give undefined
 * results; calls ordered on one stream are safe.  Nothing in the array needs to
 * start at zero (every value read is written earlier in the same call).  Other
 * arguments, results and errors as taylor_attn_prefill_into. */
int taylor_attn_prefill_into_static(const void* q, const void* k, const void* v, float* o, const float* state_in,
                                    float* state_out, int B, int H, int N, const taylor_config* cfg,
                                    hipStream_t stream);

/* Bytes of device workspace taylor_attn_prefill_varlen needs for these sizes
 * (may be 0); it depends on the sizes only, not on the individual lengths.
 * Host only.  Negative taylor_status if cfg or sizes are invalid;
 * TAYLOR_ERR_UNSUPPORTED for a config without a ragged-batch kernel (below). */
int64_t taylor_prefill_varlen_workspace_bytes(const taylor_config* cfg, int n_seqs, int H, int max_seqlen,
                                              int64_t total_tokens);

/* Causal prefill of a ragged batch: n_seqs sequences of different lengths, each
 * its own causal history (Abstract: the states sum over a sequence's past; they
 * are kept per sequence), packed back to back along the token axis.
 *   q, k       : [H][T][d_k] in cfg->in_dtype, T = total_tokens; sequence b
 *                occupies tokens cu_seqlens[b] .. cu_seqlens[b+1]-1 of every head;
 *   v          : [H][T][d_v] in cfg->in_dtype;
 *   o          : [H][T][d_v] float32, or NULL for a state-only pass;
 *   state      : [n_seqs][H][stride] float32, in/out as in taylor_attn_prefill
 *                (NULL: empty histories, final states discarded).  At least one
 *                of o and state must be non-NULL;
 *   cu_seqlens : DEVICE array of n_seqs+1 int32 offsets (4-byte aligned), read
 *                by the kernels only: 0 = cu[0] <= cu[1] <= ... <= cu[n_seqs] = T
 *                and every length cu[b+1]-cu[b] <= max_seqlen.  Violations are not
 *                detected: the kernels clamp every offset into [0, T], so no access
 *                leaves the buffers, but outputs and states are then undefined;
 *   workspace  : taylor_prefill_varlen_workspace_bytes(cfg, n_seqs, H,
 *                max_seqlen, T) bytes (NULL allowed when 0); contents on entry
 *                ignored, on return undefined.
 * Each sequence gives, up to float32 summation order, the outputs and final
 * state that taylor_attn_prefill with B = 1 gives on it alone; an empty
 * sequence leaves its state unchanged.  Compiled for d_k = 16, d_v = 64 (the
 * matrix-core kernels, n = 1..5, both input types); other configs return
 * TAYLOR_ERR_UNSUPPORTED.  T > n_seqs * max_seqlen or negative sizes:
 * TAYLOR_ERR_INVALID_ARG.  n_seqs*H == 0 or T == 0 is a no-op.  Calls sharing a
 * workspace must not overlap. */
int taylor_attn_prefill_varlen(const void* q, const void* k, const void* v, float* o, float* state, void* workspace,
                               const int32_t* cu_seqlens, int n_seqs, int H, int max_seqlen, int64_t total_tokens,
                               const taylor_config* cfg, hipStream_t stream);

/* taylor_attn_prefill_varlen with the incoming and the final states in separate
 * arrays, as taylor_attn_prefill_into: state_in [n_seqs][H][stride] read only
 * (NULL = empty histories), state_out written (NULL = discarded; the same array
 * as state_in or one that does not overlap it, else TAYLOR_ERR_INVALID_ARG).
 * Every row of state_out is written, an empty sequence's with its incoming
 * state (zero when state_in is NULL).  Other arguments, sizes and errors as
 * taylor_attn_prefill_varlen. */
int taylor_attn_prefill_varlen_into(const void* q, const void* k, const void* v, float* o, const float* state_in,
                                    float* state_out, void* workspace, const int32_t* cu_seqlens, int n_seqs, int H,
                                    int max_seqlen, int64_t total_tokens, const taylor_config* cfg,
                                    hipStream_t stream);

/* Bytes of device workspace taylor_attn_prefill_backward needs (may be 0).  Host
 * only.  Negative taylor_status if cfg or sizes are invalid, or
 * TAYLOR_ERR_UNSUPPORTED where no backward kernel is compiled (below). */
int64_t taylor_prefill_backward_workspace_bytes(const taylor_config* cfg, int B, int H, int N);

/* Gradients of one taylor_attn_prefill call (truncated-kernel readout; the pages
 * give no gradients -- they are the derivatives of the Abstract's definition).
 * With L a loss of the outputs o = taylor_attn_prefill(q, k, v | state):
 *   q, k, v : the forward's inputs, [B,H,N,d_k], [B,H,N,d_k], [B,H,N,d_v] in cfg->in_dtype;
 *   o       : the forward's outputs [B,H,N,d_v] float32;
 *   g       : dL/do, [B,H,N,d_v] float32;
 *   state   : the forward's incoming state [B,H,stride] (NULL: empty history);
 *             read only;
 *   dstate  : [B,H,stride] float32 in/out, or NULL.  On entry dL/d(the final
 *             state the forward returned) (NULL: zero); on return dL/d(the
 *             incoming state), in the state layout (S rows then z);
 *   dq, dk, dv : [B,H,N,d_k], [B,H,N,d_k], [B,H,N,d_v] float32 outputs (dq, dk
 *             include the score scale);
 *   workspace : taylor_prefill_backward_workspace_bytes(cfg, B, H, N) bytes.
 * So a sequence prefilled in pieces is differentiated piece by piece in reverse,
 * passing dstate along.  Compiled for cfg->readout = TAYLOR_READOUT_KERNEL,
 * n_terms = 1..5, d_k = 16, d_v = 64, either input type (float32 arithmetic;
 * n = 4, 5 on feature blocks, whose per-block partial gradients make the
 * workspace 5,456 (n = 4) or 12,584 (n = 5) bytes per token and head);
 * otherwise TAYLOR_ERR_UNSUPPORTED.  B*H == 0 or N == 0 is a no-op (dstate
 * unchanged).  Calls sharing a workspace must not overlap. */
int taylor_attn_prefill_backward(const void* q, const void* k, const void* v, const float* o, const float* g,
                                 const float* state, float* dstate, float* dq, float* dk, float* dv, void* workspace,
                                 int B, int H, int N, const taylor_config* cfg, hipStream_t stream);

/* One decode step per (b, h).  The Abstract of "Expanding Attention": each of
 * the n states is updated by one rank-one outer product per token, independent
 * of the context length N, so a step costs the same at any history length:
 * S += phi(k_t) [v_t | 1]^T (one rank-one update),
 * then o_t = (phi(scale*q_t)^T S)[:d_v] / (phi(scale*q_t)^T z) -- the update comes
 * first, so the current token attends to itself.  (TAYLOR_READOUT_CENTERED: the
 * same update, then the expanded-softmax output of the token over its history.)
 *   q, k, v : [B,H,d_k], [B,H,d_k], [B,H,d_v] in cfg->in_dtype;
 *   o       : [B,H,d_v] float32;
 *   state   : [B,H,stride] float32, updated in place.
 * B*H == 0 is a no-op. */
int taylor_attn_decode_step(const void* q, const void* k, const void* v, float* o, float* state, int B, int H,
                            const taylor_config* cfg, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TAYLOR_ATTN_H */
