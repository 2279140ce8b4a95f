/*
 * lcv_bsa.h -- C ABI of the LongCat-Video block-sparse 3D self-attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is the self-attention of the LongCat-Video diffusion transformer over
 * patchified video latent tokens:
 *   - tokens are the latent grid (T, H, W) flattened row-major in (t, y, x); condition
 *     frames come first along time (myzaker article on LongCat-Video, section on the
 *     technical principles: noise-free condition frames and noisy frames concatenated on
 *     the time axis; the number of condition frames selects text-, image- or
 *     video-conditioned generation);
 *   - attention runs over blocks of 64 consecutive tokens; query block i attends key
 *     block j iff |i - j| <= local_blocks or j % global_stride == 0 (longcat-video-rs page,
 *     section 02 benchmark table "block=64, local=2, stride=4" and section 03
 *     "Block-Sparse & Multi-Audio"; zhichai.net post, section "Block Sparse Attention":
 *     dense inside a block pair, sparse between blocks);
 *   - condition tokens (the first cond_len tokens) attend only to condition tokens, so
 *     their keys and values can be cached and reused across calls (myzaker article,
 *     technical principles: block attention with a KV cache);
 *   - queries and keys carry a partitioned 3D rotary embedding: channels [0,16) turn with
 *     t, [16,40) with y, [40,64) with x, adjacent channel pairs as complex numbers, pair p
 *     of a section of width d at angle pos * theta^(-2p/d) (longcat-video-rs page, section
 *     03 "Partitioned 3D-RoPE (16T+24H+24W)").
 *
 * Numerics: bf16 inputs, RoPE in fp32 rounded to bf16 before the matrix cores, scores
 * and softmax in fp32 with fp32 accumulation, probabilities rounded to bf16 for the
 * P*V product, bf16 output, fp32 natural-log LSE of the scores scaled by 1/sqrt(64).
 *
 * Conventions for every entry point:
 *   - Tensors are caller-owned device memory, contiguous, row-major, with the shapes
 *     stated below; bf16 tensors are passed as void* and must be 16-byte aligned, fp32
 *     tensors 4-byte aligned.  The library never frees them and no forward or RoPE call
 *     allocates memory.
 *   - Calls are asynchronous on the given stream (0 = the null stream) and never
 *     synchronise, except lcv_bsa_build_layout (see there).  Results are bitwise
 *     deterministic for identical inputs on the same GPU.
 *   - Every argument is validated on the host before anything is launched: on error the
 *     status says why, nothing is launched and lcv_last_error() holds a message.  HIP
 *     failures are reported as LCV_ERR_HIP.
 *   - A layout is immutable after it is built and may be shared by concurrent calls on
 *     any streams and threads.
 *   - Every call except lcv_bsa_build_layout, lcv_bsa_layout_copy_csr and
 *     lcv_bsa_layout_destroy only launches kernels on the given stream (no allocation,
 *     copy, memset or synchronisation), so it may be captured into a HIP graph and
 *     replayed; the buffers it was given stay bound to the graph.
 */
#ifndef LCV_BSA_H
#define LCV_BSA_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LCV_BSA_ABI_VERSION 11
#define LCV_HEAD_DIM 64   /* channels per head (16 + 24 + 24 rotary channels) */
#define LCV_BLOCK 64      /* tokens per attention block */

typedef enum lcv_status {
  LCV_OK = 0,
  LCV_ERR_NULL = 1,            /* a required pointer is NULL */
  LCV_ERR_INVALID_ARG = 2,     /* a value is out of range or a pointer is misaligned */
  LCV_ERR_SHAPE = 3,           /* sizes disagree (e.g. N != T*H*W) */
  LCV_ERR_LAYOUT_MISMATCH = 5, /* cond_len differs from the one the layout was built for */
  LCV_ERR_UNSUPPORTED = 6,     /* valid but beyond what the library supports (sizes) */
  LCV_ERR_OOM = 7,             /* device allocation failed (layout build only) */
  LCV_ERR_HIP = 8              /* a HIP runtime call failed */
} lcv_status;

/* flags of the forward calls: apply the 3D-RoPE to Q and/or K while loading them.
 * Without a flag the corresponding input is taken as already rotated. */
#define LCV_ROPE_Q 1u
#define LCV_ROPE_K 2u

/* Block layout parameters.  n_tokens = N >= 1; block must be 64; local_blocks = w >= 0
 * (window radius in blocks); global_stride = s >= 0 (0 disables global blocks, 1 makes
 * every key block global); cond_len = C in [0, N] (condition tokens [0, C)). */
typedef struct lcv_bsa_layout_params {
  int32_t n_tokens;
  int32_t block;
  int32_t local_blocks;
  int32_t global_stride;
  int32_t cond_len;
} lcv_bsa_layout_params;

/* Latent grid of the 3D-RoPE: tokens are (t, y, x) row-major with t < T, y < H, x < W;
 * theta is the rotary base (1e4 for LongCat-Video). */
typedef struct lcv_rope3d_grid {
  int32_t T;
  int32_t H;
  int32_t W;
  float theta;
} lcv_rope3d_grid;

typedef struct lcv_bsa_layout_info {
  int32_t n_tokens;
  int32_t n_blocks;        /* ceil(N / 64) */
  int32_t local_blocks;
  int32_t global_stride;
  int32_t cond_len;
  int32_t max_row_len;     /* longest CSR row */
  int64_t nnz;             /* CSR entries: block pairs holding >= 1 attended token pair */
  int64_t attended_pairs;  /* (q, k) token pairs attended, per (batch, head) */
} lcv_bsa_layout_info;

typedef struct lcv_bsa_layout lcv_bsa_layout; /* opaque */

/* Sizes of the layout that lcv_bsa_build_layout would build, computed on the host in
 * closed form without touching the GPU.  Errors: NULL, INVALID_ARG, UNSUPPORTED
 * (nnz >= 2^31). */
lcv_status lcv_bsa_layout_query(const lcv_bsa_layout_params* params, lcv_bsa_layout_info* info);

/* Build the block layout on the GPU: the CSR (row_ptr[n+1], ascending col_idx[nnz], int32)
 * of key blocks per query block -- block pairs of the rule above that hold at least one
 * token pair allowed by the condition rule -- plus the internal schedule the forward
 * kernels walk.  Allocates device memory owned by the returned handle and waits for the
 * stream before returning (built once per shape, reused across steps, layers, heads and
 * batch items).  Errors: NULL, INVALID_ARG, UNSUPPORTED, OOM, HIP; *out is NULL on error. */
lcv_status lcv_bsa_build_layout(const lcv_bsa_layout_params* params, hipStream_t stream,
                                lcv_bsa_layout** out);

/* Sizes of a built layout.  Errors: NULL. */
lcv_status lcv_bsa_layout_get_info(const lcv_bsa_layout* layout, lcv_bsa_layout_info* info);

/* Copy the CSR into caller-owned device buffers row_ptr[n_blocks+1] and col_idx[nnz]
 * (int32), asynchronously on stream.  Errors: NULL, INVALID_ARG (misaligned), HIP. */
lcv_status lcv_bsa_layout_copy_csr(const lcv_bsa_layout* layout, int32_t* row_ptr, int32_t* col_idx,
                                   hipStream_t stream);

/* Release a layout (NULL is a no-op).  The caller must ensure no queued call still uses it. */
void lcv_bsa_layout_destroy(lcv_bsa_layout* layout);

/* Apply the partitioned 3D-RoPE to x[n_outer, n_tokens, 64] (bf16) and write y (bf16, may be
 * equal to x for in-place use; must not otherwise overlap x).  Row r of each of the n_outer
 * slices (batch * heads) is token token_offset + r of the grid, so noise tokens of a cached
 * call pass token_offset = cond_len.  Math in fp32, result rounded to nearest even bf16.
 * Errors: NULL, INVALID_ARG (n_outer < 0, n_tokens < 0, token_offset < 0, theta <= 0,
 * misalignment), SHAPE (token_offset + n_tokens > T*H*W), UNSUPPORTED (n_outer > 131070),
 * HIP. */
lcv_status lcv_rope3d_apply(const void* x, void* y, int64_t n_outer, int32_t n_tokens,
                            int32_t token_offset, const lcv_rope3d_grid* grid, hipStream_t stream);

/* Query/key prologue of the self-attention (myzaker article, technical principles: RMSNorm
 * in the self-attention module, 3D RoPE on visual tokens).  Each 64-channel row of
 * x[n_outer, n_tokens, 64] (bf16) is RMS-normalised with the gain gamma[64] (fp32, device
 * memory): x / sqrt(mean(x^2) + eps) * gamma; when grid is not NULL the partitioned 3D-RoPE
 * then turns it by the position of token token_offset + r (row r of every slice).  The
 * result goes to y (bf16; y may equal x, otherwise the two must not overlap).  Math in fp32,
 * one rounding to nearest-even bf16 at the end.  Call it once for Q and once for K (each
 * with its own gain) before lcv_bsa_forward with flags = 0.  Errors: NULL (x, y or gamma),
 * INVALID_ARG (n_outer, n_tokens or token_offset < 0, eps < 0 or not finite, theta <= 0,
 * x or y not 16-byte aligned, gamma not 4-byte aligned), SHAPE (token_offset + n_tokens >
 * T*H*W), UNSUPPORTED (n_outer > 131070), HIP. */
lcv_status lcv_qk_rmsnorm_rope3d(const void* x, void* y, const float* gamma, float eps, int64_t n_outer,
                                 int32_t n_tokens, int32_t token_offset, const lcv_rope3d_grid* grid,
                                 hipStream_t stream);

/* Block-sparse attention over all N tokens.
 *   q, k, v : bf16 [batch, heads, N, 64], N = layout n_tokens
 *   out     : bf16 [batch, heads, N, 64]
 *   lse     : fp32 [batch, heads, N] natural-log LSE of the scaled scores, or NULL
 *   cond_len: must equal the layout's (LCV_ERR_LAYOUT_MISMATCH otherwise)
 *   flags   : LCV_ROPE_Q | LCV_ROPE_K subset; grid is required (N == T*H*W) iff a flag is set
 * A query row with no attended key (impossible with the layouts above) gets out = 0 and
 * lse = -inf.  Errors: NULL, INVALID_ARG, SHAPE, LAYOUT_MISMATCH, UNSUPPORTED, HIP. */
lcv_status lcv_bsa_forward(const void* q, const void* k, const void* v, int32_t batch, int32_t heads,
                           const lcv_bsa_layout* layout, int32_t cond_len, uint32_t flags,
                           const lcv_rope3d_grid* grid, void* out, float* lse, hipStream_t stream);

/* Block-sparse attention of the noise tokens [C, N) only, with the condition keys and
 * values taken from a cache (C = cond_len, N = layout n_tokens):
 *   q_noise, k_noise, v_noise : bf16 [batch, heads, N-C, 64] (token C+r at row r)
 *   k_cond, v_cond            : bf16 [batch, heads, C, 64], the condition K/V exactly as a
 *                               full call received them (raw K if LCV_ROPE_K is set,
 *                               pre-rotated K otherwise); may be NULL when C == 0
 *   out_noise                 : bf16 [batch, heads, N-C, 64]; lse_noise fp32 [batch, heads, N-C] or NULL
 * Results equal rows [C, N) of lcv_bsa_forward on the concatenated sequence, bitwise.
 * C == N is a valid no-op.  Errors as lcv_bsa_forward. */
lcv_status lcv_bsa_forward_cached(const void* q_noise, const void* k_noise, const void* v_noise,
                                  const void* k_cond, const void* v_cond, int32_t batch, int32_t heads,
                                  const lcv_bsa_layout* layout, int32_t cond_len, uint32_t flags,
                                  const lcv_rope3d_grid* grid, void* out_noise, float* lse_noise,
                                  hipStream_t stream);

/* Rows [row_begin, row_end) of lcv_bsa_forward: one device's share of a sequence-sharded call
 * (context-parallel attention, myzaker article, technical principles: context-parallel
 * block-sparse attention for high resolution).  q, out and lse hold only the range's rows
 * ([batch, heads, row_end - row_begin, 64] and [batch, heads, row_end - row_begin]); k and v
 * are the full [batch, heads, N, 64] tensors (on several devices, the gathered key/value
 * blocks the range's rows attend to).  The rows' results are bitwise those of the full call.
 * An empty range (row_begin == row_end) does nothing (its pointers may be NULL).
 * Errors as lcv_bsa_forward, plus INVALID_ARG for a range outside [0, N]. */
lcv_status lcv_bsa_forward_rows(const void* q, const void* k, const void* v, int32_t batch, int32_t heads,
                                const lcv_bsa_layout* layout, int32_t cond_len, uint32_t flags,
                                const lcv_rope3d_grid* grid, int32_t row_begin, int32_t row_end, void* out, float* lse,
                                hipStream_t stream);

/* Backward of lcv_qk_rmsnorm_rope3d for LoRA training of the projections before it (myzaker
 * article, technical principles: RMSNorm and 3D RoPE in the self-attention; the LoRA-trained
 * refinement expert): with n = x / sqrt(mean(x^2) + eps) and dy' = R^T dy (each channel pair
 * rotated by minus its angle; dy' = dy when grid is NULL),
 *   dgamma = sum over every row of dy' * n,  dx = (dn - n * mean(dn * n)) / sqrt(mean(x^2) + eps),
 *   dn = dy' * gamma.
 *   x, dy, dx : bf16 [n_outer, n_tokens, 64] (x the prologue's input; dx may be x or dy)
 *   gamma     : fp32 [64], 16-byte aligned;  dgamma : fp32 [64], written (not accumulated)
 *   workspace : fp32, caller-owned, at least lcv_qk_rmsnorm_rope3d_backward_workspace(n_outer,
 *               n_tokens) values (one 64-value partial per workgroup)
 * Deterministic (the partials are added in a fixed order).  Asynchronous on stream.  Errors:
 * NULL, INVALID_ARG (sizes, alignment, eps, small workspace), SHAPE, UNSUPPORTED, HIP. */
int64_t lcv_qk_rmsnorm_rope3d_backward_workspace(int64_t n_outer, int32_t n_tokens);
lcv_status lcv_qk_rmsnorm_rope3d_backward(const void* x, const void* dy, const float* gamma, float eps,
                                          int64_t n_outer, int32_t n_tokens, int32_t token_offset,
                                          const lcv_rope3d_grid* grid, void* dx, float* dgamma, float* workspace,
                                          int64_t workspace_floats, hipStream_t stream);

/* lcv_qk_rmsnorm_rope3d_backward without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  The dgamma partials go to a static
 * device array of the library (4 MiB, 1,048,576 fp32 values: one 64-value partial per
 * workgroup, i.e. sizes with lcv_qk_rmsnorm_rope3d_backward_workspace(n_outer, n_tokens) <=
 * 1,048,576), of which every GPU the library runs on holds its own copy until the process
 * ends.  Every call on a GPU shares that GPU's array: calls that overlap on one GPU (other
 * streams, other threads) race and must be serialised by the caller.  Same arguments,
 * results (bitwise) and errors as lcv_qk_rmsnorm_rope3d_backward, plus UNSUPPORTED for sizes
 * beyond the array. */
lcv_status lcv_qk_rmsnorm_rope3d_backward_noalloc(const void* x, const void* dy, const float* gamma, float eps,
                                                  int64_t n_outer, int32_t n_tokens, int32_t token_offset,
                                                  const lcv_rope3d_grid* grid, void* dx, float* dgamma,
                                                  hipStream_t stream);

/* Backward of lcv_bsa_forward (flags = 0): the gradients of the attention for the upstream
 * gradient dout, for training (myzaker article, technical principles: the LoRA-trained
 * refinement expert; SimpleTuner quickstart "LongCat-Video Edit").  With P recomputed from
 * the saved LSE: dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(dO * O)), dQ = dS K / 8,
 * dK = dS^T Q / 8, under the same layout and condition rule as the forward.  P is formed
 * from the forward's own score operands (Q rounded to bf16 after its scaling by
 * log2(e)/8, as the forward rounds it), so it agrees with the saved LSE for any score size;
 * dK takes that same rounded Q.
 *   q, k, v, out, dout : bf16 [batch, heads, N, 64]; q and k as they entered the scores (a
 *                        caller that rotates with RoPE passes the rotated tensors and
 *                        rotates dq, dk back), out the forward's output
 *   lse                : fp32 [batch, heads, N], the forward's
 *   dq, dk, dv         : bf16 [batch, heads, N, 64], written completely (fp32 accumulation)
 *   workspace          : fp32 scratch, caller-owned, 16-byte aligned, at least
 *                        lcv_bsa_backward_workspace(batch, heads, N) values (152 B per query
 *                        row: the scaled Q, two per-row terms and their folded bf16 parts;
 *                        -1 for invalid sizes)
 * Deterministic: every output row is written once, without atomics.  Asynchronous on
 * stream.  Errors: NULL, INVALID_ARG (sizes, alignment, device, small workspace),
 * LAYOUT_MISMATCH (cond_len), UNSUPPORTED (sizes), HIP. */
int64_t lcv_bsa_backward_workspace(int32_t batch, int32_t heads, int32_t n_tokens);
lcv_status lcv_bsa_backward(const void* q, const void* k, const void* v, const void* out, const float* lse,
                            const void* dout, int32_t batch, int32_t heads, const lcv_bsa_layout* layout,
                            int32_t cond_len, void* dq, void* dk, void* dv, float* workspace,
                            int64_t workspace_floats, hipStream_t stream);

/* Cross-attention of the video tokens over text states, the second attention of every DiT
 * block (myzaker article, technical principles: each block has 3D self-attention,
 * cross-attention and a SwiGLU feed-forward network): out = softmax(q k^T / 8) v, dense over
 * the text tokens, no RoPE.
 *   q, out   : bf16 [batch, heads, n_q, 64] (video queries; normalise them first with
 *              lcv_qk_rmsnorm_rope3d and grid = NULL if the model does)
 *   k, v     : bf16 [batch, heads, kv_len, 64] (projected text states, padded to kv_len)
 *   kv_lens  : device int32 [batch] valid text tokens per batch item (keys at or past it are
 *              padding and ignored; values are clamped to [0, kv_len]), or NULL for kv_len
 *   lse      : fp32 [batch, heads, n_q] natural-log LSE of the scaled scores, or NULL
 * A batch item with no valid text token gives out = 0 and lse = -inf.  With n_q = 0 every
 * pointer, with kv_len = 0 k and v may be NULL.  Caller-owned memory,
 * no allocation, asynchronous on stream, deterministic.  Errors: NULL, INVALID_ARG (sizes,
 * alignment), UNSUPPORTED (sizes), HIP. */
lcv_status lcv_cross_attention(const void* q, const void* k, const void* v, int32_t batch, int32_t heads,
                               int32_t n_q, int32_t kv_len, const int32_t* kv_lens, void* out, float* lse,
                               hipStream_t stream);

/* Backward of lcv_cross_attention, for training the projections around it (myzaker article,
 * technical principles: each block has 3D self-attention, cross-attention and a SwiGLU
 * feed-forward network; the LoRA-trained refinement expert).  With P recomputed from the
 * saved LSE over the valid text keys: dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(dO * O)),
 * dQ = dS K / 8, dK = dS^T Q / 8 (P and dK from the forward's rounded scaled Q, as in
 * lcv_bsa_backward).
 *   q, out, dout : bf16 [batch, heads, n_q, 64];  lse : fp32 [batch, heads, n_q], the forward's
 *   k, v         : bf16 [batch, heads, kv_len, 64];  kv_lens as in lcv_cross_attention
 *   dq           : bf16 [batch, heads, n_q, 64];  dk, dv : bf16 [batch, heads, kv_len, 64];
 *                  all written completely (padded text rows and a batch item without text
 *                  get zeros)
 *   workspace    : fp32, caller-owned, 16-byte aligned, at least
 *                  lcv_cross_attention_backward_workspace(batch, heads, n_q, kv_len) values
 *                  (the scaled Q, two per-row terms and their bf16 parts, 152 B per query row, and the fp32
 *                  partial dK, dV of the query chunks; -1 for invalid sizes)
 * With n_q = 0 (dk = dv = 0) the query-side pointers, with kv_len = 0 (dq = 0) the text-side
 * pointers, and a workspace of size 0 may be NULL.
 * Deterministic: the chunks' partial sums are added in a fixed order, without atomics.
 * Asynchronous on stream.  Errors: NULL, INVALID_ARG (sizes, alignment, small workspace),
 * UNSUPPORTED (sizes), HIP. */
int64_t lcv_cross_attention_backward_workspace(int32_t batch, int32_t heads, int32_t n_q, int32_t kv_len);
lcv_status lcv_cross_attention_backward(const void* q, const void* k, const void* v, const void* out,
                                        const float* lse, const void* dout, int32_t batch, int32_t heads, int32_t n_q,
                                        int32_t kv_len, const int32_t* kv_lens, void* dq, void* dk, void* dv,
                                        float* workspace, int64_t workspace_floats, hipStream_t stream);

/* Merge of attention results over disjoint key sets, the combine step of context-parallel
 * ring attention (myzaker article, technical principles: context-parallel ring block-sparse
 * attention): lse = log(sum_i exp(lse_i)), out = sum_i exp(lse_i - lse) * out_i, the
 * attention over the union of the sets.
 *   outs     : host array of n_parts device pointers, bf16 [rows, 64] each (rows = B*H*N)
 *   lses     : host array of n_parts device pointers, fp32 [rows] each (natural-log LSE;
 *              -inf marks a row with no key in that part)
 *   n_parts  : 1 .. 8
 *   out, lse : bf16 [rows, 64] and fp32 [rows] (lse may be NULL); may be outs[i] / lses[i]
 *              (in-place merge)
 * A row empty in every part gives out = 0, lse = -inf.  fp32 math, one bf16 rounding.
 * Asynchronous on stream.  Errors: NULL, INVALID_ARG (sizes, alignment), UNSUPPORTED, HIP. */
lcv_status lcv_attn_merge(const void* const* outs, const float* const* lses, int32_t n_parts, int64_t rows,
                          void* out, float* lse, hipStream_t stream);

/* Message of the last failing call on this thread ("" if none). */
const char* lcv_last_error(void);

/* LCV_BSA_ABI_VERSION of the loaded library. */
int32_t lcv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LCV_BSA_H */
