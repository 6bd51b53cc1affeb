/*
 * moe.h - C ABI of the MI355X (gfx950) fine-grained MoE FFN layer library.
 *
 * The layer is the dots.llm1 mixture-of-experts feed-forward block:
 *   - FP32 gating over E routed experts with a per-expert selection bias,
 *     top-K selection, plus S always-on shared experts
 *     ("dots.llm1 Technical Report" summary page, sections "Key claims" and
 *     "Method"; "dots.llm1: the first MoE large language model open-sourced by
 *     Little Red Book", section "Model Architecture Features");
 *   - tokens permuted into per-expert segments padded to the GEMM tile
 *     multiple, no token dropped (Technical Report summary, "Key claims" and
 *     "Method");
 *   - SwiGLU experts, each a two-layer feed-forward network (aibase news item,
 *     architecture paragraph);
 *   - the weighted combine of the K routed outputs plus the shared outputs.
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless a comment says "host".  bf16 values
 *     are passed as uint16_t bit patterns.  Every array is dense row-major.
 *   - Every device pointer is 16-byte aligned and every workspace 256-byte
 *     aligned (the kernels move rows with 16-byte vector accesses); a call
 *     with a misaligned pointer is rejected with MOE_ERR_INVALID_ARGUMENT.
 *   - The caller owns every buffer.  The library never allocates device
 *     memory on these paths, never frees, and keeps no pointer after return.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *     default stream) and performs no host<->device synchronisation.
 *   - Errors are reported by the return code only (moe_status_t); nothing is
 *     thrown across the ABI.  Argument checks run on the host before any HIP
 *     call, so a rejected call has launched nothing.  T == 0 is a valid no-op.
 *   - Outputs are deterministic: the same inputs give bit-identical outputs
 *     (no floating-point atomics anywhere).
 *   - Shape limits: H % 64 == 0, F % 32 == 0, H <= 65536, F <= 65536,
 *     F * H < 2^30 (one expert's weights below 4 GiB), 1 <= K <= E <= 128,
 *     K <= 16, align == moe_align(); row counts below 2^31; for the
 *     weight-gradient entry points m_rows * max(H, 2F) * 2 bytes below 4 GiB
 *     (each segment is addressed with 32-bit buffer offsets, 419,430 rows at
 *     H = 5120; every admitted segment is read in full and nothing past it).
 *     Calls outside these limits return MOE_ERR_UNSUPPORTED_SHAPE.
 *
 * Readings of what the pages leave open (all entry points follow them):
 *   scores are sigmoid(logit); the bias is added for selection only; the K
 *   combine weights are the selected scores normalised to sum 1; shared experts
 *   have weight 1; ties in top-K go to the lower expert index (NaN ranks
 *   lowest); the K experts of a token are listed by key descending; rows of a
 *   segment are its tokens in ascending order; an expert with no tokens owns no
 *   rows; gate = first F rows of W1 and h = silu(gate) * up; the backward is
 *   the gradient with the routing decision held fixed (no bias gradient).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status_t;
#define MOE_OK 0
#define MOE_ERR_INVALID_ARGUMENT 1   /* null pointer, negative size, K > E ... */
#define MOE_ERR_UNSUPPORTED_SHAPE 2  /* H, F, K, E or align outside the compiled limits */
#define MOE_ERR_WORKSPACE_TOO_SMALL 3
#define MOE_ERR_HIP 4                /* a HIP launch failed; see moe_last_error() */

/* host: static string for a status code. */
const char* moe_status_string(moe_status_t status);

/* host: message of the last failure on the calling thread ("" if none). */
const char* moe_last_error(void);

/* host: the segment alignment = the grouped-GEMM row tile (128). */
int32_t moe_align(void);

/* host: upper bound on the padded routed row count,
 * ceil((T*K + E*(align-1)) / align) * align.  Row buffers of the routed path
 * (x_rows, act, h, y_rows, dy_rows, dact, dx_rows) have this many rows. */
int64_t moe_capacity_rows(int32_t T, int32_t E, int32_t K);

/* host: bytes of the workspace moe_route needs for T tokens: the router
 * weight's three bf16 parts (3 * ceil(E/32)*32 * H * 2 bytes, rounded up to
 * 256) and the projection's per-slice logits (S * T * 128 * 4 bytes, where S,
 * the number of slices of h, depends on T and H).  0 for invalid arguments. */
size_t moe_route_workspace_bytes(int32_t T, int32_t H, int32_t E);

/* host: bytes of the workspace moe_permute needs (at least 256: its first
 * 16 bytes receive the data-check block, see moe_permute_check). */
size_t moe_permute_workspace_bytes(int32_t T, int32_t E, int32_t K);

/* host: bytes of the workspace moe_route_bwd needs. */
size_t moe_route_bwd_workspace_bytes(int32_t T, int32_t H, int32_t E, int32_t K);

/* host: bytes of the workspace moe_seq_balance_fwd needs (0 for invalid
 * arguments, including T % seq_len != 0). */
size_t moe_seq_balance_workspace_bytes(int32_t T, int32_t E, int32_t seq_len);

/* host: bytes of the workspace moe_route_bwd_dense needs. */
size_t moe_route_bwd_dense_workspace_bytes(int32_t T, int32_t H, int32_t E);

/*
 * moe_route - FP32 gating, selection bias, top-K, combine weights.
 * (Technical Report summary, "Method": gating projection in FP32, top-6 of 128,
 * auxiliary-loss-free balancing by a bias; model card: dynamic bias terms.)
 *
 *   logit[t,e] = sum_h x[t,h] * w_router[h,e]         (fp32 arithmetic)
 *   s[t,e]     = sigmoid(logit[t,e])
 *   v[t,e]     = s[t,e] + bias[e]                      (selection key only)
 *   topk_idx[t,:] = the K experts with the largest v, key descending, ties to
 *                   the lower index
 *   topk_s[t,k]   = s[t, topk_idx[t,k]]
 *   topk_w[t,k]   = topk_s[t,k] / sum_j topk_s[t,j]
 *
 * x [T,H] bf16; w_router [H,E] fp32; bias [E] fp32;
 * topk_idx [T,K] int32; topk_w [T,K] fp32; topk_s [T,K] fp32 (nullable);
 * scores [T,E] fp32 (nullable): every s[t,e], the input of the sequence-wise
 * balance loss (moe_seq_balance_fwd / _bwd).
 * ws: device workspace of at least moe_route_workspace_bytes(T,H,E) bytes (the
 * router weight re-encoded for the matrix cores and the partial logits of
 * each slice of h; rewritten by every call).
 * x must be finite: the projection multiplies x by the exact three-part split
 * of each weight, so an infinite input meets zero parts and gives NaN logits;
 * a NaN key ranks below every other (such a token selects experts 0..K-1 with
 * NaN weights).
 */
moe_status_t moe_route(int32_t T, int32_t H, int32_t E, int32_t K,
                       const uint16_t* x, const float* w_router, const float* bias,
                       int32_t* topk_idx, float* topk_w, float* topk_s, float* scores,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * moe_permute - token permutation into per-expert segments padded to `align`
 * rows (Technical Report summary, "Key claims" / "Method": segments padded to
 * the GEMM tile multiple; no token dropped).  Integer outputs are bit-exact:
 *
 *   counts[e]      = number of tokens that selected e                    [E]
 *   offsets[e]     = sum_{j<e} ceil(counts[j]/align)*align; offsets[E] is
 *                    the padded total                                   [E+1]
 *   row_of[t,k]    = offsets[e] + (number of tokens t' < t that selected
 *                    e = topk_idx[t,k])                                  [T,K]
 *   src_token[r]   = token held by row r, -1 for a padding row or a row
 *                    at or beyond offsets[E]                             [m_cap]
 *   tile_expert[i] = expert owning rows [i*align, (i+1)*align), -1 for
 *                    tiles at or beyond offsets[E]                  [m_cap/align]
 *   x_rows[r,:]    = x[src_token[r],:] for every non-padding row; padding rows
 *                    are left untouched                            [m_cap,H] bf16
 *
 * Data check (every call): a token whose K ids are not all in [0,E) and
 * distinct (moe_route always writes such ids) is rejected before any of its
 * ids indexes memory: it is not counted, owns no row, its row_of entries are
 * -1 and its x row is not copied; every other token is permuted as above.
 * The call records what it rejected in the first 16 bytes of ws (four int32:
 * flags, number of rejected tokens, first rejected token, a marker), which
 * moe_permute_check decodes after the caller copies them to host memory.  If
 * any token was rejected, the routing must not be passed on: the other entry
 * points read topk_idx and row_of without checking them.
 * m_cap must be >= moe_capacity_rows(T,E,K) and a multiple of align.
 * ws: device workspace of at least moe_permute_workspace_bytes(T,E,K) bytes.
 */
moe_status_t moe_permute(int32_t T, int32_t H, int32_t E, int32_t K, int32_t align,
                         const int32_t* topk_idx, const uint16_t* x, int64_t m_cap,
                         int32_t* counts, int32_t* offsets, int32_t* row_of,
                         int32_t* src_token, int32_t* tile_expert, uint16_t* x_rows,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * moe_permute_noalloc - moe_permute for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same permutation and data check, same arguments
 * and results, but no workspace argument.  Its kernels use a static device
 * array of the library (530,688 bytes on each GPU it runs on, held until the
 * process ends), which bounds T to moe_permute_noalloc_max_tokens() (131,072);
 * larger T is rejected with MOE_ERR_UNSUPPORTED_SHAPE.  The call allocates
 * nothing (no hipMalloc, no allocating library routine).  Every word of the
 * array the kernels read is written earlier in the same call, so nothing
 * carries over from the previous call; calls that overlap in time on one GPU
 * share the array and race (serialise them, e.g. on one stream).
 * status: device int32 [4] (nullable) that receives the data-check block
 * (see moe_permute / moe_permute_check); with NULL it stays in the array.
 */
int32_t moe_permute_noalloc_max_tokens(void);
moe_status_t moe_permute_noalloc(int32_t T, int32_t H, int32_t E, int32_t K, int32_t align,
                                 const int32_t* topk_idx, const uint16_t* x, int64_t m_cap,
                                 int32_t* counts, int32_t* offsets, int32_t* row_of,
                                 int32_t* src_token, int32_t* tile_expert, uint16_t* x_rows,
                                 int32_t* status, void* stream);

/*
 * moe_permute_check - host: decodes moe_permute's data-check block.
 * words: host copy of the first four int32 of moe_permute's workspace.
 * Returns MOE_OK when no token was rejected; MOE_ERR_INVALID_ARGUMENT when
 * some were (moe_last_error() then names the cause: an id outside [0,E), an
 * id repeated within a token, or both; how many tokens; the first one), or
 * when the words are not a block moe_permute wrote.  Touches no device state.
 */
moe_status_t moe_permute_check(const int32_t* words);

/*
 * moe_grouped_swiglu_fwd - grouped SwiGLU expert FFN over row segments
 * (aibase news item: each expert is two feed-forward layers with SwiGLU;
 * Technical Report summary: grouped GEMM over tile-padded expert segments).
 *
 * For every group g and every valid row r of its segment
 * (offsets[g] <= r < offsets[g]+counts[g]):
 *   [gate | up] = x_rows[r,:] . w1[g]^T      (w1 [G,2F,H]: gate rows 0..F-1)
 *   h[r,:]      = silu(gate) * up            (bf16 [m_rows,F])
 *   y_rows[r,:] = h[r,:] . w2[g]^T           (w2 [G,H,F]; bf16 [m_rows,H])
 *   act[r,:]    = [gate | up] rounded to bf16 (bf16 [m_rows,2F]; nullable, kept
 *                 for the backward)
 * bf16 operands, fp32 accumulation, bf16 outputs.  Rows outside every
 * segment are not written.
 *
 * Routed use: G = E, m_rows = m_cap, offsets/counts/tile_expert from
 * moe_permute.  Dense use (the shared experts): offsets = counts =
 * tile_expert = NULL, G = 1, m_rows = T: one segment of all T rows of x.  S
 * shared experts are passed fused as one expert of width S*F: w1 = the S gate
 * blocks stacked, then the S up blocks ([2SF,H]); w2 = the S down matrices side
 * by side ([H,SF]); this equals the sum of the S experts.
 */
moe_status_t moe_grouped_swiglu_fwd(int32_t G, int64_t m_rows, int32_t H, int32_t F,
                                    const int32_t* offsets, const int32_t* counts,
                                    const int32_t* tile_expert, const uint16_t* x_rows,
                                    const uint16_t* w1, const uint16_t* w2, uint16_t* act,
                                    uint16_t* h, uint16_t* y_rows, void* stream);

/*
 * moe_grouped_gate_up_fwd / moe_grouped_down_fwd - the two halves of
 * moe_grouped_swiglu_fwd, same arguments and results: the first computes act
 * and h (gate/up GEMM with SwiGLU fused into its epilogue), the second y_rows
 * from h (down GEMM).  moe_grouped_swiglu_fwd is exactly the first followed by
 * the second.
 */
moe_status_t moe_grouped_gate_up_fwd(int32_t G, int64_t m_rows, int32_t H, int32_t F,
                                     const int32_t* offsets, const int32_t* counts,
                                     const int32_t* tile_expert, const uint16_t* x_rows,
                                     const uint16_t* w1, uint16_t* act, uint16_t* h,
                                     void* stream);
moe_status_t moe_grouped_down_fwd(int32_t G, int64_t m_rows, int32_t H, int32_t F,
                                  const int32_t* offsets, const int32_t* counts,
                                  const int32_t* tile_expert, const uint16_t* h,
                                  const uint16_t* w2, uint16_t* y_rows, void* stream);

/*
 * moe_dense_gate_up_fwd_split / moe_dense_down_fwd_split - the dense (one
 * group, G = 1, no segments) uses of moe_grouped_gate_up_fwd and
 * moe_grouped_down_fwd, i.e. the fused shared experts over all m_rows rows of
 * x (model card: the 2 shared experts are active for every token), for
 * batches too small to fill the GPU.  Same results as the dense call up to the
 * order of the fp32 sums: when the product's 128 x 256 tiles would occupy less
 * than half of the 256 compute units, the contraction (H for gate/up, F for
 * down) is split into up to 8 slices computed by separate workgroups into fp32
 * partial products in `ws`, which a second kernel adds in slice order before
 * the SwiGLU (gate/up: act and h, each rounded to bf16 from the fp32 sums) or
 * the bf16 store (down).  Otherwise the call runs the dense call itself and
 * leaves `ws` unused.  Deterministic.
 *   x [m_rows,H], w1 [2F,H], act [m_rows,2F] (nullable), h [m_rows,F],
 *   w2 [H,F], y [m_rows,H]; all bf16, row-major.
 * ws: device workspace of at least moe_dense_fwd_split_workspace_bytes(m_rows,
 * H, F) bytes (0 when no split is taken; ws may then be NULL), 256-byte
 * aligned, rewritten by each call; calls sharing one ws must not overlap.
 * Limits as moe_grouped_gate_up_fwd (H % 64 == 0, F % 32 == 0).
 */
size_t moe_dense_fwd_split_workspace_bytes(int64_t m_rows, int32_t H, int32_t F);
moe_status_t moe_dense_gate_up_fwd_split(int64_t m_rows, int32_t H, int32_t F,
                                         const uint16_t* x, const uint16_t* w1, uint16_t* act,
                                         uint16_t* h, void* ws, size_t ws_bytes, void* stream);
moe_status_t moe_dense_down_fwd_split(int64_t m_rows, int32_t H, int32_t F, const uint16_t* h,
                                      const uint16_t* w2, uint16_t* y, void* ws,
                                      size_t ws_bytes, void* stream);

/*
 * moe_combine - weighted combine of the routed outputs plus the shared output
 * (model card: 6 routed and 2 shared experts active per token):
 *   y[t,:] = y_shared[t,:] + sum_k topk_w[t,k] * y_rows[row_of[t,k],:]
 * fp32 accumulation in k order, one bf16 rounding.  y_shared nullable (zero).
 * y_rows [*,H] bf16; row_of [T,K]; topk_w [T,K]; y_shared, y [T,H] bf16.
 */
moe_status_t moe_combine(int32_t T, int32_t H, int32_t K, const uint16_t* y_rows,
                         const int32_t* row_of, const float* topk_w,
                         const uint16_t* y_shared, uint16_t* y, void* stream);

/*
 * moe_combine_bwd - backward of moe_combine.  The pages time the layer's
 * backward (Technical Report summary, "Key claims" and "Results": the grouped
 * GEMM's forward and backward against Transformer Engine, Table 1) without
 * defining it; every backward entry point computes the true gradient of its
 * forward with the routing decision held fixed and no gradient for the
 * selection bias.  Here, of the combine (model card, "Model Architecture
 * Features": 6 routed and 2 shared experts per token):
 *   dy_rows[row_of[t,k],:] = topk_w[t,k] * dy[t,:]        (bf16)
 *   dg[t,k]                = <dy[t,:], y_rows[row_of[t,k],:]>   (fp32)
 * Padding rows of dy_rows are not written.
 */
moe_status_t moe_combine_bwd(int32_t T, int32_t H, int32_t K, const uint16_t* dy,
                             const uint16_t* y_rows, const int32_t* row_of,
                             const float* topk_w, uint16_t* dy_rows, float* dg,
                             void* stream);

/*
 * moe_grouped_swiglu_bwd - backward of moe_grouped_swiglu_fwd (the backward
 * the Technical Report summary times, "Results", Table 1; the gradient of the
 * SwiGLU experts of the aibase news item's architecture paragraph, routing
 * held fixed) over the same tile-padded segments ("Key claims" / "Method"),
 * with the same segment arguments (offsets/counts/tile_expert NULL = dense
 * single group):
 *   dh        = dy_rows . w2[g]                          (per valid row)
 *   dgate     = dh * up * silu'(gate),  silu'(z) = sig(z)(1 + z(1 - sig(z)))
 *   dup       = dh * silu(gate)
 *   dact      = [dgate | dup]                            (bf16 [m_rows,2F])
 *   dx_rows   = dact . w1[g]                             (bf16 [m_rows,H])
 *   dw2[g]    = dy_rows_g^T . h_g                        (bf16 [G,H,F])
 *   dw1[g]    = dact_g^T . x_rows_g                      (bf16 [G,2F,H])
 * act and h are the forward's outputs.  Sums over rows run over the valid rows
 * of the segment only; a group with no rows gets dw1[g] = dw2[g] = 0.
 */
moe_status_t moe_grouped_swiglu_bwd(int32_t G, int64_t m_rows, int32_t H, int32_t F,
                                    const int32_t* offsets, const int32_t* counts,
                                    const int32_t* tile_expert, const uint16_t* x_rows,
                                    const uint16_t* w1, const uint16_t* w2,
                                    const uint16_t* act, const uint16_t* h,
                                    const uint16_t* dy_rows, uint16_t* dact,
                                    uint16_t* dx_rows, uint16_t* dw1, uint16_t* dw2,
                                    void* stream);

/*
 * The four steps of moe_grouped_swiglu_bwd as entry points of their own (the
 * grouped GEMM's backward of the Technical Report summary, "Results", Table
 * 1: data and weight gradients over the tile-padded segments), same argument
 * meanings; moe_grouped_swiglu_bwd is exactly
 * down_dgrad, gate_up_dgrad, down_wgrad, gate_up_wgrad in that order.  The
 * data gradients and the weight gradients do not depend on each other once
 * dact exists, so a caller may run the weight-gradient steps on another stream.
 *   moe_grouped_down_dgrad    : dact  = SwiGLU-backward(dy_rows . w2[g], act)
 *   moe_grouped_down_wgrad    : dw2[g] = dy_rows_g^T . h_g      (zero for an empty group)
 *   moe_grouped_gate_up_dgrad : dx_rows = dact . w1[g]
 *   moe_grouped_gate_up_wgrad : dw1[g] = dact_g^T . x_rows_g    (zero for an empty group)
 * tile_expert is only validated by the weight-gradient steps.  m_rows == 0 is
 * a no-op for the data-gradient steps; the weight-gradient steps still write
 * zeros.
 */
moe_status_t moe_grouped_down_dgrad(int32_t G, int64_t m_rows, int32_t H, int32_t F,
                                    const int32_t* offsets, const int32_t* counts,
                                    const int32_t* tile_expert, const uint16_t* w2,
                                    const uint16_t* act, const uint16_t* dy_rows,
                                    uint16_t* dact, void* stream);
moe_status_t moe_grouped_down_wgrad(int32_t G, int64_t m_rows, int32_t H, int32_t F,
                                    const int32_t* offsets, const int32_t* counts,
                                    const int32_t* tile_expert, const uint16_t* dy_rows,
                                    const uint16_t* h, uint16_t* dw2, void* stream);
moe_status_t moe_grouped_gate_up_dgrad(int32_t G, int64_t m_rows, int32_t H, int32_t F,
                                       const int32_t* offsets, const int32_t* counts,
                                       const int32_t* tile_expert, const uint16_t* w1,
                                       const uint16_t* dact, uint16_t* dx_rows, void* stream);
moe_status_t moe_grouped_gate_up_wgrad(int32_t G, int64_t m_rows, int32_t H, int32_t F,
                                       const int32_t* offsets, const int32_t* counts,
                                       const int32_t* tile_expert, const uint16_t* dact,
                                       const uint16_t* x_rows, uint16_t* dw1, void* stream);

/*
 * moe_route_bwd - backward of moe_route's weights through the selected scores
 * (the FP32 gating of the Technical Report summary, "Method"; the backward is
 * timed there, "Results", not defined: routing decision held fixed, no bias
 * gradient):
 *   S_t        = sum_j topk_s[t,j],  g = topk_s / S_t
 *   ds[t,k]    = (dg[t,k] - sum_j g[t,j] dg[t,j]) / S_t
 *   dlogit[t,k]= ds[t,k] * s * (1 - s),   s = topk_s[t,k]
 *   dw_router[h,e] = sum over tokens t that selected e of x[t,h] * dlogit   (fp32 [H,E])
 *   dx_router[t,h] = sum_k dlogit[t,k] * w_router[h, topk_idx[t,k]]        (fp32 [T,H])
 * The weight gradient is summed over expert segments in fixed order, so it
 * takes the permutation from moe_permute (row_of, offsets, counts, and
 * src_token, whose entries below offsets[E] name the token of every row) and
 * gathers the token rows from x [T,H] bf16.
 * ws: device workspace of at least moe_route_bwd_workspace_bytes(T,H,E,K).
 */
moe_status_t moe_route_bwd(int32_t T, int32_t H, int32_t E, int32_t K,
                           const uint16_t* x, const float* w_router,
                           const int32_t* topk_idx, const float* topk_s, const float* dg,
                           const int32_t* row_of, const int32_t* offsets,
                           const int32_t* counts, const int32_t* src_token, float* dw_router,
                           float* dx_router, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_permute_bwd - backward of moe_permute's row gather (the tile-padded
 * segments of the Technical Report summary, "Key claims" / "Method"; the
 * backward timed in "Results", routing held fixed): un-permute and add every
 * path of the input gradient:
 *   dx[t,:] = sum_k dx_rows[row_of[t,k],:] + dx_shared[t,:] + dx_router[t,:]
 * fp32 accumulation, one bf16 rounding.  dx_shared (bf16) and dx_router (fp32)
 * are nullable.
 */
moe_status_t moe_permute_bwd(int32_t T, int32_t H, int32_t K, const uint16_t* dx_rows,
                             const int32_t* row_of, const uint16_t* dx_shared,
                             const float* dx_router, uint16_t* dx, void* stream);

/*
 * moe_route_permute_bwd - moe_route_bwd followed by moe_permute_bwd (the
 * backward timed in the Technical Report summary, "Results", routing held
 * fixed), with the router's input gradient added where dx is summed instead
 * of passing through a [T,H] fp32 buffer:
 *   dw_router as moe_route_bwd computes it;
 *   dx[t,:] = sum_k dx_rows[row_of[t,k],:] + dx_shared[t,:] + dx_router[t,:]
 * with dx_router[t,:] formed on the fly exactly as moe_route_bwd forms it, so
 * both outputs equal those of the two calls bit for bit.  Arguments as for
 * the two calls (dx_shared nullable); ws: device workspace of at least
 * moe_route_bwd_workspace_bytes(T,H,E,K) bytes.
 */
moe_status_t moe_route_permute_bwd(int32_t T, int32_t H, int32_t E, int32_t K,
                                   const uint16_t* x, const float* w_router,
                                   const int32_t* topk_idx, const float* topk_s, const float* dg,
                                   const int32_t* row_of, const int32_t* offsets,
                                   const int32_t* counts, const int32_t* src_token,
                                   const uint16_t* dx_rows, const uint16_t* dx_shared,
                                   float* dw_router, uint16_t* dx, void* ws, size_t ws_bytes,
                                   void* stream);

/*
 * Load balancing.  Technical Report summary, "Method": balancing by DeepSeek's
 * auxiliary-loss-free bias update, complemented by a sequence-wise balance
 * loss; model card, "Model Architecture Features": dynamic bias terms.  The
 * pages define neither; the entry points below take DeepSeek's published
 * forms.
 */

/*
 * moe_bias_update - one auxiliary-loss-free bias step from a batch's loads:
 *   bias[e] += gamma * sign(sum_j counts[j] / E - counts[e])
 * An expert above the mean load has its bias lowered by gamma, one below it
 * raised, one exactly at the mean unchanged; the comparison is exact (integer
 * E * counts[e] against the total) and the update is one fp32 addition.
 * counts [E] int32 (moe_permute's counts, or the caller's sum of them over
 * micro-batches or ranks); bias [E] fp32, updated in place; gamma (host) is
 * the step.  E <= 128.
 */
moe_status_t moe_bias_update(int32_t E, const int32_t* counts, float* bias, float gamma,
                             void* stream);

/*
 * moe_seq_balance_fwd - sequence-wise balance loss.  The T tokens are B =
 * T / seq_len consecutive sequences of seq_len tokens.  For sequence b:
 *   s'[t,i]  = scores[t,i] / sum_j scores[t,j]          (all E experts)
 *   P[b,i]   = mean over the sequence's tokens of s'[t,i]
 *   f[b,i]   = E / (K seq_len) * (number of its tokens with i in topk_idx[t,:])
 *   loss_b   = alpha * sum_i f[b,i] P[b,i]
 *   loss[0]  = mean over b of loss_b                     (fp32, device)
 * scores [T,E] fp32 from moe_route; topk_idx [T,K]; seq_f [B,E] fp32 receives
 * f, which moe_seq_balance_bwd takes.  ws: at least
 * moe_seq_balance_workspace_bytes(T,E,seq_len) bytes.  T % seq_len must be 0.
 */
moe_status_t moe_seq_balance_fwd(int32_t T, int32_t E, int32_t K, int32_t seq_len,
                                 const float* scores, const int32_t* topk_idx, float alpha,
                                 float* loss, float* seq_f, void* ws, size_t ws_bytes,
                                 void* stream);

/*
 * moe_seq_balance_bwd - gradient of dloss * loss with respect to the logits,
 * with the selection (and so f) held fixed.  For token t of sequence b, with
 * c_i = dloss * alpha * f[b,i] / (B seq_len) and S = sum_i scores[t,i]:
 *   dlogit[t,e] = (c_e - sum_i c_i scores[t,i] / S) / S * s (1 - s),
 *   s = scores[t,e]                                     (fp32 [T,E], written)
 * dloss: device pointer to the upstream gradient of loss[0] (NULL = 1).
 * The result is dense over all E experts; moe_route_bwd_dense turns it into
 * router-weight and input gradients.
 */
moe_status_t moe_seq_balance_bwd(int32_t T, int32_t E, int32_t K, int32_t seq_len,
                                 const float* scores, const float* seq_f, float alpha,
                                 const float* dloss, float* dlogit, void* stream);

/*
 * moe_route_dlogit - the combine path's logit gradient (moe_route_bwd's, see
 * there), ADDED into a dense logit gradient [T,E] fp32:
 *   dlogit[t, topk_idx[t,k]] += ds[t,k] * s (1 - s),   s = topk_s[t,k]
 * With the balance loss this folds the two logit gradients into one, and a
 * single moe_route_bwd_dense (accumulate = 0) then gives the router weight and
 * input gradients of both, in place of moe_route_bwd followed by
 * moe_route_bwd_dense (accumulate = 1).  The K experts of a token are
 * distinct, so every entry has one writer; T == 0 is a no-op.
 */
moe_status_t moe_route_dlogit(int32_t T, int32_t E, int32_t K, const int32_t* topk_idx,
                              const float* topk_s, const float* dg, float* dlogit,
                              void* stream);

/*
 * moe_route_bwd_dense - router gradients of a dense logit gradient, ADDED to
 * the outputs when accumulate != 0 (so it composes with moe_route_bwd, which
 * writes them), written over them when accumulate == 0:
 *   dw_router[h,e] (+)= sum_t x[t,h] * dlogit[t,e]      (fp32 [H,E])
 *   dx_router[t,h] (+)= sum_e dlogit[t,e] * w_router[h,e] (fp32 [T,H])
 * x [T,H] bf16 in token order; dlogit [T,E] fp32; dx_router 16-byte aligned.
 * The weight gradient runs over token slices of x addressed with 32-bit
 * offsets; T whose largest slice reaches 4 GiB (beyond about 5.4 million
 * tokens at H = 5120, E = 128) is rejected with MOE_ERR_UNSUPPORTED_SHAPE.
 * The products run on the bf16 matrix cores with every fp32 operand split
 * exactly into three bf16 parts (fp32-level accuracy).  Every sum runs in a
 * fixed order.  ws: at least moe_route_bwd_dense_workspace_bytes(T,H,E) bytes,
 * 256-byte aligned.  T == 0 leaves the outputs as they are when accumulating
 * and writes a zero dw_router otherwise.
 */
moe_status_t moe_route_bwd_dense(int32_t T, int32_t H, int32_t E, const uint16_t* x,
                                 const float* w_router, const float* dlogit, float* dw_router,
                                 float* dx_router, int32_t accumulate, void* ws, size_t ws_bytes,
                                 void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
