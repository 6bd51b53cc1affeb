// Internal launchers of the MoE kernels (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kAlign = 128;  // grouped-GEMM row tile = segment alignment

size_t route_workspace_bytes(int T, int H, int E);
hipError_t launch_route(int T, int H, int E, int K, const uint16_t* x, const float* w_router,
                        const float* bias, int32_t* topk_idx, float* topk_w, float* topk_s,
                        float* scores, void* ws, hipStream_t s);

// moe_permute's data-check block: the first kPermuteStatusBytes of its
// workspace, four int32 words (flags, rejected tokens, first rejected token,
// kPermuteStatusMagic), rewritten by every call
constexpr size_t kPermuteStatusBytes = 256;
constexpr int32_t kPermuteStatusMagic = 0x4D4F4550;
size_t permute_workspace_bytes(int T, int E);
hipError_t launch_permute(int T, int H, int E, int K, int align, const int32_t* topk_idx,
                          const uint16_t* x, int64_t m_cap, int32_t* counts, int32_t* offsets,
                          int32_t* row_of, int32_t* src_token, int32_t* tile_expert,
                          uint16_t* x_rows, void* ws, int32_t* status_out, hipStream_t s);
// the same without a workspace: the kernels use a file-scope device array
int permute_noalloc_max_tokens();
hipError_t launch_permute_noalloc(int T, int H, int E, int K, int align, const int32_t* topk_idx,
                                  const uint16_t* x, int64_t m_cap, int32_t* counts,
                                  int32_t* offsets, int32_t* row_of, int32_t* src_token,
                                  int32_t* tile_expert, uint16_t* x_rows, int32_t* status,
                                  hipStream_t s);

hipError_t launch_gemm_gate_up(int G, int64_t m_rows, int H, int F, const int32_t* offsets,
                               const int32_t* counts, const int32_t* tile_expert,
                               const uint16_t* x_rows, const uint16_t* w1, uint16_t* act,
                               uint16_t* h, hipStream_t s);
hipError_t launch_gemm_down(int G, int64_t m_rows, int H, int F, const int32_t* offsets,
                            const int32_t* counts, const int32_t* tile_expert,
                            const uint16_t* h, const uint16_t* w2, uint16_t* y_rows,
                            hipStream_t s);
size_t dense_fwd_split_workspace_bytes(int64_t m_rows, int H, int F);
hipError_t launch_dense_gate_up_split(int64_t m_rows, int H, int F, const uint16_t* x,
                                      const uint16_t* w1, uint16_t* act, uint16_t* h, void* ws,
                                      hipStream_t s);
hipError_t launch_dense_down_split(int64_t m_rows, int H, int F, const uint16_t* h,
                                   const uint16_t* w2, uint16_t* y, void* ws, hipStream_t s);
hipError_t launch_gemm_dgrad_down(int G, int64_t m_rows, int H, int F, const int32_t* offsets,
                                  const int32_t* counts, const int32_t* tile_expert,
                                  const uint16_t* dy_rows, const uint16_t* w2,
                                  const uint16_t* act, uint16_t* dact, hipStream_t s);
hipError_t launch_gemm_dgrad_up(int G, int64_t m_rows, int H, int F, const int32_t* offsets,
                                const int32_t* counts, const int32_t* tile_expert,
                                const uint16_t* dact, const uint16_t* w1, uint16_t* dx_rows,
                                hipStream_t s);
hipError_t launch_gemm_wgrad_down(int G, int64_t m_rows, int H, int F, const int32_t* offsets,
                                  const int32_t* counts, const uint16_t* dy_rows,
                                  const uint16_t* h, uint16_t* dw2, hipStream_t s);
hipError_t launch_gemm_wgrad_up(int G, int64_t m_rows, int H, int F, const int32_t* offsets,
                                const int32_t* counts, const uint16_t* dact,
                                const uint16_t* x_rows, uint16_t* dw1, hipStream_t s);

hipError_t launch_gemm_f32_nt(int64_t M, int N, int K, const uint16_t* A, int lda,
                              const uint16_t* B, int ldb, float* C, int ldc, bool accumulate,
                              hipStream_t s);
hipError_t launch_gemm_f32_tn_grouped(int G, const int32_t* offsets, const int32_t* counts,
                                      int64_t rows, int M, int N, const uint16_t* A, int lda,
                                      const uint16_t* B, int ldb, float* C, int ldc,
                                      int64_t strideC, hipStream_t s);

hipError_t launch_combine(int T, int H, int K, const uint16_t* y_rows, const int32_t* row_of,
                          const float* topk_w, const uint16_t* y_shared, uint16_t* y,
                          hipStream_t s);
hipError_t launch_combine_bwd(int T, int H, int K, const uint16_t* dy, const uint16_t* y_rows,
                              const int32_t* row_of, const float* topk_w, uint16_t* dy_rows,
                              float* dg, hipStream_t s);
hipError_t launch_unpermute_add(int T, int H, int K, const uint16_t* dx_rows,
                                const int32_t* row_of, const uint16_t* dx_shared,
                                const float* dx_router, uint16_t* dx, hipStream_t s);
size_t route_bwd_workspace_bytes(int64_t m_cap, int H, int E);
hipError_t launch_route_bwd(int T, int H, int E, int K, const uint16_t* x,
                            const float* w_router, const int32_t* topk_idx, const float* topk_s,
                            const float* dg, const int32_t* row_of, const int32_t* offsets,
                            const int32_t* counts, const int32_t* src_token, float* dw_router,
                            float* dx_router, void* ws, hipStream_t s);
// launch_route_bwd without materialising dx_router, then the un-permute-add
// with the router's input gradient formed from ws
hipError_t launch_route_permute_bwd(int T, int H, int E, int K, const uint16_t* x,
                                    const float* w_router, const int32_t* topk_idx,
                                    const float* topk_s, const float* dg, const int32_t* row_of,
                                    const int32_t* offsets, const int32_t* counts,
                                    const int32_t* src_token, const uint16_t* dx_rows,
                                    const uint16_t* dx_shared, float* dw_router, uint16_t* dx,
                                    void* ws, hipStream_t s);


hipError_t launch_bias_update(int E, const int32_t* counts, float* bias, float gamma,
                              hipStream_t s);
size_t seq_balance_workspace_bytes(int T, int E, int L);
hipError_t launch_seq_balance_fwd(int T, int E, int K, int L, const float* scores,
                                  const int32_t* topk_idx, float alpha, float* loss, float* seq_f,
                                  void* ws, hipStream_t s);
hipError_t launch_seq_balance_bwd(int T, int E, int L, const float* scores, const float* seq_f,
                                  float alpha, const float* dloss, float* dlogit, hipStream_t s);
size_t route_bwd_dense_workspace_bytes(int T, int H, int E);
// rows of the largest token slice of the dense router weight gradient
int64_t route_bwd_dense_slice_rows(int T, int H, int E);
hipError_t launch_route_dlogit(int T, int E, int K, const int32_t* topk_idx, const float* topk_s,
                               const float* dg, float* dlogit, hipStream_t s);
hipError_t launch_route_bwd_dense(int T, int H, int E, const uint16_t* x, const float* w_router,
                                  const float* dlogit, float* dw_router, float* dx_router,
                                  bool accumulate, void* ws, hipStream_t s);

}  // namespace moe
