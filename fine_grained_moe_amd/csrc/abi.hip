// C ABI of the MoE layer library: host-side argument checks, then launches.
// Every check runs before the first HIP call, so a rejected call launches
// nothing and touches no device state.
#include <stdio.h>
#include <stdint.h>
#include <string.h>

#include "../../include/moe.h"
#include "kernels.h"

namespace {

thread_local char g_last_error[256] = "";

moe_status_t fail(moe_status_t st, const char* fn, const char* what) {
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s", fn, what);
  return st;
}

moe_status_t hip_status(hipError_t e, const char* fn) {
  if (e == hipSuccess) return MOE_OK;
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s", fn, hipGetErrorString(e));
  return MOE_ERR_HIP;
}

#define REQUIRE(cond, st, msg) \
  do {                         \
    if (!(cond)) return fail(st, __func__, msg); \
  } while (0)

// every device pointer is read or written with 16-byte vector accesses (rows
// are multiples of 128 bytes, so a 16-byte aligned base aligns every row);
// workspaces are carved into 256-byte aligned parts.  NULL passes.
template <class... P>
bool aligned(uintptr_t a, P... p) {
  return ((((uintptr_t)p) % a == 0) && ...);
}
#define REQUIRE_ALIGNED(...)                                            \
  REQUIRE(aligned(16, __VA_ARGS__), MOE_ERR_INVALID_ARGUMENT,           \
          "device pointers must be 16-byte aligned")
#define REQUIRE_WS_ALIGNED(ws) \
  REQUIRE(aligned(256, ws), MOE_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned")

// Widths the kernels address with 32-bit buffer offsets: a row tile of up to
// 256 rows of H or 2F bf16 values, one expert's weights (4 F H bytes) and the
// router's re-encoded weight stay well below 4 GiB within these limits.
constexpr int32_t kMaxWidth = 65536;

moe_status_t check_dims(const char* fn, int32_t T, int32_t H, int32_t E, int32_t K) {
  if (T < 0 || H <= 0 || E <= 0 || K <= 0) return fail(MOE_ERR_INVALID_ARGUMENT, fn, "T<0 or H,E,K<=0");
  if (K > E) return fail(MOE_ERR_INVALID_ARGUMENT, fn, "K > E");
  if (E > 128 || K > 16) return fail(MOE_ERR_UNSUPPORTED_SHAPE, fn, "E > 128 or K > 16");
  if (H % 64 != 0) return fail(MOE_ERR_UNSUPPORTED_SHAPE, fn, "H % 64 != 0");
  if (H > kMaxWidth) return fail(MOE_ERR_UNSUPPORTED_SHAPE, fn, "H > 65536");
  if ((int64_t)T * K >= (int64_t)1 << 30) return fail(MOE_ERR_UNSUPPORTED_SHAPE, fn, "T*K too large");
  return MOE_OK;
}

int64_t capacity(int32_t T, int32_t E, int32_t K) {
  const int64_t a = moe::kAlign;
  int64_t n = (int64_t)T * K + (int64_t)E * (a - 1);
  return (n + a - 1) / a * a;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOE_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_last_error; }

int32_t moe_align(void) { return moe::kAlign; }

int64_t moe_capacity_rows(int32_t T, int32_t E, int32_t K) {
  if (T < 0 || E <= 0 || K <= 0) return -1;
  return capacity(T, E, K);
}

size_t moe_route_workspace_bytes(int32_t T, int32_t H, int32_t E) {
  if (T < 0 || H <= 0 || H % 64 != 0 || E <= 0 || E > 128) return 0;
  return moe::route_workspace_bytes(T, H, E);
}

size_t moe_permute_workspace_bytes(int32_t T, int32_t E, int32_t K) {
  (void)K;
  if (T < 0 || E <= 0) return 0;
  return moe::permute_workspace_bytes(T, E);
}

size_t moe_route_bwd_workspace_bytes(int32_t T, int32_t H, int32_t E, int32_t K) {
  if (T < 0 || H <= 0 || E <= 0 || K <= 0) return 0;
  return moe::route_bwd_workspace_bytes(capacity(T, E, K), H, E);
}

size_t moe_seq_balance_workspace_bytes(int32_t T, int32_t E, int32_t seq_len) {
  if (T < 0 || E <= 0 || E > 128 || seq_len <= 0 || T % seq_len != 0) return 0;
  return moe::seq_balance_workspace_bytes(T, E, seq_len);
}

size_t moe_route_bwd_dense_workspace_bytes(int32_t T, int32_t H, int32_t E) {
  if (T < 0 || H <= 0 || E <= 0 || E > 128) return 0;
  return moe::route_bwd_dense_workspace_bytes(T, H, E);
}

moe_status_t moe_permute_check(const int32_t* words) {
  REQUIRE(words != nullptr, MOE_ERR_INVALID_ARGUMENT, "null pointer");
  REQUIRE(words[3] == moe::kPermuteStatusMagic, MOE_ERR_INVALID_ARGUMENT,
          "not a status block written by moe_permute");
  const int32_t flags = words[0], n = words[1], first = words[2];
  if (flags == 0 && n == 0 && first == -1) return MOE_OK;
  REQUIRE(flags != 0 && (flags & ~3) == 0 && n > 0 && first >= 0, MOE_ERR_INVALID_ARGUMENT,
          "corrupt status block");
  snprintf(g_last_error, sizeof(g_last_error),
           "moe_permute rejected %d token(s), the first being token %d: %s%s%s", n, first,
           (flags & 1) ? "an expert id outside [0,E)" : "", flags == 3 ? " and " : "",
           (flags & 2) ? "an expert id repeated within a token" : "");
  return MOE_ERR_INVALID_ARGUMENT;
}

moe_status_t moe_route(int32_t T, int32_t H, int32_t E, int32_t K, const uint16_t* x,
                       const float* w_router, const float* bias, int32_t* topk_idx,
                       float* topk_w, float* topk_s, float* scores, void* ws, size_t ws_bytes,
                       void* stream) {
  moe_status_t st = check_dims(__func__, T, H, E, K);
  if (st) return st;
  if (T == 0) return MOE_OK;
  REQUIRE(x && w_router && bias && topk_idx && topk_w, MOE_ERR_INVALID_ARGUMENT, "null pointer");
  REQUIRE(ws != nullptr && ws_bytes >= moe_route_workspace_bytes(T, H, E),
          MOE_ERR_WORKSPACE_TOO_SMALL, "workspace too small");
  REQUIRE_ALIGNED(x, w_router, bias, topk_idx, topk_w, topk_s, scores);
  REQUIRE_WS_ALIGNED(ws);
  return hip_status(moe::launch_route(T, H, E, K, x, w_router, bias, topk_idx, topk_w, topk_s,
                                      scores, ws, (hipStream_t)stream),
                    __func__);
}

moe_status_t moe_permute(int32_t T, int32_t H, int32_t E, int32_t K, int32_t align,
                         const int32_t* topk_idx, const uint16_t* x, int64_t m_cap,
                         int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* src_token,
                         int32_t* tile_expert, uint16_t* x_rows, void* ws, size_t ws_bytes,
                         void* stream) {
  moe_status_t st = check_dims(__func__, T, H, E, K);
  if (st) return st;
  REQUIRE(align == moe::kAlign, MOE_ERR_UNSUPPORTED_SHAPE, "align != moe_align()");
  REQUIRE(m_cap >= capacity(T, E, K) && m_cap % align == 0 && m_cap < ((int64_t)1 << 31),
          MOE_ERR_INVALID_ARGUMENT, "m_cap below moe_capacity_rows or not a multiple of align");
  REQUIRE(counts && offsets && src_token && tile_expert, MOE_ERR_INVALID_ARGUMENT, "null pointer");
  REQUIRE(T == 0 || (topk_idx && x && row_of && x_rows), MOE_ERR_INVALID_ARGUMENT, "null pointer");
  const size_t need = moe::permute_workspace_bytes(T, E);
  REQUIRE(ws_bytes >= need && (need == 0 || ws != nullptr), MOE_ERR_WORKSPACE_TOO_SMALL,
          "workspace too small");
  REQUIRE_ALIGNED(topk_idx, x, counts, offsets, row_of, src_token, tile_expert, x_rows);
  REQUIRE_WS_ALIGNED(ws);
  return hip_status(moe::launch_permute(T, H, E, K, align, topk_idx, x, m_cap, counts, offsets,
                                        row_of, src_token, tile_expert, x_rows, ws, nullptr,
                                        (hipStream_t)stream),
                    __func__);
}

int32_t moe_permute_noalloc_max_tokens(void) { return moe::permute_noalloc_max_tokens(); }

moe_status_t moe_permute_noalloc(int32_t T, int32_t H, int32_t E, int32_t K, int32_t align,
                                 const int32_t* topk_idx, const uint16_t* x, int64_t m_cap,
                                 int32_t* counts, int32_t* offsets, int32_t* row_of,
                                 int32_t* src_token, int32_t* tile_expert, uint16_t* x_rows,
                                 int32_t* status, void* stream) {
  moe_status_t st = check_dims(__func__, T, H, E, K);
  if (st) return st;
  REQUIRE(T <= moe::permute_noalloc_max_tokens(), MOE_ERR_UNSUPPORTED_SHAPE,
          "T > moe_permute_noalloc_max_tokens() (the size of its static scratch)");
  REQUIRE(align == moe::kAlign, MOE_ERR_UNSUPPORTED_SHAPE, "align != moe_align()");
  REQUIRE(m_cap >= capacity(T, E, K) && m_cap % align == 0 && m_cap < ((int64_t)1 << 31),
          MOE_ERR_INVALID_ARGUMENT, "m_cap below moe_capacity_rows or not a multiple of align");
  REQUIRE(counts && offsets && src_token && tile_expert, MOE_ERR_INVALID_ARGUMENT, "null pointer");
  REQUIRE(T == 0 || (topk_idx && x && row_of && x_rows), MOE_ERR_INVALID_ARGUMENT, "null pointer");
  REQUIRE_ALIGNED(topk_idx, x, counts, offsets, row_of, src_token, tile_expert, x_rows, status);
  return hip_status(moe::launch_permute_noalloc(T, H, E, K, align, topk_idx, x, m_cap, counts,
                                                offsets, row_of, src_token, tile_expert, x_rows,
                                                status, (hipStream_t)stream),
                    __func__);
}

static moe_status_t check_grouped(const char* fn, int32_t G, int64_t m_rows, int32_t H, int32_t F,
                                  const int32_t* offsets, const int32_t* counts,
                                  const int32_t* tile_expert) {
  if (G <= 0 || m_rows < 0 || H <= 0 || F <= 0) return fail(MOE_ERR_INVALID_ARGUMENT, fn, "G,H,F<=0 or m_rows<0");
  if (H % 64 != 0 || F % 32 != 0) return fail(MOE_ERR_UNSUPPORTED_SHAPE, fn, "H % 64 or F % 32 != 0");
  if (H > kMaxWidth || F > kMaxWidth || (int64_t)F * H >= ((int64_t)1 << 30))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, fn, "H or F > 65536, or an expert's weights >= 4 GiB");
  if (m_rows >= ((int64_t)1 << 31)) return fail(MOE_ERR_UNSUPPORTED_SHAPE, fn, "m_rows too large");
  const bool dense = offsets == nullptr && counts == nullptr && tile_expert == nullptr;
  const bool grouped = offsets != nullptr && counts != nullptr && tile_expert != nullptr;
  if (!dense && !grouped)
    return fail(MOE_ERR_INVALID_ARGUMENT, fn, "offsets/counts/tile_expert must be all set or all NULL");
  if (dense && G != 1) return fail(MOE_ERR_INVALID_ARGUMENT, fn, "dense call needs G == 1");
  if (grouped && m_rows % moe::kAlign != 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, fn, "grouped m_rows must be a multiple of moe_align()");
  return MOE_OK;
}

// The weight gradients address a whole segment (an expert's rows, or the m_rows
// of a dense call) through one buffer resource with 32-bit byte offsets, so a
// segment of rows of up to max(H, 2F) bf16 values must stay below 4 GiB.  No
// segment holds more than m_rows rows.
static moe_status_t check_wgrad_rows(const char* fn, int64_t m_rows, int32_t H, int32_t F) {
  const int64_t row_bytes = 2 * (int64_t)(H > 2 * F ? H : 2 * F);
  if (m_rows * row_bytes >= ((int64_t)1 << 32))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, fn, "m_rows * row bytes >= 4 GiB (weight-gradient segment)");
  return MOE_OK;
}

moe_status_t moe_grouped_swiglu_fwd(int32_t G, int64_t m_rows, int32_t H, int32_t F,
                                    const int32_t* offsets, const int32_t* counts,
                                    const int32_t* tile_expert, const uint16_t* x_rows,
                                    const uint16_t* w1, const uint16_t* w2, uint16_t* act,
                                    uint16_t* h, uint16_t* y_rows, void* stream) {
  moe_status_t st = check_grouped(__func__, G, m_rows, H, F, offsets, counts, tile_expert);
  if (st) return st;
  if (m_rows == 0) return MOE_OK;
  REQUIRE(x_rows && w1 && w2 && h && y_rows, MOE_ERR_INVALID_ARGUMENT, "null pointer");
  REQUIRE_ALIGNED(offsets, counts, tile_expert, x_rows, w1, w2, act, h, y_rows);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = moe::launch_gemm_gate_up(G, m_rows, H, F, offsets, counts, tile_expert, x_rows,
                                          w1, act, h, s);
  if (e == hipSuccess)
    e = moe::launch_gemm_down(G, m_rows, H, F, offsets, counts, tile_expert, h, w2, y_rows, s);
  return hip_status(e, __func__);
}

moe_status_t moe_grouped_gate_up_fwd(int32_t G, int64_t m_rows, int32_t H, int32_t F,
                                     const int32_t* offsets, const int32_t* counts,
                                     const int32_t* tile_expert, const uint16_t* x_rows,
                                     const uint16_t* w1, uint16_t* act, uint16_t* h,
                                     void* stream) {
  moe_status_t st = check_grouped(__func__, G, m_rows, H, F, offsets, counts, tile_expert);
  if (st) return st;
  if (m_rows == 0) return MOE_OK;
  REQUIRE(x_rows && w1 && h, MOE_ERR_INVALID_ARGUMENT, "null pointer");
  REQUIRE_ALIGNED(offsets, counts, tile_expert, x_rows, w1, act, h);
  return hip_status(moe::launch_gemm_gate_up(G, m_rows, H, F, offsets, counts, tile_expert,
                                             x_rows, w1, act, h, (hipStream_t)stream),
                    __func__);
}

moe_status_t moe_grouped_down_fwd(int32_t G, int64_t m_rows, int32_t H, int32_t F,
                                  const int32_t* offsets, const int32_t* counts,
                                  const int32_t* tile_expert, const uint16_t* h,
                                  const uint16_t* w2, uint16_t* y_rows, void* stream) {
  moe_status_t st = check_grouped(__func__, G, m_rows, H, F, offsets, counts, tile_expert);
  if (st) return st;
  if (m_rows == 0) return MOE_OK;
  REQUIRE(h && w2 && y_rows, MOE_ERR_INVALID_ARGUMENT, "null pointer");
  REQUIRE_ALIGNED(offsets, counts, tile_expert, h, w2, y_rows);
  return hip_status(moe::launch_gemm_down(G, m_rows, H, F, offsets, counts, tile_expert, h, w2,
                                          y_rows, (hipStream_t)stream),
                    __func__);
}

size_t moe_dense_fwd_split_workspace_bytes(int64_t m_rows, int32_t H, int32_t F) {
  if (m_rows <= 0 || H <= 0 || F <= 0) return 0;
  return moe::dense_fwd_split_workspace_bytes(m_rows, H, F);
}

moe_status_t moe_dense_gate_up_fwd_split(int64_t m_rows, int32_t H, int32_t F, const uint16_t* x,
                                         const uint16_t* w1, uint16_t* act, uint16_t* h, void* ws,
                                         size_t ws_bytes, void* stream) {
  moe_status_t st = check_grouped(__func__, 1, m_rows, H, F, nullptr, nullptr, nullptr);
  if (st) return st;
  if (m_rows == 0) return MOE_OK;
  REQUIRE(x && w1 && h, MOE_ERR_INVALID_ARGUMENT, "null pointer");
  REQUIRE_ALIGNED(x, w1, act, h);
  REQUIRE_WS_ALIGNED(ws);
  const size_t need = moe::dense_fwd_split_workspace_bytes(m_rows, H, F);
  REQUIRE(ws_bytes >= need && (need == 0 || ws), MOE_ERR_WORKSPACE_TOO_SMALL, "workspace too small");
  return hip_status(
      moe::launch_dense_gate_up_split(m_rows, H, F, x, w1, act, h, ws, (hipStream_t)stream),
      __func__);
}

moe_status_t moe_dense_down_fwd_split(int64_t m_rows, int32_t H, int32_t F, const uint16_t* h,
                                      const uint16_t* w2, uint16_t* y, void* ws, size_t ws_bytes,
                                      void* stream) {
  moe_status_t st = check_grouped(__func__, 1, m_rows, H, F, nullptr, nullptr, nullptr);
  if (st) return st;
  if (m_rows == 0) return MOE_OK;
  REQUIRE(h && w2 && y, MOE_ERR_INVALID_ARGUMENT, "null pointer");
  REQUIRE_ALIGNED(h, w2, y);
  REQUIRE_WS_ALIGNED(ws);
  const size_t need = moe::dense_fwd_split_workspace_bytes(m_rows, H, F);
  REQUIRE(ws_bytes >= need && (need == 0 || ws), MOE_ERR_WORKSPACE_TOO_SMALL, "workspace too small");
  return hip_status(moe::launch_dense_down_split(m_rows, H, F, h, w2, y, ws, (hipStream_t)stream),
                    __func__);
}

moe_status_t moe_combine(int32_t T, int32_t H, int32_t K, const uint16_t* y_rows,
                         const int32_t* row_of, const float* topk_w, const uint16_t* y_shared,
                         uint16_t* y, void* stream) {
  REQUIRE(T >= 0 && H > 0 && K > 0, MOE_ERR_INVALID_ARGUMENT, "T<0 or H,K<=0");
  REQUIRE(H % 64 == 0 && K <= 16, MOE_ERR_UNSUPPORTED_SHAPE, "H % 64 != 0 or K > 16");
  if (T == 0) return MOE_OK;
  REQUIRE(y_rows && row_of && topk_w && y, MOE_ERR_INVALID_ARGUMENT, "null pointer");
  REQUIRE_ALIGNED(y_rows, row_of, topk_w, y_shared, y);
  return hip_status(moe::launch_combine(T, H, K, y_rows, row_of, topk_w, y_shared, y,
                                        (hipStream_t)stream),
                    __func__);
}

moe_status_t moe_combine_bwd(int32_t T, int32_t H, int32_t K, const uint16_t* dy,
                             const uint16_t* y_rows, const int32_t* row_of, const float* topk_w,
                             uint16_t* dy_rows, float* dg, void* stream) {
  REQUIRE(T >= 0 && H > 0 && K > 0, MOE_ERR_INVALID_ARGUMENT, "T<0 or H,K<=0");
  REQUIRE(H % 64 == 0 && K <= 16, MOE_ERR_UNSUPPORTED_SHAPE, "H % 64 != 0 or K > 16");
  if (T == 0) return MOE_OK;
  REQUIRE(dy && y_rows && row_of && topk_w && dy_rows && dg, MOE_ERR_INVALID_ARGUMENT,
          "null pointer");
  REQUIRE_ALIGNED(dy, y_rows, row_of, topk_w, dy_rows, dg);
  return hip_status(moe::launch_combine_bwd(T, H, K, dy, y_rows, row_of, topk_w, dy_rows, dg,
                                            (hipStream_t)stream),
                    __func__);
}

moe_status_t moe_grouped_swiglu_bwd(int32_t G, int64_t m_rows, int32_t H, int32_t F,
                                    const int32_t* offsets, const int32_t* counts,
                                    const int32_t* tile_expert, const uint16_t* x_rows,
                                    const uint16_t* w1, const uint16_t* w2, const uint16_t* act,
                                    const uint16_t* h, const uint16_t* dy_rows, uint16_t* dact,
                                    uint16_t* dx_rows, uint16_t* dw1, uint16_t* dw2,
                                    void* stream) {
  moe_status_t st = check_grouped(__func__, G, m_rows, H, F, offsets, counts, tile_expert);
  if (st) return st;
  st = check_wgrad_rows(__func__, m_rows, H, F);
  if (st) return st;
  REQUIRE(x_rows && w1 && w2 && act && h && dy_rows && dact && dx_rows && dw1 && dw2,
          MOE_ERR_INVALID_ARGUMENT, "null pointer");
  REQUIRE_ALIGNED(offsets, counts, tile_expert, x_rows, w1, w2, act, h, dy_rows, dact, dx_rows,
                  dw1, dw2);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (m_rows > 0) {
    e = moe::launch_gemm_dgrad_down(G, m_rows, H, F, offsets, counts, tile_expert, dy_rows, w2,
                                    act, dact, s);
    if (e == hipSuccess)
      e = moe::launch_gemm_dgrad_up(G, m_rows, H, F, offsets, counts, tile_expert, dact, w1,
                                    dx_rows, s);
  }
  // weight gradients are written for every group, also when it has no rows
  if (e == hipSuccess)
    e = moe::launch_gemm_wgrad_down(G, m_rows, H, F, offsets, counts, dy_rows, h, dw2, s);
  if (e == hipSuccess)
    e = moe::launch_gemm_wgrad_up(G, m_rows, H, F, offsets, counts, dact, x_rows, dw1, s);
  return hip_status(e, __func__);
}

moe_status_t moe_grouped_down_dgrad(int32_t G, int64_t m_rows, int32_t H, int32_t F,
                                    const int32_t* offsets, const int32_t* counts,
                                    const int32_t* tile_expert, const uint16_t* w2,
                                    const uint16_t* act, const uint16_t* dy_rows,
                                    uint16_t* dact, void* stream) {
  moe_status_t st = check_grouped(__func__, G, m_rows, H, F, offsets, counts, tile_expert);
  if (st) return st;
  if (m_rows == 0) return MOE_OK;
  REQUIRE(w2 && act && dy_rows && dact, MOE_ERR_INVALID_ARGUMENT, "null pointer");
  REQUIRE_ALIGNED(offsets, counts, tile_expert, w2, act, dy_rows, dact);
  return hip_status(moe::launch_gemm_dgrad_down(G, m_rows, H, F, offsets, counts, tile_expert,
                                                dy_rows, w2, act, dact, (hipStream_t)stream),
                    __func__);
}

moe_status_t moe_grouped_down_wgrad(int32_t G, int64_t m_rows, int32_t H, int32_t F,
                                    const int32_t* offsets, const int32_t* counts,
                                    const int32_t* tile_expert, const uint16_t* dy_rows,
                                    const uint16_t* h, uint16_t* dw2, void* stream) {
  moe_status_t st = check_grouped(__func__, G, m_rows, H, F, offsets, counts, tile_expert);
  if (st) return st;
  st = check_wgrad_rows(__func__, m_rows, H, F);
  if (st) return st;
  REQUIRE(dy_rows && h && dw2, MOE_ERR_INVALID_ARGUMENT, "null pointer");
  REQUIRE_ALIGNED(offsets, counts, tile_expert, dy_rows, h, dw2);
  return hip_status(moe::launch_gemm_wgrad_down(G, m_rows, H, F, offsets, counts, dy_rows, h, dw2,
                                                (hipStream_t)stream),
                    __func__);
}

moe_status_t moe_grouped_gate_up_dgrad(int32_t G, int64_t m_rows, int32_t H, int32_t F,
                                       const int32_t* offsets, const int32_t* counts,
                                       const int32_t* tile_expert, const uint16_t* w1,
                                       const uint16_t* dact, uint16_t* dx_rows, void* stream) {
  moe_status_t st = check_grouped(__func__, G, m_rows, H, F, offsets, counts, tile_expert);
  if (st) return st;
  if (m_rows == 0) return MOE_OK;
  REQUIRE(w1 && dact && dx_rows, MOE_ERR_INVALID_ARGUMENT, "null pointer");
  REQUIRE_ALIGNED(offsets, counts, tile_expert, w1, dact, dx_rows);
  return hip_status(moe::launch_gemm_dgrad_up(G, m_rows, H, F, offsets, counts, tile_expert, dact,
                                              w1, dx_rows, (hipStream_t)stream),
                    __func__);
}

moe_status_t moe_grouped_gate_up_wgrad(int32_t G, int64_t m_rows, int32_t H, int32_t F,
                                       const int32_t* offsets, const int32_t* counts,
                                       const int32_t* tile_expert, const uint16_t* dact,
                                       const uint16_t* x_rows, uint16_t* dw1, void* stream) {
  moe_status_t st = check_grouped(__func__, G, m_rows, H, F, offsets, counts, tile_expert);
  if (st) return st;
  st = check_wgrad_rows(__func__, m_rows, H, F);
  if (st) return st;
  REQUIRE(dact && x_rows && dw1, MOE_ERR_INVALID_ARGUMENT, "null pointer");
  REQUIRE_ALIGNED(offsets, counts, tile_expert, dact, x_rows, dw1);
  return hip_status(moe::launch_gemm_wgrad_up(G, m_rows, H, F, offsets, counts, dact, x_rows, dw1,
                                              (hipStream_t)stream),
                    __func__);
}

moe_status_t moe_route_bwd(int32_t T, int32_t H, int32_t E, int32_t K, const uint16_t* x,
                           const float* w_router, const int32_t* topk_idx, const float* topk_s,
                           const float* dg, const int32_t* row_of, const int32_t* offsets,
                           const int32_t* counts, const int32_t* src_token, float* dw_router,
                           float* dx_router, void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = check_dims(__func__, T, H, E, K);
  if (st) return st;
  REQUIRE(w_router && offsets && counts && dw_router, MOE_ERR_INVALID_ARGUMENT, "null pointer");
  REQUIRE(T == 0 || (x && topk_idx && topk_s && dg && row_of && src_token && dx_router),
          MOE_ERR_INVALID_ARGUMENT, "null pointer");
  REQUIRE(ws != nullptr && ws_bytes >= moe_route_bwd_workspace_bytes(T, H, E, K),
          MOE_ERR_WORKSPACE_TOO_SMALL, "workspace too small");
  REQUIRE_ALIGNED(x, w_router, topk_idx, topk_s, dg, row_of, offsets, counts, src_token, dw_router,
                  dx_router);
  REQUIRE_WS_ALIGNED(ws);
  // T == 0 still writes the (zero) router weight gradient
  return hip_status(moe::launch_route_bwd(T, H, E, K, x, w_router, topk_idx, topk_s, dg, row_of,
                                          offsets, counts, src_token, dw_router, dx_router, ws,
                                          (hipStream_t)stream),
                    __func__);
}

moe_status_t moe_permute_bwd(int32_t T, int32_t H, int32_t K, const uint16_t* dx_rows,
                             const int32_t* row_of, const uint16_t* dx_shared,
                             const float* dx_router, uint16_t* dx, void* stream) {
  REQUIRE(T >= 0 && H > 0 && K > 0, MOE_ERR_INVALID_ARGUMENT, "T<0 or H,K<=0");
  REQUIRE(H % 64 == 0 && K <= 16, MOE_ERR_UNSUPPORTED_SHAPE, "H % 64 != 0 or K > 16");
  if (T == 0) return MOE_OK;
  REQUIRE(dx_rows && row_of && dx, MOE_ERR_INVALID_ARGUMENT, "null pointer");
  REQUIRE_ALIGNED(dx_rows, row_of, dx_shared, dx_router, dx);
  return hip_status(moe::launch_unpermute_add(T, H, K, dx_rows, row_of, dx_shared, dx_router, dx,
                                              (hipStream_t)stream),
                    __func__);
}

moe_status_t moe_route_permute_bwd(int32_t T, int32_t H, int32_t E, int32_t K, const uint16_t* x,
                                   const float* w_router, const int32_t* topk_idx,
                                   const float* topk_s, const float* dg, const int32_t* row_of,
                                   const int32_t* offsets, const int32_t* counts,
                                   const int32_t* src_token, const uint16_t* dx_rows,
                                   const uint16_t* dx_shared, float* dw_router, uint16_t* dx,
                                   void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = check_dims(__func__, T, H, E, K);
  if (st) return st;
  REQUIRE(w_router && offsets && counts && dw_router, MOE_ERR_INVALID_ARGUMENT, "null pointer");
  REQUIRE(T == 0 || (x && topk_idx && topk_s && dg && row_of && src_token && dx_rows && dx),
          MOE_ERR_INVALID_ARGUMENT, "null pointer");
  REQUIRE(ws != nullptr && ws_bytes >= moe_route_bwd_workspace_bytes(T, H, E, K),
          MOE_ERR_WORKSPACE_TOO_SMALL, "workspace too small");
  REQUIRE_ALIGNED(x, w_router, topk_idx, topk_s, dg, row_of, offsets, counts, src_token, dx_rows,
                  dx_shared, dw_router, dx);
  REQUIRE_WS_ALIGNED(ws);
  return hip_status(moe::launch_route_permute_bwd(T, H, E, K, x, w_router, topk_idx, topk_s, dg,
                                                  row_of, offsets, counts, src_token, dx_rows,
                                                  dx_shared, dw_router, dx, ws,
                                                  (hipStream_t)stream),
                    __func__);
}

moe_status_t moe_bias_update(int32_t E, const int32_t* counts, float* bias, float gamma,
                             void* stream) {
  REQUIRE(E > 0, MOE_ERR_INVALID_ARGUMENT, "E <= 0");
  REQUIRE(E <= 128, MOE_ERR_UNSUPPORTED_SHAPE, "E > 128");
  REQUIRE(counts && bias, MOE_ERR_INVALID_ARGUMENT, "null pointer");
  REQUIRE_ALIGNED(counts, bias);
  return hip_status(moe::launch_bias_update(E, counts, bias, gamma, (hipStream_t)stream),
                    __func__);
}

static moe_status_t check_seq(const char* fn, int32_t T, int32_t E, int32_t K, int32_t seq_len) {
  if (T <= 0 || E <= 0 || K <= 0 || seq_len <= 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, fn, "T, E, K or seq_len <= 0");
  if (K > E) return fail(MOE_ERR_INVALID_ARGUMENT, fn, "K > E");
  if (T % seq_len != 0) return fail(MOE_ERR_INVALID_ARGUMENT, fn, "T % seq_len != 0");
  if (E > 128 || K > 16) return fail(MOE_ERR_UNSUPPORTED_SHAPE, fn, "E > 128 or K > 16");
  if ((int64_t)T * E >= (int64_t)1 << 31) return fail(MOE_ERR_UNSUPPORTED_SHAPE, fn, "T*E too large");
  return MOE_OK;
}

moe_status_t moe_seq_balance_fwd(int32_t T, int32_t E, int32_t K, int32_t seq_len,
                                 const float* scores, const int32_t* topk_idx, float alpha,
                                 float* loss, float* seq_f, void* ws, size_t ws_bytes,
                                 void* stream) {
  moe_status_t st = check_seq(__func__, T, E, K, seq_len);
  if (st) return st;
  REQUIRE(scores && topk_idx && loss && seq_f, MOE_ERR_INVALID_ARGUMENT, "null pointer");
  REQUIRE(ws != nullptr && ws_bytes >= moe_seq_balance_workspace_bytes(T, E, seq_len),
          MOE_ERR_WORKSPACE_TOO_SMALL, "workspace too small");
  REQUIRE_ALIGNED(scores, topk_idx, loss, seq_f);
  REQUIRE_WS_ALIGNED(ws);
  return hip_status(moe::launch_seq_balance_fwd(T, E, K, seq_len, scores, topk_idx, alpha, loss,
                                                seq_f, ws, (hipStream_t)stream),
                    __func__);
}

moe_status_t moe_seq_balance_bwd(int32_t T, int32_t E, int32_t K, int32_t seq_len,
                                 const float* scores, const float* seq_f, float alpha,
                                 const float* dloss, float* dlogit, void* stream) {
  moe_status_t st = check_seq(__func__, T, E, K, seq_len);
  if (st) return st;
  REQUIRE(scores && seq_f && dlogit, MOE_ERR_INVALID_ARGUMENT, "null pointer");
  REQUIRE_ALIGNED(scores, seq_f, dloss, dlogit);
  return hip_status(moe::launch_seq_balance_bwd(T, E, seq_len, scores, seq_f, alpha, dloss,
                                                dlogit, (hipStream_t)stream),
                    __func__);
}

moe_status_t moe_route_dlogit(int32_t T, int32_t E, int32_t K, const int32_t* topk_idx,
                              const float* topk_s, const float* dg, float* dlogit, void* stream) {
  REQUIRE(T >= 0 && E > 0 && K > 0, MOE_ERR_INVALID_ARGUMENT, "T<0 or E,K<=0");
  REQUIRE(K <= E, MOE_ERR_INVALID_ARGUMENT, "K > E");
  REQUIRE(E <= 128 && K <= 16, MOE_ERR_UNSUPPORTED_SHAPE, "E > 128 or K > 16");
  REQUIRE((int64_t)T * E < ((int64_t)1 << 31), MOE_ERR_UNSUPPORTED_SHAPE, "T*E too large");
  if (T == 0) return MOE_OK;
  REQUIRE(topk_idx && topk_s && dg && dlogit, MOE_ERR_INVALID_ARGUMENT, "null pointer");
  REQUIRE_ALIGNED(topk_idx, topk_s, dg, dlogit);
  return hip_status(moe::launch_route_dlogit(T, E, K, topk_idx, topk_s, dg, dlogit,
                                             (hipStream_t)stream),
                    __func__);
}

moe_status_t moe_route_bwd_dense(int32_t T, int32_t H, int32_t E, const uint16_t* x,
                                 const float* w_router, const float* dlogit, float* dw_router,
                                 float* dx_router, int32_t accumulate, void* ws, size_t ws_bytes,
                                 void* stream) {
  REQUIRE(T >= 0 && H > 0 && E > 0, MOE_ERR_INVALID_ARGUMENT, "T<0 or H,E<=0");
  REQUIRE(E <= 128 && H % 64 == 0 && H <= kMaxWidth, MOE_ERR_UNSUPPORTED_SHAPE,
          "E > 128, H % 64 != 0 or H > 65536");
  // the weight gradient addresses each token slice of its two operands (x
  // rows, and the three bf16 parts of dlogit side by side: 3 * 128 values a
  // row at most) with 32-bit offsets
  REQUIRE(T == 0 || moe::route_bwd_dense_slice_rows(T, H, E) * (H > 384 ? H : 384) * 2 <
                        ((int64_t)1 << 32),
          MOE_ERR_UNSUPPORTED_SHAPE, "token slice of x >= 4 GiB");
  if (T == 0) {
    // nothing to add; written mode still leaves a (zero) weight gradient
    if (accumulate) return MOE_OK;
    REQUIRE(dw_router, MOE_ERR_INVALID_ARGUMENT, "null pointer");
    REQUIRE_ALIGNED(dw_router);
    return hip_status(moe::launch_route_bwd_dense(0, H, E, nullptr, nullptr, nullptr, dw_router,
                                                  nullptr, false, nullptr, (hipStream_t)stream),
                      __func__);
  }
  REQUIRE(x && w_router && dlogit && dw_router && dx_router, MOE_ERR_INVALID_ARGUMENT,
          "null pointer");
  REQUIRE(ws != nullptr && ws_bytes >= moe_route_bwd_dense_workspace_bytes(T, H, E),
          MOE_ERR_WORKSPACE_TOO_SMALL, "workspace too small");
  REQUIRE_ALIGNED(x, w_router, dlogit, dw_router, dx_router);
  REQUIRE_WS_ALIGNED(ws);
  return hip_status(moe::launch_route_bwd_dense(T, H, E, x, w_router, dlogit, dw_router,
                                                dx_router, accumulate != 0, ws,
                                                (hipStream_t)stream),
                    __func__);
}

}  // extern "C"
