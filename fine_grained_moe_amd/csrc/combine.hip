// Combine, combine backward, un-permute-add and router backward: the
// HBM-bound row kernels of the MoE layer on gfx950.
//
// Combine (model card "Model Architecture Features": 6 routed + 2 shared
// experts per token) is done as the gather dual of a scatter-add: each token
// gathers its K routed rows, so every output row is written once, the sum
// order is fixed (no atomics) and every access is a coalesced 16-byte row
// chunk.  One wave per token; lane l owns chunks l, l+64, ... of the row.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace comb {

constexpr int NT = 256, TPB = NT / 64;  // tokens per workgroup (one per wave)
// threads per token in combine and un-permute-add (64: one wave; 256: the
// whole workgroup streams longer stretches of each row)
#ifndef MOE_ROW_TPT
#define MOE_ROW_TPT 256
#endif

__device__ __forceinline__ void unpack8(const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = lo_bf16(v[i]);
    f[2 * i + 1] = hi_bf16(v[i]);
  }
}
__device__ __forceinline__ u32x4 pack8(const float* f) {
  return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
               pack_bf16x2(f[6], f[7])};
}

// Every k-loop below is unrolled to KMAX with k < K guards, so a lane's K row
// loads of one chunk are all in flight together; KMAX = 8 when K <= 8 keeps
// the register count (and so the occupancy) of the common case low.
template <int KMAX, int TPT>
__global__ void __launch_bounds__(NT) combine_kernel(int T, int H, int K,
                                                     const uint16_t* __restrict__ y_rows,
                                                     const int32_t* __restrict__ row_of,
                                                     const float* __restrict__ topk_w,
                                                     const uint16_t* __restrict__ y_shared,
                                                     uint16_t* __restrict__ y) {
  const int lane = threadIdx.x % TPT;
  const int t = blockIdx.x * (NT / TPT) + threadIdx.x / TPT;
  if (t >= T) return;
  int rows[KMAX];
  float g[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    rows[k] = k < K ? row_of[(int64_t)t * K + k] : 0;
    g[k] = k < K ? topk_w[(int64_t)t * K + k] : 0.f;
  }
  const int nchunk = H / 8;
  for (int c = lane; c < nchunk; c += TPT) {
    u32x4 vr[KMAX], vs = u32x4{0u, 0u, 0u, 0u};
    // non-temporal loads: every row is read once here (alone 6 % faster)
    if (y_shared) vs = __builtin_nontemporal_load((const u32x4*)(y_shared + (int64_t)t * H) + c);
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
      if (k < K) vr[k] = __builtin_nontemporal_load((const u32x4*)(y_rows + (int64_t)rows[k] * H) + c);
    float acc[8], v[8];
    unpack8(vs, acc);
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      if (k < K) {
        unpack8(vr[k], v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(g[k], v[i], acc[i]);
      }
    }
    // written once and never read back here: streamed past the caches
    __builtin_nontemporal_store(pack8(acc), (u32x4*)(y + (int64_t)t * H) + c);
  }
}

template <int KMAX>
__global__ void __launch_bounds__(NT) combine_bwd_kernel(int T, int H, int K,
                                                         const uint16_t* __restrict__ dy,
                                                         const uint16_t* __restrict__ y_rows,
                                                         const int32_t* __restrict__ row_of,
                                                         const float* __restrict__ topk_w,
                                                         uint16_t* __restrict__ dy_rows,
                                                         float* __restrict__ dg) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * TPB + (threadIdx.x >> 6);
  if (t >= T) return;
  int rows[KMAX];
  float g[KMAX], dot[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    rows[k] = k < K ? row_of[(int64_t)t * K + k] : 0;
    g[k] = k < K ? topk_w[(int64_t)t * K + k] : 0.f;
    dot[k] = 0.f;
  }
  const int nchunk = H / 8;
  for (int c = lane; c < nchunk; c += 64) {
    const u32x4 vd = ((const u32x4*)(dy + (int64_t)t * H))[c];
    u32x4 vr[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
      if (k < K) vr[k] = ((const u32x4*)(y_rows + (int64_t)rows[k] * H))[c];
    float d[8], v[8], o[8];
    unpack8(vd, d);
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      if (k < K) {
        unpack8(vr[k], v);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          dot[k] = __builtin_fmaf(d[i], v[i], dot[k]);
          o[i] = g[k] * d[i];
        }
        ((u32x4*)(dy_rows + (int64_t)rows[k] * H))[c] = pack8(o);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (k < K) {
      float v = dot[k];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
      if (lane == 0) dg[(int64_t)t * K + k] = v;
    }
  }
}

// ROUTER: dx_router is not read; the router's input gradient is formed here
// from the route backward's workspace (wt = W_r^T, dl_row = the logit
// gradient of every row), in the order route_bwd_token_kernel forms it
template <int KMAX, int TPT, bool ROUTER>
__global__ void __launch_bounds__(NT) unpermute_add_kernel(int T, int H, int K,
                                                           const uint16_t* __restrict__ dx_rows,
                                                           const int32_t* __restrict__ row_of,
                                                           const uint16_t* __restrict__ dx_shared,
                                                           const float* __restrict__ dx_router,
                                                           const float* __restrict__ wt,
                                                           const float* __restrict__ dl_row,
                                                           const int32_t* __restrict__ topk_idx,
                                                           uint16_t* __restrict__ dx) {
  const int lane = threadIdx.x % TPT;
  const int t = blockIdx.x * (NT / TPT) + threadIdx.x / TPT;
  if (t >= T) return;
  int rows[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) rows[k] = k < K ? row_of[(int64_t)t * K + k] : 0;
  float dlk[KMAX];
  int ek[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    dlk[k] = (ROUTER && k < K) ? dl_row[rows[k]] : 0.f;
    ek[k] = (ROUTER && k < K) ? topk_idx[(int64_t)t * K + k] : 0;
  }
  const int nchunk = H / 8;
  for (int c = lane; c < nchunk; c += TPT) {
    u32x4 vr[KMAX], vs = u32x4{0u, 0u, 0u, 0u};
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
      if (k < K) vr[k] = __builtin_nontemporal_load((const u32x4*)(dx_rows + (int64_t)rows[k] * H) + c);
    // read once, as in the combine (the fused router backward + un-permute
    // alone 10 % faster; the whole step 0.2 %)
    if (dx_shared) vs = __builtin_nontemporal_load((const u32x4*)(dx_shared + (int64_t)t * H) + c);
    if (ROUTER) {
#pragma unroll
      for (int k = 0; k < KMAX; ++k) {
        if (k < K) {
          const f32x4* w = (const f32x4*)(wt + (int64_t)ek[k] * H + (int64_t)c * 8);
          const f32x4 w0 = w[0], w1 = w[1];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            a0[i] = __builtin_fmaf(dlk[k], w0[i], a0[i]);
            a1[i] = __builtin_fmaf(dlk[k], w1[i], a1[i]);
          }
        }
      }
    } else if (dx_router) {
      const f32x4* p = (const f32x4*)(dx_router + (int64_t)t * H + (int64_t)c * 8);
      a0 = p[0];
      a1 = p[1];
    }
    float acc[8], v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      if (k < K) {
        unpack8(vr[k], v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += v[i];
      }
    }
    unpack8(vs, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += v[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[i] += a0[i];
      acc[4 + i] += a1[i];
    }
    __builtin_nontemporal_store(pack8(acc), (u32x4*)(dx + (int64_t)t * H) + c);
  }
}

// ---------------------------------------------------------------------------
// Router backward (routing decision held fixed)
// ---------------------------------------------------------------------------
// W_r [H,E] -> W_r^T [E,H] through a 32x32 LDS tile
__global__ void __launch_bounds__(256) transpose_kernel(int H, int E, const float* __restrict__ w,
                                                        float* __restrict__ wt) {
  __shared__ float tile[32][33];
  const int h0 = blockIdx.x * 32, e0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int i = ty; i < 32; i += 8) {
    int h = h0 + i, e = e0 + tx;
    tile[i][tx] = (h < H && e < E) ? w[(int64_t)h * E + e] : 0.f;
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    int e = e0 + i, h = h0 + tx;
    if (e < E && h < H) wt[(int64_t)e * H + h] = tile[tx][i];
  }
}

// per token: dlogit for its K experts, dx_router row, and the per-row copy
// of dlogit used by the weight gradient
__global__ void __launch_bounds__(NT) route_bwd_token_kernel(int T, int H, int E, int K,
                                                             const float* __restrict__ wt,
                                                             const int32_t* __restrict__ topk_idx,
                                                             const float* __restrict__ topk_s,
                                                             const float* __restrict__ dg,
                                                             const int32_t* __restrict__ row_of,
                                                             float* __restrict__ dl_row,
                                                             float* __restrict__ dx_router) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * TPB + (threadIdx.x >> 6);
  if (t >= T) return;
  // lane k < K holds expert k's values
  float s = 0.f, d = 0.f;
  int e = 0;
  if (lane < K) {
    s = topk_s[(int64_t)t * K + lane];
    d = dg[(int64_t)t * K + lane];
    e = topk_idx[(int64_t)t * K + lane];
  }
  // S = sum_j s_j and sum_j s_j dg_j (fixed lane order reduction)
  float ssum = s, sdg = s * d;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    ssum += __shfl_xor(ssum, off, 64);
    sdg += __shfl_xor(sdg, off, 64);
  }
  // ds_k = (dg_k - sum_j g_j dg_j) / S with g_j = s_j / S
  const float ds = (d - sdg / ssum) / ssum;
  const float dl = ds * s * (1.0f - s);
  if (lane < K) dl_row[row_of[(int64_t)t * K + lane]] = dl;
  // without dx_router the un-permute forms the input gradient from dl_row
  if (dx_router == nullptr) return;
  float dlk[16];
  int ek[16];
  for (int k = 0; k < K; ++k) {
    dlk[k] = __shfl(dl, k, 64);
    ek[k] = __shfl(e, k, 64);
  }
  for (int h = lane * 4; h < H; h += 256) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < K; ++k) {
      f32x4 wv = *(const f32x4*)(wt + (int64_t)ek[k] * H + h);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(dlk[k], wv[i], acc[i]);
    }
    *(f32x4*)(dx_router + (int64_t)t * H + h) = acc;
  }
}

// dW_r[h,e] = sum over the valid rows r of e's segment of x[src_token[r],h] * dl_row[r]
// Workgroup (expert e, 512 columns): wave w takes the rows r0+w, r0+w+4, ...,
// each lane 8 columns (one 16-byte chunk per row, four rows in flight); the
// four partial sums are added in wave order through LDS, so the result does
// not depend on timing.  The token rows are gathered from x (84 MB at dots
// shapes, K reads of each mostly served by the caches) rather than streamed
// from the permuted copy (six times the bytes): 115 instead of 175 us.
constexpr int WG_COLS = 512, WG_WAVES = 4, WG_UNROLL = 4;
__global__ void __launch_bounds__(256) route_bwd_wgrad_kernel(int H, int E,
                                                              const uint16_t* __restrict__ x,
                                                              const int32_t* __restrict__ src_token,
                                                              const float* __restrict__ dl_row,
                                                              const int32_t* __restrict__ offsets,
                                                              const int32_t* __restrict__ counts,
                                                              float* __restrict__ dw) {
  __shared__ float part[WG_WAVES - 1][WG_COLS];
  const int e = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = blockIdx.x * WG_COLS + lane * 8;
  const bool hin = h < H;
  const int r0 = offsets[e], n = counts[e];
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int j = wave; j < n; j += WG_WAVES * WG_UNROLL) {
    u32x4 v[WG_UNROLL];
    float d[WG_UNROLL];
#pragma unroll
    for (int u = 0; u < WG_UNROLL; ++u) {
      const int jj = j + u * WG_WAVES;
      const bool ok = jj < n && hin;
      d[u] = jj < n ? dl_row[r0 + jj] : 0.f;
      v[u] = ok ? *(const u32x4*)(x + (int64_t)src_token[r0 + jj] * H + h) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < WG_UNROLL; ++u) {
      float xv[8];
      unpack8(v[u], xv);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(xv[i], d[u], acc[i]);
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) part[wave - 1][lane * 8 + i] = acc[i];
  }
  __syncthreads();
  if (wave == 0 && hin) {
#pragma unroll
    for (int w = 0; w < WG_WAVES - 1; ++w)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += part[w][lane * 8 + i];
#pragma unroll
    for (int i = 0; i < 8; ++i) dw[(int64_t)(h + i) * E + e] = acc[i];
  }
}

}  // namespace comb

hipError_t launch_combine(int T, int H, int K, const uint16_t* y_rows, const int32_t* row_of,
                          const float* topk_w, const uint16_t* y_shared, uint16_t* y,
                          hipStream_t s) {
  constexpr int TPT = MOE_ROW_TPT, TPB = comb::NT / TPT;
  const dim3 grid((T + TPB - 1) / TPB);
  if (K <= 8)
    hipLaunchKernelGGL((comb::combine_kernel<8, TPT>), grid, dim3(comb::NT), 0, s, T, H, K, y_rows,
                       row_of, topk_w, y_shared, y);
  else
    hipLaunchKernelGGL((comb::combine_kernel<16, TPT>), grid, dim3(comb::NT), 0, s, T, H, K, y_rows,
                       row_of, topk_w, y_shared, y);
  return hipGetLastError();
}

hipError_t launch_combine_bwd(int T, int H, int K, const uint16_t* dy, const uint16_t* y_rows,
                              const int32_t* row_of, const float* topk_w, uint16_t* dy_rows,
                              float* dg, hipStream_t s) {
  const dim3 grid((T + comb::TPB - 1) / comb::TPB);
  if (K <= 8)
    hipLaunchKernelGGL(comb::combine_bwd_kernel<8>, grid, dim3(comb::NT), 0, s, T, H, K, dy, y_rows,
                       row_of, topk_w, dy_rows, dg);
  else
    hipLaunchKernelGGL(comb::combine_bwd_kernel<16>, grid, dim3(comb::NT), 0, s, T, H, K, dy, y_rows,
                       row_of, topk_w, dy_rows, dg);
  return hipGetLastError();
}

static hipError_t unpermute(int T, int H, int K, const uint16_t* dx_rows, const int32_t* row_of,
                            const uint16_t* dx_shared, const float* dx_router, const float* wt,
                            const float* dl_row, const int32_t* topk_idx, uint16_t* dx,
                            hipStream_t s) {
  constexpr int TPT = MOE_ROW_TPT, TPB = comb::NT / TPT;
  const dim3 grid((T + TPB - 1) / TPB);
  const bool router = wt != nullptr;
  if (K <= 8 && !router)
    hipLaunchKernelGGL((comb::unpermute_add_kernel<8, TPT, false>), grid, dim3(comb::NT), 0, s, T,
                       H, K, dx_rows, row_of, dx_shared, dx_router, wt, dl_row, topk_idx, dx);
  else if (K <= 8)
    hipLaunchKernelGGL((comb::unpermute_add_kernel<8, TPT, true>), grid, dim3(comb::NT), 0, s, T,
                       H, K, dx_rows, row_of, dx_shared, dx_router, wt, dl_row, topk_idx, dx);
  else if (!router)
    hipLaunchKernelGGL((comb::unpermute_add_kernel<16, TPT, false>), grid, dim3(comb::NT), 0, s, T,
                       H, K, dx_rows, row_of, dx_shared, dx_router, wt, dl_row, topk_idx, dx);
  else
    hipLaunchKernelGGL((comb::unpermute_add_kernel<16, TPT, true>), grid, dim3(comb::NT), 0, s, T,
                       H, K, dx_rows, row_of, dx_shared, dx_router, wt, dl_row, topk_idx, dx);
  return hipGetLastError();
}

hipError_t launch_unpermute_add(int T, int H, int K, const uint16_t* dx_rows,
                                const int32_t* row_of, const uint16_t* dx_shared,
                                const float* dx_router, uint16_t* dx, hipStream_t s) {
  return unpermute(T, H, K, dx_rows, row_of, dx_shared, dx_router, nullptr, nullptr, nullptr, dx,
                   s);
}

size_t route_bwd_workspace_bytes(int64_t m_cap, int H, int E) {
  // W_r^T [E,H] fp32, then dl_row [m_cap] fp32 (256-byte aligned)
  size_t a = ((size_t)E * H * sizeof(float) + 255) / 256 * 256;
  return a + (size_t)m_cap * sizeof(float);
}

hipError_t launch_route_bwd(int T, int H, int E, int K, const uint16_t* x,
                            const float* w_router, const int32_t* topk_idx, const float* topk_s,
                            const float* dg, const int32_t* row_of, const int32_t* offsets,
                            const int32_t* counts, const int32_t* src_token, float* dw_router,
                            float* dx_router, void* ws, hipStream_t s) {
  float* wt = (float*)ws;
  float* dl_row = (float*)((char*)ws + ((size_t)E * H * sizeof(float) + 255) / 256 * 256);
  hipLaunchKernelGGL(comb::transpose_kernel, dim3((H + 31) / 32, (E + 31) / 32), dim3(256), 0, s, H,
                     E, w_router, wt);
  if (T > 0)
    hipLaunchKernelGGL(comb::route_bwd_token_kernel, dim3((T + comb::TPB - 1) / comb::TPB),
                       dim3(comb::NT), 0, s, T, H, E, K, wt, topk_idx, topk_s, dg, row_of, dl_row,
                       dx_router);
  hipLaunchKernelGGL(comb::route_bwd_wgrad_kernel, dim3((H + comb::WG_COLS - 1) / comb::WG_COLS, E),
                     dim3(256), 0, s, H, E, x, src_token, dl_row, offsets, counts, dw_router);
  return hipGetLastError();
}

hipError_t launch_route_permute_bwd(int T, int H, int E, int K, const uint16_t* x,
                                    const float* w_router, const int32_t* topk_idx,
                                    const float* topk_s, const float* dg, const int32_t* row_of,
                                    const int32_t* offsets, const int32_t* counts,
                                    const int32_t* src_token, const uint16_t* dx_rows,
                                    const uint16_t* dx_shared, float* dw_router, uint16_t* dx,
                                    void* ws, hipStream_t s) {
  // the router backward without its [T,H] input gradient (dl_row and W_r^T
  // stay in ws), then the un-permute forming that gradient where it adds it
  hipError_t e = launch_route_bwd(T, H, E, K, x, w_router, topk_idx, topk_s, dg, row_of, offsets,
                                  counts, src_token, dw_router, nullptr, ws, s);
  if (e != hipSuccess || T == 0) return e;
  const float* wt = (const float*)ws;
  const float* dl_row =
      (const float*)((const char*)ws + ((size_t)E * H * sizeof(float) + 255) / 256 * 256);
  return unpermute(T, H, K, dx_rows, row_of, dx_shared, nullptr, wt, dl_row, topk_idx, dx, s);
}

}  // namespace moe
