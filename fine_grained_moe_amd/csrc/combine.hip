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

__global__ void __launch_bounds__(NT) combine_kernel(int T, int H, int K,
                                                     const uint16_t* __restrict__ y_rows,
                                                     const int32_t* __restrict__ row_of,
                                                     const float* __restrict__ topk_w,
                                                     const uint16_t* __restrict__ y_shared,
                                                     uint16_t* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * TPB + (threadIdx.x >> 6);
  if (t >= T) return;
  int rows[16];
  float g[16];
  for (int k = 0; k < K; ++k) {
    rows[k] = row_of[(int64_t)t * K + k];
    g[k] = topk_w[(int64_t)t * K + k];
  }
  const int nchunk = H / 8;
  for (int c = lane; c < nchunk; c += 64) {
    float acc[8], v[8];
    if (y_shared) {
      unpack8(((const u32x4*)(y_shared + (int64_t)t * H))[c], acc);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    }
    for (int k = 0; k < K; ++k) {
      unpack8(((const u32x4*)(y_rows + (int64_t)rows[k] * H))[c], v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(g[k], v[i], acc[i]);
    }
    ((u32x4*)(y + (int64_t)t * H))[c] = pack8(acc);
  }
}

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
  const int nchunk = H / 8;
  for (int k = 0; k < K; ++k) {
    const int row = row_of[(int64_t)t * K + k];
    const float gk = topk_w[(int64_t)t * K + k];
    float dot = 0.f;
    for (int c = lane; c < nchunk; c += 64) {
      float d[8], v[8], o[8];
      unpack8(((const u32x4*)(dy + (int64_t)t * H))[c], d);
      unpack8(((const u32x4*)(y_rows + (int64_t)row * H))[c], v);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        dot = __builtin_fmaf(d[i], v[i], dot);
        o[i] = gk * d[i];
      }
      ((u32x4*)(dy_rows + (int64_t)row * H))[c] = pack8(o);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dot += __shfl_xor(dot, off, 64);
    if (lane == 0) dg[(int64_t)t * K + k] = dot;
  }
}

__global__ void __launch_bounds__(NT) unpermute_add_kernel(int T, int H, int K,
                                                           const uint16_t* __restrict__ dx_rows,
                                                           const int32_t* __restrict__ row_of,
                                                           const uint16_t* __restrict__ dx_shared,
                                                           const float* __restrict__ dx_router,
                                                           uint16_t* __restrict__ dx) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * TPB + (threadIdx.x >> 6);
  if (t >= T) return;
  int rows[16];
  for (int k = 0; k < K; ++k) rows[k] = row_of[(int64_t)t * K + k];
  const int nchunk = H / 8;
  for (int c = lane; c < nchunk; c += 64) {
    float acc[8], v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int k = 0; k < K; ++k) {
      unpack8(((const u32x4*)(dx_rows + (int64_t)rows[k] * H))[c], v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    if (dx_shared) {
      unpack8(((const u32x4*)(dx_shared + (int64_t)t * H))[c], v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    if (dx_router) {
      const f32x4* p = (const f32x4*)(dx_router + (int64_t)t * H + (int64_t)c * 8);
      f32x4 a0 = p[0], a1 = p[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] += a0[i];
        acc[4 + i] += a1[i];
      }
    }
    ((u32x4*)(dx + (int64_t)t * H))[c] = pack8(acc);
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

// dW_r[h,e] = sum over the valid rows r of e's segment of x_rows[r,h] * dl_row[r]
__global__ void __launch_bounds__(256) route_bwd_wgrad_kernel(int H, int E,
                                                              const uint16_t* __restrict__ x_rows,
                                                              const float* __restrict__ dl_row,
                                                              const int32_t* __restrict__ offsets,
                                                              const int32_t* __restrict__ counts,
                                                              float* __restrict__ dw) {
  const int e = blockIdx.y;
  const int h = (blockIdx.x * 256 + threadIdx.x) * 2;
  if (h >= H) return;
  const int r0 = offsets[e], n = counts[e];
  float a0 = 0.f, a1 = 0.f;
  for (int r = r0; r < r0 + n; ++r) {
    const float d = dl_row[r];
    const uint32_t xv = *(const uint32_t*)(x_rows + (int64_t)r * H + h);
    a0 = __builtin_fmaf(lo_bf16(xv), d, a0);
    a1 = __builtin_fmaf(hi_bf16(xv), d, a1);
  }
  dw[(int64_t)h * E + e] = a0;
  dw[(int64_t)(h + 1) * E + e] = a1;
}

}  // namespace comb

hipError_t launch_combine(int T, int H, int K, const uint16_t* y_rows, const int32_t* row_of,
                          const float* topk_w, const uint16_t* y_shared, uint16_t* y,
                          hipStream_t s) {
  hipLaunchKernelGGL(comb::combine_kernel, dim3((T + comb::TPB - 1) / comb::TPB), dim3(comb::NT), 0,
                     s, T, H, K, y_rows, row_of, topk_w, y_shared, y);
  return hipGetLastError();
}

hipError_t launch_combine_bwd(int T, int H, int K, const uint16_t* dy, const uint16_t* y_rows,
                              const int32_t* row_of, const float* topk_w, uint16_t* dy_rows,
                              float* dg, hipStream_t s) {
  hipLaunchKernelGGL(comb::combine_bwd_kernel, dim3((T + comb::TPB - 1) / comb::TPB),
                     dim3(comb::NT), 0, s, T, H, K, dy, y_rows, row_of, topk_w, dy_rows, dg);
  return hipGetLastError();
}

hipError_t launch_unpermute_add(int T, int H, int K, const uint16_t* dx_rows,
                                const int32_t* row_of, const uint16_t* dx_shared,
                                const float* dx_router, uint16_t* dx, hipStream_t s) {
  hipLaunchKernelGGL(comb::unpermute_add_kernel, dim3((T + comb::TPB - 1) / comb::TPB),
                     dim3(comb::NT), 0, s, T, H, K, dx_rows, row_of, dx_shared, dx_router, dx);
  return hipGetLastError();
}

size_t route_bwd_workspace_bytes(int64_t m_cap, int H, int E) {
  // W_r^T [E,H] fp32, then dl_row [m_cap] fp32 (256-byte aligned)
  size_t a = ((size_t)E * H * sizeof(float) + 255) / 256 * 256;
  return a + (size_t)m_cap * sizeof(float);
}

hipError_t launch_route_bwd(int T, int H, int E, int K, const uint16_t* x_rows,
                            const float* w_router, const int32_t* topk_idx, const float* topk_s,
                            const float* dg, const int32_t* row_of, const int32_t* offsets,
                            const int32_t* counts, float* dw_router, float* dx_router, void* ws,
                            hipStream_t s) {
  float* wt = (float*)ws;
  float* dl_row = (float*)((char*)ws + ((size_t)E * H * sizeof(float) + 255) / 256 * 256);
  hipLaunchKernelGGL(comb::transpose_kernel, dim3((H + 31) / 32, (E + 31) / 32), dim3(256), 0, s, H,
                     E, w_router, wt);
  if (T > 0)
    hipLaunchKernelGGL(comb::route_bwd_token_kernel, dim3((T + comb::TPB - 1) / comb::TPB),
                       dim3(comb::NT), 0, s, T, H, E, K, wt, topk_idx, topk_s, dg, row_of, dl_row,
                       dx_router);
  hipLaunchKernelGGL(comb::route_bwd_wgrad_kernel, dim3((H / 2 + 255) / 256, E), dim3(256), 0, s, H,
                     E, x_rows, dl_row, offsets, counts, dw_router);
  return hipGetLastError();
}

}  // namespace moe
