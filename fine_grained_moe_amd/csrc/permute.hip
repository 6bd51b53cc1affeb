// Permutation of tokens into per-expert row segments padded to the GEMM row
// tile ("dots.llm1 Technical Report" summary page, "Key claims" and "Method":
// expert token segments padded to tile multiples; no token is dropped).
//
// Integer-only and deterministic (the LDS atomics below only count or set
// bits, so their order cannot change a result):
//   1. count   : per 256-token chunk, a histogram of the chunk's expert ids
//   2. scan    : per expert, exclusive prefix over chunks (chunk bases) and the
//                total count; padded exclusive scan over experts (offsets)
//      fill    : -1 into every row of src_token; the tile -> expert table
//   3. scatter : per chunk, each token's rank among the chunk's earlier
//                tokens with the same expert (popcount of a per-expert token
//                bitmask), so rows of a segment are in ascending token order
//   4. rows    : copy each token's x row into its K segment rows (x read once)
#include "common.h"
#include "kernels.h"

namespace moe {
namespace perm {

constexpr int CH = 256;    // tokens per chunk = threads per workgroup
constexpr int EMAX = 128;

__global__ void __launch_bounds__(CH) count_kernel(int T, int E, int K,
                                                   const int32_t* __restrict__ topk_idx,
                                                   int32_t* __restrict__ chunk_counts) {
  __shared__ int hist[EMAX];
  const int tid = threadIdx.x, c = blockIdx.x;
  if (tid < EMAX) hist[tid] = 0;
  __syncthreads();
  const int t = c * CH + tid;
  if (t < T)
    for (int k = 0; k < K; ++k) atomicAdd(&hist[topk_idx[(int64_t)t * K + k]], 1);
  __syncthreads();
  if (tid < E) chunk_counts[(int64_t)c * E + tid] = hist[tid];
}

__global__ void __launch_bounds__(EMAX) scan_kernel(int E, int nchunks, int align,
                                                    const int32_t* __restrict__ chunk_counts,
                                                    int32_t* __restrict__ chunk_base,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets) {
  __shared__ int cnt[EMAX];
  const int tid = threadIdx.x;
  if (tid < E) {
    // exclusive prefix over chunks; eight independent loads per round
    int run = 0;
    for (int c0 = 0; c0 < nchunks; c0 += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = c0 + u < nchunks ? chunk_counts[(int64_t)(c0 + u) * E + tid] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (c0 + u < nchunks) chunk_base[(int64_t)(c0 + u) * E + tid] = run;
        run += v[u];
      }
    }
    cnt[tid] = run;
    counts[tid] = run;
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      offsets[e] = run;
      run += (cnt[e] + align - 1) / align * align;
    }
    offsets[E] = run;
  }
}

// every row of src_token to -1 (the scatter then writes the token rows) and
// the tile -> expert table (-1 past the last segment)
__global__ void __launch_bounds__(256) fill_kernel(int E, int align, int64_t m_cap,
                                                   const int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ src_token,
                                                   int32_t* __restrict__ tile_expert) {
  __shared__ int off[EMAX + 1];
  for (int i = threadIdx.x; i <= E; i += blockDim.x) off[i] = offsets[i];
  __syncthreads();
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= m_cap) return;
  src_token[r] = -1;
  if (r % align == 0) {
    const int row = (int)r;
    int e = -1;
    if (row < off[E]) {
      int lo = 0, hi = E - 1;  // last e with off[e] <= row: a non-empty segment
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= row) lo = mid; else hi = mid - 1;
      }
      e = lo;
    }
    tile_expert[r / align] = e;
  }
}

__global__ void __launch_bounds__(CH) scatter_kernel(int T, int E, int K,
                                                     const int32_t* __restrict__ topk_idx,
                                                     const int32_t* __restrict__ chunk_base,
                                                     const int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ row_of,
                                                     int32_t* __restrict__ src_token) {
  __shared__ uint32_t mask[EMAX][CH / 32];
  const int tid = threadIdx.x, c = blockIdx.x;
  for (int i = tid; i < EMAX * (CH / 32); i += CH) (&mask[0][0])[i] = 0u;
  __syncthreads();
  const int t = c * CH + tid;
  const int w = tid >> 5, bit = tid & 31;
  int ev[16];
  if (t < T) {
    for (int k = 0; k < K; ++k) {
      ev[k] = topk_idx[(int64_t)t * K + k];
      atomicOr(&mask[ev[k]][w], 1u << bit);
    }
  }
  __syncthreads();
  if (t < T) {
    for (int k = 0; k < K; ++k) {
      const int e = ev[k];
      int rank = __popc(mask[e][w] & ((1u << bit) - 1u));
      for (int q = 0; q < w; ++q) rank += __popc(mask[e][q]);
      const int row = offsets[e] + chunk_base[(int64_t)c * E + e] + rank;
      row_of[(int64_t)t * K + k] = row;
      src_token[row] = t;
    }
  }
}

// one wave per token; each lane moves 16-byte chunks of the row
__global__ void __launch_bounds__(256) rows_kernel(int T, int H, int K,
                                                   const int32_t* __restrict__ row_of,
                                                   const uint16_t* __restrict__ x,
                                                   uint16_t* __restrict__ x_rows) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int rows[16];
  for (int k = 0; k < K; ++k) rows[k] = row_of[(int64_t)t * K + k];
  const int nchunk = H / 8;
  const u32x4* src = (const u32x4*)(x + (int64_t)t * H);
  for (int c = lane; c < nchunk; c += 64) {
    u32x4 v = src[c];
    // non-temporal: the K copies of a row do not displace the lines the next
    // products read (measured: this gather 4 %, the gate/up product after it
    // 1.6 % faster; the same on the combine backward's scattered rows was slower)
    for (int k = 0; k < K; ++k) __builtin_nontemporal_store(v, (u32x4*)(x_rows + (int64_t)rows[k] * H) + c);
  }
}

}  // namespace perm

size_t permute_workspace_bytes(int T, int E) {
  const int nchunks = (T + perm::CH - 1) / perm::CH;
  return (size_t)2 * nchunks * E * sizeof(int32_t);
}

hipError_t launch_permute(int T, int H, int E, int K, int align, const int32_t* topk_idx,
                          const uint16_t* x, int64_t m_cap, int32_t* counts, int32_t* offsets,
                          int32_t* row_of, int32_t* src_token, int32_t* tile_expert,
                          uint16_t* x_rows, void* ws, hipStream_t s) {
  const int nchunks = (T + perm::CH - 1) / perm::CH;
  int32_t* chunk_counts = (int32_t*)ws;
  int32_t* chunk_base = chunk_counts + (size_t)nchunks * E;
  if (nchunks > 0)
    hipLaunchKernelGGL(perm::count_kernel, dim3(nchunks), dim3(perm::CH), 0, s, T, E, K, topk_idx,
                       chunk_counts);
  hipLaunchKernelGGL(perm::scan_kernel, dim3(1), dim3(perm::EMAX), 0, s, E, nchunks, align,
                     chunk_counts, chunk_base, counts, offsets);
  if (m_cap > 0)
    hipLaunchKernelGGL(perm::fill_kernel, dim3((unsigned)((m_cap + 255) / 256)), dim3(256), 0, s, E,
                       align, m_cap, offsets, src_token, tile_expert);
  if (nchunks > 0) {
    hipLaunchKernelGGL(perm::scatter_kernel, dim3(nchunks), dim3(perm::CH), 0, s, T, E, K,
                       topk_idx, chunk_base, offsets, row_of, src_token);
    hipLaunchKernelGGL(perm::rows_kernel, dim3((T + 3) / 4), dim3(256), 0, s, T, H, K, row_of, x,
                       x_rows);
  }
  return hipGetLastError();
}

}  // namespace moe
