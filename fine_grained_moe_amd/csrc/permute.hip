// Permutation of tokens into per-expert row segments padded to the GEMM row
// tile ("dots.llm1 Technical Report" summary page, "Key claims" and "Method":
// expert token segments padded to tile multiples; no token is dropped).
//
// Integer-only and deterministic (the LDS atomics below only count, set bits
// or take a minimum, so their order cannot change a result):
//   1. count   : per 256-token chunk, a histogram of the chunk's expert ids
//   2. scan    : per expert, exclusive prefix over chunks (chunk bases) and the
//                total count; padded exclusive scan over experts (offsets)
//      fill    : -1 into every row of src_token; the tile -> expert table
//   3. scatter : per chunk, each token's rank among the chunk's earlier
//                tokens with the same expert (popcount of a per-expert token
//                bitmask), so rows of a segment are in ascending token order
//   4. rows    : copy each token's x row into its K segment rows (x read once)
// A batch of at most one chunk (decode) runs steps 1-3 as one workgroup
// (small_kernel): the same layout from one launch instead of four.
//
// Data check: a token whose K expert ids are not all in [0,E) and distinct is
// rejected before any of its ids indexes anything: it is not counted, owns no
// row, its row_of entries are -1 and its x row is not copied.  count records
// per chunk what it rejected; scan (or small_kernel, for one chunk) folds that
// into the status block at the start of the workspace (written by every call):
//   [0] flags: bit 0 an id outside [0,E), bit 1 an id repeated in a token
//   [1] number of rejected tokens
//   [2] smallest rejected token, -1 if none
//   [3] kPermuteStatusMagic
#include <atomic>
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace perm {

constexpr int CH = 256;    // tokens per chunk = threads per workgroup
constexpr int EMAX = 128;
constexpr int kNone = 0x7fffffff;

// Loads the K expert ids of one token into ev and checks them: returns 0 if
// every id lies in [0,E) and no id repeats, else the status flags (bit 0 out
// of range, bit 1 repeated).
__device__ __forceinline__ int load_ids(const int32_t* __restrict__ p, int K, int E, int* ev) {
  int fl = 0;
  for (int k = 0; k < K; ++k) {
    const int e = p[k];
    ev[k] = e;
    if (e < 0 || e >= E) fl |= 1;
    for (int j = 0; j < k; ++j)
      if (ev[j] == e) fl |= 2;
  }
  return fl;
}

__global__ void __launch_bounds__(CH) count_kernel(int T, int E, int K,
                                                   const int32_t* __restrict__ topk_idx,
                                                   int32_t* __restrict__ chunk_counts,
                                                   int32_t* __restrict__ chunk_status) {
  __shared__ int hist[EMAX];
  __shared__ int bad_flags, bad_count, bad_first;
  const int tid = threadIdx.x, c = blockIdx.x;
  if (tid < EMAX) hist[tid] = 0;
  if (tid == 0) {
    bad_flags = 0;
    bad_count = 0;
    bad_first = kNone;
  }
  __syncthreads();
  const int t = c * CH + tid;
  if (t < T) {
    int ev[16];
    const int fl = load_ids(topk_idx + (int64_t)t * K, K, E, ev);
    if (fl == 0) {
      for (int k = 0; k < K; ++k) atomicAdd(&hist[ev[k]], 1);
    } else {
      atomicOr(&bad_flags, fl);
      atomicAdd(&bad_count, 1);
      atomicMin(&bad_first, t);
    }
  }
  __syncthreads();
  if (tid < E) chunk_counts[(int64_t)c * E + tid] = hist[tid];
  if (tid == 0) {
    chunk_status[3 * (int64_t)c + 0] = bad_flags;
    chunk_status[3 * (int64_t)c + 1] = bad_count;
    chunk_status[3 * (int64_t)c + 2] = bad_first;
  }
}

__global__ void __launch_bounds__(EMAX) scan_kernel(int E, int nchunks, int align,
                                                    const int32_t* __restrict__ chunk_counts,
                                                    const int32_t* __restrict__ chunk_status,
                                                    int32_t* __restrict__ chunk_base,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ status) {
  __shared__ int cnt[EMAX];
  __shared__ int bad_flags, bad_count, bad_first;
  const int tid = threadIdx.x;
  if (tid == 0) {
    bad_flags = 0;
    bad_count = 0;
    bad_first = kNone;
  }
  __syncthreads();
  {
    int fl = 0, n = 0, first = kNone;
    for (int c = tid; c < nchunks; c += EMAX) {
      fl |= chunk_status[3 * (int64_t)c + 0];
      n += chunk_status[3 * (int64_t)c + 1];
      first = min(first, chunk_status[3 * (int64_t)c + 2]);
    }
    if (n) {
      atomicOr(&bad_flags, fl);
      atomicAdd(&bad_count, n);
      atomicMin(&bad_first, first);
    }
  }
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
  __syncthreads();
  if (tid == 0) {
    status[0] = bad_flags;
    status[1] = bad_count;
    status[2] = bad_count ? bad_first : -1;
    status[3] = kPermuteStatusMagic;
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
  const bool ok = t < T && load_ids(topk_idx + (int64_t)t * K, K, E, ev) == 0;
  if (ok)
    for (int k = 0; k < K; ++k) atomicOr(&mask[ev[k]][w], 1u << bit);
  else if (t < T)
    for (int k = 0; k < K; ++k) row_of[(int64_t)t * K + k] = -1;   // rejected: no rows
  __syncthreads();
  if (ok) {
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

// Steps 1-3 for a batch of at most CH tokens, one token per thread: the
// histogram and the per-expert token bitmasks in LDS, the padded scan, every
// row no token fills set to -1 (each segment's padding and the rows past the
// last segment: the token rows are written by the scatter, so no row is
// written twice), the tile -> expert table, and each token's rows in
// ascending token order, as the multi-chunk path lays them out.
__global__ void __launch_bounds__(CH) small_kernel(int T, int E, int K, int align, int64_t m_cap,
                                                   const int32_t* __restrict__ topk_idx,
                                                   int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ row_of,
                                                   int32_t* __restrict__ src_token,
                                                   int32_t* __restrict__ tile_expert,
                                                   int32_t* __restrict__ status) {
  __shared__ int hist[EMAX];
  __shared__ int scan[2][EMAX];
  __shared__ int off[EMAX + 1];
  __shared__ uint32_t mask[EMAX][CH / 32];
  __shared__ int bad_flags, bad_count, bad_first;
  const int tid = threadIdx.x;
  if (tid < EMAX) hist[tid] = 0;
  for (int i = tid; i < EMAX * (CH / 32); i += CH) (&mask[0][0])[i] = 0u;
  if (tid == 0) {
    bad_flags = 0;
    bad_count = 0;
    bad_first = kNone;
  }
  __syncthreads();
  const int t = tid, w = tid >> 5, bit = tid & 31;
  int ev[16];
  bool ok = false;
  if (t < T) {
    const int fl = load_ids(topk_idx + (int64_t)t * K, K, E, ev);
    ok = fl == 0;
    if (ok) {
      for (int k = 0; k < K; ++k) {
        atomicAdd(&hist[ev[k]], 1);
        atomicOr(&mask[ev[k]][w], 1u << bit);
      }
    } else {
      atomicOr(&bad_flags, fl);
      atomicAdd(&bad_count, 1);
      atomicMin(&bad_first, t);
      for (int k = 0; k < K; ++k) row_of[(int64_t)t * K + k] = -1;   // rejected: no rows
    }
  }
  __syncthreads();
  // inclusive scan of the padded counts over experts (Hillis-Steele, in LDS)
  int cur = 0;
  if (tid < EMAX) scan[0][tid] = tid < E ? (hist[tid] + align - 1) / align * align : 0;
  __syncthreads();
  for (int d = 1; d < EMAX; d <<= 1) {
    if (tid < EMAX) scan[cur ^ 1][tid] = scan[cur][tid] + (tid >= d ? scan[cur][tid - d] : 0);
    cur ^= 1;
    __syncthreads();
  }
  if (tid <= E) off[tid] = tid == 0 ? 0 : scan[cur][tid - 1];
  __syncthreads();
  if (tid < E) counts[tid] = hist[tid];
  if (tid <= E) offsets[tid] = off[tid];
  if (tid == 0) {
    status[0] = bad_flags;
    status[1] = bad_count;
    status[2] = bad_count ? bad_first : -1;
    status[3] = kPermuteStatusMagic;
  }
  // rows no token fills: each segment's padding, one wave per expert with its
  // lanes on consecutive rows (coalesced stores); lane j of wave v first
  // fetches the bounds of expert v + 4j, so the loop reads them from registers
  {
    constexpr int NWV = CH / 64;
    const int wv = tid >> 6, ln = tid & 63;
    const int ej = wv + NWV * ln;
    const int pad_lo = ej < E ? off[ej] + hist[ej] : 0;
    const int pad_hi = ej < E ? off[ej + 1] : 0;
    for (int j = 0; wv + NWV * j < E; ++j) {
      const int lo = __builtin_amdgcn_readlane(pad_lo, j), hi = __builtin_amdgcn_readlane(pad_hi, j);
      for (int r = lo + ln; r < hi; r += 64) src_token[r] = -1;
    }
  }
  // ... and every row past the last segment
  for (int64_t r = off[E] + tid; r < m_cap; r += CH) src_token[r] = -1;
  // tile -> expert: the last expert whose segment starts at or before the
  // tile (a non-empty one), -1 past the last segment
  for (int64_t q = tid; q * align < m_cap; q += CH) {
    const int row = (int)(q * align);
    int e = -1;
    if (row < off[E]) {
      int lo = 0, hi = E - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= row) lo = mid; else hi = mid - 1;
      }
      e = lo;
    }
    tile_expert[q] = e;
  }
  if (ok) {
    for (int k = 0; k < K; ++k) {
      const int e = ev[k];
      int rank = __popc(mask[e][w] & ((1u << bit) - 1u));
      for (int q = 0; q < w; ++q) rank += __popc(mask[e][q]);
      const int row = off[e] + rank;
      row_of[(int64_t)t * K + k] = row;
      src_token[row] = t;
    }
  }
}

// `split` waves per token (1, 2 or 4: small batches spread a row over
// several waves to fill the chip); each lane moves 16-byte chunks of the row
__global__ void __launch_bounds__(256) rows_kernel(int T, int H, int K, int split,
                                                   const int32_t* __restrict__ row_of,
                                                   const uint16_t* __restrict__ x,
                                                   uint16_t* __restrict__ x_rows) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int t = gw / split, part = gw % split;
  if (t >= T || row_of[(int64_t)t * K] < 0) return;   // a rejected token owns no rows
  int rows[16];
  for (int k = 0; k < K; ++k) rows[k] = row_of[(int64_t)t * K + k];
  const int nchunk = H / 8;
  const u32x4* src = (const u32x4*)(x + (int64_t)t * H);
  for (int c = part * 64 + lane; c < nchunk; c += 64 * split) {
    u32x4 v = src[c];
    // non-temporal: the K copies of a row do not displace the lines the next
    // products read (measured: this gather 4 %, the gate/up product after it
    // 1.6 % faster; the same on the combine backward's scattered rows was slower)
    for (int k = 0; k < K; ++k) __builtin_nontemporal_store(v, (u32x4*)(x_rows + (int64_t)rows[k] * H) + c);
  }
}

}  // namespace perm

// workspace: the 256-byte status block, per-chunk status (3 ints a chunk,
// rounded up to 256 bytes), per-chunk histograms, per-chunk bases
static size_t chunk_status_bytes(int nchunks) {
  return ((size_t)3 * nchunks * sizeof(int32_t) + 255) / 256 * 256;
}

size_t permute_workspace_bytes(int T, int E) {
  const int nchunks = (T + perm::CH - 1) / perm::CH;
  return kPermuteStatusBytes + chunk_status_bytes(nchunks) + (size_t)2 * nchunks * E * sizeof(int32_t);
}

hipError_t launch_permute(int T, int H, int E, int K, int align, const int32_t* topk_idx,
                          const uint16_t* x, int64_t m_cap, int32_t* counts, int32_t* offsets,
                          int32_t* row_of, int32_t* src_token, int32_t* tile_expert,
                          uint16_t* x_rows, void* ws, int32_t* status_out, hipStream_t s) {
  const int nchunks = (T + perm::CH - 1) / perm::CH;
  int32_t* status = status_out ? status_out : (int32_t*)ws;
  if (nchunks == 1) {
    hipLaunchKernelGGL(perm::small_kernel, dim3(1), dim3(perm::CH), 0, s, T, E, K, align, m_cap,
                       topk_idx, counts, offsets, row_of, src_token, tile_expert, status);
    // four waves a token: T <= 256 tokens as up to 1,024 waves
    hipLaunchKernelGGL(perm::rows_kernel, dim3(T), dim3(256), 0, s, T, H, K, 4, row_of, x, x_rows);
    return hipGetLastError();
  }
  int32_t* chunk_status = (int32_t*)((uint8_t*)ws + kPermuteStatusBytes);
  int32_t* chunk_counts = (int32_t*)((uint8_t*)chunk_status + chunk_status_bytes(nchunks));
  int32_t* chunk_base = chunk_counts + (size_t)nchunks * E;
  if (nchunks > 0)
    hipLaunchKernelGGL(perm::count_kernel, dim3(nchunks), dim3(perm::CH), 0, s, T, E, K, topk_idx,
                       chunk_counts, chunk_status);
  hipLaunchKernelGGL(perm::scan_kernel, dim3(1), dim3(perm::EMAX), 0, s, E, nchunks, align,
                     chunk_counts, chunk_status, chunk_base, counts, offsets, status);
  if (m_cap > 0)
    hipLaunchKernelGGL(perm::fill_kernel, dim3((unsigned)((m_cap + 255) / 256)), dim3(256), 0, s, E,
                       align, m_cap, offsets, src_token, tile_expert);
  if (nchunks > 0) {
    hipLaunchKernelGGL(perm::scatter_kernel, dim3(nchunks), dim3(perm::CH), 0, s, T, E, K,
                       topk_idx, chunk_base, offsets, row_of, src_token);
    hipLaunchKernelGGL(perm::rows_kernel, dim3((T + 3) / 4), dim3(256), 0, s, T, H, K, 1, row_of, x,
                       x_rows);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The permutation without a workspace argument, for callers that cannot
// allocate (graph capture, serving loops): its workspace is this file-scope
// device array, one per GPU for the life of the process.  Every word the
// kernels read is written earlier in the same call, so nothing is cleared
// between calls; calls that overlap on one GPU share the array and race.
// ---------------------------------------------------------------------------
namespace perm {
constexpr int kNoAllocMaxTokens = 131072;
constexpr size_t kNoAllocScratchBytes =
    kPermuteStatusBytes + ((size_t)3 * (kNoAllocMaxTokens / CH) * 4 + 255) / 256 * 256 +
    (size_t)2 * (kNoAllocMaxTokens / CH) * EMAX * 4;   // 530,688 bytes
static_assert(kNoAllocMaxTokens % CH == 0, "whole chunks");

__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
}  // namespace perm

namespace {
using perm::kNoAllocMaxTokens;
using perm::kNoAllocScratchBytes;

// the array's device address on each GPU, looked up once per device (in host
// code `scratch` names a host-side stand-in, never the device memory)
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

hipError_t scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(perm::scratch));
      if (e != hipSuccess) return e;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}
}  // namespace

int permute_noalloc_max_tokens() { return kNoAllocMaxTokens; }

hipError_t launch_permute_noalloc(int T, int H, int E, int K, int align, const int32_t* topk_idx,
                                  const uint16_t* x, int64_t m_cap, int32_t* counts,
                                  int32_t* offsets, int32_t* row_of, int32_t* src_token,
                                  int32_t* tile_expert, uint16_t* x_rows, int32_t* status,
                                  hipStream_t s) {
  if (T > kNoAllocMaxTokens || E > perm::EMAX ||
      permute_workspace_bytes(T, E) > kNoAllocScratchBytes)
    return hipErrorInvalidValue;
  void* ws = nullptr;
  hipError_t e = scratch_on_current_device(&ws);
  if (e != hipSuccess) return e;
  return launch_permute(T, H, E, K, align, topk_idx, x, m_cap, counts, offsets, row_of, src_token,
                        tile_expert, x_rows, ws, status, s);
}

}  // namespace moe
