// Load balancing of the MoE router on gfx950: the auxiliary-loss-free bias
// step, the sequence-wise balance loss (forward and backward), and the
// router gradients of a dense logit gradient (into which the combine path's
// K-per-token logit gradient can first be added, so that one dense pass gives
// the router gradients of both).
//
// dots.llm1 Technical Report summary, section "Method": load balancing by
// DeepSeek's auxiliary-loss-free bias update, complemented by a sequence-wise
// balance loss for extreme imbalance within a sequence; model card, "Model
// Architecture Features": dynamic bias terms.  The pages give neither the
// update rule nor the loss, so both follow DeepSeek's published forms:
//   bias step   bias[e] += gamma * sign(mean load - load[e])
//   loss        per sequence of L tokens, alpha * sum_i f_i P_i with
//               f_i = E/(K L) * (tokens of the sequence that picked i) and
//               P_i = mean over the sequence of s[t,i] / sum_j s[t,j];
//               a batch of B sequences takes the mean over them.
// Every reduction runs in a fixed order, so results are bit-reproducible.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace bal {

constexpr int EMAX = 128;  // experts per token handled by one wave (two per lane)

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// ---- bias step ------------------------------------------------------------
// One workgroup of EMAX threads, thread e owns expert e.  The load of e is
// compared with the mean in integers (E * counts[e] against the total), so
// the decision is exact; the update is a single fp32 addition.
__global__ void __launch_bounds__(EMAX) bias_update_kernel(int E, const int32_t* __restrict__ counts,
                                                           float* __restrict__ bias, float gamma) {
  __shared__ long long wsum[EMAX / 64];
  const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
  const long long c = e < E ? (long long)counts[e] : 0;
  long long s = c;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if (lane == 0) wsum[wave] = s;
  __syncthreads();
  long long total = 0;
#pragma unroll
  for (int w = 0; w < EMAX / 64; ++w) total += wsum[w];
  if (e < E) {
    const long long excess = (long long)E * c - total;  // sign of load - mean
    const float dir = excess < 0 ? 1.0f : (excess > 0 ? -1.0f : 0.0f);
    bias[e] = bias[e] + dir * gamma;
  }
}

// ---- sequence-wise balance loss, forward ---------------------------------
// Pass 1: workgroup (sequence b, chunk c) takes CH tokens of sequence b;
// wave w takes TPW of them (all their loads issued first), lane l owns
// experts l and l + 64.  It adds up, per expert, the normalised scores
// s[t,e] / sum_j s[t,j] and the picks of its tokens in token order, then
// writes the chunk's partial sums (waves added in wave order).
constexpr int CH = 32, NT = 256, NW = NT / 64, TPW = CH / NW;

__global__ void __launch_bounds__(NT) seq_partial_kernel(int T, int E, int K, int L, int nch,
                                                         const float* __restrict__ scores,
                                                         const int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ psum,
                                                         int32_t* __restrict__ picks) {
  __shared__ float sp[NW][EMAX];
  __shared__ int32_t sk[NW][EMAX];
  const int b = blockIdx.x / nch, c = blockIdx.x % nch;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t_lo = b * L + c * CH, t_hi = min(b * L + min(L, (c + 1) * CH), T);
  float acc[2] = {0.f, 0.f};
  int cnt[2] = {0, 0};
  float s[TPW][2];
  int pick[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int t = t_lo + wave * TPW + j;
    const bool ok = t < t_hi;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = lane + 64 * q;
      s[j][q] = (ok && e < E) ? scores[(int64_t)t * E + e] : 0.f;
    }
    pick[j] = (ok && lane < K) ? topk_idx[(int64_t)t * K + lane] : -1;
  }
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    if (t_lo + wave * TPW + j >= t_hi) break;
    const float inv = 1.0f / wave_sum(s[j][0] + s[j][1]);
    for (int k = 0; k < K; ++k) {
      const int ek = __shfl(pick[j], k, 64);
      cnt[0] += ek == lane;
      cnt[1] += ek == lane + 64;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) acc[q] += s[j][q] * inv;
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    sp[wave][lane + 64 * q] = acc[q];
    sk[wave][lane + 64 * q] = cnt[q];
  }
  __syncthreads();
  if (threadIdx.x < EMAX) {
    const int e = threadIdx.x;
    float p = 0.f;
    int n = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      p += sp[w][e];
      n += sk[w][e];
    }
    if (e < E) {
      psum[(int64_t)blockIdx.x * E + e] = p;
      picks[(int64_t)blockIdx.x * E + e] = n;
    }
  }
}

// Pass 2: workgroup b adds its chunks in order and forms f, P and the
// sequence's loss alpha * sum_e f_e P_e.
__global__ void __launch_bounds__(EMAX) seq_final_kernel(int E, int K, int L, int nch, float alpha,
                                                         const float* __restrict__ psum,
                                                         const int32_t* __restrict__ picks,
                                                         float* __restrict__ seq_f,
                                                         float* __restrict__ seq_loss) {
  __shared__ float wsum[EMAX / 64];
  const int b = blockIdx.x, e = threadIdx.x, lane = e & 63, wave = e >> 6;
  float term = 0.f;
  if (e < E) {
    float p = 0.f;
    int n = 0;
#pragma unroll 8
    for (int c = 0; c < nch; ++c) {
      p += psum[((int64_t)b * nch + c) * E + e];
      n += picks[((int64_t)b * nch + c) * E + e];
    }
    const float f = (float)((double)E * n / ((double)K * L));
    seq_f[(int64_t)b * E + e] = f;
    term = f * (p / (float)L);
  }
  term = wave_sum(term);
  if (lane == 0) wsum[wave] = term;
  __syncthreads();
  if (e == 0) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < EMAX / 64; ++w) s += wsum[w];
    seq_loss[b] = alpha * s;
  }
}

// Pass 3: one workgroup, loss = mean over the B sequences (fixed order).
__global__ void __launch_bounds__(256) seq_mean_kernel(int B, const float* __restrict__ seq_loss,
                                                       float* __restrict__ loss) {
  __shared__ float part[4];
  const int tid = threadIdx.x;
  float s = 0.f;
  for (int b = tid; b < B; b += 256) s += seq_loss[b];
  s = wave_sum(s);
  if ((tid & 63) == 0) part[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) loss[0] = (part[0] + part[1] + part[2] + part[3]) / (float)B;
}

// ---- sequence-wise balance loss, backward --------------------------------
// One wave per token: with c_e = dloss * alpha * f[b,e] / (B L),
//   ds_e = (c_e - sum_i c_i s_i / S) / S,  S = sum_i s_i,
//   dlogit_e = ds_e * s_e * (1 - s_e)      for every expert e.
__global__ void __launch_bounds__(NT) seq_bwd_kernel(int T, int E, int L, int B, float alpha,
                                                     const float* __restrict__ scores,
                                                     const float* __restrict__ seq_f,
                                                     const float* __restrict__ dloss,
                                                     float* __restrict__ dlogit) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * NW + (threadIdx.x >> 6);
  if (t >= T) return;
  const int b = t / L;
  const float scale = (dloss ? dloss[0] : 1.0f) * alpha / ((float)B * (float)L);
  float s[2], c[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = lane + 64 * q;
    s[q] = e < E ? scores[(int64_t)t * E + e] : 0.f;
    c[q] = e < E ? scale * seq_f[(int64_t)b * E + e] : 0.f;
  }
  const float S = wave_sum(s[0] + s[1]);
  const float cs = wave_sum(c[0] * s[0] + c[1] * s[1]) / S;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = lane + 64 * q;
    if (e < E) dlogit[(int64_t)t * E + e] = (c[q] - cs) / S * s[q] * (1.0f - s[q]);
  }
}

// ---- router gradients of a dense logit gradient --------------------------
// Both products run on the bf16 matrix cores through the grouped-GEMM kernel.
// Every fp32 operand v is split exactly into three bf16 parts,
//   hi = bf16(v), mid = bf16(v - hi), lo = bf16(v - hi - mid),
// whose sum is v to about 2^-27 |v|.  x is bf16 already.
//   dW_r = x^T dlogit          = x^T (d_hi + d_mid + d_lo): three exact products
//   dx_r = dlogit W_r^T        = the six part products down to 2^-16 of the
//                                leading one (hi.hi, hi.mid, mid.hi, hi.lo,
//                                lo.hi, mid.mid); the three left out are below
//                                fp32 rounding
// Each part block is padded to EP = E rounded up to 8 columns (zeros).  dx_r
// takes one GEMM with the six blocks laid side by side along K; dW_r takes one
// K-grouped GEMM over G token slices with the three parts side by side along
// N, whose fp32 partial results are then added in a fixed order.
__device__ __forceinline__ void split3(float v, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
  hi = f32_to_bf16(v);
  const float r1 = v - bf16_to_f32(hi);
  mid = f32_to_bf16(r1);
  lo = f32_to_bf16(r1 - bf16_to_f32(mid));
}

// part order of the six K blocks: dlogit side and W_r side
__constant__ int kPartA[6] = {0, 0, 1, 0, 2, 1};
__constant__ int kPartB[6] = {0, 1, 0, 2, 0, 1};

// src [R, E] fp32 -> six [R, EP] blocks along each row of dst6 ([R, 6 EP],
// parts in `order`), and, when dst3 is given, the three parts in order along
// each row of dst3 ([R, 3 EP]).  Columns E..EP-1 are zero.
__global__ void __launch_bounds__(256) split_rows_kernel(int R, int E, int EP, int side,
                                                         const float* __restrict__ src,
                                                         uint16_t* __restrict__ dst6,
                                                         uint16_t* __restrict__ dst3) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)R * EP) return;
  const int64_t r = i / EP;
  const int e = (int)(i % EP);
  const float v = e < E ? src[r * E + e] : 0.f;
  uint16_t part[3];
  split3(v, part[0], part[1], part[2]);
  const int* order = side == 0 ? kPartA : kPartB;
#pragma unroll
  for (int q = 0; q < 6; ++q) dst6[r * 6 * EP + q * EP + e] = part[order[q]];
  if (dst3) {
#pragma unroll
    for (int q = 0; q < 3; ++q) dst3[r * 3 * EP + q * EP + e] = part[q];
  }
}

// token slices of the weight-gradient product
__global__ void seg_kernel(int G, int S, int T, int32_t* __restrict__ offsets,
                           int32_t* __restrict__ counts) {
  const int g = threadIdx.x;
  if (g > G) return;
  const int o = min(g * S, T);
  offsets[g] = o;
  if (g < G) counts[g] = min(S, T - o);
}

// dW_r[h,e] += sum over slices g and parts p of part[g][h][p EP + e]
__global__ void __launch_bounds__(256) dw_reduce_kernel(int H, int E, int EP, int G, int acc,
                                                        const float* __restrict__ part,
                                                        float* __restrict__ dw) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)H * E) return;
  const int64_t h = i / E;
  const int e = (int)(i % E);
  float s = acc ? dw[i] : 0.f;
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int p = 0; p < 3; ++p) s += part[((int64_t)g * H + h) * 3 * EP + p * EP + e];
  dw[i] = s;
}

// the combine path's logit gradient added into a dense [T,E] one: per token,
// S = sum_j s_j, ds_k = (dg_k - sum_j s_j dg_j / S) / S and
// dlogit[t, topk_idx[t,k]] += ds_k s_k (1 - s_k).  One thread per token; the K
// experts of a token are distinct, so every entry has one writer.
__global__ void __launch_bounds__(256) route_dlogit_kernel(int T, int E, int K,
                                                           const int32_t* __restrict__ topk_idx,
                                                           const float* __restrict__ topk_s,
                                                           const float* __restrict__ dg,
                                                           float* __restrict__ dlogit) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  const int64_t o = (int64_t)t * K;
  float ssum = 0.f, sdg = 0.f;
  for (int k = 0; k < K; ++k) {
    const float s = topk_s[o + k];
    ssum += s;
    sdg += s * dg[o + k];
  }
  for (int k = 0; k < K; ++k) {
    const float s = topk_s[o + k];
    const float ds = (dg[o + k] - sdg / ssum) / ssum;
    float* d = dlogit + (int64_t)t * E + topk_idx[o + k];
    *d += ds * s * (1.0f - s);
  }
}

// token slices for dW_r: enough workgroups for the CUs (the grouped kernel
// tiles 256 x 256), at least 256 tokens each
__host__ inline int dw_slices(int T, int H, int EP) {
  const int tiles = ((H + 255) / 256) * ((3 * EP + 255) / 256);
  int g = (512 + tiles - 1) / tiles;
  const int by_t = (T + 255) / 256;
  g = g < by_t ? g : by_t;
  g = g < 255 ? g : 255;  // seg_kernel: one thread per slice boundary
  return g < 1 ? 1 : g;
}

struct DenseWs {
  uint16_t *a6, *w6, *d3;
  int32_t *offsets, *counts;
  float* part;
  size_t bytes;
};

__host__ inline size_t al256(size_t n) { return (n + 255) / 256 * 256; }

__host__ inline DenseWs dense_ws(int T, int H, int E, void* base) {
  const int EP = (E + 7) / 8 * 8, G = dw_slices(T, H, EP);
  const uintptr_t p = (uintptr_t)base;
  DenseWs w;
  size_t o = 0;
  w.a6 = (uint16_t*)(p + o); o += al256((size_t)T * 6 * EP * 2);
  w.w6 = (uint16_t*)(p + o); o += al256((size_t)H * 6 * EP * 2);
  w.d3 = (uint16_t*)(p + o); o += al256((size_t)T * 3 * EP * 2);
  w.offsets = (int32_t*)(p + o); o += al256((size_t)(G + 1) * 4);
  w.counts = (int32_t*)(p + o); o += al256((size_t)G * 4);
  w.part = (float*)(p + o); o += al256((size_t)G * H * 3 * EP * 4);
  w.bytes = o;
  return w;
}

}  // namespace bal

hipError_t launch_bias_update(int E, const int32_t* counts, float* bias, float gamma,
                              hipStream_t s) {
  hipLaunchKernelGGL(bal::bias_update_kernel, dim3(1), dim3(bal::EMAX), 0, s, E, counts, bias,
                     gamma);
  return hipGetLastError();
}

size_t seq_balance_workspace_bytes(int T, int E, int L) {
  const int64_t B = T / L, nch = (L + bal::CH - 1) / bal::CH;
  const size_t part = (size_t)B * nch * E * 4;
  const size_t a = (part + 255) / 256 * 256;
  return 2 * a + ((size_t)B * 4 + 255) / 256 * 256;
}

hipError_t launch_seq_balance_fwd(int T, int E, int K, int L, const float* scores,
                                  const int32_t* topk_idx, float alpha, float* loss, float* seq_f,
                                  void* ws, hipStream_t s) {
  const int B = T / L, nch = (L + bal::CH - 1) / bal::CH;
  const size_t part = ((size_t)B * nch * E * 4 + 255) / 256 * 256;
  float* psum = (float*)ws;
  int32_t* picks = (int32_t*)((uint8_t*)ws + part);
  float* seq_loss = (float*)((uint8_t*)ws + 2 * part);
  hipLaunchKernelGGL(bal::seq_partial_kernel, dim3(B * nch), dim3(bal::NT), 0, s, T, E, K, L, nch,
                     scores, topk_idx, psum, picks);
  hipLaunchKernelGGL(bal::seq_final_kernel, dim3(B), dim3(bal::EMAX), 0, s, E, K, L, nch, alpha,
                     psum, picks, seq_f, seq_loss);
  hipLaunchKernelGGL(bal::seq_mean_kernel, dim3(1), dim3(256), 0, s, B, seq_loss, loss);
  return hipGetLastError();
}

hipError_t launch_seq_balance_bwd(int T, int E, int L, const float* scores, const float* seq_f,
                                  float alpha, const float* dloss, float* dlogit, hipStream_t s) {
  const int B = T / L;
  hipLaunchKernelGGL(bal::seq_bwd_kernel, dim3((T + bal::NW - 1) / bal::NW), dim3(bal::NT), 0, s,
                     T, E, L, B, alpha, scores, seq_f, dloss, dlogit);
  return hipGetLastError();
}

size_t route_bwd_dense_workspace_bytes(int T, int H, int E) {
  return bal::dense_ws(T, H, E, nullptr).bytes;
}

int64_t route_bwd_dense_slice_rows(int T, int H, int E) {
  const int G = bal::dw_slices(T, H, (E + 7) / 8 * 8);
  return ((int64_t)T + G - 1) / G;
}

hipError_t launch_route_dlogit(int T, int E, int K, const int32_t* topk_idx, const float* topk_s,
                               const float* dg, float* dlogit, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(bal::route_dlogit_kernel, dim3((T + 255) / 256), dim3(256), 0, s, T, E, K,
                     topk_idx, topk_s, dg, dlogit);
  return hipGetLastError();
}

hipError_t launch_route_bwd_dense(int T, int H, int E, const uint16_t* x, const float* w_router,
                                  const float* dlogit, float* dw_router, float* dx_router,
                                  bool accumulate, void* ws, hipStream_t s) {
  if (T == 0) {  // no tokens: the written weight gradient is zero
    if (!accumulate)
      hipLaunchKernelGGL(bal::dw_reduce_kernel, dim3((unsigned)(((int64_t)H * E + 255) / 256)),
                         dim3(256), 0, s, H, E, E, 0, 0, (const float*)nullptr, dw_router);
    return hipGetLastError();
  }
  const int EP = (E + 7) / 8 * 8, G = bal::dw_slices(T, H, EP);
  const bal::DenseWs w = bal::dense_ws(T, H, E, ws);
  const int S = (T + G - 1) / G;
  hipLaunchKernelGGL(bal::split_rows_kernel, dim3((unsigned)(((int64_t)T * EP + 255) / 256)),
                     dim3(256), 0, s, T, E, EP, 0, dlogit, w.a6, w.d3);
  hipLaunchKernelGGL(bal::split_rows_kernel, dim3((unsigned)(((int64_t)H * EP + 255) / 256)),
                     dim3(256), 0, s, H, E, EP, 1, w_router, w.w6, (uint16_t*)nullptr);
  hipLaunchKernelGGL(bal::seg_kernel, dim3(1), dim3(256), 0, s, G, S, T, w.offsets, w.counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dx_r += [d parts] . [W_r parts]^T, K = 6 EP
  e = launch_gemm_f32_nt(T, H, 6 * EP, w.a6, 6 * EP, w.w6, 6 * EP, dx_router, H, accumulate, s);
  if (e != hipSuccess) return e;
  // part[g] = x_g^T [d_hi | d_mid | d_lo]_g, then dW_r += the sum of the parts
  e = launch_gemm_f32_tn_grouped(G, w.offsets, w.counts, T, H, 3 * EP, x, H, w.d3, 3 * EP, w.part,
                                 3 * EP, (int64_t)H * 3 * EP, s);
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)H * E;
  hipLaunchKernelGGL(bal::dw_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, H,
                     E, EP, G, accumulate ? 1 : 0, w.part, dw_router);
  return hipGetLastError();
}

}  // namespace moe
