// Load balancing of the MoE router on gfx950: the auxiliary-loss-free bias
// step, the sequence-wise balance loss (forward and backward), and the
// router gradients of a dense logit gradient.
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
// fp32 products on the vector ALU, 128 x 128 output tiles of 256 threads,
// each thread an 8 x 8 block; k advances 16 at a time through a
// double-buffered LDS stage whose rows are k.  Both operands are staged
// k-major, so a thread reads its 8 rows and 8 columns as two 16-byte words
// each.
constexpr int GT = 128, GK = 16, GNT = 256;

// rows padded by 16 bytes so that the transposing stores of one k column
// fall into different banks
constexpr int GP = GT + 4;
struct alignas(16) Stage {
  float a[GK][GP];
  float b[GK][GP];
};

__device__ __forceinline__ void fma_block(const Stage& st, int ty, int tx, float (&acc)[8][8]) {
#pragma unroll
  for (int k = 0; k < GK; ++k) {
    const f32x4 a0 = *(const f32x4*)&st.a[k][ty * 4];
    const f32x4 a1 = *(const f32x4*)&st.a[k][64 + ty * 4];
    const f32x4 b0 = *(const f32x4*)&st.b[k][tx * 4];
    const f32x4 b1 = *(const f32x4*)&st.b[k][64 + tx * 4];
    const float av[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    const float bv[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
  }
}

// row i of a thread's block is tile row (i < 4 ? ty*4 + i : 64 + ty*4 + i-4)
__device__ __forceinline__ int blk_row(int t, int i) { return i < 4 ? t * 4 + i : 64 + t * 4 + i - 4; }

// dx[t,h] += sum_e dlogit[t,e] * w[h,e]: tile (128 tokens, 128 h), k = e.
// Stage loads: dlogit rows t (k contiguous) and w rows h (k contiguous), both
// transposed into the k-major stage; elements past T, H or E read as zero.
__global__ void __launch_bounds__(GNT) dense_dx_kernel(int T, int H, int E,
                                                       const float* __restrict__ dlogit,
                                                       const float* __restrict__ w,
                                                       float* __restrict__ dx) {
  __shared__ Stage st[2];
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int t0 = blockIdx.y * GT, h0 = blockIdx.x * GT;
  // loader: thread covers (row lr + 16 i, k lk) for i < 8
  const int lk = tid & 15, lr = tid >> 4;
  float acc[8][8] = {};
  auto load = [&](int buf, int k0) {
    const int k = k0 + lk;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = lr + 16 * i;
      const int t = t0 + r, h = h0 + r;
      st[buf].a[lk][r] = (t < T && k < E) ? dlogit[(int64_t)t * E + k] : 0.f;
      st[buf].b[lk][r] = (h < H && k < E) ? w[(int64_t)h * E + k] : 0.f;
    }
  };
  const int nk = (E + GK - 1) / GK;
  load(0, 0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load((kt + 1) & 1, (kt + 1) * GK);
    fma_block(st[kt & 1], ty, tx, acc);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = t0 + blk_row(ty, i);
    if (t >= T) continue;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int h = h0 + half * 64 + tx * 4;
      if (h >= H) continue;  // H % 64 == 0: a 4-column group is all in or all out
      f32x4* p = (f32x4*)(dx + (int64_t)t * H + h);
      f32x4 v = *p;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] += acc[i][half * 4 + j];
      *p = v;
    }
  }
}

// Split-k partial of dW_r: part[s][h,e] = sum over tokens t of slice s of
// x[t,h] * dlogit[t,e].  Tile (128 h, 128 e), k = t; x rows are h-contiguous
// and dlogit rows e-contiguous, so both stage without a transpose.
__global__ void __launch_bounds__(GNT) dense_dw_kernel(int T, int H, int E, int t_per_slice,
                                                       const uint16_t* __restrict__ x,
                                                       const float* __restrict__ dlogit,
                                                       float* __restrict__ part) {
  __shared__ Stage st[2];
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int h0 = blockIdx.x * GT, slice = blockIdx.y;
  const int tb = slice * t_per_slice, te = min(T, tb + t_per_slice);
  // loader: thread covers k row kr and the 8 consecutive columns lc*8
  const int kr = tid >> 4, lc = tid & 15;
  float acc[8][8] = {};
  auto load = [&](int buf, int k0) {
    {
      const int t = k0 + kr;
      const int h = h0 + lc * 8;
      float xv[8], dv[8];
      if (t < te && h < H) {
        const u32x4 raw = *(const u32x4*)(x + (int64_t)t * H + h);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          xv[2 * j] = lo_bf16(raw[j]);
          xv[2 * j + 1] = hi_bf16(raw[j]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) xv[j] = 0.f;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = lc * 8 + j;
        dv[j] = (t < te && e < E) ? dlogit[(int64_t)t * E + e] : 0.f;
      }
      *(f32x4*)&st[buf].a[kr][lc * 8] = f32x4{xv[0], xv[1], xv[2], xv[3]};
      *(f32x4*)&st[buf].a[kr][lc * 8 + 4] = f32x4{xv[4], xv[5], xv[6], xv[7]};
      *(f32x4*)&st[buf].b[kr][lc * 8] = f32x4{dv[0], dv[1], dv[2], dv[3]};
      *(f32x4*)&st[buf].b[kr][lc * 8 + 4] = f32x4{dv[4], dv[5], dv[6], dv[7]};
    }
  };
  const int nk = (te - tb + GK - 1) / GK;
  if (nk > 0) {
    load(0, tb);
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load((kt + 1) & 1, tb + (kt + 1) * GK);
    fma_block(st[kt & 1], ty, tx, acc);
    __syncthreads();
  }
  float* out = part + (int64_t)slice * H * GT;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int h = h0 + blk_row(ty, i);
    if (h >= H) continue;
#pragma unroll
    for (int half = 0; half < 2; ++half)
      *(f32x4*)(out + (int64_t)h * GT + half * 64 + tx * 4) =
          f32x4{acc[i][half * 4], acc[i][half * 4 + 1], acc[i][half * 4 + 2], acc[i][half * 4 + 3]};
  }
}

// dW_r[h,e] += sum_s part[s][h,e], slices in order.
__global__ void __launch_bounds__(256) dense_dw_reduce_kernel(int H, int E, int slices,
                                                              const float* __restrict__ part,
                                                              float* __restrict__ dw) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)H * E) return;
  const int64_t h = i / E, e = i % E;
  float s = dw[i];
  for (int k = 0; k < slices; ++k) s += part[((int64_t)k * H + h) * GT + e];
  dw[i] = s;
}

// token slices of the dW_r split: enough workgroups to cover the CUs twice
__host__ inline int dw_slices(int T, int H) {
  const int tiles = (H + GT - 1) / GT;
  int s = (512 + tiles - 1) / tiles;
  const int by_t = (T + 255) / 256;  // at least 256 tokens per slice
  s = s < by_t ? s : by_t;
  return s < 1 ? 1 : s;
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
  (void)E;
  return (size_t)bal::dw_slices(T, H) * H * bal::GT * 4;
}

hipError_t launch_route_bwd_dense(int T, int H, int E, const uint16_t* x, const float* w_router,
                                  const float* dlogit, float* dw_router, float* dx_router,
                                  void* ws, hipStream_t s) {
  const int slices = bal::dw_slices(T, H);
  const int t_per = ((T + slices - 1) / slices + bal::GK - 1) / bal::GK * bal::GK;
  float* part = (float*)ws;
  hipLaunchKernelGGL(bal::dense_dx_kernel, dim3((H + bal::GT - 1) / bal::GT, (T + bal::GT - 1) / bal::GT),
                     dim3(bal::GNT), 0, s, T, H, E, dlogit, w_router, dx_router);
  hipLaunchKernelGGL(bal::dense_dw_kernel, dim3((H + bal::GT - 1) / bal::GT, slices), dim3(bal::GNT),
                     0, s, T, H, E, t_per, x, dlogit, part);
  const int64_t n = (int64_t)H * E;
  hipLaunchKernelGGL(bal::dense_dw_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     H, E, slices, part, dw_router);
  return hipGetLastError();
}

}  // namespace moe
