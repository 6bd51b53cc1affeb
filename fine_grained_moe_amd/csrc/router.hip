// Router of the MoE layer on gfx950: FP32 gating GEMV, sigmoid scores,
// bias-adjusted top-K selection and normalised combine weights, one kernel.
//
// "dots.llm1 Technical Report" summary page, section "Method": the gating
// projection runs in FP32 for stable routing decisions; balancing uses the
// DeepSeek auxiliary-loss-free bias; top-6 of 128 routed experts.  Model card
// "Model Architecture Features": balancing through dynamic bias terms.
//
// Work split: a 256-thread workgroup owns 32 tokens and all E <= 128 experts;
// each thread holds a 4-token x 4-expert block of fp32 accumulators.  The H
// loop stages 32-wide slices of x (converted to fp32, transposed) and of
// W_r in LDS.  Summation is blocked (32-term partial sums, 16 partials per
// second-level sum) so the fp32 logit stays within ~1e-6 of the exact value.
//
// Selection: one wave per token; lane l owns experts l and l+64.  Keys
// v = s + b are turned into order-preserving 32-bit codes (NaN -> -inf) and
// packed with the inverted expert index, so one 64-bit wave max picks the
// largest key and, among equal keys, the lowest index.  K rounds.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace router {

constexpr int NT = 256, TB = 32, HC = 32, EMAX = 128;

__device__ __forceinline__ uint32_t order_code(float v) {
  if (v != v) v = -__builtin_inff();  // NaN ranks lowest
  uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    uint32_t olo = __shfl_xor(lo, off, 64), ohi = __shfl_xor(hi, off, 64);
    uint64_t o = ((uint64_t)ohi << 32) | olo;
    v = o > v ? o : v;
  }
  return v;
}

__global__ void __launch_bounds__(NT) route_kernel(int T, int H, int E, int K,
                                                   const uint16_t* __restrict__ x,
                                                   const float* __restrict__ w,
                                                   const float* __restrict__ bias,
                                                   int32_t* __restrict__ topk_idx,
                                                   float* __restrict__ topk_w,
                                                   float* __restrict__ topk_s) {
  __shared__ __attribute__((aligned(16))) float xs[2][HC][TB];      // [h][t]
  __shared__ __attribute__((aligned(16))) float ws[2][HC][EMAX];    // [h][e]
  __shared__ float lg[TB][EMAX + 1];

  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * TB;
  const int eg = tid & 31, tg = tid >> 5;  // experts eg*4.., tokens tg*4..

  // staging: x slice 32 tokens x 32 h bf16 = 1024 values -> 4 per thread
  //          w slice 32 h x 128 e fp32 = 4096 values -> 16 per thread (4 x float4)
  const int xt = tid >> 3, xh = (tid & 7) * 4;  // token, h offset (4 bf16)
  uint32_t xr[2];
  f32x4 wr[4];

  auto load = [&](int h0) {
    const int t = t0 + xt;
    if (t < T) {
      const uint32_t* p = (const uint32_t*)(x + (int64_t)t * H + h0 + xh);
      xr[0] = p[0];
      xr[1] = p[1];
    } else {
      xr[0] = xr[1] = 0;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int q = tid + i * NT;          // 0..1023 float4 slots: h = q/32, e4 = q%32
      int hh = q >> 5, e4 = (q & 31) * 4;
      if (e4 < E) {
        const float* p = w + (int64_t)(h0 + hh) * E + e4;
        if (e4 + 4 <= E && (E & 3) == 0) {
          wr[i] = *(const f32x4*)p;
        } else {
          for (int c = 0; c < 4; ++c) wr[i][c] = (e4 + c < E) ? p[c] : 0.f;
        }
      } else {
        wr[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  auto store = [&](int buf) {
    xs[buf][xh + 0][xt] = lo_bf16(xr[0]);
    xs[buf][xh + 1][xt] = hi_bf16(xr[0]);
    xs[buf][xh + 2][xt] = lo_bf16(xr[1]);
    xs[buf][xh + 3][xt] = hi_bf16(xr[1]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int q = tid + i * NT;
      *(f32x4*)&ws[buf][q >> 5][(q & 31) * 4] = wr[i];
    }
  };

  float s2[4][4], s1[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) s2[a][b] = s1[a][b] = 0.f;

  const int nch = H / HC;
  load(0);
  store(0);
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const int cur = c & 1;
    if (c + 1 < nch) load((c + 1) * HC);
    float p[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) p[a][b] = 0.f;
#pragma unroll 8
    for (int hh = 0; hh < HC; ++hh) {
      f32x4 xv = *(const f32x4*)&xs[cur][hh][tg * 4];
      f32x4 wv = *(const f32x4*)&ws[cur][hh][eg * 4];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) p[a][b] = __builtin_fmaf(xv[a], wv[b], p[a][b]);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) s1[a][b] += p[a][b];
    if ((c & 15) == 15 || c + 1 == nch) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          s2[a][b] += s1[a][b];
          s1[a][b] = 0.f;
        }
    }
    if (c + 1 < nch) store(cur ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) lg[tg * 4 + a][eg * 4 + b] = s2[a][b];
  __syncthreads();

  // ---- selection: one wave per token ---------------------------------
  const int lane = tid & 63, wave = tid >> 6;
  for (int tt = wave; tt < TB; tt += NT / 64) {
    const int t = t0 + tt;
    if (t >= T) break;
    float sc[2];
    uint64_t key[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = lane + 64 * q;
      if (e < E) {
        float z = lg[tt][e];
        sc[q] = 1.0f / (1.0f + expf(-z));
        float v = sc[q] + bias[e];
        key[q] = ((uint64_t)order_code(v) << 32) | (uint32_t)(0xFFFFu - e);
      } else {
        sc[q] = 0.f;
        key[q] = 0;
      }
    }
    float ssum = 0.f, my_s = 0.f;
    int my_e = 0;
    for (int k = 0; k < K; ++k) {
      uint64_t m = wave_max_u64(key[0] > key[1] ? key[0] : key[1]);
      const int e = 0xFFFF - (int)(uint32_t)(m & 0xFFFFFFFFu);
      // the owner lane retires the winner and broadcasts its score
      const int owner = e & 63, q = e >> 6;
      float s_own = 0.f;
      if (lane == owner) {
        s_own = sc[q];
        key[q] = 0;
      }
      const float s = __shfl(s_own, owner, 64);
      if (lane == k) {
        my_e = e;
        my_s = s;
      }
      ssum += s;
    }
    if (lane < K) {
      topk_idx[(int64_t)t * K + lane] = my_e;
      topk_w[(int64_t)t * K + lane] = my_s / ssum;
      if (topk_s) topk_s[(int64_t)t * K + lane] = my_s;
    }
  }
}

}  // namespace router

hipError_t launch_route(int T, int H, int E, int K, const uint16_t* x, const float* w_router,
                        const float* bias, int32_t* topk_idx, float* topk_w, float* topk_s,
                        hipStream_t s) {
  const int nb = (T + router::TB - 1) / router::TB;
  hipLaunchKernelGGL(router::route_kernel, dim3(nb), dim3(router::NT), 0, s, T, H, E, K, x,
                     w_router, bias, topk_idx, topk_w, topk_s);
  return hipGetLastError();
}

}  // namespace moe
