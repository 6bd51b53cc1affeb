// Router of the MoE layer on gfx950: FP32 gating projection, sigmoid scores,
// bias-adjusted top-K selection and normalised combine weights.
//
// "dots.llm1 Technical Report" summary page, section "Method": the gating
// projection runs in FP32 for stable routing decisions; balancing uses the
// DeepSeek auxiliary-loss-free bias; top-6 of 128 routed experts.  Model card
// "Model Architecture Features": balancing through dynamic bias terms.
//
// Projection on the matrix cores, exactly in fp32 terms.  x is bf16, so each
// fp32 router weight w is split into three bf16 parts w = hi + mid + lo
// (hi = bf16(w), mid = bf16(w - hi), lo = bf16(w - hi - mid); each difference
// is exact in fp32 and the three parts carry w's 24-bit significand).  Every
// product x * part is exact in the MFMA's fp32 accumulator, so
//   logit = sum_h x[h] * (hi + mid + lo)[h]
// is the fp32 dot product up to accumulation rounding.  The accumulation is
// blocked (per lane, each 32x32 block sums 512 h at a time, then adds into a
// running fp32 total) so the logit stays within a few 1e-7 of the exact value.
//
// split_kernel writes the three parts in MFMA fragment order (one 1 KB block
// per part, 32-expert block and 16-deep k-step: lane l's 16 bytes are the
// eight k of expert l%32 at k offset 8*(l/32)), so every operand load is one
// contiguous 1 KB LDS-DMA.  route_kernel: a 256-thread workgroup owns TB
// tokens and all E <= 128 experts; wave w computes the TB x 32 logit block of
// experts 32w.., with x tiles (K-contiguous, swizzled) and weight fragments
// streamed into an LDS ring (64 tokens: 5 stages of 32 h; 32 tokens: 3 of 64).
//
// Selection: one wave per token; lane l owns experts l and l+64.  Keys
// v = s + b are turned into order-preserving 32-bit codes (NaN -> -inf) and
// packed with the inverted expert index, so one 64-bit wave max picks the
// largest key and, among equal keys, the lowest index.  K rounds.
#include "common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace moe {
namespace router {

using namespace lds;

#ifndef MOE_ROUTE_TB
#define MOE_ROUTE_TB 32
#endif
constexpr int NT = 256, NW = 4, EMAX = 128, EBMAX = EMAX / 32;
constexpr int TB = MOE_ROUTE_TB;                              // tokens per workgroup
constexpr int BK = TB == 64 ? 32 : 64, STAGES = TB == 64 ? 5 : 3;
constexpr int TM = TB / 32;                                   // 32-token blocks per wave
constexpr int KK = BK / 16;                                   // k-steps per stage
constexpr int A_BYTES = TB * BK * 2;                          // x tile
constexpr int B_REGIONS = 3 * EBMAX * KK;                     // weight fragments per stage
constexpr int STAGE_BYTES = A_BYTES + B_REGIONS * 1024;
constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
constexpr int A_PER = KcLoad<TB, BK, NW>::PER;                // x regions per wave
constexpr int B_PER = B_REGIONS / NW;                         // weight regions per wave
constexpr int LOADS = A_PER + B_PER;
constexpr int SUM_BLOCK = 512 / BK;                           // stages per partial sum (512 h)
static_assert(B_REGIONS % NW == 0, "weight regions per wave");
static_assert(LDS_BYTES <= 160 * 1024, "LDS");
static_assert(TB * (EMAX + 1) * 4 <= LDS_BYTES, "logit tile fits the ring");

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

// wf[p][eb][ks][lane][8]: part p of w_router[16 ks + 8 (lane/32) + j][32 eb + lane%32]
__global__ void __launch_bounds__(64) split_kernel(int H, int E, const float* __restrict__ w,
                                                   uint16_t* __restrict__ wf) {
  const int lane = threadIdx.x;
  const int ks = blockIdx.x, eb = blockIdx.y;
  const int nks = H / 16, EB = gridDim.y;
  const int e = 32 * eb + (lane & 31);
  const int k0 = 16 * ks + 8 * (lane >> 5);
  uint32_t part[3][4];
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    float v[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) v[q] = e < E ? w[(int64_t)(k0 + j + q) * E + e] : 0.f;
    uint16_t b[3][2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint16_t hi = f32_to_bf16(v[q]);
      const float r1 = v[q] - bf16_to_f32(hi);
      const uint16_t mid = f32_to_bf16(r1);
      const float r2 = r1 - bf16_to_f32(mid);
      b[0][q] = hi;
      b[1][q] = mid;
      b[2][q] = f32_to_bf16(r2);
    }
#pragma unroll
    for (int p = 0; p < 3; ++p) part[p][j / 2] = (uint32_t)b[p][0] | ((uint32_t)b[p][1] << 16);
  }
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    const int64_t blk = ((int64_t)p * EB + eb) * nks + ks;
    *(u32x4*)(wf + blk * 512 + lane * 8) = u32x4{part[p][0], part[p][1], part[p][2], part[p][3]};
  }
}

__global__ void __launch_bounds__(NT, 1) route_kernel(int T, int H, int E, int K,
                                                      const uint16_t* __restrict__ x,
                                                      const uint16_t* __restrict__ wf,
                                                      const float* __restrict__ bias,
                                                      int32_t* __restrict__ topk_idx,
                                                      float* __restrict__ topk_w,
                                                      float* __restrict__ topk_s,
                                                      float* __restrict__ scores) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = blockIdx.x * TB;
  const int EB = (E + 31) / 32, nks = H / 16, nk = H / BK;

  // operand sources: x rows t0.. (rows past T read as zeros), weight fragments
  const int rows_valid = min(TB, T - t0);
  const u32x4 rX = make_rsrc(x + (int64_t)t0 * H, (uint32_t)(rows_valid * H * 2));
  const u32x4 rW = make_rsrc(wf, (uint32_t)(3 * EB * nks * 1024));
  KcLoad<TB, BK, NW> lx;
  lx.init([&](int r) -> uint32_t { return r < rows_valid ? (uint32_t)(r * H * 2) : kOOB; }, wave,
          lane);
  const uint32_t smem_base = lds_addr(smem);
  auto issue = [&](int kt) {
    const uint32_t As = smem_base + (kt % STAGES) * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < A_PER; ++i) lx.issue(rX, As, wave, i, kt, H);
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      const int r = i * NW + wave;                 // region: part, expert block, k-step
      const int p = r / (EBMAX * KK), eb = (r / KK) % EBMAX, kl = r % KK;
      const int ks = kt * KK + kl;
      const uint32_t off = (eb < EB && ks < nks)
                               ? (uint32_t)((((p * EB + eb) * nks) + ks) * 1024 + lane * 16)
                               : kOOB;
      dma16(rW, As + A_BYTES + r * 1024, off);
    }
  };

  f32x16 acc[TM], tot[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = tot[i][r] = 0.f;
  const bool active = wave < EB;

  // branch-free ring: loads past the last stage read as zeros
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) issue(s);
  for (int kt = 0; kt < nk; ++kt) {
    wait_vmcnt<LOADS * (STAGES - 2)>();
    lds_barrier();
    issue(kt + STAGES - 1);  // into the buffer every wave finished reading
    const uint8_t* As = smem + (kt % STAGES) * STAGE_BYTES;
    const uint8_t* Bs = As + A_BYTES;
    if (active) {
      bf16x8 af[KK][TM], bq[KK][3];
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
        for (int i = 0; i < TM; ++i) af[kk][i] = frag_kc<BK>(As, 32 * i, kk, lane);
#pragma unroll
        for (int p = 0; p < 3; ++p)
          bq[kk][p] = *(const bf16x8*)(Bs + ((p * EBMAX + wave) * KK + kk) * 1024 + lane * 16);
      }
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int p = 0; p < 3; ++p)
#pragma unroll
          for (int i = 0; i < TM; ++i)
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bq[kk][p], af[kk][i], acc[i], 0, 0, 0);
    }
    if ((kt % SUM_BLOCK) == SUM_BLOCK - 1 || kt + 1 == nk) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          tot[i][r] += acc[i][r];
          acc[i][r] = 0.f;
        }
    }
  }
  wait_vmcnt<0>();
  lds_barrier();

  // logits -> LDS [token][expert]: lane holds token 32i + l%32 and experts
  // 32w + 8(r/4) + 4(l/32) + r%4
  float* lg = (float*)smem;
  constexpr int LP = EMAX + 1;
  if (active) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        lg[(32 * i + (lane & 31)) * LP + 32 * wave + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)] =
            tot[i][r];
  }
  lds_barrier();

  // ---- selection: one wave per token ---------------------------------
  for (int tt = wave; tt < TB; tt += NW) {
    const int t = t0 + tt;
    if (t >= T) break;
    float sc[2];
    uint64_t key[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = lane + 64 * q;
      if (e < E) {
        const float z = lg[tt * LP + e];
        sc[q] = 1.0f / (1.0f + expf(-z));
        if (scores) scores[(int64_t)t * E + e] = sc[q];
        const float v = sc[q] + bias[e];
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

size_t route_workspace_bytes(int H, int E) {
  return (size_t)3 * ((E + 31) / 32) * 32 * (size_t)H * 2;
}

hipError_t launch_route(int T, int H, int E, int K, const uint16_t* x, const float* w_router,
                        const float* bias, int32_t* topk_idx, float* topk_w, float* topk_s,
                        float* scores, void* ws, hipStream_t s) {
  uint16_t* wf = (uint16_t*)ws;
  hipLaunchKernelGGL(router::split_kernel, dim3(H / 16, (E + 31) / 32), dim3(64), 0, s, H, E,
                     w_router, wf);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || T == 0) return e;
  const int nb = (T + router::TB - 1) / router::TB;
  hipLaunchKernelGGL(router::route_kernel, dim3(nb), dim3(router::NT), 0, s, T, H, E, K, x, wf,
                     bias, topk_idx, topk_w, topk_s, scores);
  return hipGetLastError();
}

}  // namespace moe
