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
// blocked: each 32x32 block sums 512 h at a time into a running fp32 total per
// slice of h, and the slices' totals are added in slice order, so the logit
// stays within a few 1e-7 of the exact value and does not depend on timing.
//
// split_kernel writes the three parts in MFMA fragment order (one 1 KB block
// per part, 32-expert block and 16-deep k-step: lane l's 16 bytes are the
// eight k of expert l%32 at k offset 8*(l/32)), so every operand load is one
// contiguous 1 KB LDS-DMA.
//
// proj_kernel: a workgroup owns 128 tokens, all E <= 128 experts and one slice
// of h (H split into S slices so that the grid has about 256 workgroups).
// Every workgroup streams the weight parts of its slice once for 128 tokens:
// with 32-token workgroups over the whole of h the weight stream (3.9 MB per
// workgroup at dots shapes) was 12x the x stream and set the kernel's time.
// Eight waves: wave w computes the 64 x 32 logit block of tokens 64 (w/4)..
// and experts 32 (w%4).., with x tiles (K-contiguous, swizzled) and weight
// fragments in a 4-stage LDS ring of 32-deep stages.  The slice's logits go to
// the workspace through LDS with coalesced row stores.
//
// select_kernel: one wave per token adds the S slice logits in slice order,
// then selects.  Lane l owns experts l and l+64.  Keys v = s + b are turned
// into order-preserving 32-bit codes (NaN -> -inf) and packed with the
// inverted expert index, so one 64-bit wave max picks the largest key and,
// among equal keys, the lowest index.  K rounds.
#include "common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace moe {
namespace router {

using namespace lds;

constexpr int NT = 512, NW = 8, EMAX = 128, EBMAX = EMAX / 32;
constexpr int TB = 128;                                       // tokens per workgroup
constexpr int BK = 32, STAGES = 4;                            // h per stage, ring depth
constexpr int TM = 2;                                         // 32-token blocks per wave
constexpr int KK = BK / 16;                                   // k-steps per stage
constexpr int A_BYTES = TB * BK * 2;                          // x tile
constexpr int B_REGIONS = 3 * EBMAX * KK;                     // weight fragments per stage
constexpr int STAGE_BYTES = A_BYTES + B_REGIONS * 1024;
constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
constexpr int A_PER = KcLoad<TB, BK, NW>::PER;                // x regions per wave
constexpr int B_PER = B_REGIONS / NW;                         // weight regions per wave
constexpr int LOADS = A_PER + B_PER;
constexpr int SUM_BLOCK = 512 / BK;                           // stages per partial sum (512 h)
constexpr int LP = EMAX + 1;                                  // LDS pitch of the logit tile
constexpr int WG_TARGET = 256;                                // workgroups to aim for
constexpr int S_MAX = 64;                                     // h slices at most
static_assert(B_REGIONS % NW == 0, "weight regions per wave");
static_assert(TM * 32 * 2 == TB && NW == 2 * EBMAX, "wave layout: 2 token halves x 4 expert blocks");
static_assert(LDS_BYTES <= 160 * 1024, "LDS");
static_assert(TB * LP * 4 <= LDS_BYTES, "logit tile fits the ring");

// number of h slices for T tokens: doubled while the grid stays below
// WG_TARGET workgroups and every slice remains a whole number of stages
__host__ __device__ inline int slices(int T, int H) {
  const int ntok = (T + TB - 1) / TB;
  int S = 1;
  while (S < S_MAX && ntok * S < WG_TARGET && H % (2 * S * BK) == 0) S *= 2;
  return S;
}

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

__global__ void __launch_bounds__(NT, 1) proj_kernel(int T, int H, int E, int S,
                                                     const uint16_t* __restrict__ x,
                                                     const uint16_t* __restrict__ wf,
                                                     float* __restrict__ part) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int eb = wave % EBMAX, th = wave / EBMAX;  // expert block, token half
  const int t0 = blockIdx.x * TB, sl = blockIdx.y;
  const int EB = (E + 31) / 32, nks = H / 16;
  const int HS = H / S, nk = HS / BK;              // h per slice, stages per slice
  const int h0 = sl * HS;

  // operand sources: x rows t0.. (rows past T read as zeros) at columns h0..,
  // weight fragments of k-steps h0/16..
  const int rows_valid = min(TB, T - t0);
  const u32x4 rX = make_rsrc(x + (int64_t)t0 * H, (uint32_t)(rows_valid * H * 2));
  const u32x4 rW = make_rsrc(wf, (uint32_t)(3 * EB * nks * 1024));
  KcLoad<TB, BK, NW> lx;
  lx.init([&](int r) -> uint32_t { return r < rows_valid ? (uint32_t)((r * H + h0) * 2) : kOOB; },
          wave, lane);
  const uint32_t smem_base = lds_addr(smem);
  auto issue = [&](int kt) {
    const uint32_t As = smem_base + (kt % STAGES) * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < A_PER; ++i) lx.issue(rX, As, wave, i, kt, HS);
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      const int r = i * NW + wave;                 // region: part, expert block, k-step
      const int p = r / (EBMAX * KK), rb = (r / KK) % EBMAX, kl = r % KK;
      const int ks = h0 / 16 + kt * KK + kl;
      const uint32_t off = (rb < EB && kt < nk && ks < nks)
                               ? (uint32_t)((((p * EB + rb) * nks) + ks) * 1024 + lane * 16)
                               : kOOB;
      dma16(rW, As + A_BYTES + r * 1024, off);
    }
  };

  f32x16 acc[TM], tot[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = tot[i][r] = 0.f;
  const bool active = eb < EB;

  // branch-free ring: loads past the slice's last stage read as zeros
#pragma unroll
  for (int st = 0; st < STAGES - 1; ++st) issue(st);
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
        for (int i = 0; i < TM; ++i) af[kk][i] = frag_kc<BK>(As, 64 * th + 32 * i, kk, lane);
#pragma unroll
        for (int p = 0; p < 3; ++p)
          bq[kk][p] = *(const bf16x8*)(Bs + ((p * EBMAX + eb) * KK + kk) * 1024 + lane * 16);
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

  // logits -> LDS [token][expert]: lane holds token 64 th + 32 i + l%32 and
  // experts 32 eb + 8(r/4) + 4(l/32) + r%4 (zeros for experts past E)
  float* lg = (float*)smem;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      lg[(64 * th + 32 * i + (lane & 31)) * LP + 32 * eb + 8 * (r >> 2) + 4 * (lane >> 5) +
         (r & 3)] = active ? tot[i][r] : 0.f;
  lds_barrier();

  // slice logits -> part[sl][t][0..EMAX): every thread moves 16-byte chunks
  constexpr int CPR = EMAX / 4;  // chunks per row
#pragma unroll 4
  for (int q = tid; q < TB * CPR; q += NT) {
    const int r = q / CPR, c = q % CPR;
    if (r < rows_valid) {
      const float* src = lg + r * LP + 4 * c;
      *(f32x4*)(part + ((int64_t)sl * T + t0 + r) * EMAX + 4 * c) =
          f32x4{src[0], src[1], src[2], src[3]};
    }
  }
}

// one wave per token: logit = sum of the S slice logits in slice order, then
// score, key, top-K and normalised weights
constexpr int SEL_NT = 256, SEL_TPB = SEL_NT / 64;
__global__ void __launch_bounds__(SEL_NT) select_kernel(int T, int E, int K, int S,
                                                        const float* __restrict__ part,
                                                        const float* __restrict__ bias,
                                                        int32_t* __restrict__ topk_idx,
                                                        float* __restrict__ topk_w,
                                                        float* __restrict__ topk_s,
                                                        float* __restrict__ scores) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * SEL_TPB + (threadIdx.x >> 6);
  if (t >= T) return;
  // slice logits: eight slices' loads in flight at a time (small batches run
  // with up to 64 slices), added in slice order
  float z[2] = {0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += 8) {
    float v[8][2];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int q = 0; q < 2; ++q)
        v[u][q] = (s0 + u < S && lane + 64 * q < E)
                      ? part[((int64_t)(s0 + u) * T + t) * EMAX + lane + 64 * q]
                      : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int q = 0; q < 2; ++q)
        if (s0 + u < S) z[q] += v[u][q];
  }
  float sc[2];
  uint64_t key[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = lane + 64 * q;
    if (e < E) {
      sc[q] = 1.0f / (1.0f + expf(-z[q]));
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

}  // namespace router

// workspace: the weight parts (3 x 32 EB x H bf16), then the slice logits
// (S x T x 128 fp32), 256-byte aligned
static size_t route_parts_bytes(int H, int E) {
  return ((size_t)3 * ((E + 31) / 32) * 32 * (size_t)H * 2 + 255) / 256 * 256;
}

size_t route_workspace_bytes(int T, int H, int E) {
  return route_parts_bytes(H, E) +
         (size_t)router::slices(T, H) * (size_t)T * router::EMAX * sizeof(float);
}

hipError_t launch_route(int T, int H, int E, int K, const uint16_t* x, const float* w_router,
                        const float* bias, int32_t* topk_idx, float* topk_w, float* topk_s,
                        float* scores, void* ws, hipStream_t s) {
  uint16_t* wf = (uint16_t*)ws;
  float* part = (float*)((char*)ws + route_parts_bytes(H, E));
  hipLaunchKernelGGL(router::split_kernel, dim3(H / 16, (E + 31) / 32), dim3(64), 0, s, H, E,
                     w_router, wf);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || T == 0) return e;
  const int S = router::slices(T, H);
  hipLaunchKernelGGL(router::proj_kernel, dim3((T + router::TB - 1) / router::TB, S),
                     dim3(router::NT), 0, s, T, H, E, S, x, wf, part);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(router::select_kernel, dim3((T + router::SEL_TPB - 1) / router::SEL_TPB),
                     dim3(router::SEL_NT), 0, s, T, E, K, S, part, bias, topk_idx, topk_w, topk_s,
                     scores);
  return hipGetLastError();
}

}  // namespace moe
