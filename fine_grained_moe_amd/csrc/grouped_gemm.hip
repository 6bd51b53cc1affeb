// Grouped bf16 GEMMs of the MoE expert FFN on gfx950 MFMA.
//
// The expert token segments are padded to the row tile, so every row tile
// belongs to exactly one expert and the grouped GEMM tiles like a plain GEMM
// ("dots.llm1 Technical Report" summary page, "Key claims" and "Method": the
// grouped GEMM pads expert token segments to tile multiples so tiling inside a
// block is uniform).  The pages built that for Hopper WGMMA tiles; here the
// tiles are sized for CDNA4 (v_mfma_f32_32x32x16_bf16, wave64, 160 KB LDS):
//   row-grouped products (rows = expert segments, 128-row aligned):
//     128 x 256 x 64 workgroup tile, 8 waves (2 per SIMD) of 64 x 64, 3 stages
//   weight gradients and the dense shared-expert products:
//     256 x 256 x 32 workgroup tile, 8 waves of 128 x 64, 4 stages
// Operands move global -> LDS with buffer_load ... lds (no VGPR staging),
// issued interleaved with the MFMAs of the current stage; a 3- or 4-deep LDS
// ring keeps two or three stages in flight.
//
// One kernel template covers the six products of the layer:
//   forward  gate/up  x_rows[M,H] . W1_e^T   (A K-contig, B K-contig) + SwiGLU epilogue
//   forward  down     h[M,F]      . W2_e^T   (A K-contig, B K-contig)
//   backward dgrad    dy_rows     . W2_e     (B N-contig)  + SwiGLU-backward epilogue
//   backward dgrad    dact        . W1_e     (B N-contig)
//   backward wgrad    dy_rows_e^T . h_e      (both M/N-contig, K = segment rows)
//   backward wgrad    dact_e^T    . x_rows_e (both M/N-contig, K = segment rows)
//
// LDS operand layouts (bf16):
//   K-contig tile  [rows][BK k]: 2*BK B per row; 16 B chunk c stored at
//                  c ^ ((row >> 1) & 7) (BK = 64) or c ^ ((row >> 2) & 3)
//                  (BK = 32).  Fragments read with ds_read_b128.
//   MN-contig tile [BK k][cols]: 2*cols B per k-row, 16 B chunk c stored at
//                  c ^ (4 * (k & 3)).  Fragments read with two
//                  ds_read_b64_tr_b16 (transposing LDS read of gfx950).
// Both layouts are free of LDS bank conflicts for these reads.
// Both give the same MFMA fragment: lane l holds Op[mn = base + l%32]
// [k = 16*kk + 8*(l/32) + 0..7].
//
// The MFMA is issued with the B-tile fragment as the first operand, so the
// accumulator of block (i,j) holds C[m][n] with m = l%32 (one row per lane)
// and n = 8*(r/4) + 4*(l/32) + r%4 (four consecutive columns per group of
// four registers): epilogues store 4 bf16 (8 bytes) per lane per group.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace gemm {

template <int BM_, int BN_, int BK_, int STAGES_, int WGM_, int WGN_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_, WGM = WGM_, WGN = WGN_;
  static constexpr int NW = WGM * WGN, NT = NW * 64;
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;  // wave tile
  static constexpr int WM = WTM / 32, WN = WTN / 32;    // 32x32 MFMA blocks per wave
  static constexpr int KK = BK / 16;                    // MFMA k-steps per stage
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
};
// Tile depth and pipeline depth are build-time tunables (defaults measured best).
#ifndef MOE_ROWS_BK
#define MOE_ROWS_BK 64
#endif
#ifndef MOE_ROWS_STAGES
#define MOE_ROWS_STAGES 3
#endif
#ifndef MOE_WIDE_BK
#define MOE_WIDE_BK 32
#endif
#ifndef MOE_WIDE_STAGES
#define MOE_WIDE_STAGES 4
#endif
// row-grouped tile order: 1 = expert-major (all m-tiles of one expert and one
// n-tile adjacent, then the next n-tile of the same expert); 0 = groups of
// GROUP_M m-tiles regardless of expert boundaries
#ifndef MOE_EXPERT_MAJOR
#define MOE_EXPERT_MAJOR 1
#endif
#ifndef MOE_ROWS_WGN
#define MOE_ROWS_WGN 4
#endif
#ifndef MOE_WIDE_WGN
#define MOE_WIDE_WGN 4
#endif
using CfgRows = TileCfg<128, 256, MOE_ROWS_BK, MOE_ROWS_STAGES, 2, MOE_ROWS_WGN>;  // 128-row segments
using CfgWide = TileCfg<256, 256, MOE_WIDE_BK, MOE_WIDE_STAGES, 2, MOE_WIDE_WGN>;  // wgrad, dense
static_assert(CfgRows::LDS_BYTES <= 160 * 1024 && CfgWide::LDS_BYTES <= 160 * 1024, "LDS");
static_assert(CfgRows::BM == kAlign, "row tile must equal the segment alignment");

constexpr int GROUP_M = 4;  // m-tiles per rasterization group

enum Src { KC = 0, MC = 1 };
enum Epi { EPI_SWIGLU_FWD = 0, EPI_STORE = 1, EPI_SWIGLU_BWD = 2 };
enum Mode { MGROUP = 0, KGROUP = 1 };

struct Args {
  const uint16_t* A;     // A operand base
  const uint16_t* B;     // B operand base (per-group stride strideB elements)
  uint16_t* C;           // output (STORE / SWIGLU_BWD: dact / SWIGLU_FWD: h)
  uint16_t* C2;          // SWIGLU_FWD: act (nullable)
  const uint16_t* aux;   // SWIGLU_BWD: act
  const int32_t* offsets;
  const int32_t* counts;
  const int32_t* tile_expert;
  int64_t m_rows;        // MGROUP: rows of A/C; dense KGROUP: rows of the segment
  int M, N, K;           // logical GEMM dims (MGROUP: M unused; KGROUP: per group)
  int lda, ldb, ldc;     // leading dims (elements)
  int64_t strideB;       // elements between consecutive groups' B
  int64_t strideC;       // KGROUP: elements between consecutive groups' C
  int F;                 // SWIGLU: expert width (gate/up split)
  int n_mtiles, n_ntiles, G;
};

// --------------------------------------------------------------------------
// Global -> LDS: buffer loads straight into LDS (buffer_load_dwordx4 ... lds)
// --------------------------------------------------------------------------
// Each wave-level load moves 64 lanes x 16 B = 1 KB into a contiguous LDS
// region whose base is wave-uniform (M0); lane l lands at base + 16*l.  The
// LDS swizzle is therefore applied on the global side: lane l fetches the
// global chunk that belongs at its LDS slot.  A lane whose element is out of
// range (rows past the segment, k past K, columns past N) gets an offset past
// the buffer's num_records, which the hardware turns into zeros (checked per
// dword), so masked rows and tails contribute exactly nothing.
constexpr uint32_t kOOB = 0x80000000u;
constexpr uint32_t kRsrcWord3 = 0x00020000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           (int)kRsrcWord3);
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, 0, 0, 0);
}

// s_waitcnt vmcnt(n) leaving expcnt/lgkmcnt unconstrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// wait until at most `ahead` stages of LOADS loads each are still in flight
template <int LOADS, int MAXA>
__device__ __forceinline__ void wait_stages(int ahead) {
  if constexpr (MAXA <= 0) {
    wait_vmcnt<0>();
  } else {
    if (ahead >= MAXA) wait_vmcnt<LOADS * MAXA>();
    else wait_stages<LOADS, MAXA - 1>(ahead);
  }
}

template <int BK>
__device__ __forceinline__ int kc_swz(int r) {
  return BK == 64 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}

// K-contig tile of R rows x BK k.  A 1 KB region holds RPR consecutive rows.
template <int R, int BK, int NW>
struct KcLoad {
  static constexpr int CPR = BK / 8;           // 16-byte chunks per row
  static constexpr int RPR = 1024 / (BK * 2);  // rows per region
  static constexpr int PER = R / RPR / NW;     // regions per wave
  static_assert(PER * RPR * NW == R, "tile rows");
  uint32_t off[PER];  // byte offset of the lane's chunk at kt = 0, or kOOB
  int kel[PER];       // k offset (elements) of the lane's chunk within a stage
  template <class RowOff>
  __device__ __forceinline__ void init(RowOff row_off, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = i * NW + wave;
      const int r = q * RPR + lane / CPR;
      const int c = (lane % CPR) ^ kc_swz<BK>(r);
      const uint32_t ro = row_off(r);
      off[i] = ro == kOOB ? kOOB : ro + c * 16;
      kel[i] = c * 8;
    }
  }
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, uint8_t* lds, int wave, int i,
                                        int kt, int K) const {
    const int q = i * NW + wave;
    const bool kin = kt * BK + kel[i] < K;
    const uint32_t v = (off[i] == kOOB || !kin) ? kOOB : off[i] + (uint32_t)kt * (BK * 2);
    dma16(rs, lds + q * 1024, v);
  }
};

// MN-contig tile of BK k-rows x C columns.  A 1 KB region holds KPR k-rows.
template <int C, int BK, int NW>
struct McLoad {
  static constexpr int CPR = C / 8;           // chunks per k-row
  static constexpr int KPR = 1024 / (2 * C);  // k-rows per region
  static constexpr int PER = BK / KPR / NW;   // regions per wave
  static_assert(PER * KPR * NW == BK, "tile k-rows");
  uint32_t coff[PER];  // byte offset of the lane's column chunk, or kOOB
  int kr[PER];         // k-row (0..BK-1) of the lane's chunk
  template <class ColOff>
  __device__ __forceinline__ void init(ColOff col_off, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = i * NW + wave;
      const int k = q * KPR + lane / CPR;
      const int c = (lane % CPR) ^ (4 * (k & 3));
      kr[i] = k;
      coff[i] = col_off(c * 8);
    }
  }
  // krow_off(k) -> byte offset of global k-row k, or kOOB
  template <class KRowOff>
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, uint8_t* lds, int wave, int i,
                                        int kt, KRowOff krow_off) const {
    const int q = i * NW + wave;
    const uint32_t ko = krow_off(kt * BK + kr[i]);
    const uint32_t v = (ko == kOOB || coff[i] == kOOB) ? kOOB : ko + coff[i];
    dma16(rs, lds + q * 1024, v);
  }
};

// --------------------------------------------------------------------------
// LDS -> fragment: lane l gets Op[mn = base + l%32][k = 16*kk + 8*(l/32) + 0..7]
// --------------------------------------------------------------------------
template <int BK>
__device__ __forceinline__ bf16x8 frag_kc(const uint8_t* lds, int base, int kk, int lane) {
  const int row = base + (lane & 31);
  const int c = 2 * kk + (lane >> 5);
  return *(const bf16x8*)(lds + row * (BK * 2) + ((c ^ kc_swz<BK>(row)) << 4));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(__attribute__((address_space(3))) const void*)p;
}

// LDS address of the first of the two transposing reads that build lane l's
// fragment of an MN-contig tile; the second read is 4 k-rows (8*C bytes) on.
template <int C>
__device__ __forceinline__ uint32_t mc_addr(const uint8_t* lds, int base, int kk, int lane) {
  const int g = lane >> 4, li = lane & 15;
  const int col = base + 16 * (g & 1) + 4 * (li & 3);
  const int k0 = 16 * kk + 8 * (g >> 1) + (li >> 2);
  const int c = col >> 3, sub = (col & 7) * 2;
  return lds_addr(lds) + k0 * (C * 2) + ((c ^ (4 * (k0 & 3))) << 4) + sub;
}

__device__ __forceinline__ bf16x8 join(s16x4 lo, s16x4 hi) {
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Fragments of an MN-contig tile via ds_read_b64_tr_b16, issued from inline
// asm together with their own s_waitcnt lgkmcnt(0): the outputs are complete
// when the block ends.  Written this way because the compiler treats the
// transposing-read builtin as possibly aliasing the in-flight LDS-DMA stores
// and would otherwise wait for every outstanding operand load before it.
template <int C>
__device__ __forceinline__ void mc_frags2(uint32_t a0, uint32_t a1, bf16x8& f0, bf16x8& f1) {
  s16x4 r0, r1, r2, r3;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %4 offset:%6\n\t"
      "ds_read_b64_tr_b16 %2, %5\n\t"
      "ds_read_b64_tr_b16 %3, %5 offset:%6\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(a0), "v"(a1), "i"(8 * C));
  f0 = join(r0, r1);
  f1 = join(r2, r3);
}
template <int C>
__device__ __forceinline__ void mc_frags4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                          bf16x8& f0, bf16x8& f1, bf16x8& f2, bf16x8& f3) {
  s16x4 r0, r1, r2, r3, r4, r5, r6, r7;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:%12\n\t"
      "ds_read_b64_tr_b16 %2, %9\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:%12\n\t"
      "ds_read_b64_tr_b16 %4, %10\n\t"
      "ds_read_b64_tr_b16 %5, %10 offset:%12\n\t"
      "ds_read_b64_tr_b16 %6, %11\n\t"
      "ds_read_b64_tr_b16 %7, %11 offset:%12\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "i"(8 * C));
  f0 = join(r0, r1);
  f1 = join(r2, r3);
  f2 = join(r4, r5);
  f3 = join(r6, r7);
}

// all NF fragments of one operand for k-step kk
template <int SRC, int NF, int C, int BK>
__device__ __forceinline__ void load_frags(const uint8_t* lds, const int* base, int kk, int lane,
                                           bf16x8* f) {
  if constexpr (SRC == KC) {
#pragma unroll
    for (int i = 0; i < NF; ++i) f[i] = frag_kc<BK>(lds, base[i], kk, lane);
  } else {
    static_assert(NF == 2 || NF == 4, "fragment count");
    if constexpr (NF == 2) {
      mc_frags2<C>(mc_addr<C>(lds, base[0], kk, lane), mc_addr<C>(lds, base[1], kk, lane), f[0], f[1]);
    } else {
      mc_frags4<C>(mc_addr<C>(lds, base[0], kk, lane), mc_addr<C>(lds, base[1], kk, lane),
                   mc_addr<C>(lds, base[2], kk, lane), mc_addr<C>(lds, base[3], kk, lane), f[0],
                   f[1], f[2], f[3]);
    }
  }
}

// --------------------------------------------------------------------------
// The kernel
// --------------------------------------------------------------------------
template <class Cfg, int ASRC, int BSRC, int EPI, int MODE>
__global__ void __launch_bounds__(Cfg::NT) grouped_gemm_kernel(Args a) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, NW = Cfg::NW, STAGES = Cfg::STAGES;
  constexpr int WM = Cfg::WM, WN = Cfg::WN, WTM = Cfg::WTM, WTN = Cfg::WTN;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[Cfg::LDS_BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / Cfg::WGN, wn = wave % Cfg::WGN;

  // ---- tile decode ---------------------------------------------------
  // Live tile count: for routed segments only the tiles below offsets[G] hold
  // rows; the grid is sized for the capacity bound.  Spreading the live tiles
  // (not the grid) over the XCDs keeps every XCD busy; the surplus ids exit.
  int n_mt = a.n_mtiles;
  if (MODE == MGROUP && a.tile_expert != nullptr) n_mt = a.offsets[a.G] / BM;
  const int ntiles_live = (MODE == MGROUP) ? n_mt * a.n_ntiles : (int)gridDim.x;
  if ((int)blockIdx.x >= ntiles_live) return;
  const int L = xcd_remap(blockIdx.x, ntiles_live);
  int e, mt, nt;
  {
    const int per_e = (MODE == KGROUP) ? a.n_mtiles * a.n_ntiles : 0x7fffffff;
    e = (MODE == KGROUP) ? L / per_e : 0;
    const int rem = (MODE == KGROUP) ? L % per_e : L;
    const int per_group = GROUP_M * a.n_ntiles;
    const int grp = rem / per_group, within = rem % per_group;
    const int gm = min(GROUP_M, n_mt - grp * GROUP_M);
    mt = grp * GROUP_M + within % gm;
    nt = within / gm;
  }
  if constexpr (MODE == MGROUP) {
    if (a.tile_expert == nullptr) {
      e = 0;
    } else if (MOE_EXPERT_MAJOR) {
      // tiles of expert e occupy [n_ntiles * mstart_e, n_ntiles * mend_e) in
      // the logical order, m-tile fastest, so the m-tiles sharing one weight
      // slice are adjacent and an expert's rows stay hot across its n-tiles
      const int mq = L / a.n_ntiles;  // some m-tile inside the same expert's range
      e = a.tile_expert[mq];
      if (e < 0) return;
      const int mstart = a.offsets[e] / BM;
      const int me = (a.offsets[e + 1] - a.offsets[e]) / BM;
      const int local = L - a.n_ntiles * mstart;
      mt = mstart + local % me;
      nt = local / me;
    } else {
      e = a.tile_expert[mt];
      if (e < 0) return;
    }
  }

  // row range of the segment (MGROUP: rows of the tile; KGROUP: the K range)
  int64_t seg_lo, seg_hi;
  if (a.offsets) {
    seg_lo = a.offsets[e];
    seg_hi = seg_lo + a.counts[e];
  } else {
    seg_lo = 0;
    seg_hi = a.m_rows;
  }

  const uint16_t* Bg = a.B + (int64_t)e * a.strideB;
  const int64_t m0 = (MODE == MGROUP) ? (int64_t)mt * BM : 0;
  const int mloc0 = (MODE == MGROUP) ? 0 : mt * BM;            // KGROUP: first output row (M dim)
  const int n0 = nt * (EPI == EPI_SWIGLU_FWD ? BN / 2 : BN);  // SWIGLU_FWD: f offset

  int nk;
  if constexpr (MODE == MGROUP) nk = (a.K + BK - 1) / BK;
  else nk = (int)((seg_hi - seg_lo + BK - 1) / BK);

  // ---- buffer resources and per-lane load offsets ----------------------
  __amdgpu_buffer_rsrc_t rA, rB;
  KcLoad<BM, BK, NW> la_kc;
  McLoad<BM, BK, NW> la_mc;
  KcLoad<BN, BK, NW> lb_kc;
  McLoad<BN, BK, NW> lb_mc;
  if constexpr (MODE == MGROUP) {
    const int rows_valid = (int)min<int64_t>(BM, seg_hi - m0);
    rA = make_rsrc(a.A + m0 * a.lda, (uint32_t)rows_valid * a.lda * 2);
    la_kc.init([&](int r) -> uint32_t { return r < rows_valid ? (uint32_t)r * a.lda * 2 : kOOB; },
               wave, lane);
    if constexpr (BSRC == KC) {
      rB = make_rsrc(Bg, (uint32_t)a.N * a.ldb * 2);
      lb_kc.init([&](int r) -> uint32_t {
        int n;
        if constexpr (EPI == EPI_SWIGLU_FWD) {
          const int f = n0 + (r & (BN / 2 - 1));
          if (f >= a.F) return kOOB;
          n = (r < BN / 2) ? f : a.F + f;
        } else {
          n = n0 + r;
          if (n >= a.N) return kOOB;
        }
        return (uint32_t)n * a.ldb * 2;
      }, wave, lane);
    } else {  // B = W [K][N], N-contig
      rB = make_rsrc(Bg, (uint32_t)a.K * a.ldb * 2);
      lb_mc.init([&](int c) -> uint32_t { return n0 + c < a.N ? (uint32_t)(n0 + c) * 2 : kOOB; },
                 wave, lane);
    }
  } else {  // KGROUP: A and B are rows of the segment, both M/N-contig
    const uint32_t nrows = (uint32_t)(seg_hi - seg_lo);
    rA = make_rsrc(a.A + seg_lo * a.lda, nrows * a.lda * 2);
    rB = make_rsrc(a.B + seg_lo * a.ldb, nrows * a.ldb * 2);
    la_mc.init([&](int c) -> uint32_t { return mloc0 + c < a.M ? (uint32_t)(mloc0 + c) * 2 : kOOB; },
               wave, lane);
    lb_mc.init([&](int c) -> uint32_t { return n0 + c < a.N ? (uint32_t)(n0 + c) * 2 : kOOB; },
               wave, lane);
  }

  constexpr int A_PER = (ASRC == KC) ? KcLoad<BM, BK, NW>::PER : McLoad<BM, BK, NW>::PER;
  constexpr int B_PER = (BSRC == KC) ? KcLoad<BN, BK, NW>::PER : McLoad<BN, BK, NW>::PER;
  constexpr int LOADS = A_PER + B_PER;  // DMA loads per wave per stage

  // load i of stage kt: i < A_PER is an A region, the rest B regions
  auto issue_one = [&](int kt, int i) {
    uint8_t* As = smem + (kt % STAGES) * Cfg::STAGE_BYTES;
    uint8_t* Bs = As + Cfg::A_BYTES;
    const int nrows = (int)(seg_hi - seg_lo);
    if (i < A_PER) {
      if constexpr (ASRC == KC) {
        la_kc.issue(rA, As, wave, i, kt, a.K);
      } else {
        la_mc.issue(rA, As, wave, i, kt, [&](int k) -> uint32_t {
          return k < nrows ? (uint32_t)k * a.lda * 2 : kOOB;
        });
      }
    } else {
      const int j = i - A_PER;
      if constexpr (BSRC == KC) {
        lb_kc.issue(rB, Bs, wave, j, kt, a.K);
      } else if constexpr (MODE == MGROUP) {
        lb_mc.issue(rB, Bs, wave, j, kt, [&](int k) -> uint32_t {
          return k < a.K ? (uint32_t)k * a.ldb * 2 : kOOB;
        });
      } else {
        lb_mc.issue(rB, Bs, wave, j, kt, [&](int k) -> uint32_t {
          return k < nrows ? (uint32_t)k * a.ldb * 2 : kOOB;
        });
      }
    }
  };

  // wave's fragment bases
  int a_base[WM], b_base[WN];
#pragma unroll
  for (int i = 0; i < WM; ++i) a_base[i] = wm * WTM + 32 * i;
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    if constexpr (EPI == EPI_SWIGLU_FWD)  // first half gate columns, second half the matching up
      b_base[j] = (j < WN / 2) ? (wn * (WTN / 2) + 32 * j)
                               : (BN / 2 + wn * (WTN / 2) + 32 * (j - WN / 2));
    else
      b_base[j] = wn * WTN + 32 * j;
  }

  f32x16 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // prologue: stages 0 .. STAGES-2 in flight
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk)
#pragma unroll
      for (int i = 0; i < LOADS; ++i) issue_one(s, i);

  for (int kt = 0; kt < nk; ++kt) {
    // stage kt has landed once only the stages issued after it are in flight
    const int ahead = min(STAGES - 2, nk - 1 - kt);
    wait_stages<LOADS, STAGES - 2>(ahead);
    // every wave's part of stage kt is in LDS, and every wave has finished
    // reading the buffer that stage kt+STAGES-1 overwrites
    __builtin_amdgcn_s_barrier();
    const int nxt = kt + STAGES - 1;
    const uint8_t* As = smem + (kt % STAGES) * Cfg::STAGE_BYTES;
    const uint8_t* Bs = As + Cfg::A_BYTES;
#pragma unroll
    for (int kk = 0; kk < Cfg::KK; ++kk) {
      bf16x8 af[WM], bfr[WN];
      load_frags<ASRC, WM, BM, BK>(As, a_base, kk, lane, af);
      load_frags<BSRC, WN, BN, BK>(Bs, b_base, kk, lane, bfr);
      // this stage's share of the next DMA loads, spread over the k-steps
      if (nxt < nk) {
#pragma unroll
        for (int i = kk * LOADS / Cfg::KK; i < (kk + 1) * LOADS / Cfg::KK; ++i) issue_one(nxt, i);
      }
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
  }

  // ---- epilogue: through LDS, coalesced 16-byte row stores ---------------
  // acc[i][j][r] holds row m = a_base[i] + (lane & 31) and column
  // n = b_base[j] + 8 (r/4) + 4 (lane/32) + r%4 of the tile.  Each output plane
  // (a BM x PC slice of one output tensor) is written to LDS as bf16 from the
  // registers, then copied out row by row with every lane moving 16 bytes, so a
  // wave's store covers whole cache lines.  The operand ring is free once all
  // waves pass the first barrier (the last stage was waited for in full).
  const int mrow = lane & 31;
  const int csub = 4 * (lane >> 5);
  constexpr int PC_FULL = (EPI == EPI_SWIGLU_FWD) ? BN / 2 : BN;  // plane columns
  constexpr int PITCH_FULL = PC_FULL * 2 + 16;
  constexpr int PC = (BM * PITCH_FULL <= Cfg::LDS_BYTES) ? PC_FULL : PC_FULL / 2;
  constexpr int PITCH = PC * 2 + 16;  // 16-byte pad: row starts rotate over the banks
  constexpr int NPART = PC_FULL / PC;
  static_assert(BM * PITCH <= Cfg::LDS_BYTES, "output plane must fit the operand ring");
  uint8_t* plane = smem;

  // column of block j, group g relative to the plane (gate/up blocks map to the
  // same plane column)
  auto pcol = [&](int j, int g) -> int {
    const int c = b_base[j] + 8 * g + csub;
    return (EPI == EPI_SWIGLU_FWD && j >= WN / 2) ? c - BN / 2 : c;
  };
  auto put4 = [&](int m, int c, float v0, float v1, float v2, float v3) {
    *(u32x2*)(plane + m * PITCH + c * 2) = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
  };
  // plane (columns [part*PC, part*PC + PC) of the tile) -> global rows
  auto store_plane = [&](uint16_t* gbase, int64_t ld, int64_t row0, int64_t row_lim, int col0,
                         int col_lim) {
    __syncthreads();
    constexpr int CPR = PC / 8;
    for (int q = tid; q < BM * CPR; q += Cfg::NT) {
      const int r = q / CPR, c = q % CPR;
      const int64_t row = row0 + r;
      const int col = col0 + c * 8;
      if (row < row_lim && col < col_lim)
        *(u32x4*)(gbase + row * ld + col) = *(const u32x4*)(plane + r * PITCH + c * 16);
    }
  };
  __syncthreads();

  if constexpr (EPI == EPI_SWIGLU_FWD) {
    // planes: h, then act's gate half, then act's up half
    const int nplanes = a.C2 ? 3 : 1;
    for (int pl = 0; pl < nplanes; ++pl) {
#pragma unroll
      for (int part = 0; part < NPART; ++part) {
        if (pl + part > 0) __syncthreads();
#pragma unroll
        for (int i = 0; i < WM; ++i)
#pragma unroll
          for (int j = 0; j < WN / 2; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int c = pcol(j, g) - part * PC;
              if (c < 0 || c >= PC) continue;
              const f32x16& G = acc[i][j];
              const f32x16& U = acc[i][j + WN / 2];
              float v[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const float gt = G[4 * g + q], up = U[4 * g + q];
                v[q] = pl == 0 ? gt / (1.0f + expf(-gt)) * up : (pl == 1 ? gt : up);
              }
              put4(a_base[i] + mrow, c, v[0], v[1], v[2], v[3]);
            }
        if (pl == 0)
          store_plane(a.C, a.ldc, m0, seg_hi, n0 + part * PC, a.F);
        else
          store_plane(a.C2 + (pl == 2 ? a.F : 0), 2 * (int64_t)a.F, m0, seg_hi, n0 + part * PC, a.F);
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU_BWD) {
    // acc = dh[row][f].  The forward's act rows ([gate | up], bf16) for this
    // tile are first copied into LDS with coalesced 16-byte loads (gate plane,
    // then up plane).  Each lane reads its own gate/up values from LDS, turns
    // dh into dgate in place, and writes dup over its own gate slots (each slot
    // has exactly one reader), so the gate plane becomes the dup plane; both
    // results then leave through the plane path into dact's two halves.
    static_assert(NPART == 1, "SwiGLU backward runs on tiles whose act planes fit LDS");
    static_assert(2 * BM * PITCH <= Cfg::LDS_BYTES, "gate and up planes must fit the ring");
    uint8_t* gplane = smem;
    uint8_t* uplane = smem + BM * PITCH;
    {
      constexpr int CPR = PC / 8;
      for (int q = tid; q < 2 * BM * CPR; q += Cfg::NT) {
        const int half = q / (BM * CPR), rq = q % (BM * CPR);
        const int r = rq / CPR, c = rq % CPR;
        const int64_t row = m0 + r;
        const int f = n0 + c * 8;
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (row < seg_hi && f < a.F) v = *(const u32x4*)(a.aux + row * (int64_t)(2 * a.F) + half * a.F + f);
        *(u32x4*)((half ? uplane : gplane) + r * PITCH + c * 16) = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int m = a_base[i] + mrow, c = pcol(j, g);
          const u32x2 gw = *(const u32x2*)(gplane + m * PITCH + c * 2);
          const u32x2 uw = *(const u32x2*)(uplane + m * PITCH + c * 2);
          const float gt[4] = {lo_bf16(gw[0]), hi_bf16(gw[0]), lo_bf16(gw[1]), hi_bf16(gw[1])};
          const float up[4] = {lo_bf16(uw[0]), hi_bf16(uw[0]), lo_bf16(uw[1]), hi_bf16(uw[1])};
          float du[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float dh = acc[i][j][4 * g + q];
            const float sg = 1.0f / (1.0f + expf(-gt[q]));
            acc[i][j][4 * g + q] = dh * up[q] * (sg * (1.0f + gt[q] * (1.0f - sg)));
            du[q] = dh * gt[q] * sg;
          }
          put4(m, c, du[0], du[1], du[2], du[3]);  // plane == gplane
        }
    store_plane(a.C + a.F, 2 * (int64_t)a.F, m0, seg_hi, n0, a.F);  // dup half
    __syncthreads();
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          put4(a_base[i] + mrow, pcol(j, g), acc[i][j][4 * g + 0], acc[i][j][4 * g + 1],
               acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
    store_plane(a.C, 2 * (int64_t)a.F, m0, seg_hi, n0, a.F);  // dgate half
  } else {  // EPI_STORE
    uint16_t* Cg = a.C + (MODE == KGROUP ? (int64_t)e * a.strideC : 0);
    const int64_t row0 = (MODE == MGROUP) ? m0 : (int64_t)mloc0;
    const int64_t rows_lim = (MODE == MGROUP) ? seg_hi : (int64_t)a.M;
#pragma unroll
    for (int part = 0; part < NPART; ++part) {
      if (part > 0) __syncthreads();
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int c = pcol(j, g) - part * PC;
            if (c < 0 || c >= PC) continue;
            put4(a_base[i] + mrow, c, acc[i][j][4 * g + 0], acc[i][j][4 * g + 1],
                 acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
          }
      store_plane(Cg, a.ldc, row0, rows_lim, n0 + part * PC, a.N);
    }
  }
}

template <class Cfg, int ASRC, int BSRC, int EPI, int MODE>
static hipError_t launch(const Args& a, int nblocks, hipStream_t s) {
  if (nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_gemm_kernel<Cfg, ASRC, BSRC, EPI, MODE>), dim3(nblocks), dim3(Cfg::NT),
                     0, s, a);
  return hipGetLastError();
}

// M-grouped launch: routed segments use the 128-row tile (= alignment), the
// dense single group (shared experts) the 256-row tile
template <int ASRC, int BSRC, int EPI>
static hipError_t launch_rows(Args a, int n_cols_per_tile_rows, int n_cols_per_tile_wide, int ncols,
                              hipStream_t s) {
  // routed segments need the 128-row tile (= alignment); the SwiGLU-backward
  // epilogue stages two act planes in LDS, which only the 128-row tile leaves
  // room for; everything else dense takes the 256-row tile
  auto rows = [&]() {
    a.n_mtiles = (int)((a.m_rows + CfgRows::BM - 1) / CfgRows::BM);
    a.n_ntiles = (ncols + n_cols_per_tile_rows - 1) / n_cols_per_tile_rows;
    return launch<CfgRows, ASRC, BSRC, EPI, MGROUP>(a, a.n_mtiles * a.n_ntiles, s);
  };
  if constexpr (EPI == EPI_SWIGLU_BWD) {
    return rows();
  } else {
    if (a.tile_expert) return rows();
    a.n_mtiles = (int)((a.m_rows + CfgWide::BM - 1) / CfgWide::BM);
    a.n_ntiles = (ncols + n_cols_per_tile_wide - 1) / n_cols_per_tile_wide;
    return launch<CfgWide, ASRC, BSRC, EPI, MGROUP>(a, a.n_mtiles * a.n_ntiles, s);
  }
}

}  // namespace gemm

using namespace gemm;

hipError_t launch_gemm_gate_up(int G, int64_t m_rows, int H, int F, const int32_t* offsets,
                               const int32_t* counts, const int32_t* tile_expert,
                               const uint16_t* x_rows, const uint16_t* w1, uint16_t* act,
                               uint16_t* h, hipStream_t s) {
  Args a = {};
  a.A = x_rows; a.B = w1; a.C = h; a.C2 = act;
  a.offsets = offsets; a.counts = counts; a.tile_expert = tile_expert;
  a.m_rows = m_rows; a.N = 2 * F; a.K = H; a.F = F;
  a.lda = H; a.ldb = H; a.ldc = F; a.strideB = (int64_t)2 * F * H; a.G = G;
  // an n-tile covers BN/2 gate columns and the matching BN/2 up columns
  return launch_rows<KC, KC, EPI_SWIGLU_FWD>(a, CfgRows::BN / 2, CfgWide::BN / 2, F, s);
}

hipError_t launch_gemm_down(int G, int64_t m_rows, int H, int F, const int32_t* offsets,
                            const int32_t* counts, const int32_t* tile_expert,
                            const uint16_t* h, const uint16_t* w2, uint16_t* y_rows,
                            hipStream_t s) {
  Args a = {};
  a.A = h; a.B = w2; a.C = y_rows;
  a.offsets = offsets; a.counts = counts; a.tile_expert = tile_expert;
  a.m_rows = m_rows; a.N = H; a.K = F; a.F = F;
  a.lda = F; a.ldb = F; a.ldc = H; a.strideB = (int64_t)H * F; a.G = G;
  return launch_rows<KC, KC, EPI_STORE>(a, CfgRows::BN, CfgWide::BN, H, s);
}

hipError_t launch_gemm_dgrad_down(int G, int64_t m_rows, int H, int F, const int32_t* offsets,
                                  const int32_t* counts, const int32_t* tile_expert,
                                  const uint16_t* dy_rows, const uint16_t* w2,
                                  const uint16_t* act, uint16_t* dact, hipStream_t s) {
  Args a = {};
  a.A = dy_rows; a.B = w2; a.C = dact; a.aux = act;
  a.offsets = offsets; a.counts = counts; a.tile_expert = tile_expert;
  a.m_rows = m_rows; a.N = F; a.K = H; a.F = F;
  a.lda = H; a.ldb = F; a.ldc = 2 * F; a.strideB = (int64_t)H * F; a.G = G;
  return launch_rows<KC, MC, EPI_SWIGLU_BWD>(a, CfgRows::BN, CfgWide::BN, F, s);
}

hipError_t launch_gemm_dgrad_up(int G, int64_t m_rows, int H, int F, const int32_t* offsets,
                                const int32_t* counts, const int32_t* tile_expert,
                                const uint16_t* dact, const uint16_t* w1, uint16_t* dx_rows,
                                hipStream_t s) {
  Args a = {};
  a.A = dact; a.B = w1; a.C = dx_rows;
  a.offsets = offsets; a.counts = counts; a.tile_expert = tile_expert;
  a.m_rows = m_rows; a.N = H; a.K = 2 * F; a.F = F;
  a.lda = 2 * F; a.ldb = H; a.ldc = H; a.strideB = (int64_t)2 * F * H; a.G = G;
  return launch_rows<KC, MC, EPI_STORE>(a, CfgRows::BN, CfgWide::BN, H, s);
}

// dW2[g] [H,F] = dy_rows_g^T [H, rows] . h_g [rows, F]
hipError_t launch_gemm_wgrad_down(int G, int64_t m_rows, int H, int F, const int32_t* offsets,
                                  const int32_t* counts, const uint16_t* dy_rows,
                                  const uint16_t* h, uint16_t* dw2, hipStream_t s) {
  Args a = {};
  a.A = dy_rows; a.B = h; a.C = dw2;
  a.offsets = offsets; a.counts = counts;
  a.m_rows = m_rows; a.M = H; a.N = F; a.F = F;
  a.lda = H; a.ldb = F; a.ldc = F; a.strideB = 0; a.strideC = (int64_t)H * F;
  a.n_mtiles = (H + CfgWide::BM - 1) / CfgWide::BM; a.n_ntiles = (F + CfgWide::BN - 1) / CfgWide::BN;
  a.G = G;
  return launch<CfgWide, MC, MC, EPI_STORE, KGROUP>(a, G * a.n_mtiles * a.n_ntiles, s);
}

// dW1[g] [2F,H] = dact_g^T [2F, rows] . x_rows_g [rows, H]
hipError_t launch_gemm_wgrad_up(int G, int64_t m_rows, int H, int F, const int32_t* offsets,
                                const int32_t* counts, const uint16_t* dact,
                                const uint16_t* x_rows, uint16_t* dw1, hipStream_t s) {
  Args a = {};
  a.A = dact; a.B = x_rows; a.C = dw1;
  a.offsets = offsets; a.counts = counts;
  a.m_rows = m_rows; a.M = 2 * F; a.N = H; a.F = F;
  a.lda = 2 * F; a.ldb = H; a.ldc = H; a.strideB = 0; a.strideC = (int64_t)2 * F * H;
  a.n_mtiles = (2 * F + CfgWide::BM - 1) / CfgWide::BM; a.n_ntiles = (H + CfgWide::BN - 1) / CfgWide::BN;
  a.G = G;
  return launch<CfgWide, MC, MC, EPI_STORE, KGROUP>(a, G * a.n_mtiles * a.n_ntiles, s);
}

}  // namespace moe
