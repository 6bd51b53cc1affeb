// Grouped bf16 GEMMs of the MoE expert FFN on gfx950 MFMA.
//
// The expert token segments are padded to the row tile, so every row tile
// belongs to exactly one expert and the grouped GEMM tiles like a plain GEMM
// ("dots.llm1 Technical Report" summary page, "Key claims" and "Method": the
// grouped GEMM pads expert token segments to tile multiples so tiling inside a
// block is uniform).  The pages built that for Hopper WGMMA tiles; here the
// tiles are sized for CDNA4 (v_mfma_f32_32x32x16_bf16, wave64, 160 KB LDS):
//   row-grouped products (rows = expert segments, 128-row aligned):
//     128 x 256 x 64 workgroup tile, 8 waves (2 per SIMD) of 64 x 64, 3 stages;
//     the gate/up data gradient 128 x 512 x 32, 8 waves of 64 x 128, 4 stages
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
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace moe {
namespace gemm {

using namespace lds;

template <int BM_, int BN_, int BK_, int STAGES_, int WGM_, int WGN_, int MINB_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_, WGM = WGM_, WGN = WGN_;
  static constexpr int MINB = MINB_;                    // workgroups resident per CU
  static constexpr int NW = WGM * WGN, NT = NW * 64;
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;  // wave tile
  static constexpr int WM = WTM / 32, WN = WTN / 32;    // 32x32 MFMA blocks per wave
  static constexpr int KK = BK / 16;                    // MFMA k-steps per stage
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static_assert(KK % 2 == 0, "fragment double buffering pairs k-steps");
  static_assert(LDS_BYTES * MINB <= 160 * 1024, "LDS per CU");
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
// 128 x 256 row tiles, 8 waves (wave tile 64 x 64), one workgroup per CU,
// 64-deep k stages (128-byte row segments per load)
using CfgRows = TileCfg<128, 256, MOE_ROWS_BK, MOE_ROWS_STAGES, 2, 4, 1>;
// 128 x 512 row tiles, 8 waves of 64 x 128, four 32-deep stages (160 KB):
// the gate/up data gradient (N = H, B N-contig), where the wider wave tile
// halves the B fragment reads per MFMA and measured 7 % faster than CfgRows
// (the down forward, B K-contig, measured 11 % slower with it, the down data
// gradient with its SwiGLU-backward epilogue 4 % slower)
using CfgRowsN = TileCfg<128, 512, 32, 4, 2, 4, 1>;
static_assert(CfgRowsN::BM == 128, "row tile must equal the segment alignment");
// 256 x 256 tiles of 8 waves (wave tile 128 x 64), one workgroup per CU
using CfgWide = TileCfg<256, 256, MOE_WIDE_BK, MOE_WIDE_STAGES, 2, 4, 1>;
// K-grouped weight-gradient products use the wide tile
using CfgWgrad = CfgWide;
static_assert(CfgRows::BM == kAlign, "row tile must equal the segment alignment");

constexpr int GROUP_M = 4;  // m-tiles per rasterization group (dense row products)
// Routed row products: the tiles of one expert run in bands of BAND_M m-tiles
// (all n-tiles of a band, m-tile fastest, before the next band).  The
// workgroups that run together on one XCD then share BAND_M row blocks of the
// row operand and a few weight slices; an expert with thousands of rows
// rastered m-fastest over its whole segment instead streams every row block
// once per n-tile (the skewed batch's gate/up forward: 14 % faster with bands
// of 4; balanced batches, at most 4 row tiles per expert, are unchanged).
constexpr int BAND_M = 4;
// K-grouped weight gradients: m-tiles per rasterization group inside one
// expert, so a column slab of the second operand is reused by several m-tiles
// while it is resident in L2
constexpr int KGROUP_GM = 4;

enum Src { KC = 0, MC = 1 };
enum Epi { EPI_SWIGLU_FWD = 0, EPI_STORE = 1, EPI_SWIGLU_BWD = 2, EPI_F32 = 3 };
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
  float* Cf;             // F32: fp32 output (row-major, ldc)
  int acc_out;           // F32: add to Cf instead of writing it
  int ksplit;            // F32, dense MGROUP: slices of the k range (0 or 1: none)
  int64_t split_stride;  // F32 with ksplit > 1: elements between slices' outputs
  int kg_chunk;          // KGROUP: logical tiles per chunk dealt round-robin to the XCDs
  int kg_tiles;          // KGROUP with kg_chunk: logical tiles (the grid is padded)
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
  __device__ __forceinline__ void issue(const u32x4& rs, uint32_t lds, int wave, int i, int kt,
                                        KRowOff krow_off) const {
    const int q = i * NW + wave;
    const uint32_t ko = krow_off(kt * BK + kr[i]);
    const uint32_t v = (ko == kOOB || coff[i] == kOOB) ? kOOB : ko + coff[i];
    dma16(rs, lds + q * 1024, v);
  }
};

// --------------------------------------------------------------------------
// LDS -> fragment: lane l gets Op[mn = base + l%32][k = 16*kk + 8*(l/32) + 0..7]
// --------------------------------------------------------------------------
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

__device__ __forceinline__ s16x4 read_tr16(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(size_t)addr);
}

// fragment of an MN-contig tile: two ds_read_b64_tr_b16 (gfx950 transposing
// LDS read), four k-rows apart
template <int C>
__device__ __forceinline__ bf16x8 frag_mc(const uint8_t* lds, int base, int kk, int lane) {
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const uint32_t a0 = mc_addr<C>(lds, base, kk, lane);
  const s16x4 lo = read_tr16(a0), hi = read_tr16(a0 + 8 * C);
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// all NF fragments of one operand for k-step kk
template <int SRC, int NF, int C, int BK>
__device__ __forceinline__ void load_frags(const uint8_t* lds, const int* base, int kk, int lane,
                                           bf16x8* f) {
#pragma unroll
  for (int i = 0; i < NF; ++i)
    f[i] = (SRC == KC) ? frag_kc<BK>(lds, base[i], kk, lane) : frag_mc<C>(lds, base[i], kk, lane);
}

// SwiGLU's logistic function in the GEMM epilogues: hardware exp2 and
// reciprocal (about 1 ulp each).  The results are rounded to bf16 next, so the
// correctly rounded library forms would only cost time.
__device__ __forceinline__ float sigmoid_fast(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.44269504088896341f));
}

// --------------------------------------------------------------------------
// The kernel
// --------------------------------------------------------------------------
// NTB: the B operand's loads are non-temporal (a weight matrix that every
// tile reads once: routed forward products at a few rows per expert)
template <class Cfg, int ASRC, int BSRC, int EPI, int MODE, bool NTB = false>
__global__ void __launch_bounds__(Cfg::NT, Cfg::MINB) grouped_gemm_kernel(Args a) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, NW = Cfg::NW, STAGES = Cfg::STAGES;
  constexpr int WM = Cfg::WM, WN = Cfg::WN, WTM = Cfg::WTM, WTN = Cfg::WTN;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[Cfg::LDS_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / Cfg::WGN, wn = wave % Cfg::WGN;

  // ---- tile decode ---------------------------------------------------
  // Live tile count: for routed segments only the tiles below offsets[G] hold
  // rows; the grid is sized for the capacity bound.  Spreading the live tiles
  // (not the grid) over the XCDs keeps every XCD busy; the surplus ids exit.
  int n_mt = a.n_mtiles;
  if (MODE == MGROUP && a.tile_expert != nullptr) n_mt = a.offsets[a.G] / BM;
  // k split (dense fp32-output products only): the grid holds ks copies of the
  // tile set, copy sp accumulating its own slice of the k stages
  constexpr bool SPLIT = EPI == EPI_F32 && MODE == MGROUP;
  const int ks = (SPLIT && a.ksplit > 1) ? a.ksplit : 1;
  const int ntiles_live = (MODE == MGROUP) ? n_mt * a.n_ntiles * ks : (int)gridDim.x;
  int L0;
  if (MODE == KGROUP && a.kg_chunk > 0) {
    // chunks of kg_chunk consecutive logical tiles go to the XCDs in turn
    // (the hardware hands consecutive workgroup ids to consecutive XCDs), so
    // that a few experts holding most rows still spread over all of them;
    // the grid is padded to whole rounds of chunks
    const int CH = a.kg_chunk;
    const int xcd = (int)blockIdx.x % kNumXcd, slot = (int)blockIdx.x / kNumXcd;
    L0 = ((slot / CH) * kNumXcd + xcd) * CH + slot % CH;
    if (L0 >= a.kg_tiles) return;
  } else {
    if ((int)blockIdx.x >= ntiles_live) return;
    L0 = xcd_remap(blockIdx.x, ntiles_live);
  }
  const int sp = SPLIT ? L0 / (n_mt * a.n_ntiles) : 0;
  const int L = SPLIT ? L0 - sp * (n_mt * a.n_ntiles) : L0;
  int e, mt, nt;
  {
    const int per_e = (MODE == KGROUP) ? a.n_mtiles * a.n_ntiles : 0x7fffffff;
    e = (MODE == KGROUP) ? L / per_e : 0;
    const int rem = (MODE == KGROUP) ? L % per_e : L;
    const int GM = (MODE == KGROUP) ? KGROUP_GM : GROUP_M;
    const int per_group = GM * a.n_ntiles;
    const int grp = rem / per_group, within = rem % per_group;
    const int gm = min(GM, n_mt - grp * GM);
    mt = grp * GM + within % gm;
    nt = within / gm;
  }
  if constexpr (MODE == MGROUP) {
    if (a.tile_expert == nullptr) {
      e = 0;
    } else {
      // tiles of expert e occupy [n_ntiles * mstart_e, n_ntiles * mend_e) in
      // the logical order, m-tile fastest, so the m-tiles sharing one weight
      // slice are adjacent and an expert's rows stay hot across its n-tiles
      const int mq = L / a.n_ntiles;  // some m-tile inside the same expert's range
      e = a.tile_expert[mq];
      if (e < 0) return;
      const int mstart = a.offsets[e] / BM;
      const int me = (a.offsets[e + 1] - a.offsets[e]) / BM;
      const int local = L - a.n_ntiles * mstart;
      // bands of BAND_M m-tiles, each band's tiles m-fastest within it and
      // the bands one after the other (a segment of at most BAND_M tiles is
      // one band)
      const int per_band = BAND_M * a.n_ntiles;
      const int band = local / per_band, within = local % per_band;
      const int bm = min(BAND_M, me - band * BAND_M);
      mt = mstart + band * BAND_M + within % bm;
      nt = within / bm;
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
  // this copy's k slice: first stage and end (elements); the whole range
  // without a split
  int kofs = 0, kend = a.K;
  if constexpr (SPLIT) {
    const int k0 = sp * nk / ks, k1 = (sp + 1) * nk / ks;
    kofs = k0;
    kend = min(a.K, k1 * BK);
    nk = k1 - k0;
  }

  // ---- buffer resources and per-lane load offsets ----------------------
  u32x4 rA, rB;
  KcLoad<BM, BK, NW> la_kc;
  McLoad<BM, BK, NW> la_mc;
  KcLoad<BN, BK, NW> lb_kc;
  McLoad<BN, BK, NW> lb_mc;
  // rows of the tile inside the segment (MGROUP)
  const int rows_valid = (MODE == MGROUP) ? (int)min<int64_t>(BM, seg_hi - m0) : BM;
  if constexpr (MODE == MGROUP) {
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
  const uint32_t smem_base = lds_addr(smem);
  auto issue_one = [&](int kt, int i) {
    const uint32_t As = smem_base + (kt % STAGES) * Cfg::STAGE_BYTES;
    const uint32_t Bs = As + Cfg::A_BYTES;
    const int nrows = (int)(seg_hi - seg_lo);
    if (i < A_PER) {
      if constexpr (ASRC == KC) {
        if constexpr (SPLIT) la_kc.issue(rA, As, wave, i, kt + kofs, kend);
        else la_kc.issue(rA, As, wave, i, kt, a.K);
      } else {
        la_mc.issue(rA, As, wave, i, kt, [&](int k) -> uint32_t {
          return k < nrows ? (uint32_t)k * a.lda * 2 : kOOB;
        });
      }
    } else {
      const int j = i - A_PER;
      if constexpr (BSRC == KC) {
        if constexpr (SPLIT) lb_kc.issue(rB, Bs, wave, j, kt + kofs, kend);
        else lb_kc.template issue<NTB>(rB, Bs, wave, j, kt, a.K);
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

  // One k-step (16 deep) of the wave tile: WM x WN MFMAs on fragments that
  // were read from LDS one k-step earlier (double-buffered registers), so the
  // LDS latency of step s+1 hides behind the MFMAs of step s.
  // (NL of the wave's WM row blocks take part, see below)
  auto frags = [&](auto nl_c, int kt, int kk, bf16x8* af, bf16x8* bfr) {
    constexpr int NL = decltype(nl_c)::value;
    const uint8_t* As = smem + (kt % STAGES) * Cfg::STAGE_BYTES;
    const uint8_t* Bs = As + Cfg::A_BYTES;
    load_frags<ASRC, NL, BM, BK>(As, a_base, kk, lane, af);
    load_frags<BSRC, WN, BN, BK>(Bs, b_base, kk, lane, bfr);
  };

  // The pipeline runs without branches: loads of stages past the last one
  // have k past K, so the hardware fills their LDS slots with zeros (nothing
  // reads them), and every wait counts the same number of loads.
  // prologue: stages 0 .. STAGES-2 in flight, stage 0 landed, its first
  // fragments in registers
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
#pragma unroll
    for (int i = 0; i < LOADS; ++i) issue_one(s, i);
  wait_vmcnt<LOADS * (STAGES - 2)>();
  lds_barrier();

  // each k-step issues PER_KK of the LOADS loads of stage kt+STAGES-1, so
  // when the last k-step of stage kt waits for stage kt+1, the loads issued
  // after stage kt+1 are the full stages kt+2 .. kt+STAGES-2 and the first
  // KK-1 shares of stage kt+STAGES-1
  // With two stages the refill of stage kt+1 must be complete when stage kt
  // ends, so its loads go out during the first KK-1 k-steps only.
  constexpr int ISSUE_KK = (STAGES == 2) ? Cfg::KK - 1 : Cfg::KK;
  constexpr int PER_KK = (LOADS + ISSUE_KK - 1) / ISSUE_KK;
  constexpr int LATER =
      (STAGES == 2) ? 0
                    : LOADS * (STAGES - 3) +
                          ((Cfg::KK - 1) * PER_KK < LOADS ? (Cfg::KK - 1) * PER_KK : LOADS);
  static_assert(STAGES >= 2 && ISSUE_KK >= 1, "pipeline depth");

  // The main loop for a wave whose first NL row blocks (of 32 rows) hold rows
  // of the segment: the other blocks are padding, whose MFMAs and fragment
  // reads it skips (their results would be dropped).  Every wave issues the
  // same loads, waits and barriers whatever its NL.
  auto main_loop = [&](auto nl_c) {
    constexpr int NL = decltype(nl_c)::value;
    bf16x8 af[2][WM], bfr[2][WN];
    if constexpr (NL > 0) frags(nl_c, 0, 0, af[0], bfr[0]);
    for (int kt = 0; kt < nk; ++kt) {
      // stage kt+STAGES-1 goes into the buffer stage kt-1 used; every wave
      // finished reading that one before the barrier that preceded stage kt
      const int nxt = kt + STAGES - 1;
#pragma unroll
      for (int kk = 0; kk < Cfg::KK; ++kk) {
        const int cur = kk & 1, nb = cur ^ 1;
        if (kk + 1 < Cfg::KK) {
          if constexpr (NL > 0) frags(nl_c, kt, kk + 1, af[nb], bfr[nb]);
        } else {
          // stage kt+1 has landed once only the loads issued after it remain
          wait_vmcnt<LATER>();
          lds_barrier();
          if constexpr (NL > 0) frags(nl_c, kt + 1, 0, af[nb], bfr[nb]);
        }
        // keep the reads ahead of the MFMAs that hide their latency
        __builtin_amdgcn_sched_barrier(0);
        // this k-step's share of the next stage's DMA loads, between MFMAs
#pragma unroll
        for (int i = 0; i < WM; ++i)
#pragma unroll
          for (int j = 0; j < WN; ++j) {
            if (i < NL)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[cur][j], af[cur][i],
                                                                  acc[i][j], 0, 0, 0);
            const int t = i * WN + j;
            const int li = kk * PER_KK + t;
            if (t < PER_KK && li < LOADS) {
              issue_one(nxt, li);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
      }
    }
  };
  // live row blocks of this wave: routed 128-row tiles skip padding blocks
  // one by one; other tiles run whole waves or none.  A wave whose columns
  // all lie past N (the last column tile of an N that is not a multiple of
  // the tile) has nothing to compute either.
  const int nl_rows = (rows_valid - wm * WTM + 31) / 32;
  const bool cols_live = (EPI == EPI_SWIGLU_FWD) || (a.N - n0 - wn * WTN > 0);
  const int nl = (nl_rows <= 0 || !cols_live) ? 0 : (nl_rows >= WM ? WM : nl_rows);
  if constexpr (MODE == MGROUP && BM == kAlign && WM == 2) {
    if (nl == 2)
      main_loop(std::integral_constant<int, 2>{});
    else if (nl == 1)
      main_loop(std::integral_constant<int, 1>{});
    else
      main_loop(std::integral_constant<int, 0>{});
  } else {
    if (nl > 0)
      main_loop(std::integral_constant<int, WM>{});
    else
      main_loop(std::integral_constant<int, 0>{});
  }
  wait_vmcnt<0>();

  // ---- epilogue: through LDS, coalesced 16-byte row stores ---------------
  // acc[i][j][r] holds row m = a_base[i] + (lane & 31) and column
  // n = b_base[j] + 8 (r/4) + 4 (lane/32) + r%4 of the tile.  Each output plane
  // (a BM x PC slice of one output tensor) is written to LDS as bf16 from the
  // registers, then copied out row by row with every lane moving 16 bytes, so a
  // wave's store covers whole cache lines.  Plane rows are unpadded; the 16-byte
  // chunks of row m are XOR-swizzled by m, which spreads the column writes of
  // the 32 rows a wave holds over the banks.  The operand ring is free once all
  // waves pass the first barrier (the last stage was waited for in full).
  // Barriers here order LDS only: the global stores are left in flight (a
  // workgroup fence would wait for each plane's stores before the next).
  const int mrow = lane & 31;
  const int csub = 4 * (lane >> 5);
  constexpr int PC_FULL = (EPI == EPI_SWIGLU_FWD) ? BN / 2 : BN;  // plane columns
  // the SwiGLU backward keeps two planes (gate and up of the forward) in LDS
  constexpr int NPL = (EPI == EPI_SWIGLU_BWD) ? 2 : 1;
  constexpr int PC = (NPL * BM * PC_FULL * 2 <= Cfg::LDS_BYTES) ? PC_FULL : PC_FULL / 2;
  constexpr int PITCH = PC * 2;
  constexpr int NPART = PC_FULL / PC;
  constexpr int CPR = PC / 8;                        // 16-byte chunks per plane row
  constexpr int SWZ = (CPR < 32 ? CPR : 32) - 1;     // chunk swizzle mask
  static_assert((CPR & (CPR - 1)) == 0, "plane rows hold a power-of-two number of chunks");
  static_assert(NPL * BM * PITCH <= Cfg::LDS_BYTES, "output planes must fit the operand ring");
  static_assert((BM * CPR) % Cfg::NT == 0, "plane copy is a whole number of rounds");
  // 16-byte copies in flight per thread in a plane copy (the SwiGLU backward
  // holds its dgate accumulators across the copies: one at a time there)
  constexpr int UNR_MAX = (EPI == EPI_SWIGLU_BWD) ? 1 : 4;
  uint8_t* plane = smem;
  auto poff = [](int m, int c) -> int {  // byte offset of element (m, c) of a plane
    return m * PITCH + ((((c >> 3) ^ (m & SWZ))) << 4) + ((c & 7) << 1);
  };

  // column of block j, group g relative to the plane (gate/up blocks map to the
  // same plane column)
  auto pcol = [&](int j, int g) -> int {
    const int c = b_base[j] + 8 * g + csub;
    return (EPI == EPI_SWIGLU_FWD && j >= WN / 2) ? c - BN / 2 : c;
  };
  auto in_part = [&](int c) -> bool { return NPART == 1 || (c >= 0 && c < PC); };
  auto put4 = [&](uint8_t* pl, int m, int c, float v0, float v1, float v2, float v3) {
    *(u32x2*)(pl + poff(m, c)) = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
  };
  // plane (columns [part*PC, part*PC + PC) of the tile) -> global rows: every
  // round's LDS reads are issued before its stores
  auto store_plane = [&](const uint8_t* pl, uint16_t* gbase, int64_t ld, int64_t row0,
                         int64_t row_lim, int col0, int col_lim) {
    lds_barrier();
    constexpr int ROUNDS = BM * CPR / Cfg::NT;
    constexpr int UNR = ROUNDS < UNR_MAX ? ROUNDS : UNR_MAX;
    static_assert(ROUNDS % UNR == 0, "plane copy batches");
#pragma unroll 1  // batches stay sequential: bounded registers
    for (int u0 = 0; u0 < ROUNDS; u0 += UNR) {
      u32x4 v[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int q = tid + (u0 + u) * Cfg::NT, r = q / CPR, c = q % CPR;
        v[u] = *(const u32x4*)(pl + r * PITCH + ((c ^ (r & SWZ)) << 4));
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int q = tid + (u0 + u) * Cfg::NT, r = q / CPR, c = q % CPR;
        const int64_t row = row0 + r;
        const int col = col0 + c * 8;
        // non-temporal: the launch never reads its outputs back, so they
        // stream out instead of displacing operand lines in the caches
        if (row < row_lim && col < col_lim)
          __builtin_nontemporal_store(v[u], (u32x4*)(gbase + row * ld + col));
      }
    }
  };
  lds_barrier();

  if constexpr (EPI == EPI_SWIGLU_FWD) {
    // planes: h, then act's gate half, then act's up half
    const int nplanes = a.C2 ? 3 : 1;
    for (int pl = 0; pl < nplanes; ++pl) {
#pragma unroll
      for (int part = 0; part < NPART; ++part) {
        if (pl + part > 0) lds_barrier();
#pragma unroll
        for (int i = 0; i < WM; ++i)
#pragma unroll
          for (int j = 0; j < WN / 2; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int c = pcol(j, g) - part * PC;
              if (!in_part(c)) continue;
              const f32x16& G = acc[i][j];
              const f32x16& U = acc[i][j + WN / 2];
              float v[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const float gt = G[4 * g + q], up = U[4 * g + q];
                v[q] = pl == 0 ? gt * sigmoid_fast(gt) * up : (pl == 1 ? gt : up);
              }
              put4(plane, a_base[i] + mrow, c, v[0], v[1], v[2], v[3]);
            }
        if (pl == 0)
          store_plane(plane, a.C, a.ldc, m0, seg_hi, n0 + part * PC, a.F);
        else
          store_plane(plane, a.C2 + (pl == 2 ? a.F : 0), 2 * (int64_t)a.F, m0, seg_hi,
                      n0 + part * PC, a.F);
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU_BWD) {
    // acc = dh[row][f].  Per part (a PC-column slice of the tile), the
    // forward's act values ([gate | up] rows, bf16) are first copied into two
    // LDS planes with coalesced 16-byte loads.  Each lane reads its own gate/up
    // values from LDS, turns dh into dgate in place, and writes dup over its own
    // gate slots (each slot has exactly one reader), so the gate plane becomes
    // the dup plane; both results then leave through the plane path into
    // dact's two halves.
    uint8_t* gplane = smem;
    uint8_t* uplane = smem + BM * PITCH;
#pragma unroll
    for (int part = 0; part < NPART; ++part) {
      if (part > 0) lds_barrier();
      {
        // act rows -> the two planes by LDS-DMA: every 1 KB region of a plane
        // is one wave-level load, each lane fetching the chunk that belongs at
        // its slot of the swizzled layout; rows past the segment and columns
        // past F read as zeros
        constexpr int RPRG = 1024 / PITCH;               // plane rows per region
        constexpr int REGIONS = 2 * BM * PITCH / 1024;   // both planes
        static_assert(RPRG * CPR == 64 && REGIONS % NW == 0, "act regions");
        const int rows_valid = (int)min<int64_t>(BM, seg_hi - m0);
        const u32x4 rAct = make_rsrc(a.aux + m0 * (int64_t)(2 * a.F),
                                     (uint32_t)(rows_valid * 2 * a.F * 2));
#pragma unroll
        for (int k = 0; k < REGIONS / NW; ++k) {
          const int q = k * NW + wave;                   // region
          const int half = q / (REGIONS / 2);
          const int r = (q % (REGIONS / 2)) * RPRG + lane / CPR;
          const int c = (lane % CPR) ^ (r & SWZ);
          const int f = n0 + part * PC + c * 8;
          const uint32_t voff = (r < rows_valid && f < a.F)
                                    ? (uint32_t)((r * 2 * a.F + half * a.F + f) * 2)
                                    : kOOB;
          dma16(rAct, lds_addr(smem) + q * 1024, voff);
        }
        wait_vmcnt<0>();
      }
      lds_barrier();
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int m = a_base[i] + mrow, c = pcol(j, g) - part * PC;
            if (!in_part(c)) continue;
            const u32x2 gw = *(const u32x2*)(gplane + poff(m, c));
            const u32x2 uw = *(const u32x2*)(uplane + poff(m, c));
            const float gt[4] = {lo_bf16(gw[0]), hi_bf16(gw[0]), lo_bf16(gw[1]), hi_bf16(gw[1])};
            const float up[4] = {lo_bf16(uw[0]), hi_bf16(uw[0]), lo_bf16(uw[1]), hi_bf16(uw[1])};
            float du[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float dh = acc[i][j][4 * g + q];
              const float sg = sigmoid_fast(gt[q]);
              acc[i][j][4 * g + q] = dh * up[q] * (sg * (1.0f + gt[q] * (1.0f - sg)));
              du[q] = dh * gt[q] * sg;
            }
            put4(gplane, m, c, du[0], du[1], du[2], du[3]);
            // one group at a time: keeps the LDS reads from all being hoisted
            __builtin_amdgcn_sched_barrier(0);
          }
      store_plane(gplane, a.C + a.F, 2 * (int64_t)a.F, m0, seg_hi, n0 + part * PC, a.F);  // dup
      lds_barrier();
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int c = pcol(j, g) - part * PC;
            if (!in_part(c)) continue;
            put4(gplane, a_base[i] + mrow, c, acc[i][j][4 * g + 0], acc[i][j][4 * g + 1],
                 acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
          }
      store_plane(gplane, a.C, 2 * (int64_t)a.F, m0, seg_hi, n0 + part * PC, a.F);  // dgate
    }
  } else if constexpr (EPI == EPI_F32) {
    // fp32 results straight from the accumulators (four consecutive columns
    // per lane and group, 16-byte accesses), written or added to the output
    float* Cf = a.Cf + (MODE == KGROUP ? (int64_t)e * a.strideC : 0) + (int64_t)sp * a.split_stride;
    const int64_t row0 = (MODE == MGROUP) ? m0 : (int64_t)mloc0;
    const int64_t rows_lim = (MODE == MGROUP) ? seg_hi : (int64_t)a.M;
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t row = row0 + a_base[i] + mrow;
          const int col = n0 + b_base[j] + 8 * g + csub;
          if (row < rows_lim && col < a.N) {
            f32x4* p = (f32x4*)(Cf + row * a.ldc + col);
            f32x4 v = {acc[i][j][4 * g + 0], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                       acc[i][j][4 * g + 3]};
            if (a.acc_out) {
              const f32x4 o = *p;
              v = f32x4{o[0] + v[0], o[1] + v[1], o[2] + v[2], o[3] + v[3]};
            }
            *p = v;
          }
        }
  } else {  // EPI_STORE
    uint16_t* Cg = a.C + (MODE == KGROUP ? (int64_t)e * a.strideC : 0);
    const int64_t row0 = (MODE == MGROUP) ? m0 : (int64_t)mloc0;
    const int64_t rows_lim = (MODE == MGROUP) ? seg_hi : (int64_t)a.M;
#pragma unroll
    for (int part = 0; part < NPART; ++part) {
      if (part > 0) lds_barrier();
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int c = pcol(j, g) - part * PC;
            if (!in_part(c)) continue;
            put4(plane, a_base[i] + mrow, c, acc[i][j][4 * g + 0], acc[i][j][4 * g + 1],
                 acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
          }
      store_plane(plane, Cg, a.ldc, row0, rows_lim, n0 + part * PC, a.N);
    }
  }
}

template <class Cfg, int ASRC, int BSRC, int EPI, int MODE, bool NTB = false>
static hipError_t launch(const Args& a, int nblocks, hipStream_t s) {
  if (nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_gemm_kernel<Cfg, ASRC, BSRC, EPI, MODE, NTB>), dim3(nblocks),
                     dim3(Cfg::NT), 0, s, a);
  return hipGetLastError();
}

// M-grouped launch: routed segments use the 128-row tile (= alignment), the
// dense single group (shared experts) the 256-row tile
template <int ASRC, int BSRC, int EPI, class CR = CfgRows>
static hipError_t launch_rows(Args a, int n_cols_per_tile_rows, int n_cols_per_tile_wide, int ncols,
                              hipStream_t s) {
  // routed segments need 128-row tiles (= alignment); the SwiGLU-backward
  // epilogue keeps two act planes in LDS, which the 128-row tile has room
  // for; everything else dense takes the 256-row tile
  auto rows = [&]() {
    a.n_mtiles = (int)((a.m_rows + CR::BM - 1) / CR::BM);
    a.n_ntiles = (ncols + n_cols_per_tile_rows - 1) / n_cols_per_tile_rows;
    if constexpr (BSRC == KC && EPI != EPI_F32) {
      // routed forward products at one row tile per expert or fewer on
      // average (m_rows is the padded capacity, at most G*(kAlign-1) rows
      // above the routed ones) read each weight slice about once: its loads
      // go non-temporal (T = 256: gate/up and down 9 % and 8 % faster; where
      // several row tiles share a weight slice, non-temporal weight loads
      // cost 3-16 %: T = 8192 and the skewed T = 16384 batch)
      if (a.tile_expert && a.m_rows - (int64_t)a.G * (kAlign - 1) <= (int64_t)kAlign * a.G)
        return launch<CR, ASRC, BSRC, EPI, MGROUP, true>(a, a.n_mtiles * a.n_ntiles, s);
    }
    return launch<CR, ASRC, BSRC, EPI, MGROUP>(a, a.n_mtiles * a.n_ntiles, s);
  };
  if constexpr (EPI == EPI_SWIGLU_BWD) {
    return rows();
  } else {
    if (a.tile_expert) return rows();
    const int mt = (int)((a.m_rows + CfgWide::BM - 1) / CfgWide::BM);
    const int ntl = (ncols + n_cols_per_tile_wide - 1) / n_cols_per_tile_wide;
    // few rows (decode-sized batches): the 256-row tile leaves most CUs idle,
    // the 128-row tile doubles the workgroups
    if (mt * ntl < 256) return rows();
    a.n_mtiles = mt;
    a.n_ntiles = ntl;
    return launch<CfgWide, ASRC, BSRC, EPI, MGROUP>(a, a.n_mtiles * a.n_ntiles, s);
  }
}

// Sums the ks fp32 slices of a k-split [M, 2F] gate|up product in slice
// order, then writes act = [gate | up] and h = silu(gate) * up, both rounded
// to bf16 from the fp32 sums as the fused epilogue does.  One thread per four
// consecutive f.
__global__ void __launch_bounds__(256) split_swiglu_kernel(int64_t M, int F, int ks, int64_t stride,
                                                           const float* __restrict__ part,
                                                           uint16_t* __restrict__ act,
                                                           uint16_t* __restrict__ h) {
  const int fq = F / 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= M * fq) return;
  const int64_t m = i / fq;
  const int f = (int)(i % fq) * 4;
  const float* pg = part + m * 2 * F + f;
  f32x4 g = *(const f32x4*)pg, u = *(const f32x4*)(pg + F);
  for (int sl = 1; sl < ks; ++sl) {
    g += *(const f32x4*)(pg + sl * stride);
    u += *(const f32x4*)(pg + sl * stride + F);
  }
  float v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = g[q] * sigmoid_fast(g[q]) * u[q];
  *(u32x2*)(h + m * F + f) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  if (act) {
    *(u32x2*)(act + m * 2 * F + f) = u32x2{pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3])};
    *(u32x2*)(act + m * 2 * F + F + f) = u32x2{pack_bf16x2(u[0], u[1]), pack_bf16x2(u[2], u[3])};
  }
}

// Sums the ks fp32 slices of a k-split [M, N] product in slice order and
// writes the bf16 result.  One thread per four consecutive columns.
__global__ void __launch_bounds__(256) split_store_kernel(int64_t M, int N, int ks, int64_t stride,
                                                          const float* __restrict__ part,
                                                          uint16_t* __restrict__ y) {
  const int nq = N / 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= M * nq) return;
  const int64_t m = i / nq;
  const int n = (int)(i % nq) * 4;
  const float* p = part + m * N + n;
  f32x4 v = *(const f32x4*)p;
  for (int sl = 1; sl < ks; ++sl) v += *(const f32x4*)(p + sl * stride);
  *(u32x2*)(y + m * N + n) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

// Slices of the k range for a dense (one-group) forward product of m_rows
// rows: when its 128 x 256 tiles fill less than half of the 256 CUs, as many
// slices as keep tiles x slices within one round of the CUs (at most 8, at
// least 4 k-stages each); otherwise 1 (no split).
static int dense_split(int64_t m_rows, int N, int K) {
  if (m_rows <= 0) return 1;
  const int64_t tiles =
      ((m_rows + CfgRows::BM - 1) / CfgRows::BM) * ((N + CfgRows::BN - 1) / CfgRows::BN);
  if (tiles >= 128) return 1;
  int ks = (int)(256 / tiles);
  ks = ks < 8 ? ks : 8;
  const int nk = (K + CfgRows::BK - 1) / CfgRows::BK;
  ks = ks < nk / 4 ? ks : nk / 4;
  return ks < 2 ? 1 : ks;
}

// k-split fp32 product into the workspace: slice sl of C[M,N] = A[M,K] . B[N,K]^T
// at ws + sl * M * N
static hipError_t launch_split_f32(int64_t M, int N, int K, const uint16_t* A, int lda,
                                   const uint16_t* B, int ldb, int ks, float* ws, hipStream_t s) {
  Args a = {};
  a.A = A; a.B = B; a.Cf = ws; a.acc_out = 0;
  a.m_rows = M; a.N = N; a.K = K; a.F = 0;
  a.lda = lda; a.ldb = ldb; a.ldc = N; a.strideB = 0; a.G = 1;
  a.ksplit = ks; a.split_stride = M * (int64_t)N;
  a.n_mtiles = (int)((M + CfgRows::BM - 1) / CfgRows::BM);
  a.n_ntiles = (N + CfgRows::BN - 1) / CfgRows::BN;
  return launch<CfgRows, KC, KC, EPI_F32, MGROUP>(a, a.n_mtiles * a.n_ntiles * ks, s);
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
  return launch_rows<KC, KC, EPI_STORE, CfgRows>(a, CfgRows::BN, CfgWide::BN, H, s);
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
  return launch_rows<KC, MC, EPI_STORE, CfgRowsN>(a, CfgRowsN::BN, CfgWide::BN, H, s);
}

// K-grouped launch over G experts' n_mtiles x n_ntiles tiles each.  The
// experts' tile ranges (chunks of the logical order) go to the XCDs in turn:
// with the whole range split into eight contiguous parts instead, a batch
// whose rows sit in a few experts ran on one XCD (the Zipf-skewed T = 16384
// batch's weight gradients: 22.5 ms, against 6.2 ms with the chunks), while
// each expert's tiles still share one L2 (T = 8192 and the expert-parallel
// shard: within 0.3 % of the contiguous split or faster).  Chunks of two
// m-groups balanced the skewed batch better (5.6 ms) but cost the balanced
// one 0.5 %.  A single group (the shared experts) keeps the contiguous split.
template <int EPI>
static hipError_t launch_kgroup(Args a, hipStream_t s) {
  const int tiles = a.G * a.n_mtiles * a.n_ntiles;
  if (a.G == 1) return launch<CfgWgrad, MC, MC, EPI, KGROUP>(a, tiles, s);
  const int ch = a.n_mtiles * a.n_ntiles;  // one expert
  const int cap = (tiles + 4 * kNumXcd - 1) / (4 * kNumXcd);  // at least four chunks per XCD
  a.kg_chunk = ch < cap ? ch : cap;
  a.kg_tiles = tiles;
  const int span = kNumXcd * a.kg_chunk;
  return launch<CfgWgrad, MC, MC, EPI, KGROUP>(a, (tiles + span - 1) / span * span, s);
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
  a.n_mtiles = (H + CfgWgrad::BM - 1) / CfgWgrad::BM; a.n_ntiles = (F + CfgWgrad::BN - 1) / CfgWgrad::BN;
  a.G = G;
  return launch_kgroup<EPI_STORE>(a, s);
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
  a.n_mtiles = (2 * F + CfgWgrad::BM - 1) / CfgWgrad::BM; a.n_ntiles = (H + CfgWgrad::BN - 1) / CfgWgrad::BN;
  a.G = G;
  return launch_kgroup<EPI_STORE>(a, s);
}

size_t dense_fwd_split_workspace_bytes(int64_t m_rows, int H, int F) {
  const int k1 = dense_split(m_rows, 2 * F, H), k2 = dense_split(m_rows, H, F);
  const size_t b1 = k1 > 1 ? (size_t)k1 * m_rows * 2 * F * sizeof(float) : 0;
  const size_t b2 = k2 > 1 ? (size_t)k2 * m_rows * H * sizeof(float) : 0;
  return b1 > b2 ? b1 : b2;
}

hipError_t launch_dense_gate_up_split(int64_t m_rows, int H, int F, const uint16_t* x,
                                      const uint16_t* w1, uint16_t* act, uint16_t* h, void* ws,
                                      hipStream_t s) {
  const int ks = dense_split(m_rows, 2 * F, H);
  if (ks == 1)
    return launch_gemm_gate_up(1, m_rows, H, F, nullptr, nullptr, nullptr, x, w1, act, h, s);
  hipError_t e = launch_split_f32(m_rows, 2 * F, H, x, H, w1, H, ks, (float*)ws, s);
  if (e != hipSuccess) return e;
  const int64_t n = m_rows * (F / 4);
  hipLaunchKernelGGL(split_swiglu_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, m_rows,
                     F, ks, m_rows * 2 * (int64_t)F, (const float*)ws, act, h);
  return hipGetLastError();
}

hipError_t launch_dense_down_split(int64_t m_rows, int H, int F, const uint16_t* h,
                                   const uint16_t* w2, uint16_t* y, void* ws, hipStream_t s) {
  const int ks = dense_split(m_rows, H, F);
  if (ks == 1) return launch_gemm_down(1, m_rows, H, F, nullptr, nullptr, nullptr, h, w2, y, s);
  hipError_t e = launch_split_f32(m_rows, H, F, h, F, w2, F, ks, (float*)ws, s);
  if (e != hipSuccess) return e;
  const int64_t n = m_rows * (H / 4);
  hipLaunchKernelGGL(split_store_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, m_rows,
                     H, ks, m_rows * (int64_t)H, (const float*)ws, y);
  return hipGetLastError();
}

// C[M,N] (+)= A[M,K] . B[N,K]^T: bf16 operands with K-contiguous rows, fp32
// output, one dense group.  K, lda, ldb multiples of 8; N, ldc multiples of 4.
hipError_t launch_gemm_f32_nt(int64_t M, int N, int K, const uint16_t* A, int lda,
                              const uint16_t* B, int ldb, float* C, int ldc, bool accumulate,
                              hipStream_t s) {
  Args a = {};
  a.A = A; a.B = B; a.Cf = C; a.acc_out = accumulate ? 1 : 0;
  a.m_rows = M; a.N = N; a.K = K; a.F = 0;
  a.lda = lda; a.ldb = ldb; a.ldc = ldc; a.strideB = 0; a.G = 1;
  return launch_rows<KC, KC, EPI_F32>(a, CfgRows::BN, CfgWide::BN, N, s);
}

// C_g[M,N] = sum over the rows r of segment g of A[r,m] . B[r,n] (A [rows,M],
// B [rows,N], bf16 row-major), fp32 C_g at C + g * strideC.  M, N, lda, ldb
// multiples of 8.
hipError_t launch_gemm_f32_tn_grouped(int G, const int32_t* offsets, const int32_t* counts,
                                      int64_t rows, int M, int N, const uint16_t* A, int lda,
                                      const uint16_t* B, int ldb, float* C, int ldc,
                                      int64_t strideC, hipStream_t s) {
  Args a = {};
  a.A = A; a.B = B; a.Cf = C; a.acc_out = 0;
  a.offsets = offsets; a.counts = counts;
  a.m_rows = rows; a.M = M; a.N = N; a.F = 0;
  a.lda = lda; a.ldb = ldb; a.ldc = ldc; a.strideB = 0; a.strideC = strideC;
  a.n_mtiles = (M + CfgWgrad::BM - 1) / CfgWgrad::BM; a.n_ntiles = (N + CfgWgrad::BN - 1) / CfgWgrad::BN;
  a.G = G;
  return launch_kgroup<EPI_F32>(a, s);
}

}  // namespace moe
