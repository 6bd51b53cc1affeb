// Grouped bf16 GEMMs of the MoE expert FFN on gfx950 MFMA.
//
// The expert token segments are padded to the row tile, so every row tile
// belongs to exactly one expert and the grouped GEMM tiles like a plain GEMM
// ("dots.llm1 Technical Report" summary page, "Key claims" and "Method": the
// grouped GEMM pads expert token segments to tile multiples so tiling inside a
// block is uniform).  The pages built that for Hopper WGMMA tiles; here the
// tile is sized for CDNA4: a 128x256 workgroup tile of four wave64 waves, each
// computing 64x128 with v_mfma_f32_32x32x16_bf16, LDS double-buffered.
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
//   K-contig tile  [rows][64 k]: 128 B per row, 16 B chunk c stored at
//                  c ^ ((row >> 1) & 7).  Fragments read with ds_read_b128.
//   MN-contig tile [64 k][cols]: 2*cols B per k-row, 16 B chunk c stored at
//                  c ^ (4 * (k & 3)).  Fragments read with two
//                  ds_read_b64_tr_b16 (transposing LDS read of gfx950).
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

constexpr int BM = 128, BN = 256, BK = 64, NT = 256;
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
  int64_t m_rows;        // MGROUP: rows of A/C; KGROUP dense: rows of the segment
  int M, N, K;           // logical GEMM dims (MGROUP: M unused; KGROUP: per group)
  int lda, ldb, ldc;     // leading dims (elements)
  int64_t strideB;       // elements between consecutive groups' B
  int64_t strideC;       // KGROUP: elements between consecutive groups' C
  int F;                 // SWIGLU: expert width (gate/up split)
  int n_mtiles, n_ntiles, G;
};

// --------------------------------------------------------------------------
// Global -> register staging of one BK slice of an operand tile
// --------------------------------------------------------------------------
// K-contig tile of R rows: chunk q -> row q/8, k-chunk q%8.
template <int R>
struct KcStage {
  static constexpr int PER = R * 8 / NT;
  u32x4 v[PER];
  // row_ptr(row) returns the global row pointer or nullptr if the row is invalid
  template <class RowFn>
  __device__ __forceinline__ void load(RowFn row_ptr, int k0, int K, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int q = tid + i * NT;
      int r = q >> 3, c = q & 7;
      const uint16_t* p = row_ptr(r);
      int k = k0 + c * 8;
      if (p != nullptr && k < K)
        v[i] = *(const u32x4*)(p + k);
      else
        v[i] = u32x4{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void store(uint8_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int q = tid + i * NT;
      int r = q >> 3, c = q & 7;
      *(u32x4*)(lds + r * 128 + ((c ^ ((r >> 1) & 7)) << 4)) = v[i];
    }
  }
};

// MN-contig tile of C columns: chunk q -> k-row q/(C/8), col-chunk q%(C/8).
template <int C>
struct McStage {
  static constexpr int CPR = C / 8;  // chunks per k-row
  static constexpr int PER = BK * CPR / NT;
  u32x4 v[PER];
  // krow_ptr(k) returns the global pointer of k-row (at the tile's first col) or nullptr
  template <class KRowFn>
  __device__ __forceinline__ void load(KRowFn krow_ptr, int col0, int ncols, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int q = tid + i * NT;
      int kr = q / CPR, c = q % CPR;
      const uint16_t* p = krow_ptr(kr);
      if (p != nullptr && col0 + c * 8 < ncols)
        v[i] = *(const u32x4*)(p + c * 8);
      else
        v[i] = u32x4{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void store(uint8_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int q = tid + i * NT;
      int kr = q / CPR, c = q % CPR;
      *(u32x4*)(lds + kr * (C * 2) + ((c ^ (4 * (kr & 3))) << 4)) = v[i];
    }
  }
};

// --------------------------------------------------------------------------
// LDS -> fragment
// --------------------------------------------------------------------------
__device__ __forceinline__ bf16x8 frag_kc(const uint8_t* lds, int base, int kk, int lane) {
  int row = base + (lane & 31);
  int c = 2 * kk + (lane >> 5);
  return *(const bf16x8*)(lds + row * 128 + ((c ^ ((row >> 1) & 7)) << 4));
}

template <int C>
__device__ __forceinline__ bf16x8 frag_mc(const uint8_t* lds, int base, int kk, int lane) {
  int g = lane >> 4, li = lane & 15;
  int col = base + 16 * (g & 1) + 4 * (li & 3);
  int kb = 16 * kk + 8 * (g >> 1) + (li >> 2);
  int c = col >> 3, sub = (col & 7) * 2;
  int k0 = kb, k1 = kb + 4;
  const uint8_t* p0 = lds + k0 * (C * 2) + ((c ^ (4 * (k0 & 3))) << 4) + sub;
  const uint8_t* p1 = lds + k1 * (C * 2) + ((c ^ (4 * (k1 & 3))) << 4) + sub;
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, p0));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, p1));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

template <int SRC, int C>
__device__ __forceinline__ bf16x8 frag(const uint8_t* lds, int base, int kk, int lane) {
  if constexpr (SRC == KC) return frag_kc(lds, base, kk, lane);
  else return frag_mc<C>(lds, base, kk, lane);
}

// --------------------------------------------------------------------------
// The kernel
// --------------------------------------------------------------------------
template <int ASRC, int BSRC, int EPI, int MODE>
__global__ void __launch_bounds__(NT, 1) grouped_gemm_kernel(Args a) {
  constexpr int A_BYTES = BM * BK * 2;  // 16 KB
  constexpr int B_BYTES = BN * BK * 2;  // 32 KB
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (A_BYTES + B_BYTES)];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- tile decode ---------------------------------------------------
  const int nblocks = gridDim.x;
  const int L = xcd_remap(blockIdx.x, nblocks);
  int e, mt, nt;
  if constexpr (MODE == MGROUP) {
    const int per_group = GROUP_M * a.n_ntiles;
    const int grp = L / per_group, within = L % per_group;
    const int gm = min(GROUP_M, a.n_mtiles - grp * GROUP_M);
    mt = grp * GROUP_M + within % gm;
    nt = within / gm;
    e = a.tile_expert ? a.tile_expert[mt] : 0;
    if (e < 0) return;
  } else {
    const int per_e = a.n_mtiles * a.n_ntiles;
    e = L / per_e;
    const int rem = L % per_e;
    const int per_group = GROUP_M * a.n_ntiles;
    const int grp = rem / per_group, within = rem % per_group;
    const int gm = min(GROUP_M, a.n_mtiles - grp * GROUP_M);
    mt = grp * GROUP_M + within % gm;
    nt = within / gm;
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
  const int mloc0 = (MODE == MGROUP) ? 0 : mt * BM;    // KGROUP: first output row (M dim)
  const int n0 = nt * (EPI == EPI_SWIGLU_FWD ? BN / 2 : BN);  // SWIGLU_FWD: f offset

  int nk;
  int64_t k_base;  // first K index (KGROUP: first segment row)
  if constexpr (MODE == MGROUP) {
    nk = (a.K + BK - 1) / BK;
    k_base = 0;
  } else {
    nk = (int)((seg_hi - seg_lo + BK - 1) / BK);
    k_base = seg_lo;
  }

  // ---- operand row/col pointer functions ------------------------------
  auto a_row_kc = [&](int r) -> const uint16_t* {   // A K-contig (MGROUP)
    int64_t row = m0 + r;
    return row < seg_hi ? a.A + row * a.lda : nullptr;
  };
  auto b_row_kc = [&](int r) -> const uint16_t* {   // B K-contig: B row n
    int n;
    if constexpr (EPI == EPI_SWIGLU_FWD) {
      int f = n0 + (r & (BN / 2 - 1));
      if (f >= a.F) return nullptr;
      n = (r < BN / 2) ? f : a.F + f;
    } else {
      n = n0 + r;
      if (n >= a.N) return nullptr;
    }
    return Bg + (int64_t)n * a.ldb;
  };

  KcStage<BM> sa_kc;
  McStage<BM> sa_mc;
  KcStage<BN> sb_kc;
  McStage<BN> sb_mc;

  auto load_tile = [&](int kt) {
    const int k0 = kt * BK;
    if constexpr (ASRC == KC) {
      sa_kc.load(a_row_kc, k0, a.K, tid);
    } else {  // A MN-contig: k-rows are segment rows (KGROUP)
      auto krow = [&](int kr) -> const uint16_t* {
        int64_t row = k_base + k0 + kr;
        return row < seg_hi ? a.A + row * a.lda + mloc0 : nullptr;
      };
      sa_mc.load(krow, mloc0, a.M, tid);
    }
    if constexpr (BSRC == KC) {
      sb_kc.load(b_row_kc, k0, a.K, tid);
    } else {
      if constexpr (MODE == MGROUP) {  // B = W [K][N] N-contig
        auto krow = [&](int kr) -> const uint16_t* {
          int k = k0 + kr;
          return k < a.K ? Bg + (int64_t)k * a.ldb + n0 : nullptr;
        };
        sb_mc.load(krow, n0, a.N, tid);
      } else {  // B = rows of the segment, N-contig
        auto krow = [&](int kr) -> const uint16_t* {
          int64_t row = k_base + k0 + kr;
          return row < seg_hi ? a.B + row * a.ldb + n0 : nullptr;
        };
        sb_mc.load(krow, n0, a.N, tid);
      }
    }
  };
  auto store_tile = [&](int buf) {
    uint8_t* As = smem + buf * (A_BYTES + B_BYTES);
    uint8_t* Bs = As + A_BYTES;
    if constexpr (ASRC == KC) sa_kc.store(As, tid); else sa_mc.store(As, tid);
    if constexpr (BSRC == KC) sb_kc.store(Bs, tid); else sb_mc.store(Bs, tid);
  };

  // wave's fragment bases
  const int a_base0 = wm * 64;  // rows of A tile
  int b_base[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (EPI == EPI_SWIGLU_FWD)
      b_base[j] = (j < 2) ? (wn * 64 + j * 32) : (BN / 2 + wn * 64 + (j - 2) * 32);
    else
      b_base[j] = wn * 128 + j * 32;
  }

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  if (nk > 0) {
    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) load_tile(kt + 1);
      const uint8_t* As = smem + cur * (A_BYTES + B_BYTES);
      const uint8_t* Bs = As + A_BYTES;
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        bf16x8 af[2], bfr[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) af[i] = frag<ASRC, BM>(As, a_base0 + i * 32, kk, lane);
#pragma unroll
        for (int j = 0; j < 4; ++j) bfr[j] = frag<BSRC, BN>(Bs, b_base[j], kk, lane);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < nk) store_tile(cur ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue --------------------------------------------------------
  // acc[i][j][r]: row m = a_base0 + 32 i + (lane & 31)
  //               col n = b_base[j] + 8 (r/4) + 4 (lane/32) + r%4
  const int mrow = lane & 31;
  const int csub = 4 * (lane >> 5);
  if constexpr (EPI == EPI_SWIGLU_FWD) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t row = m0 + a_base0 + 32 * i + mrow;
      if (row >= seg_hi) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int f = n0 + wn * 64 + j * 32 + 8 * g + csub;
          if (f >= a.F) continue;
          float hv[4];
          uint32_t gw[2], uw[2], hw[2];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float gt = acc[i][j][4 * g + q], up = acc[i][j + 2][4 * g + q];
            hv[q] = gt / (1.0f + expf(-gt)) * up;
          }
          hw[0] = pack_bf16x2(hv[0], hv[1]);
          hw[1] = pack_bf16x2(hv[2], hv[3]);
          *(u32x2*)(a.C + row * a.ldc + f) = u32x2{hw[0], hw[1]};
          if (a.C2) {
            gw[0] = pack_bf16x2(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]);
            gw[1] = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
            uw[0] = pack_bf16x2(acc[i][j + 2][4 * g + 0], acc[i][j + 2][4 * g + 1]);
            uw[1] = pack_bf16x2(acc[i][j + 2][4 * g + 2], acc[i][j + 2][4 * g + 3]);
            uint16_t* ar = a.C2 + row * (int64_t)(2 * a.F);
            *(u32x2*)(ar + f) = u32x2{gw[0], gw[1]};
            *(u32x2*)(ar + a.F + f) = u32x2{uw[0], uw[1]};
          }
        }
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU_BWD) {
    // acc = dh[row][f]; aux = act [rows][2F]; C = dact [rows][2F]
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t row = m0 + a_base0 + 32 * i + mrow;
      if (row >= seg_hi) continue;
      const uint16_t* actr = a.aux + row * (int64_t)(2 * a.F);
      uint16_t* dactr = a.C + row * (int64_t)(2 * a.F);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int f = n0 + b_base[j] + 8 * g + csub;
          if (f >= a.F) continue;
          u32x2 gw = *(const u32x2*)(actr + f);
          u32x2 uw = *(const u32x2*)(actr + a.F + f);
          float gt[4] = {lo_bf16(gw[0]), hi_bf16(gw[0]), lo_bf16(gw[1]), hi_bf16(gw[1])};
          float up[4] = {lo_bf16(uw[0]), hi_bf16(uw[0]), lo_bf16(uw[1]), hi_bf16(uw[1])};
          float dg[4], du[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float dh = acc[i][j][4 * g + q];
            float sg = 1.0f / (1.0f + expf(-gt[q]));
            dg[q] = dh * up[q] * (sg * (1.0f + gt[q] * (1.0f - sg)));
            du[q] = dh * gt[q] * sg;
          }
          *(u32x2*)(dactr + f) = u32x2{pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3])};
          *(u32x2*)(dactr + a.F + f) = u32x2{pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3])};
        }
      }
    }
  } else {  // EPI_STORE
    uint16_t* Cg = a.C + (MODE == KGROUP ? (int64_t)e * a.strideC : 0);
    const int64_t rows_lim = (MODE == MGROUP) ? seg_hi : (int64_t)a.M;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t row = (MODE == MGROUP ? m0 : (int64_t)mloc0) + a_base0 + 32 * i + mrow;
      if (row >= rows_lim) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + b_base[j] + 8 * g + csub;
          if (n >= a.N) continue;
          *(u32x2*)(Cg + row * a.ldc + n) =
              u32x2{pack_bf16x2(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]),
                    pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3])};
        }
      }
    }
  }
}

template <int ASRC, int BSRC, int EPI, int MODE>
static hipError_t launch(const Args& a, int nblocks, hipStream_t s) {
  if (nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_gemm_kernel<ASRC, BSRC, EPI, MODE>), dim3(nblocks), dim3(NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace gemm

using namespace gemm;

// M-tiles covering m_rows rows
static inline int mtiles(int64_t m_rows) { return (int)((m_rows + BM - 1) / BM); }

hipError_t launch_gemm_gate_up(int G, int64_t m_rows, int H, int F, const int32_t* offsets,
                               const int32_t* counts, const int32_t* tile_expert,
                               const uint16_t* x_rows, const uint16_t* w1, uint16_t* act,
                               uint16_t* h, hipStream_t s) {
  Args a = {};
  a.A = x_rows; a.B = w1; a.C = h; a.C2 = act;
  a.offsets = offsets; a.counts = counts; a.tile_expert = tile_expert;
  a.m_rows = m_rows; a.N = 2 * F; a.K = H; a.F = F;
  a.lda = H; a.ldb = H; a.ldc = F; a.strideB = (int64_t)2 * F * H;
  a.n_mtiles = mtiles(m_rows); a.n_ntiles = (F + BN / 2 - 1) / (BN / 2); a.G = G;
  return launch<KC, KC, EPI_SWIGLU_FWD, MGROUP>(a, a.n_mtiles * a.n_ntiles, s);
}

hipError_t launch_gemm_down(int G, int64_t m_rows, int H, int F, const int32_t* offsets,
                            const int32_t* counts, const int32_t* tile_expert,
                            const uint16_t* h, const uint16_t* w2, uint16_t* y_rows,
                            hipStream_t s) {
  Args a = {};
  a.A = h; a.B = w2; a.C = y_rows;
  a.offsets = offsets; a.counts = counts; a.tile_expert = tile_expert;
  a.m_rows = m_rows; a.N = H; a.K = F; a.F = F;
  a.lda = F; a.ldb = F; a.ldc = H; a.strideB = (int64_t)H * F;
  a.n_mtiles = mtiles(m_rows); a.n_ntiles = (H + BN - 1) / BN; a.G = G;
  return launch<KC, KC, EPI_STORE, MGROUP>(a, a.n_mtiles * a.n_ntiles, s);
}

hipError_t launch_gemm_dgrad_down(int G, int64_t m_rows, int H, int F, const int32_t* offsets,
                                  const int32_t* counts, const int32_t* tile_expert,
                                  const uint16_t* dy_rows, const uint16_t* w2,
                                  const uint16_t* act, uint16_t* dact, hipStream_t s) {
  Args a = {};
  a.A = dy_rows; a.B = w2; a.C = dact; a.aux = act;
  a.offsets = offsets; a.counts = counts; a.tile_expert = tile_expert;
  a.m_rows = m_rows; a.N = F; a.K = H; a.F = F;
  a.lda = H; a.ldb = F; a.ldc = 2 * F; a.strideB = (int64_t)H * F;
  a.n_mtiles = mtiles(m_rows); a.n_ntiles = (F + BN - 1) / BN; a.G = G;
  return launch<KC, MC, EPI_SWIGLU_BWD, MGROUP>(a, a.n_mtiles * a.n_ntiles, s);
}

hipError_t launch_gemm_dgrad_up(int G, int64_t m_rows, int H, int F, const int32_t* offsets,
                                const int32_t* counts, const int32_t* tile_expert,
                                const uint16_t* dact, const uint16_t* w1, uint16_t* dx_rows,
                                hipStream_t s) {
  Args a = {};
  a.A = dact; a.B = w1; a.C = dx_rows;
  a.offsets = offsets; a.counts = counts; a.tile_expert = tile_expert;
  a.m_rows = m_rows; a.N = H; a.K = 2 * F; a.F = F;
  a.lda = 2 * F; a.ldb = H; a.ldc = H; a.strideB = (int64_t)2 * F * H;
  a.n_mtiles = mtiles(m_rows); a.n_ntiles = (H + BN - 1) / BN; a.G = G;
  return launch<KC, MC, EPI_STORE, MGROUP>(a, a.n_mtiles * a.n_ntiles, s);
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
  a.n_mtiles = (H + BM - 1) / BM; a.n_ntiles = (F + BN - 1) / BN; a.G = G;
  return launch<MC, MC, EPI_STORE, KGROUP>(a, G * a.n_mtiles * a.n_ntiles, s);
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
  a.n_mtiles = (2 * F + BM - 1) / BM; a.n_ntiles = (H + BN - 1) / BN; a.G = G;
  return launch<MC, MC, EPI_STORE, KGROUP>(a, G * a.n_mtiles * a.n_ntiles, s);
}

}  // namespace moe
