// Global -> LDS loading (buffer_load ... lds), its waits and barriers, and
// the K-contiguous tile layout with its MFMA fragment read, shared by the
// grouped GEMMs and the router projection.
#pragma once
#include "common.h"

namespace moe {
namespace lds {

// --------------------------------------------------------------------------
// Global -> LDS: buffer loads straight into LDS (buffer_load_dwordx4 ... lds)
// --------------------------------------------------------------------------
// Each wave-level load moves 64 lanes x 16 B = 1 KB into a contiguous LDS
// region whose base is wave-uniform (M0); lane l lands at base + 16*l.  The
// LDS swizzle is therefore applied on the global side: lane l fetches the
// global chunk that belongs at its LDS slot.  A lane whose element is out of
// range (rows past the segment, k past K, columns past N) gets the offset
// kOOB, past the buffer's num_records, which the hardware turns into zeros
// (checked per dword), so masked rows and tails contribute exactly nothing.
// kOOB must lie at or above every num_records a resource here is built with:
// a resource covers whole rows, below 4 GiB in all (the host refuses larger
// segments), and every row is a multiple of 128 bytes, so num_records is at
// most 2^32 - 128 < kOOB.  kOOB + 12, the last dword of a 16-byte load, does
// not wrap in 32 bits.
constexpr uint32_t kOOB = 0xFFFFFFF0u;
static_assert(kOOB >= 0xFFFFFF80u && kOOB <= 0xFFFFFFFFu - 12u, "out-of-range offset sentinel");
constexpr uint32_t kRsrcWord3 = 0x00020000u;

// raw buffer resource: base, stride 0, num_records = bytes.  The arguments
// are workgroup-uniform; readfirstlane makes that explicit so the descriptor
// lives in SGPRs, as the buffer instruction requires.
__device__ __forceinline__ u32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(b >> 32) & 0xffffu)),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes), kRsrcWord3};
}

// One wave-level global -> LDS load of 64 x 16 B.  lds: wave-uniform LDS byte
// address of the 1 KB destination.  Issued from inline asm so that the compiler
// does not treat the LDS writes as aliasing every later LDS read (it would put
// a wait for all outstanding loads before each transposing read); the kernel
// orders them itself with explicit vmcnt waits and barriers.  M0 is used by
// nothing else in these kernels.  NT marks the load non-temporal (streamed:
// for an operand every line of which is read once).
template <bool NT = false>
__device__ __forceinline__ void dma16(const u32x4& rs_in, uint32_t lds, uint32_t voff) {
  // both are workgroup-uniform; readfirstlane keeps them in SGPRs whatever
  // the compiler concluded about their uniformity
  lds = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds);
  const u32x4 rs = {(uint32_t)__builtin_amdgcn_readfirstlane((int)rs_in[0]),
                    (uint32_t)__builtin_amdgcn_readfirstlane((int)rs_in[1]),
                    (uint32_t)__builtin_amdgcn_readfirstlane((int)rs_in[2]),
                    (uint32_t)__builtin_amdgcn_readfirstlane((int)rs_in[3])};
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen nt lds"
        :
        : "s"(lds), "v"(voff), "s"(rs)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds"
        :
        : "s"(lds), "v"(voff), "s"(rs)
        : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(__attribute__((address_space(3))) const void*)p;
}

// s_waitcnt vmcnt(n) leaving expcnt/lgkmcnt unconstrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
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

// every wave's LDS reads done, then a workgroup barrier that orders memory
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
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
  template <bool NT = false>
  __device__ __forceinline__ void issue(const u32x4& rs, uint32_t lds, int wave, int i, int kt,
                                        int K) const {
    const int q = i * NW + wave;
    const bool kin = kt * BK + kel[i] < K;
    const uint32_t v = (off[i] == kOOB || !kin) ? kOOB : off[i] + (uint32_t)kt * (BK * 2);
    dma16<NT>(rs, lds + q * 1024, v);
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

}  // namespace lds
}  // namespace moe
