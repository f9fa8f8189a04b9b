// Internal helpers shared by the HIP sources of the ring-attention library.
// gfx950 only: 64-lane waves, bf16 MFMA 32x32x16, LDS transpose reads,
// permlane32 swaps.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Finite "minus infinity" for running maxima: exp2(s - m) stays 0 for masked
// scores (s = -inf) and no (-inf) - (-inf) is ever formed.
constexpr float kNegBig = -1.0e30f;

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16).
// Lane l supplies A[l%32][8*(l/32) + i] and B[8*(l/32) + i][l%32], i = 0..7;
// it receives D[8*(r/4) + 4*(l/32) + r%4][l%32] in register r = 0..15.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// acc += A * B with the accumulator held in AGPRs (inline asm, so that the
// register allocator keeps it out of the VGPR budget).  The compiler does not
// see inside the asm: the caller must not write A or B with a vector ALU
// instruction in the two wait states before (an MFMA reading a VGPR that a
// VALU op just wrote needs them); LDS loads are covered by the compiler's
// s_waitcnt.  Consecutive uses of one accumulator need no wait (exact overlap).
__device__ __forceinline__ void mfma32_acc(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Before anything else reads accumulators written by mfma32_acc: covers the
// wait states between the last MFMA writing them and a read (the asm takes
// each accumulator as an operand, so no read is scheduled above it).
template <int N>
__device__ __forceinline__ void acc_ready(f32x16 (&x)[N], f32x16 (&y)[N]) {
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+a"(x[i]), "+a"(y[i]));
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives element i%4 of the 8-byte chunk addressed by lane
// 4*t + i/4, for t = 0..3.  If lane j of the group addresses row (r0 + j/4),
// columns (c0 + 4*(j%4)) .. +3 of a row-major 16-bit matrix, lane i receives
// column c0 + i of rows r0 .. r0 + 3: a 4x16 block read transposed.
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Value of x in lane l ^ 32, combined with x by max / add.
__device__ __forceinline__ float max_halves(float x) {
  unsigned u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_halves(float x) {
  unsigned u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Pack registers [8*half, 8*half + 8) of an fp32 accumulator into bf16 (RNE).
__device__ __forceinline__ bf16x8 to_bf16x8(const f32x16& s, int half) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (bf16)s[8 * half + i];
  return r;
}

// Workgroup -> tile mapping that keeps consecutive tiles on one XCD.  The
// dispatcher places workgroup w on XCD w % 8; with this remap XCD x runs the
// contiguous tile range [x*n/8, (x+1)*n/8), so the workgroups that share a
// head's key/value block share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int w, int n) {
  if ((n & 7) != 0) return w;
  return (w & 7) * (n >> 3) + (w >> 3);
}

// ---- tile staging: swizzled LDS rows filled by direct-to-LDS copies ------

typedef __attribute__((address_space(3))) void lvoid;

// Physical 16-byte chunk of logical chunk c in row r is c ^ swz(r).
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128)
    return ((r & 3) << 2) | ((r >> 2) & 3);
  else
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Direct-to-LDS copy of 16 bytes per lane: lane l's bytes land at LDS byte
// address lds_base + 16*l (lds_base wave-uniform).  Issued from inline asm so
// that the compiler does not order every later LDS read after it; the kernel
// waits for these loads itself (s_waitcnt vmcnt + barrier) before reading the
// stage they fill.  The instruction has no register outputs.
// NT sets the non-temporal cache policy: for data read exactly once (a
// decode step's key/value stream), which then streams past the L2 instead of
// displacing it; kernels that re-read tiles from L2 leave it off.
#define RA_DMA16(SFX) "s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" SFX
template <bool NT = false>
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  if constexpr (NT)
    asm volatile(RA_DMA16(" nt") :: "v"(src), "s"(lds_base) : "memory", "m0");
  else
    asm volatile(RA_DMA16("") :: "v"(src), "s"(lds_base) : "memory", "m0");
}
#undef RA_DMA16

// N consecutive 1 KiB direct-to-LDS copies from a wave-uniform base: copy i
// reads 16 bytes per lane at sbase + voff[i] + 1024 i and writes them to LDS
// byte address lds_base + 1024 i + 16*lane.  The instruction offset applies to
// both the global and the LDS address, so M0 is written once for the group.
#define RA_DMA16_G1(SFX) "s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" SFX
#define RA_DMA16_G2(SFX)                         \
  "s_mov_b32 m0, %3\n\t"                         \
  "global_load_lds_dwordx4 %0, %2" SFX "\n\t"    \
  "global_load_lds_dwordx4 %1, %2 offset:1024" SFX
#define RA_DMA16_G4(SFX)                                \
  "s_mov_b32 m0, %5\n\t"                                \
  "global_load_lds_dwordx4 %0, %4" SFX "\n\t"           \
  "global_load_lds_dwordx4 %1, %4 offset:1024" SFX "\n\t" \
  "global_load_lds_dwordx4 %2, %4 offset:2048" SFX "\n\t" \
  "global_load_lds_dwordx4 %3, %4 offset:3072" SFX
template <int N, bool NT = false>
__device__ __forceinline__ void dma16_group(const void* sbase, const uint32_t (&voff)[N],
                                            uint32_t lds_base) {
  static_assert(N == 1 || N == 2 || N == 4, "group size");
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
  if constexpr (N == 1) {
    if constexpr (NT)
      asm volatile(RA_DMA16_G1(" nt") :: "v"(voff[0]), "s"(sbase), "s"(m0) : "memory", "m0");
    else
      asm volatile(RA_DMA16_G1("") :: "v"(voff[0]), "s"(sbase), "s"(m0) : "memory", "m0");
  } else if constexpr (N == 2) {
    if constexpr (NT)
      asm volatile(RA_DMA16_G2(" nt") :: "v"(voff[0]), "v"(voff[1]), "s"(sbase), "s"(m0)
                   : "memory", "m0");
    else
      asm volatile(RA_DMA16_G2("") :: "v"(voff[0]), "v"(voff[1]), "s"(sbase), "s"(m0)
                   : "memory", "m0");
  } else {
    if constexpr (NT)
      asm volatile(RA_DMA16_G4(" nt") :: "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]),
                   "s"(sbase), "s"(m0) : "memory", "m0");
    else
      asm volatile(RA_DMA16_G4("") :: "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]),
                   "s"(sbase), "s"(m0) : "memory", "m0");
  }
}
#undef RA_DMA16_G1
#undef RA_DMA16_G2
#undef RA_DMA16_G4

// Direct-to-LDS copy of 4 bytes per lane: lane l's word lands at LDS byte
// address lds_base + 4*l.  Same contract as dma16.
__device__ __forceinline__ void dma4(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
               :: "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base)) : "memory", "m0");
}

// A pointer the caller knows to be wave-uniform, moved to scalar registers.
template <typename T>
__device__ __forceinline__ T* uniform(T* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}


// Source offsets of the swizzled tile copies.  Load j of a tile moves bytes
// [1024 j, 1024 j + 1024) of the LDS tile; lane l's 16 bytes come from
// source byte offset
//     1024 j + (lane_part(l) ^ (swz(1024 j / ROWB) << 4)),
// where lane_part is the offset for j = 0.  This holds because every 1 KiB
// covers whole rows (ROWB divides 1024) and the swizzle of row r + 1024j/ROWB
// differs from that of r < 1024/ROWB by swz(1024j/ROWB) (XOR-linear in the
// bits involved).  So a load costs one XOR with a wave-uniform value.
template <int D>
__device__ __forceinline__ uint32_t dma_lane_part(int lane) {
  constexpr int ROWB = D * 2;
  const int q = lane * 16;
  const int row = q / ROWB;
  return (uint32_t)(row * ROWB + ((((q % ROWB) >> 4) ^ swz<D>(row)) << 4));
}
template <int D>
__device__ __forceinline__ uint32_t dma_xor(int j) {
  return (uint32_t)(swz<D>(j * 1024 / (D * 2)) << 4);
}

// Loads j0 .. j0+N-1 of a swizzled tile copy (j0 wave-uniform): the tile's
// first row is row t0 of a [L x D] tensor A; load j fills LDS bytes
// tile_lds + 1024 j ... + 1023.  One scalar branch per call picks the full
// tile form (scalar base + one XOR-add per load) or the ragged form (rows
// past L-1 clamped to L-1).
// The same loads, each under its own full / ragged test with its own M0.
// Same effect; which form schedules better depends on the kernel.
template <int D, int BT, int N, bool NT = false>
__device__ __forceinline__ void dma_tile_loads_split(uint32_t tile_lds, const bf16* A, int t0,
                                                     int L, int j0, uint32_t lane_part) {
  constexpr int ROWB = D * 2;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int j = j0 + i;
    const uint32_t lds = __builtin_amdgcn_readfirstlane(tile_lds + (uint32_t)j * 1024);
    const uint32_t off = lane_part ^ dma_xor<D>(j);
    if (t0 + BT <= L) {
      const uint32_t voff[1] = {off + (uint32_t)j * 1024};
      dma16_group<1, NT>(uniform(A + (size_t)t0 * D), voff, lds);
    } else {
      const int row = j * (1024 / ROWB) + (int)(off / ROWB);
      dma16<NT>((const char*)(A + (size_t)min(t0 + row, L - 1) * D) + off % ROWB, lds);
    }
  }
}

template <int D, int BT, int N, bool NT = false>
__device__ __forceinline__ void dma_tile_loads(uint32_t tile_lds, const bf16* A, int t0, int L,
                                               int j0, uint32_t lane_part) {
  constexpr int ROWB = D * 2;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(tile_lds + (uint32_t)j0 * 1024);
  if (t0 + BT <= L) {
    uint32_t voff[N];  // (x ^ y) + z: one v_xad_u32 each
#pragma unroll
    for (int i = 0; i < N; ++i) voff[i] = (lane_part ^ dma_xor<D>(j0 + i)) + (uint32_t)j0 * 1024;
    dma16_group<N, NT>(uniform(A + (size_t)t0 * D), voff, lds0);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int j = j0 + i;
      const uint32_t off = lane_part ^ dma_xor<D>(j);
      const int row = j * (1024 / ROWB) + (int)(off / ROWB);
      dma16<NT>((const char*)(A + (size_t)min(t0 + row, L - 1) * D) + off % ROWB,
                lds0 + i * 1024);
    }
  }
}

// Copies one [BT x D] bf16 tile (rows t0 .. t0+BT-1 of a [L x D] tensor)
// into swizzled LDS rows with NL = TILEB / 1 KiB loads.  Either every wave
// issues LPW = NL / NW of them, or (NL < NW) waves 0 .. NL-1 issue one each
// and the rest none: a wave never has more than LPW loads per tile in
// flight, which is what a kernel counts in vmcnt.
// HOLD keeps the lane offset in a register across calls; otherwise it is
// recomputed at each call (for kernels short of registers).  SPLIT issues
// each load under its own full / ragged test (dma_tile_loads_split), which
// measured faster in the forward kernel; otherwise one test per call.  NT
// issues the copies with the non-temporal cache policy (see dma16).
template <int D, int BT, int NW, bool HOLD = true, bool SPLIT = false, bool NT = false>
struct TileLoader {
  static constexpr int ROWB = D * 2;
  static constexpr int TILEB = BT * ROWB;
  static constexpr int NL = TILEB / 1024;
  static constexpr int LPW = NL >= NW ? NL / NW : 1;
  static_assert(TILEB % 1024 == 0 && (NL % NW == 0 || NL < NW), "tile must split into 1 KiB loads");
  int wave;            // wave-uniform
  int lane;
  uint32_t lane_part;  // HOLD: one register for every load
  __device__ __forceinline__ TileLoader(int wave_, int lane_)
      : wave(__builtin_amdgcn_readfirstlane(wave_)), lane(lane_),
        lane_part(HOLD ? dma_lane_part<D>(lane_) : 0u) {}
  __device__ __forceinline__ void issue(uint32_t tile_lds, const bf16* A, int t0, int L) const {
    if (NL < NW && wave >= NL) return;
    uint32_t lp = lane_part;
    if (!HOLD) {
      int ln = lane;
      asm volatile("" : "+v"(ln));  // keep the offset from being hoisted out of the loop
      lp = dma_lane_part<D>(ln);
    }
    if constexpr (SPLIT)
      dma_tile_loads_split<D, BT, LPW, NT>(tile_lds, A, t0, L, wave * LPW, lp);
    else
      dma_tile_loads<D, BT, LPW, NT>(tile_lds, A, t0, L, wave * LPW, lp);
  }
};

// Scheduling hint for a run of NA MFMAs that take RA LDS reads each,
// followed by NB MFMAs that take RB reads each (one basic block, reads in
// the order of their use): the reads of the first LEAD MFMAs go first, then
// each MFMA is followed by the reads of the MFMA LEAD places later.  Keeps
// LDS latency off the MFMA chain without holding all operands at once.
template <int NA, int RA, int NB, int RB, int LEAD>
struct MfmaReadPipeline {
  static constexpr int reads_of(int m) { return m < NA ? RA : (m < NA + NB ? RB : 0); }
  template <int I>
  static __device__ __forceinline__ void step() {
    if constexpr (I < NA + NB) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      if constexpr (reads_of(I + LEAD) > 0)
        __builtin_amdgcn_sched_group_barrier(0x100, reads_of(I + LEAD), 0);  // its reads
      step<I + 1>();
    }
  }
  template <int I>
  static constexpr int lead_reads() {
    if constexpr (I < LEAD) return reads_of(I) + lead_reads<I + 1>();
    else return 0;
  }
  static __device__ __forceinline__ void apply() {
    __builtin_amdgcn_sched_group_barrier(0x100, lead_reads<0>(), 0);
    step<0>();
  }
};

// s_waitcnt vmcnt(N) with expcnt and lgkmcnt left at their maxima (gfx9
// encoding: vmcnt bits [3:0] and [15:14]).  Vector memory loads complete in
// issue order, so vmcnt(N) means all but the N most recent are done.
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// s_waitcnt vmcnt(0) (expcnt, lgkmcnt left at their maxima).  The builtin,
// unlike inline asm, tells the compiler that earlier global loads are done.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Per-lane byte offsets inside a swizzled [rows x D] bf16 tile:
//   row[ds]  16-byte read of row 32*k + l32, chunk 2*ds + hl (MFMA A/B rows);
//   tr[dd]   transpose read of the 4x16 block at rows 16*k + 4*hl + (lane%16)/4,
//            columns 32*dd + 16*((lane/16)%2) + 4*(lane%4);
//   trd      added to tr[dd] for the same block 8 rows further down.
// None depends on k (the swizzle only uses the low four row bits), so k goes
// into the instruction's immediate offset.  The +8-row partner differs by a
// lane constant: row 8 flips bit 1 of the swizzle, which moves the chunk by
// +-2 depending on bit 1 of (chunk ^ swizzle), a bit that no 32-column tile
// index dd touches.
template <int D>
struct LdsOffsets {
  int row[D / 16];
  int tr[D / 32];
  int trd;
  __device__ __forceinline__ explicit LdsOffsets(int lane) {
    constexpr int ROWB = D * 2;
    const int l32 = lane & 31, hl = lane >> 5;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) row[ds] = l32 * ROWB + (((2 * ds + hl) ^ swz<D>(l32)) << 4);
    const int r = 4 * hl + ((lane & 15) >> 2);
    const int c = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int dd = 0; dd < D / 32; ++dd)
      tr[dd] = r * ROWB + (((4 * dd + c) ^ swz<D>(r)) << 4) + 8 * (lane & 1);
    trd = 8 * ROWB + ((((c ^ swz<D>(r)) >> 1) & 1) ? -32 : 32);
  }
};

}  // namespace ra

#include "ra_launch.h"
