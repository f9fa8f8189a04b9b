// Blockwise feedforward of a ring member's rows, bf16 inputs, fp32
// accumulation, gfx950 MFMA.
//
// The method computes self-attention and the feedforward blockwise (Ring
// Attention with Blockwise Transformers, abstract): the feedforward is
// position-wise, so a member applies it to its own rows, a chunk of rows at a
// time, and the hidden activation never exceeds [chunk rows, d_ff].  The
// feedforward is the position-wise two-layer MLP
//     out = GELU(x W1^T) W2^T        (GELU(z) = z/2 (1 + erf(z / sqrt 2)))
// with W1 [d_ff, d_model] and W2 [d_model, d_ff] in the (out, in) layout, the
// hidden activation rounded to bf16 before the second product.
//
// Both products are C = A B^T with A [M x K] and B [N x K] row-major, so both
// MFMA operands are contiguous along K and come from 16-byte LDS reads of
// swizzled rows.  gemm_tn_kernel: one 256 x 256 output tile per workgroup,
// four waves of 128 x 128 (one wave per SIMD; the accumulators take 256
// registers), K in steps of 64 staged through two LDS stages of
// 2 x 256 x 64 bf16 filled by direct-to-LDS copies one step ahead.  Tiles
// are ordered in groups of four row tiles per XCD so that the workgroups
// running together on one XCD share A and B tiles in its L2.
#include <math.h>

#include "ra_common.h"

using namespace ra;

namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int ROWB = BK * 2;                 // bytes per staged row
constexpr int TILEB = BM * ROWB;             // one staged A (or B) tile, 32 KiB
constexpr int STAGEB = 2 * TILEB;            // A then B
constexpr int GROUP_M = 4;                   // row tiles per group in the tile order

// Copies rows [r0, r0 + 256) x columns [k0, k0 + 64) of a row-major
// [rows x ld] bf16 matrix into a swizzled [256 x 64] LDS tile: 16-byte chunk c
// of tile row r sits at physical chunk c ^ swz<64>(r).  Copy j (1 KiB) fills
// tile rows 8j .. 8j + 7; lane l writes physical chunk l & 7 of row
// 8j + (l >> 3), so it fetches logical chunk (l & 7) ^ swz<64>(8j + (l >> 3)).
// swz<64>(8j + r) = swz<64>(r) ^ 2 (j & 1) for r < 8, and ld is a multiple of
// 64 elements, so the lane offset for odd j is the even one with bit 5
// flipped.  Rows at or past `rows` are clamped to rows - 1 (their products
// are never stored).  Each wave issues copies j = 8 w .. 8 w + 7.
struct StridedTileLoader {
  uint32_t voff;    // lane byte offset for even j (row part + chunk)
  int lane_row;     // l >> 3
  int lane_chunk;   // logical chunk for even j
  int wave;
  __device__ __forceinline__ StridedTileLoader(int wave_, int lane, int ld)
      : wave(__builtin_amdgcn_readfirstlane(wave_)) {
    lane_row = lane >> 3;
    lane_chunk = (lane & 7) ^ swz<64>(lane_row);
    voff = (uint32_t)(lane_row * ld * 2 + lane_chunk * 16);
  }
  __device__ __forceinline__ void issue(uint32_t tile_lds, const bf16* src, int r0, int rows,
                                        int ld, int k0) const {
    if (r0 + 256 <= rows) {  // whole tile in range: scalar row base per copy
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = wave * 8 + i;
        const uint32_t lds = __builtin_amdgcn_readfirstlane(tile_lds + (uint32_t)j * 1024);
        const uint32_t v[1] = {voff ^ (uint32_t)((j & 1) << 5)};
        dma16_group<1>(uniform(src + (size_t)(r0 + 8 * j) * ld + k0), v, lds);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = wave * 8 + i;
        const uint32_t lds = __builtin_amdgcn_readfirstlane(tile_lds + (uint32_t)j * 1024);
        const int row = min(r0 + 8 * j + lane_row, rows - 1);
        const int chunk = lane_chunk ^ ((j & 1) << 1);
        dma16(src + (size_t)row * ld + k0 + chunk * 8, lds);
      }
    }
  }
};

__device__ __forceinline__ float gelu(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}

// C[m][n] = epi(sum_k A[m][k] B[n][k]) for m < M; N % 256 == 0, K % 64 == 0.
template <bool GELU>
__global__ __launch_bounds__(256, 1) void gemm_tn_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ B, bf16* __restrict__ C, int M,
    int N, int K, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGEB];
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(lvoid*)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hl = lane >> 5;

  // Tile order: XCD x runs a contiguous range of tile ids; within it, groups
  // of GROUP_M row tiles sweep the column tiles.
  const int ntile = tiles_m * tiles_n;
  const int t = xcd_remap(blockIdx.x, ntile);
  const int per_group = GROUP_M * tiles_n;
  const int first_m = (t / per_group) * GROUP_M;
  const int gm = min(tiles_m - first_m, GROUP_M);
  const int tm = first_m + (t % per_group) % gm;
  const int tn = (t % per_group) / gm;
  const int m0 = tm * BM, n0 = tn * BN;
  const int wm = wave >> 1, wn = wave & 1;   // the wave's 128 x 128 quadrant

  const StridedTileLoader loader(wave, lane, K);
  auto issue = [&](int kt) __attribute__((always_inline)) {
    const uint32_t st = smem_lds + (kt & 1) * STAGEB;
    loader.issue(st, A, m0, M, K, kt * BK);
    loader.issue(st + TILEB, B, n0, N, K, kt * BK);
  };
  const LdsOffsets<64> off(lane);

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  // Fragments of one 16-wide K slice: a[i] rows 32 i .. of the wave's A
  // quadrant, b[j] rows 32 j .. of its B quadrant; two sets, so the reads of
  // slice ds + 1 run under the MFMAs of slice ds.
  bf16x8 fa[2][4], fb[2][4];
  auto read = [&](int set, int stage, int ds) __attribute__((always_inline)) {
    const char* As = smem + stage * STAGEB + wm * 128 * ROWB + off.row[ds];
    const char* Bs = smem + stage * STAGEB + TILEB + wn * 128 * ROWB + off.row[ds];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[set][i] = *(const bf16x8*)(As + i * 32 * ROWB);
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[set][j] = *(const bf16x8*)(Bs + j * 32 * ROWB);
  };
  auto mfmas = [&](int set, int first, int count) __attribute__((always_inline)) {
#pragma unroll
    for (int q = first; q < first + count; ++q)
      acc[q >> 2][q & 3] = mfma32(fa[set][q >> 2], fb[set][q & 3], acc[q >> 2][q & 3]);
  };
  // One MFMA, then one LDS read, eight times; then the remaining MFMAs.
  auto interleave8 = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  };

  const int nk = K / BK;
  issue(0);
  wait_vmem();
  __syncthreads();
  read(0, 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int stage = kt & 1;
    // Stage (kt+1)&1 was last read in iteration kt-1, before the barrier in
    // its last slice; the reads since then are of stage kt&1.
    if (kt + 1 < nk) issue(kt + 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ds = 0; ds < 3; ++ds) {
      read((ds + 1) & 1, stage, ds + 1);
      mfmas(ds & 1, 0, 16);
      interleave8();
      __builtin_amdgcn_sched_barrier(0);
    }
    // Slice 3: half of its MFMAs, then (if a step follows) the wait for the
    // next stage's copies, the barrier, and the next step's slice-0 reads
    // under the other half.
    mfmas(1, 0, 8);
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 1 < nk) {
      wait_vmem();  // this wave's copies of step kt+1 have landed
      __syncthreads();
      read(0, stage ^ 1, 0);
    }
    mfmas(1, 8, 8);
    __builtin_amdgcn_sched_barrier(0);
  }

  // Lane l32 holds column n of 16 rows per accumulator: each store writes 32
  // consecutive columns of one row.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn * 128 + j * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
        float v = acc[i][j][r];
        if constexpr (GELU) v = gelu(v);
        if (m < M) C[(size_t)m * N + n] = (bf16)v;
      }
    }
}

hipError_t gemm_tn(const bf16* A, const bf16* B, bf16* C, int M, int N, int K, bool gelu_epi,
                   hipStream_t stream) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = N / BN;
  const dim3 grid((unsigned)(tiles_m * tiles_n)), block(256);
  if (gelu_epi)
    hipLaunchKernelGGL(gemm_tn_kernel<true>, grid, block, 0, stream, A, B, C, M, N, K, tiles_m,
                       tiles_n);
  else
    hipLaunchKernelGGL(gemm_tn_kernel<false>, grid, block, 0, stream, A, B, C, M, N, K, tiles_m,
                       tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t ra_launch_ffn_up(const void* x, const void* w1, void* hidden, int rows, int d_model,
                            int d_ff, hipStream_t stream) {
  if (rows < 1 || d_model % BK != 0 || d_ff % BN != 0) return hipErrorInvalidValue;
  return gemm_tn((const bf16*)x, (const bf16*)w1, (bf16*)hidden, rows, d_ff, d_model, true,
                 stream);
}

hipError_t ra_launch_ffn_down(const void* hidden, const void* w2, void* out, int rows,
                              int d_model, int d_ff, hipStream_t stream) {
  if (rows < 1 || d_ff % BK != 0 || d_model % BN != 0) return hipErrorInvalidValue;
  return gemm_tn((const bf16*)hidden, (const bf16*)w2, (bf16*)out, rows, d_model, d_ff, false,
                 stream);
}
