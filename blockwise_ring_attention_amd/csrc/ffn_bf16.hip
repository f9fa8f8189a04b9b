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
// eight waves of 128 x 64 (two per SIMD, whose MFMA streams cover each
// other's waits; the accumulators take 128 registers), K in steps of 64
// staged through two LDS stages of
// 2 x 256 x 64 bf16 filled by direct-to-LDS copies one step ahead.  Tiles
// are ordered in groups of eight row tiles per XCD so that the workgroups
// running together on one XCD share A and B tiles in its L2.  The epilogue
// stages the output tile in LDS and stores it with 16-byte writes.
#include <math.h>

#include "ra_common.h"

using namespace ra;

namespace {

constexpr int BM = 256, BN = 256;
constexpr int GROUP_M = 8;                   // row tiles per group in the tile order
// Output tile staged in LDS for the epilogue: 256 rows of 256 bf16, padded
// to 528 bytes so that the 8-byte writes of 32 consecutive rows spread over
// the banks and every 16-byte read stays aligned.
constexpr int OUT_ROWB = BN * 2 + 16;

// Staging of K steps of BK columns (32 or 64) in NSTAGE LDS stages, each an
// A tile and a B tile of 256 rows x BK bf16.
template <int BK, int NSTAGE>
struct GemmCfg {
  static constexpr int ROWB = BK * 2;               // bytes per staged row
  static constexpr int CPR = ROWB / 16;             // 16-byte chunks per row
  static constexpr int RPL = 1024 / ROWB;           // rows per 1 KiB copy
  static constexpr int LPW = BM / RPL / 8;          // copies per wave (8 waves) per tile
  static constexpr int TILEB = BM * ROWB;
  static constexpr int STAGEB = 2 * TILEB;          // A then B
  static constexpr int SMEM = NSTAGE * STAGEB > BM * OUT_ROWB ? NSTAGE * STAGEB : BM * OUT_ROWB;
  static constexpr int DS = BK / 16;                // 16-wide MFMA slices per step
};

// Physical 16-byte chunk of logical chunk c in staged row r is c ^ gswz(r):
// 64-column rows use the attention tiles' swizzle, 32-column rows (four
// chunks) XOR with bits 2-3 of the row.  Either way the 16-byte reads of 32
// consecutive rows at one logical chunk hit distinct banks.
template <int BK>
__device__ __forceinline__ int gswz(int r) {
  if constexpr (BK == 64)
    return swz<64>(r);
  else
    return (r >> 2) & 3;
}

// Copies rows [r0, r0 + 256) x columns [k0, k0 + BK) of a row-major
// [rows x ld] bf16 matrix into a swizzled LDS tile.  Copy j (1 KiB) fills
// tile rows RPL j .. RPL j + RPL - 1; lane l writes physical chunk l % CPR of
// row RPL j + l / CPR, so it fetches logical chunk
// (l % CPR) ^ gswz(RPL j + l / CPR) = (l % CPR) ^ gswz(l / CPR) ^ gswz(RPL j)
// (the swizzles are XOR-linear over these row bits; gswz(RPL j) is 2 (j & 1)
// for 64 columns and 0 for 32).  ld is a multiple of 64 elements, so that XOR
// never reaches the row part of the offset.  Rows at or past `rows` are
// clamped to rows - 1 (their products are never stored).  Wave w (of 8)
// issues copies LPW w .. LPW w + LPW - 1.
template <int BK, int NSTAGE>
struct StridedTileLoader {
  using C = GemmCfg<BK, NSTAGE>;
  uint32_t voff;    // lane byte offset for j with gswz(RPL j) = 0
  int lane_row;
  int lane_chunk;   // logical chunk for those j
  int wave;
  __device__ __forceinline__ StridedTileLoader(int wave_, int lane, int ld)
      : wave(__builtin_amdgcn_readfirstlane(wave_)) {
    lane_row = lane / C::CPR;
    lane_chunk = (lane % C::CPR) ^ gswz<BK>(lane_row);
    voff = (uint32_t)(lane_row * ld * 2 + lane_chunk * 16);
  }
  __device__ __forceinline__ void issue(uint32_t tile_lds, const bf16* src, int r0, int rows,
                                        int ld, int k0) const {
    if (r0 + BM <= rows) {  // whole tile in range: scalar row base per copy
#pragma unroll
      for (int i = 0; i < C::LPW; ++i) {
        const int j = wave * C::LPW + i;
        const uint32_t lds = __builtin_amdgcn_readfirstlane(tile_lds + (uint32_t)j * 1024);
        const uint32_t v[1] = {voff ^ (uint32_t)(gswz<BK>(C::RPL * j) << 4)};
        dma16_group<1>(uniform(src + (size_t)(r0 + C::RPL * j) * ld + k0), v, lds);
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::LPW; ++i) {
        const int j = wave * C::LPW + i;
        const uint32_t lds = __builtin_amdgcn_readfirstlane(tile_lds + (uint32_t)j * 1024);
        const int row = min(r0 + C::RPL * j + lane_row, rows - 1);
        const int chunk = lane_chunk ^ gswz<BK>(C::RPL * j);
        dma16(src + (size_t)row * ld + k0 + chunk * 8, lds);
      }
    }
  }
};

// Waits until at most `pending` (0 .. K) steps of LPT copies each are still
// in flight for this wave (copies complete in issue order).
template <int LPT, int K>
__device__ __forceinline__ void wait_steps_pending(int pending) {
  if constexpr (K == 0) {
    wait_vmem();
  } else {
    if (pending >= K)
      wait_vmem_n<K * LPT>();
    else
      wait_steps_pending<LPT, K - 1>(pending);
  }
}

// GELU(z) = z Phi(z) with Phi(z) = erfc(-z / sqrt 2) / 2.  erfc(u) for u >= 0
// from the rational approximation of Abramowitz and Stegun, Handbook of
// Mathematical Functions, formula 7.1.26 (|error of erf| <= 1.5e-7):
//   erfc(u) ~ (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-u^2),
//   t = 1 / (1 + p u).
// Phi(z) = 1 - erfc(|z|/sqrt 2)/2 for z >= 0 and erfc(|z|/sqrt 2)/2 for
// z < 0, so no 1 - erf cancellation is formed.  In fp32 with the hardware
// exp2 and reciprocal, |GELU error| < 5e-7 (checked against the exact form),
// well below the bf16 rounding of the hidden activation that follows.
__device__ __forceinline__ float normal_cdf(float z) {
  constexpr float p = 0.3275911f, a1 = 0.254829592f, a2 = -0.284496736f, a3 = 1.421413741f,
                  a4 = -1.453152027f, a5 = 1.061405429f;
  const float u = fabsf(z) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(p, u, 1.0f));
  const float poly = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, a5, a4), a3), a2), a1);
  const float ec = poly * exp2_fast(-u * u * kLog2e);
  return z >= 0.0f ? fmaf(-0.5f, ec, 1.0f) : 0.5f * ec;
}
__device__ __forceinline__ float gelu(float z) { return z * normal_cdf(z); }
// d GELU / dz = Phi(z) + z phi(z), phi the standard normal density.
__device__ __forceinline__ float gelu_grad(float z) {
  const float dens = 0.3989422804014327f * exp2_fast(-0.5f * z * z * kLog2e);
  return fmaf(z, dens, normal_cdf(z));
}

// C[m][n] = epi(sum_k A[m][k] B[n][k]) for m < M; N % 256 == 0, K % 64 == 0.
// Epilogues: bf16 store, GELU then bf16 store, or fp32 accumulate (C += AB^T).
enum { kEpiStore = 0, kEpiGelu = 1, kEpiAccF32 = 2 };

template <int EPI, int BK, int NSTAGE>
__global__ __launch_bounds__(512, 1) void gemm_tn_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ B, void* __restrict__ Cv, int M,
    int N, int K, int tiles_m, int tiles_n) {
  using G = GemmCfg<BK, NSTAGE>;
  constexpr int ROWB = G::ROWB, DS = G::DS, PF = NSTAGE - 1;
  constexpr int LPT = 2 * G::LPW;   // this wave's copies per step (A and B)
  static_assert((PF - 1) * LPT < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) char smem[G::SMEM];
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
  const int wm = wave >> 2, wn = wave & 3;   // the wave's 128 x 64 part

  const StridedTileLoader<BK, NSTAGE> loader(wave, lane, K);
  auto issue = [&](int kt) __attribute__((always_inline)) {
    const uint32_t st = smem_lds + (kt % NSTAGE) * G::STAGEB;
    loader.issue(st, A, m0, M, K, kt * BK);
    loader.issue(st + G::TILEB, B, n0, N, K, kt * BK);
  };
  // Per-lane offsets of the 16-byte MFMA operand reads: row l32 of a 32-row
  // block, logical chunk 2 ds + hl.
  int roff[DS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) roff[ds] = l32 * ROWB + (((2 * ds + hl) ^ gswz<BK>(l32)) << 4);

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  // Fragments of one 16-wide K slice: a[i] rows 32 i .. of the wave's 128
  // A rows, b[j] rows 32 j .. of its 64 B rows; two sets, so the reads of the
  // next slice run under the MFMAs of this one.
  bf16x8 fa[2][4], fb[2][2];
  auto read = [&](int set, int stage, int ds) __attribute__((always_inline)) {
    const char* As = smem + stage * G::STAGEB + wm * 128 * ROWB + roff[ds];
    const char* Bs = smem + stage * G::STAGEB + G::TILEB + wn * 64 * ROWB + roff[ds];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[set][i] = *(const bf16x8*)(As + i * 32 * ROWB);
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[set][j] = *(const bf16x8*)(Bs + j * 32 * ROWB);
  };
  // B fragments as the MFMA's first operand: lane l32 of acc[i][j] holds row
  // 32 i + l32 of the wave's part, register r its column 32 j + 8 (r / 4) +
  // 4 (lane / 32) + r % 4, so four consecutive registers are four adjacent
  // columns of one row.
  auto mfmas = [&](int set, int first, int count) __attribute__((always_inline)) {
#pragma unroll
    for (int q = first; q < first + count; ++q)
      acc[q >> 1][q & 1] = mfma32(fb[set][q & 1], fa[set][q >> 1], acc[q >> 1][q & 1]);
  };
  // One MFMA, then one LDS read, six times; then the remaining MFMAs.
  auto interleave8 = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 6; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  };

  // Steps 0 .. PF-1 before the loop; step kt issues step kt + PF into the
  // stage of step kt - 1 (last read in iteration kt - 1, before the barrier
  // in its last slice).  The copies go out together at the top of the step:
  // spreading them between the MFMAs measured slower.
  const int nk = K / BK;
#pragma unroll
  for (int s = 0; s < PF; ++s)
    if (s < nk) issue(s);
  wait_steps_pending<LPT, PF - 1>(min(nk, PF) - 1);
  __syncthreads();
  read(0, 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int stage = kt % NSTAGE;
    if (kt + PF < nk) issue(kt + PF);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ds = 0; ds + 1 < DS; ++ds) {
      read((ds + 1) & 1, stage, ds + 1);
      mfmas(ds & 1, 0, 8);
      interleave8();
      __builtin_amdgcn_sched_barrier(0);
    }
    // Last slice: half of its MFMAs, then (if a step follows) the wait for
    // the next step's copies, the barrier, and the next step's first-slice
    // reads under the other half.
    constexpr int last = (DS - 1) & 1;
    mfmas(last, 0, 4);
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 1 < nk) {
      // step kt+1 has landed; steps kt+2 .. kt+PF may stay in flight
      wait_steps_pending<LPT, PF - 1>(min(nk, kt + PF + 1) - kt - 2);
      __syncthreads();
      read(last ^ 1, (kt + 1) % NSTAGE, 0);
    }
    mfmas(last, 4, 4);
    __builtin_amdgcn_sched_barrier(0);
  }

  __syncthreads();  // every wave is done reading the last stage
  if constexpr (EPI == kEpiAccF32) {
    // fp32 accumulate, one 128-column half at a time: the waves owning that
    // half stage it in LDS (16-byte writes, four adjacent columns), then the
    // workgroup adds it to C row by row with 16-byte reads and writes.
    float* Cf = (float*)Cv;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if ((wn >> 1) == half) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                               acc[i][j][4 * g + 3]};
              const int row = wm * 128 + i * 32 + l32;
              const int col = (wn & 1) * 64 + j * 32 + 8 * g + 4 * hl;
              *(f32x4*)(smem + row * OUT_ROWB + col * 4) = v;
            }
      }
      __syncthreads();
#pragma unroll 4
      for (int it = 0; it < BM * 128 / 4 / 512; ++it) {
        const int id = it * 512 + tid;
        const int row = id >> 5, c = id & 31;   // 32 chunks of 4 columns per row
        const f32x4 v = *(const f32x4*)(smem + row * OUT_ROWB + c * 16);
        if (m0 + row < M) {
          f32x4* dst = (f32x4*)(Cf + (size_t)(m0 + row) * N + n0 + half * 128 + c * 4);
          *dst = *dst + v;
        }
      }
      __syncthreads();
    }
  } else {
    // Each wave writes its part (after the activation, as bf16) into
    // the LDS tile, four adjacent columns per 8-byte write; then the
    // workgroup stores the tile row by row, 16 bytes per lane.
    bf16* C = (bf16*)Cv;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float x = acc[i][j][4 * g + e];
            if constexpr (EPI == kEpiGelu) x = gelu(x);
            v[e] = (bf16)x;
          }
          const int row = wm * 128 + i * 32 + l32;
          const int col = wn * 64 + j * 32 + 8 * g + 4 * hl;
          *(bf16x4*)(smem + row * OUT_ROWB + col * 2) = v;
        }
    __syncthreads();
#pragma unroll 4
    for (int it = 0; it < BM * BN / 8 / 512; ++it) {
      const int id = it * 512 + tid;
      const int row = id >> 5, c = id & 31;   // 32 chunks of 8 columns per row
      const u32x4 v = *(const u32x4*)(smem + row * OUT_ROWB + c * 16);
      if (m0 + row < M) *(u32x4*)(C + (size_t)(m0 + row) * N + n0 + c * 8) = v;
    }
  }
}

// out[c][r] = in[r][c] for r < R and 0 for R <= r < Rpad: a [R x C] bf16
// matrix into a [C x Rpad] one (C and Rpad multiples of 64), one 64 x 64
// tile per workgroup through LDS, 16-byte global reads and writes.
__global__ __launch_bounds__(256) void transpose_pad_kernel(const bf16* __restrict__ in,
                                                            bf16* __restrict__ out, int R, int C,
                                                            int Rpad) {
  constexpr int TROW = 64 + 8;   // padded LDS row (elements)
  __shared__ bf16 tile[64 * TROW];
  const int tiles_c = C / 64;
  const int r0 = (blockIdx.x / tiles_c) * 64, c0 = (blockIdx.x % tiles_c) * 64;
  const int t = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int row = t / 8 + 32 * k, ch = t % 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r0 + row < R) v = *(const u32x4*)(in + (size_t)(r0 + row) * C + c0 + ch * 8);
    *(u32x4*)(tile + row * TROW + ch * 8) = v;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int orow = t / 8 + 32 * k, ch = t % 8;   // output row = input column
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tile[(ch * 8 + e) * TROW + orow];
    *(bf16x8*)(out + (size_t)(c0 + orow) * Rpad + r0 + ch * 8) = v;
  }
}

// The activation gradient and both transposes the weight gradients need, in
// one pass over a 64 x 64 tile of the [R x C] chunk: per element
// h = GELU(z) and g <- g * GELU'(z) (the gradient with respect to the
// pre-activation, written back in place, row-major, for the dx product),
// and the tile's g and h written transposed into Gt and Ht [C x Rpad], rows
// R .. Rpad-1 of those zero.  C and Rpad multiples of 64.
__global__ __launch_bounds__(256) void gelu_grad_transpose_kernel(
    const bf16* __restrict__ Z, bf16* __restrict__ G, bf16* __restrict__ Gt,
    bf16* __restrict__ Ht, int R, int C, int Rpad) {
  constexpr int TROW = 64 + 8;   // padded LDS row (elements)
  __shared__ bf16 tg[64 * TROW], th[64 * TROW];
  const int tiles_c = C / 64;
  const int r0 = (blockIdx.x / tiles_c) * 64, c0 = (blockIdx.x % tiles_c) * 64;
  const int t = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int row = t / 8 + 32 * k, ch = t % 8;
    bf16x8 dz = {}, h = {};
    if (r0 + row < R) {
      const size_t at = (size_t)(r0 + row) * C + c0 + ch * 8;
      const bf16x8 z = *(const bf16x8*)(Z + at);
      const bf16x8 g = *(const bf16x8*)(G + at);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float zf = (float)z[e];
        h[e] = (bf16)gelu(zf);
        dz[e] = (bf16)((float)g[e] * gelu_grad(zf));
      }
      *(bf16x8*)(G + at) = dz;
    }
    *(bf16x8*)(tg + row * TROW + ch * 8) = dz;
    *(bf16x8*)(th + row * TROW + ch * 8) = h;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int orow = t / 8 + 32 * k, ch = t % 8;   // output row = input column
    bf16x8 vg, vh;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      vg[e] = tg[(ch * 8 + e) * TROW + orow];
      vh[e] = th[(ch * 8 + e) * TROW + orow];
    }
    const size_t at = (size_t)(c0 + orow) * Rpad + r0 + ch * 8;
    *(bf16x8*)(Gt + at) = vg;
    *(bf16x8*)(Ht + at) = vh;
  }
}

constexpr int kBK = 64, kStages = 2;

template <int EPI>
hipError_t gemm_tn(const bf16* A, const bf16* B, void* C, int M, int N, int K,
                   hipStream_t stream) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = N / BN;
  hipLaunchKernelGGL((gemm_tn_kernel<EPI, kBK, kStages>), dim3((unsigned)(tiles_m * tiles_n)),
                     dim3(512), 0, stream, A, B, C, M, N, K, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t ra_launch_ffn_up(const void* x, const void* w1, void* hidden, int rows, int d_model,
                            int d_ff, hipStream_t stream) {
  if (rows < 1 || d_model % 64 != 0 || d_ff % BN != 0) return hipErrorInvalidValue;
  return gemm_tn<kEpiGelu>((const bf16*)x, (const bf16*)w1, hidden, rows, d_ff, d_model, stream);
}

hipError_t ra_launch_ffn_down(const void* hidden, const void* w2, void* out, int rows,
                              int d_model, int d_ff, hipStream_t stream) {
  if (rows < 1 || d_ff % 64 != 0 || d_model % BN != 0) return hipErrorInvalidValue;
  return gemm_tn<kEpiStore>((const bf16*)hidden, (const bf16*)w2, out, rows, d_model, d_ff,
                            stream);
}

hipError_t ra_launch_gemm_tn(const void* a, const void* b, void* c, int m, int n, int k,
                             int accumulate_f32, hipStream_t stream) {
  if (m < 1 || n % BN != 0 || k % 64 != 0 || k < 64) return hipErrorInvalidValue;
  return accumulate_f32
             ? gemm_tn<kEpiAccF32>((const bf16*)a, (const bf16*)b, c, m, n, k, stream)
             : gemm_tn<kEpiStore>((const bf16*)a, (const bf16*)b, c, m, n, k, stream);
}

hipError_t ra_launch_transpose_pad(const void* in, void* out, int rows, int cols, int rows_pad,
                                   hipStream_t stream) {
  if (rows < 0 || cols % 64 != 0 || rows_pad % 64 != 0 || rows_pad < rows)
    return hipErrorInvalidValue;
  const long long tiles = (long long)(rows_pad / 64) * (cols / 64);
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_pad_kernel, dim3((unsigned)tiles), dim3(256), 0, stream,
                     (const bf16*)in, (bf16*)out, rows, cols, rows_pad);
  return hipGetLastError();
}

hipError_t ra_launch_gelu_grad_transpose(const void* z, void* g, void* gt, void* ht, int rows,
                                         int cols, int rows_pad, hipStream_t stream) {
  if (rows < 0 || cols % 64 != 0 || rows_pad % 64 != 0 || rows_pad < rows)
    return hipErrorInvalidValue;
  const long long tiles = (long long)(rows_pad / 64) * (cols / 64);
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(gelu_grad_transpose_kernel, dim3((unsigned)tiles), dim3(256), 0, stream,
                     (const bf16*)z, (bf16*)g, (bf16*)gt, (bf16*)ht, rows, cols, rows_pad);
  return hipGetLastError();
}
