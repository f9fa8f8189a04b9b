// Decode-shaped forward step, bf16 inputs, fp32 accumulation, gfx950 MFMA.
//
// A few query rows (one decode step, or a short draft of Lq tokens) against
// one long key/value block: the same blockwise pass and associative fold as
// the forward ring step (Ring Attention keyword page, definition; darcstar
// commentary on the associative combine), for the "inference" use of the
// method (Ring Attention with Blockwise Transformers, abstract: training and
// inference).  The query rows come after every key of the block, so no key
// is masked.
//
// With so few rows the work is bound by streaming the key/value block from
// HBM, so the block's keys are split: workgroup (b, key/value head, split s)
// attends every query row of the head's group (G query heads x Lq rows, at
// most 64) to keys [s*k_chunk, min(Lk, (s+1)*k_chunk)) and writes a
// normalised partial (o, lse) for split s.  fold_kernel then folds the S
// split partials and the running accumulator (o_acc, lse_acc), in order,
// with the same combine as ring_attn_combine.
//
// Inside a workgroup, key tiles of 128 keys move global -> LDS with
// non-temporal direct-to-LDS copies (each byte is read once, so it streams
// past the L2) into two stages (swizzled rows, as in the forward kernels):
// the next tile is in flight while the current one is used, 64 KiB per
// compute unit.  Each of the four waves takes 32 keys of a tile, holds the
// query rows in registers (B operand of S^T = K Q^T, one or two blocks of 32
// rows), and keeps its own online softmax; the waves' partials are merged
// through LDS at the end.
#include <math.h>

#include <mutex>

#include "ra_common.h"
#include "ring_attn.h"

using namespace ra;

// Split partials of ring_attn_fwd_decode_noalloc: a device-resident array,
// one copy per GPU, that lives until the process ends.  Host code never uses
// the name below as an address (on the host it is only a stand-in symbol);
// ra_decode_scratch() looks up each device's own address once and hands
// that out.
static __device__ __align__(256) char scratch[RA_DECODE_SCRATCH_BYTES];

namespace {

constexpr float kRescaleThresh = 8.0f;  // log2 units

template <int D>
struct DecCfg {
  static constexpr int NW = 4;                  // waves; each takes 32 keys of a tile
  static constexpr int BT = NW * 32;            // keys per tile
  static constexpr int ROWB = D * 2;
  static constexpr int TILEB = BT * ROWB;       // one K (or V) tile
  static constexpr int STAGEB = 2 * TILEB;      // K then V
  static constexpr int NSTAGE = 2;
  static constexpr int PF = NSTAGE - 1;         // tiles issued ahead of the one in use
  static constexpr int SMEM = NSTAGE * STAGEB;
};

// Waits until at most `pending` (0 .. K) tiles of LPT copies each are still
// in flight for this wave (copies complete in issue order).
template <int LPT, int K>
__device__ __forceinline__ void wait_tiles_pending(int pending) {
  if constexpr (K == 0) {
    wait_vmem();
  } else {
    if (pending >= K)
      wait_vmem_n<K * LPT>();
    else
      wait_tiles_pending<LPT, K - 1>(pending);
  }
}

// RB: blocks of 32 query rows (rows = G * Lq <= 32 * RB).
template <int D, int RB>
__global__ __launch_bounds__(DecCfg<D>::NW * 64, 1) void decode_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ KV, float* __restrict__ Opart,
    float* __restrict__ LSEpart, int B, int H, int G, int Lq, int Lk, int k_chunk, int S,
    float c2) {
  using C = DecCfg<D>;
  constexpr int NW = C::NW, BT = C::BT, DS = D / 16, DD = D / 32;
  // the tile stages, later reused for the merge of the waves' partials
  constexpr int MERGEB = (2 * NW * RB * 32 + NW * RB * 32 * D) * 4;
  __shared__ __attribute__((aligned(1024))) char smem[C::SMEM > MERGEB ? C::SMEM : MERGEB];
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(lvoid*)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hl = lane >> 5;

  const int s = blockIdx.x % S;      // key split
  const int bkv = blockIdx.x / S;    // b * Hkv + key/value head
  const int Hkv = H / G;
  const int b = bkv / Hkv, kvh = bkv % Hkv;
  const int R = G * Lq;              // query rows of the group
  const int k0 = s * k_chunk, k1 = min(Lk, k0 + k_chunk);
  const int ntiles = (k1 - k0 + BT - 1) / BT;
  const bf16* Kp = KV + (size_t)bkv * Lk * D;
  const bf16* Vp = KV + ((size_t)B * Hkv + bkv) * Lk * D;

  // Row r of the group: query head kvh*G + r / Lq, query r % Lq.
  auto row_index = [&](int r) -> size_t {
    return ((size_t)b * H + kvh * G + r / Lq) * Lq + r % Lq;
  };
  bf16x8 qreg[RB][DS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = rb * 32 + l32;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
      qreg[rb][ds] = r < R ? *(const bf16x8*)(Q + row_index(r) * D + ds * 16 + hl * 8)
                           : bf16x8{};
  }

  // Wait for q here, with the builtin, before any direct-to-LDS copy is in
  // flight: the compiler does not see those copies, and a wait it placed for
  // q inside the loop would be vmcnt(0), draining the prefetched tiles too.
  wait_vmem();

  const LdsOffsets<D> off(lane);
  const TileLoader<D, BT, NW, true, true, true> loader(wave, lane);  // read once: non-temporal
  constexpr int LPT = 2 * decltype(loader)::LPW;  // copies per wave per tile (K and V)
  auto issue = [&](int t) __attribute__((always_inline)) {
    const uint32_t st = smem_lds + (t % C::NSTAGE) * C::STAGEB;
    loader.issue(st, Kp, k0 + t * BT, Lk);
    loader.issue(st + C::TILEB, Vp, k0 + t * BT, Lk);
  };

  f32x16 oacc[RB][DD];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int dd = 0; dd < DD; ++dd) oacc[rb][dd] = f32x16{};
  float m[RB], lsum[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) m[rb] = kNegBig, lsum[rb] = 0.f;

  // Tiles 0 .. PF-1 before the loop; iteration t issues tile t+PF into the
  // stage of tile t-1 (read in iteration t-1, before its barrier).  The wave
  // waits for its own copies of the next tile; the barrier makes the other
  // waves' copies visible too.
  constexpr int PF = C::PF;
  static_assert((PF - 1) * LPT < 64, "vmcnt range");
#pragma unroll
  for (int t = 0; t < PF; ++t)
    if (t < ntiles) issue(t);
  wait_tiles_pending<LPT, PF - 1>(min(ntiles, PF) - 1);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    if (t + PF < ntiles) issue(t + PF);
    const char* kt = smem + (t % C::NSTAGE) * C::STAGEB + wave * 32 * C::ROWB;
    const char* vt = kt + C::TILEB;
    const int kw0 = k0 + t * BT + wave * 32;  // this wave's first key
    // S^T = K Q^T for this wave's 32 keys and each block of 32 rows.
    f32x16 sc[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) sc[rb] = f32x16{};
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const bf16x8 a = *(const bf16x8*)(kt + off.row[ds]);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) sc[rb] = mfma32(a, qreg[rb][ds], sc[rb]);
    }
    // keys past the split's end (the ragged last tile) take no part
    if (__builtin_amdgcn_readfirstlane(kw0 + 32 > k1)) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kw0 + 8 * (r >> 2) + 4 * hl + (r & 3) >= k1) sc[rb][r] = -INFINITY;
    }
    // online softmax (log2 units; lazy rescale above a growth of 2^8)
    bf16x8 pb[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[rb][r]);
      mx = max_halves(mx) * c2;
      if (__builtin_amdgcn_ballot_w64(mx > m[rb] + kRescaleThresh)) {
        const float mnew = fmaxf(m[rb], mx);
        const float alpha = exp2_fast(m[rb] - mnew);
        m[rb] = mnew;
        lsum[rb] *= alpha;
#pragma unroll
        for (int dd = 0; dd < DD; ++dd) oacc[rb][dd] *= alpha;
      }
      f32x16 p;
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = exp2_fast(fmaf(sc[rb][r], c2, -m[rb]));
        rs += p[r];
      }
      lsum[rb] += rs;
      pb[rb][0] = to_bf16x8(p, 0);
      pb[rb][1] = to_bf16x8(p, 1);
    }
    // O^T += V^T P^T over this wave's 32 keys.
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const char* vb = vt + 16 * half * C::ROWB;
#pragma unroll
      for (int dd = 0; dd < DD; ++dd) {
        const bf16x4 lo = lds_read_tr((const bf16*)(vb + off.tr[dd]));
        const bf16x4 hi = lds_read_tr((const bf16*)(vb + off.tr[dd] + off.trd));
        const bf16x8 a = cat(lo, hi);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) oacc[rb][dd] = mfma32(a, pb[rb][half], oacc[rb][dd]);
      }
    }
    // Tile t+1 must have landed; tiles t+2 .. t+PF may stay in flight.
    wait_tiles_pending<LPT, PF - 1>(min(ntiles, t + PF + 1) - t - 2);
    __syncthreads();
  }

  // Merge the waves' partials through LDS (the tile buffers are free):
  // per wave and row its max (log2 units), sum and unnormalised output.
  float* cm = (float*)smem;                          // [NW][RB*32]
  float* cl = cm + NW * RB * 32;                     // [NW][RB*32]
  float* co = cl + NW * RB * 32;                     // [NW][RB*32][D]
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = rb * 32 + l32;
    const float lt = add_halves(lsum[rb]);
    if (hl == 0) {
      cm[wave * RB * 32 + r] = m[rb];
      cl[wave * RB * 32 + r] = lt;
    }
    float* orow = co + ((size_t)wave * RB * 32 + r) * D;
#pragma unroll
    for (int dd = 0; dd < DD; ++dd)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(f32x4*)(orow + dd * 32 + 8 * g + 4 * hl) =
            f32x4{oacc[rb][dd][4 * g], oacc[rb][dd][4 * g + 1], oacc[rb][dd][4 * g + 2],
                  oacc[rb][dd][4 * g + 3]};
  }
  __syncthreads();
  // D/4 threads per row, four columns each.
  constexpr int TPR = D / 4;
  for (int idx = tid; idx < R * TPR; idx += NW * 64) {
    const int r = idx / TPR, c = (idx % TPR) * 4;
    float mw[NW], M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      mw[w] = cm[w * RB * 32 + r];
      M = fmaxf(M, mw[w]);
    }
    float Ls = 0.f;
    f32x4 o = {};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float e = exp2_fast(mw[w] - M);
      Ls += e * cl[w * RB * 32 + r];
      o += e * *(const f32x4*)(co + ((size_t)w * RB * 32 + r) * D + c);
    }
    const size_t prow = (size_t)s * B * H * Lq + row_index(r);
    *(f32x4*)(Opart + prow * D + c) = o / Ls;
    if (c == 0) LSEpart[prow] = (M + log2f(Ls)) * kLn2;
  }
}

// (o_acc, lse_acc) <- (o_acc, lse_acc) (+) partial 0 (+) ... (+) partial S-1,
// the combine of ring_attn_combine extended to S + 1 terms: one thread per
// four columns of a row.
template <int D>
__global__ void fold_kernel(float* __restrict__ o_acc, float* __restrict__ lse_acc,
                            const float* __restrict__ Opart,
                            const float* __restrict__ LSEpart, int64_t rows, int S) {
  constexpr int TPR = D / 4;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = g / TPR;
  if (row >= rows) return;
  const int c = (int)(g % TPR) * 4;
  const float la = lse_acc[row];
  float mu = la;
  for (int s = 0; s < S; ++s) mu = fmaxf(mu, LSEpart[(int64_t)s * rows + row]);
  if (mu == -INFINITY) return;  // every term empty: unchanged
  float z = 0.f;
  f32x4 o = {};
  if (la != -INFINITY) {
    const float w = expf(la - mu);
    z += w;
    o += w * *(const f32x4*)(o_acc + row * D + c);
  }
  for (int s = 0; s < S; ++s) {
    const float ls = LSEpart[(int64_t)s * rows + row];
    if (ls == -INFINITY) continue;
    const float w = expf(ls - mu);
    z += w;
    o += w * *(const f32x4*)(Opart + ((int64_t)s * rows + row) * D + c);
  }
  *(f32x4*)(o_acc + row * D + c) = o / z;
  // The threads of one row lie in one wave and all load lse_acc[row] above,
  // before this store in program order.
  if (c == 0) lse_acc[row] = mu + logf(z);
}

template <int D, int RB>
hipError_t launch(const void* q, const void* kv, float* o_part, float* lse_part, int k_chunk,
                  int S, const ra_launch& a) {
  const int G = a.H / a.Hkv;
  const long long grid = (long long)a.B * a.Hkv * S;
  hipLaunchKernelGGL((decode_kernel<D, RB>), dim3((unsigned)grid), dim3(DecCfg<D>::NW * 64), 0,
                     a.stream, (const bf16*)q, (const bf16*)kv, o_part, lse_part, a.B, a.H, G,
                     a.Lq, a.Lk, k_chunk, S, a.scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t ra_launch_decode_split(const void* q, const void* kv, float* o_part, float* lse_part,
                                  int k_chunk, int splits, const ra_launch& a) {
  const int R = (a.H / a.Hkv) * a.Lq;
  if (R <= 0 || R > 64 || k_chunk < 1 || splits < 1) return hipErrorInvalidValue;
  if (a.D == 128)
    return R <= 32 ? launch<128, 1>(q, kv, o_part, lse_part, k_chunk, splits, a)
                   : launch<128, 2>(q, kv, o_part, lse_part, k_chunk, splits, a);
  if (a.D == 64)
    return R <= 32 ? launch<64, 1>(q, kv, o_part, lse_part, k_chunk, splits, a)
                   : launch<64, 2>(q, kv, o_part, lse_part, k_chunk, splits, a);
  return hipErrorInvalidValue;
}

hipError_t ra_launch_decode_fold(float* o_acc, float* lse_acc, const float* o_part,
                                 const float* lse_part, int64_t rows, int D, int splits,
                                 hipStream_t stream) {
  const int64_t threads = rows * (D / 4);
  const unsigned grid = (unsigned)((threads + 255) / 256);
  if (D == 128)
    hipLaunchKernelGGL((fold_kernel<128>), dim3(grid), dim3(256), 0, stream, o_acc, lse_acc,
                       o_part, lse_part, rows, splits);
  else if (D == 64)
    hipLaunchKernelGGL((fold_kernel<64>), dim3(grid), dim3(256), 0, stream, o_acc, lse_acc,
                       o_part, lse_part, rows, splits);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// Device address of this GPU's copy of `scratch`, looked up with
// hipGetSymbolAddress on the first call made while that device is current
// and kept for later calls.
hipError_t ra_decode_scratch(void** ptr, size_t* bytes) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = RA_DECODE_SCRATCH_BYTES;
  return hipSuccess;
}
