// Backward ring step, bf16 inputs, fp32 accumulation, gfx950 MFMA.
//
// The gradient is that of sum(dO * O) over the member's rows, with O the
// exact attention of the forward share.  For one key/value block, with
// P = exp(scale * Q K^T - lse) recomputed from the saved final LSE (the
// memory-efficient method never keeps P; Blockwise RingAttention keyword
// page, definition) and delta_i = <dO_i, O_i>:
//     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - delta),
//     dQ = scale * dS K,  dK = scale * dS^T Q.
// Two kernels and no atomics, so every result is deterministic:
//   * dq_kernel (query-major, the forward's structure): a wave keeps 32
//     queries and their dO rows in registers and sweeps the block's key /
//     value tiles through LDS, forming S^T = K Q^T and dP^T = V dO^T (16-byte
//     LDS reads), dS^T in registers, and dQ^T += K^T dS^T (K^T by LDS
//     transpose reads).  Eight waves ping-pong as in the forward (group
//     B's MFMA phase at the higher wave priority).
//   * dkv_kernel (key-major): a wave keeps 32 keys and their values in
//     registers and sweeps the query tiles (Q, dO, lse, delta) through LDS,
//     forming S = Q K^T and dP = dO V^T, then dV += P^T dO and dK += dS^T Q
//     with dO^T and Q^T by LDS transpose reads.  Four waves, one per SIMD;
//     each wave overlaps the products of tile t with the scores of t+1.
// Tiles move global -> LDS with direct-to-LDS copies into XOR-swizzled rows
// (see ra_common.h); each kernel keeps two tiles of prefetch in flight.
// The causal diagonal block masks key j > query i; past blocks are dense.
#include <math.h>

#include "ra_common.h"

using namespace ra;

namespace {

template <int D, int BT, int NW>
struct TileCfg {
  static constexpr int NT = NW * 64;
  static constexpr int ROWB = D * 2;
  static constexpr int TILEB = BT * ROWB;      // one [BT x D] bf16 tile
  static constexpr int STAGEB = 2 * TILEB;     // two tiles per stage
  static constexpr int NSTAGE = 4;
  static constexpr int LPW = STAGEB / (NW * 1024);
  static_assert(STAGEB % (NW * 1024) == 0 && LPW >= 1, "tile must split into 1 KiB loads");
  static_assert(TILEB % 1024 == 0, "a load must not straddle the two tiles");
};

// Wave priority of group B's MFMA phase in the dQ ping-pong, above group A's
// (1) and the gradient phases (0): B opens each tile with its MFMA phase, and
// at equal priority A's MFMA phase, starting when its shorter gradient phase
// ends, would take the MFMA pipe from B's unfinished one.
constexpr int kPrioB = 2;

// ---------------------------------------------------------------- dQ ------
template <int D, int BN, int NW>
__global__ __launch_bounds__(NW * 64, 1) void dq_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ KV,
    const bf16* __restrict__ dO, const float* __restrict__ LSE,
    const float* __restrict__ Delta, float* __restrict__ dQacc, int BH, int H, int G, int Lq,
    int Lk, int n_qt, int diag, float c2, float scale) {
  using C = TileCfg<D, BN, NW>;
  constexpr int BM = NW * 32;
  constexpr int KK = BN / 32, DS = D / 16, DD = D / 32;
  // Ring of NR slots, each a K tile followed by its V tile.  Iteration t
  // reads K tiles t-1 .. t+1 and V tiles t, t+1, has tiles t+2 in flight and
  // issues t+3.  A V tile sits a fixed TILEB after its K tile, so both
  // are addressed from one register plus an immediate offset.
  constexpr int NR = 5;
  __shared__ __attribute__((aligned(1024))) char smem[NR * 2 * C::TILEB];
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(lvoid*)smem;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const bool group_b = NW == 8 && wave >= 4;
  const int rblk = NW == 8 ? 2 * (wave & 3) + (wave >> 2) : wave;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / n_qt;
  int qt = tile % n_qt;
  if (diag) qt = n_qt - 1 - qt;
  const int q0 = qt * BM;
  const int qw0 = q0 + rblk * 32;
  const int qi = qw0 + l32;

  // Groups of G query heads share one key/value head.
  const int kvbh = (bh / H) * (H / G) + (bh % H) / G;
  const bf16* Qp = Q + (size_t)bh * Lq * D;
  const bf16* dOp = dO + (size_t)bh * Lq * D;
  const bf16* Kp = KV + (size_t)kvbh * Lk * D;
  const bf16* Vp = KV + ((size_t)(BH / G) + kvbh) * Lk * D;

  // diag == 2 (no skipping): every tile, the ones above the diagonal fully masked
  const int kend = diag == 1 ? min(Lk, q0 + BM) : Lk;
  const int ntiles = (kend + BN - 1) / BN;
  const int qw_last = min(qw0 + 31, Lq - 1);
  int ntw = 0;
  if (qw0 < Lq) ntw = diag == 1 ? min(ntiles, qw_last / BN + 1) : ntiles;

  const LdsOffsets<D> off(lane);
  using Loader = TileLoader<D, BN, NW, false>;
  const Loader loader(wave, lane);
  auto issue_k = [&](int t) __attribute__((always_inline)) {
    loader.issue(smem_lds + (t % NR) * 2 * C::TILEB, Kp, t * BN, Lk);
  };
  auto issue_v = [&](int t) __attribute__((always_inline)) {
    loader.issue(smem_lds + (t % NR) * 2 * C::TILEB + C::TILEB, Vp, t * BN, Lk);
  };
  // Iteration 0 needs K and V tiles 0 and 1 (group A's scores of tile 1);
  // tiles 2 may stay in flight until its end.
  for (int t = 0; t < 2; ++t)
    if (t < ntiles) {
      issue_k(t);
      issue_v(t);
    }

  bf16x8 qreg[DS], doreg[DS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) {
    qreg[ds] = qi < Lq ? *(const bf16x8*)(Qp + (size_t)qi * D + ds * 16 + hl * 8) : bf16x8{};
    doreg[ds] = qi < Lq ? *(const bf16x8*)(dOp + (size_t)qi * D + ds * 16 + hl * 8) : bf16x8{};
  }
  // A row that saw no key (lse = -inf) or lies past the end gets an
  // exponent offset of +inf, so its probabilities are exactly zero.
  const float lse_raw = qi < Lq ? LSE[(size_t)bh * Lq + qi] : -INFINITY;
  const float neg_lse2 = lse_raw == -INFINITY ? -INFINITY : -lse_raw * kLog2e;
  const float delta = qi < Lq ? Delta[(size_t)bh * Lq + qi] : 0.f;

  f32x16 dq[DD];
#pragma unroll
  for (int dd = 0; dd < DD; ++dd) dq[dd] = f32x16{};
  f32x16 s[KK], dp[KK];
  bf16x8 pb[KK][2];

  wait_vmem();
  if (ntiles > 2) {
    issue_k(2);
    issue_v(2);
  }
  __syncthreads();

  auto k_of = [&](int t) __attribute__((always_inline)) -> const char* {
    return smem + (t % NR) * 2 * C::TILEB;
  };
  auto v_of = [&](int t) __attribute__((always_inline)) -> const char* {
    return smem + (t % NR) * 2 * C::TILEB + C::TILEB;
  };
  auto scores = [&](const char* kt, const char* vt) __attribute__((always_inline)) {  // S^T, dP^T
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      s[kk] = f32x16{};
      dp[kk] = f32x16{};
    }
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int ro = kk * 32 * C::ROWB + off.row[ds];
        s[kk] = mfma32(*(const bf16x8*)(kt + ro), qreg[ds], s[kk]);
        dp[kk] = mfma32(*(const bf16x8*)(vt + ro), doreg[ds], dp[kk]);
      }
  };
  auto grad = [&](int t) __attribute__((always_inline)) {  // dS^T -> pb
    const int kt0 = t * BN;
    if (__builtin_amdgcn_readfirstlane((kt0 + BN > Lk) || (diag && kt0 + BN - 1 > qw0))) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kj = kt0 + kk * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (kj >= Lk || (diag && kj > qi)) s[kk][r] = -INFINITY;
        }
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      f32x16 g;  // not written back into s: s is dead until the next scores
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2_fast(fmaf(s[kk][r], c2, neg_lse2));
        g[r] = p * (dp[kk][r] - delta);
      }
      pb[kk][0] = to_bf16x8(g, 0);
      pb[kk][1] = to_bf16x8(g, 1);
    }
  };
  auto value = [&](const char* kt) __attribute__((always_inline)) {  // dQ^T += K^T dS^T
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const char* kb = kt + (kk * 32 + 16 * half) * C::ROWB;
#pragma unroll
        for (int dd = 0; dd < DD; ++dd) {
          const bf16x4 lo = lds_read_tr((const bf16*)(kb + off.tr[dd]));
          const bf16x4 hi = lds_read_tr((const bf16*)(kb + off.tr[dd] + off.trd));
          dq[dd] = mfma32(cat(lo, hi), pb[kk][half], dq[dd]);
        }
      }
  };

  // value: KK*2*DD MFMAs with two transpose reads each; scores: DS*KK*2
  // MFMAs with one 16-byte read each.
  using Pipe = MfmaReadPipeline<KK * 2 * DD, 2, DS * KK * 2, 1, 4>;
  if (!group_b && ntw > 0) scores(k_of(0), v_of(0));
  for (int t = 0; t < ntiles; ++t) {
    // Slot (t+3)%5 last served iteration t-1 (K tile t-2, group B's value;
    // its V tile was last read in iteration t-3).
    if (t + 3 < ntiles) {
      issue_k(t + 3);
      issue_v(t + 3);
    }
    if (!group_b) {
      if (t < ntw) {
        grad(t);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
        value(k_of(t));
        // Unconditional: past the wave's last tile the scores are unused, and
        // a branch here would keep the previous tile's registers alive.
        scores(k_of(t + 1), v_of(t + 1));
        Pipe::apply();
        __builtin_amdgcn_s_setprio(0);
      }
    } else {
      if (t >= 1 && t - 1 < ntw) {
        __builtin_amdgcn_s_setprio(kPrioB);
        value(k_of(t - 1));
        scores(k_of(t), v_of(t));
        Pipe::apply();
        __builtin_amdgcn_s_setprio(0);
      } else if (t == 0 && ntw > 0) {
        __builtin_amdgcn_s_setprio(kPrioB);
        scores(k_of(0), v_of(0));
        __builtin_amdgcn_s_setprio(0);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (t < ntw) grad(t);
    }
    // Iteration t+1 reads K and V tile t+2 (issued in iteration t-1); this
    // iteration's loads may stay in flight.
    if (t + 3 < ntiles)
      wait_vmem_n<2 * Loader::LPW>();
    else
      wait_vmem();
    __syncthreads();
  }
  // Group B still owes the value product of its last tile; no load touched
  // that K slot after the loop.
  if (group_b && ntw == ntiles && ntw > 0) value(k_of(ntw - 1));

  if (qi < Lq) {
    float* row = dQacc + ((size_t)bh * Lq + qi) * D;
    f32x4 old[DD][4];  // all loads first, then the stores
#pragma unroll
    for (int dd = 0; dd < DD; ++dd)
#pragma unroll
      for (int g = 0; g < 4; ++g) old[dd][g] = *(const f32x4*)(row + dd * 32 + 8 * g + 4 * hl);
#pragma unroll
    for (int dd = 0; dd < DD; ++dd)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 v = {dq[dd][4 * g], dq[dd][4 * g + 1], dq[dd][4 * g + 2], dq[dd][4 * g + 3]};
        *(f32x4*)(row + dd * 32 + 8 * g + 4 * hl) = old[dd][g] + v * scale;
      }
  }
}

// --------------------------------------------------------------- dK, dV ---
// Key-major.  A wave owns 32 keys (K, V rows in registers) and walks the
// query tiles of its block in 32-query sub-tiles n = 0, 1, 2, ... (two per
// 64-query LDS tile).  Per sub-tile:
//     scores(n):   S = Q K^T, dP = dO V^T             (16 MFMAs, row reads)
//     grad(n):     P = exp2(S*c2 - lse*log2e), dS = P (dP - delta)   (VALU)
//     products(n): dV += P^T dO, dK += dS^T Q         (16 MFMAs, transpose reads)
// With one wave per SIMD the only overlap is within the wave, so the work is
// software-pipelined: step n issues scores(n), then products(n-1) with the
// VALU work of grad(n) interleaved between its MFMAs.  P and dS alternate
// between two register sets (grad(n) writes one while products(n-1) reads the
// other).
//
// Memory pipeline: four LDS stages of (Q tile, dO tile).  Iteration t (steps
// 2t, 2t+1) reads stages t-1 (products(2t-1)) and t, copies tile t+2 into
// the slot of tile t-2, and at its end waits for tile t+1 only.  Each wave
// keeps a private copy of the tile's lse / delta rows (two 4-byte
// direct-to-LDS copies, issued for tile t+3) and converts it in place one
// iteration before the tile is used, so no extra barrier is needed.  Where
// every tile ahead is full, the copies and the conversion are placed between
// the MFMAs of the steps instead of in a burst after the barrier.
template <int D, int BQ, int NW>
__global__ __launch_bounds__(NW * 64, 1) void dkv_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ KV,
    const bf16* __restrict__ dO, const float* __restrict__ LSE,
    const float* __restrict__ Delta, float* __restrict__ dKV, float* __restrict__ WS, int BH, int H,
    int G, int qj, int ws_store, int Lq, int Lk, int n_kt, int diag, float c2, float scale) {
  using C = TileCfg<D, BQ, NW>;
  constexpr int BK = NW * 32;  // keys per workgroup
  constexpr int DS = D / 16, DD = D / 32;
  static_assert(BQ == 64, "two 32-query sub-tiles per LDS tile");
  __shared__ __attribute__((aligned(1024))) char smem[C::NSTAGE * C::STAGEB];
  // Per stage and wave: row 0 lse (converted in place to -lse*log2e), row 1 delta.
  __shared__ __attribute__((aligned(1024))) float s_ld[C::NSTAGE][NW][2][BQ];
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(lvoid*)smem;
  const uint32_t sld_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) float*)&s_ld[0][0][0][0];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: loop bounds derive from it
  const int l32 = lane & 31, hl = lane >> 5;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  // This workgroup's split sp, key/value head and key tile.  A launch handles
  // query heads qj .. qj + nsplit - 1 of every group, split sp taking member
  // qj + sp; split 0 adds into dKV, split sp > 0 into its own copy of dKV in
  // WS (stored rather than added when ws_store is set).  Consecutive
  // workgroups (one XCD) share the split and head, so they stream the same
  // query rows.
  const int per_split = (BH / G) * n_kt;
  const int sp = tile / per_split;
  const int kvbh = (tile % per_split) / n_kt;
  const int bh = (kvbh / (H / G)) * H + (kvbh % (H / G)) * G + qj + sp;
  const int k0 = (tile % n_kt) * BK;  // small k0 first: the most causal work
  const int kw0 = k0 + wave * 32;
  const int kj = kw0 + l32;

  const bf16* Qp = Q + (size_t)bh * Lq * D;
  const bf16* dOp = dO + (size_t)bh * Lq * D;
  const bf16* Kp = KV + (size_t)kvbh * Lk * D;
  const bf16* Vp = KV + ((size_t)(BH / G) + kvbh) * Lk * D;
  const float* Lp = LSE + (size_t)bh * Lq;
  const float* Dp = Delta + (size_t)bh * Lq;

  // Under the causal mask only queries at or after the first key matter.
  // (diag == 2, no skipping: every query tile, the earlier ones fully masked)
  const int qstart = diag == 1 ? (k0 / BQ) * BQ : 0;
  const int ntiles = qstart < Lq ? (Lq - qstart + BQ - 1) / BQ : 0;
  const int kw_last = min(kw0 + 31, Lk - 1);
  // This wave's active tiles are a suffix [ft, ntiles): query tiles that
  // end before its first key contribute nothing.
  int ft = diag == 1 ? max(0, (kw0 - qstart) / BQ) : 0;
  if (kw0 >= Lk) ft = ntiles;

  const LdsOffsets<D> off(lane);
  using Loader = TileLoader<D, BQ, NW>;
  const Loader loader(wave, lane);
  // Per iteration t each wave issues VPT copies: LPW of Q and LPW of dO for
  // tile t+2, and its own lse and delta rows for tile t+3 (they are converted
  // an iteration before the tile's stage is read).  Copy k < 2 LPW is a Q / dO
  // copy, 2 LPW and 2 LPW + 1 the lse / delta rows; vmcnt counts them.
  constexpr int LPW = Loader::LPW;
  constexpr int VPT = 2 * LPW + 2;
  auto issue_copy = [&](int t, int k) __attribute__((always_inline)) {
    if (k < 2 * LPW) {
      const int tt = t + 2;
      const uint32_t base = smem_lds + (tt % C::NSTAGE) * C::STAGEB + (k < LPW ? 0 : C::TILEB);
      dma_tile_loads_split<D, BQ, 1>(base, k < LPW ? Qp : dOp, qstart + tt * BQ, Lq,
                                     wave * LPW + k % LPW, loader.lane_part);
    } else {
      const int tt = t + 3;
      const int q = min(qstart + tt * BQ + lane, Lq - 1);
      const uint32_t row = sld_lds + (uint32_t)(((tt % C::NSTAGE) * NW + wave) * 2 * BQ * 4);
      if (k == 2 * LPW)
        dma4(Lp + q, row);
      else
        dma4(Dp + q, row + BQ * 4);
    }
  };
  // Copies of iteration t that exist: Q / dO while t + 2 < ntiles, lse /
  // delta while t + 3 < ntiles.
  auto copy_live = [&](int t, int k) __attribute__((always_inline)) -> bool {
    return k < 2 * LPW ? t + 2 < ntiles : t + 3 < ntiles;
  };
  // The same copy when the caller knows it exists and its tile has no rows
  // past the end: no test, no branch (placed between MFMAs).
  auto issue_copy_full = [&](int t, int k) __attribute__((always_inline)) {
    if (k < 2 * LPW) {
      const int tt = t + 2;
      const uint32_t base = smem_lds + (tt % C::NSTAGE) * C::STAGEB + (k < LPW ? 0 : C::TILEB);
      const int j = wave * LPW + k % LPW;
      const uint32_t voff[1] = {(loader.lane_part ^ dma_xor<D>(j)) + (uint32_t)j * 1024};
      dma16_group<1>(uniform((k < LPW ? Qp : dOp) + (size_t)(qstart + tt * BQ) * D), voff,
                     base + (uint32_t)j * 1024);
    } else {
      issue_copy(t, k);  // lse / delta rows: clamped, branch-free already
    }
  };
  // Tiles with no rows past the end of the block.
  const int nfull = qstart < Lq ? (Lq - qstart) / BQ : 0;
  // In-place conversion of this wave's copy for tile t (one lse and one
  // delta per lane): lse -> -lse*log2e, where -inf (a row that saw no key)
  // and rows past the end give P = 0; delta -> -delta, 0 past the end.
  float ld_l = 0.f, ld_d = 0.f;
  auto convert_read = [&](int t) __attribute__((always_inline)) {
    const float* row = &s_ld[t % C::NSTAGE][wave][0][0];
    ld_l = row[lane];
    ld_d = row[BQ + lane];
  };
  auto convert_write = [&](int t) __attribute__((always_inline)) {
    float* row = &s_ld[t % C::NSTAGE][wave][0][0];
    const bool valid = qstart + t * BQ + lane < Lq;
    row[lane] = (!valid || ld_l == -INFINITY) ? -INFINITY : -ld_l * kLog2e;
    row[BQ + lane] = valid ? -ld_d : 0.f;
  };

  // Prologue: Q / dO of tiles 0, 1 and lse / delta of tiles 0, 1, 2 (the
  // copies iterations -2 and -1 would have issued).
  for (int k = 0; k < VPT; ++k) {
    if (k < 2 * LPW) {
      if (copy_live(-2, k)) issue_copy(-2, k);
      if (copy_live(-1, k)) issue_copy(-1, k);
    } else {
      if (copy_live(-3, k)) issue_copy(-3, k);
      if (copy_live(-2, k)) issue_copy(-2, k);
      if (copy_live(-1, k)) issue_copy(-1, k);
    }
  }

  bf16x8 kreg[DS], vreg[DS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) {
    kreg[ds] = kj < Lk ? *(const bf16x8*)(Kp + (size_t)kj * D + ds * 16 + hl * 8) : bf16x8{};
    vreg[ds] = kj < Lk ? *(const bf16x8*)(Vp + (size_t)kj * D + ds * 16 + hl * 8) : bf16x8{};
  }
  f32x16 dk[DD], dv[DD];
#pragma unroll
  for (int dd = 0; dd < DD; ++dd) {
    dk[dd] = f32x16{};
    dv[dd] = f32x16{};
  }
  f32x16 s;                   // S of the newest scored sub-tile
  bf16x8 pbf[2][2], dsbf[2][2];  // P and dS of two sub-tiles ([set][16-query half])

  wait_vmem();
  __syncthreads();
  if (ntiles > 0) {
    convert_read(0);
    convert_write(0);
  }

  auto stage_of = [&](int t) __attribute__((always_inline)) -> const char* {
    return smem + (t % C::NSTAGE) * C::STAGEB;
  };
  // Operands.  Scores MFMA m of sub-tile (t, qs): m < DS accumulates S over
  // head-dim slice m (Q rows), DS <= m < 2 DS accumulates dP - delta over
  // slice m - DS (dO rows, starting from -delta); 16-byte row reads.  Product MFMA i: i = 2*(DD*p + dd) + w, p
  // the 16-query half, w = 0 the dO^T operand of dV[dd], w = 1 the Q^T
  // operand of dK[dd]; transpose reads.
  auto score_operand = [&](int t, int qs, int m) __attribute__((always_inline)) -> bf16x8 {
    const char* b = stage_of(t) + qs * 32 * C::ROWB + (m >= DS ? C::TILEB : 0);
    return *(const bf16x8*)(b + off.row[m % DS]);
  };
  auto prod_operand = [&](int t, int qs, int i) __attribute__((always_inline)) -> bf16x8 {
    const int p = i / (2 * DD), dd = (i / 2) % DD, w = i & 1;
    const char* b = stage_of(t) + (qs * 32 + 16 * p) * C::ROWB + (w == 0 ? C::TILEB : 0);
    return cat(lds_read_tr((const bf16*)(b + off.tr[dd])),
               lds_read_tr((const bf16*)(b + off.tr[dd] + off.trd)));
  };
  constexpr int NS = 2 * DS, NP = 4 * DD, LEAD = 4;
  constexpr int EPC = 16 / NP;  // gradient elements per product MFMA
  static_assert(16 % NP == 0, "gradient chunking");
  // -lse*log2e (nl) and -delta (ndl) of the 16 query rows a lane holds, one
  // set per step of an iteration.  ndl[qs] is also step qs's dP accumulator:
  // the dP MFMAs start from -delta in place, and the next rows are loaded
  // into the other set.
  f32x4 nl[2][4];
  f32x16 ndl[2];
  auto ld_rows = [&](int t, int qs, int g) __attribute__((always_inline)) {  // 1 of 4 read pairs
    const float* row = &s_ld[t % C::NSTAGE][wave][0][0];
    nl[qs][g] = *(const f32x4*)&row[qs * 32 + 8 * g + 4 * hl];
    const f32x4 d = *(const f32x4*)&row[BQ + qs * 32 + 8 * g + 4 * hl];
#pragma unroll
    for (int i = 0; i < 4; ++i) ndl[qs][4 * g + i] = d[i];
  };
  bf16x8 sop[LEAD];    // first scores operands of the next step, read ahead
  // One step, scheduled by hand as NS + NP chunks separated by scheduling
  // barriers.  Chunk c issues MFMA c of the step (scores of sub-tile (t, qs)
  // for c < NS, then products of sub-tile (pt, pqs) from P / dS set 1 - set,
  // accumulating in AGPRs, see mfma32_acc), the operand reads of MFMA c + LEAD
  // (for the last chunks: the next step's first scores operands, when it reads
  // the same, already visible, stage), and in the product chunks EPC
  // elements of the gradient of (t, qs) into set `set`: exp2 as soon as S is
  // complete, dS and the bf16 rounding two chunks later, once dP is.
  // Side work placed in the chunks of a step (`side`): 1 in step qs = 0 of
  // iteration t issues the iteration's copies (one per chunk, spread over the
  // step; only where all of them exist and are full tiles) and reads the lse
  // / delta rows of step qs = 1; 3 only reads those rows (the copies were
  // issued before the step); 2 in step qs = 1
  // converts tile t+1's lse / delta (read early, written later) and then
  // reads the rows of the next iteration's step qs = 0; 0 does nothing.
  auto side_work = [&](int side, int t, int c) __attribute__((always_inline)) {
    constexpr int SPREAD = (NS + NP) / VPT;  // chunks between copies
    if (side == 1 || side == 3) {
      if (side == 1 && c % SPREAD == 1 && c / SPREAD < VPT) issue_copy_full(t, c / SPREAD);
      if (c >= NS + 2 && c < NS + 6) ld_rows(t, 1, c - NS - 2);
    } else if (side == 2 && t + 1 < ntiles) {
      if (c == 2) convert_read(t + 1);
      if (c == NS - 2) convert_write(t + 1);
      if (c >= NS + 2 && c < NS + 6) ld_rows(t + 1, 0, c - NS - 2);
    }
  };
  auto step = [&](int t, int qs, int set, bool prod, int pt, int pqs, bool pre_in,
                  bool pre_out, int nt, int nqs, int side) __attribute__((always_inline)) {
    bf16x8 op[NS + NP];
#pragma unroll
    for (int i = 0; i < LEAD; ++i) op[i] = pre_in ? sop[i] : score_operand(t, qs, i);
    f32x16 pr, dsr;
    u32x4 pw[2], dw[2];
    auto finish = [&](int r) __attribute__((always_inline)) {  // dS and rounding of element r
      dsr[r] = pr[r] * ndl[qs][r];  // dP already holds dO V^T - delta
      if (r & 1) {
        const bf16x2 pp = {(bf16)pr[r - 1], (bf16)pr[r]};
        const bf16x2 d2 = {(bf16)dsr[r - 1], (bf16)dsr[r]};
        pw[r >> 3][(r & 7) >> 1] = __builtin_bit_cast(uint32_t, pp);
        dw[r >> 3][(r & 7) >> 1] = __builtin_bit_cast(uint32_t, d2);
      }
    };
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < NS + NP; ++c) {
      if (c < DS) {
        s = mfma32(op[c], kreg[c], c == 0 ? f32x16{} : s);
      } else if (c < NS) {
        ndl[qs] = mfma32(op[c], vreg[c - DS], ndl[qs]);
      } else if (prod) {
        const int i = c - NS, p = i / (2 * DD), dd = (i / 2) % DD;
        if ((i & 1) == 0)
          mfma32_acc(dv[dd], pbf[1 - set][p], op[c]);
        else
          mfma32_acc(dk[dd], dsbf[1 - set][p], op[c]);
      }
      const int j = c + LEAD;
      if (j < NS)
        op[j] = score_operand(t, qs, j);
      else if (j < NS + NP) {
        if (prod) op[j] = prod_operand(pt, pqs, j - NS);
      } else if (pre_out) {
        sop[j - NS - NP] = score_operand(nt, nqs, j - NS - NP);
      }
      if (c >= NS) {
        const int k = c - NS;
#pragma unroll
        for (int e = k * EPC; e < (k + 1) * EPC; ++e) pr[e] = exp2_fast(fmaf(s[e], c2, nl[qs][e >> 2][e & 3]));
        if (k >= 2) {
#pragma unroll
          for (int e = (k - 2) * EPC; e < (k - 1) * EPC; ++e) finish(e);
        }
      }
      side_work(side, t, c);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int e = 16 - 2 * EPC; e < 16; ++e) finish(e);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      pbf[set][h] = __builtin_bit_cast(bf16x8, pw[h]);
      dsbf[set][h] = __builtin_bit_cast(bf16x8, dw[h]);
    }
  };
  // Products of the last sub-tile (after the loop; no scores, no gradient).
  auto last_products = [&](int pt, int pqs, int pset) __attribute__((always_inline)) {
    bf16x8 op[NP];
#pragma unroll
    for (int i = 0; i < LEAD; ++i) op[i] = prod_operand(pt, pqs, i);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = i / (2 * DD), dd = (i / 2) % DD;
      if ((i & 1) == 0)
        mfma32_acc(dv[dd], pbf[pset][p], op[i]);
      else
        mfma32_acc(dk[dd], dsbf[pset][p], op[i]);
      if (i + LEAD < NP) op[i + LEAD] = prod_operand(pt, pqs, i + LEAD);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Keys past the end, or after the query on the diagonal block, take no
  // part: their P and dS (already rounded to bf16) are cleared bit-wise, which
  // also discards any overflow in them.  Only sub-tiles that straddle the
  // diagonal or the end of the block need it; the test is wave-uniform and
  // made scalar, so elsewhere the mask is a skipped branch.
  auto mask_grad = [&](int t, int qs, int set) __attribute__((always_inline)) {
    const int qt0 = qstart + t * BQ + qs * 32;
    if (__builtin_amdgcn_readfirstlane((kw0 + 31 >= Lk) || (diag && kw_last > qt0))) {
      auto dead = [&](int r) { return kj >= Lk || (diag && kj > qt0 + 8 * (r >> 2) + 4 * hl + (r & 3)); };
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 pw = __builtin_bit_cast(u32x4, pbf[set][half]);
        u32x4 dw = __builtin_bit_cast(u32x4, dsbf[set][half]);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int r = 8 * half + 2 * k;  // low half-word: element r, high: r + 1
          const uint32_t keep = (dead(r) ? 0u : 0x0000FFFFu) | (dead(r + 1) ? 0u : 0xFFFF0000u);
          pw[k] &= keep;
          dw[k] &= keep;
        }
        pbf[set][half] = __builtin_bit_cast(bf16x8, pw);
        dsbf[set][half] = __builtin_bit_cast(bf16x8, dw);
      }
    }
  };
  auto end_iter = [&](int t) __attribute__((always_inline)) {
    // Iteration t+1 reads stage t+1 and converts tile t+2's lse / delta, both
    // copied in iteration t-1; this iteration's copies may stay in flight.
    if (t + 3 < ntiles)
      wait_vmem_n<VPT>();
    else if (t + 2 < ntiles)
      wait_vmem_n<2 * LPW>();
    else
      wait_vmem();
    __syncthreads();
  };

  // Tiles before this wave's first active tile: keep the pipeline moving
  // (copies, and the conversion of the next tile's lse / delta).
  int t = 0;
  for (; t < min(ft, ntiles); ++t) {
    for (int k = 0; k < VPT; ++k)
      if (copy_live(t, k)) issue_copy(t, k);
    if (t + 1 < ntiles) {
      convert_read(t + 1);
      convert_write(t + 1);
    }
    end_iter(t);
  }
  auto top_copies = [&](int t) __attribute__((always_inline)) {
    for (int k = 0; k < VPT; ++k)
      if (copy_live(t, k)) issue_copy(t, k);
  };
  if (t < ntiles) {  // first active tile: nothing to multiply before it
#pragma unroll
    for (int g = 0; g < 4; ++g) ld_rows(t, 0, g);
    if (t + 3 < nfull) {
      step(t, 0, 0, false, 0, 0, false, true, t, 1, 1);
    } else {
      top_copies(t);
      step(t, 0, 0, false, 0, 0, false, true, t, 1, 3);
    }
    mask_grad(t, 0, 0);
    step(t, 1, 1, true, t, 0, true, false, 0, 0, 2);
    mask_grad(t, 1, 1);
    end_iter(t);
    ++t;
  }
  // Steady state: every copy exists and is a full tile.
  for (; t + 3 < nfull; ++t) {
    step(t, 0, 0, true, t - 1, 1, false, true, t, 1, 1);
    mask_grad(t, 0, 0);
    step(t, 1, 1, true, t, 0, true, false, 0, 0, 2);
    mask_grad(t, 1, 1);
    end_iter(t);
  }
  for (; t < ntiles; ++t) {
    top_copies(t);
    step(t, 0, 0, true, t - 1, 1, false, true, t, 1, 3);
    mask_grad(t, 0, 0);
    step(t, 1, 1, true, t, 0, true, false, 0, 0, 2);
    mask_grad(t, 1, 1);
    end_iter(t);
  }
  // The last sub-tile's products (its stage is not reloaded after the loop).
  if (ft < ntiles) last_products(ntiles - 1, 1, 1);
  acc_ready(dk, dv);

  // dK / dV rows: lane holds head-dim column dd*32 + l32 of keys
  // kw0 + 8*(r/4) + 4*hl + r%4.
  float* out = sp == 0 ? dKV : WS + (size_t)(sp - 1) * 2 * (BH / G) * Lk * D;
  const bool add = sp == 0 || !ws_store;
  float* dKp = out + (size_t)kvbh * Lk * D;
  float* dVp = out + ((size_t)(BH / G) + kvbh) * Lk * D;
#pragma unroll
  for (int dd = 0; dd < DD; ++dd) {
    // all loads of this head-dim tile first, then the stores
    float ok[16], ov[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kw0 + 8 * (r >> 2) + 4 * hl + (r & 3);
      const size_t o = (size_t)min(key, Lk - 1) * D + dd * 32 + l32;
      ok[r] = add ? dKp[o] : 0.f;
      ov[r] = add ? dVp[o] : 0.f;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kw0 + 8 * (r >> 2) + 4 * hl + (r & 3);
      if (key < Lk) {
        const size_t o = (size_t)key * D + dd * 32 + l32;
        dKp[o] = ok[r] + dk[dd][r] * scale;
        dVp[o] = ov[r] + dv[dd][r];
      }
    }
  }
}

}  // namespace

// BN = 64 keys per dQ tile with eight waves (256 query rows per workgroup);
// BQ = 64 queries per dK/dV tile with four waves (128 keys per workgroup).
// With G query heads per key/value head, the dK/dV kernel runs over the
// members of a group in launches of nsplit members each (the last one may
// hold fewer); split 0 adds into dkv, split s > 0 into copy s - 1 of dkv in
// ws, which the first launch stores and the later ones add to, and a last
// pass adds the copies into dkv in copy order.  Every sum is taken in a
// fixed order, so results are deterministic.
hipError_t ra_launch_bwd_dq(const void* q, const void* kv, const void* dout,
                            const float* lse, const float* delta, float* dq_acc,
                            const ra_launch& a) {
  constexpr int NW = 8, BM = NW * 32;
  const int BH = a.B * a.H;
  const int n_qt = (a.Lq + BM - 1) / BM;
  if ((long long)n_qt * BH <= 0) return hipSuccess;
  const float c2 = a.scale * kLog2e;
#define RA_DQ(DD)                                                                         \
  hipLaunchKernelGGL((dq_kernel<DD, 64, NW>), dim3(n_qt * BH), dim3(NW * 64), 0, a.stream, \
                     (const bf16*)q, (const bf16*)kv, (const bf16*)dout, lse, delta, dq_acc, \
                     BH, a.H, a.H / a.Hkv, a.Lq, a.Lk, n_qt, a.diag, c2, a.scale)
  if (a.D == 128) RA_DQ(128);
  else if (a.D == 64) RA_DQ(64);
  else return hipErrorInvalidValue;
#undef RA_DQ
  return hipGetLastError();
}

hipError_t ra_launch_bwd_dkv(const void* q, const void* kv, const void* dout,
                             const float* lse, const float* delta, float* dkv, float* ws,
                             int nsplit, const ra_launch& a) {
  constexpr int NW = 4, BK = NW * 32;
  const int BH = a.B * a.H, G = a.H / a.Hkv, BHkv = a.B * a.Hkv;
  const int n_kt = (a.Lk + BK - 1) / BK;
  if ((long long)n_kt * BHkv <= 0) return hipSuccess;
  if (nsplit < 1 || nsplit > G || (nsplit > 1 && !ws)) return hipErrorInvalidValue;
  const float c2 = a.scale * kLog2e;
  if (a.D != 128 && a.D != 64) return hipErrorInvalidValue;
  for (int qj = 0; qj < G; qj += nsplit) {
    const int ns = min(nsplit, G - qj);
    const unsigned grid = (unsigned)(n_kt * BHkv * ns);
#define RA_DKV(DD)                                                                             \
  hipLaunchKernelGGL((dkv_kernel<DD, 64, NW>), dim3(grid), dim3(NW * 64), 0, a.stream,          \
                     (const bf16*)q, (const bf16*)kv, (const bf16*)dout, lse, delta, dkv, ws,   \
                     BH, a.H, G, qj, qj == 0 ? 1 : 0, a.Lq, a.Lk, n_kt, a.diag, c2, a.scale)
    if (a.D == 128) RA_DKV(128);
    else RA_DKV(64);
#undef RA_DKV
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (nsplit > 1)
    return ra_launch_add_copies(dkv, ws, nsplit - 1, (int64_t)2 * BHkv * a.Lk * a.D, a.stream);
  return hipSuccess;
}
