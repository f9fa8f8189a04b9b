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
//     transpose reads).  Eight waves ping-pong as in the forward.
//   * dkv_kernel (key-major): a wave keeps 32 keys and their values in
//     registers and sweeps the query tiles (Q, dO, lse, delta) through LDS,
//     forming S = Q K^T and dP = dO V^T, then dV += P^T dO and dK += dS^T Q
//     with dO^T and Q^T by LDS transpose reads.  Four waves, one per SIMD;
//     each wave overlaps the products of tile t with the scores of t+1.
// Tiles move global -> LDS with direct-to-LDS copies into XOR-swizzled rows
// (see ra_common.h), four stages deep, one tile of prefetch.
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

// ---------------------------------------------------------------- dQ ------
template <int D, int BN, int NW>
__global__ __launch_bounds__(NW * 64, 1) void dq_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ KV,
    const bf16* __restrict__ dO, const float* __restrict__ LSE,
    const float* __restrict__ Delta, float* __restrict__ dQacc, int BH, int Lq,
    int Lk, int n_qt, int diag, float c2, float scale) {
  using C = TileCfg<D, BN, NW>;
  constexpr int BM = NW * 32;
  constexpr int KK = BN / 32, DS = D / 16, DD = D / 32;
  // K ring: iteration t reads K tiles t-1 .. t+1, has t+2 in flight and
  // issues t+3.  V ring: reads t, t+1, t+2 in flight, issues t+3.
  constexpr int NK = 5, NV = 4;
  constexpr int VBASE = NK * C::TILEB;
  __shared__ __attribute__((aligned(1024))) char smem[(NK + NV) * C::TILEB];
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

  const bf16* Qp = Q + (size_t)bh * Lq * D;
  const bf16* dOp = dO + (size_t)bh * Lq * D;
  const bf16* Kp = KV + (size_t)bh * Lk * D;
  const bf16* Vp = KV + ((size_t)BH + bh) * Lk * D;

  const int kend = diag ? min(Lk, q0 + BM) : Lk;
  const int ntiles = (kend + BN - 1) / BN;
  const int qw_last = min(qw0 + 31, Lq - 1);
  int ntw = 0;
  if (qw0 < Lq) ntw = diag ? min(ntiles, qw_last / BN + 1) : ntiles;

  const LdsOffsets<D> off(lane);
  using Loader = TileLoader<D, BN, NW, false>;
  const Loader loader(wave, lane);
  auto issue_k = [&](int t) __attribute__((always_inline)) {
    loader.issue(smem_lds + (t % NK) * C::TILEB, Kp, t * BN, Lk);
  };
  auto issue_v = [&](int t) __attribute__((always_inline)) {
    loader.issue(smem_lds + VBASE + (t % NV) * C::TILEB, Vp, t * BN, Lk);
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
    return smem + (t % NK) * C::TILEB;
  };
  auto v_of = [&](int t) __attribute__((always_inline)) -> const char* {
    return smem + VBASE + (t % NV) * C::TILEB;
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
    // K slot (t+3)%5 last served iteration t-1 (K tile t-2, group B's
    // value); V slot (t+3)%4 last served iteration t-1 (V tile t-1).
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
        __builtin_amdgcn_s_setprio(1);
        value(k_of(t - 1));
        scores(k_of(t), v_of(t));
        Pipe::apply();
        __builtin_amdgcn_s_setprio(0);
      } else if (t == 0 && ntw > 0) {
        __builtin_amdgcn_s_setprio(1);
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
template <int D, int BQ, int NW>
__global__ __launch_bounds__(NW * 64, 1) void dkv_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ KV,
    const bf16* __restrict__ dO, const float* __restrict__ LSE,
    const float* __restrict__ Delta, float* __restrict__ dKV, int BH, int Lq,
    int Lk, int n_kt, int diag, float c2, float scale) {
  using C = TileCfg<D, BQ, NW>;
  constexpr int BK = NW * 32;  // keys per workgroup
  constexpr int DS = D / 16, DD = D / 32;
  static_assert(BQ == 64 && NW == 4, "two 32-query sub-tiles per LDS tile; one lse/delta load per wave");
  __shared__ __attribute__((aligned(1024))) char smem[C::NSTAGE * C::STAGEB];
  // Per stage: row 0 lse (converted in place to -lse*log2e), row 1 delta,
  // rows 2-3 written by the other two waves' copies and never read.
  __shared__ __attribute__((aligned(1024))) float s_ld[C::NSTAGE][4][BQ];
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(lvoid*)smem;
  const uint32_t sld_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) float*)&s_ld[0][0][0];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: loop bounds derive from it
  const int l32 = lane & 31, hl = lane >> 5;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / n_kt;
  const int k0 = (tile % n_kt) * BK;  // small k0 first: the most causal work
  const int kw0 = k0 + wave * 32;
  const int kj = kw0 + l32;

  const bf16* Qp = Q + (size_t)bh * Lq * D;
  const bf16* dOp = dO + (size_t)bh * Lq * D;
  const bf16* Kp = KV + (size_t)bh * Lk * D;
  const bf16* Vp = KV + ((size_t)BH + bh) * Lk * D;
  const float* Lp = LSE + (size_t)bh * Lq;
  const float* Dp = Delta + (size_t)bh * Lq;

  // Under the causal mask only queries at or after the first key matter.
  const int qstart = diag ? (k0 / BQ) * BQ : 0;
  const int ntiles = qstart < Lq ? (Lq - qstart + BQ - 1) / BQ : 0;
  const int kw_last = min(kw0 + 31, Lk - 1);
  // This wave's active tiles are a suffix [ft, ntiles): query tiles that
  // end before its first key contribute nothing.
  int ft = diag ? max(0, (kw0 - qstart) / BQ) : 0;
  if (kw0 >= Lk) ft = ntiles;

  const LdsOffsets<D> off(lane);
  using Loader = TileLoader<D, BQ, NW, false>;
  const Loader loader(wave, lane);
  // Per tile each wave issues LPW loads of Q, LPW of dO and one 256-byte
  // copy of lse (waves 0, 2) or delta (waves 1, 3): VPT loads, counted in
  // vmcnt.  Iteration t reads stages t and t+1, has t+2 in flight and
  // issues t+3 into the slot of tile t-1.
  constexpr int VPT = 2 * Loader::LPW + 1;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  auto issue = [&](int t) __attribute__((always_inline)) {
    const int st = t % C::NSTAGE;
    const int q0t = qstart + t * BQ;
    loader.issue(smem_lds + st * C::STAGEB, Qp, q0t, Lq);
    loader.issue(smem_lds + st * C::STAGEB + C::TILEB, dOp, q0t, Lq);
    dma4((wave_u & 1 ? Dp : Lp) + min(q0t + lane, Lq - 1), sld_lds + (st * 4 + wave_u) * BQ * 4);
  };
  // In-place conversion of a landed tile's lse / delta (waves 0 and 1, one
  // value per lane): lse -> -lse*log2e, with -inf (a row that saw no key, or
  // past the end) giving P = 0; delta past the end -> 0.  The read is issued
  // early and the write late in an iteration.
  float ld_raw = 0.f;
  auto ld_read = [&](int t) __attribute__((always_inline)) {
    if (wave_u < 2) ld_raw = s_ld[t % C::NSTAGE][wave_u][lane];
  };
  auto ld_write = [&](int t) __attribute__((always_inline)) {
    if (wave_u < 2) {
      const bool valid = qstart + t * BQ + lane < Lq;
      float v;
      if (wave_u == 0)
        v = (!valid || ld_raw == -INFINITY) ? -INFINITY : -ld_raw * kLog2e;
      else
        v = valid ? ld_raw : 0.f;
      s_ld[t % C::NSTAGE][wave_u][lane] = v;
    }
  };

  if (ntiles > 0) issue(0);
  if (ntiles > 1) issue(1);

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
  // Work runs in 32-query sub-tiles (qs = 0, 1) of the 64-query LDS tiles.
  f32x16 s, dp;            // S and dP of the sub-tile to be softmaxed next
  bf16x8 pbf[2], dsbf[2];  // P and dS of the sub-tile being multiplied
  bf16x8 ob[2][8];         // LDS operands, one MFMA step ahead

  wait_vmem();
  __syncthreads();
  if (ntiles > 0) {
    ld_read(0);
    ld_write(0);
  }
  if (ntiles > 2) issue(2);
  __syncthreads();

  auto stage_of = [&](int t) __attribute__((always_inline)) -> const char* {
    return smem + (t % C::NSTAGE) * C::STAGEB;
  };
  // P = exp(S*scale - lse), dS = P (dP - delta) for sub-tile qs of tile t.
  auto grad = [&](int t, int qs) __attribute__((always_inline)) {
    const int qt0 = qstart + t * BQ + qs * 32;
    const int st = t % C::NSTAGE;
    f32x4 nl[4], dl[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      nl[g] = *(const f32x4*)&s_ld[st][0][qs * 32 + 8 * g + 4 * hl];
      dl[g] = *(const f32x4*)&s_ld[st][1][qs * 32 + 8 * g + 4 * hl];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = exp2_fast(fmaf(s[r], c2, nl[r >> 2][r & 3]));
    if (__builtin_amdgcn_readfirstlane((kw0 + 31 >= Lk) || (diag && kw_last > qt0))) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = qt0 + 8 * (r >> 2) + 4 * hl + (r & 3);
        if (kj >= Lk || (diag && kj > q)) s[r] = 0.f;
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) dp[r] = s[r] * (dp[r] - dl[r >> 2][r & 3]);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      pbf[half] = to_bf16x8(s, half);
      dsbf[half] = to_bf16x8(dp, half);
    }
  };
  // MFMA steps of 8.  Product steps p = 0, 1 (rows 16*p of the sub-tile):
  // dV += P^T dO and dK += dS^T Q over the head-dim tiles, operands by
  // transpose reads.  Score steps p = 2, 3 (head-dim slices (p-2)*DS/2 ..):
  // S = Q K^T and dP = dO V^T, operands by 16-byte row reads; step 2 starts
  // the accumulators from zero.
  auto load_step = [&](int p, const char* st, int qs, bf16x8* o) __attribute__((always_inline)) {
    if (p < 2) {
      const char* qb = st + (qs * 32 + 16 * p) * C::ROWB;
#pragma unroll
      for (int dd = 0; dd < DD; ++dd) {
        o[2 * dd] = cat(lds_read_tr((const bf16*)(qb + C::TILEB + off.tr[dd])),
                        lds_read_tr((const bf16*)(qb + C::TILEB + off.tr[dd] + off.trd)));
        o[2 * dd + 1] = cat(lds_read_tr((const bf16*)(qb + off.tr[dd])),
                            lds_read_tr((const bf16*)(qb + off.tr[dd] + off.trd)));
      }
    } else {
#pragma unroll
      for (int j = 0; j < DS / 2; ++j) {
        const char* rb = st + qs * 32 * C::ROWB + off.row[(DS / 2) * (p - 2) + j];
        o[2 * j] = *(const bf16x8*)rb;
        o[2 * j + 1] = *(const bf16x8*)(rb + C::TILEB);
      }
    }
  };
  auto mfma_step = [&](int p, const bf16x8* o) __attribute__((always_inline)) {
    if (p < 2) {
#pragma unroll
      for (int dd = 0; dd < DD; ++dd) {
        dv[dd] = mfma32(pbf[p], o[2 * dd], dv[dd]);
        dk[dd] = mfma32(dsbf[p], o[2 * dd + 1], dk[dd]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < DS / 2; ++j) {
        const int ds = (DS / 2) * (p - 2) + j;
        const bool first = ds == 0;
        s = mfma32(o[2 * j], kreg[ds], first ? f32x16{} : s);
        dp = mfma32(o[2 * j + 1], vreg[ds], first ? f32x16{} : dp);
      }
    }
  };
  // Runs steps [p0, p1); the operands of step p0 must already be in ob[p0&1].
  auto steps = [&](int p0, int p1, const char* pst, int pqs, const char* sst, int sqs)
      __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      if (p >= p0 && p < p1) {
        if (p + 1 < p1) load_step(p + 1, p + 1 < 2 ? pst : sst, p + 1 < 2 ? pqs : sqs, ob[(p + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);  // keep the next step's reads ahead
        mfma_step(p, ob[p & 1]);
      }
    }
  };
  // Multiply sub-tile (t, qs), then score the next sub-tile (tn, 1 - qs).
  auto full_phase = [&](int t, int qs, int tn) __attribute__((always_inline)) {
    grad(t, qs);
    __builtin_amdgcn_sched_barrier(0);
    load_step(0, stage_of(t), qs, ob[0]);
    steps(0, 4, stage_of(t), qs, stage_of(tn), 1 - qs);
  };
  auto score_phase = [&](int tn, int sqs) __attribute__((always_inline)) {
    load_step(2, stage_of(tn), sqs, ob[0]);
    steps(2, 4, nullptr, 0, stage_of(tn), sqs);
  };
  auto prod_phase = [&](int t, int qs) __attribute__((always_inline)) {
    grad(t, qs);
    __builtin_amdgcn_sched_barrier(0);
    load_step(0, stage_of(t), qs, ob[0]);
    steps(0, 2, stage_of(t), qs, nullptr, 0);
  };
  auto end_tile = [&](int t) __attribute__((always_inline)) {
    if (t + 1 < ntiles) ld_write(t + 1);
    // Iteration t+1 reads stage t+2 (issued in iteration t-1); this
    // iteration's loads may stay in flight.
    if (t + 3 < ntiles)
      wait_vmem_n<VPT>();
    else
      wait_vmem();
    __syncthreads();
  };
  auto begin_tile = [&](int t) __attribute__((always_inline)) {
    if (t + 3 < ntiles) issue(t + 3);
    if (t + 1 < ntiles) ld_read(t + 1);
  };

  // Tiles before this wave's first active tile: only keep the pipeline
  // moving; the last of them scores sub-tile (ft, 0).
  int t = 0;
  for (; t < min(ft, ntiles); ++t) {
    begin_tile(t);
    if (t + 1 == ft && ft < ntiles) score_phase(ft, 0);
    end_tile(t);
  }
  if (ft == 0 && ntiles > 0) score_phase(0, 0);
  // Steady state: both sub-tiles multiplied, the next two scored.
  for (; t + 1 < ntiles; ++t) {
    begin_tile(t);
    full_phase(t, 0, t);
    full_phase(t, 1, t + 1);
    end_tile(t);
  }
  // Last tile: nothing left to score after its second sub-tile.
  if (t < ntiles) {
    begin_tile(t);
    full_phase(t, 0, t);
    prod_phase(t, 1);
    end_tile(t);
  }

  // dK / dV rows: lane holds head-dim column dd*32 + l32 of keys
  // kw0 + 8*(r/4) + 4*hl + r%4.
  float* dKp = dKV + (size_t)bh * Lk * D;
  float* dVp = dKV + ((size_t)BH + bh) * Lk * D;
#pragma unroll
  for (int dd = 0; dd < DD; ++dd) {
    // all loads of this head-dim tile first, then the stores
    float ok[16], ov[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kw0 + 8 * (r >> 2) + 4 * hl + (r & 3);
      const size_t o = (size_t)min(key, Lk - 1) * D + dd * 32 + l32;
      ok[r] = dKp[o];
      ov[r] = dVp[o];
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
                     BH, a.Lq, a.Lk, n_qt, a.diag, c2, a.scale)
  if (a.D == 128) RA_DQ(128);
  else if (a.D == 64) RA_DQ(64);
  else return hipErrorInvalidValue;
#undef RA_DQ
  return hipGetLastError();
}

hipError_t ra_launch_bwd_dkv(const void* q, const void* kv, const void* dout,
                             const float* lse, const float* delta, float* dkv,
                             const ra_launch& a) {
  constexpr int NW = 4, BK = NW * 32;
  const int BH = a.B * a.H;
  const int n_kt = (a.Lk + BK - 1) / BK;
  if ((long long)n_kt * BH <= 0) return hipSuccess;
  const float c2 = a.scale * kLog2e;
#define RA_DKV(DD)                                                                          \
  hipLaunchKernelGGL((dkv_kernel<DD, 64, NW>), dim3(n_kt * BH), dim3(NW * 64), 0, a.stream, \
                     (const bf16*)q, (const bf16*)kv, (const bf16*)dout, lse, delta, dkv, BH, \
                     a.Lq, a.Lk, n_kt, a.diag, c2, a.scale)
  if (a.D == 128) RA_DKV(128);
  else if (a.D == 64) RA_DKV(64);
  else return hipErrorInvalidValue;
#undef RA_DKV
  return hipGetLastError();
}
