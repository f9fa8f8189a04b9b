// Forward ring step, bf16 inputs, fp32 accumulation, gfx950 MFMA.
//
// One launch attends the member's query block to one key/value block and
// folds the normalised result into (o_acc, lse_acc): the blockwise pass and
// the associative online-softmax combine of a ring member (Ring Attention
// keyword page, definition; darcstar commentary on the associative combine
// and exact seams).
//
// Work decomposition.  A workgroup owns BM = NW*32 query rows of one
// (batch, head); each wave owns 32 rows and keeps their queries in registers
// as the B operand of
//     S^T = K_tile Q^T          (32x32x16 bf16 MFMA, fp32 accumulators)
// so that a lane holds one query and 16 keys of every 32x32 score tile: the
// row max and row sum are in-lane reductions plus one permlane32 swap.  The
// probabilities P^T are rounded to bf16 in registers and feed
//     O^T += V_tile^T P^T
// directly as the B operand; the V^T operand comes from LDS transpose reads,
// with the key order permuted to match the accumulator layout (the
// contraction runs over keys, so a common permutation of both operands
// leaves the sum unchanged).
//
// Memory pipeline.  Key and value tiles of BN keys are copied global -> LDS
// with direct-to-LDS loads (no registers, no LDS store instructions) into two
// rings of four tiles.  Iteration t reads K tiles t, t+1 and V tiles t-1, t,
// issues K tile t+3 and V tile t+2, and at its end waits only for the loads
// issued one iteration earlier: every load has two iterations to land.
// Rows are XOR-swizzled in 16-byte chunks so that both the 16-byte K reads (16 rows per LDS cycle) and the
// V transpose reads (4 rows x 32 columns per half-wave) touch every bank
// once.  Keys past the end of the block load a clamped valid row; the mask
// zeroes their probabilities.
//
// Ping-pong.  On gfx950 a wave's vector ALU work does not run under its own
// MFMAs, but work of a second wave on the same SIMD largely does.  With
// eight waves, each SIMD hosts one wave of group A (waves 0..3) and one of
// group B (waves 4..7).  Per key tile t, each wave runs an MFMA phase (the
// value product of tile t-1 or t and the scores of the next tile; B issues
// its scores first) and a VALU phase (softmax of tile t), in opposite orders
// in the two groups, so the softmax of one wave fills the other wave's MFMA
// phase.  Both groups
// meet at one barrier per tile.  MFMA phases run at a raised wave priority,
// group B's (which opens the tile) above group A's.
//
// Softmax.  The running max is kept in log2 units (scores scaled by
// scale*log2(e), folded into the exponent's FMA).  A tile's probabilities
// are first taken against the running max as it stands, with no row max at
// all; only when some lane's partial row sum exceeds 2^16 (some score rose
// more than 16 above the max, or the first tile, whose sentinel max makes
// the sum infinite) is the row max taken, the accumulators rescaled and the
// tile's probabilities recomputed.  Every probability stays <= 2^16, and the
// final normalisation with the same max keeps the result exact.  Row sums
// add the fp32 probabilities in four independent chains.
//
// Causal seam.  For the diagonal block (query and key positions share the
// block offset) key j is visible to query i iff j <= i; a workgroup only
// visits tiles up to its last row, a wave skips the MFMA work of tiles past
// its last row, and the element mask runs only on tiles that straddle the
// diagonal or the ragged end of the block.  Past blocks need no mask; future
// blocks are never launched.
//
// Epilogue.  The block partial (o_b = acc / l, lse_b = m + log l) is folded
// into the fp32 accumulators with mu = max(lse_a, lse_b):
//     o <- (e^{lse_a-mu} o_a + e^{lse_b-mu} o_b) / (e^{lse_a-mu} + e^{lse_b-mu})
// treating lse_a = -inf as the empty partial.
#include <math.h>

#include "ra_common.h"

using namespace ra;

namespace {

// A tile's probabilities are taken against the running max as it stands
// while this lane's share of their sum stays at most kSumLimit.
constexpr float kSumLimit = 65536.0f;

// Wave priority of group B's MFMA phase, above group A's (1) and the softmax
// phases (0).  B opens each tile with its MFMA phase; A's softmax is shorter,
// and at equal priority A's MFMA phase would take the MFMA pipe from B's
// unfinished one, so that B's softmax later ran with no MFMA work beside it.
constexpr int kPrioB = 2;

template <int D, int BN, int NW>
struct FwdCfg {
  static constexpr int BM = NW * 32;         // query rows per workgroup
  static constexpr int NT = NW * 64;         // threads per workgroup
  static constexpr int ROWB = D * 2;         // bytes per K or V row
  static constexpr int TILEB = BN * ROWB;    // bytes per K (or V) tile
  static constexpr int NSLOT = 4;            // K ring and V ring, 4 tiles each
  static constexpr int VBASE = NSLOT * TILEB;  // V ring after the K ring
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
};

template <int D, int BN, int NW>
__global__ __launch_bounds__(NW * 64, 1) void fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ KV,
    float* __restrict__ Oacc, float* __restrict__ LSEacc, int BH, int H, int G, int Lq,
    int Lk, int n_qt, int diag, float c2) {
  using C = FwdCfg<D, BN, NW>;
  constexpr int KK = BN / 32;  // 32-key sub-tiles per tile
  constexpr int DS = D / 16;   // 16-wide head-dim slices (S contraction)
  constexpr int DD = D / 32;   // 32-wide head-dim tiles (O^T rows)
  __shared__ __attribute__((aligned(1024))) char smem[2 * C::NSLOT * C::TILEB];
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(lvoid*)smem;  // LDS byte address

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  // Group B (second wave on each SIMD) runs its phases in the other order.
  const bool group_b = NW == 8 && wave >= 4;
  // Paired waves of a SIMD take adjacent 32-row blocks (similar causal work).
  const int rblk = NW == 8 ? 2 * (wave & 3) + (wave >> 2) : wave;

  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / n_qt;
  int qt = tile % n_qt;
  if (diag) qt = n_qt - 1 - qt;  // longest causal rows first
  const int q0 = qt * C::BM;
  const int qw0 = q0 + rblk * 32;
  const int qi = qw0 + l32;

  // Groups of G query heads share one key/value head.
  const int kvbh = (bh / H) * (H / G) + (bh % H) / G;
  const bf16* Qp = Q + (size_t)bh * Lq * D;
  const bf16* Kp = KV + (size_t)kvbh * Lk * D;
  const bf16* Vp = KV + ((size_t)(BH / G) + kvbh) * Lk * D;

  // diag == 2 (no skipping): every tile, the ones above the diagonal fully masked
  const int kend = diag == 1 ? min(Lk, q0 + C::BM) : Lk;
  const int ntiles = (kend + BN - 1) / BN;
  // tiles this wave computes: a prefix [0, ntw)
  const int qw_last = min(qw0 + 31, Lq - 1);
  int ntw = 0;
  if (qw0 < Lq) ntw = diag == 1 ? min(ntiles, qw_last / BN + 1) : ntiles;

  const LdsOffsets<D> off(lane);

  const TileLoader<D, BN, NW, true, true> loader(wave, lane);
  // Branch-free single copies (the caller guarantees that the tile exists
  // and has no keys past the end).  With eight waves and only full tiles
  // ahead, each wave issues half of its copies at the top of the iteration
  // and half between its two phases, which stalls less than a burst of
  // copies after the barrier.
  auto copy1 = [&](bool isv, int t, int i) __attribute__((always_inline)) {
    constexpr int LPW = decltype(loader)::LPW;
    const uint32_t base = smem_lds + (isv ? C::VBASE : 0) + (t % C::NSLOT) * C::TILEB;
    const int j = wave * LPW + i;
    const uint32_t voff[1] = {(loader.lane_part ^ dma_xor<D>(j)) + (uint32_t)j * 1024};
    dma16_group<1>(uniform((isv ? Vp : Kp) + (size_t)t * BN * D), voff, base + (uint32_t)j * 1024);
  };
  const int nfull = Lk / BN;
  // (every wave issues exactly two copies per tile in this configuration)
  constexpr bool kSplitCopies = NW == 8 && decltype(loader)::NL == 2 * NW;
  auto issue_k = [&](int t) __attribute__((always_inline)) {
    loader.issue(smem_lds + (t % C::NSLOT) * C::TILEB, Kp, t * BN, Lk);
  };
  auto issue_v = [&](int t) __attribute__((always_inline)) {
    loader.issue(smem_lds + C::VBASE + (t % C::NSLOT) * C::TILEB, Vp, t * BN, Lk);
  };

  // Iteration 0 needs K tiles 0, 1 and V tile 0; K 2 and V 1 may stay in
  // flight until its end.
  if (ntiles > 0) issue_k(0);
  if (ntiles > 0) issue_v(0);
  if (ntiles > 1) issue_k(1);

  // Queries of this wave: B operand of S^T = K Q^T.
  bf16x8 qreg[DS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds)
    qreg[ds] = qi < Lq ? *(const bf16x8*)(Qp + (size_t)qi * D + ds * 16 + hl * 8) : bf16x8{};

  f32x16 oacc[DD];
#pragma unroll
  for (int dd = 0; dd < DD; ++dd) oacc[dd] = f32x16{};
  float m = kNegBig, lsum = 0.f;
  f32x16 s[KK];      // scores of the tile being softmaxed
  bf16x8 pb[KK][2];  // its probabilities, bf16, as PV B operands

  wait_vmem();
  if (ntiles > 2) issue_k(2);
  if (ntiles > 1) issue_v(1);
  __syncthreads();

  auto scores = [&](const char* kt) __attribute__((always_inline)) {  // s = K Q^T
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) s[kk] = f32x16{};
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const bf16x8 a = *(const bf16x8*)(kt + kk * 32 * C::ROWB + off.row[ds]);
        s[kk] = mfma32(a, qreg[ds], s[kk]);
      }
  };
  auto value = [&](const char* vt) __attribute__((always_inline)) {  // O^T += V^T P^T
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const char* vb = vt + (kk * 32 + 16 * half) * C::ROWB;
#pragma unroll
        for (int dd = 0; dd < DD; ++dd) {
          const bf16x4 lo = lds_read_tr((const bf16*)(vb + off.tr[dd]));
          const bf16x4 hi = lds_read_tr((const bf16*)(vb + off.tr[dd] + off.trd));
          oacc[dd] = mfma32(cat(lo, hi), pb[kk][half], oacc[dd]);
        }
      }
  };
  // value: KK*2*DD MFMAs with two transpose reads each; scores: DS*KK MFMAs
  // with one 16-byte read each.
  using Pipe = MfmaReadPipeline<KK * 2 * DD, 2, DS * KK, 1, 4>;
  using PipeSV = MfmaReadPipeline<DS * KK, 1, KK * 2 * DD, 2, 4>;  // scores first
  // s (raw scores) -> pb = bf16(exp2(s*c2 - m)); returns this lane's share of
  // the row sum of the fp32 probabilities, added in four independent chains.
  auto probs = [&]() __attribute__((always_inline)) -> float {
    const float negm = -m;
    float r[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      f32x16 p;  // not written back into s: s stays valid for the rescale path
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = exp2_fast(fmaf(s[kk][i], c2, negm));
        r[i & 3] += p[i];
      }
      pb[kk][0] = to_bf16x8(p, 0);
      pb[kk][1] = to_bf16x8(p, 1);
    }
    return (r[0] + r[1]) + (r[2] + r[3]);
  };
  auto softmax = [&](int t) __attribute__((always_inline)) {  // s (raw scores of tile t) -> pb, m, lsum
    const int kt0 = t * BN;
    // (wave-uniform; made scalar so the mask is a skipped branch, not selects)
    if (__builtin_amdgcn_readfirstlane((kt0 + BN > Lk) || (diag && kt0 + BN - 1 > qw0))) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kj = kt0 + kk * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (kj >= Lk || (diag && kj > qi)) s[kk][r] = -INFINITY;
        }
    }
    // Probabilities against the running max as it stands.  Only if some lane's
    // sum exceeds kSumLimit (a score more than log2(kSumLimit) above the max,
    // or the first tile, where the max is still the sentinel and the sum is
    // infinite) is the row max taken, the accumulators rescaled and the
    // probabilities recomputed.  Every probability stays <= kSumLimit.
    float rs = probs();
    if (__builtin_amdgcn_ballot_w64(!(rs <= kSumLimit))) {
      float mx = -INFINITY;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kk][r]);
      mx = max_halves(mx) * c2;
      const float mnew = fmaxf(m, mx);
      const float alpha = exp2_fast(m - mnew);
      m = mnew;
      lsum *= alpha;
#pragma unroll
      for (int dd = 0; dd < DD; ++dd) oacc[dd] *= alpha;
      rs = probs();
    }
    lsum += rs;
  };

  auto k_of = [&](int t) __attribute__((always_inline)) -> const char* {
    return smem + (t % C::NSLOT) * C::TILEB;
  };
  auto v_of = [&](int t) __attribute__((always_inline)) -> const char* {
    return smem + C::VBASE + (t % C::NSLOT) * C::TILEB;
  };

  // Group A computes the scores of tile 0 before the loop; group B computes
  // the scores of tile t inside iteration t.
  if (!group_b && ntw > 0) scores(k_of(0));

  for (int t = 0; t < ntiles; ++t) {
    // K slot (t+3)%4 last served iteration t-1 (K tile t-1); V slot
    // (t+2)%4 last served iteration t-1 (V tile t-2).
    const bool steady = kSplitCopies && t + 3 < nfull;
    if (steady) {
      copy1(false, t + 3, 0);
      copy1(true, t + 2, 0);
    } else {
      if (t + 3 < ntiles) issue_k(t + 3);
      if (t + 2 < ntiles) issue_v(t + 2);
    }
    if (!group_b) {
      // A: softmax(t), then value(t) + scores(t+1)
      if (t < ntw) {
        softmax(t);
        __builtin_amdgcn_sched_barrier(0);
        if (steady) {
          copy1(false, t + 3, 1);
          copy1(true, t + 2, 1);
          __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(1);
        value(v_of(t));
        // Unconditional: past the wave's last tile the scores are unused, and
        // a branch here would keep the previous tile's registers alive.
        scores(k_of(t + 1));
        Pipe::apply();
        __builtin_amdgcn_s_setprio(0);
      } else if (steady) {  // past this wave's last tile: its copies still go out
        copy1(false, t + 3, 1);
        copy1(true, t + 2, 1);
      }
    } else {
      // B: scores(t) + value(t-1), then softmax(t).  (Scores first: the
      // tile then opens with 16-byte K reads; measured 0.3-0.7 % faster than
      // value first.)
      if (t >= 1 && t - 1 < ntw) {
        __builtin_amdgcn_s_setprio(kPrioB);
        scores(k_of(t));
        value(v_of(t - 1));
        PipeSV::apply();
        __builtin_amdgcn_s_setprio(0);
      } else if (t == 0 && ntw > 0) {
        __builtin_amdgcn_s_setprio(kPrioB);
        scores(k_of(0));
        __builtin_amdgcn_s_setprio(0);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (steady) {
        copy1(false, t + 3, 1);
        copy1(true, t + 2, 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (t < ntw) softmax(t);
    }
    // Iteration t+1 reads K tile t+2 and V tile t+1 (issued in iteration
    // t-1); this iteration's loads may stay in flight.
    if (t + 3 < ntiles)
      wait_vmem_n<2 * decltype(loader)::LPW>();
    else if (t + 2 < ntiles)
      wait_vmem_n<decltype(loader)::LPW>();
    else
      wait_vmem();
    __syncthreads();
  }
  // Group B still owes the value product of its last tile; no load touched
  // that V slot after the loop.
  if (group_b && ntw == ntiles && ntw > 0) value(v_of(ntw - 1));

  // Fold the block partial into the running accumulators.
  const float ltot = add_halves(lsum);
  if (qi < Lq && ltot > 0.f) {
    const float lse_b = (m + log2f(ltot)) * kLn2;
    float* lse_p = LSEacc + (size_t)bh * Lq + qi;
    const float lse_a = *lse_p;
    const float inv = 1.f / ltot;
    float wa, wb, lse_new;
    if (lse_a == -INFINITY) {
      wa = 0.f;
      wb = inv;
      lse_new = lse_b;
    } else {
      const float mu = fmaxf(lse_a, lse_b);
      const float ea = expf(lse_a - mu), eb = expf(lse_b - mu);
      const float z = ea + eb;
      lse_new = mu + logf(z);
      wa = ea / z;
      wb = eb / z * inv;
    }
    float* orow = Oacc + ((size_t)bh * Lq + qi) * D;
    f32x4 oa[DD][4];  // all loads first, then the stores
#pragma unroll
    for (int dd = 0; dd < DD; ++dd)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        oa[dd][g] = wa != 0.f ? *(const f32x4*)(orow + dd * 32 + 8 * g + 4 * hl) : f32x4{};
#pragma unroll
    for (int dd = 0; dd < DD; ++dd)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 acc = {oacc[dd][4 * g], oacc[dd][4 * g + 1], oacc[dd][4 * g + 2],
                           oacc[dd][4 * g + 3]};
        *(f32x4*)(orow + dd * 32 + 8 * g + 4 * hl) = acc * wb + oa[dd][g] * wa;
      }
    if (hl == 0) *lse_p = lse_new;
  }
}

template <int D, int BN, int NW>
hipError_t launch(const void* q, const void* kv, float* o_acc, float* lse_acc,
                  const ra_launch& a) {
  using C = FwdCfg<D, BN, NW>;
  const int n_qt = (a.Lq + C::BM - 1) / C::BM;
  const int BH = a.B * a.H;
  const long long grid = (long long)n_qt * BH;
  if (grid <= 0) return hipSuccess;
  const float c2 = a.scale * kLog2e;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, BN, NW>), dim3((unsigned)grid), dim3(C::NT), 0,
                     a.stream, (const bf16*)q, (const bf16*)kv, o_acc, lse_acc, BH, a.H,
                     a.H / a.Hkv, a.Lq, a.Lk, n_qt, a.diag, c2);
  return hipGetLastError();
}

// q_chunk >= 256 selects 256 query rows per workgroup (eight waves, ping-pong),
// else 128 (four waves); k_chunk >= 64 selects 64-key tiles, else 32.
template <int D>
hipError_t launch_d(const void* q, const void* kv, float* o_acc, float* lse_acc,
                    const ra_launch& a) {
  const bool wide_q = a.q_chunk >= 256;
  const bool wide_k = a.k_chunk >= 64;
  if (wide_q)
    return wide_k ? launch<D, 64, 8>(q, kv, o_acc, lse_acc, a)
                  : launch<D, 32, 8>(q, kv, o_acc, lse_acc, a);
  return wide_k ? launch<D, 64, 4>(q, kv, o_acc, lse_acc, a)
                : launch<D, 32, 4>(q, kv, o_acc, lse_acc, a);
}

}  // namespace

hipError_t ra_launch_fwd_bf16(const void* q, const void* kv, float* o_acc,
                              float* lse_acc, const ra_launch& a) {
  if (a.D == 128) return launch_d<128>(q, kv, o_acc, lse_acc, a);
  if (a.D == 64) return launch_d<64>(q, kv, o_acc, lse_acc, a);
  return hipErrorInvalidValue;
}
