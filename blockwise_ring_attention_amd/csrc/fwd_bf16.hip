// Forward ring step, bf16 inputs, fp32 accumulation, gfx950 MFMA.
//
// One launch attends the member's query block to one key/value block and
// folds the normalised result into (o_acc, lse_acc): the blockwise pass and
// the associative online-softmax combine of a ring member (Ring Attention
// keyword page, definition; darcstar commentary on the associative combine
// and exact seams).
//
// Work decomposition.  A workgroup owns BM = NW*QT*32 query rows of one
// (batch, head); each of its NW waves owns QT sub-tiles of 32 rows and keeps
// their queries in registers for the whole sweep.  Key/value tiles of BN
// keys are staged through LDS (double-buffered, one barrier per tile) and
// every wave computes
//     S^T = K_tile Q^T          (32x32x16 bf16 MFMA, fp32 accumulators)
// so that each lane holds one query and 16 keys of every 32x32 score tile:
// the row max and row sum are in-lane reductions plus one permlane32 swap.
// The probabilities P^T are rounded to bf16 in registers and feed
//     O^T += V_tile^T P^T
// directly as the B operand; the matching V^T operand comes from LDS with
// transpose reads, with the key order permuted to match the accumulator
// layout (the contraction is over keys, so any common key permutation of
// both operands gives the same sum).
//
// Causal seam.  For the diagonal block (query and key positions share the
// block offset) key j is visible to query i iff j <= i; the launch only
// visits key tiles up to the workgroup's last row, a wave skips the MFMA
// work of tiles that lie entirely after its last row, and the element mask
// is evaluated only on tiles that straddle the diagonal or the ragged end of
// the block.  Past blocks need no mask; future blocks are never launched.
//
// Epilogue.  The block partial (o_b = acc / l, lse_b = m + log l) is folded
// into the fp32 accumulators with mu = max(lse_a, lse_b):
//     o <- (e^{lse_a-mu} o_a + e^{lse_b-mu} o_b) / (e^{lse_a-mu} + e^{lse_b-mu})
// treating lse_a = -inf as the empty partial.
#include <math.h>

#include "ra_common.h"

using namespace ra;

namespace {

template <int D, int QT, int BN, int NW>
struct FwdCfg {
  static constexpr int BM = NW * QT * 32;  // query rows per workgroup
  static constexpr int LDW = D + 8;        // LDS row stride (16-byte pad vs bank conflicts)
  static constexpr int NT = NW * 64;       // threads per workgroup
  static constexpr int CH = BN * D / 8;    // 16-byte chunks per K (or V) tile
  static constexpr int PT = CH / NT;       // chunks per thread per tensor
  static_assert(CH % NT == 0, "a tile must split evenly over the threads");
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
};

template <int D, int QT, int BN, int NW>
__global__ __launch_bounds__(NW * 64, 1) void fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ KV,
    float* __restrict__ Oacc, float* __restrict__ LSEacc, int BH, int Lq,
    int Lk, int n_qt, int diag, float c2) {
  using C = FwdCfg<D, QT, BN, NW>;
  __shared__ __attribute__((aligned(16))) bf16 smem[2][2][BN * C::LDW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / n_qt;
  int qt = tile % n_qt;
  if (diag) qt = n_qt - 1 - qt;  // longest causal rows first
  const int q0 = qt * C::BM;
  const int qw0 = q0 + wave * QT * 32;

  const bf16* Qp = Q + (size_t)bh * Lq * D;
  const bf16* Kp = KV + (size_t)bh * Lk * D;
  const bf16* Vp = KV + ((size_t)BH + bh) * Lk * D;

  // Queries of this wave: B operand of S^T = K Q^T (lane: query l32,
  // head-dim elements 8*hl .. 8*hl+7 of every 16-wide slice).
  bf16x8 qreg[QT][D / 16];
#pragma unroll
  for (int qq = 0; qq < QT; ++qq) {
    const int row = qw0 + qq * 32 + l32;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      if (row < Lq)
        qreg[qq][ds] = *(const bf16x8*)(Qp + (size_t)row * D + ds * 16 + hl * 8);
      else
        qreg[qq][ds] = bf16x8{};
    }
  }

  f32x16 oacc[QT][D / 32];
  float m[QT], lsum[QT];
#pragma unroll
  for (int qq = 0; qq < QT; ++qq) {
    m[qq] = kNegBig;
    lsum[qq] = 0.f;
#pragma unroll
    for (int dd = 0; dd < D / 32; ++dd) oacc[qq][dd] = f32x16{};
  }

  const int kend = diag ? min(Lk, q0 + C::BM) : Lk;
  const int ntiles = (kend + BN - 1) / BN;
  const int qw_last = min(qw0 + QT * 32, Lq) - 1;

  bf16x8 pk[C::PT], pv[C::PT];
  auto gload = [&](int kt0) {
#pragma unroll
    for (int i = 0; i < C::PT; ++i) {
      const int c = tid + i * C::NT;
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      const int key = kt0 + row;
      if (key < Lk) {
        pk[i] = *(const bf16x8*)(Kp + (size_t)key * D + col);
        pv[i] = *(const bf16x8*)(Vp + (size_t)key * D + col);
      } else {  // ragged end: zeros keep 0 * V finite
        pk[i] = bf16x8{};
        pv[i] = bf16x8{};
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::PT; ++i) {
      const int c = tid + i * C::NT;
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      *(bf16x8*)&smem[buf][0][row * C::LDW + col] = pk[i];
      *(bf16x8*)&smem[buf][1][row * C::LDW + col] = pv[i];
    }
  };

  if (ntiles > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int kt0 = t * BN;
    if (t + 1 < ntiles) gload(kt0 + BN);
    const bool active = (qw0 < Lq) && (!diag || kt0 <= qw_last);
    if (active) {
      const bf16* Ks = smem[buf][0];
      const bf16* Vs = smem[buf][1];
      f32x16 s[BN / 32][QT];
#pragma unroll
      for (int kk = 0; kk < BN / 32; ++kk)
#pragma unroll
        for (int qq = 0; qq < QT; ++qq) s[kk][qq] = f32x16{};
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds) {
#pragma unroll
        for (int kk = 0; kk < BN / 32; ++kk) {
          const bf16x8 a = *(const bf16x8*)(Ks + (kk * 32 + l32) * C::LDW + ds * 16 + hl * 8);
#pragma unroll
          for (int qq = 0; qq < QT; ++qq) s[kk][qq] = mfma32(a, qreg[qq][ds], s[kk][qq]);
        }
      }

      const bool need_mask = (kt0 + BN > Lk) || (diag && kt0 + BN - 1 > qw0);
#pragma unroll
      for (int qq = 0; qq < QT; ++qq) {
        const int qi = qw0 + qq * 32 + l32;
        float mx = -INFINITY;
#pragma unroll
        for (int kk = 0; kk < BN / 32; ++kk)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float x = s[kk][qq][r] * c2;
            if (need_mask) {
              const int kj = kt0 + kk * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
              if (kj >= Lk || (diag && kj > qi)) x = -INFINITY;
            }
            s[kk][qq][r] = x;
            mx = fmaxf(mx, x);
          }
        mx = max_halves(mx);
        const float mnew = fmaxf(m[qq], mx);
        const float alpha = exp2_fast(m[qq] - mnew);
        m[qq] = mnew;
        float rs = 0.f;
#pragma unroll
        for (int kk = 0; kk < BN / 32; ++kk)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = exp2_fast(s[kk][qq][r] - mnew);
            s[kk][qq][r] = p;
            rs += p;
          }
        lsum[qq] = lsum[qq] * alpha + rs;
#pragma unroll
        for (int dd = 0; dd < D / 32; ++dd) oacc[qq][dd] *= alpha;
      }

      // O^T += V^T P^T.  Registers 8*half .. 8*half+7 of score tile kk hold
      // keys kk*32 + 16*half + {4*hl + 0..3, 8 + 4*hl + 0..3}; the two
      // transpose reads fetch V at exactly those keys for head-dim column
      // dd*32 + l32.
#pragma unroll
      for (int kk = 0; kk < BN / 32; ++kk) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          bf16x8 pb[QT];
#pragma unroll
          for (int qq = 0; qq < QT; ++qq) pb[qq] = to_bf16x8(s[kk][qq], half);
          const int rowA = kk * 32 + 16 * half + 4 * hl + ((lane & 15) >> 2);
#pragma unroll
          for (int dd = 0; dd < D / 32; ++dd) {
            const int col = dd * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
            const bf16x4 lo = lds_read_tr(Vs + rowA * C::LDW + col);
            const bf16x4 hi = lds_read_tr(Vs + (rowA + 8) * C::LDW + col);
            const bf16x8 a = cat(lo, hi);
#pragma unroll
            for (int qq = 0; qq < QT; ++qq) oacc[qq][dd] = mfma32(a, pb[qq], oacc[qq][dd]);
          }
        }
      }
    }
    if (t + 1 < ntiles) sstore(buf ^ 1);
    __syncthreads();
  }

  // Fold the block partial into the running accumulators.
#pragma unroll
  for (int qq = 0; qq < QT; ++qq) {
    const int qi = qw0 + qq * 32 + l32;
    const float ltot = add_halves(lsum[qq]);
    if (qi < Lq && ltot > 0.f) {
      const float lse_b = (m[qq] + log2f(ltot)) * kLn2;
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
#pragma unroll
      for (int dd = 0; dd < D / 32; ++dd)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = dd * 32 + 8 * g + 4 * hl;
          const f32x4 acc = {oacc[qq][dd][4 * g], oacc[qq][dd][4 * g + 1],
                             oacc[qq][dd][4 * g + 2], oacc[qq][dd][4 * g + 3]};
          f32x4 res = acc * wb;
          if (wa != 0.f) res += *(const f32x4*)(orow + d) * wa;
          *(f32x4*)(orow + d) = res;
        }
      if (hl == 0) *lse_p = lse_new;
    }
  }
}

template <int D, int QT, int BN>
hipError_t launch(const void* q, const void* kv, float* o_acc, float* lse_acc,
                  const ra_launch& a) {
  constexpr int NW = 4;
  using C = FwdCfg<D, QT, BN, NW>;
  const int n_qt = (a.Lq + C::BM - 1) / C::BM;
  const int BH = a.B * a.H;
  const long long grid = (long long)n_qt * BH;
  if (grid <= 0) return hipSuccess;
  const float c2 = a.scale * kLog2e;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, QT, BN, NW>), dim3((unsigned)grid),
                     dim3(C::NT), 0, a.stream, (const bf16*)q, (const bf16*)kv,
                     o_acc, lse_acc, BH, a.Lq, a.Lk, n_qt, a.diag, c2);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const void* q, const void* kv, float* o_acc, float* lse_acc,
                    const ra_launch& a) {
  const bool wide_q = a.q_chunk >= 256;
  const bool wide_k = a.k_chunk >= 64;
  if (wide_q) {
    return wide_k ? launch<D, 2, 64>(q, kv, o_acc, lse_acc, a)
                  : launch<D, 2, 32>(q, kv, o_acc, lse_acc, a);
  }
  return wide_k ? launch<D, 1, 64>(q, kv, o_acc, lse_acc, a)
                : launch<D, 1, 32>(q, kv, o_acc, lse_acc, a);
}

}  // namespace

hipError_t ra_launch_fwd_bf16(const void* q, const void* kv, float* o_acc,
                              float* lse_acc, const ra_launch& a) {
  if (a.D == 128) return launch_d<128>(q, kv, o_acc, lse_acc, a);
  if (a.D == 64) return launch_d<64>(q, kv, o_acc, lse_acc, a);
  return hipErrorInvalidValue;
}
