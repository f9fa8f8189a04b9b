// Backward ring step, bf16 inputs, fp32 accumulation, gfx950 MFMA.
//
// The gradient is that of sum(dO * O) over the member's rows, with O the
// exact attention of the forward share.  For one key/value block, with
// P = exp(scale * Q K^T - lse) recomputed from the saved final LSE (the
// memory-efficient method never keeps P; Blockwise RingAttention keyword
// page, definition) and delta_i = <dO_i, O_i>:
//     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - delta),
//     dQ = scale * dS K,  dK = scale * dS^T Q.
// Two kernels, no atomics, so every result is deterministic:
//   * dq_kernel (query-major): a wave keeps 32 queries and their dO rows in
//     registers, sweeps the key tiles of the block through LDS and
//     accumulates dQ^T = K^T dS^T, reusing the forward's operand layout
//     (S^T = K Q^T, dP^T = V dO^T; K^T from LDS transpose reads);
//   * dkv_kernel (key-major): a wave keeps 32 keys and their values in
//     registers, sweeps the query tiles (Q, dO, lse, delta) through LDS and
//     accumulates dV = P^T dO and dK = dS^T Q, with dO^T and Q^T read
//     transposed from LDS.
// The causal diagonal block masks key j > query i; past blocks are dense.
#include <math.h>

#include "ra_common.h"

using namespace ra;

namespace {

constexpr int kNW = 4;  // waves per workgroup

// ---------------------------------------------------------------- dQ ------
template <int D, int BN>
__global__ __launch_bounds__(kNW * 64, 1) void dq_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ KV,
    const bf16* __restrict__ dO, const float* __restrict__ LSE,
    const float* __restrict__ Delta, float* __restrict__ dQacc, int BH, int Lq,
    int Lk, int n_qt, int diag, float c2, float scale) {
  constexpr int BM = kNW * 32;
  constexpr int LDW = D + 8;
  constexpr int NT = kNW * 64;
  constexpr int PT = BN * D / 8 / NT;
  static_assert(BN * D / 8 % NT == 0, "tile split");
  __shared__ __attribute__((aligned(16))) bf16 smem[2][2][BN * LDW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / n_qt;
  int qt = tile % n_qt;
  if (diag) qt = n_qt - 1 - qt;
  const int q0 = qt * BM;
  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + l32;

  const bf16* Qp = Q + (size_t)bh * Lq * D;
  const bf16* dOp = dO + (size_t)bh * Lq * D;
  const bf16* Kp = KV + (size_t)bh * Lk * D;
  const bf16* Vp = KV + ((size_t)BH + bh) * Lk * D;

  bf16x8 qreg[D / 16], doreg[D / 16];
#pragma unroll
  for (int ds = 0; ds < D / 16; ++ds) {
    if (qi < Lq) {
      qreg[ds] = *(const bf16x8*)(Qp + (size_t)qi * D + ds * 16 + hl * 8);
      doreg[ds] = *(const bf16x8*)(dOp + (size_t)qi * D + ds * 16 + hl * 8);
    } else {
      qreg[ds] = bf16x8{};
      doreg[ds] = bf16x8{};
    }
  }
  // Rows that saw no key (lse = -inf) cannot occur in a causal share, but
  // keep them harmless: their probabilities are forced to zero.
  const float lse_raw = qi < Lq ? LSE[(size_t)bh * Lq + qi] : -INFINITY;
  const bool row_live = lse_raw != -INFINITY;
  const float lse2 = row_live ? lse_raw * kLog2e : 0.f;
  const float delta = qi < Lq ? Delta[(size_t)bh * Lq + qi] : 0.f;

  f32x16 dq[D / 32];
#pragma unroll
  for (int dd = 0; dd < D / 32; ++dd) dq[dd] = f32x16{};

  const int kend = diag ? min(Lk, q0 + BM) : Lk;
  const int ntiles = (kend + BN - 1) / BN;
  const int qw_last = min(qw0 + 32, Lq) - 1;

  bf16x8 pk[PT], pv[PT];
  auto gload = [&](int kt0) {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int c = tid + i * NT;
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      const int key = kt0 + row;
      if (key < Lk) {
        pk[i] = *(const bf16x8*)(Kp + (size_t)key * D + col);
        pv[i] = *(const bf16x8*)(Vp + (size_t)key * D + col);
      } else {
        pk[i] = bf16x8{};
        pv[i] = bf16x8{};
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int c = tid + i * NT;
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      *(bf16x8*)&smem[buf][0][row * LDW + col] = pk[i];
      *(bf16x8*)&smem[buf][1][row * LDW + col] = pv[i];
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
      f32x16 s[BN / 32], dp[BN / 32];
#pragma unroll
      for (int kk = 0; kk < BN / 32; ++kk) {
        s[kk] = f32x16{};
        dp[kk] = f32x16{};
      }
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds)
#pragma unroll
        for (int kk = 0; kk < BN / 32; ++kk) {
          const int off = (kk * 32 + l32) * LDW + ds * 16 + hl * 8;
          s[kk] = mfma32(*(const bf16x8*)(Ks + off), qreg[ds], s[kk]);
          dp[kk] = mfma32(*(const bf16x8*)(Vs + off), doreg[ds], dp[kk]);
        }
      const bool need_mask = (kt0 + BN > Lk) || (diag && kt0 + BN - 1 > qw0);
#pragma unroll
      for (int kk = 0; kk < BN / 32; ++kk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = exp2_fast(s[kk][r] * c2 - lse2);
          if (!row_live) p = 0.f;
          if (need_mask) {
            const int kj = kt0 + kk * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
            if (kj >= Lk || (diag && kj > qi)) p = 0.f;
          }
          s[kk][r] = p * (dp[kk][r] - delta);  // dS^T
        }
      // dQ^T += K^T dS^T (K^T operand by transpose reads, keys permuted to
      // match the dS^T register layout).
#pragma unroll
      for (int kk = 0; kk < BN / 32; ++kk)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const bf16x8 b = to_bf16x8(s[kk], half);
          const int rowA = kk * 32 + 16 * half + 4 * hl + ((lane & 15) >> 2);
#pragma unroll
          for (int dd = 0; dd < D / 32; ++dd) {
            const int col = dd * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
            const bf16x8 a = cat(lds_read_tr(Ks + rowA * LDW + col),
                                 lds_read_tr(Ks + (rowA + 8) * LDW + col));
            dq[dd] = mfma32(a, b, dq[dd]);
          }
        }
    }
    if (t + 1 < ntiles) sstore(buf ^ 1);
    __syncthreads();
  }

  if (qi < Lq) {
    float* row = dQacc + ((size_t)bh * Lq + qi) * D;
#pragma unroll
    for (int dd = 0; dd < D / 32; ++dd)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = dd * 32 + 8 * g + 4 * hl;
        const f32x4 v = {dq[dd][4 * g], dq[dd][4 * g + 1], dq[dd][4 * g + 2], dq[dd][4 * g + 3]};
        *(f32x4*)(row + d) += v * scale;
      }
  }
}

// --------------------------------------------------------------- dK, dV ---
template <int D, int BQ>
__global__ __launch_bounds__(kNW * 64, 1) void dkv_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ KV,
    const bf16* __restrict__ dO, const float* __restrict__ LSE,
    const float* __restrict__ Delta, float* __restrict__ dKV, int BH, int Lq,
    int Lk, int n_kt, int diag, float c2, float scale) {
  constexpr int BK = kNW * 32;  // keys per workgroup
  constexpr int LDW = D + 8;
  constexpr int NT = kNW * 64;
  constexpr int PT = BQ * D / 8 / NT;
  static_assert(BQ * D / 8 % NT == 0, "tile split");
  static_assert(BQ <= NT, "one thread per row of lse / delta");
  __shared__ __attribute__((aligned(16))) bf16 smem[2][2][BQ * LDW];
  __shared__ float s_lse[2][BQ], s_delta[2][BQ];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / n_kt;
  const int k0 = (tile % n_kt) * BK;
  const int kw0 = k0 + wave * 32;
  const int kj = kw0 + l32;  // this lane's key (as the MFMA n index)

  const bf16* Qp = Q + (size_t)bh * Lq * D;
  const bf16* dOp = dO + (size_t)bh * Lq * D;
  const bf16* Kp = KV + (size_t)bh * Lk * D;
  const bf16* Vp = KV + ((size_t)BH + bh) * Lk * D;
  const float* Lp = LSE + (size_t)bh * Lq;
  const float* Dp = Delta + (size_t)bh * Lq;

  bf16x8 kreg[D / 16], vreg[D / 16];
#pragma unroll
  for (int ds = 0; ds < D / 16; ++ds) {
    if (kj < Lk) {
      kreg[ds] = *(const bf16x8*)(Kp + (size_t)kj * D + ds * 16 + hl * 8);
      vreg[ds] = *(const bf16x8*)(Vp + (size_t)kj * D + ds * 16 + hl * 8);
    } else {
      kreg[ds] = bf16x8{};
      vreg[ds] = bf16x8{};
    }
  }
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int dd = 0; dd < D / 32; ++dd) {
    dk[dd] = f32x16{};
    dv[dd] = f32x16{};
  }

  // Under the causal mask only queries at or after the first key matter.
  const int qstart = diag ? (k0 / BQ) * BQ : 0;
  const int ntiles = qstart < Lq ? (Lq - qstart + BQ - 1) / BQ : 0;
  const int kw_last = min(kw0 + 32, Lk) - 1;

  bf16x8 pq[PT], pd[PT];
  float pl = 0.f, pdl = 0.f;
  auto gload = [&](int qt0) {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int c = tid + i * NT;
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      const int q = qt0 + row;
      if (q < Lq) {
        pq[i] = *(const bf16x8*)(Qp + (size_t)q * D + col);
        pd[i] = *(const bf16x8*)(dOp + (size_t)q * D + col);
      } else {
        pq[i] = bf16x8{};
        pd[i] = bf16x8{};
      }
    }
    if (tid < BQ) {
      const int q = qt0 + tid;
      const float l = q < Lq ? Lp[q] : -INFINITY;
      pl = l;
      pdl = q < Lq ? Dp[q] : 0.f;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int c = tid + i * NT;
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      *(bf16x8*)&smem[buf][0][row * LDW + col] = pq[i];
      *(bf16x8*)&smem[buf][1][row * LDW + col] = pd[i];
    }
    if (tid < BQ) {
      // -inf (an empty or out-of-range row) becomes +inf in the exponent
      // offset, so that row's probabilities come out as exactly zero.
      s_lse[buf][tid] = pl == -INFINITY ? INFINITY : pl * kLog2e;
      s_delta[buf][tid] = pdl;
    }
  };

  if (ntiles > 0) {
    gload(qstart);
    sstore(0);
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int qt0 = qstart + t * BQ;
    if (t + 1 < ntiles) gload(qt0 + BQ);
    // skip query tiles that end before this wave's first key
    const bool active = (kw0 < Lk) && (!diag || qt0 + BQ - 1 >= kw0);
    if (active) {
      const bf16* Qs = smem[buf][0];
      const bf16* dOs = smem[buf][1];
      f32x16 s[BQ / 32], dp[BQ / 32];
#pragma unroll
      for (int qs = 0; qs < BQ / 32; ++qs) {
        s[qs] = f32x16{};
        dp[qs] = f32x16{};
      }
      // S = Q K^T and dP = dO V^T: lane holds key l32 and 16 queries.
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds)
#pragma unroll
        for (int qs = 0; qs < BQ / 32; ++qs) {
          const int off = (qs * 32 + l32) * LDW + ds * 16 + hl * 8;
          s[qs] = mfma32(*(const bf16x8*)(Qs + off), kreg[ds], s[qs]);
          dp[qs] = mfma32(*(const bf16x8*)(dOs + off), vreg[ds], dp[qs]);
        }
      const bool need_mask = (kw0 + 31 >= Lk) || (diag && kw_last > qt0);
#pragma unroll
      for (int qs = 0; qs < BQ / 32; ++qs)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ql = qs * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
          float p = exp2_fast(s[qs][r] * c2 - s_lse[buf][ql]);
          if (need_mask && (kj >= Lk || (diag && kj > qt0 + ql))) p = 0.f;
          s[qs][r] = p;                                   // P
          dp[qs][r] = p * (dp[qs][r] - s_delta[buf][ql]);  // dS
        }
      // dV += P^T dO and dK += dS^T Q; the B operands (dO, Q with queries
      // permuted to match the register layout) come from transpose reads.
#pragma unroll
      for (int qs = 0; qs < BQ / 32; ++qs)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const bf16x8 ap = to_bf16x8(s[qs], half);
          const bf16x8 ads = to_bf16x8(dp[qs], half);
          const int rowB = qs * 32 + 16 * half + 4 * hl + ((lane & 15) >> 2);
#pragma unroll
          for (int dd = 0; dd < D / 32; ++dd) {
            const int col = dd * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
            const bf16x8 bdo = cat(lds_read_tr(dOs + rowB * LDW + col),
                                   lds_read_tr(dOs + (rowB + 8) * LDW + col));
            const bf16x8 bq = cat(lds_read_tr(Qs + rowB * LDW + col),
                                  lds_read_tr(Qs + (rowB + 8) * LDW + col));
            dv[dd] = mfma32(ap, bdo, dv[dd]);
            dk[dd] = mfma32(ads, bq, dk[dd]);
          }
        }
    }
    if (t + 1 < ntiles) sstore(buf ^ 1);
    __syncthreads();
  }

  // dK/dV rows: lane holds head-dim column dd*32 + l32 of keys
  // kw0 + 8*(r/4) + 4*hl + r%4.
  float* dKp = dKV + (size_t)bh * Lk * D;
  float* dVp = dKV + ((size_t)BH + bh) * Lk * D;
#pragma unroll
  for (int dd = 0; dd < D / 32; ++dd)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kw0 + 8 * (r >> 2) + 4 * hl + (r & 3);
      if (key < Lk) {
        const size_t off = (size_t)key * D + dd * 32 + l32;
        dKp[off] += dk[dd][r] * scale;
        dVp[off] += dv[dd][r];
      }
    }
}

template <int D>
hipError_t launch_dq(const void* q, const void* kv, const void* dout, const float* lse,
                     const float* delta, float* dq, const ra_launch& a) {
  const int BH = a.B * a.H;
  constexpr int BM = kNW * 32;
  const int n_qt = (a.Lq + BM - 1) / BM;
  if ((long long)n_qt * BH <= 0) return hipSuccess;
  hipLaunchKernelGGL((dq_kernel<D, 64>), dim3(n_qt * BH), dim3(kNW * 64), 0, a.stream,
                     (const bf16*)q, (const bf16*)kv, (const bf16*)dout, lse, delta, dq, BH,
                     a.Lq, a.Lk, n_qt, a.diag, a.scale * kLog2e, a.scale);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dkv(const void* q, const void* kv, const void* dout, const float* lse,
                      const float* delta, float* dkv, const ra_launch& a) {
  const int BH = a.B * a.H;
  constexpr int BK = kNW * 32;
  const int n_kt = (a.Lk + BK - 1) / BK;
  if ((long long)n_kt * BH <= 0) return hipSuccess;
  hipLaunchKernelGGL((dkv_kernel<D, 64>), dim3(n_kt * BH), dim3(kNW * 64), 0, a.stream,
                     (const bf16*)q, (const bf16*)kv, (const bf16*)dout, lse, delta, dkv, BH,
                     a.Lq, a.Lk, n_kt, a.diag, a.scale * kLog2e, a.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t ra_launch_bwd_dq(const void* q, const void* kv, const void* dout,
                            const float* lse, const float* delta, float* dq_acc,
                            const ra_launch& a) {
  if (a.D == 128) return launch_dq<128>(q, kv, dout, lse, delta, dq_acc, a);
  if (a.D == 64) return launch_dq<64>(q, kv, dout, lse, delta, dq_acc, a);
  return hipErrorInvalidValue;
}

hipError_t ra_launch_bwd_dkv(const void* q, const void* kv, const void* dout,
                             const float* lse, const float* delta, float* dkv,
                             const ra_launch& a) {
  if (a.D == 128) return launch_dkv<128>(q, kv, dout, lse, delta, dkv, a);
  if (a.D == 64) return launch_dkv<64>(q, kv, dout, lse, delta, dkv, a);
  return hipErrorInvalidValue;
}
