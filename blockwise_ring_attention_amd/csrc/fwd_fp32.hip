// Forward ring step for fp32 inputs, computed in fp32 on the vector ALUs.
//
// Same method as the bf16 path (blockwise pass over one key/value block,
// online softmax, fold into the running accumulators; Ring Attention keyword
// page, definition; darcstar commentary), without any rounding to bf16, for
// callers that need fp32 accuracy.  One thread owns one query row; key/value
// tiles of BN keys are staged in LDS and read as broadcasts.  Scores are
// formed for a whole tile before the running max is updated, so the
// accumulator is rescaled once per tile.
#include <math.h>

#include "ra_common.h"

using namespace ra;

namespace {

constexpr int kRows = 64;  // query rows per workgroup (one wave)

template <int D, int BN>
__global__ __launch_bounds__(kRows) void fwd_fp32_kernel(
    const float* __restrict__ Q, const float* __restrict__ KV,
    float* __restrict__ Oacc, float* __restrict__ LSEacc, int BH, int H, int G, int Lq,
    int Lk, int n_qt, int diag, float c2) {
  __shared__ float ks[BN][D];
  __shared__ float vs[BN][D];
  const int lane = threadIdx.x;
  const int bh = blockIdx.x / n_qt;
  const int q0 = (blockIdx.x % n_qt) * kRows;
  const int qi = q0 + lane;
  // Groups of G query heads share one key/value head.
  const int kvbh = (bh / H) * (H / G) + (bh % H) / G;
  const float* Qp = Q + (size_t)bh * Lq * D;
  const float* Kp = KV + (size_t)kvbh * Lk * D;
  const float* Vp = KV + ((size_t)(BH / G) + kvbh) * Lk * D;

  float qr[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qr[d] = qi < Lq ? Qp[(size_t)qi * D + d] * c2 : 0.f;
    acc[d] = 0.f;
  }
  float m = kNegBig, l = 0.f;
  const int kend = diag == 1 ? min(Lk, q0 + kRows) : Lk;  // 2: no skipping

  for (int t0 = 0; t0 < kend; t0 += BN) {
    __syncthreads();
    for (int e = lane; e < BN * D; e += kRows) {
      const int j = e / D, d = e % D, key = t0 + j;
      ks[j][d] = key < Lk ? Kp[(size_t)key * D + d] : 0.f;
      vs[j][d] = key < Lk ? Vp[(size_t)key * D + d] : 0.f;
    }
    __syncthreads();
    float s[BN];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      float x = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) x = fmaf(qr[d], ks[j][d], x);
      const int key = t0 + j;
      if (key >= Lk || (diag && key > qi)) x = -INFINITY;
      s[j] = x;
      mx = fmaxf(mx, x);
    }
    const float mnew = fmaxf(m, mx);
    const float alpha = exp2f(m - mnew);
    m = mnew;
    l *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      const float p = exp2f(s[j] - mnew);
      l += p;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vs[j][d], acc[d]);
    }
  }

  if (qi < Lq && l > 0.f) {
    const float lse_b = (m + log2f(l)) * kLn2;
    float* lse_p = LSEacc + (size_t)bh * Lq + qi;
    const float lse_a = *lse_p;
    const float inv = 1.f / l;
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
    for (int d = 0; d < D; ++d) {
      float r = acc[d] * wb;
      if (wa != 0.f) r = fmaf(orow[d], wa, r);
      orow[d] = r;
    }
    *lse_p = lse_new;
  }
}

template <int D, int BN>
hipError_t launch(const float* q, const float* kv, float* o, float* lse,
                  const ra_launch& a) {
  const int n_qt = (a.Lq + kRows - 1) / kRows;
  const int BH = a.B * a.H;
  const long long grid = (long long)n_qt * BH;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_fp32_kernel<D, BN>), dim3((unsigned)grid), dim3(kRows),
                     0, a.stream, q, kv, o, lse, BH, a.H, a.H / a.Hkv, a.Lq, a.Lk, n_qt, a.diag,
                     a.scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t ra_launch_fwd_fp32(const float* q, const float* kv, float* o_acc,
                              float* lse_acc, const ra_launch& a) {
  if (a.D == 64) return launch<64, 32>(q, kv, o_acc, lse_acc, a);
  if (a.D == 128) return launch<128, 16>(q, kv, o_acc, lse_acc, a);
  return hipErrorInvalidValue;
}
