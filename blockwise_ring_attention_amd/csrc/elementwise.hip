// Memory-bound helpers of the ring share: accumulator initialisation, the
// associative combine of two partials, the final cast, and the backward
// row dot products.  Each is one coalesced pass over its tensors.
#include <math.h>

#include "ra_common.h"

using namespace ra;

namespace {

constexpr int kThreads = 256;

inline unsigned blocks_for(int64_t n, int per_block) {
  int64_t b = (n + per_block - 1) / per_block;
  return (unsigned)(b < 1 ? 1 : b);
}

// (0, -inf): the empty partial.  A fill kernel rather than hipMemset so the
// call can be captured in a HIP graph.
__global__ void init_acc_kernel(f32x4* __restrict__ o, int64_t n4,
                                float* __restrict__ lse, int64_t rows) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
    o[i] = f32x4{};
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows; i += stride)
    lse[i] = -INFINITY;
}

// a <- a (+) b for normalised partials over disjoint key sets (darcstar
// commentary: online softmax is associative).  One thread per 4 columns of
// one row; the row's weights are recomputed by each of its threads.
template <int D>
__global__ void combine_kernel(float* __restrict__ o_a, float* __restrict__ lse_a,
                               const float* __restrict__ o_b,
                               const float* __restrict__ lse_b, int64_t rows) {
  constexpr int TPR = D / 4;  // threads per row
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = g / TPR;
  if (row >= rows) return;
  const int c = (int)(g % TPR) * 4;
  const float la = lse_a[row], lb = lse_b[row];
  if (lb == -INFINITY) return;  // b empty: a unchanged
  f32x4* pa = (f32x4*)(o_a + row * D + c);
  const f32x4 ob = *(const f32x4*)(o_b + row * D + c);
  float lse;
  if (la == -INFINITY) {  // a empty: take b
    *pa = ob;
    lse = lb;
  } else {
    const float mu = fmaxf(la, lb);
    const float wa = expf(la - mu), wb = expf(lb - mu);
    const float z = wa + wb;
    *pa = (*pa * wa + ob * wb) / z;
    lse = mu + logf(z);
  }
  // The threads of one row lie in one wave (TPR divides 64) and all of them
  // load lse_a[row] above, before this store in program order.
  if (c == 0) lse_a[row] = lse;
}

__global__ void finalize_bf16_kernel(const f32x4* __restrict__ in,
                                     bf16x4* __restrict__ out, int64_t n4) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const f32x4 v = in[i];
    out[i] = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  }
}

__global__ void finalize_fp32_kernel(const f32x4* __restrict__ in,
                                     f32x4* __restrict__ out, int64_t n4) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
    out[i] = in[i];
}

// delta[row] = <dO[row], O[row]>: one wave per 4 rows, 16 lanes per row,
// D/16 columns per lane, reduced with cross-lane shuffles.
template <int D, typename T>
__global__ void bwd_prep_kernel(const float* __restrict__ o, const T* __restrict__ dout,
                                float* __restrict__ delta, int64_t rows) {
  constexpr int PER = D / 16;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = g / 16;
  const int sub = (int)(g % 16);
  float acc = 0.f;
  if (row < rows) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = sub * PER + i;
      acc = fmaf(o[row * D + c], (float)dout[row * D + c], acc);
    }
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
  if (row < rows && sub == 0) delta[row] = acc;
}

// acc <- acc + c_0 + c_1 + ... in copy order (n4 float4 per copy): the
// dK/dV copies of the query heads that ran side by side.
__global__ void add_copies_kernel(f32x4* __restrict__ acc, const f32x4* __restrict__ copies,
                                  int ncopies, int64_t n4) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    f32x4 v = acc[i];
    for (int c = 0; c < ncopies; ++c) v += copies[c * n4 + i];
    acc[i] = v;
  }
}

}  // namespace

hipError_t ra_launch_add_copies(float* acc, const float* copies, int ncopies, int64_t n,
                                hipStream_t s) {
  const int64_t n4 = n / 4;  // head_dim is a multiple of 4
  unsigned grid = blocks_for(n4, kThreads);
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(add_copies_kernel, dim3(grid), dim3(kThreads), 0, s, (f32x4*)acc,
                     (const f32x4*)copies, ncopies, n4);
  return hipGetLastError();
}

hipError_t ra_launch_init_acc(float* o_acc, float* lse_acc, int64_t rows, int D,
                              hipStream_t s) {
  const int64_t n4 = rows * D / 4;
  const int64_t work = n4 > rows ? n4 : rows;
  unsigned grid = blocks_for(work, kThreads);
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(init_acc_kernel, dim3(grid), dim3(kThreads), 0, s,
                     (f32x4*)o_acc, n4, lse_acc, rows);
  return hipGetLastError();
}

hipError_t ra_launch_combine(float* o_a, float* lse_a, const float* o_b,
                             const float* lse_b, int64_t rows, int D,
                             hipStream_t s) {
  const int64_t threads = rows * (D / 4);
  if (D == 128)
    hipLaunchKernelGGL(combine_kernel<128>, dim3(blocks_for(threads, kThreads)),
                       dim3(kThreads), 0, s, o_a, lse_a, o_b, lse_b, rows);
  else if (D == 64)
    hipLaunchKernelGGL(combine_kernel<64>, dim3(blocks_for(threads, kThreads)),
                       dim3(kThreads), 0, s, o_a, lse_a, o_b, lse_b, rows);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t ra_launch_finalize(const float* acc, void* out, int out_dtype,
                              int64_t n, hipStream_t s) {
  const int64_t n4 = n / 4;  // head_dim is a multiple of 4
  unsigned grid = blocks_for(n4, kThreads);
  if (grid > 65536) grid = 65536;
  if (out_dtype == 0)
    hipLaunchKernelGGL(finalize_bf16_kernel, dim3(grid), dim3(kThreads), 0, s,
                       (const f32x4*)acc, (bf16x4*)out, n4);
  else
    hipLaunchKernelGGL(finalize_fp32_kernel, dim3(grid), dim3(kThreads), 0, s,
                       (const f32x4*)acc, (f32x4*)out, n4);
  return hipGetLastError();
}

hipError_t ra_launch_bwd_prep(const float* o, const void* dout, int dtype,
                              float* delta, int64_t rows, int D, hipStream_t s) {
  const unsigned grid = blocks_for(rows * 16, kThreads);
#define RA_PREP(DD, T)                                                          \
  hipLaunchKernelGGL((bwd_prep_kernel<DD, T>), dim3(grid), dim3(kThreads), 0, s, \
                     o, (const T*)dout, delta, rows)
  if (D == 128 && dtype == 0) RA_PREP(128, bf16);
  else if (D == 128) RA_PREP(128, float);
  else if (D == 64 && dtype == 0) RA_PREP(64, bf16);
  else if (D == 64) RA_PREP(64, float);
  else return hipErrorInvalidValue;
#undef RA_PREP
  return hipGetLastError();
}
