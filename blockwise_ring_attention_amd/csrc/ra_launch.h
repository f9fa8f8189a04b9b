// Host-side launchers of the library's kernels (defined in the .hip sources)
// and the launch descriptor they share.  Kept apart from the device helpers
// in ra_common.h so that adding a launcher leaves those untouched.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

struct ra_launch {
  int B, H, Lq, Lk, D;
  int Hkv;           // key/value heads (divides H)
  float scale;       // resolved (never 0)
  int diag;          // causal diagonal block: mask key j > query i (local); 1 skips
                     // tiles wholly above the diagonal, 2 computes them masked
  int q_chunk, k_chunk;
  hipStream_t stream;
};

hipError_t ra_launch_fwd_bf16(const void* q, const void* kv, float* o_acc,
                              float* lse_acc, const ra_launch& a);
// Decode-shaped forward.  ra_launch_decode_split attends the (H / Hkv) * Lq
// <= 64 rows of each key/value head group to `splits` key splits of k_chunk
// keys, writing o_part [splits, B, H, Lq, d] / lse_part [splits, B, H, Lq];
// ra_launch_decode_fold folds them, in split order, into (o_acc, lse_acc).
hipError_t ra_launch_decode_split(const void* q, const void* kv, float* o_part, float* lse_part,
                                  int k_chunk, int splits, const ra_launch& a);
// This device's copy of the decode scratch array (RA_DECODE_SCRATCH_BYTES).
hipError_t ra_decode_scratch(void** ptr, size_t* bytes);
hipError_t ra_launch_decode_fold(float* o_acc, float* lse_acc, const float* o_part,
                                 const float* lse_part, int64_t rows, int D, int splits,
                                 hipStream_t stream);
// Blockwise feedforward products (bf16, fp32 accumulation):
//   ffn_up:   hidden[r][f] = bf16(GELU(sum_c x[r][c] w1[f][c]))   rows x d_ff
//   ffn_down: out[r][c]    = bf16(sum_f hidden[r][f] w2[c][f])    rows x d_model
// d_model and d_ff multiples of 256, rows >= 1.
hipError_t ra_launch_ffn_up(const void* x, const void* w1, void* hidden, int rows, int d_model,
                            int d_ff, hipStream_t stream);
hipError_t ra_launch_ffn_down(const void* hidden, const void* w2, void* out, int rows,
                              int d_model, int d_ff, hipStream_t stream);
// Feedforward backward building blocks (bf16 in, fp32 accumulation):
//   gemm_tn:       c[i][j] (=|+=) sum_k a[i][k] b[j][k]; a [m x k], b [n x k];
//                  c bf16 [m x n] (store) or fp32 (accumulate_f32 != 0);
//                  n % 256 == 0, k % 64 == 0, m >= 1
//   transpose_pad: out [cols x rows_pad] = in [rows x cols] transposed, rows
//                  rows .. rows_pad-1 of the result zero; cols, rows_pad % 64 == 0
//   gelu_grad_transpose: per element h = GELU(z), g <- g * GELU'(z) (in
//                  place, [rows x cols]), and g, h written transposed into
//                  gt, ht [cols x rows_pad] (rows .. rows_pad-1 zero)
hipError_t ra_launch_gemm_tn(const void* a, const void* b, void* c, int m, int n, int k,
                             int accumulate_f32, hipStream_t stream);
hipError_t ra_launch_transpose_pad(const void* in, void* out, int rows, int cols, int rows_pad,
                                   hipStream_t stream);
hipError_t ra_launch_gelu_grad_transpose(const void* z, void* g, void* gt, void* ht, int rows,
                                         int cols, int rows_pad, hipStream_t stream);
hipError_t ra_launch_fwd_fp32(const float* q, const float* kv, float* o_acc,
                              float* lse_acc, const ra_launch& a);
hipError_t ra_launch_init_acc(float* o_acc, float* lse_acc, int64_t rows,
                              int D, hipStream_t s);
hipError_t ra_launch_combine(float* o_a, float* lse_a, const float* o_b,
                             const float* lse_b, int64_t rows, int D,
                             hipStream_t s);
hipError_t ra_launch_finalize(const float* acc, void* out, int out_dtype,
                              int64_t n, hipStream_t s);
hipError_t ra_launch_bwd_prep(const float* o, const void* dout, int dtype,
                              float* delta, int64_t rows, int D, hipStream_t s);
hipError_t ra_launch_bwd_dq(const void* q, const void* kv, const void* dout,
                            const float* lse, const float* delta, float* dq_acc,
                            const ra_launch& a);
// dK/dV over the G query heads of each key/value head, nsplit heads side by
// side per launch; nsplit > 1 needs ws, (nsplit - 1) fp32 copies of dkv.
hipError_t ra_launch_bwd_dkv(const void* q, const void* kv, const void* dout,
                             const float* lse, const float* delta, float* dkv, float* ws,
                             int nsplit, const ra_launch& a);
// acc[i] += copies[0][i] + copies[1][i] + ... (in copy order), n floats per copy.
hipError_t ra_launch_add_copies(float* acc, const float* copies, int ncopies, int64_t n,
                                hipStream_t s);
