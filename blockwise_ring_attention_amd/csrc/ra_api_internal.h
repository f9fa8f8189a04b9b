// Host-side helpers shared by the C ABI and the ring emulator.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ring_attn.h"

// Validated, resolved shape of one call.
struct ra_shape {
  int B, H, Hkv, Lq, Lk, D, dtype, elem;  // Hkv divides H
  float scale;
  int64_t bh, q_rows, kv_rows;  // bh = B*H; kv_rows = B*Hkv*Lk
};

int ra_fail(int code, const char* fmt, ...);
int ra_hip_fail(hipError_t e, const char* what);
int ra_check_dims(const ra_dims* d, ra_shape* s);
int ra_check_ring(int rank, int step, int size, int causal, int q_chunk, int k_chunk,
                  const ra_shape& s);
int ra_block_of_step(int rank, int step, int size);
int ra_check_fwd_buffers(const void* q, const void* kv, const float* o_acc,
                         const float* lse_acc, const ra_shape& s);
int ra_check_bwd_buffers(const void* q, const void* kv, const void* dout,
                         const float* lse, const float* delta, const float* dq,
                         const float* dkv, const ra_shape& s);
// Attend to block kb and fold (forward) / accumulate gradients (backward).
// A block in the causal future, an empty block or an empty query set is a
// no-op.  Arguments are assumed validated.
int ra_fwd_block(const void* q, const void* kv, int kb, int rank, int causal,
                 int q_chunk, int k_chunk, float* o_acc, float* lse_acc,
                 const ra_shape& s, hipStream_t stream);
// ws: (nsplit - 1) fp32 copies of dkv, or nullptr with nsplit == 1.
int ra_bwd_block(const void* q, const void* kv, const void* dout, const float* lse,
                 const float* delta, int kb, int rank, int causal, int q_chunk,
                 int k_chunk, float* dq_acc, float* dkv, float* ws, int nsplit,
                 const ra_shape& s, hipStream_t stream);
// Query heads of a group whose dK/dV run side by side, for about one
// workgroup per compute unit (1 when every head has its own key/value head).
int ra_bwd_dkv_splits(const ra_shape& s);
// Copies a backward call can use from a workspace of work_bytes (validated:
// sign, NULL, 16-byte alignment, no overlap with the nother given buffers).
int ra_bwd_ws_plan(const ra_shape& s, const void* work, int64_t work_bytes,
                   const void* const* other, const size_t* othersz, int nother, int* nsplit);
