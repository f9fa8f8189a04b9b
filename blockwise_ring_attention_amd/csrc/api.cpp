// C ABI of the ring-attention library: argument validation, the ring
// schedule (which block a member holds at a step, and whether the causal
// mask hides it), and kernel dispatch.  No exception crosses this boundary
// and nothing here allocates device memory.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "ra_api_internal.h"
#include "ra_launch.h"
#include "ring_attn.h"

namespace {

thread_local std::string g_last_error;

// ---- kernel timing: event pairs around launches, kept until read ---------
enum Kind {
  kFwdBf16 = 0, kFwdFp32, kBwdDq, kBwdDkv, kDecode, kDecodeFold, kFfnUp, kFfnDown,
  kFfnBwdGemm, kFfnBwdAux, kKinds
};
const char* const kKindNames[kKinds] = {"fwd_bf16",   "fwd_fp32",    "bwd_dq",       "bwd_dkv",
                                        "fwd_decode", "decode_fold", "ffn_up",       "ffn_down",
                                        "ffn_bwd_gemm", "ffn_bwd_aux"};

struct TimingRec {
  int kind;
  hipEvent_t start, stop;
};

std::mutex g_tmu;
bool g_timing = false;
std::vector<TimingRec> g_recs;
std::vector<hipEvent_t> g_spare;

hipEvent_t take_event() {  // caller holds g_tmu
  if (!g_spare.empty()) {
    hipEvent_t e = g_spare.back();
    g_spare.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Brackets one kernel launch when timing is on; a no-op otherwise.
class Timed {
 public:
  Timed(int kind, hipStream_t s) : kind_(kind), s_(s) {
    std::lock_guard<std::mutex> g(g_tmu);
    if (!g_timing) return;
    start_ = take_event();
    if (start_ && hipEventRecord(start_, s_) != hipSuccess) {
      g_spare.push_back(start_);
      start_ = nullptr;
    }
  }
  void done() {
    if (!start_) return;
    std::lock_guard<std::mutex> g(g_tmu);
    hipEvent_t stop = take_event();
    if (stop && hipEventRecord(stop, s_) == hipSuccess) {
      g_recs.push_back({kind_, start_, stop});
    } else {
      g_spare.push_back(start_);
      if (stop) g_spare.push_back(stop);
    }
    start_ = nullptr;
  }

 private:
  int kind_;
  hipStream_t s_;
  hipEvent_t start_ = nullptr;
};

}  // namespace

int ra_fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ra_hip_fail(hipError_t e, const char* what) {
  return ra_fail(RA_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

static bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const char* pa = (const char*)a;
  const char* pb = (const char*)b;
  return pa < pb + nb && pb < pa + na;
}

int ra_check_dims(const ra_dims* d, ra_shape* s) {
  if (!d) return ra_fail(RA_ERR_INVALID, "dims is NULL");
  if (d->batch < 0 || d->heads < 0 || d->q_len < 0 || d->kv_len < 0)
    return ra_fail(RA_ERR_INVALID, "negative size in dims (B=%d H=%d Lq=%d Lk=%d)",
                   d->batch, d->heads, d->q_len, d->kv_len);
  if (d->head_dim != 64 && d->head_dim != 128)
    return ra_fail(RA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", d->head_dim);
  if (d->dtype != RA_BF16 && d->dtype != RA_FP32)
    return ra_fail(RA_ERR_UNSUPPORTED, "dtype %d not supported", d->dtype);
  if (!isfinite(d->scale) || d->scale < 0.f)
    return ra_fail(RA_ERR_INVALID, "scale must be finite and positive (0 = default)");
  const int hkv = d->kv_heads != 0 ? d->kv_heads : d->heads;
  if (hkv < 0 || (d->heads > 0 && (hkv == 0 || d->heads % hkv != 0)))
    return ra_fail(RA_ERR_INVALID, "kv_heads %d must divide heads %d (0 = heads)",
                   d->kv_heads, d->heads);
  s->B = d->batch;
  s->H = d->heads;
  s->Hkv = hkv;
  s->Lq = d->q_len;
  s->Lk = d->kv_len;
  s->D = d->head_dim;
  s->dtype = d->dtype;
  s->elem = d->dtype == RA_BF16 ? 2 : 4;
  s->scale = d->scale != 0.f ? d->scale : 1.0f / sqrtf((float)d->head_dim);
  s->bh = (int64_t)s->B * s->H;
  s->q_rows = s->bh * s->Lq;
  s->kv_rows = (int64_t)s->B * s->Hkv * s->Lk;
  // every row index handled by a kernel must fit a 32-bit grid
  if (s->q_rows > (int64_t)1 << 40 || s->kv_rows > (int64_t)1 << 40 ||
      (s->bh > 0 && (s->Lq > (1 << 30) || s->Lk > (1 << 30))))
    return ra_fail(RA_ERR_INVALID, "problem too large");
  if (s->bh * ((int64_t)s->Lq + 127) / 128 > 0x7fffffffLL ||
      s->bh * ((int64_t)s->Lk + 127) / 128 > 0x7fffffffLL)
    return ra_fail(RA_ERR_INVALID, "problem too large for one launch");
  return RA_OK;
}

int ra_check_ring(int rank, int step, int size, int causal, int q_chunk,
                  int k_chunk, const ra_shape& s) {
  if (size < 1) return ra_fail(RA_ERR_INVALID, "ring_size %d < 1", size);
  if (rank < 0 || rank >= size)
    return ra_fail(RA_ERR_INVALID, "ring_rank %d outside [0, %d)", rank, size);
  if (step < 0 || step >= size)
    return ra_fail(RA_ERR_INVALID, "ring_step %d outside [0, %d)", step, size);
  if (q_chunk < 1 || k_chunk < 1)
    return ra_fail(RA_ERR_INVALID, "q_chunk %d / k_chunk %d must be >= 1", q_chunk, k_chunk);
  if (causal && s.Lq != s.Lk)
    return ra_fail(RA_ERR_INVALID,
                   "causal ring step needs equal blocks (Lq %d != Lk %d)", s.Lq, s.Lk);
  return RA_OK;
}

int ra_block_of_step(int rank, int step, int size) {
  int kb = (rank - step) % size;
  return kb < 0 ? kb + size : kb;
}

// Diagonal-block mode: 1 skips the tiles wholly above the diagonal; with the
// environment variable RA_NO_SKIP set (to anything but "0") every tile is
// computed and masked instead, a debug switch that shows the skip changes no
// result.  Read at every call, so a process can switch it.
static int ra_diag_mode() {
  const char* e = getenv("RA_NO_SKIP");
  return (e && *e && strcmp(e, "0") != 0) ? 2 : 1;
}

int ra_fwd_block(const void* q, const void* kv, int kb, int rank, int causal,
                 int q_chunk, int k_chunk, float* o_acc, float* lse_acc,
                 const ra_shape& s, hipStream_t stream) {
  if (s.q_rows == 0 || s.Lk == 0) return RA_OK;  // empty block: identity
  if (causal && kb > rank) return RA_OK;         // entirely in the future
  ra_launch L{s.B, s.H, s.Lq, s.Lk, s.D, s.Hkv, s.scale, causal && kb == rank ? ra_diag_mode() : 0,
              q_chunk, k_chunk, stream};
  Timed t(s.dtype == RA_BF16 ? kFwdBf16 : kFwdFp32, stream);
  hipError_t e = s.dtype == RA_BF16
                     ? ra_launch_fwd_bf16(q, kv, o_acc, lse_acc, L)
                     : ra_launch_fwd_fp32((const float*)q, (const float*)kv, o_acc, lse_acc, L);
  t.done();
  return e == hipSuccess ? RA_OK : ra_hip_fail(e, "forward kernel launch");
}

int ra_bwd_dkv_splits(const ra_shape& s) {
  const int G = s.Hkv > 0 ? s.H / s.Hkv : 1;
  const int64_t wgs = (int64_t)s.B * s.Hkv * ((s.Lk + 127) / 128);  // 128 keys per workgroup
  int S = 1;
  while (S < G && wgs * S < 256) S *= 2;  // about one workgroup per compute unit
  return S < G ? S : G;
}

int ra_bwd_ws_plan(const ra_shape& s, const void* work, int64_t work_bytes,
                   const void* const* other, const size_t* othersz, int nother, int* nsplit) {
  *nsplit = 1;
  if (work_bytes < 0)
    return ra_fail(RA_ERR_INVALID, "work_bytes %lld is negative", (long long)work_bytes);
  if (work_bytes > 0 && !work) return ra_fail(RA_ERR_INVALID, "NULL workspace");
  // As many dK/dV copies as the workspace holds, up to the preferred count.
  const int64_t copyb = (int64_t)2 * s.kv_rows * s.D * 4;
  if (copyb == 0) return RA_OK;
  const int n = std::min<int64_t>(ra_bwd_dkv_splits(s), 1 + work_bytes / copyb);
  if (n > 1) {
    if ((uintptr_t)work % 16 != 0)
      return ra_fail(RA_ERR_INVALID, "workspace must be 16-byte aligned");
    const size_t wb = (size_t)(n - 1) * (size_t)copyb;
    for (int i = 0; i < nother; ++i)
      if (overlaps(work, wb, other[i], othersz[i]))
        return ra_fail(RA_ERR_INVALID, "the workspace overlaps an input or an output");
  }
  *nsplit = n;
  return RA_OK;
}

int ra_bwd_block(const void* q, const void* kv, const void* dout, const float* lse,
                 const float* delta, int kb, int rank, int causal, int q_chunk,
                 int k_chunk, float* dq_acc, float* dkv, float* ws, int nsplit,
                 const ra_shape& s, hipStream_t stream) {
  if (s.q_rows == 0 || s.Lk == 0) return RA_OK;
  if (causal && kb > rank) return RA_OK;
  ra_launch L{s.B, s.H, s.Lq, s.Lk, s.D, s.Hkv, s.scale, causal && kb == rank ? ra_diag_mode() : 0,
              q_chunk, k_chunk, stream};
  Timed tq(kBwdDq, stream);
  hipError_t e = ra_launch_bwd_dq(q, kv, dout, lse, delta, dq_acc, L);
  tq.done();
  if (e != hipSuccess) return ra_hip_fail(e, "backward dQ kernel launch");
  Timed tkv(kBwdDkv, stream);
  e = ra_launch_bwd_dkv(q, kv, dout, lse, delta, dkv, ws, nsplit, L);
  tkv.done();
  return e == hipSuccess ? RA_OK : ra_hip_fail(e, "backward dK/dV kernel launch");
}

int ra_check_fwd_buffers(const void* q, const void* kv, const float* o_acc,
                         const float* lse_acc, const ra_shape& s) {
  if (s.q_rows == 0) return RA_OK;
  if (!q || !o_acc || !lse_acc || (s.Lk > 0 && !kv))
    return ra_fail(RA_ERR_INVALID, "NULL tensor pointer");
  const size_t qb = (size_t)s.q_rows * s.D * s.elem;
  const size_t kvb = (size_t)2 * s.kv_rows * s.D * s.elem;
  const size_t ob = (size_t)s.q_rows * s.D * 4;
  const size_t lb = (size_t)s.q_rows * 4;
  if (overlaps(o_acc, ob, q, qb) || overlaps(o_acc, ob, kv, kvb) ||
      overlaps(lse_acc, lb, q, qb) || overlaps(lse_acc, lb, kv, kvb) ||
      overlaps(lse_acc, lb, o_acc, ob))
    return ra_fail(RA_ERR_INVALID, "accumulators overlap an input or each other");
  return RA_OK;
}

int ra_check_bwd_buffers(const void* q, const void* kv, const void* dout,
                         const float* lse, const float* delta, const float* dq,
                         const float* dkv, const ra_shape& s) {
  if (s.q_rows == 0) return RA_OK;
  if (!q || !dout || !lse || !delta || !dq || (s.Lk > 0 && (!kv || !dkv)))
    return ra_fail(RA_ERR_INVALID, "NULL tensor pointer");
  const size_t qb = (size_t)s.q_rows * s.D * s.elem;
  const size_t kvb = (size_t)2 * s.kv_rows * s.D * s.elem;
  const size_t dqb = (size_t)s.q_rows * s.D * 4;
  const size_t dkvb = (size_t)2 * s.kv_rows * s.D * 4;
  const size_t lb = (size_t)s.q_rows * 4;
  const void* ins[5] = {q, kv, dout, lse, delta};
  const size_t insz[5] = {qb, kvb, qb, lb, lb};
  for (int i = 0; i < 5; ++i)
    if (overlaps(dq, dqb, ins[i], insz[i]) || overlaps(dkv, dkvb, ins[i], insz[i]))
      return ra_fail(RA_ERR_INVALID, "a gradient output overlaps an input");
  if (overlaps(dq, dqb, dkv, dkvb))
    return ra_fail(RA_ERR_INVALID, "dq_acc overlaps dkv_io");
  return RA_OK;
}

namespace {

// Decode-shaped calls: rows of one key/value head group and split limits.
constexpr int kDecodeMaxRows = 64;
constexpr int kDecodeMaxSplits = 1 << 16;
constexpr int kDecodeTileKeys = 128;
constexpr int kDecodeMaxChunkKeys = 8192;

int ra_check_decode(const ra_shape& s) {
  if (s.dtype != RA_BF16)
    return ra_fail(RA_ERR_UNSUPPORTED, "decode step is implemented for bf16 inputs only");
  if (s.q_rows == 0) return RA_OK;  // (Hkv may be 0 when H is)
  const int64_t rows = (int64_t)(s.H / s.Hkv) * s.Lq;
  if (rows > kDecodeMaxRows)
    return ra_fail(RA_ERR_UNSUPPORTED,
                   "decode step takes at most %d rows per key/value head group "
                   "((heads / kv_heads) * q_len = %lld)",
                   kDecodeMaxRows, (long long)rows);
  return RA_OK;
}

// Feedforward shapes shared by the forward and backward entry points.
int ra_check_ffn(int64_t rows, int d_model, int d_ff, int chunk_rows) {
  if (rows < 0 || rows > 0x7fffffffLL)
    return ra_fail(RA_ERR_INVALID, "rows %lld outside [0, 2^31)", (long long)rows);
  if (d_model < 256 || d_ff < 256 || d_model % 256 != 0 || d_ff % 256 != 0)
    return ra_fail(RA_ERR_UNSUPPORTED, "d_model %d and d_ff %d must be positive multiples of 256",
                   d_model, d_ff);
  if (chunk_rows < 1) return ra_fail(RA_ERR_INVALID, "chunk_rows %d must be >= 1", chunk_rows);
  const int64_t chunk = std::min<int64_t>(chunk_rows, std::max<int64_t>(rows, 1));
  // Largest grids: a product over a chunk, the weight-gradient products
  // (d_ff x d_model tiles of 256) and the weight transposes (tiles of 64).
  if (((chunk + 255) / 256) * (int64_t)(std::max(d_model, d_ff) / 256) > 0x7fffffffLL ||
      (int64_t)(d_ff / 64) * (d_model / 64) > 0x7fffffffLL)
    return ra_fail(RA_ERR_INVALID, "problem too large for one launch");
  return RA_OK;
}

// Backward workspace, in order (each part 256-byte aligned): W1^T [dm x dff],
// W2^T [dff x dm], Z and G (the hidden gradient) [c x dff], and the
// zero-padded transposes x^T, dout^T [dm x cp], G^T, H^T [dff x cp], with
// c = min(rows, chunk_rows) and cp = c rounded up to a multiple of 64.
struct FfnBwdWork {
  size_t w1t, w2t, z, g, xt, dot, gt, ht, total;
};
FfnBwdWork ra_ffn_bwd_layout(int64_t rows, int d_model, int d_ff, int chunk_rows) {
  const int64_t c = std::min<int64_t>(chunk_rows, std::max<int64_t>(rows, 1));
  const int64_t cp = (c + 63) / 64 * 64;
  const size_t dm = (size_t)d_model, df = (size_t)d_ff;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  FfnBwdWork w;
  size_t off = 0;
  w.w1t = off; off += up(dm * df * 2);
  w.w2t = off; off += up(dm * df * 2);
  w.z = off;   off += up((size_t)c * df * 2);
  w.g = off;   off += up((size_t)c * df * 2);
  w.xt = off;  off += up(dm * (size_t)cp * 2);
  w.dot = off; off += up(dm * (size_t)cp * 2);
  w.gt = off;  off += up(df * (size_t)cp * 2);
  w.ht = off;  off += up(df * (size_t)cp * 2);
  w.total = off;
  return w;
}

int ra_decode_splits(const ra_shape& s, int k_chunk) {
  return (int)(((int64_t)s.Lk + k_chunk - 1) / k_chunk);
}

// Validation shared by the two decode entry points.  On RA_OK, *S is the
// number of key splits, or 0 when the call has nothing to attend (the
// accumulators are then left as they are).
int ra_check_decode_call(const void* q, const void* kv_block, int k_chunk, const float* o_acc,
                         const float* lse_acc, const ra_dims* dims, ra_shape* s, int* S) {
  *S = 0;
  int rc = ra_check_dims(dims, s);
  if (rc) return rc;
  if ((rc = ra_check_decode(*s))) return rc;
  if (k_chunk < 1) return ra_fail(RA_ERR_INVALID, "k_chunk %d must be >= 1", k_chunk);
  if ((rc = ra_check_fwd_buffers(q, kv_block, o_acc, lse_acc, *s))) return rc;
  if (s->q_rows == 0 || s->Lk == 0) return RA_OK;  // nothing to attend: identity
  const int n = ra_decode_splits(*s, k_chunk);
  if (n > kDecodeMaxSplits)
    return ra_fail(RA_ERR_INVALID, "k_chunk %d gives %d key splits (at most %d)", k_chunk, n,
                   kDecodeMaxSplits);
  if ((int64_t)s->B * s->Hkv * n > 0x7fffffffLL || s->q_rows * (s->D / 4) / 256 >= 0x7fffffffLL)
    return ra_fail(RA_ERR_INVALID, "problem too large for one launch");
  *S = n;
  return RA_OK;
}

// The split kernel and the fold, with the partials in o_part / lse_part.
int ra_decode_step(const void* q, const void* kv_block, int k_chunk, int S, float* o_acc,
                   float* lse_acc, float* o_part, float* lse_part, const ra_shape& s,
                   hipStream_t stream) {
  ra_launch L{s.B, s.H, s.Lq, s.Lk, s.D, s.Hkv, s.scale, 0, 0, k_chunk, stream};
  Timed t(kDecode, L.stream);
  hipError_t e = ra_launch_decode_split(q, kv_block, o_part, lse_part, k_chunk, S, L);
  t.done();
  if (e != hipSuccess) return ra_hip_fail(e, "decode kernel launch");
  Timed tf(kDecodeFold, L.stream);
  e = ra_launch_decode_fold(o_acc, lse_acc, o_part, lse_part, s.q_rows, s.D, S, L.stream);
  tf.done();
  return e == hipSuccess ? RA_OK : ra_hip_fail(e, "decode fold kernel launch");
}

}  // namespace

extern "C" {

int ring_attn_version(void) { return 204; }

int ring_attn_timing_enable(int on) {
  std::lock_guard<std::mutex> g(g_tmu);
  if (on) {
    for (const TimingRec& r : g_recs) {
      (void)hipEventSynchronize(r.stop);
      g_spare.push_back(r.start);
      g_spare.push_back(r.stop);
    }
    g_recs.clear();
  }
  g_timing = on != 0;
  return RA_OK;
}

int ring_attn_timing_read(const char* name, int* launches, double* total_ms) {
  if (!name || !launches || !total_ms) return ra_fail(RA_ERR_INVALID, "NULL argument");
  int kind = -1;
  for (int k = 0; k < kKinds; ++k)
    if (std::string(name) == kKindNames[k]) kind = k;
  if (kind < 0) return ra_fail(RA_ERR_INVALID, "unknown kernel family '%s'", name);
  std::lock_guard<std::mutex> g(g_tmu);
  int n = 0;
  double total = 0.0;
  for (const TimingRec& r : g_recs) {
    if (r.kind != kind) continue;
    hipError_t e = hipEventSynchronize(r.stop);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) return ra_hip_fail(e, "reading kernel timing events");
    ++n;
    total += ms;
  }
  *launches = n;
  *total_ms = total;
  return RA_OK;
}

const char* ring_attn_last_error(void) { return g_last_error.c_str(); }

int ring_attn_init_acc(float* o_acc, float* lse_acc, const ra_dims* dims, void* stream) {
  ra_shape s;
  int rc = ra_check_dims(dims, &s);
  if (rc) return rc;
  if (s.q_rows == 0) return RA_OK;
  if (!o_acc || !lse_acc) return ra_fail(RA_ERR_INVALID, "NULL accumulator");
  if (overlaps(o_acc, (size_t)s.q_rows * s.D * 4, lse_acc, (size_t)s.q_rows * 4))
    return ra_fail(RA_ERR_INVALID, "o_acc overlaps lse_acc");
  hipError_t e = ra_launch_init_acc(o_acc, lse_acc, s.q_rows, s.D, (hipStream_t)stream);
  return e == hipSuccess ? RA_OK : ra_hip_fail(e, "init kernel launch");
}

int ring_attn_fwd(const void* q, const void* kv_block, int ring_rank, int ring_step,
                  int ring_size, int causal, int q_chunk, int k_chunk, float* o_acc,
                  float* lse_acc, const ra_dims* dims, void* stream) {
  ra_shape s;
  int rc = ra_check_dims(dims, &s);
  if (rc) return rc;
  if ((rc = ra_check_ring(ring_rank, ring_step, ring_size, causal, q_chunk, k_chunk, s)))
    return rc;
  if ((rc = ra_check_fwd_buffers(q, kv_block, o_acc, lse_acc, s))) return rc;
  const int kb = ra_block_of_step(ring_rank, ring_step, ring_size);
  return ra_fwd_block(q, kv_block, kb, ring_rank, causal, q_chunk, k_chunk, o_acc,
                      lse_acc, s, (hipStream_t)stream);
}

int ring_attn_combine(float* o_a, float* lse_a, const float* o_b, const float* lse_b,
                      const ra_dims* dims, void* stream) {
  ra_shape s;
  int rc = ra_check_dims(dims, &s);
  if (rc) return rc;
  if (s.q_rows == 0) return RA_OK;
  if (!o_a || !lse_a || !o_b || !lse_b) return ra_fail(RA_ERR_INVALID, "NULL tensor pointer");
  const size_t ob = (size_t)s.q_rows * s.D * 4, lb = (size_t)s.q_rows * 4;
  if (overlaps(o_a, ob, o_b, ob) || overlaps(o_a, ob, lse_b, lb) ||
      overlaps(lse_a, lb, o_b, ob) || overlaps(lse_a, lb, lse_b, lb) ||
      overlaps(o_a, ob, lse_a, lb))
    return ra_fail(RA_ERR_INVALID, "partials a and b overlap");
  hipError_t e = ra_launch_combine(o_a, lse_a, o_b, lse_b, s.q_rows, s.D, (hipStream_t)stream);
  return e == hipSuccess ? RA_OK : ra_hip_fail(e, "combine kernel launch");
}

int ring_attn_finalize(const float* acc, void* out, int out_dtype, const ra_dims* dims,
                       void* stream) {
  ra_shape s;
  int rc = ra_check_dims(dims, &s);
  if (rc) return rc;
  if (out_dtype != RA_BF16 && out_dtype != RA_FP32)
    return ra_fail(RA_ERR_UNSUPPORTED, "out_dtype %d not supported", out_dtype);
  if (s.q_rows == 0) return RA_OK;
  if (!acc || !out) return ra_fail(RA_ERR_INVALID, "NULL tensor pointer");
  const size_t n = (size_t)s.q_rows * s.D;
  if (overlaps(acc, n * 4, out, n * (out_dtype == RA_BF16 ? 2 : 4)))
    return ra_fail(RA_ERR_INVALID, "out overlaps acc");
  hipError_t e = ra_launch_finalize(acc, out, out_dtype == RA_BF16 ? 0 : 1, (int64_t)n,
                                    (hipStream_t)stream);
  return e == hipSuccess ? RA_OK : ra_hip_fail(e, "finalize kernel launch");
}

int ring_attn_bwd_prep(const float* o, const void* dout, float* delta, const ra_dims* dims,
                       void* stream) {
  ra_shape s;
  int rc = ra_check_dims(dims, &s);
  if (rc) return rc;
  if (s.q_rows == 0) return RA_OK;
  if (!o || !dout || !delta) return ra_fail(RA_ERR_INVALID, "NULL tensor pointer");
  if (overlaps(delta, (size_t)s.q_rows * 4, o, (size_t)s.q_rows * s.D * 4) ||
      overlaps(delta, (size_t)s.q_rows * 4, dout, (size_t)s.q_rows * s.D * s.elem))
    return ra_fail(RA_ERR_INVALID, "delta overlaps an input");
  hipError_t e = ra_launch_bwd_prep(o, dout, s.dtype == RA_BF16 ? 0 : 1, delta, s.q_rows,
                                    s.D, (hipStream_t)stream);
  return e == hipSuccess ? RA_OK : ra_hip_fail(e, "bwd_prep kernel launch");
}

int ring_attn_bwd(const void* q, const void* kv_block, const void* dout, const float* lse,
                  const float* delta, int ring_rank, int ring_step, int ring_size,
                  int causal, int q_chunk, int k_chunk, float* dq_acc, float* dkv_io,
                  const ra_dims* dims, void* stream) {
  ra_shape s;
  int rc = ra_check_dims(dims, &s);
  if (rc) return rc;
  if (s.dtype != RA_BF16)
    return ra_fail(RA_ERR_UNSUPPORTED, "backward is implemented for bf16 inputs only");
  if ((rc = ra_check_ring(ring_rank, ring_step, ring_size, causal, q_chunk, k_chunk, s)))
    return rc;
  if ((rc = ra_check_bwd_buffers(q, kv_block, dout, lse, delta, dq_acc, dkv_io, s)))
    return rc;
  const int kb = ra_block_of_step(ring_rank, ring_step, ring_size);
  return ra_bwd_block(q, kv_block, dout, lse, delta, kb, ring_rank, causal, q_chunk,
                      k_chunk, dq_acc, dkv_io, nullptr, 1, s, (hipStream_t)stream);
}

int64_t ring_attn_bwd_workspace(const ra_dims* dims) {
  ra_shape s;
  int rc = ra_check_dims(dims, &s);
  if (rc) return rc;
  return (int64_t)(ra_bwd_dkv_splits(s) - 1) * 2 * s.kv_rows * s.D * 4;
}

int ring_attn_bwd_ws(const void* q, const void* kv_block, const void* dout, const float* lse,
                     const float* delta, int ring_rank, int ring_step, int ring_size,
                     int causal, int q_chunk, int k_chunk, float* dq_acc, float* dkv_io,
                     void* work, int64_t work_bytes, const ra_dims* dims, void* stream) {
  ra_shape s;
  int rc = ra_check_dims(dims, &s);
  if (rc) return rc;
  if (s.dtype != RA_BF16)
    return ra_fail(RA_ERR_UNSUPPORTED, "backward is implemented for bf16 inputs only");
  if ((rc = ra_check_ring(ring_rank, ring_step, ring_size, causal, q_chunk, k_chunk, s)))
    return rc;
  if ((rc = ra_check_bwd_buffers(q, kv_block, dout, lse, delta, dq_acc, dkv_io, s)))
    return rc;
  const size_t qb = (size_t)s.q_rows * s.D * s.elem;
  const size_t kvb = (size_t)2 * s.kv_rows * s.D * s.elem;
  const size_t lb = (size_t)s.q_rows * 4, dqb = (size_t)s.q_rows * s.D * 4;
  const size_t dkvb = (size_t)2 * s.kv_rows * s.D * 4;
  const void* other[7] = {q, kv_block, dout, lse, delta, dq_acc, dkv_io};
  const size_t othersz[7] = {qb, kvb, qb, lb, lb, dqb, dkvb};
  int nsplit = 1;
  if ((rc = ra_bwd_ws_plan(s, work, work_bytes, other, othersz, 7, &nsplit))) return rc;
  const int kb = ra_block_of_step(ring_rank, ring_step, ring_size);
  return ra_bwd_block(q, kv_block, dout, lse, delta, kb, ring_rank, causal, q_chunk,
                      k_chunk, dq_acc, dkv_io, (float*)work, nsplit, s, (hipStream_t)stream);
}

int ring_attn_decode_chunk(const ra_dims* dims) {
  ra_shape s;
  int rc = ra_check_dims(dims, &s);
  if (rc) return rc;
  if ((rc = ra_check_decode(s))) return rc;
  // Enough splits for about one workgroup per compute unit of the chip (256)
  // and at most kDecodeMaxChunkKeys keys per split, whole key tiles, and at
  // least four tiles per split.
  const int64_t groups = std::max<int64_t>(1, (int64_t)s.B * s.Hkv);
  const int64_t want = std::max<int64_t>({(int64_t)1, (256 + groups - 1) / groups,
                                          ((int64_t)s.Lk + kDecodeMaxChunkKeys - 1) /
                                              kDecodeMaxChunkKeys});
  int64_t chunk = ((int64_t)s.Lk + want - 1) / want;
  chunk = (chunk + kDecodeTileKeys - 1) / kDecodeTileKeys * kDecodeTileKeys;
  chunk = std::max<int64_t>(chunk, 4 * kDecodeTileKeys);
  return (int)std::min<int64_t>(chunk, std::max<int64_t>(s.Lk, 4 * kDecodeTileKeys));
}

int ring_attn_decode_splits(const ra_dims* dims, int k_chunk) {
  ra_shape s;
  int rc = ra_check_dims(dims, &s);
  if (rc) return rc;
  if (k_chunk < 1) return ra_fail(RA_ERR_INVALID, "k_chunk %d must be >= 1", k_chunk);
  return ra_decode_splits(s, k_chunk);
}

int ring_attn_fwd_decode(const void* q, const void* kv_block, int k_chunk, float* o_acc,
                         float* lse_acc, float* o_part, float* lse_part, const ra_dims* dims,
                         void* stream) {
  ra_shape s;
  int S = 0;
  int rc = ra_check_decode_call(q, kv_block, k_chunk, o_acc, lse_acc, dims, &s, &S);
  if (rc || S == 0) return rc;
  if (!o_part || !lse_part) return ra_fail(RA_ERR_INVALID, "NULL tensor pointer");
  const size_t qb = (size_t)s.q_rows * s.D * s.elem;
  const size_t kvb = (size_t)2 * s.kv_rows * s.D * s.elem;
  const size_t ob = (size_t)s.q_rows * s.D * 4, lb = (size_t)s.q_rows * 4;
  const size_t opb = ob * S, lpb = lb * S;
  const void* other[4] = {q, kv_block, o_acc, lse_acc};
  const size_t othersz[4] = {qb, kvb, ob, lb};
  for (int i = 0; i < 4; ++i)
    if (overlaps(o_part, opb, other[i], othersz[i]) ||
        overlaps(lse_part, lpb, other[i], othersz[i]))
      return ra_fail(RA_ERR_INVALID, "o_part / lse_part overlap another buffer");
  if (overlaps(o_part, opb, lse_part, lpb))
    return ra_fail(RA_ERR_INVALID, "o_part overlaps lse_part");
  return ra_decode_step(q, kv_block, k_chunk, S, o_acc, lse_acc, o_part, lse_part, s,
                        (hipStream_t)stream);
}

int ring_attn_fwd_decode_noalloc(const void* q, const void* kv_block, int k_chunk,
                                 float* o_acc, float* lse_acc, const ra_dims* dims,
                                 void* stream) {
  ra_shape s;
  int S = 0;
  int rc = ra_check_decode_call(q, kv_block, k_chunk, o_acc, lse_acc, dims, &s, &S);
  if (rc || S == 0) return rc;
  // o_part [S, B, H, Lq, d] at the start of the array, lse_part [S, B, H, Lq]
  // after it on a 256-byte boundary.
  const uint64_t opb = (uint64_t)S * (uint64_t)s.q_rows * s.D * 4;
  const uint64_t lp_off = (opb + 255) / 256 * 256;
  const uint64_t need = lp_off + (uint64_t)S * (uint64_t)s.q_rows * 4;
  if (need > (uint64_t)RA_DECODE_SCRATCH_BYTES)
    return ra_fail(RA_ERR_INVALID,
                   "the %d key splits of k_chunk %d need %llu bytes of partials, more than "
                   "the %u of the library's scratch array; use a larger k_chunk or "
                   "ring_attn_fwd_decode",
                   S, k_chunk, (unsigned long long)need, (unsigned)RA_DECODE_SCRATCH_BYTES);
  void* base = nullptr;
  size_t bytes = 0;
  hipError_t e = ra_decode_scratch(&base, &bytes);
  if (e != hipSuccess) return ra_hip_fail(e, "decode scratch array address");
  if (need > bytes) return ra_fail(RA_ERR_INVALID, "decode scratch array too small");
  float* o_part = (float*)base;
  float* lse_part = (float*)((char*)base + lp_off);
  return ra_decode_step(q, kv_block, k_chunk, S, o_acc, lse_acc, o_part, lse_part, s,
                        (hipStream_t)stream);
}

int ring_ffn_fwd(const void* x, const void* w1, const void* w2, void* hidden, void* out,
                 int64_t rows, int d_model, int d_ff, int chunk_rows, void* stream) {
  int rc = ra_check_ffn(rows, d_model, d_ff, chunk_rows);
  if (rc) return rc;
  if (rows == 0) return RA_OK;
  if (!x || !w1 || !w2 || !hidden || !out) return ra_fail(RA_ERR_INVALID, "NULL tensor pointer");
  const int64_t chunk = std::min<int64_t>(chunk_rows, rows);
  const size_t xb = (size_t)rows * d_model * 2, w1b = (size_t)d_ff * d_model * 2,
               w2b = w1b, hb = (size_t)chunk * d_ff * 2, ob = xb;
  const void* ins[3] = {x, w1, w2};
  const size_t insz[3] = {xb, w1b, w2b};
  for (int i = 0; i < 3; ++i)
    if (overlaps(hidden, hb, ins[i], insz[i]) || overlaps(out, ob, ins[i], insz[i]))
      return ra_fail(RA_ERR_INVALID, "hidden / out overlap an input");
  if (overlaps(hidden, hb, out, ob)) return ra_fail(RA_ERR_INVALID, "hidden overlaps out");
  hipStream_t st = (hipStream_t)stream;
  for (int64_t r0 = 0; r0 < rows; r0 += chunk) {
    const int m = (int)std::min<int64_t>(chunk, rows - r0);
    Timed tu(kFfnUp, st);
    hipError_t e = ra_launch_ffn_up((const char*)x + (size_t)r0 * d_model * 2, w1, hidden, m,
                                    d_model, d_ff, st);
    tu.done();
    if (e != hipSuccess) return ra_hip_fail(e, "feedforward up-projection launch");
    Timed td(kFfnDown, st);
    e = ra_launch_ffn_down(hidden, w2, (char*)out + (size_t)r0 * d_model * 2, m, d_model, d_ff,
                           st);
    td.done();
    if (e != hipSuccess) return ra_hip_fail(e, "feedforward down-projection launch");
  }
  return RA_OK;
}

int64_t ring_ffn_bwd_workspace(int64_t rows, int d_model, int d_ff, int chunk_rows) {
  int rc = ra_check_ffn(rows, d_model, d_ff, chunk_rows);
  if (rc) return rc;
  return (int64_t)ra_ffn_bwd_layout(rows, d_model, d_ff, chunk_rows).total;
}

int ring_ffn_bwd(const void* x, const void* w1, const void* w2, const void* dout, void* dx,
                 float* dw1, float* dw2, void* work, int64_t work_bytes, int64_t rows,
                 int d_model, int d_ff, int chunk_rows, void* stream) {
  int rc = ra_check_ffn(rows, d_model, d_ff, chunk_rows);
  if (rc) return rc;
  if (rows == 0) return RA_OK;
  if (!x || !w1 || !w2 || !dout || !dx || !dw1 || !dw2 || !work)
    return ra_fail(RA_ERR_INVALID, "NULL tensor pointer");
  const FfnBwdWork L = ra_ffn_bwd_layout(rows, d_model, d_ff, chunk_rows);
  if (work_bytes < (int64_t)L.total)
    return ra_fail(RA_ERR_INVALID, "workspace of %lld bytes is smaller than the %lld needed",
                   (long long)work_bytes, (long long)L.total);
  const size_t xb = (size_t)rows * d_model * 2, wb = (size_t)d_ff * d_model * 2;
  const void* ins[4] = {x, w1, w2, dout};
  const size_t insz[4] = {xb, wb, wb, xb};
  void* outs[4] = {dx, dw1, dw2, work};
  const size_t outsz[4] = {xb, wb * 2, wb * 2, L.total};
  for (int o = 0; o < 4; ++o) {
    for (int i = 0; i < 4; ++i)
      if (overlaps(outs[o], outsz[o], ins[i], insz[i]))
        return ra_fail(RA_ERR_INVALID, "an output or the workspace overlaps an input");
    for (int p = o + 1; p < 4; ++p)
      if (overlaps(outs[o], outsz[o], outs[p], outsz[p]))
        return ra_fail(RA_ERR_INVALID, "outputs or the workspace overlap each other");
  }
  hipStream_t st = (hipStream_t)stream;
  char* wk = (char*)work;
  void *w1t = wk + L.w1t, *w2t = wk + L.w2t, *z = wk + L.z, *g = wk + L.g;
  void *xt = wk + L.xt, *dot = wk + L.dot, *gt = wk + L.gt, *ht = wk + L.ht;
  auto fail = [](hipError_t e, const char* what) { return ra_hip_fail(e, what); };
  hipError_t e;
  {
    Timed t(kFfnBwdAux, st);
    e = ra_launch_transpose_pad(w1, w1t, d_ff, d_model, d_ff, st);  // W1^T [dm x dff]
    if (e == hipSuccess) e = ra_launch_transpose_pad(w2, w2t, d_model, d_ff, d_model, st);
    t.done();
    if (e != hipSuccess) return fail(e, "weight transpose launch");
  }
  const int64_t chunk = std::min<int64_t>(chunk_rows, rows);
  for (int64_t r0 = 0; r0 < rows; r0 += chunk) {
    const int m = (int)std::min<int64_t>(chunk, rows - r0);
    const int mp = (m + 63) / 64 * 64;
    const char* xc = (const char*)x + (size_t)r0 * d_model * 2;
    const char* dc = (const char*)dout + (size_t)r0 * d_model * 2;
    char* dxc = (char*)dx + (size_t)r0 * d_model * 2;
    {
      Timed t(kFfnBwdGemm, st);
      e = ra_launch_gemm_tn(xc, w1, z, m, d_ff, d_model, 0, st);          // Z = x W1^T
      if (e == hipSuccess) e = ra_launch_gemm_tn(dc, w2t, g, m, d_ff, d_model, 0, st);  // G = dout W2
      t.done();
      if (e != hipSuccess) return fail(e, "feedforward backward product launch");
    }
    {
      Timed t(kFfnBwdAux, st);
      // G <- G GELU'(Z) in place; G^T and GELU(Z)^T for the weight gradients
      e = ra_launch_gelu_grad_transpose(z, g, gt, ht, m, d_ff, mp, st);
      if (e == hipSuccess) e = ra_launch_transpose_pad(xc, xt, m, d_model, mp, st);
      if (e == hipSuccess) e = ra_launch_transpose_pad(dc, dot, m, d_model, mp, st);
      t.done();
      if (e != hipSuccess) return fail(e, "feedforward backward elementwise launch");
    }
    {
      Timed t(kFfnBwdGemm, st);
      e = ra_launch_gemm_tn(g, w1t, dxc, m, d_model, d_ff, 0, st);        // dx = G W1
      if (e == hipSuccess) e = ra_launch_gemm_tn(gt, xt, dw1, d_ff, d_model, mp, 1, st);  // dW1 += G^T x
      if (e == hipSuccess) e = ra_launch_gemm_tn(dot, ht, dw2, d_model, d_ff, mp, 1, st);  // dW2 += dout^T H
      t.done();
      if (e != hipSuccess) return fail(e, "feedforward backward product launch");
    }
  }
  return RA_OK;
}

}  // extern "C"
