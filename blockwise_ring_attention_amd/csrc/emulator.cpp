// Single-GPU ring emulator: plays one member of a ring.
//
// The other members' key/value blocks sit in a device pool.  The hop that
// would bring the next block from the predecessor over the interconnect is
// a device-to-device hipMemcpyAsync into one of two receive slots, issued on
// a side stream so that it overlaps the attention of the current block on
// the main stream (Ring Attention with Blockwise Transformers, abstract:
// key/value communication fully overlapped with blockwise computation; Ring
// Attention keyword page, definition: each device keeps its queries while the
// key/value blocks circulate).  Two events per slot order the hazards:
//   copied[i]   : compute on slot i waits for the copy into it;
//   consumed[i] : the next copy into slot i waits for the compute reading it.
// On entry the side stream waits for everything already queued on the main
// stream, so back-to-back calls (a forward share followed by its backward
// share, or the next step) never overwrite a slot that is still being read.
// RA_EMU_UNSAFE is a negative control: the consumed[] waits are dropped and
// each recycled slot is filled with NaN before its next copy, so a step that
// reads a slot after it was recycled sees poison or another block, and the
// parity tests show they can tell.  Each compute step is bracketed by a roctx
// range ("ring fwd|bwd step s: block kb"), visible in a marker trace.
// Only two slots ever exist, so the member never holds the whole sequence
// (darcstar commentary: an all-gather of every block would discard the
// method's memory saving).
#include <hip/hip_runtime.h>
#include <rocprofiler-sdk-roctx/roctx.h>
#include <stdio.h>

#include <vector>

#include "ra_api_internal.h"
#include "ring_attn.h"

namespace {

struct Events {
  hipEvent_t e[6] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  int n = 0;
  int create(int count) {
    for (n = 0; n < count; ++n) {
      hipError_t err = hipEventCreateWithFlags(&e[n], hipEventDisableTiming);
      if (err != hipSuccess) return ra_hip_fail(err, "hipEventCreate");
    }
    return RA_OK;
  }
  ~Events() {
    for (int i = 0; i < n; ++i) (void)hipEventDestroy(e[i]);
  }
};

// Steps the member computes, in arrival order: block ids, with the causal
// future dropped.
int build_schedule(int rank, int size, int causal, const int32_t* order,
                   std::vector<int>* blocks) {
  std::vector<char> seen(size, 0);
  for (int s = 0; s < size; ++s) {
    int kb = order ? order[s] : ra_block_of_step(rank, s, size);
    if (kb < 0 || kb >= size || seen[kb])
      return ra_fail(RA_ERR_INVALID, "order is not a permutation of 0..%d", size - 1);
    seen[kb] = 1;
    if (causal && kb > rank) continue;
    blocks->push_back(kb);
  }
  return RA_OK;
}

// Host-side roctx range around the enqueue of one ring step.
struct StepRange {
  StepRange(const char* pass, int step, int kb) {
    char name[64];
    snprintf(name, sizeof name, "ring %s step %d: block %d", pass, step, kb);
    roctxRangePushA(name);
  }
  ~StepRange() { roctxRangePop(); }
};

bool valid_mode(int mode) {
  return mode == RA_EMU_OVERLAP || mode == RA_EMU_SERIALIZE || mode == RA_EMU_UNSAFE;
}

#define RA_HIP(call, what)                             \
  do {                                                 \
    hipError_t _e = (call);                            \
    if (_e != hipSuccess) return ra_hip_fail(_e, what); \
  } while (0)

}  // namespace

extern "C" int ring_emu_fwd(const void* q, const void* const* kv_pool, void* slot0,
                            void* slot1, int ring_rank, int ring_size, int causal,
                            int q_chunk, int k_chunk, float* o_acc, float* lse_acc,
                            const ra_dims* dims, const int32_t* order, int mode,
                            void* main_stream, void* side_stream) {
  ra_shape s;
  int rc = ra_check_dims(dims, &s);
  if (rc) return rc;
  if ((rc = ra_check_ring(ring_rank, 0, ring_size, causal, q_chunk, k_chunk, s))) return rc;
  if (!valid_mode(mode)) return ra_fail(RA_ERR_INVALID, "unknown emulator mode %d", mode);
  if (!kv_pool) return ra_fail(RA_ERR_INVALID, "kv_pool is NULL");
  std::vector<int> blocks;
  if ((rc = build_schedule(ring_rank, ring_size, causal, order, &blocks))) return rc;
  if (s.q_rows == 0 || s.Lk == 0) return RA_OK;
  const size_t bytes = (size_t)2 * s.kv_rows * s.D * s.elem;
  void* slots[2] = {slot0, slot1};
  int ncopies = 0;
  for (int kb : blocks) {
    if (!kv_pool[kb]) return ra_fail(RA_ERR_INVALID, "kv_pool[%d] is NULL but needed", kb);
    if ((rc = ra_check_fwd_buffers(q, kv_pool[kb], o_acc, lse_acc, s))) return rc;
    if (kb != ring_rank) ++ncopies;
  }
  if (ncopies > 0 && (!slot0 || (ncopies > 1 && !slot1)))
    return ra_fail(RA_ERR_INVALID, "receive slot is NULL");
  for (int i = 0; i < 2 && i < ncopies; ++i)
    if ((rc = ra_check_fwd_buffers(q, slots[i], o_acc, lse_acc, s))) return rc;

  // async: hops on the side stream ordered by events (overlap, unsafe);
  // guarded: a slot is recycled only after its compute (overlap).
  const bool async = mode != RA_EMU_SERIALIZE, guarded = mode == RA_EMU_OVERLAP;
  hipStream_t main = (hipStream_t)main_stream;
  hipStream_t side = async ? (hipStream_t)side_stream : main;
  if (async && side == main)
    return ra_fail(RA_ERR_INVALID, "overlap mode needs a side stream distinct from main");

  // copy index -> block id, in arrival order
  std::vector<int> copy_block;
  for (int kb : blocks)
    if (kb != ring_rank) copy_block.push_back(kb);

  Events ev;  // 0,1: copied[slot]; 2,3: consumed[slot]; 4: entry
  if (async) {
    if ((rc = ev.create(5))) return rc;
    // Work already queued on main (an earlier share still reading the slots,
    // the caller's writes to the pool) precedes every hop of this call.
    RA_HIP(hipEventRecord(ev.e[4], main), "hipEventRecord");
    RA_HIP(hipStreamWaitEvent(side, ev.e[4], 0), "hipStreamWaitEvent");
  }
  auto issue_copy = [&](int ci) -> int {
    const int slot = ci & 1;
    if (guarded && ci >= 2)
      RA_HIP(hipStreamWaitEvent(side, ev.e[2 + slot], 0), "hipStreamWaitEvent");
    if (!guarded && async && ci >= 2)
      RA_HIP(hipMemsetAsync(slots[slot], 0xFF, bytes, side), "poison fill");
    RA_HIP(hipMemcpyAsync(slots[slot], kv_pool[copy_block[ci]], bytes,
                          hipMemcpyDeviceToDevice, side),
           "ring hop copy");
    if (async) RA_HIP(hipEventRecord(ev.e[slot], side), "hipEventRecord");
    return RA_OK;
  };

  // Overlap: the first two hops are in flight before any compute; the copy
  // into a slot is issued as soon as the compute reading its previous block
  // has been enqueued.  Serialize: each copy is issued just before its use.
  const int nc = (int)copy_block.size();
  int issued = 0;
  if (async)
    for (; issued < 2 && issued < nc; ++issued)
      if ((rc = issue_copy(issued))) return rc;
  int ci = 0, step = 0;
  for (int kb : blocks) {
    const StepRange range("fwd", step++, kb);
    const void* src = kv_pool[kb];
    int slot = -1;
    if (kb != ring_rank) {
      slot = ci & 1;
      if (mode == RA_EMU_SERIALIZE) {
        if ((rc = issue_copy(ci))) return rc;
      } else {
        RA_HIP(hipStreamWaitEvent(main, ev.e[slot], 0), "hipStreamWaitEvent");
      }
      src = slots[slot];
    }
    if ((rc = ra_fwd_block(q, src, kb, ring_rank, causal, q_chunk, k_chunk, o_acc, lse_acc,
                           s, main)))
      return rc;
    if (slot >= 0) {
      if (async) {
        RA_HIP(hipEventRecord(ev.e[2 + slot], main), "hipEventRecord");
        if (issued < nc && issued == ci + 2) {
          if ((rc = issue_copy(issued))) return rc;
          ++issued;
        }
      }
      ++ci;
    }
  }
  return RA_OK;
}

extern "C" int ring_emu_bwd(const void* q, const void* const* kv_pool, void* slot0,
                            void* slot1, const void* dout, const float* lse,
                            const float* delta, float* const* dkv_pool, float* dkv_slot0,
                            float* dkv_slot1, int ring_rank, int ring_size, int causal,
                            int q_chunk, int k_chunk, float* dq_acc, void* work,
                            int64_t work_bytes, const ra_dims* dims, const int32_t* order,
                            int mode, void* main_stream, void* side_stream) {
  ra_shape s;
  int rc = ra_check_dims(dims, &s);
  if (rc) return rc;
  if (s.dtype != RA_BF16)
    return ra_fail(RA_ERR_UNSUPPORTED, "backward is implemented for bf16 inputs only");
  if ((rc = ra_check_ring(ring_rank, 0, ring_size, causal, q_chunk, k_chunk, s))) return rc;
  if (!valid_mode(mode)) return ra_fail(RA_ERR_INVALID, "unknown emulator mode %d", mode);
  if (!kv_pool || !dkv_pool) return ra_fail(RA_ERR_INVALID, "pool is NULL");
  std::vector<int> blocks;
  if ((rc = build_schedule(ring_rank, ring_size, causal, order, &blocks))) return rc;
  if (s.q_rows == 0 || s.Lk == 0) return RA_OK;
  const size_t kv_bytes = (size_t)2 * s.kv_rows * s.D * s.elem;
  const size_t dkv_bytes = (size_t)2 * s.kv_rows * s.D * 4;
  void* slots[2] = {slot0, slot1};
  float* dslots[2] = {dkv_slot0, dkv_slot1};
  int nsplit = 1;
  std::vector<int> copy_block;
  for (int kb : blocks) {
    if (!kv_pool[kb] || !dkv_pool[kb])
      return ra_fail(RA_ERR_INVALID, "pool entry %d is NULL but needed", kb);
    if ((rc = ra_check_bwd_buffers(q, kv_pool[kb], dout, lse, delta, dq_acc, dkv_pool[kb], s)))
      return rc;
    if (kb != ring_rank) copy_block.push_back(kb);
  }
  const int nc = (int)copy_block.size();
  if (nc > 0 && (!slot0 || !dkv_slot0 || (nc > 1 && (!slot1 || !dkv_slot1))))
    return ra_fail(RA_ERR_INVALID, "receive slot is NULL");
  for (int i = 0; i < 2 && i < nc; ++i)
    if ((rc = ra_check_bwd_buffers(q, slots[i], dout, lse, delta, dq_acc, dslots[i], s)))
      return rc;
  // The workspace must stay clear of every buffer of the share.
  {
    const size_t qb = (size_t)s.q_rows * s.D * s.elem, lb = (size_t)s.q_rows * 4;
    const size_t dqb = (size_t)s.q_rows * s.D * 4;
    std::vector<const void*> other = {q, dout, lse, delta, dq_acc};
    std::vector<size_t> othersz = {qb, qb, lb, lb, dqb};
    for (int kb : blocks) {
      other.push_back(kv_pool[kb]);
      othersz.push_back(kv_bytes);
      other.push_back(dkv_pool[kb]);
      othersz.push_back(dkv_bytes);
    }
    for (int i = 0; i < 2 && i < nc; ++i) {
      other.push_back(slots[i]);
      othersz.push_back(kv_bytes);
      other.push_back(dslots[i]);
      othersz.push_back(dkv_bytes);
    }
    if ((rc = ra_bwd_ws_plan(s, work, work_bytes, other.data(), othersz.data(),
                             (int)other.size(), &nsplit)))
      return rc;
  }

  // async: hops on the side stream ordered by events (overlap, unsafe);
  // guarded: a slot is recycled only after its compute (overlap).
  const bool async = mode != RA_EMU_SERIALIZE, guarded = mode == RA_EMU_OVERLAP;
  hipStream_t main = (hipStream_t)main_stream;
  hipStream_t side = async ? (hipStream_t)side_stream : main;
  if (async && side == main)
    return ra_fail(RA_ERR_INVALID, "overlap mode needs a side stream distinct from main");

  Events ev;  // 0,1 copied; 2,3 consumed; 4 side done; 5 entry
  if (async) {
    if ((rc = ev.create(6))) return rc;
    RA_HIP(hipEventRecord(ev.e[5], main), "hipEventRecord");
    RA_HIP(hipStreamWaitEvent(side, ev.e[5], 0), "hipStreamWaitEvent");
  }
  // Receive: the key/value block and its travelling dK/dV partial.
  auto issue_in = [&](int ci) -> int {
    const int slot = ci & 1;
    // the previous user of this slot finished its compute and its copy-out
    // was issued earlier on the same (side) stream, so ordering is implied
    // (unsafe: that copy-out did not wait, and the slot is poisoned first)
    if (!guarded && async && ci >= 2) {
      RA_HIP(hipMemsetAsync(slots[slot], 0xFF, kv_bytes, side), "poison fill");
      RA_HIP(hipMemsetAsync(dslots[slot], 0xFF, dkv_bytes, side), "poison fill");
    }
    RA_HIP(hipMemcpyAsync(slots[slot], kv_pool[copy_block[ci]], kv_bytes,
                          hipMemcpyDeviceToDevice, side),
           "ring hop copy (kv)");
    RA_HIP(hipMemcpyAsync(dslots[slot], dkv_pool[copy_block[ci]], dkv_bytes,
                          hipMemcpyDeviceToDevice, side),
           "ring hop copy (dkv in)");
    if (async) RA_HIP(hipEventRecord(ev.e[slot], side), "hipEventRecord");
    return RA_OK;
  };
  // Send: the partial, now holding this member's contribution, moves on.
  auto issue_out = [&](int ci) -> int {
    const int slot = ci & 1;
    if (guarded) RA_HIP(hipStreamWaitEvent(side, ev.e[2 + slot], 0), "hipStreamWaitEvent");
    RA_HIP(hipMemcpyAsync(dkv_pool[copy_block[ci]], dslots[slot], dkv_bytes,
                          hipMemcpyDeviceToDevice, side),
           "ring hop copy (dkv out)");
    return RA_OK;
  };

  int issued = 0;
  if (async)
    for (; issued < 2 && issued < nc; ++issued)
      if ((rc = issue_in(issued))) return rc;
  int ci = 0, step = 0;
  for (int kb : blocks) {
    const StepRange range("bwd", step++, kb);
    const void* src = kv_pool[kb];
    float* dsrc = dkv_pool[kb];
    int slot = -1;
    if (kb != ring_rank) {
      slot = ci & 1;
      if (mode == RA_EMU_SERIALIZE) {
        if ((rc = issue_in(ci))) return rc;
      } else {
        RA_HIP(hipStreamWaitEvent(main, ev.e[slot], 0), "hipStreamWaitEvent");
      }
      src = slots[slot];
      dsrc = dslots[slot];
    }
    if ((rc = ra_bwd_block(q, src, dout, lse, delta, kb, ring_rank, causal, q_chunk, k_chunk,
                           dq_acc, dsrc, (float*)work, nsplit, s, main)))
      return rc;
    if (slot >= 0) {
      if (async) RA_HIP(hipEventRecord(ev.e[2 + slot], main), "hipEventRecord");
      if ((rc = issue_out(ci))) return rc;
      if (async && issued < nc && issued == ci + 2) {
        if ((rc = issue_in(issued))) return rc;
        ++issued;
      }
      ++ci;
    }
  }
  if (async && nc > 0) {
    // the caller's main stream completes only after the last hop has landed
    RA_HIP(hipEventRecord(ev.e[4], side), "hipEventRecord");
    RA_HIP(hipStreamWaitEvent(main, ev.e[4], 0), "hipStreamWaitEvent");
  }
  return RA_OK;
}
