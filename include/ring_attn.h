/*
 * ring_attn.h -- C ABI for one ring member's share of exact blockwise
 * softmax attention on AMD Instinct MI355X (gfx950).
 *
 * The method (Ring Attention with Blockwise Transformers; "Ring Attention"
 * and "Blockwise RingAttention" keyword pages, definitions): a sequence is
 * split into equal contiguous blocks, one per ring member.  A member keeps
 * its query block while the key/value blocks circulate around the ring; each
 * arriving block is attended blockwise and folded into a running result.
 * The fold is the associative online-softmax combine of partial attentions,
 * and the causal mask and softmax denominator are applied exactly across
 * block and chunk seams (darcstar research page, commentary).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers on the current HIP device.  The
 *   caller allocates and frees every buffer, workspaces included; the
 *   library allocates no device memory (its only device storage is the fixed
 *   scratch array of ring_attn_fwd_decode_noalloc, part of the loaded code
 *   object).  All work is enqueued asynchronously on the given hipStream_t
 *   (passed as void*; NULL = the null stream); a device fault surfaces at the
 *   caller's next synchronisation.
 * - Every compute entry point (ring_attn_init_acc, ring_attn_fwd,
 *   ring_attn_fwd_decode, ring_attn_fwd_decode_noalloc, ring_attn_combine,
 *   ring_attn_finalize, ring_attn_bwd_prep, ring_attn_bwd, ring_attn_bwd_ws,
 *   ring_ffn_fwd, ring_ffn_bwd) only
 *   launches kernels on the given stream: no allocation, no hipMemset, no
 *   synchronisation, so a sequence of them may be captured into a HIP graph
 *   and replayed.  Timing (ring_attn_timing_enable) records events and must
 *   be off while capturing.  The ring emulator entry points create events
 *   and use a second stream; they are not meant for capture.
 * - Layouts are dense row-major, no strides (H = ra_dims.heads query heads,
 *   Hkv = ra_dims.kv_heads key/value heads):
 *     q, dout          [B, H, Lq, d]        (dtype of ra_dims.dtype)
 *     kv_block         [2, B, Hkv, Lk, d]   (index 0 = K, 1 = V; one copy moves it)
 *     o_acc, dq_acc    [B, H, Lq, d]        float32
 *     lse_acc, delta   [B, H, Lq]           float32
 *     dkv_io           [2, B, Hkv, Lk, d]   float32 (0 = dK, 1 = dV)
 * - Shared key/value heads (MQA / GQA: several query heads share one
 *   key/value head; kongchang "Ring Attention" knowledge page, facts list):
 *   query head h attends to key/value head h / (H / Hkv), i.e. consecutive
 *   groups of H / Hkv query heads share one.  Hkv == H is ordinary multi-head
 *   attention, Hkv == 1 is MQA.
 * - Positions are global: member r's query i sits at r*Lq + i and key j of
 *   block kb at kb*Lk + j.  Under the causal mask key j is visible to query
 *   i iff its position is <= the query's (the diagonal is visible).  Causal
 *   calls therefore require Lq == Lk (equal blocks).
 * - Ring schedule: at ring step s a member of rank r holds block
 *   kb = (r - s) mod N (it receives from its predecessor; step 0 is its own
 *   block).  Under the causal mask a block with kb > r is entirely in the
 *   future: the call is a no-op that launches nothing.
 * - Debug switch: with the environment variable RA_NO_SKIP set (to anything
 *   but "0") at the time of a call, the causal diagonal block computes every
 *   tile, the ones wholly above the diagonal fully masked, instead of
 *   skipping them (ring_attn_fwd, ring_attn_bwd, ring_attn_bwd_ws and the
 *   emulator).  Results are bitwise those of the skipping path.
 * - Scores are scale * <q_i, k_j> with scale = ra_dims.scale, or 1/sqrt(d)
 *   when ra_dims.scale == 0.  LSE is the natural-log log-sum-exp of the
 *   scores over the keys a row has seen so far.
 * - (o_acc, lse_acc) always hold a NORMALISED partial: o over the keys seen
 *   so far and its LSE.  The empty partial is (0, -inf); initialise with
 *   ring_attn_init_acc.
 * - q_chunk / k_chunk are the query and key chunk sizes of the blockwise
 *   decomposition (sourcepulse project page, Highlighted Details: tuning
 *   knobs).  They must be >= 1; they need not divide the lengths (ragged
 *   last chunks are handled).  They select the kernels' tile shapes and never
 *   change the result beyond rounding: for bf16 ring steps q_chunk >= 256
 *   selects 256 query rows per workgroup (8 waves), otherwise 128 (4 waves);
 *   k_chunk >= 64 selects 64-key tiles, otherwise 32.  Larger chunks (cfg
 *   "512 / 1024") therefore run as 256 / 64: a chunk of 1024 keys of d = 128
 *   in K and V is 512 KiB, more than the 160 KiB of LDS a compute unit has.
 *   The backward always uses 256-row dQ tiles and 128-key dK/dV tiles; the
 *   fp32 forward, one query row per thread.
 *
 * Errors: every entry point returns RA_OK (0) or a negative code, and never
 * throws.  Invalid arguments and unsupported shapes are detected on the host
 * before anything is enqueued; ring_attn_last_error() then returns a
 * thread-local message describing the most recent failure on this thread.
 * Calls on different streams may run concurrently from different threads,
 * provided their output buffers do not overlap.
 */
#ifndef RING_ATTN_H
#define RING_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  RA_OK = 0,
  RA_ERR_INVALID = -1,      /* null pointer, bad rank/step/size, bad chunk, aliasing */
  RA_ERR_UNSUPPORTED = -2,  /* head_dim or dtype the kernels do not implement */
  RA_ERR_HIP = -3           /* a HIP launch or copy failed */
};

enum { RA_BF16 = 0, RA_FP32 = 1 };

/* Problem shape of one call.  head_dim must be 64 or 128.  batch, heads and
 * the lengths may be 0 (then the call does nothing and returns RA_OK). */
typedef struct ra_dims {
  int32_t batch;
  int32_t heads;     /* H: query heads */
  int32_t q_len;     /* Lq: query rows held by the member */
  int32_t kv_len;    /* Lk: tokens per key/value block */
  int32_t head_dim;  /* d */
  int32_t dtype;     /* RA_BF16 or RA_FP32: dtype of q, kv_block and dout */
  float scale;       /* > 0; 0 => 1/sqrt(head_dim); negative is rejected */
  int32_t kv_heads;  /* Hkv: key/value heads, dividing heads; 0 => heads */
} ra_dims;

/* Version of this ABI (major * 100 + minor). */
int ring_attn_version(void);

/* Message for the most recent failing call on this thread ("" if none). */
const char* ring_attn_last_error(void);

/* Set (o_acc, lse_acc) to the empty partial (0, -inf) with a fill kernel
 * (no hipMemset, so the call may be captured in a HIP graph). */
int ring_attn_init_acc(float* o_acc, float* lse_acc, const ra_dims* dims,
                       void* stream);

/* Forward ring step (blockwise pass + fold; Ring Attention keyword page,
 * definition; darcstar commentary on the associative combine and exact seams).
 * Attends q to key/value block kb = (ring_rank - ring_step) mod ring_size and
 * folds the result into (o_acc, lse_acc) in place:
 *     (o_acc, lse_acc) <- (o_acc, lse_acc) (+) attention(q, kv_block)
 * where (+) is the combine of ring_attn_combine.  Requirements:
 * 0 <= ring_rank, ring_step < ring_size; Lq == Lk if causal; o_acc and
 * lse_acc must not overlap q or kv_block.  A future block under the causal
 * mask returns RA_OK and leaves the accumulators bitwise unchanged.
 * bf16 inputs run on bf16 MFMA with fp32 accumulation (the probabilities are
 * rounded to bf16 before the value product); fp32 inputs run in fp32. */
int ring_attn_fwd(const void* q, const void* kv_block, int ring_rank,
                  int ring_step, int ring_size, int causal, int q_chunk,
                  int k_chunk, float* o_acc, float* lse_acc,
                  const ra_dims* dims, void* stream);

/* Associative combine of two normalised partials over disjoint key sets
 * (darcstar commentary: online softmax is associative).  In place on a:
 *     mu = max(lse_a, lse_b), w_x = exp(lse_x - mu),
 *     lse_a <- mu + ln(w_a + w_b),  o_a <- (w_a o_a + w_b o_b) / (w_a + w_b)
 * with (0, -inf) as the identity on either side.  Shapes: o [B,H,Lq,d],
 * lse [B,H,Lq] (kv_len and kv_heads are ignored).  a and b must not overlap. */
int ring_attn_combine(float* o_a, float* lse_a, const float* o_b,
                      const float* lse_b, const ra_dims* dims, void* stream);

/* Cast an fp32 [B, H, Lq, d] accumulator (o_acc or dq_acc) to out_dtype
 * (RA_BF16 with round-to-nearest-even, or RA_FP32 copy).  The pages fix no
 * output precision; the bf16 output with an fp32 running accumulator is the
 * reading used (the accumulator stays fp32 across every ring step, so the
 * blockwise fold adds no rounding of its own).  acc and out must not
 * overlap (RA_ERR_INVALID). */
int ring_attn_finalize(const float* acc, void* out, int out_dtype,
                       const ra_dims* dims, void* stream);

/* Backward preparation: delta[b,h,i] = sum_c dout[b,h,i,c] * o[b,h,i,c], with
 * o the final fp32 o_acc of the forward share.  The gradient is that of
 * sum(dO * O) over the member's rows; the pages do not discuss the backward,
 * so this follows from the exactness of the forward. */
int ring_attn_bwd_prep(const float* o, const void* dout, float* delta,
                       const ra_dims* dims, void* stream);

/* Backward ring step for block kb = (ring_rank - ring_step) mod ring_size.
 * The pages do not discuss the backward; this is the exact gradient of
 * sum(dO * O) for the forward above, computed blockwise with the
 * probabilities recomputed per block rather than stored (the memory-efficient
 * method keeps no attention matrix; Blockwise RingAttention keyword page,
 * definition).  Recomputes the probabilities from the saved final lse
 * (natural log, as left in lse_acc by the forward) and accumulates
 *     dq_acc += dQ  (this block's contribution to the member's dQ)
 *     dkv_io += [dK_kb, dV_kb]  (this member's contribution to block kb)
 * so a travelling dK/dV partial can collect every member's contribution.
 * With shared key/value heads, dK/dV of a key/value head sums the
 * contributions of every query head of its group.
 * bf16 only (RA_ERR_UNSUPPORTED for fp32).  A future block under the causal
 * mask is a no-op.  dq_acc and dkv_io must not overlap each other or any
 * input. */
int ring_attn_bwd(const void* q, const void* kv_block, const void* dout,
                  const float* lse, const float* delta, int ring_rank,
                  int ring_step, int ring_size, int causal, int q_chunk,
                  int k_chunk, float* dq_acc, float* dkv_io,
                  const ra_dims* dims, void* stream);

/* The same backward step with a caller-provided workspace, for shared
 * key/value heads.  The dK/dV of a key/value head sums the contributions of
 * the G = H / Hkv query heads of its group (definition above); ring_attn_bwd
 * takes them one query head after another over the head's key tiles of 128
 * keys, so with few key/value heads (MQA: B * Hkv * ceil(Lk / 128)
 * workgroups) part of the chip idles.  ring_attn_bwd_ws runs S query heads of
 * each group side by side: the first adds into dkv_io as before, each other
 * one into a private fp32 copy of dkv_io in `work` ([S-1][2, B, Hkv, Lk, d]),
 * and the copies are added into dkv_io at the end of the call, in copy
 * order.  Every sum is taken in a fixed order, so the result is
 * deterministic for a given S; it differs from ring_attn_bwd only by the
 * order of fp32 additions.
 *   ring_attn_bwd_workspace(dims) returns the bytes of `work` for the
 *   preferred S (about one workgroup per compute unit, at most G; 0 when
 *   S = 1, e.g. Hkv == H), or a negative error code.
 *   ring_attn_bwd_ws uses as many copies as work_bytes holds, up to that
 *   preferred count (work_bytes == 0 is ring_attn_bwd).  work must be
 *   16-byte aligned and must not overlap any other argument; its contents on
 *   return are unspecified; work_bytes < 0, or work == NULL with
 *   work_bytes > 0, is RA_ERR_INVALID.  All other arguments and errors as
 *   ring_attn_bwd. */
int64_t ring_attn_bwd_workspace(const ra_dims* dims);
int ring_attn_bwd_ws(const void* q, const void* kv_block, const void* dout,
                     const float* lse, const float* delta, int ring_rank,
                     int ring_step, int ring_size, int causal, int q_chunk,
                     int k_chunk, float* dq_acc, float* dkv_io, void* work,
                     int64_t work_bytes, const ra_dims* dims, void* stream);

/* ---- decode-shaped step ---------------------------------------------------
 * The inference use of the method (Ring Attention with Blockwise
 * Transformers, abstract: training and inference of long sequences): a few
 * new query rows -- one decode step, or a short run of Lq draft tokens --
 * that come after every key of kv_block attend to the whole block, which
 * may be one member's share of a long key/value cache.  There is no mask
 * inside the block: every key precedes every query row.  As in
 * ring_attn_fwd,
 *     (o_acc, lse_acc) <- (o_acc, lse_acc) (+) attention(q, kv_block)
 * so blocks arriving around the ring fold in the same way.
 *
 * With so few rows the step streams the key/value block from HBM once; to
 * spread that over the chip the block's keys are split into
 * S = ceil(Lk / k_chunk) splits of k_chunk keys, attended in parallel, each
 * giving a normalised partial; the S partials are then folded into the
 * accumulator in split order.  The caller provides the partials' storage:
 *     o_part   [S, B, H, Lq, d]  float32
 *     lse_part [S, B, H, Lq]     float32
 * which must not overlap each other or any other argument; their contents
 * on return are unspecified.  Requirements: bf16 inputs
 * (RA_ERR_UNSUPPORTED otherwise); (H / Hkv) * Lq <= 64, the query rows that
 * share one key/value head (RA_ERR_UNSUPPORTED otherwise); k_chunk >= 1 and
 * S <= 65536 (RA_ERR_INVALID).  Lk == 0 leaves the accumulators unchanged.
 * ring_attn_decode_chunk(dims) returns a k_chunk (> 0) that spreads the
 * splits over the chip for these dims, or a negative error code;
 * ring_attn_decode_splits(dims, k_chunk) returns S (>= 0), or a negative
 * error code. */
int ring_attn_decode_chunk(const ra_dims* dims);
int ring_attn_decode_splits(const ra_dims* dims, int k_chunk);
int ring_attn_fwd_decode(const void* q, const void* kv_block, int k_chunk,
                         float* o_acc, float* lse_acc, float* o_part,
                         float* lse_part, const ra_dims* dims, void* stream);

/* The same decode-shaped step for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): identical to ring_attn_fwd_decode with the same k_chunk --
 * same kernels, bitwise the same result -- except that the split partials
 * live in a device-resident array of RA_DECODE_SCRATCH_BYTES bytes owned by
 * the library (one copy per GPU, held from the first call on that GPU until
 * the process ends).  It calls no allocating routine.  The partials need
 *     align256(S * B * H * Lq * d * 4) + S * B * H * Lq * 4
 * bytes with S = ceil(Lk / k_chunk); a call needing more returns
 * RA_ERR_INVALID before anything is enqueued (take a larger k_chunk, or
 * ring_attn_fwd_decode with caller-provided partials).  Every call on one
 * GPU uses that GPU's one array: calls that may overlap in time on the same
 * GPU (different streams, or different host threads) race and give
 * undefined results; serialise them.  The array keeps the last call's
 * contents; each call writes every partial it reads, so nothing needs
 * clearing.  Other requirements and errors as for ring_attn_fwd_decode;
 * RA_ERR_HIP if the array's address cannot be obtained on this device. */
#define RA_DECODE_SCRATCH_BYTES (16u << 20)
int ring_attn_fwd_decode_noalloc(const void* q, const void* kv_block,
                                 int k_chunk, float* o_acc, float* lse_acc,
                                 const ra_dims* dims, void* stream);

/* ---- blockwise feedforward ----------------------------------------------
 * The method computes self-attention and the feedforward blockwise (Ring
 * Attention with Blockwise Transformers, abstract; sourcepulse project page,
 * How It Works: attention and feedforward are both distributed).  The
 * feedforward is position-wise, so a member applies it to its own rows with
 * no communication, chunk_rows rows at a time, and the hidden activation
 * never exceeds [chunk_rows, d_ff].  The pages do not give its form; this is
 * the position-wise two-layer MLP
 *     out = GELU(x W1^T) W2^T,   GELU(z) = z/2 (1 + erf(z / sqrt 2)),
 * with the hidden activation rounded to bf16 (RNE) before the second
 * product and out rounded to bf16 (RNE); products accumulate in fp32.
 *   x      [rows, d_model]  bf16 (device)
 *   w1     [d_ff, d_model]  bf16 (out x in, the layout of a linear layer)
 *   w2     [d_model, d_ff]  bf16
 *   hidden [min(rows, chunk_rows), d_ff]  bf16 workspace owned by the caller;
 *          its contents on return are unspecified
 *   out    [rows, d_model]  bf16
 * d_model and d_ff must be positive multiples of 256 (RA_ERR_UNSUPPORTED);
 * chunk_rows >= 1 (RA_ERR_INVALID); hidden and out must not overlap each
 * other or any input (RA_ERR_INVALID).  Each row's result is bitwise
 * independent of chunk_rows.  rows == 0 does nothing. */
int ring_ffn_fwd(const void* x, const void* w1, const void* w2, void* hidden,
                 void* out, int64_t rows, int d_model, int d_ff, int chunk_rows,
                 void* stream);

/* Backward of ring_ffn_fwd for the same rows and chunking: given
 * dout = d loss / d out [rows, d_model] bf16,
 *   dx   = dZ W1                    [rows, d_model]  bf16 (written)
 *   dw1 += dZ^T x                   [d_ff, d_model]  fp32 (accumulated)
 *   dw2 += dout^T GELU(Z)           [d_model, d_ff]  fp32 (accumulated)
 * with Z = x W1^T recomputed per chunk, dH = dout W2 and
 * dZ = dH * GELU'(Z), GELU'(z) = Phi(z) + z phi(z) (the pages do not
 * discuss the backward; this is the exact gradient of the forward above).
 * Z, GELU(Z) and dZ are held in bf16; products accumulate in fp32, and dw1
 * / dw2 gather every chunk's contribution, so callers zero them first (or
 * keep accumulating over several blocks).  work is a caller-provided device
 * workspace of ring_ffn_bwd_workspace(rows, d_model, d_ff, chunk_rows)
 * bytes (transposed weights and per-chunk activations; contents on return
 * are unspecified); a smaller work_bytes is RA_ERR_INVALID.  Outputs and
 * the workspace must not overlap each other or any input.  Shape rules as
 * for ring_ffn_fwd.  ring_ffn_bwd_workspace returns the byte count (>= 0) or
 * a negative error code. */
int64_t ring_ffn_bwd_workspace(int64_t rows, int d_model, int d_ff,
                               int chunk_rows);
int ring_ffn_bwd(const void* x, const void* w1, const void* w2,
                 const void* dout, void* dx, float* dw1, float* dw2, void* work,
                 int64_t work_bytes, int64_t rows, int d_model, int d_ff,
                 int chunk_rows, void* stream);

/* ---- single-GPU ring emulator ------------------------------------------
 * Plays one member of a ring of ring_size members on one GPU.  The other
 * members' key/value blocks live in a device pool; the "hop" that would
 * bring the next block over the interconnect is a device-to-device
 * hipMemcpyAsync into one of two receive slots, issued on side_stream and
 * overlapped with the attention of the current block on main_stream
 * (Ring Attention with Blockwise Transformers, abstract: the key/value
 * transfers hide behind the blockwise compute).  Events order
 * copy-after-consume and compute-after-copy.  Only two slots exist: there
 * is never a gather of all blocks.
 *
 * kv_pool: HOST array of ring_size device pointers; kv_pool[kb] is block kb
 *          ([2,B,Hkv,Lk,d]).  Entries that the causal mask never needs (kb >
 *          ring_rank) may be NULL.  kv_pool[ring_rank] is used in place
 *          (the member's own block needs no hop).
 * slots:   two device buffers of one block each.
 * order:   NULL for the ring schedule, else a HOST array of ring_size block
 *          ids giving the arrival order (any permutation; the result is
 *          order-invariant because the combine is commutative).
 * mode:    RA_EMU_OVERLAP (side-stream copies) or RA_EMU_SERIALIZE (all on
 *          main_stream; must match OVERLAP bitwise), or RA_EMU_UNSAFE, a
 *          negative control for tests: as OVERLAP but a slot is recycled
 *          without waiting for the step that reads it and is filled with NaN
 *          before its next copy, so results are wrong (never a fault: every
 *          access stays inside the caller's buffers).
 * Each step's enqueue is bracketed by a roctx range "ring fwd|bwd step s:
 * block kb" (host side; shown by a profiler's marker trace). */
enum { RA_EMU_OVERLAP = 0, RA_EMU_SERIALIZE = 1, RA_EMU_UNSAFE = 2 };

int ring_emu_fwd(const void* q, const void* const* kv_pool, void* slot0,
                 void* slot1, int ring_rank, int ring_size, int causal,
                 int q_chunk, int k_chunk, float* o_acc, float* lse_acc,
                 const ra_dims* dims, const int32_t* order, int mode,
                 void* main_stream, void* side_stream);

/* Backward share through the emulator.  For each step the block's travelling
 * dK/dV partial dkv_pool[kb] (fp32 [2,B,Hkv,Lk,d], device) is brought into a
 * receive slot with the key/value block, this member's contribution is added
 * there, and the slot is copied back to dkv_pool[kb] (the hop to the next
 * member), so on return dkv_pool[kb] += this member's dK/dV for every block
 * it sees, in ring order.  dq_acc += the member's dQ.  dkv_slot0/1 are two
 * fp32 device buffers of one dK/dV block each.  lse and delta are those of
 * the finished forward share (ring_attn_bwd_prep).  work / work_bytes: the
 * optional dK/dV workspace of ring_attn_bwd_ws (NULL / 0 for none), reused
 * by every block; it must not overlap any other buffer of the share. */
int ring_emu_bwd(const void* q, const void* const* kv_pool, void* slot0,
                 void* slot1, const void* dout, const float* lse,
                 const float* delta, float* const* dkv_pool, float* dkv_slot0,
                 float* dkv_slot1, int ring_rank, int ring_size, int causal,
                 int q_chunk, int k_chunk, float* dq_acc, void* work,
                 int64_t work_bytes, const ra_dims* dims, const int32_t* order,
                 int mode, void* main_stream, void* side_stream);

/* ---- kernel timing (diagnostics) ---------------------------------------
 * While enabled, each attention kernel the library launches is bracketed by
 * a pair of HIP events recorded on the stream the kernel runs on.  Kernel
 * families: "fwd_bf16", "fwd_fp32", "bwd_dq", "bwd_dkv", "fwd_decode" (the
 * split kernel of ring_attn_fwd_decode), "decode_fold" (its fold), and
 * "ffn_up" / "ffn_down" (the two products of ring_ffn_fwd, per chunk),
 * "ffn_bwd_gemm" / "ffn_bwd_aux" (ring_ffn_bwd's products, and its
 * transposes and activation-gradient passes, in groups).
 * ring_attn_timing_enable(on): on != 0 discards earlier records and starts
 * collecting; 0 stops collecting (records are kept).
 * ring_attn_timing_read(name, &launches, &total_ms): waits for the recorded
 * events of that family and returns the launch count and summed durations.
 * Returns RA_ERR_INVALID for an unknown family or NULL outputs. */
int ring_attn_timing_enable(int on);
int ring_attn_timing_read(const char* name, int* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* RING_ATTN_H */
