/*
 * ring_attn.h -- C ABI of the MI355X (gfx950) ring-attention step library.
 *
 * The method (close-reading notes on "Ring Attention with Blockwise
 * Transformers for Near-Infinite Context", llm-papers-study, §3.1-§3.5):
 * the sequence is split into D equal blocks, one per host of a logical ring.
 * A host keeps its query block Q_r and, round after round, computes blockwise
 * attention of Q_r against the key/value block it currently holds while
 * forwarding that block to the next host and receiving the previous host's
 * (§3.2).  Blocks may be absorbed in any order as long as the per-row
 * statistics (running max and running sum) rescale what was accumulated
 * (§3.1), so the result is exact attention, not an approximation
 * ("什么是环形注意力（Ring Attention）？", aiboss88 wiki, "边界与常见误解").
 *
 * This library runs ONE rank's share of that ring on one GPU.  The link to the
 * previous host is emulated by an asynchronous device-to-device copy of the
 * next K/V block into a double-buffered staging area on a library-owned side
 * stream, overlapped with the attention kernel of the current block on the
 * caller's stream (the "six resident blocks" budget of §3.4: Q, O, the K/V
 * block in use and the K/V block in flight).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Batch is 1.  Layouts are token-major and dense:
 *      q, dout, out, dq        [block_len][heads][head_dim]
 *      each K/V block, dk, dv  [block_len][kv_heads][head_dim]
 *      lse                     [heads][block_len]
 *  - bf16 entry points take bfloat16 q/k/v/dout; *_f32 twins take float32.
 *    out, lse and all gradients are float32 in both.
 *  - Scores are scaled by 1/sqrt(head_dim).  lse is the natural log of the
 *    sum of exp(scaled score) over the visible keys of the row.
 *  - Query head h uses K/V head h / (heads / kv_heads) (contiguous groups).
 *  - causal != 0: key position p_k is visible to query position p_q iff
 *    p_k <= p_q, where block j covers positions j*block_len .. (j+1)*block_len-1.
 *  - k_blocks / v_blocks / dk_blocks / dv_blocks are HOST arrays of n_blocks
 *    DEVICE pointers, indexed by sequence block id j (not by arrival order).
 *  - stream is a hipStream_t (NULL = the legacy default stream).  Every call
 *    only enqueues work and returns; the caller orders against `stream` only.
 *    Library side-stream copies first wait for everything already enqueued on
 *    `stream`, and `stream` waits for the side stream before the call returns.
 *  - Pointers are caller-owned device memory (no ownership transfer).  The
 *    library owns one side stream, a few events and the K/V staging buffers
 *    per device (created lazily, released by ring_attn_shutdown).
 *  - Calls on one device share the library's staging and workspace buffers.
 *    Calls issued on different streams of the device are serialised on the
 *    GPU: a call's work starts only after the previous call's work (on
 *    whichever stream it was issued) has finished, so they never race; the
 *    price is that they do not overlap.  ring_attn_merge uses no library
 *    buffer and is not ordered against other calls.
 *  - Errors: every entry point returns RA_OK (0) or an ra_status code and
 *    never aborts.  Arguments are validated on the host before anything is
 *    enqueued; on a validation error nothing is enqueued and no output is
 *    touched.  ring_attn_last_error() returns a message for the last failure
 *    on the calling thread.
 */
#ifndef RING_ATTN_H
#define RING_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* ra_stream_t; /* hipStream_t */

typedef enum {
  RA_OK = 0,
  RA_ERR_INVALID_ARG = 1, /* null pointer, bad size/rank, aliasing */
  RA_ERR_UNSUPPORTED = 2, /* head_dim not in {64, 128}            */
  RA_ERR_HIP = 3,         /* a HIP runtime call failed             */
  RA_ERR_OOM = 4          /* staging allocation failed             */
} ra_status;

/*
 * ring_attn_fwd -- one rank's forward ring step (bf16 inputs).
 *
 * Computes exact attention of this rank's query block over every visible K/V
 * block, visiting them in ring order: round s uses block (rank - s) mod
 * n_blocks (round 0 is the rank's own block, §3.5 walk-through).  With causal
 * != 0, rounds whose block lies in the future (j > rank) are skipped and the
 * rank's own (diagonal) block is masked.  Rounds s >= 1 read their block from
 * a staging buffer filled by the side-stream copy started while round s-1
 * computes.  Each round folds its block into (out, lse) with the rescaled
 * merge of §3.1, so after the last round out/lse hold the final result.
 *
 *   q          device, bf16 [block_len][heads][head_dim], this rank's Q block
 *   k_blocks   host array[n_blocks] of device bf16 [block_len][kv_heads][head_dim]
 *   v_blocks   likewise for V
 *   n_blocks   ring size D >= 1;   0 <= rank < n_blocks
 *   block_len  tokens per block, >= 1 (any value; tiles are ragged-safe)
 *   heads, kv_heads  heads % kv_heads == 0;   head_dim in {64, 128}
 *   out        device, fp32 [block_len][heads][head_dim], overwritten
 *   lse        device, fp32 [heads][block_len], overwritten
 * out/lse must not overlap q or any K/V block.
 */
int ring_attn_fwd(const void* q, const void* const* k_blocks, const void* const* v_blocks,
                  int n_blocks, int block_len, int heads, int kv_heads, int head_dim,
                  int causal, int rank, float* out, float* lse, ra_stream_t stream);

/* Same as ring_attn_fwd with float32 q and K/V blocks (fp32 MFMA throughout). */
int ring_attn_fwd_f32(const float* q, const float* const* k_blocks, const float* const* v_blocks,
                      int n_blocks, int block_len, int heads, int kv_heads, int head_dim,
                      int causal, int rank, float* out, float* lse, ra_stream_t stream);

/*
 * ring_attn_merge -- combine two normalised partial results over disjoint key
 * sets (the statistic merge of §3.1 in log form):
 *   lse = log(exp(lse_a) + exp(lse_b))
 *   out = exp(lse_a - lse) * out_a + exp(lse_b - lse) * out_b
 * A partial with lse = -inf is empty (weight 0); two empty partials give
 * out = 0, lse = -inf.  All buffers fp32 on the device:
 *   out_a, out_b, out  [rows][heads][head_dim]     lse_a, lse_b, lse [heads][rows]
 * out/lse may alias out_a/lse_a or out_b/lse_b exactly (in-place merge);
 * partial overlaps are rejected.  rows >= 0 (0 is a no-op), heads >= 1,
 * head_dim >= 1.
 */
int ring_attn_merge(const float* out_a, const float* lse_a, const float* out_b,
                    const float* lse_b, int rows, int heads, int head_dim, float* out, float* lse,
                    ra_stream_t stream);

/*
 * ring_attn_bwd -- one rank's backward ring step (bf16 inputs), recomputing the
 * attention probabilities from the saved lse of the forward.  The method is a
 * training method: the ring runs inside every transformer layer (close-reading
 * notes, abstract and the §3.5 algorithm), so the gradients flow through the
 * same blockwise ring as the forward, with the same K/V rotation.
 *
 * With P = softmax of the visible scaled scores (rebuilt as exp(S - lse)),
 * Delta_i = sum_d dout_i * out_i, dS = P * (dout V^T - Delta):
 *   dq               = sum over visible blocks of dS K / sqrt(d)   (OVERWRITTEN)
 *   dk_blocks[j]    += dS^T q / sqrt(d)   for every visible block j  (ACCUMULATED)
 *   dv_blocks[j]    += P^T dout                                     (ACCUMULATED)
 * K/V blocks travel the same ring (same schedule and staging) as the forward.
 * For grouped heads the dk/dv of a K/V head sum over its query heads.  Run
 * over every rank, the accumulated dk/dv are the full-sequence gradients; the
 * caller zeroes them once before the first rank.
 *
 * Precision: the kernels convert q, the K/V blocks and dout exactly to IEEE
 * half and run every contraction on fp16 matrix cores with fp32
 * accumulation, so the probabilities and dS they round for the matrix core
 * keep 11 significant bits (bf16 would keep 8).  Inputs must be finite and
 * below 65504 in magnitude (the half range), as must dS; values below 2^-14
 * keep an absolute step of 2^-24.  The library holds, per device, a
 * workspace of the row terms (8 bytes per query row and head) and the half
 * copies of q, dout and one K/V block.
 *
 *   out, lse   the forward's fp32 outputs for this rank
 *   dout       device, bf16 [block_len][heads][head_dim]
 *   dq         device, fp32 [block_len][heads][head_dim]
 *   dk_blocks, dv_blocks  host arrays[n_blocks] of device fp32
 *              [block_len][kv_heads][head_dim]
 * Other arguments as ring_attn_fwd.  Gradient buffers must not overlap inputs.
 */
int ring_attn_bwd(const void* q, const void* const* k_blocks, const void* const* v_blocks,
                  const float* out, const void* dout, const float* lse, int n_blocks,
                  int block_len, int heads, int kv_heads, int head_dim, int causal, int rank,
                  float* dq, float* const* dk_blocks, float* const* dv_blocks,
                  ra_stream_t stream);

/* Same as ring_attn_bwd with float32 q, K/V blocks and dout. */
int ring_attn_bwd_f32(const float* q, const float* const* k_blocks, const float* const* v_blocks,
                      const float* out, const float* dout, const float* lse, int n_blocks,
                      int block_len, int heads, int kv_heads, int head_dim, int causal, int rank,
                      float* dq, float* const* dk_blocks, float* const* dv_blocks,
                      ra_stream_t stream);

/*
 * Zig-zag (load-balanced causal) layout of the same two steps.  The sequence
 * is cut into 2 * n_blocks chunks of block_len / 2 tokens; block b -- rank b's
 * query block and K/V block b alike -- holds chunk b in its first half and
 * chunk 2 * n_blocks - 1 - b in its second half.  With a causal mask every
 * rank then owns the same amount of work (each ring round pairs one early
 * and one late chunk), instead of rank r doing r + 1 rounds of the
 * contiguous layout; the ring visits every block in every rank.  Chunk pairs
 * are the units of work: a key chunk later than the query chunk is skipped,
 * the same chunk is the masked diagonal, an earlier one is full.  Where one
 * query chunk sees both key chunks of a block off the diagonal (for dK/dV:
 * one key chunk is seen by both query chunks), the two pairs run as one step
 * over the whole block, so a round is never split into more kernel steps than
 * its diagonal requires.
 * Arguments, layouts, ownership and errors are those of ring_attn_fwd and
 * ring_attn_bwd (bf16), except that block_len must be even
 * (RA_ERR_INVALID_ARG otherwise) and row i of every per-block tensor sits at
 * the global position of its chunk.
 */
int ring_attn_fwd_zigzag(const void* q, const void* const* k_blocks, const void* const* v_blocks,
                         int n_blocks, int block_len, int heads, int kv_heads, int head_dim,
                         int causal, int rank, float* out, float* lse, ra_stream_t stream);
int ring_attn_bwd_zigzag(const void* q, const void* const* k_blocks, const void* const* v_blocks,
                         const float* out, const void* dout, const float* lse,
                         int n_blocks, int block_len, int heads, int kv_heads, int head_dim,
                         int causal, int rank, float* dq, float* const* dk_blocks,
                         float* const* dv_blocks, ra_stream_t stream);

/*
 * The ring order used by ring_attn_fwd/ring_attn_bwd for one rank: writes the
 * sequence-block id of every executed round to steps[0..] (round s uses block
 * (rank - s) mod n_blocks; causal drops blocks j > rank) and returns the number
 * of rounds, or a negative ra_status on bad arguments (steps may be NULL to
 * query the count; otherwise it must hold max_steps >= the count).
 */
int ring_attn_schedule(int rank, int n_blocks, int causal, int* steps, int max_steps);

/*
 * Diagnostics for the rotation pipeline (off by default):
 *   poison != 0     after a staging buffer's last reader finishes, fill it with
 *                   NaN bytes on the side stream before its next copy, so any
 *                   read that escapes the event ordering shows up as NaN;
 *   delay_cycles>0  spin the side stream for that many GPU clock cycles before
 *                   every staging copy (a slow link); results must not change.
 * Applies to subsequent calls from any thread.
 */
int ring_attn_debug(int poison, long long delay_cycles);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char* ring_attn_last_error(void);

/*
 * Bytes of library-owned staging for a block shape: two K and two V blocks.
 * This is the resident-block budget of the close-reading notes, §3.4: besides
 * Q and the output, a host holds the K/V block in use and the K/V block in
 * flight from the previous host (the block in use by the kernel is either the
 * rank's own or a staged one; the in-flight block goes to the other half).
 * elem_bytes is 2 (bf16) or 4.  Returns 0 for non-positive sizes or an
 * elem_bytes other than 2 or 4.
 */
size_t ring_attn_workspace_bytes(int block_len, int kv_heads, int head_dim, int elem_bytes);

/*
 * Hand the library caller-owned device memory (on the current device) to use
 * as the K/V staging instead of its own lazily allocated buffer.  `dev_ptr`
 * must be 256-byte aligned and stay valid until it is replaced, reset or
 * ring_attn_shutdown() runs; the library never frees it.  Calls whose shape
 * needs more than `bytes` (ring_attn_workspace_bytes) return
 * RA_ERR_INVALID_ARG and enqueue nothing.  (NULL, 0) returns to library-owned
 * staging.  The call synchronises the device first, so no earlier call still
 * uses the old buffer, and frees the library's own buffer if it had one.
 * The backward's workspace (row terms and half copies) stays library-owned.  Errors: RA_ERR_INVALID_ARG (pointer/size mismatch,
 * misalignment), RA_ERR_HIP.
 */
int ring_attn_set_workspace(void* dev_ptr, size_t bytes);

/*
 * Profiling of the library's own launches (measurement support).  While
 * enabled, the library records HIP events around every attention kernel it
 * launches (on the stream it launches on) and around every staging copy (on
 * the side stream).  ring_attn_profile_read() synchronises those events and
 * fills, for each kind, the summed duration in milliseconds and the count:
 *   kinds: 0 = forward step kernel, 1 = backward dK/dV kernel,
 *          2 = backward dQ kernel, 3 = backward preprocess kernel,
 *          4 = merge kernel, 5 = staging copy (K+V of one block),
 *          6 = decode partial kernel, 7 = decode merge kernel,
 *          8 = feedforward up-projection GEMM, 9 = down-projection GEMM
 * and `hidden_ms`, the part of all copy time that overlaps a kernel interval
 * of the same call (copy/compute overlap on the device timeline).
 * `ms` and `count` must hold at least 10 entries.  Reading resets the records.
 */
int ring_attn_profile_enable(int enable);
int ring_attn_profile_read(double* ms, int* count, double* copy_ms, double* hidden_ms);

/*
 * ring_attn_decode -- long-context decode: a few new query rows against the
 * whole context held as ring blocks (inference use of the method; the
 * per-block statistics combine exactly with the merge of §3.1).  Each host
 * keeps its K/V block; only the few query rows and their per-block partials
 * move, so the step reads every K/V byte once and is HBM-bound.  On one GPU
 * all blocks are processed by one split-key launch (one wavefront per K/V
 * head and key chunk of a block) followed by a log-sum-exp merge of the
 * partials.
 *
 *   q          device, bf16 [q_len][heads][head_dim]; query i sits at global
 *              position q_pos0 + i
 *   k_blocks   host array[n_blocks] of device bf16 [block_len][kv_heads][head_dim];
 *   v_blocks   key t of block j sits at global position j * block_len + t
 *   n_blocks   1 .. 64;  block_len >= 1;  q_len >= 1;  q_pos0 >= 0
 *   heads, kv_heads  heads % kv_heads == 0 and heads / kv_heads <= 32
 *              (RA_ERR_UNSUPPORTED otherwise);  head_dim in {64, 128}.  One pass
 *              serves at most 32 query rows per K/V head ((heads / kv_heads) x
 *              rows); a longer q_len runs as successive passes of
 *              floor(32 / (heads / kv_heads)) rows, each of which streams the K/V
 *              blocks again
 *   out        device, fp32 [q_len][heads][head_dim], overwritten
 *   lse        device, fp32 [heads][q_len] (natural log), overwritten
 * A key is visible to a query iff its position is <= the query's (q_pos0 >=
 * n_blocks * block_len - 1 makes every key visible).  A row with no visible
 * key gets out = 0 and lse = -inf.  out/lse must not overlap each other, q or
 * any K/V block.  The library keeps a lazily grown device buffer for the
 * partials (about kv_heads * partials * rows * (head_dim + 1) floats).
 * Errors: RA_ERR_INVALID_ARG, RA_ERR_UNSUPPORTED, RA_ERR_OOM, RA_ERR_HIP;
 * nothing is enqueued on error.
 */
int ring_attn_decode(const void* q, const void* const* k_blocks, const void* const* v_blocks,
                     int n_blocks, int block_len, int q_len, int heads, int kv_heads, int head_dim,
                     long long q_pos0, float* out, float* lse, ra_stream_t stream);

/*
 * ring_attn_decode_noalloc -- ring_attn_decode for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments, layouts, results and
 * errors as ring_attn_decode (it runs the same kernels), but the split-key
 * partials go to a fixed device array compiled into the library,
 * RA_DECODE_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends,
 * instead of a lazily grown buffer; the call performs no allocation and
 * creates no library stream or event.  A shape whose partials need more than
 * that (about kv_heads * partials * rows * (head_dim + 1) floats; the 512k
 * GQA 32/8 workload with 4 query rows needs 8.5 MB) returns
 * RA_ERR_INVALID_ARG and enqueues nothing.  Every such call on one GPU shares
 * the array, which keeps the last call's contents: calls that overlap in time
 * on one GPU (different streams) race on it and must be serialised by the
 * caller; unlike the other entry points this one is not ordered against
 * other library calls.
 */
#define RA_DECODE_NOALLOC_SCRATCH_BYTES (32u << 20)
int ring_attn_decode_noalloc(const void* q, const void* const* k_blocks, const void* const* v_blocks,
                             int n_blocks, int block_len, int q_len, int heads, int kv_heads,
                             int head_dim, long long q_pos0, float* out, float* lse,
                             ra_stream_t stream);

/*
 * ring_attn_ffn_blockwise -- the feedforward half of a blockwise transformer
 * layer, computed block by block ("Ring Attention with Blockwise Transformers
 * for Near-Infinite Context" close-reading notes, §2.2: computing the
 * feedforward in blocks caps its largest activation at one block of the
 * 4h-wide intermediate rather than the whole sequence's):
 *
 *   y = GELU(x W1^T + b1) W2^T + b2        GELU(z) = z * Phi(z) (exact, erf form)
 *
 *   x    device bf16 [rows][hidden]     (e.g. a rank's attention block, rows = block_len)
 *   w1   device bf16 [ffn][hidden]      w2  device bf16 [hidden][ffn]   (weights [out][in])
 *   b1   device fp32 [ffn] or NULL      b2  device fp32 [hidden] or NULL
 *   y    device fp32 [rows][hidden], overwritten; must not overlap any input
 *   chunk_rows  rows per block (0 = all rows at once).  The library keeps one
 *        bf16 [chunk_rows][ffn] intermediate, rounds GELU's output to bf16
 *        there, and runs two MFMA GEMMs per chunk on `stream`.
 * hidden and ffn must be positive multiples of 128 (RA_ERR_UNSUPPORTED);
 * rows >= 1; operands must stay under 4 GiB each (RA_ERR_INVALID_ARG).
 * Errors: RA_ERR_INVALID_ARG, RA_ERR_UNSUPPORTED, RA_ERR_OOM, RA_ERR_HIP;
 * nothing is enqueued on error.
 */
int ring_attn_ffn_blockwise(const void* x, const void* w1, const float* b1, const void* w2,
                            const float* b2, int rows, int hidden, int ffn, int chunk_rows,
                            float* y, ra_stream_t stream);

/*
 * Matrix-core rate probe (measurement support): runs RA_MFMA_RATE_SINK_FLOATS
 * workgroups of 8 waves, each wave issuing `iters` rounds of four independent
 * bf16 32x32x16 MFMAs from registers, on `stream`, and waits for it.  Writes
 * the achieved dense bf16 TFLOP/s to *tflops: the practical ceiling at the
 * clock the card sustains under matrix load.  `sink` is caller device memory
 * of RA_MFMA_RATE_SINK_FLOATS floats that receives one checksum per
 * workgroup.  Errors: RA_ERR_INVALID_ARG (iters outside [1, 2^24], NULL
 * pointers), RA_ERR_HIP.
 */
#define RA_MFMA_RATE_SINK_FLOATS 1024
int ring_attn_mfma_rate(int iters, float* sink, double* tflops, ra_stream_t stream);

/* Release every library-owned stream, event and staging buffer (all devices). */
void ring_attn_shutdown(void);

#ifdef __cplusplus
}
#endif

#endif /* RING_ATTN_H */
