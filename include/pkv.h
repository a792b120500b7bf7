/*
 * pkv.h - single-token decode attention over a block-paged KV cache, for AMD
 * Instinct MI355X (gfx950).  C ABI; every entry point is extern "C".
 *
 * The problem, as the pages state it:
 *   - spindle, "Paging": each sequence's keys/values live in fixed-size blocks
 *     (16 tokens) drawn from a shared pool and are addressed through a
 *     per-sequence block table; forked sequences share blocks copy-on-write
 *     through reference counts.
 *   - spindle, "Two bugs worth recording": where a write lands and how many
 *     tokens a read covers are arguments, and lengths move forward in the
 *     caller, once per step, never in the cache.  Nothing here ever infers or
 *     advances a length.
 *   - mlsystems topic listing, flash-decoding entry: at q_len = 1 the KV
 *     length is split into partitions processed in parallel, whose partial
 *     results are merged afterwards (log-sum-exp combine).
 *
 * Layout (one transformer layer; every call works on one layer's caches):
 *   k_cache, v_cache : [num_blocks][num_kv_heads][block_size][head_dim]
 *                      elements of `dtype`, contiguous.  Block b, KV head h
 *                      is one contiguous run of block_size * head_dim
 *                      elements.
 *   block_tables     : int32 [batch][bt_stride], row s = sequence s's
 *                      physical block ids in logical order; each row holds
 *                      bt_stride entries, so a sequence can hold at most
 *                      bt_stride * block_size tokens.
 *   context_lens     : int32 [batch], tokens each sequence attends to.
 *   q                : [batch][num_q_heads][head_dim] of `dtype`.
 *   out              : float32 [batch][num_q_heads][head_dim].
 *   lse              : float32 [batch][num_q_heads], natural-log
 *                      log-sum-exp of the scaled scores.
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 *
 * Pointers are device pointers unless marked "host".  The caller owns and
 * allocates every buffer (workspace included); the library allocates no
 * device memory and keeps no state between calls.  Work is enqueued on
 * `stream` (a hipStream_t; NULL = the null stream) and returns without
 * synchronising; buffers must stay alive until the stream has finished.
 *
 * Errors: each call returns PKV_OK (0) or a negative PKV_ERR_* code after
 * checking its host-side arguments; nothing is enqueued on error.  Device
 * data (block ids, positions, lengths) is checked by the kernels themselves:
 * an out-of-range value is never dereferenced; the offending unit is skipped
 * or clamped and a bit is set in a per-device error word that
 * pkv_device_error() reads back.  Outputs of a call that set such a bit are
 * unspecified.
 *
 * Supported shapes: block_size 16; head_dim 64 or 128; num_q_heads a
 * multiple of num_kv_heads with a group size of 1..8; partition_size 0 or a
 * multiple of 16.  dtype PKV_F32 or PKV_BF16 (bfloat16 bit patterns).
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* pkv_stream_t; /* hipStream_t */

typedef enum pkv_dtype { PKV_F32 = 0, PKV_BF16 = 1 } pkv_dtype;

enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_NULL = -1,          /* a required pointer is NULL                     */
  PKV_ERR_DTYPE = -2,         /* unknown dtype                                  */
  PKV_ERR_SHAPE = -3,         /* unsupported size/shape combination             */
  PKV_ERR_WORKSPACE = -4,     /* workspace missing or smaller than required     */
  PKV_ERR_LAUNCH = -5,        /* the HIP runtime rejected a launch              */
  PKV_ERR_DEVICE = -6,        /* a HIP runtime call failed                      */
  PKV_ERR_OUT_OF_BLOCKS = -7, /* block manager: pool exhausted (nothing changed)*/
  PKV_ERR_ARG = -8,           /* bad argument value (alignment, range, id)      */
  PKV_ERR_SCRATCH = -9        /* needs more than PKV_STATIC_SCRATCH_BYTES       */
};

/* Size of the library's static per-device scratch buffer (see
 * pkv_append_paged_decode_static). */
#define PKV_STATIC_SCRATCH_BYTES ((size_t)16 << 20)

/* Bits of the device error word. */
enum pkv_device_error_bits {
  PKV_DEVERR_BLOCK_ID = 1,      /* a block-table entry outside [0, num_blocks)   */
  PKV_DEVERR_POSITION = 2,      /* an append position outside the table row      */
  PKV_DEVERR_CONTEXT = 4,       /* context_lens[s] < 0 or > bt_stride*block_size */
  PKV_DEVERR_MAX_CONTEXT = 8,   /* context_lens[s] > the max_context_len given   */
  PKV_DEVERR_CU = 16,           /* cu_new_tokens not non-decreasing / bad total  */
  PKV_DEVERR_GROUPS = 32        /* fork groups do not tile the batch in order    */
};

/* Library version, e.g. 100 for 1.0.0. */
int pkv_version(void);

/* Static description of a status code. Never NULL. */
const char* pkv_status_string(int status);

/*
 * KV append (spindle, "Two bugs worth recording": the write position is an
 * argument, never derived from a stored length).
 *
 * For each sequence s and i in [0, cu_new_tokens[s+1] - cu_new_tokens[s]):
 *   pos = start_pos[s] + i,
 *   block = block_tables[s][pos / block_size], slot = pos % block_size,
 *   k_cache[block][h][slot][:] = k_new[cu_new_tokens[s] + i][h][:]  for every
 *   KV head h, and the same for v.
 * A bit-exact copy; no other cache element is written; no length is read or
 * advanced.  The target blocks must be exclusively owned by s (copy-on-write
 * already resolved) and distinct across sequences, otherwise writes race.
 *
 *   k_new, v_new    : [total_new][num_kv_heads][head_dim] of dtype.
 *   start_pos       : int32 [batch].
 *   cu_new_tokens   : int32 [batch + 1], cu[0] = 0, non-decreasing,
 *                     cu[batch] = total_new.
 * total_new = 0 is a no-op.
 */
int pkv_kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                  const int32_t* block_tables, int64_t bt_stride, const int32_t* start_pos,
                  const int32_t* cu_new_tokens, int32_t batch, int32_t total_new,
                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                  int32_t num_blocks, int32_t dtype, pkv_stream_t stream);

/*
 * Bytes of device workspace the decode calls need (> 0 whenever batch > 0):
 * the work plan (a count and batch * P unit entries) and, when the context is
 * split into P = ceil(max_context_len / partition_size) > 1 partitions, the
 * per-partition partial outputs and log-sum-exps, batch * num_q_heads * P *
 * (head_dim + 1) floats, and batch * num_q_heads int32 merge counters; each
 * part 256-byte aligned.  The workspace itself must be 256-byte aligned.
 */
size_t pkv_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t head_dim,
                                  int32_t max_context_len, int32_t partition_size);

/*
 * A partition size for pkv_paged_decode and its variants, from the crossover the first
 * pass measures on MI355X (uniform and long-tailed lengths, 1 to 256 sequences, 512 to
 * 32768 tokens; mlsystems topic listing, flash-decoding entry: past some point, splitting
 * the KV length beats one unit per sequence):
 *   - 0 (one unit per sequence and KV head) when max_context_len <= 512, or when
 *     batch * num_kv_heads >= 512 (two units per compute unit already);
 *   - else P = the power of two in [256, 8192] at or below the call's K/V bytes divided
 *     by 256 units (about one per compute unit), counted in tokens of a 128-dim head:
 *     total_context_tokens * num_kv_heads * head_dim / 32768;
 *   - raised to the smallest power of two that leaves at most 8 partitions per sequence
 *     (merged inside the pass, no combine launch) when that at most doubles it;
 *   - 0 when P >= max_context_len.
 * total_context_tokens: sum of the batch's context lengths, as the host knows it; <= 0
 * takes batch * max_context_len.  A host computation: no device access, no error.
 */
int32_t pkv_decode_partition_size(int32_t batch, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_context_len, int64_t total_context_tokens);

/*
 * Which engine runs the first pass of pkv_paged_decode and its variants for these
 * shapes: PKV_ENGINE_VALU (the vector-ALU pass, decode_pass1_kernel) or
 * PKV_ENGINE_MATRIX (the bf16 matrix-core tile, decode_mfma_kernel, used when a KV
 * head serves 7 or 8 query heads).  Both compute the same attention; the choice
 * follows a measured sweep over group sizes on MI355X.  A host computation:
 * PKV_ERR_DTYPE or PKV_ERR_SHAPE for shapes the decode calls refuse.
 */
#define PKV_ENGINE_VALU 0
#define PKV_ENGINE_MATRIX 1
int32_t pkv_decode_engine(int32_t kv_dtype, int32_t head_dim, int32_t num_q_heads,
                          int32_t num_kv_heads);

/*
 * Work plan of the decode's first pass, written into `workspace`: the
 * (sequence, partition) units in longest-first order (every full partition,
 * then the last partition of every split sequence, so that its merge is done
 * early, then the other sequences by decreasing length).  The
 * order decides only which workgroup runs when; results never depend on it.
 * Reads context_lens; lengths are clamped to bt_stride * 16.  A plan stays
 * valid for every pkv_paged_decode_planned call with the same context_lens
 * contents, batch, max_context_len, partition_size and workspace, e.g. all the
 * layers of one decode step.
 */
int pkv_decode_plan(void* workspace, size_t workspace_bytes, const int32_t* context_lens,
                    int64_t bt_stride, int32_t batch, int32_t num_q_heads, int32_t head_dim,
                    int32_t max_context_len, int32_t partition_size, pkv_stream_t stream);

/*
 * Paged decode attention (spindle: gather by block table with an explicit
 * length, then attend; flash-decoding split for long contexts).
 *
 * For each sequence s with n = context_lens[s] and each query head h
 * (KV head kh = h / G):
 *   score_t = scale * dot(q[s][h], K_s[kh][t]),  t in [0, n),
 *   out[s][h] = sum_t softmax(score)_t * V_s[kh][t],
 *   lse[s][h] = ln sum_t exp(score_t),
 * where K_s[kh][t] = k_cache[block_tables[s][t / 16]][kh][t % 16].
 * n = 0 gives out = 0 and lse = -inf.  Slots at or past n (the unused tail
 * of the last block, stale or NaN data) never influence the result.
 *
 * max_context_len (host) must be >= every context_lens[s]; it sizes the grid
 * so that no device-to-host synchronisation is needed.
 * partition_size = 0: one pass per (sequence, KV head) over the whole
 * context.  partition_size = P > 0 (multiple of 16): the context is split
 * into partitions of P tokens, each attended independently, then merged by
 * their log-sum-exps, in the same launch: the last of a sequence's partition
 * workgroups to finish (a per-(sequence, KV head) counter in the workspace)
 * merges them, with the arithmetic and order of pkv_lse_combine, so the
 * result equals pkv_paged_decode_partials followed by pkv_lse_combine bit for
 * bit.  Past 8 partitions per sequence the merge is a second launch (the
 * combine kernel, same result), whose rows run in parallel.  Sequences that
 * fit in one partition are written directly.  Calls
 * that overlap in time must not share a workspace.  Ordering of the in-launch
 * merge: each split unit writes its partial result with device-scope stores,
 * waits until they have completed, then takes a ticket from a device-scope
 * counter with a relaxed atomic; the last ticket's workgroup reads the slots with
 * device-scope loads.  There is no release/acquire fence (on gfx950 those write
 * back and invalidate the whole L2 of an XCD); the ordering rests on how gfx950
 * completes device-scope stores before the wait returns, which is why the
 * library builds for gfx950 only.  The result does not depend on
 * the batch: a sequence decoded alone or in any batch, with the same
 * partition_size, gives bit-identical out and lse.
 * lse may be NULL.  workspace: pkv_decode_workspace_bytes(...) bytes,
 * 256-byte aligned, owned by the caller; its previous contents do not matter.
 * Launches, on `stream`: the plan kernel (which also zeroes the merge
 * counters), the first pass, and past 8 partitions the combine.
 */
int pkv_paged_decode(float* out, float* lse, const void* q, const void* k_cache,
                     const void* v_cache, const int32_t* block_tables, int64_t bt_stride,
                     const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int32_t num_blocks, int32_t max_context_len, float scale,
                     int32_t partition_size, void* workspace, size_t workspace_bytes,
                     int32_t dtype, pkv_stream_t stream);

/*
 * One decode step in fewer launches: exactly pkv_kv_append(k_cache, v_cache,
 * k_new, v_new, block_tables, bt_stride, start_pos, cu_new_tokens, batch,
 * total_new, ...) followed by pkv_paged_decode(...) on the same stream, with
 * the same arguments, results and errors.  The append and the work plan share
 * one launch (they touch disjoint memory), then comes the first pass, which
 * also merges split sequences.  context_lens must already count the appended
 * tokens; the caller advances lengths, never the library.
 */
int pkv_append_paged_decode(float* out, float* lse, const void* q, void* k_cache, void* v_cache,
                            const void* k_new, const void* v_new, const int32_t* block_tables,
                            int64_t bt_stride, const int32_t* start_pos,
                            const int32_t* cu_new_tokens, int32_t total_new,
                            const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t num_blocks, int32_t max_context_len, float scale,
                            int32_t partition_size, void* workspace, size_t workspace_bytes,
                            int32_t dtype, pkv_stream_t stream);

/*
 * pkv_append_paged_decode without a workspace argument, for callers that cannot
 * allocate device memory: code being captured into a HIP graph, tight serving
 * loops, harnesses that forbid hipMalloc.  Nothing is allocated: the plan,
 * partial results and merge counters live in a static device array of
 * PKV_STATIC_SCRATCH_BYTES bytes per GPU, which the library holds until the
 * process ends.  Its device address is looked up once per device, on the first
 * call made with that device current.  Arguments, results and device errors are
 * those of pkv_append_paged_decode.  A call whose workspace
 * (pkv_decode_workspace_bytes of the same sizes) would exceed
 * PKV_STATIC_SCRATCH_BYTES returns PKV_ERR_SCRATCH and enqueues nothing.  Every
 * call on one GPU uses the same array, and each call rewrites what it reads
 * (its plan and merge counters are set by its own first launch): calls that
 * overlap in time on one GPU (two streams, or two host threads) race and must
 * be serialised by the caller.
 */
int pkv_append_paged_decode_static(float* out, float* lse, const void* q, void* k_cache,
                                   void* v_cache, const void* k_new, const void* v_new,
                                   const int32_t* block_tables, int64_t bt_stride,
                                   const int32_t* start_pos, const int32_t* cu_new_tokens,
                                   int32_t total_new, const int32_t* context_lens,
                                   int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                   int32_t max_context_len, float scale,
                                   int32_t partition_size, int32_t dtype, pkv_stream_t stream);

/*
 * One decode step of one layer in one launch, on a plan made beforehand: exactly
 * pkv_kv_append(...) followed by pkv_paged_decode_planned(...) with the same arguments,
 * results and errors.  The plan must come from pkv_decode_plan on the same stream, into
 * the same workspace, for the same context_lens contents, batch, max_context_len and
 * partition_size; one plan serves every layer of a step (lengths advance once per step,
 * spindle, "Two bugs worth recording").  The first pass writes the new tokens itself:
 * sequence s's token i (row cu_new_tokens[s] + i of k_new / v_new, [total_new,
 * num_kv_heads, head_dim]) goes to position start_pos[s] + i, explicit, never inferred;
 * the workgroup whose token range holds that position stores it before streaming, and
 * a position past context_lens[s] is stored by the sequence's last workgroup.  No other
 * sequence of the call may attend an appended slot (copy-on-write: a block held by
 * several sequences is copied with pkv_copy_blocks before it is written).  Device
 * errors (bad cu_new_tokens, positions outside the table row, block ids outside the pool)
 * set the same bits as pkv_kv_append.  Past 8 partitions per sequence the combine
 * follows as a second launch.
 */
int pkv_append_paged_decode_planned(float* out, float* lse, const void* q, void* k_cache,
                                    void* v_cache, const void* k_new, const void* v_new,
                                    const int32_t* block_tables, int64_t bt_stride,
                                    const int32_t* start_pos, const int32_t* cu_new_tokens,
                                    int32_t total_new, const int32_t* context_lens,
                                    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                    int32_t max_context_len, float scale,
                                    int32_t partition_size, void* workspace,
                                    size_t workspace_bytes, int32_t dtype, pkv_stream_t stream);

/*
 * Every layer of one decode step in one call: for l = 0 .. num_layers - 1,
 * exactly pkv_append_paged_decode_planned on layer l's tensors, in order, with
 * the same results and errors (the first failing layer's code is returned and
 * the later layers are not launched).  Layer l's tensors start at the first
 * layer's pointer plus l times its layer stride, in elements: out and lse
 * (float; stride 0 lets every layer write one buffer), q, k_cache / v_cache
 * (one stride for both) and k_new / v_new (one stride), in the cache dtype.
 * Everything else (tables, positions, lengths, the plan in `workspace`) is
 * shared by the layers, as in one step of a model (spindle, "Two bugs worth
 * recording": lengths advance once per step).  For callers that issue a
 * step's layers back to back: one host call instead of num_layers.
 */
int pkv_append_paged_decode_planned_layers(
    int32_t num_layers, float* out, int64_t out_layer_stride, float* lse,
    int64_t lse_layer_stride, const void* q, int64_t q_layer_stride, void* k_cache,
    void* v_cache, int64_t cache_layer_stride, const void* k_new, const void* v_new,
    int64_t new_layer_stride, const int32_t* block_tables, int64_t bt_stride,
    const int32_t* start_pos, const int32_t* cu_new_tokens, int32_t total_new,
    const int32_t* context_lens, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_context_len,
    float scale, int32_t partition_size, void* workspace, size_t workspace_bytes, int32_t dtype,
    pkv_stream_t stream);

/*
 * Decode for a batch holding copy-on-write fork groups (spindle, "Paging":
 * forked sequences share blocks through reference counts).  Computes the
 * same out and lse as pkv_paged_decode (equal within rounding; the shared
 * prefix adds a partition boundary and, for bf16 caches, the scores and the
 * weighted sum run on matrix cores, so not bit for bit), but each group's
 * shared leading blocks are streamed once for all its members.
 *
 *   group_starts        : int32 [num_groups + 1]: group g is sequences
 *                         [group_starts[g], group_starts[g + 1]); the groups
 *                         tile 0..batch-1 in order (group_starts[0] = 0,
 *                         group_starts[num_groups] = batch).  A sequence that
 *                         shares nothing is a group of one.
 *   group_shared_blocks : int32 [num_groups]: leading logical blocks that
 *                         every member of g holds in common (same block ids).
 *                         A hint for efficiency only: a member whose ids
 *                         differ is detected and attended through its own
 *                         table row, so results never depend on it.  Values
 *                         above max_shared_blocks (host) are clamped; the
 *                         rest is attended as private context.
 * Each member's tokens [shared, context_lens[s]) are split into partitions
 * of partition_size (0: one) after the shared prefix's own partitions.
 * workspace: pkv_shared_prefix_workspace_bytes(...) bytes, 256-byte aligned.
 * Malformed groups set PKV_DEVERR_GROUPS (results then unspecified; every
 * access stays in bounds).
 * Launches: plan; then for bf16 one kernel for the shared prefixes and the
 * private ranges (fp32: the shared-prefix pass, then the first pass); then
 * the combine.
 */
size_t pkv_shared_prefix_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t head_dim,
                                         int32_t max_context_len, int32_t partition_size);

int pkv_paged_decode_shared_prefix(float* out, float* lse, const void* q, const void* k_cache,
                                   const void* v_cache, const int32_t* block_tables,
                                   int64_t bt_stride, const int32_t* context_lens,
                                   const int32_t* group_starts,
                                   const int32_t* group_shared_blocks, int32_t num_groups,
                                   int32_t max_shared_blocks, int32_t batch,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t num_blocks,
                                   int32_t max_context_len, float scale, int32_t partition_size,
                                   void* workspace, size_t workspace_bytes, int32_t dtype,
                                   pkv_stream_t stream);

/*
 * pkv_kv_append followed by pkv_paged_decode_shared_prefix, with the append
 * and the work plan in one launch (as pkv_append_paged_decode does for the
 * plain decode).  The appended tokens must not land in a block that several
 * sequences hold (copy-on-write: the caller copies such a block first, see
 * pkv_copy_blocks).  Arguments as in those two calls.
 */
int pkv_append_paged_decode_shared_prefix(
    float* out, float* lse, const void* q, void* k_cache, void* v_cache, const void* k_new,
    const void* v_new, const int32_t* block_tables, int64_t bt_stride, const int32_t* start_pos,
    const int32_t* cu_new_tokens, int32_t total_new, const int32_t* context_lens,
    const int32_t* group_starts, const int32_t* group_shared_blocks, int32_t num_groups,
    int32_t max_shared_blocks, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_context_len,
    float scale, int32_t partition_size, void* workspace, size_t workspace_bytes, int32_t dtype,
    pkv_stream_t stream);

/*
 * Paged (chunked) prefill attention (spindle, "Why write the forward pass":
 * the prompt runs through the same forward pass over the block cache;
 * "Two bugs worth recording": explicit positions and lengths).  Sequence s
 * owns query rows cu_q[s] .. cu_q[s+1]-1 of q; they are the LAST
 * q_len = cu_q[s+1] - cu_q[s] tokens of its context of context_lens[s]
 * tokens, whose K/V must already be in the cache (pkv_kv_append first).
 * Query i attends causally to tokens [0, context_lens[s] - q_len + i].
 *
 *   out : float32 [total_q][num_q_heads][head_dim]   (16-byte aligned)
 *   lse : float32 [total_q][num_q_heads], natural log; may be NULL
 *   q   : [total_q][num_q_heads][head_dim] in the cache dtype
 *   cu_q: int32 [batch + 1], non-decreasing, cu_q[0] = 0, cu_q[batch] = total_q
 *   max_q_len : host bound on every chunk's length (grid size)
 * Caches, tables, head and block sizes as in pkv_paged_decode.  bf16 caches
 * run on the matrix cores (16 (token, head) rows of one sequence per tile),
 * fp32 caches on the VALU (one wave per query token).  One launch; no
 * workspace.  Device-side violations (cu_q malformed, a chunk longer than
 * its context or than max_q_len, context beyond the table, bad block ids)
 * set PKV_DEVERR_* bits; affected rows are then unspecified, every access
 * stays in bounds.
 */
int pkv_paged_prefill(float* out, float* lse, const void* q, const void* k_cache,
                      const void* v_cache, const int32_t* block_tables, int64_t bt_stride,
                      const int32_t* cu_q, const int32_t* context_lens, int32_t batch,
                      int32_t total_q, int32_t max_q_len, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int32_t num_blocks, float scale, int32_t dtype, pkv_stream_t stream);

/*
 * First pass only: per-partition attention, no merge.
 *   part_out : float32 [batch][num_q_heads][max_partitions][head_dim]
 *   part_lse : float32 [batch][num_q_heads][max_partitions]
 * Partition p of sequence s covers tokens [p*P, min((p+1)*P, n)); its entry
 * holds that range's normalised attention output and log-sum-exp.  For
 * n = 0, entry 0 is out = 0, lse = -inf.  Entries p >= max(1, ceil(n / P))
 * are not written (pkv_lse_combine never reads them).  Exactly one kernel
 * is launched: the first pass of pkv_paged_decode.  plan_workspace: NULL, or
 * a workspace holding a pkv_decode_plan made with the same context_lens
 * contents, batch, max_context_len and this partition_size (> 0) — the
 * first pass then runs in the plan's order, as inside pkv_paged_decode.
 * Requires max_partitions >= ceil(max_context_len / partition_size) >= 1
 * and partition_size > 0.
 */
int pkv_paged_decode_partials(float* part_out, float* part_lse, const void* q,
                              const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, int64_t bt_stride,
                              const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int32_t num_blocks, int32_t max_context_len, float scale,
                              int32_t partition_size, int32_t max_partitions,
                              const void* plan_workspace, int32_t dtype, pkv_stream_t stream);

/*
 * pkv_paged_decode without the plan kernel: the first pass takes its work
 * order from a plan that pkv_decode_plan wrote earlier (same stream order)
 * into the same workspace for the same context_lens contents, batch,
 * max_context_len and partition_size.  Results are those of pkv_paged_decode.
 * One launch: the merge counters that pkv_decode_plan zeroed are reset by each
 * call's merging workgroups, so any number of planned calls may follow a plan.
 */
int pkv_paged_decode_planned(float* out, float* lse, const void* q, const void* k_cache,
                             const void* v_cache, const int32_t* block_tables, int64_t bt_stride,
                             const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t num_blocks, int32_t max_context_len, float scale,
                             int32_t partition_size, void* workspace, size_t workspace_bytes,
                             int32_t dtype, pkv_stream_t stream);

/*
 * Second pass: merge partitions by log-sum-exp (flash-decoding combine).
 * For each (s, h), over p < ceil(context_lens[s] / partition_size) with
 * part_lse > -inf:  M = max lse_p, w_p = exp(lse_p - M),
 *   out = sum w_p part_out_p / sum w_p,  lse = M + ln sum w_p;
 * no live partition gives out = 0, lse = -inf.  Rounding order: a row of 9 to
 * 64 partitions is merged in two steps, each group of 8 consecutive
 * partitions by the formula above, then the group results by the same
 * formula (the same value in exact arithmetic); other rows in one step.  A
 * call with max_partitions from 9 to 64 runs one workgroup per row, one wave
 * per group.  Layouts as in pkv_paged_decode_partials.  lse may be NULL.
 */
int pkv_lse_combine(float* out, float* lse, const float* part_out, const float* part_lse,
                    const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                    int32_t head_dim, int32_t partition_size, int32_t max_partitions,
                    pkv_stream_t stream);

/*
 * Copy-on-write block copy (spindle, "Paging": reference counts give
 * copy-on-write forking).  For i in [0, n) and every layer l in
 * [0, num_layers):  block dst[i] := block src[i] (all KV heads, all slots)
 * in both caches, bit-exact.  Layer l's caches start layer_stride elements
 * after layer l-1's (layer_stride is ignored when num_layers = 1).
 * src and dst are int32 [n] device arrays; the dst ids must be distinct and
 * disjoint from the src ids (otherwise copies race).
 */
int pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src, const int32_t* dst,
                    int32_t n, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int32_t num_blocks, int32_t num_layers, int64_t layer_stride, int32_t dtype,
                    pkv_stream_t stream);

/*
 * Synchronises `stream`, then returns (in *flags, host) and clears the
 * current device's error word: an OR of PKV_DEVERR_* bits set by kernels
 * since the last call.  Returns PKV_OK or PKV_ERR_DEVICE.
 */
int pkv_device_error(pkv_stream_t stream, int32_t* flags);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
