/*
 * pkv_replay.h - replay of a request stream through a KV allocator (host only).
 *
 * spindle, section "Paging", compares a contiguous per-sequence buffer with
 * the block pool (64 requests, 8192 token slots, 16-token blocks) by peak
 * slots held, mean slot utilisation and steps to drain.  A contiguous buffer
 * must be sized at admission to prompt + max_new_tokens and is held whole for
 * the request's lifetime; the pool hands out blocks as tokens arrive, so a
 * sequence wastes at most its final partial block.  The page gives neither
 * the workload nor the step model; this call runs the following one:
 *
 *   - requests wait in a FIFO queue, in index order, and are admitted at the
 *     start of a step while memory allows; the first that does not fit stops
 *     admission;
 *   - a request admitted in a step holds prompt + 1 tokens after it; every
 *     later step adds one token; a request leaves at the end of the step in
 *     which it holds prompt + gen tokens;
 *   - PKV_REPLAY_CONTIGUOUS: admission needs a free run of prompt +
 *     max_new_tokens slots (first fit, lowest address), held until the
 *     request leaves; freed runs merge with their neighbours;
 *   - PKV_REPLAY_PAGED: the native block manager (pkv_bm_*, FIFO free list
 *     over 0..total_slots/block_size-1); admission needs the blocks covering
 *     prompt + 1 tokens; a running request whose next token starts a new
 *     block takes one first, in admission order; with the pool empty, the most
 *     recently admitted running request is preempted (blocks freed, progress
 *     dropped, back to the front of the queue) until a block is free or the
 *     request itself was preempted;
 *   - per step, after the writes and before leaving requests release memory:
 *     slots held (reserved slots, or blocks x block_size) and tokens held over
 *     running requests.  peak_slots is the maximum, mean_utilisation the mean
 *     over steps of tokens / slots (0 for a step with nothing running), steps
 *     the number of steps until no request remains.
 *
 * Arguments: prompt_lens / gen_lens host int32 [num_requests] with
 * prompt >= 0 and 1 <= gen <= max_new_tokens; total_slots a multiple of
 * block_size.  Every request must fit an empty pool on its own
 * (PKV_ERR_SHAPE otherwise).  trace_cap >= 0 and the three trace arrays
 * (host, nullable together) receive the first trace_cap steps' slots held,
 * tokens held and running count.  Host memory and host code only.
 */
#ifndef PKV_REPLAY_H_
#define PKV_REPLAY_H_

#include <stdint.h>

#include "pkv.h"

#ifdef __cplusplus
extern "C" {
#endif

enum { PKV_REPLAY_CONTIGUOUS = 0, PKV_REPLAY_PAGED = 1 };

typedef struct pkv_replay_result {
  int64_t peak_slots;
  double mean_utilisation;
  int32_t steps;
  int32_t preemptions;
} pkv_replay_result;

int pkv_replay_allocator(int32_t policy, int32_t num_requests, const int32_t* prompt_lens,
                         const int32_t* gen_lens, int32_t max_new_tokens, int32_t total_slots,
                         int32_t block_size, int64_t* slots_trace, int64_t* tokens_trace,
                         int32_t* running_trace, int32_t trace_cap, pkv_replay_result* out);

#ifdef __cplusplus
}
#endif

#endif /* PKV_REPLAY_H_ */
