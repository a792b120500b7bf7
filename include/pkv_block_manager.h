/*
 * pkv_block_manager.h - host-side bookkeeping of the paged KV pool.
 *
 * spindle, "Paging": one pool of fixed-size blocks, a table per sequence
 * listing its blocks, blocks taken only as tokens arrive (so a sequence wastes
 * at most its last, partly filled block), and blocks shared by reference count
 * between forks (copy-on-write); the page's example is a 16-token parent forked
 * four ways: 64 tokens attended, 16 stored.
 * spindle, "Two bugs worth recording": the cache never infers a length; the
 * caller names the token range it is about to write.
 *
 * Readings where the page is silent:
 *   - the free list is FIFO over an initial order (default 0..num_blocks-1);
 *     freed blocks go to its tail;
 *   - pkv_bm_prepare_write makes the blocks covering [start, start+n)
 *     present and exclusively owned: missing logical blocks are taken from
 *     the free list; a present block with reference count > 1 is replaced by
 *     a fresh block, and the (old -> new) pair is returned for the caller to
 *     copy with pkv_copy_blocks before writing.  All or nothing: on
 *     PKV_ERR_OUT_OF_BLOCKS nothing changed.
 *
 * Everything here is host memory and host code; no GPU call is made.  A
 * pkv_bm handle is not thread-safe.  All functions return PKV_OK or a
 * negative PKV_ERR_* code (see pkv.h); PKV_ERR_ARG for an unknown sequence
 * or block id, PKV_ERR_NULL for a NULL required pointer.
 */
#ifndef PKV_BLOCK_MANAGER_H_
#define PKV_BLOCK_MANAGER_H_

#include <stdint.h>

#include "pkv.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pkv_bm pkv_bm;

/* free_order: host int32 [num_blocks], a permutation of 0..num_blocks-1, or NULL. */
int pkv_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                  pkv_bm** out);
void pkv_bm_destroy(pkv_bm* bm);

/* A new, empty sequence; ids are assigned 0, 1, 2, ... and never reused. */
int pkv_bm_add_sequence(pkv_bm* bm, int32_t* seq_out);

/*
 * Make token positions [start, start + n) of `seq` writable (see above).
 * start must not leave a hole: start / block_size <= current table length.
 * Copies needed are written to copy_src/copy_dst (host int32, capacity
 * copy_cap; at most ceil(n / block_size) + 1 are ever needed) and their
 * count to *n_copies.  n = 0 is a no-op.
 */
int pkv_bm_prepare_write(pkv_bm* bm, int32_t seq, int32_t start, int32_t n, int32_t* copy_src,
                         int32_t* copy_dst, int32_t copy_cap, int32_t* n_copies);

/*
 * One decode step's bookkeeping in one call: pkv_bm_prepare_write(seqs[r],
 * starts[r], counts[r]) for r = 0 .. nseq-1 in order, the copies of all of them
 * appended to copy_src/copy_dst (capacity copy_cap in total), then (tables not
 * NULL) pkv_bm_fill_tables(seqs, nseq, tables, width, pad_id).  *n_done counts
 * the sequences prepared; on an error (PKV_ERR_OUT_OF_BLOCKS included) the
 * first *n_done writes stay done, sequence *n_done is unchanged and the rest
 * are not attempted, and the tables are not filled.
 */
int pkv_bm_prepare_step(pkv_bm* bm, const int32_t* seqs, const int32_t* starts,
                        const int32_t* counts, int32_t nseq, int32_t* tables, int32_t width,
                        int32_t pad_id, int32_t* copy_src, int32_t* copy_dst, int32_t copy_cap,
                        int32_t* n_copies, int32_t* n_done);

/* New sequence sharing every block of `parent`; each shared block's count +1. */
int pkv_bm_fork(pkv_bm* bm, int32_t parent, int32_t* child_out);

/* Drop one reference from each of seq's blocks (count 0 -> free-list tail); forget seq. */
int pkv_bm_free_sequence(pkv_bm* bm, int32_t seq);

/* Number of blocks in seq's table. */
int pkv_bm_num_blocks_of(const pkv_bm* bm, int32_t seq, int32_t* n);

/*
 * Dense tables for a batch: row r (host int32 [nseq][width]) receives
 * seqs[r]'s block ids followed by pad_id up to `width`.  PKV_ERR_SHAPE if a
 * table is longer than width.
 */
int pkv_bm_fill_tables(const pkv_bm* bm, const int32_t* seqs, int32_t nseq, int32_t* tables,
                       int32_t width, int32_t pad_id);

int pkv_bm_refcount(const pkv_bm* bm, int32_t block, int32_t* count);
int pkv_bm_num_free(const pkv_bm* bm, int32_t* n);

/* Free-list contents in order (host int32, capacity cap); *n = list length. */
int pkv_bm_free_list(const pkv_bm* bm, int32_t* ids, int32_t cap, int32_t* n);

#ifdef __cplusplus
}
#endif

#endif /* PKV_BLOCK_MANAGER_H_ */
