// One wavefront writes one new token's K and V rows (every KV head) into the cache at
// the position the caller names (spindle, "Two bugs worth recording": the write position
// is an argument, never derived from a stored length).  Shared by the standalone append kernel and the decode prologue.
// The including file defines the device error word used by PKV_FLAG_ERROR.
#pragma once

#include "common.h"

namespace pkv {

// Sequence of token i: the largest s with cu[s] <= i, i.e. (number of entries of the
// non-decreasing cu[0..batch-1] that are <= i) - 1, counted with ballots.  A decode step
// appends one token per sequence, so token i is first tried as sequence i: for a
// non-decreasing cu, cu[i] <= i < cu[i + 1] makes i that largest s (every later entry is
// at least cu[i + 1]), found in one memory round trip.  Returns -1 (and the caller flags)
// when cu is malformed; else the sequence, with cu[s] in *first.
__device__ __forceinline__ int append_sequence_of(const int32_t* __restrict__ cu, int batch,
                                                  int total, int i, int lane, int* first) {
  if (i < batch) {
    // the three loads issued together: the test combines them without short-circuit
    const int a = cu[i], b = cu[i + 1], t = cu[batch];
    if ((a <= i) & (i < b) & (t == total)) {
      *first = a;
      return i;
    }
  }
  int count = 0;
  for (int j0 = 0; j0 < batch; j0 += kWave) {
    const int j = j0 + lane;
    const bool le = j < batch && cu[j] <= i;
    count += __popcll(__ballot(le));
  }
  const int s = max(count - 1, 0);
  const int a = cu[s];
  if (a > i || cu[s + 1] <= i || cu[batch] != total) return -1;
  *first = a;
  return s;
}

// Copy token i's rows: k_new/v_new [total][num_kv_heads][row_vecs] (16-byte vectors)
// into [num_blocks][num_kv_heads][16][row_vecs] at block table[s][pos / 16], slot pos % 16.
__device__ __forceinline__ void append_token(
    uint4* __restrict__ kc, uint4* __restrict__ vc, const uint4* __restrict__ kn,
    const uint4* __restrict__ vn, const int32_t* __restrict__ tables, int W,
    const int32_t* __restrict__ start_pos, const int32_t* __restrict__ cu, int batch, int total,
    int num_kv_heads, int row_vecs, int num_blocks, int i, int lane, unsigned* err) {
  // the position of sequence i, loaded with the lookup's loads (right for a decode step)
  const int start_i = i < batch ? start_pos[i] : 0;
  int first = 0;
  const int s = append_sequence_of(cu, batch, total, i, lane, &first);
  if (s < 0) {
    if (lane == 0) atomicOr(err, static_cast<unsigned>(PKV_DEVERR_CU));
    return;
  }
  const int pos = (s == i ? start_i : start_pos[s]) + (i - first);
  if (pos < 0 || pos >= W * kBlockTokens) {
    if (lane == 0) atomicOr(err, static_cast<unsigned>(PKV_DEVERR_POSITION));
    return;
  }
  const int blk = tables[static_cast<size_t>(s) * W + pos / kBlockTokens];
  if (static_cast<unsigned>(blk) >= static_cast<unsigned>(num_blocks)) {
    if (lane == 0) atomicOr(err, static_cast<unsigned>(PKV_DEVERR_BLOCK_ID));
    return;
  }
  const int slot = pos % kBlockTokens;
  const int n_vec = num_kv_heads * row_vecs;
  for (int v = lane; v < n_vec; v += kWave) {
    const int h = v / row_vecs;
    const int j = v % row_vecs;
    const size_t dst =
        ((static_cast<size_t>(blk) * num_kv_heads + h) * kBlockTokens + slot) * row_vecs + j;
    const size_t src = static_cast<size_t>(i) * n_vec + v;
    kc[dst] = kn[src];
    vc[dst] = vn[src];
  }
}

}  // namespace pkv
