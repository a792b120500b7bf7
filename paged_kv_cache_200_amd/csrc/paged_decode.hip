// Paged decode attention for gfx950: first pass (per KV partition) and the
// log-sum-exp combine.
//
// What is computed (spindle, "Paging" and "Two bugs worth recording"): for a
// sequence with explicit length n, gather the K/V of tokens [0, n) through
// its block table and run softmax attention of the single query token
// against them.  Long contexts are split flash-decoding style (mlsystems topic
// listing, flash-decoding entry): each KV partition is attended on its own
// and the partial results are merged by their log-sum-exps.
//
// Work decomposition.  One workgroup = (sequence, KV head, partition), four
// wavefronts.  Every query head of the KV head's GQA group is handled by the
// same workgroup, so each K/V byte is read from HBM once per call.  Wave w
// takes the partition's blocks w, w+4, w+8, ...; one 16-token block of one KV
// head is a contiguous 16*D run, read whole with 16-byte loads.
//
// Inside a wave, 8 lanes share one token: a lane holds D/8 elements of that
// token (two 16-byte chunks for bf16 D=128), so a block is 2 tokens per lane.
// The QK dot product is a per-lane partial (bf16 pairs through the dot2
// instruction, fp32 through FMA) finished by a 3-step DPP sum over the 8
// lanes.  Each 8-lane group keeps its own online-softmax state (max m, sum l,
// accumulator over its dims) for every query head of the group, so the hot
// loop needs no other cross-lane traffic.  The running max is lazy: it is
// only raised when a score exceeds it by more than 2^8, which keeps the
// accumulator rescale off the common path while all exponentials stay <= 2^8.
// At the end the 8 groups of a wave are merged with lane shuffles and the 4
// waves through LDS, by the same log-sum-exp rule as the combine.
//
// Scores are kept in log2 units (scale * log2(e) folded in) so every
// exponential is one v_exp_f32.

#include "common.h"

// The merge of split sequences inside the first pass orders its partial-result stores
// before the merge ticket without a release/acquire pair: device-scope (sc1) stores, a
// wait for their completion and a relaxed device-scope ticket, read back through
// device-scope loads.  That this suffices is a property of how gfx950 executes those
// instructions, not a guarantee of the HIP memory model, so the file builds for gfx950
// only.
#if defined(__HIP_DEVICE_COMPILE__) && !defined(__gfx950__)
#error "paged_decode.hip: the in-pass merge's memory ordering is established for gfx950 only"
#endif

PKV_DEFINE_ERROR_WORD(decode)

#include "append_row.h"
#include "mfma_tile.h"
#include "valu_attend.h"

namespace pkv {
namespace {

// Log-sum-exp merge of one (sequence, query head)'s partition results, by one wavefront:
// lane p holds partition p's log-sum-exp (64 partitions per round), so the max and the
// weight sum are wave reductions; the weighted sum of the partial outputs then streams
// the partitions with every lane owning D/64 output dims, four partitions per step.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) x += __shfl_xor(x, m);
  return x;
}

// kAgent: read the partial results through device-scope loads (global_load ... sc1), which
// miss in this XCD's L2 when another XCD wrote them in the same launch; else plain loads.
template <bool kAgent>
__device__ __forceinline__ float load_partial(const float* p) {
  if constexpr (kAgent)
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    return *p;
}

// Most partial-result slots per sequence merged inside the first pass (decode_impl
// launches the combine kernel past that), and the slots whose partial outputs the merging
// workgroup loads together.
#ifndef PKV_IN_PASS_MERGE_MAX
#define PKV_IN_PASS_MERGE_MAX 8
#endif
constexpr int kMaxInPassMergeSlots = PKV_IN_PASS_MERGE_MAX;

// The combine merges a row of more than kMaxInPassMergeSlots partitions, up to
// kMergeGroups groups of kMaxInPassMergeSlots consecutive partitions, in two steps: each
// group into one result, then the groups (the same identity, applied twice).  The groups
// of a row then run on waves of their own (lse_combine_grouped_kernel).  Longer rows are
// merged in one step.
constexpr int kMergeGroups = kMaxInPassMergeSlots;
constexpr int kMaxTwoLevelSlots = kMergeGroups * kMaxInPassMergeSlots;

__host__ __device__ constexpr int merge_group_count(int slots) {
  return (slots + kMaxInPassMergeSlots - 1) / kMaxInPassMergeSlots;
}

// One merge step over at most kMaxInPassMergeSlots results: lane u < n holds result u's
// log-sum-exp (-inf on the other lanes) and x[u] that result's D/64 output dims of this
// lane (0 past n).  The weighted sum runs over the results in order.
template <int kPer>
__device__ __forceinline__ void merge_step(float lp, const float (&x)[kMaxInPassMergeSlots][kPer],
                                           float (&o)[kPer], float& ls) {
  constexpr float kLog2e = 1.44269504088896340736f;
  const float M = wave_max(lp);
  const float w = lp == -INFINITY ? 0.0f : fast_exp2((lp - M) * kLog2e);
  const float den = wave_sum(w);
  float acc[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) acc[j] = 0.0f;
#pragma unroll
  for (int u = 0; u < kMaxInPassMergeSlots; ++u) {
    const float wp = __shfl(w, u);
#pragma unroll
    for (int j = 0; j < kPer; ++j) acc[j] = fmaf(wp, x[u][j], acc[j]);
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) o[j] = den > 0.0f ? acc[j] / den : 0.0f;
  ls = den > 0.0f ? M + __logf(den) : -INFINITY;
}

// Group g (partitions g * kMaxInPassMergeSlots ..) of a row of nparts partitions, merged
// by one wave into o (this lane's dims) and ls.
template <int D>
__device__ __forceinline__ void merge_group(const float* __restrict__ pl,
                                            const float* __restrict__ po, int nparts, int g,
                                            int lane, float (&o)[D / kWave], float& ls) {
  constexpr int kS = kMaxInPassMergeSlots;
  constexpr int kPer = D / kWave;
  const int p0 = g * kS;
  const int cnt = min(kS, nparts - p0);
  const float lp = lane < cnt ? pl[p0 + lane] : -INFINITY;
  float x[kS][kPer];
#pragma unroll
  for (int u = 0; u < kS; ++u)
#pragma unroll
    for (int j = 0; j < kPer; ++j) x[u][j] = u < cnt ? po[(p0 + u) * D + j * kWave + lane] : 0.0f;
  merge_step<kPer>(lp, x, o, ls);
}

// The combine of one (sequence, head) row by one wave.  Up to kMaxInPassMergeSlots
// partitions: one merge step, the arithmetic of the first pass's own merge, so both give
// the same bits.  Up to kMaxTwoLevelSlots: two steps (groups, then the groups).  Longer
// rows: one step over all partitions, kChunk partitions' outputs loaded together.
template <int D, int kChunk = 32>
__device__ __forceinline__ void combine_row(float* __restrict__ out_row, float* __restrict__ lse_el,
                                            const float* __restrict__ pl,
                                            const float* __restrict__ po, int nparts, int lane) {
  constexpr int kPer = D / kWave;  // output dims per lane
  constexpr float kLog2e = 1.44269504088896340736f;
  if (nparts <= kMaxInPassMergeSlots) {
    // one step, every load issued before the first wait (as in the first pass's merge)
    float o[kPer], ls;
    merge_group<D>(pl, po, nparts, 0, lane, o, ls);
#pragma unroll
    for (int j = 0; j < kPer; ++j) out_row[j * kWave + lane] = o[j];
    if (lse_el != nullptr && lane == 0) *lse_el = ls;
    return;
  }
  if (nparts <= kMaxTwoLevelSlots) {
    // two steps: lane g ends up with group g's log-sum-exp, go[g] with its dims
    const int ng = merge_group_count(nparts);
    float gl = -INFINITY;
    float go[kMergeGroups][kPer];
#pragma unroll
    for (int g = 0; g < kMergeGroups; ++g) {
      if (g < ng) {
        float ls;
        merge_group<D>(pl, po, nparts, g, lane, go[g], ls);
        if (lane == g) gl = ls;
      } else {
#pragma unroll
        for (int j = 0; j < kPer; ++j) go[g][j] = 0.0f;
      }
    }
    float o[kPer], ls;
    merge_step<kPer>(gl, go, o, ls);
#pragma unroll
    for (int j = 0; j < kPer; ++j) out_row[j * kWave + lane] = o[j];
    if (lse_el != nullptr && lane == 0) *lse_el = ls;
    return;
  }
  // One step over every partition: the max of the log-sum-exps (64 per wave load), then
  // the weights and the weighted sum in chunks.
  const float lp0 = lane < nparts ? pl[lane] : -INFINITY;
  float M = wave_max(lp0);
  for (int p0 = kWave; p0 < nparts; p0 += kWave)
    M = fmaxf(M, wave_max(p0 + lane < nparts ? pl[p0 + lane] : -INFINITY));
  float acc[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) acc[j] = 0.0f;
  float den = 0.0f;
  for (int p0 = 0; p0 < nparts; p0 += kWave) {
    const int cnt = min(kWave, nparts - p0);
    const float lp = p0 == 0 ? lp0 : lane < cnt ? pl[p0 + lane] : -INFINITY;
    const float w = (lp == -INFINITY) ? 0.0f : fast_exp2((lp - M) * kLog2e);
    den += wave_sum(w);
    // kChunk partitions' loads in flight at a time; past the last partition the weight is
    // 0 and nothing is loaded, so the step adds 0 (every chunk is whole, no serial tail)
    for (int p = 0; p < cnt; p += kChunk) {
      float wp[kChunk];
      float x[kChunk][kPer];
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        const bool live = p + u < cnt;
        wp[u] = __shfl(w, (p + u) % kWave);
#pragma unroll
        for (int j = 0; j < kPer; ++j)
          x[u][j] = live ? po[(p0 + p + u) * D + j * kWave + lane] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < kChunk; ++u)
#pragma unroll
        for (int j = 0; j < kPer; ++j) acc[j] = fmaf(wp[u], x[u][j], acc[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) out_row[j * kWave + lane] = den > 0.0f ? acc[j] / den : 0.0f;
  if (lse_el != nullptr && lane == 0) *lse_el = den > 0.0f ? M + __logf(den) : -INFINITY;
}

// Second pass as its own kernel: one wavefront per (sequence, query head), four per
// workgroup.
constexpr int kCombineWaves = 4;

// Partitions to merge for sequence s, 0 when there is nothing to do.  nslots (nullable):
// per sequence, the number of slots to merge, 0 when the first pass wrote the sequence's
// result itself; without it the count follows from the length.
__device__ __forceinline__ int combine_parts(int s, const int32_t* __restrict__ ctx_lens,
                                             const int32_t* __restrict__ nslots, int cap,
                                             int part_tokens, int max_parts, int skip_single) {
  if (nslots != nullptr) return max(0, min(nslots[s], max_parts));
  int n = ctx_lens[s];
  n = n < 0 ? 0 : min(n, cap);
  const int nparts = min(n > 0 ? (n + part_tokens - 1) / part_tokens : 1, max_parts);
  return skip_single && nparts == 1 ? 0 : nparts;
}

template <int D>
__global__ __launch_bounds__(kCombineWaves * kWave) void lse_combine_kernel(
    float* __restrict__ out, float* __restrict__ lse, const float* __restrict__ part_out,
    const float* __restrict__ part_lse, const int32_t* __restrict__ ctx_lens,
    const int32_t* __restrict__ nslots, int batch, int cap, int num_q_heads, int part_tokens,
    int max_parts, int skip_single) {
  const int row = blockIdx.x * kCombineWaves + threadIdx.x / kWave;  // (s, h) flattened
  const int lane = threadIdx.x % kWave;
  if (row >= batch * num_q_heads) return;
  const int nparts = combine_parts(row / num_q_heads, ctx_lens, nslots, cap, part_tokens,
                                   max_parts, skip_single);
  if (nparts <= 0) return;
  const size_t sh = static_cast<size_t>(row);
  combine_row<D>(out + sh * D, lse != nullptr ? lse + sh : nullptr, part_lse + sh * max_parts,
                 part_out + sh * max_parts * D, nparts, lane);
}

// The combine when no row has more than kMaxTwoLevelSlots partitions: one workgroup of
// kMergeGroups waves per (sequence, query head).  A row of more than
// kMaxInPassMergeSlots partitions has wave g merge group g, then wave 0 merge the groups
// through LDS: the steps of combine_row, so the same bits, with the groups' loads in
// flight on several waves at once.  Shorter rows are combine_row on wave 0.
template <int D>
__global__ __launch_bounds__(kMergeGroups * kWave) void lse_combine_grouped_kernel(
    float* __restrict__ out, float* __restrict__ lse, const float* __restrict__ part_out,
    const float* __restrict__ part_lse, const int32_t* __restrict__ ctx_lens,
    const int32_t* __restrict__ nslots, int batch, int cap, int num_q_heads, int part_tokens,
    int max_parts, int skip_single) {
  constexpr int kPer = D / kWave;
  __shared__ float s_o[kMergeGroups][D];
  __shared__ float s_l[kMergeGroups];
  const int row = blockIdx.x;  // (s, h) flattened; the grid has batch * num_q_heads
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int nparts = combine_parts(row / num_q_heads, ctx_lens, nslots, cap, part_tokens,
                                   max_parts, skip_single);
  if (nparts <= 0) return;
  const size_t sh = static_cast<size_t>(row);
  const float* pl = part_lse + sh * max_parts;
  const float* po = part_out + sh * max_parts * D;
  if (nparts <= kMaxInPassMergeSlots) {
    if (wave == 0) combine_row<D>(out + sh * D, lse != nullptr ? lse + sh : nullptr, pl, po,
                                  nparts, lane);
    return;
  }
  const int ng = merge_group_count(nparts);
  if (wave < ng) {
    float o[kPer], ls;
    merge_group<D>(pl, po, nparts, wave, lane, o, ls);
#pragma unroll
    for (int j = 0; j < kPer; ++j) s_o[wave][j * kWave + lane] = o[j];
    if (lane == 0) s_l[wave] = ls;
  }
  __syncthreads();
  if (wave == 0) {
    const float gl = lane < ng ? s_l[lane] : -INFINITY;
    float go[kMergeGroups][kPer];
#pragma unroll
    for (int u = 0; u < kMergeGroups; ++u)
#pragma unroll
      for (int j = 0; j < kPer; ++j) go[u][j] = u < ng ? s_o[u][j * kWave + lane] : 0.0f;
    float o[kPer], ls;
    merge_step<kPer>(gl, go, o, ls);
    float* out_row = out + sh * D;
#pragma unroll
    for (int j = 0; j < kPer; ++j) out_row[j * kWave + lane] = o[j];
    if (lse != nullptr && lane == 0) lse[sh] = ls;
  }
}

// Grid layouts of the first pass.
//   kOrderPartMinor: x = partition, y = KV-head group, z = sequence.
//   kOrderPartMajorReversed: x = KV-head group, y = sequence, z = partition counted from
//     the last one, so the later partitions of the longest sequences are dispatched first
//     and every sequence's first (often shortest) partition last.
//   kOrderPlanned: x = work unit * num_kv_heads + KV head, the units taken in the order a
//     plan kernel wrote them (longest first, see plan_kernel).
constexpr int kOrderPartMinor = 0;
constexpr int kOrderPartMajorReversed = 1;
constexpr int kOrderPlanned = 2;
// Plan entry {sequence, first token, end token, slot | kDirectFlag}: the unit's token range,
// the partial-result slot it fills, and whether it is its sequence's only unit (then it
// writes out / lse itself).
constexpr int kDirectFlag = 1 << 30;
constexpr int kSlotMask = kDirectFlag - 1;

// NW wavefronts per workgroup.  NW > 1: the waves share one (sequence, KV head,
// partition) and take its blocks round-robin, merging through LDS at the end.  NW == 1:
// one wave owns the unit and writes its result straight from registers.  Each wave keeps
// two 16-token blocks in flight.
//
// Workgroups per compute unit the register allocation is held to: two (eight waves, at
// most 256 registers per lane) where that fits without spilling, measured per shape with
// the compiler's resource report; the other shapes take what their registers allow.
// A decode step's KV append folded into the first pass (spindle, "Two bugs worth
// recording": append writes at an explicit start position).  Sequence s's new tokens,
// rows cu[s] .. cu[s + 1] - 1 of k_new / v_new at positions start_pos[s] + i, are written
// by the unit whose token range holds their position, or by the sequence's last unit when
// the position lies past the attended range.  Inside that unit each 16-byte chunk is
// stored by the lane of the wave that later loads it as part of its block (same lane,
// same address), so the attention reads the new token without a barrier: a thread always
// sees its own earlier write.  No other workgroup may read the written slot in the same
// launch, which copy-on-write guarantees (a block held by several sequences is copied
// before any of them writes into it).  Errors are flagged like the standalone append's.
struct PassAppend {
  const void* k_new;  // [total][num_kv_heads][head_dim], nullptr: nothing to append
  const void* v_new;
  const int32_t* start_pos;
  const int32_t* cu;
  int total;
};

template <typename T, int D, int NW>
__device__ __forceinline__ void append_in_unit(
    T* kc, T* vc, const PassAppend& ap, const int32_t* __restrict__ tables, int W,
    const int32_t* __restrict__ ctx_lens, int s, int kvh, int num_kv_heads, int num_blocks,
    int tok0, int tok1, int wave, int lane) {
  using Gm = Geom<T, D>;
  const int c0 = ap.cu[s];
  const int c1 = ap.cu[s + 1];
  if (c0 < 0 || c1 < c0 || c1 > ap.total) {
    if (wave == 0 && lane == 0 && kvh == 0) PKV_FLAG_ERROR(PKV_DEVERR_CU);
    return;
  }
  const int cap = W * kBlockTokens;
  int n = ctx_lens[s];
  n = n < 0 ? 0 : min(n, cap);
  const bool last_unit = tok1 >= n;
  const int p0 = ap.start_pos[s];
  const int b_begin = tok0 / kBlockTokens;
  const int grp = lane / kLanesPerToken;
  const int sub = lane % kLanesPerToken;
  const T* kn = static_cast<const T*>(ap.k_new);
  const T* vn = static_cast<const T*>(ap.v_new);
  for (int t = c0; t < c1; ++t) {
    const int pos = p0 + (t - c0);
    const bool inside = pos >= tok0 && pos < tok1;
    if (!inside && !(last_unit && pos >= tok1)) continue;
    if (pos < 0 || pos >= cap) {
      if (wave == 0 && lane == 0) PKV_FLAG_ERROR(PKV_DEVERR_POSITION);
      continue;
    }
    const int bi = pos / kBlockTokens;
    // the unit's blocks go round-robin over its waves from b_begin
    const int owner = inside ? (bi - b_begin) % NW : 0;
    const int slot = pos % kBlockTokens;
    // lanes of token group slot % 8 hold slot as their token slot / 8 of the block
    if (wave != owner || grp != slot % kGroups) continue;
    const int id = tables[static_cast<size_t>(s) * W + bi];
    if (static_cast<unsigned>(id) >= static_cast<unsigned>(num_blocks)) {
      if (sub == 0) PKV_FLAG_ERROR(PKV_DEVERR_BLOCK_ID);
      continue;
    }
    const size_t row = ((static_cast<size_t>(id) * num_kv_heads + kvh) * kBlockTokens + slot) * D;
    const size_t src = (static_cast<size_t>(t) * num_kv_heads + kvh) * D;
#pragma unroll
    for (int c = 0; c < Gm::kChunks; ++c) {
      const int e = sub * Gm::kChunkElems + c * Gm::kChunkStride;
      *reinterpret_cast<uint4*>(kc + row + e) = *reinterpret_cast<const uint4*>(kn + src + e);
      *reinterpret_cast<uint4*>(vc + row + e) = *reinterpret_cast<const uint4*>(vn + src + e);
    }
  }
}

// The work unit of a first-pass workgroup: which sequence, KV head and token range it
// attends, which partial-result slot it fills (unless `direct`: its sequence's only unit,
// written straight to out / lse), and whether its sequence is merged in this launch.
struct Unit {
  int part, kvh, s;  // part: the partial-result slot written unless `direct`
  int tok0, tok1;    // the unit's token range
  bool direct;
  bool merge;
};

// Returns false when the workgroup has no unit (past the plan's count or the sequence's
// partitions).
__device__ __forceinline__ bool resolve_unit(Unit& un, int order, int num_kv_heads,
                                             const int4* __restrict__ plan,
                                             const int* __restrict__ plan_count,
                                             const int32_t* __restrict__ ctx_lens, int W,
                                             int part_tokens, const float* out,
                                             const int* merge_ctr) {
  const bool leader = threadIdx.x == 0;
  un.merge = false;
  if (order == kOrderPlanned) {
    // The plan entry carries the unit's (range-checked) token range and slot: one load
    // instead of dependent ones before the first block-table read.
    const int unit = blockIdx.x / num_kv_heads;
    un.kvh = blockIdx.x - unit * num_kv_heads;
    // both loads at once: the grid never exceeds the plan's batch * np entries, so the
    // entry is readable (stale) even past the count
    const int count = *plan_count;
    const int4 u = plan[unit];
    if (unit >= count) return false;
    un.s = u.x;
    un.tok0 = u.y;
    un.tok1 = u.z;
    un.part = u.w & kSlotMask;
    un.direct = (u.w & kDirectFlag) != 0 && out != nullptr;
    un.merge = !un.direct && merge_ctr != nullptr && out != nullptr;
    return true;
  }
  int nx_parts;
  if (order == kOrderPartMinor) {
    un.part = blockIdx.x; un.kvh = blockIdx.y; un.s = blockIdx.z; nx_parts = gridDim.x;
  } else {
    un.kvh = blockIdx.x; un.s = blockIdx.y; un.part = gridDim.z - 1 - blockIdx.z;
    nx_parts = gridDim.z;
  }
  int n = ctx_lens[un.s];
  const int cap = W * kBlockTokens;
  if (n < 0 || n > cap) {
    if (leader && un.part == 0 && un.kvh == 0) PKV_FLAG_ERROR(PKV_DEVERR_CONTEXT);
    n = n < 0 ? 0 : cap;
  }
  int nparts = 1;
  un.tok0 = 0;
  un.tok1 = n;
  if (part_tokens > 0) {
    nparts = n > 0 ? (n + part_tokens - 1) / part_tokens : 1;
    un.tok0 = un.part * part_tokens;
    un.tok1 = min(n, un.tok0 + part_tokens);
  }
  if (un.part == nx_parts - 1 && nparts > nx_parts && leader && un.kvh == 0)
    PKV_FLAG_ERROR(PKV_DEVERR_MAX_CONTEXT);
  if (un.part >= nparts) return false;
  un.direct = nparts == 1 && out != nullptr;
  return true;
}

// Epilogue of a split unit whose sequence is merged in this launch, after its partial
// results were stored with device-scope stores: wait until those stores have completed,
// take one ticket per workgroup from the (sequence, KV head) counter, and if it is the
// last of the sequence's n_merge units (n_merge <= kMaxInPassMergeSlots), merge every slot
// (the log-sum-exp combine in the combine kernel's arithmetic and order; wave w merges
// query heads w, w + NW, ...) and reset the counter.  The counter is zeroed by the plan,
// so a reused plan starts from zero too.  Called by all threads of the workgroup.
//
// The merging wave issues every load of its heads (log-sum-exps and partial outputs of
// all slots) before it waits for any: one round trip to memory instead of one for the
// log-sum-exps and another for the outputs, per head.
template <int D, int G, int NW>
__device__ __forceinline__ void merge_when_last(int n_merge, int* __restrict__ merge_ctr, int s,
                                                int kvh, int num_q_heads, int num_kv_heads,
                                                int max_parts, float* __restrict__ out,
                                                float* __restrict__ lse,
                                                const float* __restrict__ part_out,
                                                const float* __restrict__ part_lse, int wave,
                                                int lane) {
  __shared__ int s_ticket;
  const bool leader = threadIdx.x == 0;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int* ctr = merge_ctr + static_cast<size_t>(s) * num_kv_heads + kvh;
  if (leader) s_ticket = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (s_ticket == n_merge - 1) {
    constexpr int kRows = (G + NW - 1) / NW;  // heads per wave
    constexpr int kSlots = kMaxInPassMergeSlots;
    constexpr int kPer = D / kWave;           // output dims per lane
    constexpr float kLog2e = 1.44269504088896340736f;
    float lp[kRows];
    float x[kRows][kSlots][kPer];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int g = wave + r * NW;
      const size_t sh = static_cast<size_t>(s) * num_q_heads + kvh * G + min(g, G - 1);
      const float* pl = part_lse + sh * max_parts;
      const float* po = part_out + sh * max_parts * D;
      lp[r] = g < G && lane < n_merge ? load_partial<true>(pl + lane) : -INFINITY;
#pragma unroll
      for (int u = 0; u < kSlots; ++u)
#pragma unroll
        for (int j = 0; j < kPer; ++j)
          x[r][u][j] = g < G && u < n_merge ? load_partial<true>(po + u * D + j * kWave + lane)
                                            : 0.0f;
    }
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int g = wave + r * NW;
      if (g >= G) continue;
      const size_t sh = static_cast<size_t>(s) * num_q_heads + kvh * G + g;
      const float M = wave_max(lp[r]);
      const float w = lp[r] == -INFINITY ? 0.0f : fast_exp2((lp[r] - M) * kLog2e);
      const float den = wave_sum(w);
      float acc[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) acc[j] = 0.0f;
#pragma unroll
      for (int u = 0; u < kSlots; ++u) {
        const float wp = __shfl(w, u);
#pragma unroll
        for (int j = 0; j < kPer; ++j) acc[j] = fmaf(wp, x[r][u][j], acc[j]);
      }
      float* out_row = out + sh * D;
#pragma unroll
      for (int j = 0; j < kPer; ++j) out_row[j * kWave + lane] = den > 0.0f ? acc[j] / den : 0.0f;
      if (lse != nullptr && lane == 0) lse[sh] = den > 0.0f ? M + __logf(den) : -INFINITY;
    }
    if (leader) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <typename T, int D, int G>
constexpr int pass1_min_workgroups() {
  constexpr int max_g = sizeof(T) == 2 ? (D == 64 ? 7 : 4) : (D == 64 ? 5 : 2);
  return G <= max_g ? 2 : 1;
}

template <typename T, int D, int G, int NW>
__global__ __launch_bounds__(NW * kWave, (pass1_min_workgroups<T, D, G>())) void decode_pass1_kernel(
    const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc,
    const int32_t* __restrict__ tables, int W, const int32_t* __restrict__ ctx_lens,
    int num_q_heads, int num_kv_heads, int num_blocks, float scale_log2, int part_tokens,
    int max_parts, float* __restrict__ part_out, float* __restrict__ part_lse,
    float* __restrict__ out, float* __restrict__ lse, int order,
    const int4* __restrict__ plan, const int* __restrict__ plan_count,
    const int32_t* __restrict__ nslots, int* __restrict__ merge_ctr, const PassAppend ap) {
  using Gm = Geom<T, D>;
  Unit un;
  if (!resolve_unit(un, order, num_kv_heads, plan, plan_count, ctx_lens, W, part_tokens, out,
                    merge_ctr))
    return;
  const int part = un.part, kvh = un.kvh, s = un.s, tok0 = un.tok0, tok1 = un.tok1;
  const bool direct = un.direct, merge = un.merge;
  const int wave = NW == 1 ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  // (marked unlikely, which keeps the block loop's register allocation that of plain
  // decode)
  if (__builtin_expect(ap.k_new != nullptr, 0))
    append_in_unit<T, D, NW>(const_cast<T*>(kc), const_cast<T*>(vc), ap, tables, W, ctx_lens, s,
                             kvh, num_kv_heads, num_blocks, tok0, tok1, wave, lane);

  GroupState<T, D, G> st;
  attend_range<T, D, G, NW, true>(st, q, kc, vc, tables, W, s, s, kvh, num_q_heads,
                                  num_kv_heads, num_blocks, scale_log2, tok0, tok1, wave, lane);
  const int grp = lane / kLanesPerToken;
  const int sub = lane % kLanesPerToken;

  if constexpr (NW == 1) {
    // Lanes of token group 0 hold the totals for their dims: write them.
    if (grp == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float L = st.l[g];
        const float ls = L > 0.0f ? (st.m[g] + __log2f(L)) * kLn2 : -INFINITY;
        const size_t sh = static_cast<size_t>(s) * num_q_heads + kvh * G + g;
        float* dst = direct ? out + sh * D : part_out + (sh * max_parts + part) * D;
#pragma unroll
        for (int e = 0; e < Gm::kElems; e += 4) {
          float4 v;
          v.x = L > 0.0f ? st.acc[g][e + 0] / L : 0.0f;
          v.y = L > 0.0f ? st.acc[g][e + 1] / L : 0.0f;
          v.z = L > 0.0f ? st.acc[g][e + 2] / L : 0.0f;
          v.w = L > 0.0f ? st.acc[g][e + 3] / L : 0.0f;
          *reinterpret_cast<float4*>(dst + lane_dim<T, D>(sub, e)) = v;
        }
        if (sub == 0) {
          if (direct) {
            if (lse != nullptr) lse[sh] = ls;
          } else {
            part_lse[sh * max_parts + part] = ls;
          }
        }
      }
    }
  } else {
    // Merge the waves through LDS.
    __shared__ float s_m[NW][G];
    __shared__ float s_l[NW][G];
    __shared__ float s_acc[NW][G][D];
    if (grp == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int e = 0; e < Gm::kElems; ++e)
          s_acc[wave][g][lane_dim<T, D>(sub, e)] = st.acc[g][e];
        if (sub == 0) {
          s_m[wave][g] = st.m[g];
          s_l[wave][g] = st.l[g];
        }
      }
    }
    // slots of a split sequence; the last of its units to finish merges them
    const int n_merge = merge ? min(nslots[s], max_parts) : 0;
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += NW * kWave) {
      const int g = idx / D;
      const int d = idx % D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][g]);
      float L = 0.0f, O = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float a = (s_m[w][g] == -INFINITY) ? 0.0f : fast_exp2(s_m[w][g] - M);
        L = fmaf(s_l[w][g], a, L);
        O = fmaf(s_acc[w][g][d], a, O);
      }
      const float o = L > 0.0f ? O / L : 0.0f;
      const float ls = L > 0.0f ? (M + __log2f(L)) * kLn2 : -INFINITY;
      const size_t sh = static_cast<size_t>(s) * num_q_heads + kvh * G + g;
      if (direct) {
        out[sh * D + d] = o;
        if (lse != nullptr && d == 0) lse[sh] = ls;
      } else if (n_merge > 0) {
        // device-scope stores (global_store ... sc1): written through to where every XCD's
        // device-scope loads see them, so the merging workgroup needs no cache flush
        float* po = part_out + (sh * max_parts + part) * D + d;
        __hip_atomic_store(po, o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (d == 0)
          __hip_atomic_store(part_lse + sh * max_parts + part, ls, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      } else {
        part_out[(sh * max_parts + part) * D + d] = o;
        if (d == 0) part_lse[sh * max_parts + part] = ls;
      }
    }
    // (marked unlikely: with the merge on the cold path the register allocation of the
    // block loop matches the kernel without it, which has no spill at 256 VGPRs)
    if (__builtin_expect(n_merge > 0, 0))
      merge_when_last<D, G, NW>(n_merge, merge_ctr, s, kvh, num_q_heads, num_kv_heads, max_parts,
                                out, lse, part_out, part_lse, wave, lane);
  }

}

void combine_launch(hipStream_t stream, float* out, float* lse, const float* part_out,
                    const float* part_lse, const int32_t* ctx, const int32_t* nslots, int batch,
                    int cap, int hq, int D, int part_tokens, int max_parts, int skip_single) {
  const int rows = batch * hq;
  if (max_parts > kMaxInPassMergeSlots && max_parts <= kMaxTwoLevelSlots) {
    if (D == 64)
      hipLaunchKernelGGL(lse_combine_grouped_kernel<64>, dim3(rows), dim3(kMergeGroups * kWave), 0,
                         stream, out, lse, part_out, part_lse, ctx, nslots, batch, cap, hq,
                         part_tokens, max_parts, skip_single);
    else
      hipLaunchKernelGGL(lse_combine_grouped_kernel<128>, dim3(rows), dim3(kMergeGroups * kWave),
                         0, stream, out, lse, part_out, part_lse, ctx, nslots, batch, cap, hq,
                         part_tokens, max_parts, skip_single);
    return;
  }
  const dim3 grid((rows + kCombineWaves - 1) / kCombineWaves);
  if (D == 64)
    hipLaunchKernelGGL(lse_combine_kernel<64>, grid, dim3(kCombineWaves * kWave), 0, stream, out,
                       lse, part_out, part_lse, ctx, nslots, batch, cap, hq, part_tokens,
                       max_parts, skip_single);
  else
    hipLaunchKernelGGL(lse_combine_kernel<128>, grid, dim3(kCombineWaves * kWave), 0, stream,
                       out, lse, part_out, part_lse, ctx, nslots, batch, cap, hq, part_tokens,
                       max_parts, skip_single);
}

// Work plan of the first pass: the (sequence, partition) units in longest-first order,
// each entry {sequence, partition, context length clamped to the table, 0},
// so the hardware dispatcher, which hands out workgroups in grid order, schedules them
// like longest-processing-time-first list scheduling.  Every full partition (exactly
// part_tokens tokens) comes first, in sequence order; then the last partition of every
// split sequence (so its merge happens early); then each other sequence's only unit,
// bucketed by its length in 16-token blocks (>> key_shift), longest bucket first.
// part_tokens = 0 means one unit per sequence, bucketed by its whole length.
// The order only changes which workgroup runs when, never a unit's result.
// One workgroup; plan holds at most batch * np entries.
constexpr int kPlanThreads = 1024;
constexpr int kPlanBuckets = kPlanThreads;

// Inclusive prefix sum over the workgroup (thread order); every thread gets its own.
// Wave-level shuffles, then one pass over the per-wave totals: two barriers.
__device__ __forceinline__ int block_scan_inclusive(int* s_wave, int v) {
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int x = __shfl_up(v, off);
    if (lane >= off) v += x;
  }
  if (lane == kWave - 1) s_wave[wave] = v;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += s_wave[w];
  __syncthreads();
  return v + before;
}

// What the plan needs to know about one call.  With fork groups (shared-prefix decode),
// every sequence's leading group_shared_blocks[g] blocks are attended by the shared
// kernel into slots [0, nsp), and only the rest of its context becomes plan units.
struct PlanInput {
  const int32_t* ctx;
  int batch;
  int cap;          // table capacity in tokens: lengths are clamped to it
  int part_tokens;  // 0: one unit per sequence (or per private range)
  int max_slots;    // partial-result slots per (sequence, head)
  int key_shift;    // length bucket = blocks >> key_shift
  const int32_t* group_starts;         // nullable: no fork groups
  const int32_t* group_shared_blocks;
  int num_groups;
  int max_shared_blocks;  // shared lengths are clamped to this and to the table width
  int* merge_ctr;         // nullable: per (sequence, KV head) merge counters, zeroed here
  int ctr_count;
};

// Tokens of group g's shared prefix that the shared pass attends, clamped exactly as the
// shared pass clamps them (blocks past the bound stay private: still correct, less shared).
__device__ __forceinline__ int shared_prefix_tokens(int blocks, int max_blocks, int W) {
  return max(0, min(blocks, min(max_blocks, W))) * kBlockTokens;
}

// A sequence's units: `full` partitions of part_tokens tokens starting at `base`, then
// (tail == 1) one shorter unit of tail_len tokens (an empty one when the sequence has no
// tokens and nothing shared).  Slots: nsp shared ones first, then one per unit.
struct SeqUnits {
  int n, base, nsp, full, tail, tail_len;
};

// Largest g with starts[g] <= s; `starts` is the group start array or its LDS copy.
__device__ __forceinline__ int group_of(const int32_t* starts, int num_groups, int s) {
  int lo = 0, hi = num_groups;
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (starts[mid] <= s) lo = mid; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ int shared_slots(int shared_tokens, int part_tokens) {
  if (shared_tokens <= 0) return 0;
  return part_tokens > 0 ? (shared_tokens + part_tokens - 1) / part_tokens : 1;
}

__device__ __forceinline__ SeqUnits seq_units(const PlanInput& in, int s,
                                              const int32_t* starts) {
  SeqUnits u;
  int n = in.ctx[s];
  u.n = n < 0 ? 0 : min(n, in.cap);
  int shared = 0;
  if (in.group_starts != nullptr) {
    const int g = group_of(starts, in.num_groups, s);
    shared = shared_prefix_tokens(in.group_shared_blocks[g], in.max_shared_blocks,
                                  in.cap / kBlockTokens);
  }
  u.nsp = min(shared_slots(shared, in.part_tokens), in.max_slots);
  u.base = min(shared, u.n);
  const int priv = u.n - u.base;
  const int room = in.max_slots - u.nsp;  // slots left for the private range
  if (in.part_tokens > 0) {
    u.full = min(priv / in.part_tokens, room);
    u.tail_len = priv - u.full * in.part_tokens;
    u.tail = (u.full < room) && (u.tail_len > 0 || (u.nsp == 0 && u.full == 0));
  } else {
    u.full = 0;
    u.tail_len = priv;
    u.tail = room > 0 && (priv > 0 || u.nsp == 0);
  }
  return u;
}

__device__ __forceinline__ int unit_slot(const SeqUnits& u, int p) {
  const bool only = u.nsp == 0 && u.full + u.tail == 1;
  return (u.nsp + p) | (only ? kDirectFlag : 0);
}

// Writes plan entries {sequence, first token, end token, slot | kDirectFlag}, their count,
// and per sequence the number of partial slots the combine must merge (0: the sequence's
// only unit writes out / lse itself).
// Group starts are searched in an LDS copy when they fit (one load wave instead of a
// chain of dependent global loads per sequence).
constexpr int kPlanLdsGroups = 2047;
constexpr int kPlanLaneRun = 16;

__device__ __forceinline__ void build_plan(int4* __restrict__ plan, int* __restrict__ plan_count,
                                           int* __restrict__ nslots, const PlanInput in) {
  __shared__ int s_cursor[kPlanBuckets];
  __shared__ int s_scan[kPlanThreads / kWave];
  __shared__ int s_full_total;
  __shared__ int s_starts[kPlanLdsGroups + 1];
  const int tid = threadIdx.x;
  s_cursor[tid] = 0;
  if (tid == 0) s_full_total = 0;
  if (in.merge_ctr != nullptr)
    for (int i = tid; i < in.ctr_count; i += kPlanThreads) in.merge_ctr[i] = 0;
  const bool lds_starts = in.group_starts != nullptr && in.num_groups <= kPlanLdsGroups;
  if (lds_starts)
    for (int g = tid; g <= in.num_groups; g += kPlanThreads) s_starts[g] = in.group_starts[g];
  const int32_t* starts = lds_starts ? s_starts : in.group_starts;
  __syncthreads();
  const int P = in.part_tokens;
  if (in.group_starts != nullptr) {  // groups must tile 0..batch-1 in order
    for (int g = tid; g < in.num_groups; g += kPlanThreads) {
      const bool bad = in.group_starts[g] > in.group_starts[g + 1] ||
                       (g == 0 && in.group_starts[0] != 0) ||
                       (g == in.num_groups - 1 && in.group_starts[in.num_groups] != in.batch);
      if (bad) PKV_FLAG_ERROR(PKV_DEVERR_GROUPS);
    }
  }
  // The last unit of a split sequence goes in the first bucket, right after the full
  // partitions: the sequence's partial results are then complete, and merged, long before
  // the end of the pass instead of on its critical path.
  auto key_of = [&](const SeqUnits& u) {
    if (u.full > 0) return kPlanBuckets - 1;
    return min(kPlanBuckets - 1, ((u.tail_len + kBlockTokens - 1) / kBlockTokens) >> in.key_shift);
  };
  SeqUnits first = {0, 0, 0, 0, 0, 0};  // this thread's sequence of the first round
  for (int base = 0; base < in.batch; base += kPlanThreads) {
    const int s = base + tid;
    SeqUnits u = {0, 0, 0, 0, 0, 0};
    if (s < in.batch) {
      const int raw = in.ctx[s];
      if (raw < 0 || raw > in.cap) PKV_FLAG_ERROR(PKV_DEVERR_CONTEXT);
      u = seq_units(in, s, starts);
      if (base == 0) first = u;
      const int units = u.full + u.tail;
      const int covered = u.base + u.full * P + (u.tail ? u.tail_len : 0);
      if (covered < u.n) PKV_FLAG_ERROR(PKV_DEVERR_MAX_CONTEXT);
      nslots[s] = (u.nsp == 0 && units == 1) ? 0 : u.nsp + units;
      if (u.tail) atomicAdd(&s_cursor[key_of(u)], 1);
    }
    if (P == 0) {  // one unit per sequence: no full partitions to place
      __syncthreads();
      continue;
    }
    const int incl = block_scan_inclusive(s_scan, u.full);
    const int first = s_full_total + incl - u.full;
    // The full partitions' entries.  A thread stores its sequence's when they are few; a
    // sequence with more than kPlanLaneRun (64 for 32768 tokens at P = 512: one thread
    // storing them in a row was the plan's longest chain) has them stored by every lane
    // of the wave, one such sequence at a time.  unit_slot(u, p) is unit_slot(u, 0) + p:
    // the direct flag is only set for a sequence's single unit.
    const bool own = u.full <= kPlanLaneRun;
    for (int p = 0; p < (own ? u.full : 0); ++p) {
      const int t0 = u.base + p * P;
      plan[first + p] = make_int4(s, t0, t0 + P, unit_slot(u, p));
    }
    {
      const int lane = tid % kWave;
      const int slot0 = u.full > 0 ? unit_slot(u, 0) : 0;
      unsigned long long pending = __ballot(!own);
      while (pending != 0) {
        const int j = __builtin_ctzll(pending);
        pending &= pending - 1;
        const int sj = __shfl(s, j), fj = __shfl(first, j), nj = __shfl(u.full, j);
        const int bj = __shfl(u.base, j), slj = __shfl(slot0, j);
        for (int p = lane; p < nj; p += kWave) {
          const int t0 = bj + p * P;
          plan[fj + p] = make_int4(sj, t0, t0 + P, slj + p);
        }
      }
    }
    __syncthreads();
    if (tid == kPlanThreads - 1) s_full_total += incl;
    __syncthreads();
  }
  // Bucket start offsets, longest bucket first; thread t owns bucket kPlanBuckets-1-t.
  const int kb = kPlanBuckets - 1 - tid;
  const int h = s_cursor[kb];
  const int incl = block_scan_inclusive(s_scan, h);
  s_cursor[kb] = s_full_total + incl - h;
  if (tid == kPlanThreads - 1) *plan_count = s_full_total + incl;
  __syncthreads();
  for (int s = tid; s < in.batch; s += kPlanThreads) {
    const SeqUnits u = s == tid ? first : seq_units(in, s, starts);
    if (u.tail) {
      const int t0 = u.base + u.full * P;
      const int i = atomicAdd(&s_cursor[key_of(u)], 1);
      plan[i] = make_int4(s, t0, t0 + u.tail_len, unit_slot(u, u.full));
    }
  }
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(int4* __restrict__ plan,
                                                             int* __restrict__ plan_count,
                                                             int* __restrict__ nslots,
                                                             const PlanInput in) {
  build_plan(plan, plan_count, nslots, in);
}

// Prologue of an append-and-decode step in one launch: workgroup 0 writes the work
// plan (it only reads the context lengths); every other workgroup appends one new
// token per wavefront.  The two jobs touch disjoint memory.
constexpr int kAppendPerGroup = kPlanThreads / kWave;

__global__ __launch_bounds__(kPlanThreads) void prologue_kernel(
    int4* __restrict__ plan, int* __restrict__ plan_count, int* __restrict__ nslots,
    const PlanInput in, uint4* __restrict__ kc,
    uint4* __restrict__ vc, const uint4* __restrict__ kn, const uint4* __restrict__ vn,
    const int32_t* __restrict__ tables, int W, const int32_t* __restrict__ start_pos,
    const int32_t* __restrict__ cu, int total, int num_kv_heads, int row_vecs,
    int num_blocks) {
  if (blockIdx.x == 0) {
    build_plan(plan, plan_count, nslots, in);
    return;
  }
  const int i = (blockIdx.x - 1) * kAppendPerGroup + static_cast<int>(threadIdx.x) / kWave;
  if (i >= total) return;
  append_token(kc, vc, kn, vn, tables, W, start_pos, cu, in.batch, total, num_kv_heads,
               row_vecs, num_blocks, i, static_cast<int>(threadIdx.x) % kWave, &g_pkv_error_word);
}

// First pass over fork groups' shared prefixes (spindle, "Paging": forks share blocks
// copy-on-write).  Workgroup = (shared partition, KV head, group).  Partition `part`
// covers shared tokens [part * P, min((part + 1) * P, shared)); every member of the group
// gets its partial result for that range in slot `part`, the plan puts its private range
// in the slots after the shared ones, and the combine merges them.
constexpr int kSharedWaves = 4;

// Slot `part` of member s over shared tokens [tok0, tok1) by one wave, through the
// member's own table row (plain loads, so sibling waves find the blocks cached).
template <typename T, int D, int G>
__device__ __forceinline__ void shared_member(
    const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc,
    const int32_t* __restrict__ tables, int W, int s, int n, int kvh, int num_q_heads,
    int num_kv_heads, int num_blocks, float scale_log2, int tok0, int tok1, int part,
    int max_parts, float* __restrict__ part_out, float* __restrict__ part_lse, int lane) {
  using Gm = Geom<T, D>;
  const int grp = lane / kLanesPerToken;
  const int sub = lane % kLanesPerToken;
  // A member shorter than this slot's start gets an empty range that still begins on
  // the block boundary tok0 (attend_range needs a block-aligned start).
  const int t1 = max(tok0, min(tok1, n));
  GroupState<T, D, G> st;
  attend_range<T, D, G, 1, false>(st, q, kc, vc, tables, W, s, s, kvh, num_q_heads,
                                     num_kv_heads, num_blocks, scale_log2, tok0, t1, 0, lane);
  if (grp != 0) return;
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    const float L = st.l[gg];
    const float ls = L > 0.0f ? (st.m[gg] + __log2f(L)) * kLn2 : -INFINITY;
    const size_t sh = static_cast<size_t>(s) * num_q_heads + kvh * G + gg;
    float* dst = part_out + (sh * max_parts + part) * D;
#pragma unroll
    for (int e = 0; e < Gm::kElems; e += 4) {
      float4 v;
      v.x = L > 0.0f ? st.acc[gg][e + 0] / L : 0.0f;
      v.y = L > 0.0f ? st.acc[gg][e + 1] / L : 0.0f;
      v.z = L > 0.0f ? st.acc[gg][e + 2] / L : 0.0f;
      v.w = L > 0.0f ? st.acc[gg][e + 3] / L : 0.0f;
      *reinterpret_cast<float4*>(dst + lane_dim<T, D>(sub, e)) = v;
    }
    if (sub == 0) part_lse[sh * max_parts + part] = ls;
  }
}

struct SharedRange {
  int tok0, tok1;  // shared tokens of this workgroup's slot
  int m0, m1;      // the group's members, clamped to [0, batch)
  bool live;
};

__device__ __forceinline__ SharedRange shared_range(const int32_t* __restrict__ group_starts,
                                                    const int32_t* __restrict__ group_shared,
                                                    int g, int part, int part_tokens,
                                                    int max_parts, int max_shared_blocks, int W,
                                                    int batch) {
  SharedRange r;
  const int shared = shared_prefix_tokens(group_shared[g], max_shared_blocks, W);
  const int nsp = min(shared_slots(shared, part_tokens), max_parts);
  r.live = part < nsp;
  const int P = part_tokens > 0 ? part_tokens : shared;
  r.tok0 = part * P;
  r.tok1 = min(shared, r.tok0 + P);
  r.m0 = max(group_starts[g], 0);  // malformed groups (flagged by the plan): stay in range
  r.m1 = min(group_starts[g + 1], batch);
  return r;
}

// Generic version: wave w attends for members w, w + kSharedWaves, ..., each through its
// own table row.  Sibling waves fetch the same blocks, so HBM serves most of them once.
template <typename T, int D, int G>
__global__ __launch_bounds__(kSharedWaves * kWave) void decode_shared_kernel(
    const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc,
    const int32_t* __restrict__ tables, int W, const int32_t* __restrict__ ctx_lens,
    const int32_t* __restrict__ group_starts, const int32_t* __restrict__ group_shared_blocks,
    int num_q_heads, int num_kv_heads, int num_blocks, float scale_log2, int part_tokens,
    int max_parts, int max_shared_blocks, int batch, float* __restrict__ part_out,
    float* __restrict__ part_lse) {
  const SharedRange r = shared_range(group_starts, group_shared_blocks, blockIdx.z, blockIdx.x,
                                     part_tokens, max_parts, max_shared_blocks, W, batch);
  if (!r.live) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int cap = W * kBlockTokens;
  for (int s = r.m0 + wave; s < r.m1; s += kSharedWaves) {
    int n = ctx_lens[s];
    n = n < 0 ? 0 : min(n, cap);
    shared_member<T, D, G>(q, kc, vc, tables, W, s, n, blockIdx.y, num_q_heads, num_kv_heads,
                           num_blocks, scale_log2, r.tok0, r.tok1, blockIdx.x, max_parts,
                           part_out, part_lse, lane);
  }
}

// One launch for a batch of fork groups: workgroups [0, shared_wgs) are (shared partition,
// KV head, group) = (x % nsp, x / nsp % Hkv, x / (nsp * Hkv)); the rest take the plan's
// units (each sequence's private range, and whole sequences of groups that share nothing),
// unit (x - shared_wgs) / Hkv for KV head (x - shared_wgs) % Hkv, as one-member tiles
// through the member's own table row.  The private units' short latency chains overlap
// the shared stream instead of following it.
// Token limits of members base .. base + kMembers - 1 of a decode tile: each member's
// context length clamped to the table and to `tok1`, 0 for members not taken.
template <int G>
__device__ __forceinline__ void decode_limits(int (&lim)[kMfmaRows / G],
                                              const int32_t* __restrict__ ctx_lens, int base,
                                              unsigned take, int cap, int tok1) {
#pragma unroll
  for (int mi = 0; mi < kMfmaRows / G; ++mi) {
    int n = 0;
    if ((take >> mi) & 1u) {
      n = ctx_lens[base + mi];
      n = n < 0 ? 0 : min(min(n, cap), tok1);
    }
    lim[mi] = n;
  }
}

template <int D, int G>
__global__ __launch_bounds__(kTileWaves * kWave) void decode_shared_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ tables, int W,
    const int32_t* __restrict__ ctx_lens, const int32_t* __restrict__ group_starts,
    const int32_t* __restrict__ group_shared_blocks, int num_groups, int nsp_grid,
    int num_q_heads, int num_kv_heads, int num_blocks, float scale_log2, int part_tokens,
    int max_parts, int max_shared_blocks, int batch, float* __restrict__ part_out,
    float* __restrict__ part_lse, float* __restrict__ out, float* __restrict__ lse,
    const int4* __restrict__ plan, const int* __restrict__ plan_count) {
  constexpr int kMembers = kMfmaRows / G;  // members per row tile
  __shared__ MfmaShared<D> sm;
  const int cap = W * kBlockTokens;
  const int shared_wgs = nsp_grid * num_kv_heads * num_groups;
  const int x = blockIdx.x;
  int lim[kMembers];
  if (x >= shared_wgs) {
    const int u = (x - shared_wgs) / num_kv_heads;
    const int kvh = (x - shared_wgs) % num_kv_heads;
    if (u >= *plan_count) return;
    const int4 e = plan[u];
    const bool direct = (e.w & kDirectFlag) != 0;
    decode_limits<G>(lim, ctx_lens, e.x, 1u, cap, e.z);
    mfma_tile<D, G>(sm, q, kc, vc, tables + static_cast<size_t>(e.x) * W, nullptr, W, lim, 1u,
                    e.x, kvh, num_q_heads, num_kv_heads, num_blocks, scale_log2, e.y,
                    direct ? 0 : e.w & kSlotMask, direct ? 1 : max_parts,
                    direct ? out : part_out, direct ? lse : part_lse);
    return;
  }
  const int part = x % nsp_grid;
  const int kvh = (x / nsp_grid) % num_kv_heads;
  const SharedRange r = shared_range(group_starts, group_shared_blocks, x / (nsp_grid * num_kv_heads),
                                     part, part_tokens, max_parts, max_shared_blocks, W, batch);
  if (!r.live) return;
  for (int base = r.m0; base < r.m1; base += kMembers) {
    const int cnt = min(kMembers, r.m1 - base);
    const unsigned all = (1u << cnt) - 1u;
    const int32_t* rows = tables + static_cast<size_t>(base) * W;
    decode_limits<G>(lim, ctx_lens, base, all, cap, r.tok1);
    // The tile's members through the first one's row; if the sharing hint was wrong for
    // some, the others again without them, then each of them through its own row.
    unsigned differ = mfma_tile<D, G>(sm, q, kc, vc, rows, rows, W, lim, all, base, kvh,
                                      num_q_heads, num_kv_heads, num_blocks, scale_log2, r.tok0,
                                      part, max_parts, part_out, part_lse);
    if (differ != 0 && (all & ~differ) != 0)
      mfma_tile<D, G>(sm, q, kc, vc, rows, nullptr, W, lim, all & ~differ, base, kvh,
                      num_q_heads, num_kv_heads, num_blocks, scale_log2, r.tok0, part, max_parts,
                      part_out, part_lse);
    while (differ != 0) {
      const int mi = __builtin_ctz(differ);
      differ &= differ - 1u;
      mfma_tile<D, G>(sm, q, kc, vc, rows + static_cast<size_t>(mi) * W, nullptr, W, lim,
                      1u << mi, base, kvh, num_q_heads, num_kv_heads, num_blocks, scale_log2,
                      r.tok0, part, max_parts, part_out, part_lse);
    }
  }
}

// The first pass's in-launch append (see append_in_unit) for the matrix-core tile's lane
// layout: a new token's K chunk of score step k (dims 32k + 8h .. + 7) is stored by lane
// (c = slot, h), its V dims c * D/16 .. by lane (c, h = slot / 4), in the wave that takes
// the token's block, which are the lanes that load those bytes in mfma_load_block.
template <int D>
__device__ __forceinline__ void mfma_append_in_unit(
    uint16_t* kc, uint16_t* vc, const PassAppend& ap, const int32_t* __restrict__ tables, int W,
    const int32_t* __restrict__ ctx_lens, int s, int kvh, int num_kv_heads, int num_blocks,
    int tok0, int tok1, int wave, int lane) {
  using Mg = MfmaGeom<D>;
  const int c0 = ap.cu[s];
  const int c1 = ap.cu[s + 1];
  if (c0 < 0 || c1 < c0 || c1 > ap.total) {
    if (wave == 0 && lane == 0 && kvh == 0) PKV_FLAG_ERROR(PKV_DEVERR_CU);
    return;
  }
  const int cap = W * kBlockTokens;
  int n = ctx_lens[s];
  n = n < 0 ? 0 : min(n, cap);
  const bool last_unit = tok1 >= n;
  const int p0 = ap.start_pos[s];
  const int b0 = tok0 / kBlockTokens;
  const int c = lane % 16;
  const int h = lane / 16;
  const uint16_t* kn = static_cast<const uint16_t*>(ap.k_new);
  const uint16_t* vn = static_cast<const uint16_t*>(ap.v_new);
  for (int t = c0; t < c1; ++t) {
    const int pos = p0 + (t - c0);
    const bool inside = pos >= tok0 && pos < tok1;
    if (!inside && !(last_unit && pos >= tok1)) continue;
    if (pos < 0 || pos >= cap) {
      if (wave == 0 && lane == 0) PKV_FLAG_ERROR(PKV_DEVERR_POSITION);
      continue;
    }
    const int bi = pos / kBlockTokens;
    const int owner = inside ? (bi - b0) % kTileWaves : 0;
    if (wave != owner) continue;
    const int slot = pos % kBlockTokens;
    const int id = tables[static_cast<size_t>(s) * W + bi];
    if (static_cast<unsigned>(id) >= static_cast<unsigned>(num_blocks)) {
      if (lane == 0) PKV_FLAG_ERROR(PKV_DEVERR_BLOCK_ID);
      continue;
    }
    const size_t row = ((static_cast<size_t>(id) * num_kv_heads + kvh) * kBlockTokens + slot) * D;
    const size_t src = (static_cast<size_t>(t) * num_kv_heads + kvh) * D;
    if (c == slot) {
#pragma unroll
      for (int k = 0; k < Mg::kQkSteps; ++k)
        *reinterpret_cast<u32x4_t*>(kc + row + 32 * k + 8 * h) =
            *reinterpret_cast<const u32x4_t*>(kn + src + 32 * k + 8 * h);
    }
    if (h == slot / 4) {
      const size_t e = static_cast<size_t>(c) * Mg::kTiles;
      if constexpr (Mg::kVWords == 4)
        *reinterpret_cast<u32x4_t*>(vc + row + e) = *reinterpret_cast<const u32x4_t*>(vn + src + e);
      else
        *reinterpret_cast<u32x2_t*>(vc + row + e) = *reinterpret_cast<const u32x2_t*>(vn + src + e);
    }
  }
}

// Plain decode on the matrix cores, for GQA groups large enough that one 16-row tile of a
// sequence's G query heads (the rows past G idle) costs fewer instructions per block than
// the VALU pass's G dot products per token: one workgroup per work unit and KV head, in
// the plan's order (or the grid orders of the first pass), with the first pass's
// in-launch append and merge.  Results equal the first pass's within rounding (the scores
// and the weighted sum run on the matrix cores), not bit for bit.
template <int D, int G, bool kAppend>
__global__ __launch_bounds__(kTileWaves * kWave) void decode_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ tables, int W,
    const int32_t* __restrict__ ctx_lens, int num_q_heads, int num_kv_heads, int num_blocks,
    float scale_log2, int part_tokens, int max_parts, float* __restrict__ part_out,
    float* __restrict__ part_lse, float* __restrict__ out, float* __restrict__ lse, int order,
    const int4* __restrict__ plan, const int* __restrict__ plan_count,
    const int32_t* __restrict__ nslots, int* __restrict__ merge_ctr, const PassAppend ap) {
  __shared__ MfmaShared<D> sm;
  Unit un;
  if (!resolve_unit(un, order, num_kv_heads, plan, plan_count, ctx_lens, W, part_tokens, out,
                    merge_ctr))
    return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  uint16_t* kw = const_cast<uint16_t*>(kc);
  uint16_t* vw = const_cast<uint16_t*>(vc);
  // The step's new token: a sequence appending one token inside this unit's range gets it
  // into the tile from registers (loaded now, unconditionally, from a row that is always
  // valid) and writes the cache after the tile, so the tile's loads never wait for the
  // write.  Several new tokens in one sequence are written before the tile and read back.
  MfmaNewToken<D> nt;
  nt.pos = -1;
  bool write_first = false;
  if constexpr (kAppend) {
    using Mg = MfmaGeom<D>;
    const int c0 = ap.cu[un.s];
    const int c1 = ap.cu[un.s + 1];
    const int p0 = ap.start_pos[un.s];
    const int row = min(max(c0, 0), ap.total - 1);
    const size_t src = (static_cast<size_t>(row) * num_kv_heads + un.kvh) * D;
    const uint16_t* kn = static_cast<const uint16_t*>(ap.k_new) + src;
    const uint16_t* vn = static_cast<const uint16_t*>(ap.v_new) + src;
    const int c = lane % 16;
    const int h = lane / 16;
#pragma unroll
    for (int k = 0; k < Mg::kQkSteps; ++k)
      nt.k[k] = *reinterpret_cast<const u32x4_t*>(kn + 32 * k + 8 * h);
    if constexpr (Mg::kVWords == 4) {
      const u32x4_t w = *reinterpret_cast<const u32x4_t*>(vn + c * Mg::kTiles);
#pragma unroll
      for (int j = 0; j < 4; ++j) nt.v[j] = w[j];
    } else {
      const u32x2_t w = *reinterpret_cast<const u32x2_t*>(vn + c * Mg::kTiles);
      nt.v[0] = w[0];
      nt.v[1] = w[1];
    }
    const bool valid = c0 >= 0 && c1 <= ap.total;
    if (valid && c1 - c0 == 1 && p0 >= un.tok0 && p0 < un.tok1)
      nt.pos = p0;
    else
      write_first = valid && c1 - c0 > 1;
    if (write_first)
      mfma_append_in_unit<D>(kw, vw, ap, tables, W, ctx_lens, un.s, un.kvh, num_kv_heads,
                             num_blocks, un.tok0, un.tok1, wave, lane);
  }
  int lim[kMfmaRows / G];
  decode_limits<G>(lim, ctx_lens, un.s, 1u, W * kBlockTokens, un.tok1);
  // device-scope stores throughout, so that a merging workgroup of this launch reads the
  // partial results wherever they were written
  mfma_tile<D, G, true, true>(sm, q, kc, vc, tables + static_cast<size_t>(un.s) * W, nullptr,
                              W, lim, 1u, un.s, un.kvh, num_q_heads, num_kv_heads, num_blocks,
                              scale_log2, un.tok0, un.direct ? 0 : un.part,
                              un.direct ? 1 : max_parts, un.direct ? out : part_out,
                              un.direct ? lse : part_lse, kAppend ? &nt : nullptr);
  if constexpr (kAppend) {
    if (!write_first)
      mfma_append_in_unit<D>(kw, vw, ap, tables, W, ctx_lens, un.s, un.kvh, num_kv_heads,
                             num_blocks, un.tok0, un.tok1, wave, lane);
  }
  if (un.merge) {
    const int n_merge = min(nslots[un.s], max_parts);
    if (n_merge > 0)
      merge_when_last<D, G, kTileWaves>(n_merge, merge_ctr, un.s, un.kvh, num_q_heads,
                                        num_kv_heads, max_parts, out, lse, part_out, part_lse,
                                        wave, lane);
  }
}

using LaunchFn = void (*)(int, int, int, int, hipStream_t, const void*, const void*, const void*,
                          const int32_t*, int, const int32_t*, int, int, int, float, int, int,
                          float*, float*, float*, float*, const int4*, const int*,
                          const int32_t*, int*, const PassAppend&);

// order = kOrderPlanned: plan/plan_count from plan_kernel, grid of batch * np units.
template <int NW, typename T, int D, int G>
void pass1_launch(int order, int np, int num_kv_heads, int batch, hipStream_t stream,
                  const void* q, const void* kc, const void* vc, const int32_t* tables, int W,
                  const int32_t* ctx, int hq, int hkv, int nb, float scale_log2,
                  int part_tokens, int max_parts, float* part_out, float* part_lse, float* out,
                  float* lse, const int4* plan, const int* plan_count, const int32_t* nslots,
                  int* merge_ctr, const PassAppend& ap) {
  static_assert(NW > 1, "split sequences are merged in the multi-wave epilogue");
  dim3 grid;
  if (order == kOrderPlanned)
    grid = dim3(static_cast<unsigned>(num_kv_heads) * batch * np);
  else if (order == kOrderPartMinor)
    grid = dim3(np, num_kv_heads, batch);
  else
    grid = dim3(num_kv_heads, batch, np);
  hipLaunchKernelGGL((decode_pass1_kernel<T, D, G, NW>), grid, dim3(NW * kWave), 0,
                     stream, static_cast<const T*>(q), static_cast<const T*>(kc),
                     static_cast<const T*>(vc), tables, W, ctx, hq, hkv, nb, scale_log2,
                     part_tokens, max_parts, part_out, part_lse, out, lse, order, plan,
                     plan_count, nslots, merge_ctr, ap);
}

// The configuration the library ships: four waves share a (sequence, KV head,
// partition) unit, two blocks in flight per wave.
template <typename T, int D, int G>
void pass1_default(int order, int np, int num_kv_heads, int batch, hipStream_t stream,
                   const void* q, const void* kc, const void* vc, const int32_t* tables, int W,
                   const int32_t* ctx, int hq, int hkv, int nb, float scale_log2,
                   int part_tokens, int max_parts, float* part_out, float* part_lse, float* out,
                   float* lse, const int4* plan, const int* plan_count, const int32_t* nslots,
                   int* merge_ctr, const PassAppend& ap) {
  pass1_launch<4, T, D, G>(order, np, num_kv_heads, batch, stream, q, kc, vc, tables, W, ctx, hq,
                           hkv, nb, scale_log2, part_tokens, max_parts, part_out, part_lse, out,
                           lse, plan, plan_count, nslots, merge_ctr, ap);
}

// The matrix-core first pass (bf16 only), in the launch shapes of pass1_launch.
template <typename T, int D, int G>
void mfma_pass_launch(int order, int np, int num_kv_heads, int batch, hipStream_t stream,
                      const void* q, const void* kc, const void* vc, const int32_t* tables, int W,
                      const int32_t* ctx, int hq, int hkv, int nb, float scale_log2,
                      int part_tokens, int max_parts, float* part_out, float* part_lse,
                      float* out, float* lse, const int4* plan, const int* plan_count,
                      const int32_t* nslots, int* merge_ctr, const PassAppend& ap) {
  static_assert(sizeof(T) == 2, "the matrix-core pass reads bf16 caches");
  dim3 grid;
  if (order == kOrderPlanned)
    grid = dim3(static_cast<unsigned>(num_kv_heads) * batch * np);
  else if (order == kOrderPartMinor)
    grid = dim3(np, num_kv_heads, batch);
  else
    grid = dim3(num_kv_heads, batch, np);
  auto kernel = ap.k_new != nullptr ? decode_mfma_kernel<D, G, true>
                                    : decode_mfma_kernel<D, G, false>;
  hipLaunchKernelGGL(kernel, grid, dim3(kTileWaves * kWave), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kc),
                     static_cast<const uint16_t*>(vc), tables, W, ctx, hq, hkv, nb, scale_log2,
                     part_tokens, max_parts, part_out, part_lse, out, lse, order, plan,
                     plan_count, nslots, merge_ctr, ap);
}

struct SharedArgs {
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* tables;
  int W;
  const int32_t* ctx;
  const int32_t* group_starts;
  const int32_t* group_shared;
  int num_groups;
  int nsp;  // shared partitions per group in the grid (0: nothing shared)
  int hq, hkv, num_blocks;
  float scale_log2;
  int part_tokens, max_slots, max_shared_blocks, batch;
  float* part_out;
  float* part_lse;
  float* out;
  float* lse;
  const int4* plan;
  const int* plan_count;
};

// Launches the shared-prefix pass; returns true when that launch also ran the plan's
// units (bf16: one matrix-core launch for both), false when the first pass must follow.
using SharedFn = bool (*)(const SharedArgs&, hipStream_t);

template <typename T, int D, int G>
bool shared_launch(const SharedArgs& a, hipStream_t stream) {
  if constexpr (sizeof(T) == 2) {
    const dim3 block(kTileWaves * kWave);
    const int groups = a.nsp > 0 ? a.num_groups : 0;
    const long long wgs = static_cast<long long>(a.nsp) * a.hkv * groups +
                          static_cast<long long>(a.batch) * a.max_slots * a.hkv;
    hipLaunchKernelGGL((decode_shared_mfma_kernel<D, G>), dim3(static_cast<unsigned>(wgs)), block,
                       0, stream, static_cast<const uint16_t*>(a.q),
                       static_cast<const uint16_t*>(a.kc), static_cast<const uint16_t*>(a.vc),
                       a.tables, a.W, a.ctx, a.group_starts, a.group_shared, groups,
                       max(a.nsp, 1), a.hq, a.hkv, a.num_blocks, a.scale_log2, a.part_tokens,
                       a.max_slots, a.max_shared_blocks, a.batch, a.part_out, a.part_lse, a.out,
                       a.lse, a.plan, a.plan_count);
    return true;
  } else {
    const dim3 block(kSharedWaves * kWave);
    if (a.nsp > 0)
      hipLaunchKernelGGL((decode_shared_kernel<T, D, G>), dim3(a.nsp, a.hkv, a.num_groups), block,
                         0, stream, static_cast<const T*>(a.q), static_cast<const T*>(a.kc),
                         static_cast<const T*>(a.vc), a.tables, a.W, a.ctx, a.group_starts,
                         a.group_shared, a.hq, a.hkv, a.num_blocks, a.scale_log2, a.part_tokens,
                         a.max_slots, a.max_shared_blocks, a.batch, a.part_out, a.part_lse);
    return false;
  }
}

template <typename T, int D>
SharedFn pick_shared(int G) {
  switch (G) {
    case 1: return shared_launch<T, D, 1>;
    case 2: return shared_launch<T, D, 2>;
    case 3: return shared_launch<T, D, 3>;
    case 4: return shared_launch<T, D, 4>;
    case 5: return shared_launch<T, D, 5>;
    case 6: return shared_launch<T, D, 6>;
    case 7: return shared_launch<T, D, 7>;
    case 8: return shared_launch<T, D, 8>;
    default: return nullptr;
  }
}

// Smallest GQA group whose bf16 first pass runs on the matrix cores, per head_dim.
#ifndef PKV_MFMA_MIN_GROUP_D64
#define PKV_MFMA_MIN_GROUP_D64 7
#endif
#ifndef PKV_MFMA_MIN_GROUP_D128
#define PKV_MFMA_MIN_GROUP_D128 7
#endif

template <typename T, int D>
constexpr bool mfma_pass(int G) {
  return sizeof(T) == 2 && G >= (D == 64 ? PKV_MFMA_MIN_GROUP_D64 : PKV_MFMA_MIN_GROUP_D128);
}

template <typename T, int D, int G>
LaunchFn pass_for_group() {
  if constexpr (mfma_pass<T, D>(G))
    return mfma_pass_launch<T, D, G>;
  else
    return pass1_default<T, D, G>;
}

template <typename T, int D>
bool pick_group(int G, LaunchFn* fn) {
  switch (G) {
    case 1: *fn = pass_for_group<T, D, 1>(); return true;
    case 2: *fn = pass_for_group<T, D, 2>(); return true;
    case 3: *fn = pass_for_group<T, D, 3>(); return true;
    case 4: *fn = pass_for_group<T, D, 4>(); return true;
    case 5: *fn = pass_for_group<T, D, 5>(); return true;
    case 6: *fn = pass_for_group<T, D, 6>(); return true;
    case 7: *fn = pass_for_group<T, D, 7>(); return true;
    case 8: *fn = pass_for_group<T, D, 8>(); return true;
    default: return false;
  }
}

int check_decode_args(const void* q, const void* kc, const void* vc, const int32_t* tables,
                      int64_t bt_stride, const int32_t* ctx, int32_t batch, int32_t hq,
                      int32_t hkv, int32_t D, int32_t bs, int32_t nb, int32_t max_ctx,
                      int32_t part_tokens, int32_t dtype, LaunchFn* fn) {
  if (!q || !kc || !vc || !tables || !ctx) return PKV_ERR_NULL;
  if (dtype != PKV_F32 && dtype != PKV_BF16) return PKV_ERR_DTYPE;
  if (batch < 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0 || bs != kBlockTokens || nb <= 0 ||
      max_ctx < 0 || bt_stride <= 0 || bt_stride > (1 << 26) || part_tokens < 0 ||
      part_tokens % kBlockTokens != 0)
    return PKV_ERR_SHAPE;
  if (D != 64 && D != 128) return PKV_ERR_SHAPE;
  if (static_cast<int64_t>(max_ctx) > bt_stride * kBlockTokens) return PKV_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(kc) || !aligned16(vc)) return PKV_ERR_ARG;
  const int G = hq / hkv;
  bool ok;
  if (dtype == PKV_F32)
    ok = D == 64 ? pick_group<float, 64>(G, fn) : pick_group<float, 128>(G, fn);
  else
    ok = D == 64 ? pick_group<uint16_t, 64>(G, fn) : pick_group<uint16_t, 128>(G, fn);
  return ok ? PKV_OK : PKV_ERR_SHAPE;
}

int num_partitions(int32_t max_ctx, int32_t part_tokens) {
  if (part_tokens <= 0) return 1;
  return max_ctx > 0 ? (max_ctx + part_tokens - 1) / part_tokens : 1;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Partitioning of one call.  Plain decode: P = ceil(max_context_len / partition_size)
// partitions of partition_size tokens when that exceeds one (else one unit per sequence,
// written straight).  Shared-prefix decode: a sequence's slots are the shared prefix's
// partitions followed by its private range's, at most P + 1.
struct Geometry {
  int tokens;      // partition size used by the units (0: a whole sequence / range)
  int max_slots;   // partial-result slots per (sequence, query head)
  bool partials;   // partial-result arrays (and the combine) are needed
};

Geometry decode_geometry(int32_t max_ctx, int32_t partition_size, bool shared) {
  const int np = num_partitions(max_ctx, partition_size);
  Geometry g;
  if (shared) {
    g.tokens = partition_size;
    g.max_slots = (partition_size > 0 ? np : 1) + 1;
    g.partials = true;
  } else {
    const bool split = partition_size > 0 && np > 1;
    g.tokens = split ? partition_size : 0;
    g.max_slots = split ? np : 1;
    g.partials = split;
  }
  return g;
}

// Workspace: [plan count | plan entries (int4, batch * max_slots) | per-sequence slot counts
// (int32, batch) | partial outputs | partial lse | merge counters (int32, batch * num_q_heads)],
// each part 256-byte aligned.
struct Workspace {
  int* plan_count = nullptr;
  int4* plan = nullptr;
  int* nslots = nullptr;
  float* part_out = nullptr;
  float* part_lse = nullptr;
  int* merge_ctr = nullptr;  // batch * num_q_heads counters (indexed s * Hkv + KV head)
  size_t bytes = 0;
};

Workspace workspace_layout(void* base, int32_t batch, int32_t hq, int32_t D, const Geometry& g) {
  Workspace w;
  char* p = static_cast<char*>(base);
  size_t off = 0;
  w.plan_count = reinterpret_cast<int*>(p + off);
  off += kAlign;
  w.plan = reinterpret_cast<int4*>(p + off);
  off += align_up(static_cast<size_t>(batch) * g.max_slots * sizeof(int4));
  w.nslots = reinterpret_cast<int*>(p + off);
  off += align_up(static_cast<size_t>(batch) * sizeof(int));
  if (g.partials) {
    const size_t rows = static_cast<size_t>(batch) * hq * g.max_slots;
    w.part_out = reinterpret_cast<float*>(p + off);
    off += align_up(rows * D * sizeof(float));
    w.part_lse = reinterpret_cast<float*>(p + off);
    off += align_up(rows * sizeof(float));
    w.merge_ctr = reinterpret_cast<int*>(p + off);
    off += align_up(static_cast<size_t>(batch) * hq * sizeof(int));
  }
  w.bytes = off;
  return w;
}

int plan_key_shift(int32_t max_context_len, int32_t part_tokens) {
  const int longest = part_tokens > 0 ? part_tokens : max_context_len;
  int blocks = (longest + kBlockTokens - 1) / kBlockTokens;
  int shift = 0;
  while ((blocks >> shift) >= kPlanBuckets) ++shift;
  return shift;
}

PlanInput plan_input(const int32_t* ctx, int32_t batch, int cap, const Geometry& g,
                     int32_t max_context_len, const int32_t* group_starts,
                     const int32_t* group_shared_blocks, int32_t num_groups,
                     int32_t max_shared_blocks, int* merge_ctr = nullptr, int ctr_count = 0) {
  PlanInput in;
  in.ctx = ctx;
  in.batch = batch;
  in.cap = cap;
  in.part_tokens = g.tokens;
  in.max_slots = g.max_slots;
  in.key_shift = plan_key_shift(max_context_len, g.tokens);
  in.group_starts = group_starts;
  in.group_shared_blocks = group_shared_blocks;
  in.num_groups = num_groups;
  in.max_shared_blocks = max_shared_blocks;
  in.merge_ctr = merge_ctr;
  in.ctr_count = ctr_count;
  return in;
}

struct AppendArgs {
  const void* k_new = nullptr;
  const void* v_new = nullptr;
  const int32_t* start_pos = nullptr;
  const int32_t* cu = nullptr;
  int32_t total = 0;
};

struct Groups {
  const int32_t* starts = nullptr;         // null: no fork groups
  const int32_t* shared_blocks = nullptr;
  int32_t count = 0;
  int32_t max_shared_blocks = 0;           // host bound of shared_blocks[]
};

// Shared by the decode entry points: validates, then runs [plan or prologue] +
// [shared-prefix pass] + first pass + [combine].
int decode_impl(bool make_plan, float* out, float* lse, const void* q, const void* k_cache,
                const void* v_cache, const int32_t* block_tables, int64_t bt_stride,
                const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                int32_t max_context_len, float scale, int32_t partition_size, void* workspace,
                size_t workspace_bytes, int32_t dtype, pkv_stream_t stream,
                const AppendArgs* append = nullptr, const Groups* groups = nullptr,
                bool append_in_pass = false) {
  LaunchFn fn = nullptr;
  int st = check_decode_args(q, k_cache, v_cache, block_tables, bt_stride, context_lens, batch,
                             num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                             max_context_len, partition_size, dtype, &fn);
  if (st != PKV_OK) return st;
  if (!out) return PKV_ERR_NULL;
  if (batch == 0) return PKV_OK;
  const bool shared = groups != nullptr;
  const Geometry geo = decode_geometry(max_context_len, partition_size, shared);
  const Workspace need = workspace_layout(nullptr, batch, num_q_heads, head_dim, geo);
  if (workspace == nullptr || workspace_bytes < need.bytes) return PKV_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return PKV_ERR_ARG;
  const Workspace w = workspace_layout(workspace, batch, num_q_heads, head_dim, geo);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int cap = static_cast<int>(bt_stride) * kBlockTokens;
  // Plain decode merges split sequences inside the first pass when they have few slots.
  // Past kMaxInPassMergeSlots the merging workgroup's serial walk over the slots costs
  // more than the combine launch, whose (sequence, head) rows run in parallel; the
  // shared-prefix kernels always leave the merge to the combine launch.
  const bool in_pass_merge = !shared && geo.partials && geo.max_slots <= kMaxInPassMergeSlots;
  const PlanInput in = plan_input(context_lens, batch, cap, geo, max_context_len,
                                  shared ? groups->starts : nullptr,
                                  shared ? groups->shared_blocks : nullptr,
                                  shared ? groups->count : 0,
                                  shared ? groups->max_shared_blocks : 0,
                                  in_pass_merge ? w.merge_ctr : nullptr,
                                  in_pass_merge ? batch * num_q_heads : 0);
  // The append runs inside the first pass (plan made beforehand), or beside the plan in
  // one prologue launch, or on its own.
  PassAppend pa{nullptr, nullptr, nullptr, nullptr, 0};
  if (append_in_pass) {
    if (shared || make_plan) return PKV_ERR_ARG;
    if (append != nullptr && append->total > 0)
      pa = PassAppend{append->k_new, append->v_new, append->start_pos, append->cu, append->total};
  } else if (append != nullptr && append->total > 0) {
    const int eb = elem_bytes(dtype);
    const int wgs = 1 + (append->total + kAppendPerGroup - 1) / kAppendPerGroup;
    hipLaunchKernelGGL(prologue_kernel, dim3(wgs), dim3(kPlanThreads), 0, s, w.plan,
                       w.plan_count, w.nslots, in,
                       static_cast<uint4*>(const_cast<void*>(k_cache)),
                       static_cast<uint4*>(const_cast<void*>(v_cache)),
                       static_cast<const uint4*>(append->k_new),
                       static_cast<const uint4*>(append->v_new), block_tables,
                       static_cast<int>(bt_stride), append->start_pos, append->cu, append->total,
                       num_kv_heads, head_dim * eb / 16, num_blocks);
    if ((st = launch_status()) != PKV_OK) return st;
  } else if (make_plan) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, w.plan, w.plan_count,
                       w.nslots, in);
    if ((st = launch_status()) != PKV_OK) return st;
  }
  const float scale_log2 = scale_to_log2(scale);
  bool units_done = false;
  if (shared) {
    int nsp = 0;
    if (groups->count > 0 && groups->max_shared_blocks > 0) {
      const int shared_tokens =
          min(groups->max_shared_blocks, static_cast<int>(bt_stride)) * kBlockTokens;
      nsp = min(geo.tokens > 0 ? (shared_tokens + geo.tokens - 1) / geo.tokens : 1,
                geo.max_slots);
    }
    const int G = num_q_heads / num_kv_heads;
    SharedFn sf = dtype == PKV_F32
                      ? (head_dim == 64 ? pick_shared<float, 64>(G) : pick_shared<float, 128>(G))
                      : (head_dim == 64 ? pick_shared<uint16_t, 64>(G)
                                        : pick_shared<uint16_t, 128>(G));
    const SharedArgs a{q, k_cache, v_cache, block_tables, static_cast<int>(bt_stride),
                       context_lens, groups->starts, groups->shared_blocks, groups->count, nsp,
                       num_q_heads, num_kv_heads, num_blocks, scale_log2, geo.tokens,
                       geo.max_slots, groups->max_shared_blocks, batch, w.part_out, w.part_lse,
                       out, lse, w.plan, w.plan_count};
    units_done = sf(a, s);
    if ((st = launch_status()) != PKV_OK) return st;
  }
  if (!units_done) {
    fn(kOrderPlanned, geo.max_slots, num_kv_heads, batch, s, q, k_cache, v_cache, block_tables,
       static_cast<int>(bt_stride), context_lens, num_q_heads, num_kv_heads, num_blocks,
       scale_log2, geo.tokens, geo.max_slots, w.part_out, w.part_lse, out, lse, w.plan,
       w.plan_count, w.nslots, in_pass_merge ? w.merge_ctr : nullptr, pa);
    if ((st = launch_status()) != PKV_OK) return st;
  }
  if (geo.partials && !in_pass_merge) {
    combine_launch(s, out, lse, w.part_out, w.part_lse, context_lens, w.nslots, batch, cap,
                   num_q_heads, head_dim, geo.tokens, geo.max_slots, 1);
    st = launch_status();
  }
  return st;
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" size_t pkv_decode_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                             int32_t head_dim, int32_t max_context_len,
                                             int32_t partition_size) {
  if (batch <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0) return 0;
  return workspace_layout(nullptr, batch, num_q_heads, head_dim,
                          decode_geometry(max_context_len, partition_size, false))
      .bytes;
}

extern "C" int32_t pkv_decode_partition_size(int32_t batch, int32_t num_kv_heads,
                                             int32_t head_dim, int32_t max_context_len,
                                             int64_t total_context_tokens) {
  if (batch <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_context_len <= 512) return 0;
  // One unit per (sequence, KV head) already gives two workgroups per compute unit.
  if (static_cast<int64_t>(batch) * num_kv_heads >= 512) return 0;
  const int64_t total = total_context_tokens > 0
                            ? total_context_tokens
                            : static_cast<int64_t>(batch) * max_context_len;
  // The pass's bytes spread over about one unit per compute unit, counted in tokens of a
  // 128-dim head: a power of two in [256, 8192].
  const int64_t share = total * num_kv_heads * head_dim / (256 * 128);
  int32_t P = 256;
  while (P < 8192 && 2 * static_cast<int64_t>(P) <= share) P *= 2;
  // Few enough partitions to merge inside the pass, if that costs at most one doubling.
  const int32_t per_merge = (max_context_len + kMaxInPassMergeSlots - 1) / kMaxInPassMergeSlots;
  int32_t merge_p = kBlockTokens;
  while (merge_p < per_merge) merge_p *= 2;
  if (merge_p <= 2 * P) P = min(max(P, merge_p), 8192);
  return P >= max_context_len ? 0 : P;
}

extern "C" int32_t pkv_decode_engine(int32_t dtype, int32_t head_dim, int32_t num_q_heads,
                                     int32_t num_kv_heads) {
  if (dtype != PKV_F32 && dtype != PKV_BF16) return PKV_ERR_DTYPE;
  if ((head_dim != 64 && head_dim != 128) || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || num_q_heads / num_kv_heads > 8)
    return PKV_ERR_SHAPE;
  const int G = num_q_heads / num_kv_heads;
  const bool tile = dtype == PKV_BF16 &&
                    (head_dim == 64 ? pkv::mfma_pass<uint16_t, 64>(G) : pkv::mfma_pass<uint16_t, 128>(G));
  return tile ? PKV_ENGINE_MATRIX : PKV_ENGINE_VALU;
}

extern "C" size_t pkv_shared_prefix_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                                    int32_t head_dim, int32_t max_context_len,
                                                    int32_t partition_size) {
  if (batch <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0) return 0;
  return workspace_layout(nullptr, batch, num_q_heads, head_dim,
                          decode_geometry(max_context_len, partition_size, true))
      .bytes;
}

extern "C" int pkv_decode_plan(void* workspace, size_t workspace_bytes,
                               const int32_t* context_lens, int64_t bt_stride, int32_t batch,
                               int32_t num_q_heads, int32_t head_dim, int32_t max_context_len,
                               int32_t partition_size, pkv_stream_t stream) {
  if (!workspace || !context_lens) return PKV_ERR_NULL;
  if (batch < 0 || num_q_heads <= 0 || (head_dim != 64 && head_dim != 128) ||
      max_context_len < 0 || partition_size < 0 || partition_size % kBlockTokens != 0 ||
      bt_stride <= 0 || bt_stride > (1 << 26))
    return PKV_ERR_SHAPE;
  if (batch == 0) return PKV_OK;
  if (workspace_bytes <
      pkv_decode_workspace_bytes(batch, num_q_heads, head_dim, max_context_len, partition_size))
    return PKV_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return PKV_ERR_ARG;
  const Geometry geo = decode_geometry(max_context_len, partition_size, false);
  const Workspace w = workspace_layout(workspace, batch, num_q_heads, head_dim, geo);
  const PlanInput in = plan_input(context_lens, batch, static_cast<int>(bt_stride) * kBlockTokens,
                                  geo, max_context_len, nullptr, nullptr, 0, 0, w.merge_ctr,
                                  geo.partials ? batch * num_q_heads : 0);
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0,
                     static_cast<hipStream_t>(stream), w.plan, w.plan_count, w.nslots, in);
  return launch_status();
}

extern "C" int pkv_paged_decode(float* out, float* lse, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* block_tables,
                                int64_t bt_stride, const int32_t* context_lens, int32_t batch,
                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, int32_t num_blocks, int32_t max_context_len,
                                float scale, int32_t partition_size, void* workspace,
                                size_t workspace_bytes, int32_t dtype, pkv_stream_t stream) {
  return decode_impl(true, out, lse, q, k_cache, v_cache, block_tables, bt_stride, context_lens,
                     batch, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_context_len, scale, partition_size, workspace, workspace_bytes, dtype,
                     stream);
}

extern "C" int pkv_paged_decode_planned(float* out, float* lse, const void* q,
                                        const void* k_cache, const void* v_cache,
                                        const int32_t* block_tables, int64_t bt_stride,
                                        const int32_t* context_lens, int32_t batch,
                                        int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                        int32_t max_context_len, float scale,
                                        int32_t partition_size, void* workspace,
                                        size_t workspace_bytes, int32_t dtype,
                                        pkv_stream_t stream) {
  return decode_impl(false, out, lse, q, k_cache, v_cache, block_tables, bt_stride,
                     context_lens, batch, num_q_heads, num_kv_heads, head_dim, block_size,
                     num_blocks, max_context_len, scale, partition_size, workspace,
                     workspace_bytes, dtype, stream);
}

namespace {
// Validates and packs the append arguments of the append-and-decode entry points.
int make_append(const void* k_new, const void* v_new, const int32_t* start_pos,
                const int32_t* cu_new_tokens, int32_t total_new, AppendArgs* a) {
  if (total_new < 0) return PKV_ERR_SHAPE;
  if (total_new > 0) {
    if (!k_new || !v_new || !start_pos || !cu_new_tokens) return PKV_ERR_NULL;
    if (!aligned16(k_new) || !aligned16(v_new)) return PKV_ERR_ARG;
    a->k_new = k_new;
    a->v_new = v_new;
    a->start_pos = start_pos;
    a->cu = cu_new_tokens;
    a->total = total_new;
  }
  return PKV_OK;
}

int make_groups(const int32_t* group_starts, const int32_t* group_shared_blocks,
                int32_t num_groups, int32_t max_shared_blocks, int32_t batch, Groups* g) {
  if (num_groups < 0 || max_shared_blocks < 0 || num_groups > batch) return PKV_ERR_SHAPE;
  if (batch > 0 && (!group_starts || !group_shared_blocks)) return PKV_ERR_NULL;
  g->starts = group_starts;
  g->shared_blocks = group_shared_blocks;
  g->count = num_groups;
  g->max_shared_blocks = max_shared_blocks;
  return PKV_OK;
}
}  // namespace

extern "C" int pkv_append_paged_decode(
    float* out, float* lse, const void* q, void* k_cache, void* v_cache, const void* k_new,
    const void* v_new, const int32_t* block_tables, int64_t bt_stride, const int32_t* start_pos,
    const int32_t* cu_new_tokens, int32_t total_new, const int32_t* context_lens, int32_t batch,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_context_len, float scale, int32_t partition_size,
    void* workspace, size_t workspace_bytes, int32_t dtype, pkv_stream_t stream) {
  AppendArgs a;
  const int st = make_append(k_new, v_new, start_pos, cu_new_tokens, total_new, &a);
  if (st != PKV_OK) return st;
  return decode_impl(true, out, lse, q, k_cache, v_cache, block_tables, bt_stride, context_lens,
                     batch, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_context_len, scale, partition_size, workspace, workspace_bytes, dtype,
                     stream, &a);
}

extern "C" int pkv_append_paged_decode_planned(
    float* out, float* lse, const void* q, void* k_cache, void* v_cache, const void* k_new,
    const void* v_new, const int32_t* block_tables, int64_t bt_stride, const int32_t* start_pos,
    const int32_t* cu_new_tokens, int32_t total_new, const int32_t* context_lens, int32_t batch,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_context_len, float scale, int32_t partition_size,
    void* workspace, size_t workspace_bytes, int32_t dtype, pkv_stream_t stream) {
  AppendArgs a;
  const int st = make_append(k_new, v_new, start_pos, cu_new_tokens, total_new, &a);
  if (st != PKV_OK) return st;
  return decode_impl(false, out, lse, q, k_cache, v_cache, block_tables, bt_stride,
                     context_lens, batch, num_q_heads, num_kv_heads, head_dim, block_size,
                     num_blocks, max_context_len, scale, partition_size, workspace,
                     workspace_bytes, dtype, stream, &a, nullptr, true);
}

extern "C" int pkv_paged_decode_shared_prefix(
    float* out, float* lse, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, int64_t bt_stride, const int32_t* context_lens,
    const int32_t* group_starts, const int32_t* group_shared_blocks, int32_t num_groups,
    int32_t max_shared_blocks, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_context_len,
    float scale, int32_t partition_size, void* workspace, size_t workspace_bytes, int32_t dtype,
    pkv_stream_t stream) {
  Groups g;
  const int st =
      make_groups(group_starts, group_shared_blocks, num_groups, max_shared_blocks, batch, &g);
  if (st != PKV_OK) return st;
  return decode_impl(true, out, lse, q, k_cache, v_cache, block_tables, bt_stride, context_lens,
                     batch, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_context_len, scale, partition_size, workspace, workspace_bytes, dtype,
                     stream, nullptr, &g);
}

extern "C" int pkv_append_paged_decode_shared_prefix(
    float* out, float* lse, const void* q, void* k_cache, void* v_cache, const void* k_new,
    const void* v_new, const int32_t* block_tables, int64_t bt_stride, const int32_t* start_pos,
    const int32_t* cu_new_tokens, int32_t total_new, const int32_t* context_lens,
    const int32_t* group_starts, const int32_t* group_shared_blocks, int32_t num_groups,
    int32_t max_shared_blocks, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_context_len,
    float scale, int32_t partition_size, void* workspace, size_t workspace_bytes, int32_t dtype,
    pkv_stream_t stream) {
  AppendArgs a;
  Groups g;
  int st = make_append(k_new, v_new, start_pos, cu_new_tokens, total_new, &a);
  if (st != PKV_OK) return st;
  st = make_groups(group_starts, group_shared_blocks, num_groups, max_shared_blocks, batch, &g);
  if (st != PKV_OK) return st;
  return decode_impl(true, out, lse, q, k_cache, v_cache, block_tables, bt_stride, context_lens,
                     batch, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_context_len, scale, partition_size, workspace, workspace_bytes, dtype,
                     stream, &a, &g);
}

extern "C" int pkv_paged_decode_partials(float* part_out, float* part_lse, const void* q,
                                         const void* k_cache, const void* v_cache,
                                         const int32_t* block_tables, int64_t bt_stride,
                                         const int32_t* context_lens, int32_t batch,
                                         int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t block_size,
                                         int32_t num_blocks, int32_t max_context_len,
                                         float scale, int32_t partition_size,
                                         int32_t max_partitions, const void* plan_workspace,
                                         int32_t dtype, pkv_stream_t stream) {
  LaunchFn fn = nullptr;
  int st = check_decode_args(q, k_cache, v_cache, block_tables, bt_stride, context_lens, batch,
                             num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                             max_context_len, partition_size, dtype, &fn);
  if (st != PKV_OK) return st;
  if (!part_out || !part_lse) return PKV_ERR_NULL;
  if (partition_size <= 0) return PKV_ERR_SHAPE;
  const int np = num_partitions(max_context_len, partition_size);
  if (max_partitions < np) return PKV_ERR_SHAPE;
  if (batch == 0) return PKV_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int4* plan = nullptr;
  const int* plan_count = nullptr;
  int order = kOrderPartMajorReversed;
  int grid_slots = np;
  if (plan_workspace != nullptr) {
    // A plan from pkv_decode_plan for the same lengths and partition size: its units
    // are exactly the partitions (a single-partition plan covers whole sequences, which
    // is the same range).
    if ((reinterpret_cast<uintptr_t>(plan_workspace) & (kAlign - 1)) != 0) return PKV_ERR_ARG;
    const Geometry geo = decode_geometry(max_context_len, partition_size, false);
    const Workspace w = workspace_layout(const_cast<void*>(plan_workspace), batch, num_q_heads,
                                         head_dim, geo);
    plan = w.plan;
    plan_count = w.plan_count;
    order = kOrderPlanned;
    grid_slots = geo.max_slots;
  }
  fn(order, grid_slots, num_kv_heads, batch, s, q, k_cache, v_cache, block_tables,
     static_cast<int>(bt_stride), context_lens, num_q_heads, num_kv_heads, num_blocks,
     scale_to_log2(scale), partition_size, max_partitions, part_out, part_lse, nullptr, nullptr,
     plan, plan_count, nullptr, nullptr, PassAppend{nullptr, nullptr, nullptr, nullptr, 0});
  return launch_status();
}

extern "C" int pkv_lse_combine(float* out, float* lse, const float* part_out,
                               const float* part_lse, const int32_t* context_lens, int32_t batch,
                               int32_t num_q_heads, int32_t head_dim, int32_t partition_size,
                               int32_t max_partitions, pkv_stream_t stream) {
  if (!out || !part_out || !part_lse || !context_lens) return PKV_ERR_NULL;
  if (batch < 0 || num_q_heads <= 0 || (head_dim != 64 && head_dim != 128) ||
      partition_size <= 0 || max_partitions <= 0)
    return PKV_ERR_SHAPE;
  if (batch == 0) return PKV_OK;
  // Lengths above max_partitions * partition_size are clamped to it.
  const int64_t cap64 = static_cast<int64_t>(max_partitions) * partition_size;
  const int cap = cap64 > (1 << 30) ? (1 << 30) : static_cast<int>(cap64);
  combine_launch(static_cast<hipStream_t>(stream), out, lse, part_out, part_lse, context_lens,
                 nullptr, batch, cap, num_q_heads, head_dim, partition_size, max_partitions, 0);
  return launch_status();
}
