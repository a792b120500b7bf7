// Paged (chunked) prefill attention for gfx950.
//
// What is computed (spindle, "Why write the forward pass" and "Two bugs worth
// recording"): a sequence's new chunk of q_len query tokens, already appended to the
// block cache, attends causally over the sequence's context of n tokens (the chunk
// included): query i sits at position n - q_len + i and attends to tokens [0, that
// position], through the block table, with explicit lengths.
//
// bf16 caches: matrix-core row tiles of 16 (token, query head) rows of one sequence for
// one KV head, each row with its own causal limit; a workgroup's four waves take
// consecutive tiles and share every K/V block through LDS.  fp32 caches: the VALU
// routine of the decode, one wave per query token.

#include "common.h"

PKV_DEFINE_ERROR_WORD(prefill)

#include "mfma_tile.h"
#include "valu_attend.h"

namespace pkv {
namespace {

// The chunk of sequence s: rows [r0, r0 + len) of q/out, positions [n - len, n).  A
// malformed chunk (negative length, rows past total_q, longer than the context or the
// table) sets an error bit and is cut to what can be attended safely.
struct Chunk {
  int r0, len, n;
};

__device__ __forceinline__ Chunk chunk_of(const int32_t* __restrict__ cu_q,
                                          const int32_t* __restrict__ ctx_lens, int s,
                                          int total_q, int max_q_len, int cap, bool report) {
  Chunk c;
  c.r0 = cu_q[s];
  int r1 = cu_q[s + 1];
  int n = ctx_lens[s];
  bool bad_cu = c.r0 < 0 || r1 < c.r0 || r1 > total_q;
  bool bad_ctx = n < 0 || n > cap;
  if (bad_cu) {
    c.r0 = 0;
    r1 = 0;
  }
  n = n < 0 ? 0 : min(n, cap);
  if (r1 - c.r0 > n) {
    bad_ctx = true;
    r1 = c.r0 + n;
  }
  if (report && bad_cu) PKV_FLAG_ERROR(PKV_DEVERR_CU);
  if (report && bad_ctx) PKV_FLAG_ERROR(PKV_DEVERR_CONTEXT);
  // the grid covers max_q_len tokens per sequence, counted from the chunk's end
  if (report && r1 - c.r0 > max_q_len) PKV_FLAG_ERROR(PKV_DEVERR_MAX_CONTEXT);
  c.len = r1 - c.r0;
  c.n = n;
  return c;
}

// bf16, LDS-staged: a workgroup of four waves takes kR row tiles per wave, i.e.
// 4 * kR * (16 / G) consecutive query tokens of one sequence for one KV head.  Each block
// of the causal range is loaded once per workgroup (every thread fetches 16 bytes of K
// and of V, so the loads in flight cost few registers), stored to LDS with rows padded by
// 32 bytes (both operand reads and the stores then touch distinct banks), and read by
// every wave for all its row tiles: one block load serves 64 * kR rows.  Three LDS stages
// and three register sets: a block's loads are issued two blocks before it is stored, the
// next block is stored while the current one is read, one barrier per block.
constexpr int kLdsWaves = 4;
constexpr int kLdsThreads = kLdsWaves * kWave;

template <int D>
struct LdsStage {
  // K rows: 32-byte pad per token row.  With a 16-byte pad the K operand reads (16 bytes
  // per lane, rows c = 0..15) conflicted on the banks: 37 M conflict cycles per call of
  // the 16 x 512-token chunked prefill, 0 with this pad, and the call ran 2-3% faster.
  static constexpr int kRowElems = D + 16;
  static constexpr int kVRowElems = D + 16;  // V rows: 32-byte pad (the transpose reads below
                                             // then touch each bank window once per pass)
  alignas(16) uint16_t k[kBlockTokens * kRowElems];
  alignas(16) uint16_t v[kBlockTokens * kVRowElems];
};

template <int D>
struct StageRegs {
  static constexpr int kChunks = 2 * kBlockTokens * D / 8;  // 16-byte chunks of K and V
  static constexpr int kPerThread = (kChunks + kLdsThreads - 1) / kLdsThreads;
  u32x4_t w[kPerThread];
};

// Chunk i of a block: i < 2D covers K (token i / (D/8), dims 8 * (i % (D/8)) ..), the rest V.
template <int D>
__device__ __forceinline__ void stage_load(StageRegs<D>& r, const uint16_t* __restrict__ kt,
                                           const uint16_t* __restrict__ vt, int tid) {
  constexpr int kHalf = StageRegs<D>::kChunks / 2;
#pragma unroll
  for (int j = 0; j < StageRegs<D>::kPerThread; ++j) {
    const int i = tid + j * kLdsThreads;
    const uint16_t* src = i < kHalf ? kt + i * 8 : vt + (i - kHalf) * 8;
    r.w[j] = *reinterpret_cast<const u32x4_t*>(src);
  }
}

template <int D>
__device__ __forceinline__ void stage_store(LdsStage<D>& st, const StageRegs<D>& r, int tid) {
  constexpr int kHalf = StageRegs<D>::kChunks / 2;
  constexpr int kRowChunks = D / 8;
#pragma unroll
  for (int j = 0; j < StageRegs<D>::kPerThread; ++j) {
    const int i = tid + j * kLdsThreads;
    const int ii = i < kHalf ? i : i - kHalf;
    uint16_t* dst = (i < kHalf ? st.k : st.v) +
                    (ii / kRowChunks) * (i < kHalf ? LdsStage<D>::kRowElems
                                                   : LdsStage<D>::kVRowElems) +
                    (ii % kRowChunks) * 8;
    *reinterpret_cast<u32x4_t*>(dst) = r.w[j];
  }
}

// The lane's MFMA operands of a staged block.  K as in mfma_load_block.  V through the
// gfx950 LDS transpose read: within each 16-lane group, ds_read_b64_tr_b16 gives lane i
// element i % 4 of the 8-byte chunks addressed by lanes i / 4 + 4k (k = 0..3), so lane
// (c, h) addressing V[4h + c / 4][16j + 4 (c % 4)] receives V[4h .. 4h + 3][16j + c]: the
// B operand of output tile j (dims 16j .. 16j + 15, lane c holding dim 16j + c), with no
// repacking on the VALU.
typedef short v4i16_t __attribute__((ext_vector_type(4)));

template <int D>
struct TrBlock {
  u32x4_t k[MfmaGeom<D>::kQkSteps];
  u32x2_t vt[MfmaGeom<D>::kTiles];  // tile j: V[4h .. 4h + 3][16j + c], two tokens a word
};

template <int D>
__device__ __forceinline__ void stage_read_tr(TrBlock<D>& b, const LdsStage<D>& st, int c,
                                              int h) {
  using Mg = MfmaGeom<D>;
  constexpr int RS = LdsStage<D>::kRowElems;
  constexpr int RV = LdsStage<D>::kVRowElems;
#pragma unroll
  for (int k = 0; k < Mg::kQkSteps; ++k)
    b.k[k] = *reinterpret_cast<const u32x4_t*>(st.k + c * RS + 32 * k + 8 * h);
  const uint16_t* vrow = st.v + (4 * h + c / 4) * RV + 4 * (c % 4);
#pragma unroll
  for (int j = 0; j < Mg::kTiles; ++j) {
    const v4i16_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16_t*)(vrow + 16 * j));
    b.vt[j] = __builtin_bit_cast(u32x2_t, t);
  }
}

// One block for a wave's 16 rows on a transpose-read block: scores as in mfma_rows_block,
// then P rounded once to bf16 (round to nearest even, two values per v_cvt_pk_bf16_f32) as
// the A operand of a 16x16x16 product per output tile, whose B operand is the transposed
// V pair as read (output tile j holds dims 16j + c).  kMasked: some row's causal limit or
// the chunk's end falls inside the block, so scores are masked per row; blocks below every
// row's limit skip the compares.
typedef short v4i16_t2 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t2 __attribute__((ext_vector_type(2)));

template <int D>
__device__ __forceinline__ void tr_rows_block(MfmaRows<D>& r, TrBlock<D>& cur,
                                              const u32x4_t (&qr)[MfmaGeom<D>::kQkSteps],
                                              int t_base, int n_c, int n_max, int h,
                                              float scale_log2, bool masked) {
  using Mg = MfmaGeom<D>;
  f32x4_t sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < Mg::kQkSteps; ++s)
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, cur.k[s]),
                                                 __builtin_bit_cast(bf16x8_t, qr[s]), sc, 0, 0,
                                                 0);
  float x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = sc[i] * scale_log2;
  if (masked) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (t_base + 4 * h + i < n_c) ? x[i] : -INFINITY;
  }
  float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  bm = max_xor32(max_xor16(bm));
  const bool raise = bm > r.m_c + kLazyMaxSlack;
  if (__any(raise)) {
    float a = 1.0f;
    if (raise) {
      a = r.m_c == -INFINITY ? 0.0f : fast_exp2(r.m_c - bm);
      r.m_c = bm;
    }
    r.l_part *= a;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ai = __shfl(a, 4 * h + i);
#pragma unroll
      for (int j = 0; j < Mg::kTiles; ++j) r.o[j][i] *= ai;
    }
  }
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // No select for masked scores: exp2(-inf - m) is 0 once m is finite, and every live
    // row's m is finite from block 0 on (block 0 comes first and holds token 0, which every
    // causal row attends).  Rows past the chunk's last token keep m = -inf and turn NaN;
    // matrix-core rows are independent and those rows are never written.
    p[i] = fast_exp2(x[i] - r.m_c);
    r.l_part += p[i];
  }
  bf16x2_t2 p01, p23;
  p01[0] = static_cast<__bf16>(p[0]);
  p01[1] = static_cast<__bf16>(p[1]);
  p23[0] = static_cast<__bf16>(p[2]);
  p23[1] = static_cast<__bf16>(p[3]);
  const v4i16_t2 a = __builtin_bit_cast(
      v4i16_t2, u32x2_t{__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23)});
  // Tokens past every taken row's end hold stale data: zero their V (0 * NaN); word 0 holds
  // tokens 4h, 4h + 1 (low, high half), word 1 tokens 4h + 2, 4h + 3.
  if (t_base + kBlockTokens > n_max) {
    const int t0 = t_base + 4 * h;
    const uint32_t m0 = (t0 < n_max ? 0x0000ffffu : 0u) | (t0 + 1 < n_max ? 0xffff0000u : 0u);
    const uint32_t m1 = (t0 + 2 < n_max ? 0x0000ffffu : 0u) | (t0 + 3 < n_max ? 0xffff0000u : 0u);
#pragma unroll
    for (int j = 0; j < Mg::kTiles; ++j) {
      cur.vt[j][0] &= m0;
      cur.vt[j][1] &= m1;
    }
  }
#pragma unroll
  for (int j = 0; j < Mg::kTiles; ++j)
    r.o[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, __builtin_bit_cast(v4i16_t2, cur.vt[j]),
                                                       r.o[j], 0, 0, 0);
}

// Row tiles per wave of the bf16 prefill (each LDS read of a block serves kR tiles), and
// workgroups per compute unit the register allocation is held to.
#ifndef PKV_PREFILL_ROW_TILES
#define PKV_PREFILL_ROW_TILES 1
#endif
constexpr int kPrefillRowTiles = PKV_PREFILL_ROW_TILES;

template <int D, int G, int kR>
__global__ __launch_bounds__(kLdsThreads, kR == 1 ? 4 : 2) void prefill_lds_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ tables, int W,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ ctx_lens, int total_q,
    int max_q_len, int num_q_heads, int num_kv_heads, int num_blocks, float scale_log2,
    float* __restrict__ out, float* __restrict__ lse) {
  using Mg = MfmaGeom<D>;
  constexpr int kMembers = kMfmaRows / G;  // query tokens per row tile
  constexpr int kRows = kMembers * G;
  constexpr int kGroupTokens = kMembers * kR * kLdsWaves;
  __shared__ LdsStage<D> stage[3];
  __shared__ int s_ids[kLdsThreads];
  const int s = blockIdx.y;
  const int kvh = blockIdx.z;
  const int tid = threadIdx.x;
  const bool first = blockIdx.x == 0 && kvh == 0 && tid == 0;
  const Chunk ch = chunk_of(cu_q, ctx_lens, s, total_q, max_q_len, W * kBlockTokens, first);
  const int groups = (ch.len + kGroupTokens - 1) / kGroupTokens;
  if (static_cast<int>(blockIdx.x) >= groups) return;  // whole workgroup: uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int c = lane % 16;
  const int h = lane / 16;
  const int tg = (groups - 1 - static_cast<int>(blockIdx.x)) * kGroupTokens;  // group's first
  const int pos_g = ch.n - ch.len + tg;
  // The group's causal range ends at its last live token.
  const int g_members = min(kGroupTokens, ch.len - tg);
  const int n_group = pos_g + g_members;
  const int nblk = (n_group + kBlockTokens - 1) / kBlockTokens;

  // This wave's row tiles: tokens tg + (wave * kR + r) * kMembers + c / G.
  int n_c[kR], members[kR], tile_end[kR];
  int tile_lim0[kR];  // the smallest causal limit of the tile's rows (its first token's)
  int n_wave = 0;
  u32x4_t qr[kR][Mg::kQkSteps];
  MfmaRows<D> rows[kR];
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const int t0 = tg + (wave * kR + r) * kMembers;
    members[r] = max(0, min(kMembers, ch.len - t0));
    const int pos0 = ch.n - ch.len + t0;
    const bool live = c < kRows && c / G < members[r];
    n_c[r] = live ? pos0 + c / G + 1 : 0;
    tile_end[r] = members[r] > 0 ? pos0 + members[r] : 0;
    tile_lim0[r] = pos0 + 1;
    n_wave = max(n_wave, tile_end[r]);
#pragma unroll
    for (int k = 0; k < Mg::kQkSteps; ++k) qr[r][k] = u32x4_t{0u, 0u, 0u, 0u};
    if (live) {
      const uint16_t* qrow = q + (static_cast<size_t>(ch.r0 + t0 + c / G) * num_q_heads +
                                  kvh * G + c % G) * D + 8 * h;
#pragma unroll
      for (int k = 0; k < Mg::kQkSteps; ++k)
        qr[r][k] = *reinterpret_cast<const u32x4_t*>(qrow + 32 * k);
    }
    mfma_rows_init<D>(rows[r]);
  }
  // The query loads above are conditional; without this wait the compiler cannot prove
  // them complete at the block loop's head and waits for every outstanding load (the
  // staged blocks' too) before each block's first matrix product.
  __builtin_amdgcn_s_waitcnt(0);

  const size_t head_elems = static_cast<size_t>(kBlockTokens) * D;
  const size_t block_elems = static_cast<size_t>(num_kv_heads) * head_elems;
  const int32_t* trow = tables + static_cast<size_t>(s) * W;
  // Block ids, a window of kLdsThreads at a time (one per thread), in LDS.  Each window
  // is streamed on its own, so the block loop itself holds no table read.
  auto block_ptr = [&](int id, const uint16_t* base) {
    return base + static_cast<size_t>(id) * block_elems + kvh * head_elems;
  };
  auto fetch_ids = [&](int from) {
    const int k = from + tid;
    const int id = k < nblk ? trow[k] : 0;
    const bool bad = static_cast<unsigned>(id) >= static_cast<unsigned>(num_blocks);
    if (__any(bad) && lane == 0) PKV_FLAG_ERROR(PKV_DEVERR_BLOCK_ID);
    s_ids[tid] = bad ? 0 : id;
  };
  auto compute = [&](const LdsStage<D>& st, int b) {
    const int t_base = b * kBlockTokens;
    if (t_base >= n_wave) return;  // past every row of this wave (causal): nothing to add
    TrBlock<D> cur;
    stage_read_tr<D>(cur, st, c, h);
#pragma unroll
    for (int r = 0; r < kR; ++r)
      if (t_base < tile_end[r])
        tr_rows_block<D>(rows[r], cur, qr[r], t_base, n_c[r], n_wave, h, scale_log2,
                         t_base + kBlockTokens > tile_lim0[r]);
  };

  // Three LDS stages, three register sets: the loads of block j are issued two blocks
  // before it is stored to LDS (block j lives in stage (j - w0) % 3).  Past the window's
  // last block that block is loaded and stored again (a cache hit, never read): every
  // load and store of the loop is then unconditional, so the compiler's wait before a
  // stage store counts only the loads that filled it, not the ones issued after.
  StageRegs<D> r0, r1, r2;
  for (int w0 = 0; w0 < nblk; w0 += kLdsThreads) {
    const int w1 = min(nblk, w0 + kLdsThreads);
    __syncthreads();  // the previous window's ids and stages are no longer read
    fetch_ids(w0);
    __syncthreads();
    auto issue = [&](int j, StageRegs<D>& r) {
      // uniform: the block's base address is computed on the scalar unit
      const int id = __builtin_amdgcn_readfirstlane(s_ids[min(j, w1 - 1) - w0]);
      stage_load<D>(r, block_ptr(id, kc), block_ptr(id, vc), tid);
    };
    issue(w0, r0);
    issue(w0 + 1, r1);
    issue(w0 + 2, r2);
    stage_store<D>(stage[0], r0, tid);
    __syncthreads();
    for (int b = w0; b < w1; b += 3) {
      // stage[0] holds block b; r1, r2 hold blocks b + 1, b + 2 in flight
      issue(b + 3, r0);
      compute(stage[0], b);
      stage_store<D>(stage[1], r1, tid);
      __syncthreads();
      if (b + 1 >= w1) break;
      issue(b + 4, r1);
      compute(stage[1], b + 1);
      stage_store<D>(stage[2], r2, tid);
      __syncthreads();
      if (b + 2 >= w1) break;
      issue(b + 5, r2);
      compute(stage[2], b + 2);
      stage_store<D>(stage[0], r0, tid);
      __syncthreads();
    }
  }

  // Row c's totals live on the four lanes with lane % 16 == c; output row 4h + i's on
  // lane (c, h), dims 16j + c.  Each output row takes its max and sum from a lane owning its score row.
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    float l_c = rows[r].l_part;
        l_c = sum_xor32(sum_xor16(l_c));
    const int t0 = tg + (wave * kR + r) * kMembers;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 4 * h + i;
      const float L = __shfl(l_c, rr);
      const float M = __shfl(rows[r].m_c, rr);
      if (rr >= kRows || rr / G >= members[r]) continue;
      const float inv = L > 0.0f ? 1.0f / L : 0.0f;
      const size_t sh =
          static_cast<size_t>(ch.r0 + t0 + rr / G) * num_q_heads + kvh * G + rr % G;
      // output tile j holds dims 16j + c: each store writes 16 consecutive floats of a row
      float* dst = out + sh * D + c;
#pragma unroll
      for (int j = 0; j < Mg::kTiles; ++j) dst[16 * j] = rows[r].o[j][i] * inv;
      if (c == 0 && lse != nullptr) lse[sh] = L > 0.0f ? (M + __log2f(L)) * kLn2 : -INFINITY;
    }
  }
}

constexpr int kPrefillWaves = 4;

// One wave per query token (fp32 caches): the decode's VALU routine over [0, position].
template <typename T, int D, int G>
__global__ __launch_bounds__(kPrefillWaves * kWave) void prefill_valu_kernel(
    const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc,
    const int32_t* __restrict__ tables, int W, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ ctx_lens, int total_q, int max_q_len, int num_q_heads,
    int num_kv_heads, int num_blocks, float scale_log2, float* __restrict__ out,
    float* __restrict__ lse) {
  using Gm = Geom<T, D>;
  const int s = blockIdx.y;
  const int kvh = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const bool first = blockIdx.x == 0 && kvh == 0 && threadIdx.x == 0;
  const Chunk c = chunk_of(cu_q, ctx_lens, s, total_q, max_q_len, W * kBlockTokens, first);
  const int groups = (c.len + kPrefillWaves - 1) / kPrefillWaves;
  if (static_cast<int>(blockIdx.x) >= groups) return;
  const int t = (groups - 1 - static_cast<int>(blockIdx.x)) * kPrefillWaves + wave;
  if (t >= c.len) return;
  const int row = c.r0 + t;
  GroupState<T, D, G> st;
  attend_range<T, D, G, 1, false>(st, q, kc, vc, tables, W, s, row, kvh, num_q_heads,
                                     num_kv_heads, num_blocks, scale_log2, 0,
                                     c.n - c.len + t + 1, 0, lane);
  const int grp = lane / kLanesPerToken;
  const int sub = lane % kLanesPerToken;
  if (grp != 0) return;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float L = st.l[g];
    const size_t sh = static_cast<size_t>(row) * num_q_heads + kvh * G + g;
    float* dst = out + sh * D;
#pragma unroll
    for (int e = 0; e < Gm::kElems; e += 4) {
      float4 v;
      v.x = L > 0.0f ? st.acc[g][e + 0] / L : 0.0f;
      v.y = L > 0.0f ? st.acc[g][e + 1] / L : 0.0f;
      v.z = L > 0.0f ? st.acc[g][e + 2] / L : 0.0f;
      v.w = L > 0.0f ? st.acc[g][e + 3] / L : 0.0f;
      *reinterpret_cast<float4*>(dst + lane_dim<T, D>(sub, e)) = v;
    }
    if (sub == 0 && lse != nullptr)
      lse[sh] = L > 0.0f ? (st.m[g] + __log2f(L)) * kLn2 : -INFINITY;
  }
}

struct PrefillArgs {
  float* out;
  float* lse;
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* tables;
  int W;
  const int32_t* cu_q;
  const int32_t* ctx;
  int batch, total_q, max_q_len, hq, hkv, nb;
  float scale_log2;
};

template <typename T, int D, int G>
void prefill_launch(const PrefillArgs& a, hipStream_t stream) {
  if constexpr (sizeof(T) == 2) {
    constexpr int kR = kPrefillRowTiles;
    constexpr int kGroupTokens = kMfmaRows / G * kR * kLdsWaves;
    const dim3 grid((a.max_q_len + kGroupTokens - 1) / kGroupTokens, a.batch, a.hkv);
    hipLaunchKernelGGL((prefill_lds_kernel<D, G, kR>), grid, dim3(kLdsThreads), 0, stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.kc),
                       static_cast<const uint16_t*>(a.vc), a.tables, a.W, a.cu_q, a.ctx,
                       a.total_q, a.max_q_len, a.hq, a.hkv, a.nb, a.scale_log2, a.out, a.lse);
  } else {
    const dim3 grid((a.max_q_len + kPrefillWaves - 1) / kPrefillWaves, a.batch, a.hkv);
    hipLaunchKernelGGL((prefill_valu_kernel<T, D, G>), grid, dim3(kPrefillWaves * kWave), 0,
                       stream, static_cast<const T*>(a.q), static_cast<const T*>(a.kc),
                       static_cast<const T*>(a.vc), a.tables, a.W, a.cu_q, a.ctx, a.total_q,
                       a.max_q_len, a.hq, a.hkv, a.nb, a.scale_log2, a.out, a.lse);
  }
}

using PrefillFn = void (*)(const PrefillArgs&, hipStream_t);

template <typename T, int D>
PrefillFn pick_prefill(int G) {
  switch (G) {
    case 1: return prefill_launch<T, D, 1>;
    case 2: return prefill_launch<T, D, 2>;
    case 3: return prefill_launch<T, D, 3>;
    case 4: return prefill_launch<T, D, 4>;
    case 5: return prefill_launch<T, D, 5>;
    case 6: return prefill_launch<T, D, 6>;
    case 7: return prefill_launch<T, D, 7>;
    case 8: return prefill_launch<T, D, 8>;
    default: return nullptr;
  }
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int pkv_paged_prefill(float* out, float* lse, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_tables,
                                 int64_t bt_stride, const int32_t* cu_q,
                                 const int32_t* context_lens, int32_t batch, int32_t total_q,
                                 int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                 float scale, int32_t dtype, pkv_stream_t stream) {
  if (!out || !q || !k_cache || !v_cache || !block_tables || !cu_q || !context_lens)
    return PKV_ERR_NULL;
  if (dtype != PKV_F32 && dtype != PKV_BF16) return PKV_ERR_DTYPE;
  if (batch < 0 || total_q < 0 || max_q_len < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || block_size != kBlockTokens || num_blocks <= 0 ||
      bt_stride <= 0 || bt_stride > (1 << 26) || (head_dim != 64 && head_dim != 128))
    return PKV_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return PKV_ERR_ARG;
  const int G = num_q_heads / num_kv_heads;
  PrefillFn fn = dtype == PKV_F32
                     ? (head_dim == 64 ? pick_prefill<float, 64>(G) : pick_prefill<float, 128>(G))
                     : (head_dim == 64 ? pick_prefill<uint16_t, 64>(G)
                                       : pick_prefill<uint16_t, 128>(G));
  if (fn == nullptr) return PKV_ERR_SHAPE;
  if (batch == 0 || total_q == 0 || max_q_len == 0) return PKV_OK;
  const PrefillArgs a{out, lse, q, k_cache, v_cache, block_tables, static_cast<int>(bt_stride),
                      cu_q, context_lens, batch, total_q, max_q_len, num_q_heads, num_kv_heads,
                      num_blocks, scale_to_log2(scale)};
  fn(a, static_cast<hipStream_t>(stream));
  return launch_status();
}
