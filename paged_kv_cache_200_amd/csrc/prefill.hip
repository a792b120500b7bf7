// Paged (chunked) prefill attention for gfx950.
//
// What is computed (spindle, "Why write the forward pass" and "Two bugs worth
// recording"): a sequence's new chunk of q_len query tokens, already appended to the
// block cache, attends causally over the sequence's context of n tokens (the chunk
// included): query i sits at position n - q_len + i and attends to tokens [0, that
// position], through the block table, with explicit lengths.
//
// bf16 caches: matrix-core tiles of 32 (token, query head) rows of one sequence for one
// KV head on the 32x32x16 shape, each row with its own causal limit; a workgroup's four
// waves take consecutive tiles and share every pair of K/V blocks through LDS, and all
// workgroups of one (sequence, KV head) run on one XCD so its blocks are reused from one
// L2.  fp32 caches: the VALU routine of the decode, one wave per query token.

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

// bf16: four waves per workgroup (kLdsThreads threads), each wave 32 (token, query head)
// rows of one sequence for one KV head, i.e. 4 * (32 / G) consecutive query tokens.  Each
// pair of cache blocks in the group's causal range is loaded once per workgroup into LDS
// and read by all four waves.
constexpr int kLdsWaves = 4;
constexpr int kLdsThreads = kLdsWaves * kWave;

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t2 __attribute__((ext_vector_type(2)));

// ---- 32-row tiles on the 32x32x16 matrix-core shape ----
//
// A wave owns 32 (token, query head) rows; each step takes 32 keys (two cache blocks).
// Scores are computed transposed, S^T = K Q^T: lane l holds row l % 32's scores for keys
// 8i + 4(l / 32) + j (i, j < 4), so every softmax statistic of a row lives on lanes l and
// l ^ 32.  The output is held transposed too, O^T = V^T P^T, so a lane's accumulators all
// belong to its row and a rescale is one multiply per accumulator.  The contraction runs
// over the keys in the order the score tile holds them: per 16-key step, lanes below 32
// take keys {0..3, 8..11}, the others {4..7, 12..15}; the V^T operand follows that order
// through two LDS transpose reads per product.
typedef float f32x16_t __attribute__((ext_vector_type(16)));
constexpr int kT32Rows = 32;
constexpr int kPairTokens = 2 * kBlockTokens;
constexpr int kXcds = 8;  // MI355X: eight accelerator complex dies

// LDS image of a staged pair: K rows then V rows, 32 tokens each.  K rows are padded by
// 16 bytes and V rows by 32; V row t sits at position vpos(t), the order 0, 4, 1, 5, 2, 6,
// 3, 7 within each 8 tokens, so the four consecutive rows one transpose read meets sit two
// positions apart.  With these pads neither the K operand reads nor the V transpose reads
// meet a bank conflict (shader counters on the 16 x 512-token chunked prefill: 0 conflict
// cycles, against 18.7 M with 32-byte K pads and 37 M with 32-byte pads and V in order).
template <int D>
struct PairLayout {
  static constexpr int kRowElems = D + 8;
  static constexpr int kVRowElems = D + 16;
  static constexpr int kVBase = kPairTokens * kRowElems;                // elements
  static constexpr int kStage = kPairTokens * (kRowElems + kVRowElems);  // per stage
  static constexpr int kPartChunks = kBlockTokens * D / 8;     // one block's K (or V) slice
  static constexpr int kPerThread = 4 * kPartChunks / kLdsThreads;
  static_assert(4 * kPartChunks % kLdsThreads == 0 && kLdsThreads % kPartChunks == 0,
                "a thread's chunks sit at one offset of every part they touch");
};
__device__ __forceinline__ int vpos(int row) {
  return (row & ~7) | ((row & 3) << 1) | ((row >> 2) & 1);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t2 v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

// The sequence of rank r when sequences are ordered by causal work, largest first (ties
// by index): a chunk of L tokens ending at context length n costs about L (2n - L + 1)
// key-query pairs.  Each workgroup ranks the (few) sequences itself in LDS; the ranks
// only order the launch, so a malformed length just misorders it.  Past kSortedBatch
// sequences the launch keeps sequence order.  Called by all threads of the workgroup.
constexpr int kSortedBatch = kLdsThreads;

__device__ __forceinline__ int sequence_by_work(int r, const int32_t* __restrict__ cu_q,
                                                const int32_t* __restrict__ ctx_lens, int batch,
                                                int total_q, int tid) {
  if (batch > kSortedBatch) return r;
  __shared__ long long s_work[kSortedBatch];
  __shared__ int s_seq;
  long long w = -1;
  if (tid < batch) {
    const long long len = max(0, min(cu_q[tid + 1], total_q) - max(cu_q[tid], 0));
    const long long n = max(ctx_lens[tid], 0);
    w = len * (2 * n - len + 1);
    s_work[tid] = w;
  }
  __syncthreads();
  if (tid < batch) {
    int rank = 0;
    for (int t = 0; t < batch; ++t) {
      const long long wt = s_work[t];
      rank += (wt > w || (wt == w && t < tid)) ? 1 : 0;
    }
    if (rank == r) s_seq = tid;
  }
  __syncthreads();
  return s_seq;
}

template <int D, int G>
__global__ __launch_bounds__(kLdsThreads, 3) void prefill_t32_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ tables, int W,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ ctx_lens, int total_q,
    int max_q_len, int num_q_heads, int num_kv_heads, int num_blocks, float scale_log2,
    float* __restrict__ out, float* __restrict__ lse, int batch) {
  using Ly = PairLayout<D>;
  constexpr int kSteps = D / 16;          // 32x32x16 products per score tile
  constexpr int kDimTiles = D / 32;       // output tiles of 32 dims
  constexpr int kMembers = kT32Rows / G;  // query tokens per wave
  constexpr int kRows = kMembers * G;
  constexpr int kGroupTokens = kMembers * kLdsWaves;
  constexpr int RS = Ly::kRowElems;
  constexpr int kRowChunks = D / 8;
  __shared__ alignas(16) uint16_t smem[2 * Ly::kStage];
  // Workgroups go to the eight XCDs round-robin in launch order (workgroup L to XCD
  // L % 8), each XCD with its own L2.  All row groups of one (sequence, KV head) unit are
  // placed on one XCD, so the unit's K/V blocks are fetched into one L2 and reused there:
  // unit u = 8j + x runs on XCD x as its j-th unit, groups consecutively (longest causal
  // range first).  Units are numbered sequence-major in order of causal work.
  const int n_groups = (max_q_len + kGroupTokens - 1) / kGroupTokens;
  const int wg = blockIdx.x;
  const int xk = wg / kXcds;
  const int unit = (xk / n_groups) * kXcds + wg % kXcds;
  const int gx = xk % n_groups;
  if (unit >= batch * num_kv_heads) return;  // padding of the last round: uniform
  const int tid = threadIdx.x;
  // Units in order of their sequence's causal work, largest first (up to kSortedBatch
  // sequences; sequence order past that), so the last workgroups an XCD starts are short.
  const int s = sequence_by_work(unit / num_kv_heads, cu_q, ctx_lens, batch, total_q, tid);
  const int kvh = unit % num_kv_heads;
  const bool first = gx == 0 && kvh == 0 && tid == 0;
  const Chunk ch = chunk_of(cu_q, ctx_lens, s, total_q, max_q_len, W * kBlockTokens, first);
  const int groups = (ch.len + kGroupTokens - 1) / kGroupTokens;
  if (gx >= groups) return;  // whole workgroup: uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int r = lane % 32;  // the lane's row
  const int h = lane / 32;  // which half of each 8-key run the lane holds
  const int tg = (groups - 1 - gx) * kGroupTokens;
  const int pos_g = ch.n - ch.len + tg;
  const int g_members = min(kGroupTokens, ch.len - tg);
  const int n_group = pos_g + g_members;
  const int nblk = (n_group + kBlockTokens - 1) / kBlockTokens;

  // This wave's rows: tokens t0 + r / G, heads r % G.
  const int t0 = tg + wave * kMembers;
  const int members = max(0, min(kMembers, ch.len - t0));
  const int pos0 = ch.n - ch.len + t0;
  const bool live = r < kRows && r / G < members;
  const int n_c = live ? pos0 + r / G + 1 : 0;
  const int n_wave = members > 0 ? pos0 + members : 0;
  const int lim0 = pos0 + 1;  // the smallest causal limit of the wave's rows
  u32x4_t qr[kSteps];
#pragma unroll
  for (int k = 0; k < kSteps; ++k) qr[k] = u32x4_t{0u, 0u, 0u, 0u};
  if (live) {
    const uint16_t* qrow =
        q + (static_cast<size_t>(ch.r0 + t0 + r / G) * num_q_heads + kvh * G + r % G) * D + 8 * h;
#pragma unroll
    for (int k = 0; k < kSteps; ++k)
      qr[k] = *reinterpret_cast<const u32x4_t*>(qrow + 16 * k);
  }
  // The softmax below scales raw scores inside the exponent and scales their max once,
  // which needs a scale >= 0: a negative one is applied as its magnitude to -q (the sign
  // flip of a bf16 word is exact, and so is the negated product).
  float sl2 = scale_log2;
  if (sl2 < 0.0f) {
    sl2 = -sl2;
#pragma unroll
    for (int k = 0; k < kSteps; ++k)
      qr[k] = qr[k] ^ u32x4_t{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
  }
  f32x16_t o[kDimTiles];
#pragma unroll
  for (int dt = 0; dt < kDimTiles; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[dt][e] = 0.0f;
  float m = -INFINITY, l = 0.0f;
  const bf16x2_t2 kOnes2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  // The query loads above are conditional; without this wait the compiler cannot prove
  // them complete at the loop's head and waits for every load in flight (the staged
  // pairs' too) before each pair's first product.
  __builtin_amdgcn_s_waitcnt(0);

  const size_t head_elems = static_cast<size_t>(kBlockTokens) * D;
  const size_t block_elems = static_cast<size_t>(num_kv_heads) * head_elems;
  const int32_t* trow = tables + static_cast<size_t>(s) * W;
  // Block b's id, read one pair ahead of its use (b clamped to the range: past the end
  // the last block is loaded again and never read); uniform, so a scalar load.  At use a
  // bad id is flagged and read as block 0.
  auto raw_id = [&](int b) { return trow[min(b, nblk - 1)]; };
  auto checked = [&](int raw) {
    const bool bad = static_cast<unsigned>(raw) >= static_cast<unsigned>(num_blocks);
    if (bad && lane == 0) PKV_FLAG_ERROR(PKV_DEVERR_BLOCK_ID);
    return __builtin_amdgcn_readfirstlane(bad ? 0 : raw);
  };

  // Staging: a pair is four parts of 16-byte chunks (K of block 0, K of block 1, V of
  // block 0, V of block 1; 16 rows x D/8 chunks each).  Chunk j * 256 + tid goes through
  // thread tid, so a wave's chunks lie in one part (uniform base address) and the
  // thread's offset into every part is the same: chunk c of row c_row.
  const int c = tid % Ly::kPartChunks;
  const int c_row = c / kRowChunks;
  const uint32_t g_off = 16u * c;                    // bytes into the part
  const uint32_t g_off0 = 16u * (c % kRowChunks);    // the same column of the block's row 0
  const int s_k = c_row * RS + 8 * (c % kRowChunks);          // LDS element offsets
  constexpr int RV = Ly::kVRowElems;
  const int s_v = Ly::kVBase + vpos(c_row) * RV + 8 * (c % kRowChunks);
  u32x4_t rr[Ly::kPerThread];
  // Part of chunk j * 256 + tid (0: K of block 0, 1: K of block 1, 2: V of block 0, 3: V
  // of block 1), written so that the compiler sees it is uniform.
  auto part_of = [&](int j) {
    return Ly::kPartChunks >= kLdsThreads ? j * (kLdsThreads / Ly::kPartChunks)
                                          : j * (kLdsThreads / Ly::kPartChunks) +
                                                wave / (Ly::kPartChunks / kWave);
  };
  // V rows at or past `lim` (pair-relative: past the context's end, stale slots) are
  // fetched from the block's first row instead, which holds a real token, so their zero
  // weights meet finite values.
  auto pair_load = [&](int id0, int id1, int lim) {
    const size_t o0 = static_cast<size_t>(id0) * block_elems + kvh * head_elems;
    const size_t o1 = static_cast<size_t>(id1) * block_elems + kvh * head_elems;
#pragma unroll
    for (int j = 0; j < Ly::kPerThread; ++j) {
      const int part = part_of(j);  // uniform
      const char* base =
          reinterpret_cast<const char*>((part < 2 ? kc : vc) + (part % 2 ? o1 : o0));
      const uint32_t off =
          part >= 2 && (part - 2) * kBlockTokens + c_row >= lim ? g_off0 : g_off;
      rr[j] = *reinterpret_cast<const u32x4_t*>(base + off);
    }
  };
  auto pair_store = [&](int stage) {
#pragma unroll
    for (int j = 0; j < Ly::kPerThread; ++j) {
      const int part = part_of(j);  // uniform
      const int at = stage * Ly::kStage + (part < 2 ? s_k + (part % 2) * kBlockTokens * RS
                                                    : s_v + (part % 2) * kBlockTokens * RV);
      *reinterpret_cast<u32x4_t*>(smem + at) = rr[j];
    }
  };

  // K operand: row r, dims 16k + 8h ..; V^T operand reads: lane (g = lane / 16,
  // q = lane % 16) addresses V[16t + 4h + q / 4 (+ 8)][32 dt + 16 (g % 2) + 4 (q % 4)] and
  // receives four keys of dim 32 dt + r.
  const int k_at = r * RS + 8 * h;
  const int vq = lane % 16;
  const int v_at = Ly::kVBase + vpos(4 * h + vq / 4) * RV + 16 * ((lane / 16) % 2) + 4 * (vq % 4);
  auto scores = [&](int stage, f32x16_t& sc) {
#pragma unroll
    for (int e = 0; e < 16; ++e) sc[e] = 0.0f;
#pragma unroll
    for (int k = 0; k < kSteps; ++k) {
      const u32x4_t a =
          *reinterpret_cast<const u32x4_t*>(smem + k_at + stage * Ly::kStage + 16 * k);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, qr[k]), sc, 0,
                                                   0, 0);
    }
  };
  auto attend = [&](int stage, const f32x16_t& sc, int t_base) {
    // Raw scores, masked ones -inf (a select, so stale keys' NaN scores drop out).  The
    // max is taken on them and scaled once (rounding is monotonic, so that is the max of
    // the scaled scores); each weight is exp2(score * scale - m) with the scale inside
    // the exponent's FMA.  The max key's exponent is then the rounding residual of its
    // own scaled score, and its weight rounds to exactly 1 in bf16.
    float x[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) x[e] = sc[e];
    const bool masked = t_base + kPairTokens > lim0;  // uniform
    if (masked) {
      const int lim = n_c - t_base - 4 * h;  // keys 8i + j of the lane below lim are attended
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) x[4 * i + j] = (8 * i + j < lim) ? x[4 * i + j] : -INFINITY;
    }
    float bm = x[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) bm = fmaxf(bm, x[e]);
    bm = max_xor32(bm) * sl2;
    const bool raise = bm > m + kLazyMaxSlack;
    if (__any(raise)) {
      float a = 1.0f;
      if (raise) {
        a = m == -INFINITY ? 0.0f : fast_exp2(m - bm);
        m = bm;
      }
      l *= a;
#pragma unroll
      for (int dt = 0; dt < kDimTiles; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[dt][e] *= a;
    }
    // Masked weights are set to 0 by a select, in the pairs that have masks only.  Every
    // live row's m is finite from pair 0 on (it holds token 0, which every causal row
    // attends); rows past the chunk's last token may turn NaN, the products keep rows
    // (columns of the transposed tiles) apart, and those rows are never written.
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = fast_exp2(fmaf(x[8 * t + e], sl2, -m));
      if (masked) {  // a masked key's weight is 0 also at scale 0 (-inf * 0 is NaN)
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = x[8 * t + e] == -INFINITY ? 0.0f : p[e];
      }
      // (The packed words are kept as four scalars: read back as elements of the operand
      // vector, the ROCm 7.2 compiler fed the first word to all four dot products.)
      uint32_t pw[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) pw[w] = pack_bf16x2(p[2 * w], p[2 * w + 1]);
      // The row sum takes the weights as the products do, rounded to bf16: the output is
      // an exact convex combination of V rows under the rounded weights (a key whose
      // weight rounds to 1 alone returns its V row exactly).
#pragma unroll
      for (int w = 0; w < 4; ++w)
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t2, pw[w]), kOnes2, l,
                                            false);
      const u32x4_t pb = {pw[0], pw[1], pw[2], pw[3]};
#pragma unroll
      for (int dt = 0; dt < kDimTiles; ++dt) {
        const uint16_t* vp = smem + v_at + stage * Ly::kStage + 16 * t * RV + 32 * dt;
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16_t*)(vp));
        const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16_t*)(vp + 8 * RV));
        const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo);
        const u32x2_t h2 = __builtin_bit_cast(u32x2_t, hi);
        const u32x4_t a = {l2[0], l2[1], h2[0], h2[1]};
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                        __builtin_bit_cast(bf16x8_t, pb), o[dt],
                                                        0, 0, 0);
      }
    }
  };

  // Two LDS stages and one register set: pair p + 1's loads are issued after pair p - 1's
  // products and stored to the free stage once pair p's scores are read, so the staging
  // registers are not live while pair p's products hold theirs.  One barrier per pair.
  // Block ids are read one pair ahead of their loads.  Past the last block the last block
  // is loaded again (never read), so every load and store of the loop is unconditional.
  int id_a = raw_id(0), id_b = raw_id(1);
  pair_load(checked(id_a), checked(id_b), ch.n);
  pair_store(0);
  id_a = raw_id(2);
  id_b = raw_id(3);
  pair_load(checked(id_a), checked(id_b), ch.n - 2 * kBlockTokens);
  id_a = raw_id(4);
  id_b = raw_id(5);
  __syncthreads();
  auto step = [&](int cur, int b) {
    const int t_base = b * kBlockTokens;
    f32x16_t sc;
    const bool act = t_base < n_wave;  // causal: past every row of this wave, nothing to add
    if (act) scores(cur, sc);
    pair_store(cur ^ 1);
    if (act) attend(cur, sc, t_base);
    pair_load(checked(id_a), checked(id_b), ch.n - (b + 4) * kBlockTokens);
    id_a = raw_id(b + 6);
    id_b = raw_id(b + 7);
    __syncthreads();
  };
  for (int b = 0;;) {
    step(0, b);
    if ((b += 2) >= nblk) break;
    step(1, b);
    if ((b += 2) >= nblk) break;
  }

  const float L = sum_xor32(l);
  if (live) {
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    const size_t sh = static_cast<size_t>(ch.r0 + t0 + r / G) * num_q_heads + kvh * G + r % G;
    float* dst = out + sh * D + 4 * h;
#pragma unroll
    for (int dt = 0; dt < kDimTiles; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float4 v;
        v.x = o[dt][4 * i + 0] * inv;
        v.y = o[dt][4 * i + 1] * inv;
        v.z = o[dt][4 * i + 2] * inv;
        v.w = o[dt][4 * i + 3] * inv;
        *reinterpret_cast<float4*>(dst + 32 * dt + 8 * i) = v;
      }
    if (h == 0 && lse != nullptr) lse[sh] = L > 0.0f ? (m + __log2f(L)) * kLn2 : -INFINITY;
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
    // one workgroup per (row group, unit), grouped per XCD as the kernel decodes it
    constexpr int kGroupTokens = kT32Rows / G * kLdsWaves;
    const int n_groups = (a.max_q_len + kGroupTokens - 1) / kGroupTokens;
    const int units = a.batch * a.hkv;
    const dim3 grid(kXcds * ((units + kXcds - 1) / kXcds) * n_groups);
    hipLaunchKernelGGL((prefill_t32_kernel<D, G>), grid, dim3(kLdsThreads), 0, stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.kc),
                       static_cast<const uint16_t*>(a.vc), a.tables, a.W, a.cu_q, a.ctx,
                       a.total_q, a.max_q_len, a.hq, a.hkv, a.nb, a.scale_log2, a.out, a.lse,
                       a.batch);
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
