// Matrix-core attention tile over the block-paged cache (gfx950), shared by the
// shared-prefix decode and the paged prefill.  Internal; included by the HIP sources of
// libpkv after their error word is defined.
#pragma once

#include "common.h"

namespace pkv {
namespace {

constexpr int kTileWaves = 4;  // waves of a tile workgroup

// Matrix-core attention tile for bf16 caches: up to 16 query rows that read the same
// blocks, (member, query head) pairs, attended together against each block, which is read
// once per tile: 16 x 16 score tiles S^T = K Q^T on the bf16 MFMA (16x16x32), then
// O += P V on the bf16 MFMA (16x16x16) with P carried as a sum of two bf16 terms.  Four
// waves take the range's blocks round-robin, each with its own online softmax per row,
// and are merged through LDS.  Members are the forks of a copy-on-write group in the
// shared-prefix decode and the query tokens of one sequence in the paged prefill.
//
// Lane layouts (c = lane % 16, h = lane / 16):
//   S^T tile: lane holds rows c, tokens 4h + r (r = 0..3) of the block.  Score step k
//     contracts dims 32k .. 32k + 31, lane h-group taking 8 of them: K[token c][32k + 8h ..]
//     and Q[row c][32k + 8h ..], so one load instruction reads 64 contiguous bytes of
//     every token row.
//   P V, output tile j: A = P[row c][tokens 4h .. 4h + 3] (the lane's own scores),
//     B = V[tokens 4h .. 4h + 3][c * D/16 + j], so lane loads the D/16 contiguous dims
//     c * D/16 .. of 4 tokens.
//   O tile j: lane holds rows 4h + r, dim c * D/16 + j.
constexpr int kMfmaRows = 16;
// Blocks in flight per wave in the plain-decode tile.
#ifndef PKV_MFMA_PLAIN_DEPTH
#define PKV_MFMA_PLAIN_DEPTH 4
#endif
constexpr int kPlainDepth = PKV_MFMA_PLAIN_DEPTH;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <int D>
struct MfmaGeom {
  static constexpr int kQkSteps = D / 32;   // 16x16x32 steps over the head dim
  static constexpr int kTiles = D / 16;     // output tiles of 16 dims
  static constexpr int kVWords = D / 32;    // 32-bit words of V per lane and token
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
};

template <int D>
struct MfmaBlock {
  u32x4_t k[MfmaGeom<D>::kQkSteps];
  uint32_t v[4][MfmaGeom<D>::kVWords];
};

template <int D>
__device__ __forceinline__ void mfma_load_block(MfmaBlock<D>& b, const uint16_t* __restrict__ kt,
                                                const uint16_t* __restrict__ vt, int c, int h) {
  using Mg = MfmaGeom<D>;
#pragma unroll
  for (int k = 0; k < Mg::kQkSteps; ++k)
    b.k[k] = *reinterpret_cast<const u32x4_t*>(kt + c * D + 32 * k + 8 * h);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint16_t* src = vt + (4 * h + k) * D + c * Mg::kTiles;
    if constexpr (Mg::kVWords == 4) {
      const u32x4_t w = *reinterpret_cast<const u32x4_t*>(src);
#pragma unroll
      for (int j = 0; j < 4; ++j) b.v[k][j] = w[j];
    } else {
      const u32x2_t w = *reinterpret_cast<const u32x2_t*>(src);
      b.v[k][0] = w[0];
      b.v[k][1] = w[1];
    }
  }
}

// v_perm_b32 selectors for perm(hi_word, lo_word, sel): result byte k is byte sel[k] of
// the 8-byte value hi_word:lo_word (0-3 lo_word, 4-7 hi_word).
constexpr uint32_t kLowHalves = 0x05040100u;   // lo16(lo_word) | lo16(hi_word) << 16
constexpr uint32_t kHighHalves = 0x07060302u;  // hi16(lo_word) | hi16(hi_word) << 16

// Softmax state of one wave's 16 score rows: lane (c, h) holds row c's running max
// (log2 units, lazy as in the first pass) and its share of the row's exp-sum, and the
// unnormalised output of rows 4h .. 4h + 3 at dims c * D/16 + j (tile j).
template <int D>
struct MfmaRows {
  float m_c;
  float l_part;
  f32x4_t o[MfmaGeom<D>::kTiles];
};

template <int D>
__device__ __forceinline__ void mfma_rows_init(MfmaRows<D>& r) {
  r.m_c = -INFINITY;
  r.l_part = 0.0f;
#pragma unroll
  for (int j = 0; j < MfmaGeom<D>::kTiles; ++j) r.o[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
}

// One 16-token block (token t_base .. t_base + 15) for the wave's 16 rows: row c attends
// the block's tokens below n_c (its own limit); V of tokens at or past n_max (every row's
// end) is zeroed first, since a zero weight times a stale NaN would spoil the rows.
// P enters P V as two bf16 terms (truncated value + truncated remainder, about 2^-16
// relative).  (A single rounded bf16 term measured 8% faster in the prefill but put the
// error at 4e-3, a thousand times higher.)
// x combined with the value of lane ^ 16, then of lane ^ 32 (gfx950 lane swaps, in the
// VALU).  A swap returns the lane's own value and its partner's in some order; the sum
// and the max are commutative, so each step equals x op x[lane ^ k] bit for bit.
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int D>
__device__ __forceinline__ void mfma_rows_block(MfmaRows<D>& r, MfmaBlock<D>& cur,
                                                const u32x4_t (&qr)[MfmaGeom<D>::kQkSteps],
                                                int t_base, int n_c, int n_max, int h,
                                                float scale_log2) {
  using Mg = MfmaGeom<D>;
  f32x4_t sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < Mg::kQkSteps; ++s)
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, cur.k[s]),
                                                 __builtin_bit_cast(bf16x8_t, qr[s]), sc, 0, 0,
                                                 0);
  // Scores of row c for tokens 4h + i, masked by the row's own length (select, so
  // stale or NaN slots never pass).
  float x[4];
  float bm = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = (t_base + 4 * h + i < n_c) ? sc[i] * scale_log2 : -INFINITY;
    bm = fmaxf(bm, x[i]);
  }
  bm = max_xor32(max_xor16(bm));  // the row's four lanes c + 16 h
  const bool raise = bm > r.m_c + kLazyMaxSlack;
  if (__any(raise)) {
    float a = 1.0f;
    if (raise) {
      a = r.m_c == -INFINITY ? 0.0f : fast_exp2(r.m_c - bm);
      r.m_c = bm;
    }
    r.l_part *= a;
    // Output rows 4h + i take the factor of the lanes that own score row 4h + i.
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
    p[i] = x[i] == -INFINITY ? 0.0f : fast_exp2(x[i] - r.m_c);
    r.l_part += p[i];
  }
  // P V on the bf16 MFMA with P split into two bf16 terms, hi = P truncated and
  // lo = (P - hi) truncated (P - hi is exact in fp32), so the product sees P to about
  // 2^-16 relative.  Both terms go through one 16x16x32 product: its 32-long k runs over
  // (term, token) pairs, lane (c, h) supplying k = 8h .. 8h + 7 as P_hi[c][4h .. 4h + 3]
  // then P_lo[c][4h .. 4h + 3] (the lane's own scores), and the B operand of lane
  // (n, h) the matching V[4h .. 4h + 3][n] twice.  Any order of k is the same sum, so
  // no lane needs another lane's scores.
  // (v_perm_b32 byte selects: kHighHalves packs the high 16 bits of two words, low word
  // first; kLowHalves their low 16 bits.)
  uint32_t pw[4], rw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pw[i] = __float_as_uint(p[i]);
    rw[i] = __float_as_uint(p[i] - __uint_as_float(pw[i] & 0xffff0000u));  // exact remainder
  }
  const bf16x8_t a = __builtin_bit_cast(
      bf16x8_t, u32x4_t{__builtin_amdgcn_perm(pw[1], pw[0], kHighHalves),
                        __builtin_amdgcn_perm(pw[3], pw[2], kHighHalves),
                        __builtin_amdgcn_perm(rw[1], rw[0], kHighHalves),
                        __builtin_amdgcn_perm(rw[3], rw[2], kHighHalves)});
  // Tokens past every taken row's end hold stale data: zero their V (0 * NaN).
  if (t_base + kBlockTokens > n_max) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool vok = t_base + 4 * h + i < n_max;
#pragma unroll
      for (int w = 0; w < Mg::kVWords; ++w) cur.v[i][w] = vok ? cur.v[i][w] : 0u;
    }
  }
  const auto& v = cur.v;
  // B operand of tile j: V[tokens 4h .. 4h + 3][dim c * D/16 + j], the even tiles from
  // the low halves of the lane's words, the odd ones from the high halves.
#pragma unroll
  for (int w = 0; w < Mg::kVWords; ++w) {
    const uint32_t e0 = __builtin_amdgcn_perm(v[1][w], v[0][w], kLowHalves);
    const uint32_t e1 = __builtin_amdgcn_perm(v[3][w], v[2][w], kLowHalves);
    const uint32_t o0 = __builtin_amdgcn_perm(v[1][w], v[0][w], kHighHalves);
    const uint32_t o1 = __builtin_amdgcn_perm(v[3][w], v[2][w], kHighHalves);
    const bf16x8_t b_even = __builtin_bit_cast(bf16x8_t, u32x4_t{e0, e1, e0, e1});
    const bf16x8_t b_odd = __builtin_bit_cast(bf16x8_t, u32x4_t{o0, o1, o0, o1});
    r.o[2 * w] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b_even, r.o[2 * w], 0, 0, 0);
    r.o[2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b_odd, r.o[2 * w + 1], 0, 0, 0);
  }
}

// A token appended in the same launch, as the tile's lanes hold it once loaded: lane
// (c, h) keeps the K chunks of score steps k (dims 32k + 8h ..), used where c is the
// token's slot, and the V dims c * D/16 .., used where h is its slot / 4.  The tile puts
// them into the block holding `pos` in place of what it loaded from the cache there, so
// the cache write of the token need not precede the tile's loads.  pos < 0: none.
template <int D>
struct MfmaNewToken {
  int pos;
  u32x4_t k[MfmaGeom<D>::kQkSteps];
  uint32_t v[MfmaGeom<D>::kVWords];
};

// LDS of one row tile: per wave the members found not to share the leader's blocks, and
// per wave and row the softmax state and the unnormalised output.
template <int D>
struct MfmaShared {
  unsigned mismatch[kTileWaves];
  float m[kTileWaves][kMfmaRows];
  float l[kTileWaves][kMfmaRows];
  float4 o[kTileWaves][kMfmaRows][D / 4];
};

// Attends the rows of the members selected by `take` (bit mi: member mi, whose query
// rows are q rows row0 + mi, heads kvh * G .. kvh * G + G - 1) over tokens
// [tok0, lim[mi]) through the block-table row `lead`, and writes each row (r, h) to
// dst_out[(r * Hq + h) * slots + slot] (D floats) and dst_lse[...] (nullable).  A taken
// member with nothing to attend gets out = 0, lse = -inf.
//
// member_rows (nullable): member mi's own table row is member_rows + mi * W; every taken
// member's block ids are then compared with the leader's over its share of the range (in
// the same loads that fetch the leader's ids).  Members that differ come back as the
// result; if there are any, nothing is written, and the caller redoes the others
// without them and each of them through its own row.  Called by all threads of the
// workgroup (it synchronises).  kAgentStores: results are written with device-scope
// stores (written through to where every XCD's device-scope loads read them), for a
// merge by another workgroup of the same launch.  kPlain: one member (take = 1) and no
// sharing check (member_rows unused); the query rows are then loaded by every lane (lanes
// of rows not taken load member 0's and zero them), so no load of the tile's start is
// conditional and the first block's loads need not wait for all earlier memory work (a
// caller's stores included).
template <int D, int G, bool kAgentStores = false, bool kPlain = false>
__device__ __forceinline__ unsigned mfma_tile(
    MfmaShared<D>& sm, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ lead,
    const int32_t* __restrict__ member_rows, int W, const int (&lim)[kMfmaRows / G],
    unsigned take, int row0, int kvh, int num_q_heads, int num_kv_heads, int num_blocks,
    float scale_log2, int tok0, int slot, int slots, float* __restrict__ dst_out,
    float* __restrict__ dst_lse, const MfmaNewToken<D>* nt = nullptr) {
  using Mg = MfmaGeom<D>;
  constexpr int kMembers = kMfmaRows / G;
  constexpr int kRows = kMembers * G;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int c = lane % 16;
  const int h = lane / 16;
  const size_t head_elems = static_cast<size_t>(kBlockTokens) * D;
  const size_t block_elems = static_cast<size_t>(num_kv_heads) * head_elems;
  const int b0 = tok0 / kBlockTokens;

  // The largest token limit of the taken members, and this lane's score row's.
  int n_max = 0;
  int n_c = 0;
#pragma unroll
  for (int mi = 0; mi < kMembers; ++mi) {
    const int n = ((take >> mi) & 1u) ? lim[mi] : 0;
    n_max = max(n_max, n);
    if (c < kRows && c / G == mi) n_c = n;
  }

  // Query rows as the B operand of the score step (zero for rows not taken).
  u32x4_t qr[Mg::kQkSteps];
  if constexpr (kPlain) {
    const bool live = c < G;
    const uint16_t* qrow =
        q + (static_cast<size_t>(row0) * num_q_heads + kvh * G + c % G) * D + 8 * h;
#pragma unroll
    for (int k = 0; k < Mg::kQkSteps; ++k) {
      const u32x4_t w = *reinterpret_cast<const u32x4_t*>(qrow + 32 * k);
      qr[k] = live ? w : u32x4_t{0u, 0u, 0u, 0u};
    }
  } else {
#pragma unroll
    for (int k = 0; k < Mg::kQkSteps; ++k) qr[k] = u32x4_t{0u, 0u, 0u, 0u};
    if (c < kRows && ((take >> (c / G)) & 1u)) {
      const uint16_t* qrow =
          q + (static_cast<size_t>(row0 + c / G) * num_q_heads + kvh * G + c % G) * D + 8 * h;
#pragma unroll
      for (int k = 0; k < Mg::kQkSteps; ++k)
        qr[k] = *reinterpret_cast<const u32x4_t*>(qrow + 32 * k);
    }
  }

  MfmaRows<D> rows;
  mfma_rows_init<D>(rows);

  const int nblk = n_max > tok0 ? (n_max - tok0 + kBlockTokens - 1) / kBlockTokens : 0;
  const int nw = nblk > wave ? (nblk - wave + kTileWaves - 1) / kTileWaves : 0;
  unsigned mism = 0;  // members whose ids differ on this wave's blocks
  // Block ids of this wave's blocks, 64 at a time, one per lane.
  auto fetch_ids = [&](int from) -> int {
    const int k = from + lane;
    const bool live = k < nw;
    const int b = b0 + wave + kTileWaves * k;
    int id = live ? lead[b] : 0;
    if (!kPlain && member_rows != nullptr) {
#pragma unroll
      for (int mi = 0; mi < kMembers; ++mi) {
        const bool differs = live && ((take >> mi) & 1u) && b * kBlockTokens < lim[mi] &&
                             member_rows[static_cast<size_t>(mi) * W + b] != id;
        if (__any(differs)) mism |= 1u << mi;
      }
    }
    const bool bad = static_cast<unsigned>(id) >= static_cast<unsigned>(num_blocks);
    id = bad ? 0 : id;
    if (__any(bad) && lane == 0) PKV_FLAG_ERROR(PKV_DEVERR_BLOCK_ID);
    return id;
  };
  int ids = fetch_ids(0);
  // The query loads above are conditional unless kPlain: without this wait the compiler
  // cannot prove them complete at the block loop's head and waits there for every
  // outstanding load, the block in flight included.
  if constexpr (!kPlain) __builtin_amdgcn_s_waitcnt(0);
  auto load = [&](MfmaBlock<D>& bl, int k) {  // block k of the current id window
    const int id = __builtin_amdgcn_readlane(ids, k);
    const size_t off = static_cast<size_t>(id) * block_elems + kvh * head_elems;
    mfma_load_block<D>(bl, kc + off, vc + off, c, h);
  };
  auto process = [&](MfmaBlock<D>& cur, int k) {
    const int t_base = (b0 + wave + kTileWaves * k) * kBlockTokens;  // token of slot 0
    if constexpr (kPlain) {
      if (nt != nullptr && nt->pos >= t_base && nt->pos < t_base + kBlockTokens) {
        const int ts = nt->pos - t_base;
        if (c == ts) {
#pragma unroll
          for (int kk = 0; kk < Mg::kQkSteps; ++kk) cur.k[kk] = nt->k[kk];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (h == ts / 4 && i == ts % 4) {
#pragma unroll
            for (int w = 0; w < Mg::kVWords; ++w) cur.v[i][w] = nt->v[w];
          }
        }
      }
    }
    mfma_rows_block<D>(rows, cur, qr, t_base, n_c, n_max, h, scale_log2);
  };
  // Two blocks in flight: the next block's loads are issued before this one's math.  The
  // loads of the steady loop are unconditional (a conditional one would make the
  // compiler's wait before the math cover the block in flight too); each window of 64
  // blocks, one id per lane, is streamed on its own.
  if constexpr (kPlain) {
    // A plain decode unit is a short chain of blocks per wave (8 for 512 tokens): keep
    // kPlainDepth of them in flight.  Loads past the window's last block load that block
    // again (a cache hit, never processed), so every load is unconditional; only the
    // processing of those slots is skipped.
    MfmaBlock<D> buf[kPlainDepth];
    for (int wb = 0; wb < nw; wb += kWave) {
      if (wb > 0) ids = fetch_ids(wb);
      const int n = min(kWave, nw - wb);
#pragma unroll
      for (int i = 0; i < kPlainDepth - 1; ++i) load(buf[i], min(i, n - 1));
      for (int k = 0; k < n; k += kPlainDepth) {
#pragma unroll
        for (int u = 0; u < kPlainDepth; ++u) {
          load(buf[(u + kPlainDepth - 1) % kPlainDepth], min(k + u + kPlainDepth - 1, n - 1));
          if (k + u < n) process(buf[u], wb + k + u);
        }
      }
    }
  } else {
    MfmaBlock<D> bufa, bufb;
    for (int wb = 0; wb < nw; wb += kWave) {
      if (wb > 0) ids = fetch_ids(wb);
      const int n = min(kWave, nw - wb);
      load(bufa, 0);
      int k = 0;  // window block k is in bufa
      for (; k + 2 < n; k += 2) {
        load(bufb, k + 1);
        process(bufa, wb + k);
        load(bufa, k + 2);
        process(bufb, wb + k + 1);
      }
      if (n - k == 2) {
        load(bufb, k + 1);
        process(bufa, wb + k);
        process(bufb, wb + k + 1);
      } else {
        process(bufa, wb + k);
      }
    }
  }
  float l_c = rows.l_part;
    l_c = sum_xor32(sum_xor16(l_c));
  const float m_c = rows.m_c;
  const auto& o = rows.o;

  // Merge the waves: each publishes (m, l) per row and its unnormalised rows.
  constexpr int kQuads = Mg::kTiles / 4;  // float4s per lane and row
  if (h == 0) {
    sm.m[wave][c] = m_c;
    sm.l[wave][c] = l_c;
  }
  if (lane == 0) sm.mismatch[wave] = mism;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int u = 0; u < kQuads; ++u)
      sm.o[wave][4 * h + i][c * kQuads + u] =
          make_float4(o[4 * u][i], o[4 * u + 1][i], o[4 * u + 2][i], o[4 * u + 3][i]);
  }
  __syncthreads();
  unsigned differ = 0;
#pragma unroll
  for (int w = 0; w < kTileWaves; ++w) differ |= sm.mismatch[w];
  differ &= take;
  // A member that does not share streamed the leader's blocks up to its own length,
  // which can include slots stale for everyone (NaN V times a zero weight spoils every
  // row), so a tile with any such member writes nothing and is redone without it.
  const unsigned write = differ != 0 ? 0u : take;
  const int row = tid / 16;  // 16 rows x 16 threads of D/16 dims
  const int cc = tid % 16;
  const int mi = row / G;
  if (row < kRows && ((write >> mi) & 1u)) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kTileWaves; ++w) M = fmaxf(M, sm.m[w][row]);
    float e[kTileWaves];
    float L = 0.0f;
#pragma unroll
    for (int w = 0; w < kTileWaves; ++w) {
      e[w] = sm.m[w][row] == -INFINITY ? 0.0f : fast_exp2(sm.m[w][row] - M);
      L += sm.l[w][row] * e[w];
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    const size_t sh = static_cast<size_t>(row0 + mi) * num_q_heads + kvh * G + row % G;
    float* dst = dst_out + (sh * slots + slot) * D + cc * Mg::kTiles;
    if constexpr (kAgentStores) {
      // Device-scope stores write through one 4-byte store per lane and instruction:
      // thread cc takes dims cc, cc + 16, ... so that each instruction covers 16
      // consecutive floats of the row (the same sums as below, element by element).
      float* drow = dst_out + (sh * slots + slot) * D;
#pragma unroll
      for (int k = 0; k < Mg::kTiles; ++k) {
        float acc = 0.0f;
#pragma unroll
        for (int w = 0; w < kTileWaves; ++w)
          acc = fmaf(e[w], reinterpret_cast<const float*>(&sm.o[w][row][0])[cc + 16 * k], acc);
        __hip_atomic_store(drow + cc + 16 * k, acc * inv, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
#pragma unroll
    for (int u = 0; u < (kAgentStores ? 0 : kQuads); ++u) {
      float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
      for (int w = 0; w < kTileWaves; ++w) {
        const float4 x = sm.o[w][row][cc * kQuads + u];
        acc.x = fmaf(e[w], x.x, acc.x);
        acc.y = fmaf(e[w], x.y, acc.y);
        acc.z = fmaf(e[w], x.z, acc.z);
        acc.w = fmaf(e[w], x.w, acc.w);
      }
      acc.x *= inv; acc.y *= inv; acc.z *= inv; acc.w *= inv;
      // dims cc * D/16 + j of tile j: float4 u holds tiles 4u .. 4u + 3
      *reinterpret_cast<float4*>(dst + 4 * u) = acc;
    }
    if (cc == 0 && dst_lse != nullptr) {
      const float ls = L > 0.0f ? (M + __log2f(L)) * kLn2 : -INFINITY;
      if constexpr (kAgentStores)
        __hip_atomic_store(dst_lse + sh * slots + slot, ls, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      else
        dst_lse[sh * slots + slot] = ls;
    }
  }
  __syncthreads();  // LDS reused by the next call
  return differ;
}


}  // namespace
}  // namespace pkv
