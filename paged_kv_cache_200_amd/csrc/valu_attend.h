// VALU attention over the block-paged cache (gfx950): 8 lanes per token, per-group online
// softmax, bf16 pairs through the dot2 instruction.  Internal; included by the HIP
// sources of libpkv after their error word is defined.
#pragma once

#include "common.h"

namespace pkv {
namespace {

constexpr int kLanesPerToken = 8;
constexpr int kGroups = kWave / kLanesPerToken;  // token groups per wave

template <typename T, int D>
struct Geom {
  static constexpr int kChunkElems = 16 / static_cast<int>(sizeof(T));  // elems per 16 B
  static constexpr int kChunks = D * static_cast<int>(sizeof(T)) / (16 * kLanesPerToken);
  static constexpr int kElems = kChunks * kChunkElems;                   // elems per lane
  static constexpr int kWords = kChunks * 4;                             // 32-bit words per lane
  static constexpr int kChunkStride = kLanesPerToken * kChunkElems;     // elems between chunks
  static_assert(kChunks >= 1, "head_dim too small for 8 lanes per token");
};

// Dimension held by element e of a lane with sub-index `sub` (0..7).
template <typename T, int D>
__device__ __forceinline__ int lane_dim(int sub, int e) {
  using Gm = Geom<T, D>;
  return (e / Gm::kChunkElems) * Gm::kChunkStride + sub * Gm::kChunkElems + (e % Gm::kChunkElems);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <typename T>
__device__ __forceinline__ float dot_word(uint32_t qw, uint32_t kw, float acc);

template <>
__device__ __forceinline__ float dot_word<uint16_t>(uint32_t qw, uint32_t kw, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qw),
                                         __builtin_bit_cast(bf16x2_t, kw), acc, false);
}

template <>
__device__ __forceinline__ float dot_word<float>(uint32_t qw, uint32_t kw, float acc) {
  return fmaf(__uint_as_float(qw), __uint_as_float(kw), acc);
}

// Element e of a token's words as float32 (e compile-time after unrolling).
template <typename T, int N>
__device__ __forceinline__ float elem_of(const uint32_t (&w)[N], int e) {
  if constexpr (sizeof(T) == 2)
    return (e & 1) ? bf16_hi(w[e / 2]) : bf16_lo(w[e / 2]);
  else
    return __uint_as_float(w[e]);
}

template <typename T, int D>
struct TokenRegs {
  uint32_t k[2][Geom<T, D>::kWords];  // [token in block: grp, grp+8][words]
  uint32_t v[2][Geom<T, D>::kWords];
};

template <typename T, int D, int G>
struct GroupState {
  float m[G];                       // lazy running max, log2 units
  float l[G];                       // sum of exp2(score - m)
  float acc[G][Geom<T, D>::kElems]; // sum of exp2(score - m) * V over this lane's dims
};


// K/V that are read exactly once per call go through non-temporal 16-byte loads, which
// keep the stream from displacing other data in the caches (measured ~10% more HBM
// throughput on gfx950 for random 4 KiB tiles than plain loads).  Blocks shared by
// several sequences are read with plain loads so sibling waves find them cached.
template <bool kStreaming>
__device__ __forceinline__ u32x4_t load16(const void* p) {
  if constexpr (kStreaming)
    return __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  else
    return *static_cast<const u32x4_t*>(p);
}

template <typename T, int D, bool kStreaming>
__device__ __forceinline__ void load_block(TokenRegs<T, D>& r, const T* __restrict__ kt,
                                           const T* __restrict__ vt, int lane_off) {
  using Gm = Geom<T, D>;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int c = 0; c < Gm::kChunks; ++c) {
      const int off = lane_off + i * kGroups * D + c * Gm::kChunkStride;
      const u32x4_t kk = load16<kStreaming>(kt + off);
      const u32x4_t vv = load16<kStreaming>(vt + off);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        r.k[i][4 * c + j] = kk[j];
        r.v[i][4 * c + j] = vv[j];
      }
    }
  }
}

// One 16-token block: 2 tokens per lane (token grp and grp + 8 of the block).
// kMasked: only the first n_valid tokens of the block count.
template <typename T, int D, int G, bool kMasked>
__device__ __forceinline__ void process_block(const TokenRegs<T, D>& r,
                                              const uint32_t (&q)[G][Geom<T, D>::kWords],
                                              GroupState<T, D, G>& st, float scale_log2,
                                              int grp, int n_valid) {
  using Gm = Geom<T, D>;
  float sc[2][G];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float a = 0.0f;
#pragma unroll
      for (int j = 0; j < Gm::kWords; ++j) a = dot_word<T>(q[g][j], r.k[i][j], a);
      sc[i][g] = a;
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int g = 0; g < G; ++g) sc[i][g] = group8_sum(sc[i][g]) * scale_log2;
  }
  bool valid[2] = {true, true};
  if constexpr (kMasked) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      valid[i] = (i * kGroups + grp) < n_valid;
#pragma unroll
      for (int g = 0; g < G; ++g) sc[i][g] = valid[i] ? sc[i][g] : -INFINITY;
    }
  }
  bool raise = false;
#pragma unroll
  for (int g = 0; g < G; ++g) raise |= fmaxf(sc[0][g], sc[1][g]) > st.m[g] + kLazyMaxSlack;
  if (raise) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mn = fmaxf(st.m[g], fmaxf(sc[0][g], sc[1][g]));
      const float a = (st.m[g] == -INFINITY) ? 0.0f : fast_exp2(st.m[g] - mn);
      st.l[g] *= a;
#pragma unroll
      for (int e = 0; e < Gm::kElems; ++e) st.acc[g][e] *= a;
      st.m[g] = mn;
    }
  }
  float p[2][G];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float e = fast_exp2(sc[i][g] - st.m[g]);
      p[i][g] = (kMasked && !valid[i]) ? 0.0f : e;
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) st.l[g] += p[0][g] + p[1][g];
  // V is widened one element at a time, right before its G uses, which keeps the
  // widened block out of the register file while the next block's loads are in flight.
#pragma unroll
  for (int e = 0; e < Gm::kElems; ++e) {
    float x0 = elem_of<T>(r.v[0], e);
    float x1 = elem_of<T>(r.v[1], e);
    if constexpr (kMasked) {
      // select, not multiply: stale or NaN slots must not reach the accumulator
      x0 = valid[0] ? x0 : 0.0f;
      x1 = valid[1] ? x1 : 0.0f;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) st.acc[g][e] = fmaf(p[1][g], x1, fmaf(p[0][g], x0, st.acc[g][e]));
  }
}

// One wave's share of a unit: attend this KV head's G query rows of q row `qrow` over
// the tokens [tok0, tok1) of the sequence whose block-table row is `s` (tok0 a multiple
// of the block size, tok0 <= tok1), taking the range's blocks wave, wave + NW, ... (the
// last one partial when it holds the range end), then merge the wave's 8 token groups so
// that every lane holds the wave's totals (m, l, acc) for its dims.
//
// Blocks stream two deep: block k + 1's loads are in flight while block k is processed.
// Every K/V load of the steady loop is unconditional and shares straight-line code with
// the processing it overlaps: at a join after a conditional load the compiler's wait
// counts must hold on both paths, so it would wait for the prefetched block as well.
// Block ids come 64 at a time, one per lane, and are read from the register with
// readlane.
template <typename T, int D, int G, int NW, bool kStreaming>
__device__ __forceinline__ void attend_range(GroupState<T, D, G>& st, const T* __restrict__ q,
                                             const T* __restrict__ kc, const T* __restrict__ vc,
                                             const int32_t* __restrict__ tables, int W, int s,
                                             int qrow, int kvh, int num_q_heads, int num_kv_heads,
                                             int num_blocks, float scale_log2, int tok0,
                                             int tok1, int wave, int lane) {
  using Gm = Geom<T, D>;
  const int grp = lane / kLanesPerToken;
  const int sub = lane % kLanesPerToken;
  const int b_begin = tok0 / kBlockTokens;
  const int nfull = tok1 / kBlockTokens - b_begin;  // blocks wholly inside [tok0, tok1)
  const int tail = tok1 % kBlockTokens;             // valid tokens of a trailing partial block
  const int nb = nfull + (tail != 0 ? 1 : 0);
  const int n_w = nb > wave ? (nb - wave + NW - 1) / NW : 0;  // this wave's blocks
  // The partial block (index nfull) is the last block of wave nfull % NW.
  const int last_valid =
      (tail != 0 && n_w > 0 && wave + NW * (n_w - 1) == nfull) ? tail : kBlockTokens;

  const size_t head_elems = static_cast<size_t>(kBlockTokens) * D;
  const size_t block_elems = static_cast<size_t>(num_kv_heads) * head_elems;
  const T* kbase = kc + kvh * head_elems;
  const T* vbase = vc + kvh * head_elems;
  const int lane_off = grp * D + sub * Gm::kChunkElems;
  // The wave's k-th block id is trow[NW * k].
  const int32_t* trow = tables + static_cast<size_t>(s) * W + b_begin + wave;

  // An id outside the pool reads block 0 instead and is reported once, at the end.
  bool bad_id = false;
  auto fetch_ids = [&](int base) {  // lane j: raw id of the wave's block base + j
    const int k = base + lane;
    return k < n_w ? trow[NW * k] : 0;
  };
  auto load = [&](TokenRegs<T, D>& r, int raw_id) {
    const bool bad = static_cast<unsigned>(raw_id) >= static_cast<unsigned>(num_blocks);
    bad_id |= bad;
    const size_t blk = bad ? 0 : static_cast<size_t>(raw_id);
    load_block<T, D, kStreaming>(r, kbase + blk * block_elems, vbase + blk * block_elems,
                                 lane_off);
  };

  // The first window's ids, then its first block, then the query rows.
  TokenRegs<T, D> r0, r1;
  int ids = fetch_ids(0);
  if (n_w > 0) load(r0, __builtin_amdgcn_readlane(ids, 0));

  // Query rows of this KV head's group, this lane's dims, raw bits.
  uint32_t qr[G][Gm::kWords];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const T* qg = q + (static_cast<size_t>(qrow) * num_q_heads + kvh * G + g) * D;
#pragma unroll
    for (int c = 0; c < Gm::kChunks; ++c) {
      const uint4 w = *reinterpret_cast<const uint4*>(qg + c * Gm::kChunkStride +
                                                      sub * Gm::kChunkElems);
      qr[g][4 * c + 0] = w.x; qr[g][4 * c + 1] = w.y;
      qr[g][4 * c + 2] = w.z; qr[g][4 * c + 3] = w.w;
    }
  }

#pragma unroll
  for (int g = 0; g < G; ++g) {
    st.m[g] = -INFINITY;
    st.l[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < Gm::kElems; ++e) st.acc[g][e] = 0.0f;
  }

  auto process = [&](const TokenRegs<T, D>& r) {
    process_block<T, D, G, false>(r, qr, st, scale_log2, grp, kBlockTokens);
  };
  auto process_last = [&](const TokenRegs<T, D>& r, int valid) {
    if (valid == kBlockTokens)
      process_block<T, D, G, false>(r, qr, st, scale_log2, grp, kBlockTokens);
    else
      process_block<T, D, G, true>(r, qr, st, scale_log2, grp, valid);
  };

  // Windows of 64 blocks; a window's first block is already loading into r0 when it
  // starts.
  for (int wb = 0; wb < n_w; wb += kWave) {
    const int n = min(kWave, n_w - wb);
    const int valid = wb + n == n_w ? last_valid : kBlockTokens;
    auto id = [&](int k) { return __builtin_amdgcn_readlane(ids, k); };
    int k = 0;  // block k is in r0
    for (; k + 2 < n; k += 2) {
      load(r1, id(k + 1));
      process(r0);  // block k
      load(r0, id(k + 2));
      process(r1);  // block k + 1
    }
    // One or two blocks of the window remain; block k is in r0.
    if (n - k == 2) {
      load(r1, id(k + 1));
      process(r0);
      if (wb + kWave < n_w) {  // next window: its ids, then its first block
        ids = fetch_ids(wb + kWave);
        load(r0, __builtin_amdgcn_readlane(ids, 0));
      }
      process_last(r1, valid);
    } else {  // only in the last window: a full window has an even count
      process_last(r0, valid);
    }
  }
  if (bad_id && lane == 0) PKV_FLAG_ERROR(PKV_DEVERR_BLOCK_ID);

  // Merge the 8 token groups of the wave (lanes with equal `sub` hold the same dims).
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float mx = st.m[g];
    mx = fmaxf(mx, __shfl_xor(mx, 8));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float a = (st.m[g] == -INFINITY) ? 0.0f : fast_exp2(st.m[g] - mx);
    float l = st.l[g] * a;
    l += __shfl_xor(l, 8);
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    st.l[g] = l;
#pragma unroll
    for (int e = 0; e < Gm::kElems; ++e) {
      float x = st.acc[g][e] * a;
      x += __shfl_xor(x, 8);
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      st.acc[g][e] = x;
    }
    st.m[g] = mx;
  }

}

}  // namespace
}  // namespace pkv
