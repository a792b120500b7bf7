// Paged (chunked) prefill attention for gfx950.
//
// What is computed (spindle, "Why write the forward pass" and "Two bugs worth
// recording"): a sequence's new chunk of q_len query tokens, already appended to the
// block cache, attends causally over the sequence's context of n tokens (the chunk
// included): query i sits at position n - q_len + i and attends to tokens [0, that
// position], through the block table, with explicit lengths.
//
// bf16 caches: the matrix-core tile.  A workgroup takes 16 / G consecutive query tokens
// of one sequence for one KV head, i.e. 16 (token, query head) rows that read the same
// blocks; each row carries its own causal limit, so one pass over the blocks serves all
// of them.  fp32 caches: the VALU routine of the decode, one wave per query token.

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

// Work item w = (tile x, sequence, KV head), x fastest.  The hardware hands workgroups
// to the eight XCDs round-robin by id, so workgroup b takes item (b % 8) * per + b / 8:
// the tiles of one (sequence, KV head), which read the same blocks, run on one XCD and
// share its L2.  Tiles are taken from the chunk's end (the longest causal ranges) first.
constexpr int kXcds = 8;

template <int D, int G>
__global__ __launch_bounds__(kTileWaves * kWave) void prefill_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ tables, int W,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ ctx_lens, int total_q,
    int max_q_len, int tiles_x, int batch, int num_q_heads, int num_kv_heads, int num_blocks,
    float scale_log2, float* __restrict__ out, float* __restrict__ lse) {
  constexpr int kMembers = kMfmaRows / G;  // query tokens per tile
  __shared__ MfmaShared<D> sm;
  const int items = tiles_x * batch * num_kv_heads;
  const int per = gridDim.x / kXcds;
  const int w = static_cast<int>(blockIdx.x % kXcds) * per + static_cast<int>(blockIdx.x / kXcds);
  if (w >= items) return;
  const int x = w % tiles_x;
  const int s = (w / tiles_x) % batch;
  const int kvh = w / (tiles_x * batch);
  const bool first = x == 0 && kvh == 0 && threadIdx.x == 0;
  const Chunk c = chunk_of(cu_q, ctx_lens, s, total_q, max_q_len, W * kBlockTokens, first);
  const int tiles = (c.len + kMembers - 1) / kMembers;
  if (x >= tiles) return;
  const int t0 = (tiles - 1 - x) * kMembers;
  int lim[kMembers];
  unsigned take = 0;
#pragma unroll
  for (int mi = 0; mi < kMembers; ++mi) {
    const int t = t0 + mi;
    lim[mi] = t < c.len ? c.n - c.len + t + 1 : 0;
    if (t < c.len) take |= 1u << mi;
  }
  mfma_tile<D, G>(sm, q, kc, vc, tables + static_cast<size_t>(s) * W, nullptr, W, lim, take,
                  c.r0 + t0, kvh, num_q_heads, num_kv_heads, num_blocks, scale_log2, 0, 0, 1,
                  out, lse);
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
  attend_range<T, D, G, 1, 2, false>(st, q, kc, vc, tables, W, s, row, kvh, num_q_heads,
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
    constexpr int kMembers = kMfmaRows / G;
    const int tiles_x = (a.max_q_len + kMembers - 1) / kMembers;
    const long long items = static_cast<long long>(tiles_x) * a.batch * a.hkv;
    const long long per = (items + kXcds - 1) / kXcds;
    hipLaunchKernelGGL((prefill_mfma_kernel<D, G>), dim3(static_cast<unsigned>(per * kXcds)),
                       dim3(kTileWaves * kWave), 0, stream, static_cast<const uint16_t*>(a.q),
                       static_cast<const uint16_t*>(a.kc), static_cast<const uint16_t*>(a.vc),
                       a.tables, a.W, a.cu_q, a.ctx, a.total_q, a.max_q_len, tiles_x, a.batch,
                       a.hq, a.hkv, a.nb, a.scale_log2, a.out, a.lse);
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
