// KV append: write new tokens' K/V into their cache blocks at an explicit
// start position (spindle, "Two bugs worth recording": append takes an
// explicit start position; the cache never infers or advances a length).
//
// One workgroup (one wavefront) per new token.  The token's sequence is found by
// counting the cu_new_tokens entries at or below its index; its position gives
// (block, slot) through the block table; then every KV head's D-element row is
// copied with 16-byte vector moves, bit-exact.  Out-of-range positions or block ids
// are never written: the token is skipped and an error bit is set.

#include "common.h"

PKV_DEFINE_ERROR_WORD(append)

#include "append_row.h"

namespace pkv {
namespace {

constexpr int kThreads = kWave;

__global__ __launch_bounds__(kThreads) void kv_append_kernel(
    uint4* __restrict__ kc, uint4* __restrict__ vc, const uint4* __restrict__ kn,
    const uint4* __restrict__ vn, const int32_t* __restrict__ tables, int W,
    const int32_t* __restrict__ start_pos, const int32_t* __restrict__ cu, int batch,
    int total, int num_kv_heads, int row_vecs, int num_blocks) {
  append_token(kc, vc, kn, vn, tables, W, start_pos, cu, batch, total, num_kv_heads, row_vecs,
               num_blocks, blockIdx.x, threadIdx.x, &g_pkv_error_word);
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int pkv_kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                             const int32_t* block_tables, int64_t bt_stride,
                             const int32_t* start_pos, const int32_t* cu_new_tokens,
                             int32_t batch, int32_t total_new, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int32_t num_blocks,
                             int32_t dtype, pkv_stream_t stream) {
  if (batch < 0 || total_new < 0) return PKV_ERR_SHAPE;
  if (total_new == 0) return PKV_OK;
  if (!k_cache || !v_cache || !k_new || !v_new || !block_tables || !start_pos || !cu_new_tokens)
    return PKV_ERR_NULL;
  const int eb = elem_bytes(dtype);
  if (eb == 0) return PKV_ERR_DTYPE;
  if (batch == 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size != kBlockTokens ||
      num_blocks <= 0 || bt_stride <= 0 || bt_stride > (1 << 26) ||
      (head_dim * eb) % 16 != 0)
    return PKV_ERR_SHAPE;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
    return PKV_ERR_ARG;
  hipLaunchKernelGGL(kv_append_kernel, dim3(total_new), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint4*>(k_cache),
                     static_cast<uint4*>(v_cache), static_cast<const uint4*>(k_new),
                     static_cast<const uint4*>(v_new), block_tables,
                     static_cast<int>(bt_stride), start_pos, cu_new_tokens, batch, total_new,
                     num_kv_heads, head_dim * eb / 16, num_blocks);
  return launch_status();
}
