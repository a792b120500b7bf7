// One decode step's layers issued by one host call: each layer is the planned
// append + decode call on that layer's slice of stacked tensors (spindle,
// "Paging": every layer attends over its own cache through the step's shared
// block tables).  Host code only; the kernels are those of that call.

#include "pkv.h"

extern "C" int pkv_append_paged_decode_planned_layers(
    int32_t num_layers, float* out, int64_t out_layer_stride, float* lse,
    int64_t lse_layer_stride, const void* q, int64_t q_layer_stride, void* k_cache,
    void* v_cache, int64_t cache_layer_stride, const void* k_new, const void* v_new,
    int64_t new_layer_stride, const int32_t* block_tables, int64_t bt_stride,
    const int32_t* start_pos, const int32_t* cu_new_tokens, int32_t total_new,
    const int32_t* context_lens, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_context_len,
    float scale, int32_t partition_size, void* workspace, size_t workspace_bytes, int32_t dtype,
    pkv_stream_t stream) {
  if (num_layers < 0 || out_layer_stride < 0 || lse_layer_stride < 0 || q_layer_stride < 0 ||
      cache_layer_stride < 0 || new_layer_stride < 0)
    return PKV_ERR_SHAPE;
  if (dtype != PKV_F32 && dtype != PKV_BF16) return PKV_ERR_DTYPE;
  // strides count elements of the cache dtype (float for out and lse)
  const int64_t eb = dtype == PKV_F32 ? 4 : 2;
  for (int32_t l = 0; l < num_layers; ++l) {
    const int64_t L = l;
    const int st = pkv_append_paged_decode_planned(
        out != nullptr ? out + L * out_layer_stride : nullptr,
        lse != nullptr ? lse + L * lse_layer_stride : nullptr,
        static_cast<const char*>(q) + L * q_layer_stride * eb,
        static_cast<char*>(k_cache) + L * cache_layer_stride * eb,
        static_cast<char*>(v_cache) + L * cache_layer_stride * eb,
        k_new != nullptr ? static_cast<const char*>(k_new) + L * new_layer_stride * eb : nullptr,
        v_new != nullptr ? static_cast<const char*>(v_new) + L * new_layer_stride * eb : nullptr,
        block_tables, bt_stride, start_pos, cu_new_tokens, total_new, context_lens, batch,
        num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_context_len, scale,
        partition_size, workspace, workspace_bytes, dtype, stream);
    if (st != PKV_OK) return st;
  }
  return PKV_OK;
}
