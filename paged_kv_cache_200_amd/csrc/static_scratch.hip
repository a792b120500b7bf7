// The decode step for callers that cannot allocate device memory (graph capture, serving
// loops, harnesses that forbid hipMalloc): pkv_append_paged_decode with its workspace in a
// static device array of this file, one per GPU.  The array lives in a code object of its
// own, apart from the kernels, which take its address as their workspace argument.

#include <mutex>

#include "common.h"

namespace {

// Host code never uses the array's name as an address (on the host it names a stand-in,
// not device memory): the device address comes from hipGetSymbolAddress, once per device,
// with that device current.
static __device__ __align__(256) unsigned char scratch[PKV_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up

int scratch_of_current_device(void** ptr) {
  int device = -1;
  if (hipGetDevice(&device) != hipSuccess || device < 0 || device >= kMaxDevices)
    return PKV_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[device] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return PKV_ERR_DEVICE;
    g_scratch_ptr[device] = p;
  }
  *ptr = g_scratch_ptr[device];
  return PKV_OK;
}

}  // namespace

extern "C" int pkv_append_paged_decode_static(
    float* out, float* lse, const void* q, void* k_cache, void* v_cache, const void* k_new,
    const void* v_new, const int32_t* block_tables, int64_t bt_stride, const int32_t* start_pos,
    const int32_t* cu_new_tokens, int32_t total_new, const int32_t* context_lens, int32_t batch,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_context_len, float scale, int32_t partition_size,
    int32_t dtype, pkv_stream_t stream) {
  if (batch < 0 || num_q_heads <= 0 || max_context_len < 0) return PKV_ERR_SHAPE;
  const size_t need = pkv_decode_workspace_bytes(batch, num_q_heads, head_dim, max_context_len,
                                                 partition_size);
  if (need > PKV_STATIC_SCRATCH_BYTES) return PKV_ERR_SCRATCH;
  void* ws = nullptr;
  const int st = scratch_of_current_device(&ws);
  if (st != PKV_OK) return st;
  return pkv_append_paged_decode(out, lse, q, k_cache, v_cache, k_new, v_new, block_tables,
                                 bt_stride, start_pos, cu_new_tokens, total_new, context_lens,
                                 batch, num_q_heads, num_kv_heads, head_dim, block_size,
                                 num_blocks, max_context_len, scale, partition_size, ws,
                                 PKV_STATIC_SCRATCH_BYTES, dtype, stream);
}
