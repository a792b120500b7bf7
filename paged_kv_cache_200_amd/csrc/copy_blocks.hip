// Copy-on-write block copy (spindle, "Paging": reference counts give
// copy-on-write forking).  Before a sequence writes into a block it shares,
// the host block manager hands it a fresh block; this kernel copies the old
// block's contents (every KV head, every slot, K and V, every layer) into it.
//
// Grid: (pair, layer).  A workgroup streams one block of one layer with
// 16-byte vector moves.  Ids outside [0, num_blocks) are skipped and flagged.

#include "common.h"

PKV_DEFINE_ERROR_WORD(copy)

namespace pkv {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(
    uint4* __restrict__ kc, uint4* __restrict__ vc, const int32_t* __restrict__ src,
    const int32_t* __restrict__ dst, int block_vecs, int num_blocks, int64_t layer_vecs) {
  const int i = blockIdx.x;
  const int layer = blockIdx.y;
  const int a = src[i];
  const int b = dst[i];
  if (static_cast<unsigned>(a) >= static_cast<unsigned>(num_blocks) ||
      static_cast<unsigned>(b) >= static_cast<unsigned>(num_blocks)) {
    if (threadIdx.x == 0 && layer == 0) PKV_FLAG_ERROR(PKV_DEVERR_BLOCK_ID);
    return;
  }
  const size_t base = static_cast<size_t>(layer) * layer_vecs;
  const uint4* ks = kc + base + static_cast<size_t>(a) * block_vecs;
  const uint4* vs = vc + base + static_cast<size_t>(a) * block_vecs;
  uint4* kd = kc + base + static_cast<size_t>(b) * block_vecs;
  uint4* vd = vc + base + static_cast<size_t>(b) * block_vecs;
  for (int j = threadIdx.x; j < block_vecs; j += kThreads) {
    kd[j] = ks[j];
    vd[j] = vs[j];
  }
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src,
                               const int32_t* dst, int32_t n, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int32_t num_blocks,
                               int32_t num_layers, int64_t layer_stride, int32_t dtype,
                               pkv_stream_t stream) {
  if (n < 0 || num_layers < 1) return PKV_ERR_SHAPE;
  if (n == 0) return PKV_OK;
  if (!k_cache || !v_cache || !src || !dst) return PKV_ERR_NULL;
  const int eb = elem_bytes(dtype);
  if (eb == 0) return PKV_ERR_DTYPE;
  if (num_kv_heads <= 0 || head_dim <= 0 || block_size != kBlockTokens || num_blocks <= 0 ||
      (head_dim * eb) % 16 != 0 || num_layers > 65535)
    return PKV_ERR_SHAPE;
  const int64_t block_elems = static_cast<int64_t>(num_kv_heads) * block_size * head_dim;
  if (num_layers > 1 && layer_stride < block_elems * num_blocks) return PKV_ERR_SHAPE;
  if (num_layers > 1 && (layer_stride * eb) % 16 != 0) return PKV_ERR_ARG;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_ARG;
  const int block_vecs = static_cast<int>(block_elems * eb / 16);
  const int64_t layer_vecs = num_layers > 1 ? layer_stride * eb / 16 : 0;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(n, num_layers), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint4*>(k_cache),
                     static_cast<uint4*>(v_cache), src, dst, block_vecs, num_blocks,
                     layer_vecs);
  return launch_status();
}
