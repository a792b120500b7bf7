// Internal helpers shared by the HIP sources of libpkv (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

constexpr int kBlockTokens = 16;  // tokens per cache block (spindle, "Paging")
constexpr int kWave = 64;         // CDNA wavefront width
constexpr float kLn2 = 0.69314718055994530942f;
// Online softmax: the running max (log2 units) is raised only when a score exceeds it
// by more than this, so the rescale stays off the common path and every exponential
// stays <= 2^8.
constexpr float kLazyMaxSlack = 8.0f;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// bfloat16 halves of a packed 32-bit word, widened exactly to float32.
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// DPP lane moves (all 64 lanes must be active).
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_amdgcn_update_dpp(0.0f, x, kCtrl, 0xf, 0xf, false);
}
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <- lane 7-i within each 8 lanes

// Sum over each aligned group of 8 lanes; every lane of the group gets the sum.
__device__ __forceinline__ float group8_sum(float x) {
  x += dpp_mov<kDppQuadXor1>(x);
  x += dpp_mov<kDppQuadXor2>(x);
  x += dpp_mov<kDppRowHalfMirror>(x);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Scores are kept in log2 units: scale * log2(e), rounded once to float32.
inline float scale_to_log2(float scale) {
  return static_cast<float>(static_cast<double>(scale) * 1.4426950408889634074);
}

inline int elem_bytes(int32_t dtype) {
  return dtype == PKV_F32 ? 4 : dtype == PKV_BF16 ? 2 : 0;
}

}  // namespace pkv

// Each translation unit keeps its own device error word and exposes a reader.
extern "C" int pkv_internal_take_error_decode(int32_t* flags);
extern "C" int pkv_internal_take_error_append(int32_t* flags);
extern "C" int pkv_internal_take_error_copy(int32_t* flags);
extern "C" int pkv_internal_take_error_prefill(int32_t* flags);

#define PKV_DEFINE_ERROR_WORD(NAME)                                                  \
  namespace {                                                                        \
  __device__ unsigned int g_pkv_error_word;                                          \
  }                                                                                  \
  extern "C" int pkv_internal_take_error_##NAME(int32_t* flags) {                    \
    unsigned int v = 0, zero = 0;                                                    \
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_pkv_error_word), sizeof(v), 0,          \
                            hipMemcpyDeviceToHost) != hipSuccess)                    \
      return PKV_ERR_DEVICE;                                                         \
    if (v && hipMemcpyToSymbol(HIP_SYMBOL(g_pkv_error_word), &zero, sizeof(zero), 0, \
                               hipMemcpyHostToDevice) != hipSuccess)                 \
      return PKV_ERR_DEVICE;                                                         \
    *flags |= static_cast<int32_t>(v);                                               \
    return PKV_OK;                                                                   \
  }

#define PKV_FLAG_ERROR(bits) atomicOr(&g_pkv_error_word, static_cast<unsigned int>(bits))
