// Device-side helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_internal.h"

namespace mla {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));

#define MLA_LDS __attribute__((address_space(3)))

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;

// Storage access: fp32 or bf16 elements, fp32 arithmetic.
__device__ __forceinline__ float ld(const float* p) { return *p; }
__device__ __forceinline__ float ld(const __bf16* p) { return static_cast<float>(*p); }
__device__ __forceinline__ void st(float* p, float v) { *p = v; }
__device__ __forceinline__ void st(__bf16* p, float v) { *p = static_cast<__bf16>(v); }

// Physical row index of logical token t of request b.
__device__ __forceinline__ size_t cache_row_index(const CacheView& c, int b, int t) {
  if (c.page_table == nullptr) return static_cast<size_t>(b) * c.max_len + t;
  const int page = c.page_table[static_cast<size_t>(b) * c.max_pages + t / c.page_size];
  return static_cast<size_t>(page) * c.page_size + (t % c.page_size);
}

// Byte address of logical token t of request b.
__device__ __forceinline__ const uint8_t* cache_row(const CacheView& c, int b, int t,
                                                    int row_bytes) {
  return c.data + cache_row_index(c, b, t) * row_bytes;
}

// Value of an OCP E4M3 byte (the low-bit cache), without its row scale.
__device__ __forceinline__ float ld_e4m3(const uint8_t* p) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(*p), 0);
}

// 16-byte direct-to-LDS load: lane l's 16 bytes land at lds_base +
// 16 * l (M0 holds the wave's base).  Issued as inline asm; the caller waits
// for it with an explicit s_waitcnt vmcnt(0) before the barrier that
// publishes the LDS contents.
__device__ __forceinline__ void load_to_lds16(const void* src, unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// v_permlane32_swap(v, v) yields, in every lane l, the pair
// (v[l % 32], v[l % 32 + 32]); combining the pair with a symmetric operation
// reduces over the two wave halves, bitwise identically in both halves.
__device__ __forceinline__ float halves_max(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, static_cast<unsigned>(r[0])),
               __builtin_bit_cast(float, static_cast<unsigned>(r[1])));
}
__device__ __forceinline__ float halves_sum(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, static_cast<unsigned>(r[0])) +
         __builtin_bit_cast(float, static_cast<unsigned>(r[1]));
}

}  // namespace mla
