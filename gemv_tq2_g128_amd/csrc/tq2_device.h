// Device helpers shared by the GEMV and GEMM translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq2 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Cache policy operand of a buffer load for data that one launch reads once
// (a weight streamed by the decode kernels): the non-temporal hint, so the
// stream is not kept in the caches at the expense of reused data (x).
constexpr int kStreamOnce = 2;

// Raw buffer resource over `bytes` bytes at `base`: a load whose per-lane
// offset (plus the instruction offset) reaches past the end returns zeros.
// The hardware range check does not include the scalar offset operand, so a
// variable offset that must be range-checked goes into the per-lane offset.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes),
                                           0x00020000);
}

// v_and_or_b32 with the mask in an SGPR (gfx9 VOP3 takes no literal).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(magic));
  return r;
}

// One DPP lane move of a float (lanes outside ROW_MASK read 0).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_move(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xF, false));
}

// Largest value over the wave (v >= 0): the quad permutes, the 8- and 16-lane
// mirrors and the row broadcasts of lanes 15 and 31 leave it in lane 63.
__device__ __forceinline__ float wave_max_nonneg(float v) {
  v = fmaxf(v, dpp_move<0xB1, 0xF>(v));
  v = fmaxf(v, dpp_move<0x4E, 0xF>(v));
  v = fmaxf(v, dpp_move<0x141, 0xF>(v));
  v = fmaxf(v, dpp_move<0x140, 0xF>(v));
  v = fmaxf(v, dpp_move<0x142, 0xA>(v));
  v = fmaxf(v, dpp_move<0x143, 0xC>(v));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

}  // namespace tq2
