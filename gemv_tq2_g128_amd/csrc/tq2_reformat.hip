// AoS -> SoA weight reformat (one pass per weight, off the per-call path),
// for TQ2_0_g128 and for the Q1_g128 sibling format.
//
// The pages feed the raw 34-byte blocks to a kernel-side reformat named
// `reformat_tq2_aos_to_soa` (oxibonsai-image 0.2.2, src/gpu.rs, doc of
// `blocks_as_bytes`) and keep the reformatted buffer resident for every later
// matmul (doc of `ternary_matmul_gpu`).  The target layout here is this
// library's own; it is described in tq2_internal.h.
#include "tq2_internal.h"

namespace tq2 {
namespace {

// Move the 2-bit field of t (t = 0..15, at bit 2t) to bit 2*(t>>1) + 16*(t&1)
// after mapping the reserved code 3 to code 1.
__device__ __forceinline__ uint32_t relayout_word(uint32_t w) {
  const uint32_t both = w & (w >> 1) & 0x55555555u;   // low bit of every field equal to 3
  w &= ~(both << 1);                                  // 3 -> 1
  uint32_t r = 0;
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const uint32_t c = (w >> (2 * t)) & 3u;
    r |= c << (2 * (t >> 1) + 16 * (t & 1));
  }
  return r;
}

// One thread per 34-byte block.  The block is read as 17 half-words (blocks
// start at even byte offsets) and written as 32 code bytes plus one scale.
__global__ __launch_bounds__(256) void reformat_kernel(const uint16_t* __restrict__ aos,
                                                       uint32_t* __restrict__ codes,
                                                       uint16_t* __restrict__ scales,
                                                       int64_t nblocks) {
  const int64_t b = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const uint16_t* src = aos + b * (kBlockBytes / 2);
  uint32_t words[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t lo = src[2 * i], hi = src[2 * i + 1];
    words[i] = relayout_word(lo | (hi << 16));
  }
  uint4* dst = reinterpret_cast<uint4*>(codes + b * 8);
  dst[0] = make_uint4(words[0], words[1], words[2], words[3]);
  dst[1] = make_uint4(words[4], words[5], words[6], words[7]);
  scales[b] = src[16];
}

// Q1_g128: move bit t of a 32-weight word (t = 0..31) to bit
// (t >> 1) + 16*(t & 1): even weights to the low half-word, odd to the high.
__device__ __forceinline__ uint32_t relayout_word_q1(uint32_t w) {
  uint32_t r = 0;
#pragma unroll
  for (int t = 0; t < 32; ++t) r |= ((w >> t) & 1u) << ((t >> 1) + 16 * (t & 1));
  return r;
}

// One thread per 18-byte Q1 block (nine half-words, even byte offsets).
__global__ __launch_bounds__(256) void reformat_q1_kernel(const uint16_t* __restrict__ aos,
                                                          uint32_t* __restrict__ bits,
                                                          uint16_t* __restrict__ scales,
                                                          int64_t nblocks) {
  const int64_t b = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const uint16_t* src = aos + b * (kQ1BlockBytes / 2);
  uint32_t words[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = src[2 * i], hi = src[2 * i + 1];
    words[i] = relayout_word_q1(lo | (hi << 16));
  }
  reinterpret_cast<uint4*>(bits)[b] = make_uint4(words[0], words[1], words[2], words[3]);
  scales[b] = src[8];
}

}  // namespace

hipError_t launch_reformat_q1(const uint16_t* aos, uint8_t* soa, int64_t n, int64_t k,
                              hipStream_t stream) {
  const int64_t nblocks = n * (k / kBlockWeights);
  const int64_t grid = (nblocks + 255) / 256;
  uint32_t* bits = reinterpret_cast<uint32_t*>(soa);
  uint16_t* scales = reinterpret_cast<uint16_t*>(soa + scales_offset(Fmt::kQ1, n, k));
  hipLaunchKernelGGL(reformat_q1_kernel, dim3(unsigned(grid)), dim3(256), 0, stream, aos, bits,
                     scales, nblocks);
  return hipGetLastError();
}

hipError_t launch_reformat(const uint16_t* aos, uint8_t* soa, int64_t n, int64_t k,
                           hipStream_t stream) {
  const int64_t nblocks = n * (k / kBlockWeights);
  const int64_t grid = (nblocks + 255) / 256;
  uint32_t* codes = reinterpret_cast<uint32_t*>(soa);
  uint16_t* scales = reinterpret_cast<uint16_t*>(soa + scales_offset(n, k));
  hipLaunchKernelGGL(reformat_kernel, dim3(unsigned(grid)), dim3(256), 0, stream, aos, codes,
                     scales, nblocks);
  return hipGetLastError();
}

}  // namespace tq2
