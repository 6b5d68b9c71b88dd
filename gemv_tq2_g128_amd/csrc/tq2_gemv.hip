// Decode GEMV (M = 1): out[n] = residual[n] + sum_k x[k] * w[n, k].
//
// The pages' decode kernel is `gemv_tq2_g128_v1` (oxibonsai-kernels 0.1.5,
// pipelines.rs, `MetalPipelines`, ternary section); its source is not on the
// pages.  The optional fused residual follows the `gemv_q1_g128_v7_residual`
// entry of the same table.  This kernel is designed for gfx950 on its own:
//
//  * HBM stream: every lane reads 16 contiguous code bytes (64 weights) of a
//    row per load, lanes of a row read consecutive 16-byte chunks, so a wave
//    instruction moves whole 64-byte segments; all of a block's code and
//    scale loads are issued before any arithmetic.
//  * x stays in registers: the 4 waves of a block split K into quarters and a
//    lane keeps the 64 x values of its chunk for every row it visits, so x
//    is read from L2 once per block, not once per row.
//  * Arithmetic is f32: a 2-bit code c (stored canonical, 0..2) becomes the
//    float c - 1 exactly via the bit pattern 0x4B000000 | c (= 2^23 + c)
//    minus 2^23 + 1; each lane sums its 64 products in f32, scales the chunk
//    sum by the block's d once, and the per-row partials are reduced with
//    cross-lane shuffles and a 4-wave LDS step.
#include "tq2_internal.h"

namespace tq2 {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float code_minus_one(uint32_t c) {
  return __uint_as_float(0x4B000000u | c) - 8388609.0f;
}

// Sum over the 64 weights of one 16-byte chunk of  x[k] * (code(k) - 1).
__device__ __forceinline__ float chunk_dot(const uint4& cw, const float (&xv)[64]) {
  const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t w = words[q];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      s0 = fmaf(xv[16 * q + 2 * p], code_minus_one((w >> (2 * p)) & 3u), s0);
      s1 = fmaf(xv[16 * q + 2 * p + 1], code_minus_one((w >> (2 * p + 16)) & 3u), s1);
    }
  }
  return s0 + s1;
}

// RPW rows per wave pass (64 / RPW lanes per row), PASSES passes per block.
template <int RPW, int PASSES>
__global__ __launch_bounds__(kThreads) void gemv_kernel(const uint32_t* __restrict__ codes,
                                                        const uint16_t* __restrict__ scales,
                                                        const float* __restrict__ x,
                                                        const float* __restrict__ residual,
                                                        float* __restrict__ out, int n_rows,
                                                        int k) {
  constexpr int LPR = 64 / RPW;
  constexpr int R = RPW * PASSES;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int rs = lane / LPR;
  const int lc = lane % LPR;
  const int chunks = k >> 6;
  const int kb_count = k >> 7;
  const int words_per_row = k >> 4;
  const int row0 = blockIdx.x * R;

  float acc[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) acc[p] = 0.f;

  for (int seg = 0; seg < chunks; seg += 4 * LPR) {
    const int j = seg + wave * LPR + lc;
    const bool active = j < chunks;
    uint4 cw[PASSES];
    float dv[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = row0 + p * RPW + rs;
      if (active && row < n_rows) {
        cw[p] = *reinterpret_cast<const uint4*>(codes + size_t(row) * words_per_row + 4 * j);
        const _Float16 d = __builtin_bit_cast(_Float16, scales[size_t(row) * kb_count + (j >> 1)]);
        dv[p] = float(d);
      } else {
        cw[p] = make_uint4(0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u);
        dv[p] = 0.f;
      }
    }
    float xv[64];
    if (active) {
      const float4* xp = reinterpret_cast<const float4*>(x + 64 * j);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float4 v = xp[i];
        xv[4 * i] = v.x;
        xv[4 * i + 1] = v.y;
        xv[4 * i + 2] = v.z;
        xv[4 * i + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 64; ++i) xv[i] = 0.f;
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) acc[p] = fmaf(chunk_dot(cw[p], xv), dv[p], acc[p]);
  }

#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) acc[p] += __shfl_xor(acc[p], off, 64);
  }

  __shared__ float red[4][R];
  if (lc == 0) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) red[wave][p * RPW + rs] = acc[p];
  }
  __syncthreads();
  if (threadIdx.x < R) {
    const int row = row0 + threadIdx.x;
    if (row < n_rows) {
      float v = (red[0][threadIdx.x] + red[1][threadIdx.x]) +
                (red[2][threadIdx.x] + red[3][threadIdx.x]);
      if (residual) v = residual[row] + v;
      out[row] = v;
    }
  }
}

template <int RPW>
hipError_t launch_rpw(int passes, const uint32_t* codes, const uint16_t* scales, const float* x,
                      const float* residual, float* out, int n, int k, hipStream_t stream) {
  const int rows_per_block = RPW * passes;
  const dim3 grid((n + rows_per_block - 1) / rows_per_block);
  switch (passes) {
    case 1:
      hipLaunchKernelGGL((gemv_kernel<RPW, 1>), grid, dim3(kThreads), 0, stream, codes, scales,
                         x, residual, out, n, k);
      break;
    case 2:
      hipLaunchKernelGGL((gemv_kernel<RPW, 2>), grid, dim3(kThreads), 0, stream, codes, scales,
                         x, residual, out, n, k);
      break;
    default:
      hipLaunchKernelGGL((gemv_kernel<RPW, 4>), grid, dim3(kThreads), 0, stream, codes, scales,
                         x, residual, out, n, k);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const uint8_t* soa, const float* x, const float* residual, float* out,
                       int64_t n, int64_t k, hipStream_t stream) {
  const uint32_t* codes = reinterpret_cast<const uint32_t*>(soa);
  const uint16_t* scales = reinterpret_cast<const uint16_t*>(soa + scales_offset(n, k));
  // Lanes per row: enough 16-byte chunks for one quarter of K, a power of two, <= 64.
  const int64_t chunks = k / 64;
  const int64_t quarter = (chunks + 3) / 4;
  int lpr = 1;
  while (lpr < quarter && lpr < 64) lpr <<= 1;
  const int rpw = 64 / lpr;
  // Passes: keep at least ~512 blocks in flight where the row count allows.
  int passes = 4;
  while (passes > 1 && (n + int64_t(rpw) * passes - 1) / (int64_t(rpw) * passes) < 512) passes >>= 1;
  const int ni = int(n), ki = int(k);
  switch (rpw) {
    case 64: return launch_rpw<64>(passes, codes, scales, x, residual, out, ni, ki, stream);
    case 32: return launch_rpw<32>(passes, codes, scales, x, residual, out, ni, ki, stream);
    case 16: return launch_rpw<16>(passes, codes, scales, x, residual, out, ni, ki, stream);
    case 8: return launch_rpw<8>(passes, codes, scales, x, residual, out, ni, ki, stream);
    case 4: return launch_rpw<4>(passes, codes, scales, x, residual, out, ni, ki, stream);
    case 2: return launch_rpw<2>(passes, codes, scales, x, residual, out, ni, ki, stream);
    default: return launch_rpw<1>(passes, codes, scales, x, residual, out, ni, ki, stream);
  }
}

}  // namespace tq2
