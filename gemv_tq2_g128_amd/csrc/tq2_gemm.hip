// Batched ternary matmul on the CDNA4 matrix cores:
//     out[m, n] = residual[m, n] + sum_k x[m, k] * w[n, k].
//
// Prior art on the pages (oxibonsai-kernels 0.1.5, pipelines.rs,
// `MetalPipelines`, ternary section): v8 decodes each weight block once per
// M-tile; v9 drives the matrix units with f16-staged operands and f32
// accumulation; v10 stages the dequantised weight as binary16 -- exact, since
// code * d is +-d or 0 -- and double-buffers the K staging.  This kernel keeps
// those properties and lays the work out for gfx950:
//
//  * v_mfma_f32_16x16x32_f16, one wave per SIMD, 4 waves per block.  A block
//    owns an MT x (4*NW) output tile; each wave owns MT rows x NW columns.
//  * x (f32) is staged through LDS once per block per 256-wide K chunk,
//    converted to binary16 with round-to-nearest-even on the way in, double
//    buffered so the next chunk's global loads overlap the current MFMAs.
//  * Weights go straight from the SoA codes to MFMA operand registers: a lane
//    reads 16 code bytes (64 weights of one column) per chunk and decodes them
//    into exact binary16 (c - 1) * d with an AND-OR into the mantissa of a
//    binary16 pair, one packed FMA and one packed multiply.  Each weight is
//    decoded once per block and never touches LDS.
//  * LIMBS = 2 is the f32-class variant for small M: x = hi + lo with
//    hi = f16(x), lo = f16(x - hi); both parts hit the same exact weight
//    operand and accumulate in f32 (relative error of x about 2^-22).
//  * Blocks are numbered so that the N-tiles of the same M rows land on the
//    same XCD (the dispatcher deals block ids round-robin over 8 XCDs): x, at
//    4 bytes per element, is the costly operand to re-fetch, so an XCD's L2
//    serves its few x row-blocks to many weight column-blocks.
//
// K-chunk bookkeeping.  A chunk is 256 consecutive k (two 128-weight blocks).
// Lane l of a wave has column (l & 15) of its 16-column group and k-group
// g = l >> 4, covering chunk positions 64g .. 64g+63 (block 2c + (g >> 1)).
// MFMA step s (0..7) takes from every lane the 8 positions 64g + 8s .. +7; the
// A operand uses the same positions, so each step contracts 32 k's.
#include "tq2_internal.h"

namespace tq2 {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kChunk = 256;            // k per pipeline stage
constexpr int kLdsRow = kChunk + 8;    // binary16 per LDS row (16-byte pad vs bank conflicts)

__device__ __forceinline__ half2_t as_half2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

// Four binary16 pairs (8 weights) of one MFMA step from one code word.
// `word` holds the step's codes in fields r = 0..3 at bits 2r (first weight
// of pair r) and 2r + 16 (second weight).  (1024 + 4^r c) * 4^-r - (1024 *
// 4^-r + 1) = c - 1 exactly; times d stays exact (+-d or 0).
__device__ __forceinline__ half8_t decode_step(uint32_t word, half2_t d2) {
  half8_t b;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t mask = (3u << (2 * r)) | (3u << (2 * r + 16));
    const half2_t v = as_half2((word & mask) | 0x64006400u);
    const _Float16 sc = _Float16(1.0f / float(1 << (2 * r)));
    const _Float16 off = _Float16(-(1024.0f / float(1 << (2 * r)) + 1.0f));
    const half2_t scv = {sc, sc};
    const half2_t offv = {off, off};
    const half2_t val = (v * scv + offv) * d2;
    b[2 * r] = val[0];
    b[2 * r + 1] = val[1];
  }
  return b;
}

template <int MT, int NW, int LIMBS>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const uint32_t* __restrict__ codes,
                                                        const uint16_t* __restrict__ scales,
                                                        const float* __restrict__ x,
                                                        const float* __restrict__ residual,
                                                        float* __restrict__ out, int M, int N,
                                                        int K, int tiles_m, int tiles_n) {
  constexpr int RT = MT / 16;            // 16-row MFMA tiles per wave
  constexpr int CG = NW / 16;            // 16-column groups per wave
  constexpr int NT = 4 * NW;
  constexpr int AV = MT * (kChunk / 4) / kThreads;   // float4 A loads per thread per chunk
  static_assert(MT % 16 == 0 && NW % 16 == 0, "tile shape");
  static_assert((MT * (kChunk / 4)) % kThreads == 0, "A staging split");

  __shared__ _Float16 As[2][LIMBS][MT][kLdsRow];

  // XCD-aware tile order: block id b runs on XCD b % 8; give each XCD a
  // contiguous range of logical tiles (N-tiles of one M row-block adjacent).
  const int ntiles = tiles_m * tiles_n;
  int t = blockIdx.x;
  if ((ntiles & 7) == 0) t = (t & 7) * (ntiles >> 3) + (t >> 3);
  const int mt = t / tiles_n;
  const int nt = t - mt * tiles_n;
  const int m0 = mt * MT;
  const int n0 = nt * NT;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int KB = K >> 7;
  const int words_per_row = K >> 4;
  const int nchunks = (K + kChunk - 1) / kChunk;

  // ---- staging helpers -------------------------------------------------
  float4 areg[AV];
  auto load_a = [&](int c) {
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const int f = tid + kThreads * i;
      const int r = f >> 6;              // kChunk / 4 = 64 float4 per row
      const int c4 = f & 63;
      const int m = m0 + r;
      const int kk = c * kChunk + 4 * c4;
      if (m < M && kk < K)
        areg[i] = *reinterpret_cast<const float4*>(x + size_t(m) * K + kk);
      else
        areg[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const int f = tid + kThreads * i;
      const int r = f >> 6;
      const int c4 = f & 63;
      const float4 v = areg[i];
      half4_t h = {_Float16(v.x), _Float16(v.y), _Float16(v.z), _Float16(v.w)};
      *reinterpret_cast<half4_t*>(&As[buf][0][r][4 * c4]) = h;
      if constexpr (LIMBS == 2) {
        half4_t l = {_Float16(v.x - float(h[0])), _Float16(v.y - float(h[1])),
                     _Float16(v.z - float(h[2])), _Float16(v.w - float(h[3]))};
        *reinterpret_cast<half4_t*>(&As[buf][LIMBS - 1][r][4 * c4]) = l;
      }
    }
  };

  uint4 cw[CG];
  uint32_t dw[CG];
  auto load_w = [&](int c, uint4 (&cwo)[CG], uint32_t (&dwo)[CG]) {
#pragma unroll
    for (int j = 0; j < CG; ++j) {
      const int n = n0 + wave * NW + j * 16 + col;
      const int kk = c * kChunk + 64 * g;
      if (n < N && kk < K) {
        cwo[j] = *reinterpret_cast<const uint4*>(codes + size_t(n) * words_per_row +
                                                 (c * kChunk + 64 * g) / 16);
        const uint32_t d = scales[size_t(n) * KB + 2 * c + (g >> 1)];
        dwo[j] = d | (d << 16);
      } else {
        cwo[j] = make_uint4(0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u);
        dwo[j] = 0u;
      }
    }
  };

  floatx4_t acc[RT][CG];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < CG; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  // ---- prologue ---------------------------------------------------------
  load_a(0);
  load_w(0, cw, dw);
  store_a(0);
  __syncthreads();

  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    uint4 cwn[CG];
    uint32_t dwn[CG];
    const bool more = c + 1 < nchunks;
    if (more) {
      load_a(c + 1);
      load_w(c + 1, cwn, dwn);
    }

#pragma unroll
    for (int s = 0; s < 8; ++s) {
      half8_t bop[CG];
#pragma unroll
      for (int j = 0; j < CG; ++j) {
        const uint32_t words[4] = {cw[j].x, cw[j].y, cw[j].z, cw[j].w};
        uint32_t w = words[s >> 1];
        if (s & 1) w >>= 8;
        bop[j] = decode_step(w, as_half2(dw[j]));
      }
#pragma unroll
      for (int i = 0; i < RT; ++i) {
#pragma unroll
        for (int l = 0; l < LIMBS; ++l) {
          const half8_t aop =
              *reinterpret_cast<const half8_t*>(&As[buf][l][i * 16 + col][64 * g + 8 * s]);
#pragma unroll
          for (int j = 0; j < CG; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop[j], acc[i][j], 0, 0, 0);
        }
      }
    }

    if (more) {
      store_a(buf ^ 1);
#pragma unroll
      for (int j = 0; j < CG; ++j) {
        cw[j] = cwn[j];
        dw[j] = dwn[j];
      }
    }
    __syncthreads();
  }

  // ---- epilogue: D[row = 4g + e][col] of each 16x16 tile -----------------
#pragma unroll
  for (int i = 0; i < RT; ++i) {
#pragma unroll
    for (int j = 0; j < CG; ++j) {
      const int n = n0 + wave * NW + j * 16 + col;
      if (n >= N) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + i * 16 + 4 * g + e;
        if (m < M) {
          float v = acc[i][j][e];
          const size_t o = size_t(m) * N + n;
          if (residual) v = residual[o] + v;
          out[o] = v;
        }
      }
    }
  }
}

template <int MT, int NW, int LIMBS>
hipError_t launch_tile(const uint32_t* codes, const uint16_t* scales, const float* x,
                       const float* residual, float* out, int64_t m, int64_t n, int64_t k,
                       hipStream_t stream) {
  const int64_t tm = (m + MT - 1) / MT;
  const int64_t tn = (n + 4 * NW - 1) / (4 * NW);
  if (tm * tn > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int tiles_m = int(tm), tiles_n = int(tn);
  const dim3 grid(unsigned(tm * tn));
  hipLaunchKernelGGL((gemm_kernel<MT, NW, LIMBS>), grid, dim3(kThreads), 0, stream, codes,
                     scales, x, residual, out, int(m), int(n), int(k), tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int path, const uint8_t* soa, const float* x, const float* residual,
                       float* out, int64_t m, int64_t n, int64_t k, hipStream_t stream) {
  const uint32_t* codes = reinterpret_cast<const uint32_t*>(soa);
  const uint16_t* scales = reinterpret_cast<const uint16_t*>(soa + scales_offset(n, k));
  if (path == 1) return launch_tile<16, 16, 2>(codes, scales, x, residual, out, m, n, k, stream);
  if (m <= 32) return launch_tile<32, 16, 1>(codes, scales, x, residual, out, m, n, k, stream);
  if (m <= 64) return launch_tile<64, 16, 1>(codes, scales, x, residual, out, m, n, k, stream);
  if (m <= 128) return launch_tile<128, 16, 1>(codes, scales, x, residual, out, m, n, k, stream);
  return launch_tile<96, 48, 1>(codes, scales, x, residual, out, m, n, k, stream);
}

}  // namespace tq2
