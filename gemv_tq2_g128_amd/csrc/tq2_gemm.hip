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
// v_and_or_b32 with the mask in an SGPR and the constant in a VGPR (gfx9 VOP3
// instructions take no literal operand).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(magic));
  return r;
}

// Four binary16 pairs (8 weights) of one MFMA step from one code word.
// `word` holds the step's codes in fields r = 0..3 at bits 2r (first weight
// of pair r) and 2r + 16 (second weight).  (1024 + 4^r c) * 4^-r - (1024 *
// 4^-r + 1) = c - 1 exactly; times d stays exact (+-d or 0).
__device__ __forceinline__ half8_t decode_step(uint32_t word, half2_t d2, uint32_t magic) {
  half8_t b;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t mask = (3u << (2 * r)) | (3u << (2 * r + 16));
    const half2_t v = as_half2(and_or(word, mask, magic));
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

// Wait for this wave's LDS accesses, then join the workgroup barrier.  The
// asm's memory clobber keeps the compiler from moving memory accesses across
// it; unlike __syncthreads() it leaves the wave's global loads in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Raw buffer resource over `bytes` bytes at `base`: loads past the end
// return zero, loads take a 32-bit per-lane offset plus a scalar offset.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes),
                                           0x00020000);
}

// Block tile MT x (WN*NW); WN waves split the columns, WK waves split each
// 256-wide chunk's eight MFMA steps (their partial sums meet in LDS at the
// end).  Each wave owns MT rows x NW columns of the tile.
template <int MT, int NW, int WN, int WK, int LIMBS>
__global__ __launch_bounds__(64 * WN * WK) void gemm_kernel(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales,
                                                            const float* __restrict__ x,
                                                            const float* __restrict__ residual,
                                                            float* __restrict__ out, int M, int N,
                                                            int K, int tiles_m, int tiles_n) {
  constexpr int THREADS = 64 * WN * WK;
  constexpr int RT = MT / 16;            // 16-row MFMA tiles per wave
  constexpr int CG = NW / 16;            // 16-column groups per wave
  constexpr int NT = WN * NW;
  constexpr int STEPS = 8 / WK;          // MFMA k-steps per wave per chunk
  constexpr int QW = 4 / WK;             // code dwords per lane per chunk
  constexpr int AV = MT * (kChunk / 4) / THREADS;   // float4 A loads per thread per chunk
  static_assert(MT % 16 == 0 && NW % 16 == 0, "tile shape");
  static_assert(WK == 1 || WK == 2, "k split");
  static_assert((MT * (kChunk / 4)) % THREADS == 0, "A staging split");

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
  const int wn = wave % WN;              // column share
  const int wk = wave / WN;              // share of the chunk's steps
  const int lane = tid & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int KB = K >> 7;
  typedef uint32_t codes_t[QW];
  const int nchunks = (K + kChunk - 1) / kChunk;

  // x rows m0 .. m0+MT-1 (rows past M read as zero).
  const rsrc_t rx = make_rsrc(x + size_t(m0) * K, uint32_t(min(MT, M - m0)) * uint32_t(K) * 4u);
  const rsrc_t rc = make_rsrc(codes, uint32_t(N) * uint32_t(K / 4));
  const rsrc_t rs = make_rsrc(scales, uint32_t(N) * uint32_t(KB) * 2u);

  // Per-thread byte offsets, fixed for the whole K loop; a chunk, an A row
  // step and a column group add scalar offsets.  Columns past N read as zero
  // codes and zero scales.
  const uint32_t aoff = uint32_t(tid >> 6) * uint32_t(K) * 4u + 16u * uint32_t(tid & 63);
  constexpr int AROWS = THREADS / 64;    // A rows staged per load instruction

  auto load_a = [&](int c, float4 (&areg)[AV]) {
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(
          rx, aoff, i * AROWS * K * 4 + c * kChunk * 4, 0);
      areg[i] = __builtin_bit_cast(float4, v);
    }
  };
  auto store_a = [&](int buf, const float4 (&areg)[AV]) {
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const int f = tid + THREADS * i;
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

  // Weight loads of chunk c straight into registers: each lane takes the
  // QW code dwords of its column and k-group that this wave's steps use, and
  // the raw binary16 scale of the block they fall in.  Columns past N read as
  // zero codes and zero scales.
  const uint32_t nl = uint32_t(n0 + wn * NW + col);
  const uint32_t code_voff = nl * uint32_t(K / 4) + 16u * uint32_t(g) + 4u * QW * uint32_t(wk);
  const uint32_t scale_voff = (nl * uint32_t(KB) + uint32_t(g >> 1)) * 2u;
  auto load_w = [&](int c, codes_t (&cw)[CG], _Float16 (&dsc)[CG]) {
#pragma unroll
    for (int j = 0; j < CG; ++j) {
      if constexpr (QW == 4) {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rc, code_voff,
                                                                j * 16 * (K / 4) + c * 64, 0);
        cw[j][0] = v[0]; cw[j][1] = v[1]; cw[j][2] = v[2]; cw[j][3] = v[3];
      } else {
        const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rc, code_voff,
                                                               j * 16 * (K / 4) + c * 64, 0);
        cw[j][0] = v[0]; cw[j][1] = v[1];
      }
      dsc[j] = __builtin_bit_cast(
          _Float16, __builtin_amdgcn_raw_buffer_load_b16(rs, scale_voff, j * 16 * KB * 2 + c * 4, 0));
    }
  };

  floatx4_t acc[RT][CG];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < CG; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  const uint32_t magic = 0x64006400u;     // binary16 pair (1024, 1024)
  // Operands of one MFMA step: A fragments from LDS, B fragments decoded
  // from the code words.
  auto load_afrags = [&](int buf, int s, half8_t (&a)[RT][LIMBS]) {
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int l = 0; l < LIMBS; ++l)
        a[i][l] = *reinterpret_cast<const half8_t*>(&As[buf][l][i * 16 + col][64 * g + 8 * s]);
  };
  auto decode_bfrags = [&](int ss, const codes_t (&cw)[CG], const half2_t (&d2)[CG],
                           half8_t (&b)[CG]) {
#pragma unroll
    for (int j = 0; j < CG; ++j) {
      uint32_t w = cw[j][ss >> 1];
      if (ss & 1) w >>= 8;
      b[j] = decode_step(w, d2[j], magic);
    }
  };
  auto mfmas = [&](const half8_t (&a)[RT][LIMBS], const half8_t (&b)[CG]) {
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int l = 0; l < LIMBS; ++l)
#pragma unroll
        for (int j = 0; j < CG; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b[j], a[i][l], acc[i][j], 0, 0, 0);
  };
  // Ask the scheduler to interleave one step's MFMAs with the next step's
  // operand work: per MFMA about VALU/MFMA decode instructions and an LDS
  // read every few MFMAs, instead of long runs of either.
  constexpr int NMFMA = RT * LIMBS * CG;
  constexpr int NDSR = RT * LIMBS;
  auto interleave = [&]() {
#pragma unroll
    for (int q = 0; q < NMFMA; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // one MFMA
      if (q % ((NMFMA + NDSR - 1) / NDSR) == 0)
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);        // one LDS read
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);          // up to three VALU
    }
  };

  auto compute = [&](int c, int buf, const codes_t (&cw)[CG], const _Float16 (&dsc)[CG]) {
    // binary16 pair (d, d), or (0, 0) where k runs past K in the last chunk.
    const bool live = c * kChunk + 64 * g < K;
    half2_t dw[CG];
#pragma unroll
    for (int j = 0; j < CG; ++j) {
      const _Float16 d = live ? dsc[j] : _Float16(0.0f);
      dw[j] = half2_t{d, d};
    }
    half8_t a0[RT][LIMBS], a1[RT][LIMBS], b0[CG], b1[CG];
    load_afrags(buf, wk * STEPS, a0);
    decode_bfrags(0, cw, dw, b0);
#pragma unroll
    for (int ss = 0; ss < STEPS; ++ss) {
      const int s = wk * STEPS + ss;     // chunk step: k = 64g + 8s .. +7
      if ((ss & 1) == 0) {
        if (ss + 1 < STEPS) {
          load_afrags(buf, s + 1, a1);
          decode_bfrags(ss + 1, cw, dw, b1);
        }
        mfmas(a0, b0);
      } else {
        if (ss + 1 < STEPS) {
          load_afrags(buf, s + 1, a0);
          decode_bfrags(ss + 1, cw, dw, b0);
        }
        mfmas(a1, b1);
      }
      interleave();
      // Keep the next step's operand loads inside this step's region so
      // their latency hides behind this step's MFMAs.
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- software pipeline -------------------------------------------------
  // Iteration c computes chunk c from A buffer c % 2 and weight register set
  // c % 2.  At its start it converts and stores x chunk c + 1 (loaded during
  // iteration c - 1) and issues the loads of x chunk c + 2; after its MFMAs it
  // loads weight chunk c + 2 into the register set it has just used.  Every
  // load therefore has a whole iteration to land.  The loads are issued even
  // past the last chunk (the buffer resources return zeros out of range, and
  // the values are never used) so that every iteration has the same number
  // of loads in flight and the compiler's wait counts stay exact.  The
  // closing barrier only waits for this wave's LDS stores (a plain
  // s_barrier: __syncthreads()'s fence would also drain the loads in flight).
  float4 areg[AV];
  codes_t cw0[CG], cw1[CG];
  _Float16 dr0[CG], dr1[CG];
  // The loop starts at c = -2 (the first two passes only fill the pipeline)
  // and always runs both passes of a pair (a pass past the last chunk only
  // issues loads), so every pass issues the same loads in the same place and
  // the wait counts the compiler derives hold on every path through the loop.
  auto iteration = [&](int c, codes_t (&cw)[CG], _Float16 (&dsc)[CG]) {
    if (c + 1 >= 0 && c + 1 < nchunks) store_a((c + 1) & 1, areg);
    load_a(c + 2, areg);
    if (c >= 0 && c < nchunks) compute(c, c & 1, cw, dsc);
    load_w(c + 2, cw, dsc);
    lds_barrier();
  };
  for (int c = -2; c < nchunks; c += 2) {
    iteration(c, cw0, dr0);
    iteration(c + 1, cw1, dr1);
  }

  // ---- K-split reduction: the wk = 1 waves hand their sums to wk = 0 -----
  if constexpr (WK == 2) {
    float* red = reinterpret_cast<float*>(&As[0][0][0][0]);
    static_assert(WN * RT * CG * 4 * 64 * 4 <= sizeof(As), "reduction buffer");
    if (wk == 1) {
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < CG; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            red[(((wn * RT + i) * CG + j) * 4 + e) * 64 + lane] = acc[i][j][e];
    }
    __syncthreads();
    if (wk == 1) return;
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int j = 0; j < CG; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[i][j][e] += red[(((wn * RT + i) * CG + j) * 4 + e) * 64 + lane];
  }

  // ---- epilogue ------------------------------------------------------------
  // The weight operand is the MFMA's first (row) operand, so each 16x16
  // result holds D[n = 4g + e][m = col]: a lane owns four consecutive output
  // columns of one row and writes them (and reads the residual) as one
  // 16-byte access when the row pitch allows it.
  const bool vec = (N & 3) == 0;
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    const int m = m0 + i * 16 + col;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < CG; ++j) {
      const int n = n0 + wn * NW + j * 16 + 4 * g;
      const size_t o = size_t(m) * N + n;
      if (vec && n + 3 < N) {
        float4 v = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        if (residual) {
          const float4 r = *reinterpret_cast<const float4*>(residual + o);
          v = make_float4(r.x + v.x, r.y + v.y, r.z + v.z, r.w + v.w);
        }
        *reinterpret_cast<float4*>(out + o) = v;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (n + e < N) {
            float v = acc[i][j][e];
            if (residual) v = residual[o + e] + v;
            out[o + e] = v;
          }
        }
      }
    }
  }
}

template <int MT, int NW, int WN, int WK, int LIMBS>
hipError_t launch_tile(const uint8_t* soa, const float* x, const float* residual, float* out,
                       int64_t m, int64_t n, int64_t k, hipStream_t stream) {
  const int64_t tm = (m + MT - 1) / MT;
  const int64_t tn = (n + WN * NW - 1) / (WN * NW);
  if (tm * tn > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int tiles_m = int(tm), tiles_n = int(tn);
  const dim3 grid(unsigned(tm * tn));
  hipLaunchKernelGGL((gemm_kernel<MT, NW, WN, WK, LIMBS>), grid, dim3(64 * WN * WK), 0, stream,
                     soa, soa + scales_offset(n, k), x, residual, out, int(m), int(n), int(k),
                     tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int path, const uint8_t* soa, const float* x, const float* residual,
                       float* out, int64_t m, int64_t n, int64_t k, hipStream_t stream) {
  if (path == 1) return launch_tile<16, 16, 4, 2, 2>(soa, x, residual, out, m, n, k, stream);
  if (m <= 32) return launch_tile<32, 16, 4, 2, 1>(soa, x, residual, out, m, n, k, stream);
  if (m <= 64) return launch_tile<64, 16, 4, 2, 1>(soa, x, residual, out, m, n, k, stream);
  if (m <= 128) return launch_tile<128, 16, 4, 2, 1>(soa, x, residual, out, m, n, k, stream);
  return launch_tile<96, 48, 4, 2, 1>(soa, x, residual, out, m, n, k, stream);
}

}  // namespace tq2
