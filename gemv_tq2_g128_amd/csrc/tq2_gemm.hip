// Batched ternary matmul on the CDNA4 matrix cores:
//     out[m, n] = residual[m, n] + sum_k x[m, k] * w[n, k].
//
// Prior art on the pages (oxibonsai-kernels 0.1.5, pipelines.rs,
// `MetalPipelines`, ternary section): v8 decodes each weight block once per
// M-tile; v9 drives the matrix units with f16-staged operands and f32
// accumulation; v10 stages the dequantised weight as binary16 -- exact, since
// code * d is +-d or 0 -- and double-buffers the K staging.  These kernels
// keep those properties and lay the work out for gfx950:
//
//  * v_mfma_f32_16x16x32_f16 with the weight as the first operand, 64-wide
//    waves, 8 waves per block (two per SIMD).  Each wave owns MT rows x NW
//    columns of the block tile and half of the MFMA steps of each 256-wide K
//    chunk; the two halves' partial sums meet in LDS at the end.
//  * x (f32) is loaded a chunk ahead into registers, converted to binary16
//    with round-to-nearest-even and stored into a double-buffered LDS tile.
//  * Weights go from the SoA code words straight into MFMA operand registers:
//    one AND-OR into the mantissa of a binary16 pair, one packed FMA and one
//    packed multiply give the exact binary16 (c - 1) * d of two weights.
//    Each weight is decoded once per block and never touches LDS.
//  * LIMBS = 2 (small M) splits x = hi + lo into two binary16 parts that hit
//    the same exact weight operand: f32-class accuracy (about 2^-22).
//  * gemm_pp_kernel (M > 128) runs its two wave groups half a chunk apart:
//    one group issues MFMAs while the other decodes, converts and loads.
//  * gemm_sp_kernel (16 < M <= 128) splits the waves by role instead: x
//    waves only stream and convert x, MFMA waves only decode and multiply.
//  * gemm_kernel serves tq2_gemm_precise beyond M = 16 (x = hi + lo).
//  * SWIGLU (the ternary counterpart of `fused_gate_up_swiglu_gemm_q1` in the
//    same table): half of the block's waves take gate-weight columns and the
//    other half the same columns of the up weight, on the same x tile; the
//    epilogue meets each pair in LDS and stores silu(g) * u, silu(z) =
//    z / (1 + e^-z).  Neither projection goes to memory.
//  * F = Fmt::kQ1 runs the same kernels on Q1_g128 (1-bit) weights (the
//    pages' `gemm_q1_g128_v7` / `_residual` / `fused_gate_up_swiglu_gemm_q1`):
//    a lane's word holds four steps' bits; shifting a pair's two bits onto
//    the binary16 sign positions and OR-ing |d| gives the exact pair
//    (+-|d|, +-|d|) in two instructions (the word is complemented once per
//    chunk when d > 0, so the sign bit marks the negative weights).
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
#include "tq2_device.h"

namespace tq2 {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kChunk = 256;            // k per pipeline stage
constexpr int kLdsRow = kChunk + 8;    // binary16 per LDS row (16-byte pad vs bank conflicts)
constexpr int kPpMaxKB = 96;           // scale blocks per row the ping-pong kernel can keep in LDS (K <= 12288)

__device__ __forceinline__ half2_t as_half2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

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

// The same four pairs as exact binary16 (c - 1), for a kernel that applies
// the block scale to the MFMA's result instead.
__device__ __forceinline__ half8_t decode_step_unit(uint32_t word, uint32_t magic) {
  half8_t b;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t mask = (3u << (2 * r)) | (3u << (2 * r + 16));
    const half2_t v = as_half2(and_or(word, mask, magic));
    const _Float16 sc = _Float16(1.0f / float(1 << (2 * r)));
    const _Float16 off = _Float16(-(1024.0f / float(1 << (2 * r)) + 1.0f));
    const half2_t scv = {sc, sc};
    const half2_t offv = {off, off};
    const half2_t val = v * scv + offv;
    b[2 * r] = val[0];
    b[2 * r + 1] = val[1];
  }
  return b;
}

// Q1: four binary16 pairs (8 weights) of one MFMA step.  Pair p = base + r
// of `word` has its bits at p and p + 16; shifting left by 15 - p puts them
// on the two sign bits and the AND-OR adds the magnitude pair `dabs2`
// (|d|, |d|).  `word` is complemented beforehand when d is positive, so a set
// sign bit is exactly a negative weight: the pair is ((2b-1) d, (2b'-1) d).
__device__ __forceinline__ half8_t decode_step_q1(uint32_t word, int base, uint32_t dabs2) {
  half8_t b;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int p = base + r;
    const half2_t val = as_half2(and_or(word << (15 - p), 0x80008000u, dabs2));
    b[2 * r] = val[0];
    b[2 * r + 1] = val[1];
  }
  return b;
}

// Q1 decode operands of one block scale: the |d| pair and the word mask that
// complements the bits when d is positive (sign bit clear).
__device__ __forceinline__ uint32_t q1_dabs2(uint32_t dbits) { return (dbits & 0x7FFFu) * 0x10001u; }
__device__ __forceinline__ uint32_t q1_fold(uint32_t dbits) { return ((dbits >> 15) & 1u) - 1u; }

// Wait for this wave's LDS accesses, then join the workgroup barrier.  The
// asm's memory clobber keeps the compiler from moving memory accesses across
// it; unlike __syncthreads() it leaves the wave's global loads in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// x = hi + lo for a pair of f32: hi = binary16(x) (round to nearest even),
// lo = binary16(x - hi), where x - hi is exact in f32 and comes from one
// v_fma_mix_f32 per element (hi read as binary16 from the packed pair).
__device__ __forceinline__ void split_limbs(float a, float b, uint32_t& hi, uint32_t& lo) {
  const half2_t h = {_Float16(a), _Float16(b)};
  hi = __builtin_bit_cast(uint32_t, h);
  float ra, rb;
  asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(ra) : "v"(hi), "v"(a));
  asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(rb) : "v"(hi), "v"(b));
  const half2_t l = {_Float16(ra), _Float16(rb)};
  lo = __builtin_bit_cast(uint32_t, l);
}

// max(m, |a|, |b|) in one instruction.  fmaxf compiles to one extra
// instruction per input (IEEE-mode canonicalisation); the hardware max
// itself already returns the other operand for a quiet NaN.
__device__ __forceinline__ float max3_abs(float m, float a, float b) {
  float r;
  asm("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(r) : "v"(m), "v"(a), "v"(b));
  return r;
}

// Largest value over the wave (v >= 0, not NaN), left in lane 63 and read
// from there: the same lane moves as wave_max_nonneg, with integer maxima
// of the bit patterns (which order non-negative floats as the floats).
__device__ __forceinline__ float wave_max_nonneg_bits(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  u = max(u, uint32_t(__builtin_amdgcn_update_dpp(0, int(u), 0xB1, 0xF, 0xF, false)));
  u = max(u, uint32_t(__builtin_amdgcn_update_dpp(0, int(u), 0x4E, 0xF, 0xF, false)));
  u = max(u, uint32_t(__builtin_amdgcn_update_dpp(0, int(u), 0x141, 0xF, 0xF, false)));
  u = max(u, uint32_t(__builtin_amdgcn_update_dpp(0, int(u), 0x140, 0xF, 0xF, false)));
  u = max(u, uint32_t(__builtin_amdgcn_update_dpp(0, int(u), 0x142, 0xA, 0xF, false)));
  u = max(u, uint32_t(__builtin_amdgcn_update_dpp(0, int(u), 0x143, 0xC, 0xF, false)));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(int(u), 63));
}

// Power-of-two prescale of x for the two-limb (hi + lo) paths: 2^e takes a
// largest |x| of mx into [2^14, 2^15), so that hi and lo stay clear of
// binary16's subnormal range whatever the magnitude of x (the scaling is
// exact, and the sums are scaled back by 2^-e).  mx = 0 gives e = 15.
__device__ __forceinline__ int prescale_exponent(float mx) {
  return 15 - __builtin_amdgcn_frexp_expf(mx);
}

// Store an MT x NO f32 result tile, staged row-major in LDS with row pitch
// NO + 4, to out[m0 + r][n0 + c] (plus the residual): THREADS threads walk
// the tile in whole rows, 16 bytes per lane, so each store instruction
// writes contiguous row segments.  The output is written once and not read
// again here, so the full-vector stores are non-temporal.
template <int MT, int NO, int THREADS>
__device__ __forceinline__ void store_tile(const float* tile, int tid, int m0, int n0, int M,
                                           int N, const float* __restrict__ residual,
                                           float* __restrict__ out) {
  constexpr int TP = NO + 4;
  constexpr int C4 = NO / 4;             // float4 per tile row
  const bool vec = (N & 3) == 0;
#pragma unroll
  for (int it = 0; it < (MT * C4 + THREADS - 1) / THREADS; ++it) {
    const int idx = tid + THREADS * it;
    if ((MT * C4) % THREADS != 0 && idx >= MT * C4) break;
    const int r = idx / C4;
    const int c4 = idx - r * C4;
    const int m = m0 + r, n = n0 + 4 * c4;
    if (m >= M || n >= N) continue;
    const float4 t4 = *reinterpret_cast<const float4*>(&tile[r * TP + 4 * c4]);
    const size_t o = size_t(m) * N + n;
    if (vec && n + 3 < N) {
      floatx4_t v = {t4.x, t4.y, t4.z, t4.w};
      if (residual) {
        const float4 rr = *reinterpret_cast<const float4*>(residual + o);
        v = floatx4_t{rr.x + v[0], rr.y + v[1], rr.z + v[2], rr.w + v[3]};
      }
      __builtin_nontemporal_store(v, reinterpret_cast<floatx4_t*>(out + o));
    } else {
      const float tv[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (n + e < N) {
          float v = tv[e];
          if (residual) v = residual[o + e] + v;
          out[o + e] = v;
        }
      }
    }
  }
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Buffer loads (make_rsrc) keep every variable offset in the per-lane
// offset and the scalar offset 0, so ragged tails read zeros.

// Block tile MT x (WN*NW); WN waves split the columns, WK waves split each
// 256-wide chunk's eight MFMA steps (their partial sums meet in LDS at the
// end).  Each wave owns MT rows x NW columns of the tile.  With SWIGLU the
// waves wn < WN/2 read the gate weight (codes, scales) and the others the
// same columns of the up weight (ucodes, uscales): the output tile is
// MT x (WN/2 * NW).
template <int MT, int NW, int WN, int WK, int LIMBS, bool SWIGLU, Fmt F>
__global__ __launch_bounds__(64 * WN * WK) void gemm_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const uint8_t* __restrict__ ucodes, const uint8_t* __restrict__ uscales,
    const float* __restrict__ x, const float* __restrict__ residual, float* __restrict__ out,
    int M, int N, int K, int tiles_m, int tiles_n) {
  constexpr int THREADS = 64 * WN * WK;
  constexpr int RT = MT / 16;            // 16-row MFMA tiles per wave
  constexpr int CG = NW / 16;            // 16-column groups per wave
  constexpr int NT = SWIGLU ? WN / 2 * NW : WN * NW;   // output columns per block
  constexpr int STEPS = 8 / WK;          // MFMA k-steps per wave per chunk
  constexpr int BITS = int(F);           // code bits per weight
  constexpr int QW = BITS * 2 / WK;      // code dwords per lane per chunk
  constexpr int AV = MT * (kChunk / 4) / THREADS;   // float4 A loads per thread per chunk
  static_assert(MT % 16 == 0 && NW % 16 == 0, "tile shape");
  static_assert(WK == 1 || WK == 2, "k split");
  static_assert(!SWIGLU || WN % 2 == 0, "gate/up wave split");
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
  // Gate or up weight (wave-uniform), and the column share inside it.
  const bool upw = SWIGLU && __builtin_amdgcn_readfirstlane(wn) >= WN / 2;
  const int wc = SWIGLU ? wn % (WN / 2) : wn;
  const int lane = tid & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int KB = K >> 7;
  typedef uint32_t codes_t[QW];
  const int nchunks = (K + kChunk - 1) / kChunk;

  // x rows m0 .. m0+MT-1 (rows past M read as zero).
  const rsrc_t rx = make_rsrc(x + size_t(m0) * K, uint32_t(min(MT, M - m0)) * uint32_t(K) * 4u);
  const uint32_t row_bytes = uint32_t(K / 8) * uint32_t(BITS);   // codes per weight row
  const rsrc_t rc = make_rsrc(upw ? ucodes : codes, uint32_t(N) * row_bytes);
  const rsrc_t rs = make_rsrc(upw ? uscales : scales, uint32_t(N) * uint32_t(KB) * 2u);

  // Per-thread byte offsets, fixed for the whole K loop; a chunk, an A row
  // step and a column group add scalar offsets.  Columns past N read as zero
  // codes and zero scales.
  const uint32_t aoff = uint32_t(tid >> 6) * uint32_t(K) * 4u + 16u * uint32_t(tid & 63);
  constexpr int AROWS = THREADS / 64;    // A rows staged per load instruction

  auto load_a = [&](int c, float4 (&areg)[AV]) {
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(
          rx, aoff + uint32_t(i * AROWS * K * 4 + c * kChunk * 4), 0, 0);
      areg[i] = __builtin_bit_cast(float4, v);
    }
  };
  // LIMBS = 2: the rows a wave stages (wave w stages rows w + THREADS/64 i)
  // are scaled by 2^xexp[c & 1][w] in chunk c before the split into hi and
  // lo.  The wave keeps a running exponent: the prescale_exponent of the
  // largest |x| it has staged so far (chunks of zeros leave it alone), which
  // can only fall from chunk to chunk.  The computing lanes bring their sums
  // of a row to the chunk's exponent of that row before its MFMAs (an exact
  // power-of-two rescale) and scale the finished sums back at the end.
  // Positions past K in a partial last chunk hold the next row's x; they are
  // zeroed, so that the scaling cannot take them past the binary16 range
  // (their weights are zero, and Inf * 0 would not be).
  constexpr int SW = THREADS / 64;       // staging waves; row r is staged by wave r % SW
  __shared__ int xexp[2][LIMBS == 2 ? SW : 1];
  int erun = 1 << 20;
  auto store_a = [&](int c, int buf, const float4 (&areg)[AV]) {
    float4 va[AV];
#pragma unroll
    for (int i = 0; i < AV; ++i) va[i] = areg[i];
    if constexpr (LIMBS == 2) {
      float mh = 0.f;
#pragma unroll
      for (int i = 0; i < AV; ++i) {
        const int c4 = (tid + THREADS * i) & 63;
        if (c * kChunk + 4 * c4 >= K) va[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        mh = max3_abs(mh, va[i].x, va[i].y);
        mh = max3_abs(mh, va[i].z, va[i].w);
      }
      const float mr = wave_max_nonneg_bits(mh);
      if (mr > 0.f) erun = min(erun, prescale_exponent(mr));   // a zero chunk says nothing
      if (lane == 0) xexp[buf][wave] = erun;
#pragma unroll
      for (int i = 0; i < AV; ++i) {
        va[i].x = __builtin_amdgcn_ldexpf(va[i].x, erun);
        va[i].y = __builtin_amdgcn_ldexpf(va[i].y, erun);
        va[i].z = __builtin_amdgcn_ldexpf(va[i].z, erun);
        va[i].w = __builtin_amdgcn_ldexpf(va[i].w, erun);
      }
    }
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const int f = tid + THREADS * i;
      const int r = f >> 6;
      const int c4 = f & 63;
      const float4 v = va[i];
      if constexpr (LIMBS == 2) {
        uint32_t hi[2], lo[2];
        split_limbs(v.x, v.y, hi[0], lo[0]);
        split_limbs(v.z, v.w, hi[1], lo[1]);
        *reinterpret_cast<u32x2_t*>(&As[buf][0][r][4 * c4]) = u32x2_t{hi[0], hi[1]};
        *reinterpret_cast<u32x2_t*>(&As[buf][1][r][4 * c4]) = u32x2_t{lo[0], lo[1]};
      } else {
        const half4_t h = {_Float16(v.x), _Float16(v.y), _Float16(v.z), _Float16(v.w)};
        *reinterpret_cast<half4_t*>(&As[buf][0][r][4 * c4]) = h;
      }
    }
  };

  // Weight loads of chunk c straight into registers: each lane takes the
  // QW code dwords of its column and k-group that this wave's steps use, and
  // the raw binary16 scale of the block they fall in.  Columns past N read as
  // zero codes and zero scales.
  const uint32_t nl = uint32_t(n0 + wc * NW + col);
  const uint32_t code_voff = nl * row_bytes + 8u * BITS * uint32_t(g) + 4u * QW * uint32_t(wk);
  const uint32_t scale_voff = (nl * uint32_t(KB) + uint32_t(g >> 1)) * 2u;
  auto load_w = [&](int c, codes_t (&cw)[CG], _Float16 (&dsc)[CG]) {
#pragma unroll
    for (int j = 0; j < CG; ++j) {
      const uint32_t off = code_voff + uint32_t(j * 16) * row_bytes + uint32_t(c * 32 * BITS);
      if constexpr (QW == 4) {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rc, off, 0, 0);
        cw[j][0] = v[0]; cw[j][1] = v[1]; cw[j][2] = v[2]; cw[j][3] = v[3];
      } else if constexpr (QW == 2) {
        const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rc, off, 0, 0);
        cw[j][0] = v[0]; cw[j][1] = v[1];
      } else {
        cw[j][0] = __builtin_amdgcn_raw_buffer_load_b32(rc, off, 0, 0);
      }
      dsc[j] = __builtin_bit_cast(
          _Float16, __builtin_amdgcn_raw_buffer_load_b16(
              rs, scale_voff + uint32_t(j * 16 * KB * 2 + c * 4), 0, 0));
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
  // TQ2: d2 is the pair (d, d) and cw the raw words.  Q1: d2 holds the bits
  // of (|d|, |d|) and cw the words after the sign fold.
  auto decode_bfrags = [&](int ss, const codes_t (&cw)[CG], const half2_t (&d2)[CG],
                           half8_t (&b)[CG]) {
#pragma unroll
    for (int j = 0; j < CG; ++j) {
      if constexpr (F == Fmt::kQ1) {
        b[j] = decode_step_q1(cw[j][ss >> 2], 4 * (ss & 3), __builtin_bit_cast(uint32_t, d2[j]));
      } else {
        uint32_t w = cw[j][ss >> 1];
        if (ss & 1) w >>= 8;
        b[j] = decode_step(w, d2[j], magic);
      }
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

  int ecur[RT];                          // LIMBS = 2: exponent of acc[i][.]'s x row
#pragma unroll
  for (int i = 0; i < RT; ++i) ecur[i] = 0;
  auto compute = [&](int c, int buf, const codes_t (&cw_raw)[CG], const _Float16 (&dsc)[CG]) {
    if constexpr (LIMBS == 2) {
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        const int en = xexp[buf][(i * 16 + col) % SW];
        const int dl = en - ecur[i];
        ecur[i] = en;
        if (dl != 0) {                   // skipped by the wave once no exponent moves
#pragma unroll
          for (int j = 0; j < CG; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_amdgcn_ldexpf(acc[i][j][e], dl);
        }
      }
    }
    // binary16 pair (d, d), or (0, 0) where k runs past K in the last chunk
    // (Q1: the |d| pair, and the words folded by the sign of d).
    const bool live = c * kChunk + 64 * g < K;
    half2_t dw[CG];
    codes_t cf[CG];
#pragma unroll
    for (int j = 0; j < CG; ++j) {
      const _Float16 d = live ? dsc[j] : _Float16(0.0f);
      if constexpr (F == Fmt::kQ1) {
        const uint32_t db = __builtin_bit_cast(uint16_t, d);
        dw[j] = __builtin_bit_cast(half2_t, q1_dabs2(db));
        const uint32_t fold = q1_fold(db);
#pragma unroll
        for (int q = 0; q < QW; ++q) cf[j][q] = cw_raw[j][q] ^ fold;
      } else {
        dw[j] = half2_t{d, d};
#pragma unroll
        for (int q = 0; q < QW; ++q) cf[j][q] = cw_raw[j][q];
      }
    }
    const codes_t (&cw)[CG] = cf;
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
    if (c + 1 >= 0 && c + 1 < nchunks) store_a(c + 1, (c + 1) & 1, areg);
    load_a(c + 2, areg);
    if (c >= 0 && c < nchunks) compute(c, c & 1, cw, dsc);
    load_w(c + 2, cw, dsc);
    lds_barrier();
  };
  for (int c = -2; c < nchunks; c += 2) {
    iteration(c, cw0, dr0);
    iteration(c + 1, cw1, dr1);
  }
  if constexpr (LIMBS == 2) {
    // acc[i][.] holds sums of x row i * 16 + col times 2^ecur[i].
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int j = 0; j < CG; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_amdgcn_ldexpf(acc[i][j][e], -ecur[i]);
  }

  // ---- K-split reduction: the wk = 1 waves hand their sums to wk = 0 -----
  float* red = reinterpret_cast<float*>(&As[0][0][0][0]);
  static_assert(WN * RT * CG * 4 * 64 * 4 <= sizeof(As), "reduction buffer");
  if constexpr (WK == 2) {
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
    if (wk == 0) {
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < CG; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[i][j][e] += red[(((wn * RT + i) * CG + j) * 4 + e) * 64 + lane];
    }
  }

  // ---- SwiGLU: each up wave hands its sums to the gate wave of its columns -
  if constexpr (SWIGLU) {
    // An up wave overwrites only the slots its own lanes have just read.
    if (wk == 0 && upw) {
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < CG; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            red[(((wn * RT + i) * CG + j) * 4 + e) * 64 + lane] = acc[i][j][e];
    }
    __syncthreads();
    if (wk == 0 && !upw) {
      const int wu = wn + WN / 2;
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < CG; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[i][j][e] =
                silu(acc[i][j][e]) * red[(((wu * RT + i) * CG + j) * 4 + e) * 64 + lane];
    }
  }

  // ---- epilogue ------------------------------------------------------------
  // The weight operand is the MFMA's first (row) operand, so each 16x16
  // result holds D[n = 4g + e][m = col]: the waves holding finished sums lay
  // them out row-major in LDS (tile row i * 16 + col, columns
  // wc * NW + j * 16 + 4g .. + 3), and every thread then stores whole rows.
  constexpr int TP = NT + 4;
  static_assert(MT * TP * 4 <= sizeof(As), "output tile");
  float* tile = red;
  __syncthreads();                       // every read of the reduction slots is done
  if (wk == 0 && !upw) {
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int j = 0; j < CG; ++j)
        *reinterpret_cast<float4*>(&tile[(i * 16 + col) * TP + wc * NW + j * 16 + 4 * g]) =
            make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
  }
  __syncthreads();
  store_tile<MT, NT, THREADS>(tile, tid, m0, n0, M, N, residual, out);
}

// ---------------------------------------------------------------------------
// Warp-specialised variant for 16 < M <= 128 (path 2).  4 + XW waves in two
// roles (a block's wave w runs on SIMD w % 4):
//  * waves 0..3, the MFMA waves, one per SIMD: with WR = 2 they split the
//    MT x (2 NW) block tile into four MT/2 x NW quarters (WR = 1: four
//    MT x NW column slices); each owns all eight MFMA steps of every
//    256-wide chunk, loads and decodes its weights (two chunks ahead) and
//    issues the MFMAs, reading x fragments from LDS;
//  * waves 4 .. 3 + XW, the x waves, only stream x: each a contiguous run
//    of XR rows of f32 from global memory (two chunks in registers),
//    converted to binary16 (RNE) into the double-buffered LDS tile.  XR is
//    MT / XW, or 13 for the 128-row tile when M <= 104 (104 rows staged).
//    A run that lies wholly past M is not loaded at all.  Against rows
//    interleaved over the waves: 27.2 -> 25.3 us at M = 100, N = 11008,
//    K = 4096, and 24.6 us with XR = 13.
// x is the largest operand (4 bytes per element, read by every block of an
// M row block), and each CU's texture unit takes its loads at a fixed rate;
// when the waves that issue MFMAs also issue those loads, in-order issue
// holds the MFMAs back behind them.  Split by role, the x waves wait on the
// texture unit and the MFMA waves on nothing but their own operands.  One
// barrier per chunk: in iteration c the MFMA waves compute chunk c from
// buffer c % 2 while the x waves store chunk c + 1 into the other buffer
// (loaded during iteration c - 1) and issue the loads of chunk c + 2.
//
// The 2 x 2 split halves the LDS fragment reads of the M <= 128 tiles (each
// MFMA wave reads half of the x rows) for twice the weight decode per block,
// which these short tiles can afford (measured, same process: M = 100,
// N = 11008, K = 4096 29.6 us against 32.9 us for the 16-column-wave tile
// kernel; four 1 x 4 MFMA waves with four x waves took 37.4 us).
//
// SWIGLU: the MFMA waves of the first half of the column slots read
// gate-weight columns, the others the same columns of the up weight; the
// output tile is MT x (NT / 2).  Scales: as in gemm_pp_kernel (LDS_SCALES:
// preloaded for the whole K, else per chunk).
template <int MT, int NW, int WR, int XW, bool SWIGLU, Fmt F, bool LDS_SCALES, int XR>
__global__ __launch_bounds__(64 * (4 + XW)) void gemm_sp_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const uint8_t* __restrict__ ucodes, const uint8_t* __restrict__ uscales,
    const float* __restrict__ x, const float* __restrict__ residual, float* __restrict__ out,
    int M, int N, int K, int tiles_m, int tiles_n) {
  constexpr int CS = 4 / WR;             // column slots of MFMA waves
  constexpr int MR = MT / WR;            // rows per MFMA wave
  constexpr int RT = MR / 16;            // 16-row MFMA tiles per MFMA wave
  constexpr int CG = NW / 16;            // 16-column groups per MFMA wave
  constexpr int NT = CS * NW;            // weight rows per block
  constexpr int NO = SWIGLU ? NT / 2 : NT;   // output columns per block
  constexpr int BITS = int(F);           // code bits per weight
  constexpr int QW = 2 * BITS;           // code dwords per lane per chunk
  constexpr int THREADS = 64 * (4 + XW);
  // XR: x rows per x wave per chunk (one 1 KB load each).  XR * XW may be
  // smaller than MT when the caller's M fits in XR * XW rows; the tile rows
  // past XR * XW are then never staged and reach only results that are not
  // stored.
  static_assert(XR * XW <= MT && XR * XW > MT - 32, "x rows per x wave");
  static_assert(MR % 16 == 0 && NW % 16 == 0 && (WR == 1 || WR == 2), "tile shape");
  static_assert(!SWIGLU || CS % 2 == 0, "gate/up column slots");

  __shared__ _Float16 As[2][MT][kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t Ls[LDS_SCALES ? NT * kPpMaxKB : 8];

  const int ntiles = tiles_m * tiles_n;
  int t = blockIdx.x;
  if ((ntiles & 7) == 0) t = (t & 7) * (ntiles >> 3) + (t >> 3);
  const int mt = t / tiles_n;
  const int nt = t - mt * tiles_n;
  const int m0 = mt * MT;
  const int n0 = nt * NO;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const bool xwave = __builtin_amdgcn_readfirstlane(wave) >= 4;
  const int wn = wave & 3;                // MFMA waves: wave slot
  const int xw = wave - 4;                // x waves: rows xw XR .. xw XR + XR - 1
  const int rh = wn % WR;                 // MFMA waves: row share (rows rh * MR ..)
  const int cs = wn / WR;                 // MFMA waves: column slot
  const bool upw = SWIGLU && __builtin_amdgcn_readfirstlane(cs) >= CS / 2;
  const int wc = SWIGLU ? cs % (CS / 2) : cs;
  const int lane = tid & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int KB = K >> 7;
  const int nchunks = (K + kChunk - 1) / kChunk;
  const int mrows = min(MT, M - m0);      // x rows of this block that exist

  // ---- x waves: rows xw XR + i of the block (a contiguous run per wave),
  // float4 `lane` of the chunk row.  Two register sets, so that a chunk's
  // loads are issued before the previous chunk's data is waited for.  Rows
  // past M read zeros (buffer range check); every pass issues the same loads,
  // so the compiler's wait counts stay exact.  A wave whose rows all lie past
  // M issues none (below).
  const rsrc_t rx = make_rsrc(x + size_t(m0) * K, uint32_t(mrows) * uint32_t(K) * 4u);
  const uint32_t xoff = uint32_t(xw * XR) * uint32_t(K) * 4u + 16u * uint32_t(lane);
  typedef float4 xregs_t[XR];
  auto load_x = [&](int c, xregs_t& xr) {
#pragma unroll
    for (int i = 0; i < XR; ++i)
      xr[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                             rx, xoff + uint32_t(i * K * 4 + c * kChunk * 4), 0, 0));
  };
  auto store_x = [&](int buf, const xregs_t& xr) {
#pragma unroll
    for (int i = 0; i < XR; ++i) {
      const float4 v = xr[i];
      const half4_t h = {_Float16(v.x), _Float16(v.y), _Float16(v.z), _Float16(v.w)};
      *reinterpret_cast<half4_t*>(&As[buf][xw * XR + i][4 * lane]) = h;
    }
  };

  // ---- MFMA waves: weights of column n0 + wc*NW + 16j + col, k-group g.
  typedef uint32_t codes_t[QW];
  const uint32_t row_bytes = uint32_t(K / 8) * uint32_t(BITS);
  const rsrc_t rc = make_rsrc(upw ? ucodes : codes, uint32_t(N) * row_bytes);
  const rsrc_t rs = make_rsrc(upw ? uscales : scales, uint32_t(N) * uint32_t(KB) * 2u);
  const uint32_t nl = uint32_t(n0 + wc * NW + col);
  const uint32_t code_voff = nl * row_bytes + 8u * BITS * uint32_t(g);
  const uint32_t scale_voff = (nl * uint32_t(KB) + uint32_t(g >> 1)) * 2u;
  auto load_w = [&](int c, codes_t (&cw)[CG], uint32_t (&dsc)[CG]) {
#pragma unroll
    for (int j = 0; j < CG; ++j) {
      const uint32_t off = code_voff + uint32_t(j * 16) * row_bytes + uint32_t(c * 32 * BITS);
      if constexpr (QW == 4) {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rc, off, 0, 0);
        cw[j][0] = v[0]; cw[j][1] = v[1]; cw[j][2] = v[2]; cw[j][3] = v[3];
      } else {
        const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rc, off, 0, 0);
        cw[j][0] = v[0]; cw[j][1] = v[1];
      }
      if constexpr (!LDS_SCALES)
        dsc[j] = __builtin_amdgcn_raw_buffer_load_b16(
            rs, scale_voff + uint32_t(j * 16 * KB * 2 + c * 4), 0, 0);
    }
  };
  // LDS_SCALES: scale of column group j and chunk c (block 2c + (g >> 1));
  // the chunk is clamped for the passes past the end, and an odd block
  // count's last second block reads the next row's first scale, which the
  // caller zeroes.
  const int ls_base = (cs * NW + col) * KB + (g >> 1);
  auto scale_bits = [&](int j, int c, const uint32_t (&dsc)[CG]) -> uint32_t {
    if constexpr (LDS_SCALES) return Ls[ls_base + j * 16 * KB + 2 * min(c, nchunks - 1)];
    return dsc[j];
  };

  // Set only by the MFMA waves (in their own loop), so that the x waves'
  // registers are not held for it during theirs.
  floatx4_t acc[RT][CG];

  const uint32_t magic = 0x64006400u;
  auto load_afrags = [&](int buf, int s, half8_t (&a)[RT]) {
#pragma unroll
    for (int i = 0; i < RT; ++i)
      a[i] = *reinterpret_cast<const half8_t*>(&As[buf][rh * MR + i * 16 + col][64 * g + 8 * s]);
  };
  auto decode_bfrags = [&](int s, const codes_t (&cw)[CG], const half2_t (&d2)[CG],
                           half8_t (&b)[CG]) {
#pragma unroll
    for (int j = 0; j < CG; ++j) {
      if constexpr (F == Fmt::kQ1) {
        b[j] = decode_step_q1(cw[j][s >> 2], 4 * (s & 3), __builtin_bit_cast(uint32_t, d2[j]));
      } else {
        uint32_t w = cw[j][s >> 1];
        if (s & 1) w >>= 8;
        b[j] = decode_step(w, d2[j], magic);
      }
    }
  };
  auto mfmas = [&](const half8_t (&a)[RT], const half8_t (&b)[CG]) {
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int j = 0; j < CG; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b[j], a[i], acc[i][j], 0, 0, 0);
  };
  // Per step about VALU/MFMA decode instructions and an LDS read every few
  // MFMAs, instead of long runs of either.
  constexpr int NMFMA = RT * CG;
  auto interleave = [&]() {
#pragma unroll
    for (int q = 0; q < NMFMA; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // one MFMA
      if (q % ((NMFMA + RT - 1) / RT) == 0)
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);        // one LDS read
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);          // up to three VALU
    }
  };
  auto compute = [&](int c, int buf, const codes_t (&cw_raw)[CG], const uint32_t (&dsc)[CG]) {
    // binary16 pair (d, d), or (0, 0) where k runs past K in the last chunk
    // (Q1: the |d| pair, and the words folded by the sign of d).
    const bool live = c * kChunk + 64 * g < K;
    half2_t dw[CG];
    codes_t cw[CG];
#pragma unroll
    for (int j = 0; j < CG; ++j) {
      const uint32_t db = live ? scale_bits(j, c, dsc) & 0xFFFFu : 0u;
      if constexpr (F == Fmt::kQ1) {
        dw[j] = __builtin_bit_cast(half2_t, q1_dabs2(db));
        const uint32_t fold = q1_fold(db);
#pragma unroll
        for (int q = 0; q < QW; ++q) cw[j][q] = cw_raw[j][q] ^ fold;
      } else {
        const _Float16 d = __builtin_bit_cast(_Float16, uint16_t(db));
        dw[j] = half2_t{d, d};
#pragma unroll
        for (int q = 0; q < QW; ++q) cw[j][q] = cw_raw[j][q];
      }
    }
    half8_t a0[RT], a1[RT], b0[CG], b1[CG];
    load_afrags(buf, 0, a0);
    decode_bfrags(0, cw, dw, b0);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if ((s & 1) == 0) {
        if (s + 1 < 8) {
          load_afrags(buf, s + 1, a1);
          decode_bfrags(s + 1, cw, dw, b1);
        }
        mfmas(a0, b0);
      } else {
        if (s + 1 < 8) {
          load_afrags(buf, s + 1, a0);
          decode_bfrags(s + 1, cw, dw, b0);
        }
        mfmas(a1, b1);
      }
      interleave();
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- prologue: (LDS_SCALES) the block's scales into LDS, x chunk 0 in
  // buffer 0 and chunk 1 in flight, weight chunks 0 and 1 in flight.
  if constexpr (LDS_SCALES) {
    auto preload = [&](const uint8_t* plane, int rows, int dst) {
      const uint32_t valid = uint32_t(min(rows, N - n0)) * uint32_t(KB) * 2u;
      const uint32_t full = valid & ~15u;
      const rsrc_t rsb = make_rsrc(plane + size_t(n0) * KB * 2, valid);
      uint8_t* ls = reinterpret_cast<uint8_t*>(Ls + dst);
      for (uint32_t o = 16u * uint32_t(tid); o < full; o += 16u * THREADS) {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rsb, o, 0, 0);
        *reinterpret_cast<u32x4_t*>(ls + o) = v;
      }
      const uint32_t o2 = full + 2u * uint32_t(tid);
      if (o2 < valid)
        *reinterpret_cast<uint16_t*>(ls + o2) = __builtin_amdgcn_raw_buffer_load_b16(rsb, o2, 0, 0);
    };
    if constexpr (SWIGLU) {
      preload(scales, NO, 0);
      preload(uscales, NO, NO * KB);
    } else {
      preload(scales, NT, 0);
    }
  }
  // ---- main loops: each role runs its own, with the same number of passes
  // and barriers (a pass past the last chunk only issues loads); the values
  // each loop keeps live are then not held by the other role's waves.
  if (xwave && __builtin_amdgcn_readfirstlane(xw * XR) >= mrows) {
    // An x wave whose rows all lie past M stages nothing (its LDS rows reach
    // only results that are not stored) and only keeps the barrier count:
    // one wave-uniform branch, so the loads of the other waves stay
    // unconditional.
    lds_barrier();
    for (int c = 0; c < nchunks; c += 2) {
      lds_barrier();
      lds_barrier();
    }
  } else if (xwave) {
    // x chunk q lives in set q % 2: pass c stores chunk c + 1 and reloads its
    // set with chunk c + 3.
    xregs_t xa, xb;
    load_x(0, xa);
    load_x(1, xb);
    store_x(0, xa);
    load_x(2, xa);
    lds_barrier();
    for (int c = 0; c < nchunks; c += 2) {
      if (c + 1 < nchunks) store_x(1, xb);
      load_x(c + 3, xb);
      lds_barrier();
      if (c + 2 < nchunks) store_x(0, xa);
      load_x(c + 4, xa);
      lds_barrier();
    }
  } else {
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int j = 0; j < CG; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    codes_t cw0[CG], cw1[CG];
    uint32_t dr0[CG], dr1[CG];
    load_w(0, cw0, dr0);
    load_w(1, cw1, dr1);
    lds_barrier();
    auto pass = [&](int c, codes_t (&cw)[CG], uint32_t (&dsc)[CG]) {
      if (c < nchunks) compute(c, c & 1, cw, dsc);
      load_w(c + 2, cw, dsc);
      lds_barrier();
    };
    for (int c = 0; c < nchunks; c += 2) {
      pass(c, cw0, dr0);
      pass(c + 1, cw1, dr1);
    }
  }

  // ---- epilogue --------------------------------------------------------------
  // (SWIGLU: the up waves hand their sums to the gate waves.)  The finished
  // MT x NO tile is laid out row-major in LDS and all 512 threads store it in
  // whole rows, 16 bytes per lane, reading the residual the same way.
  float* red = reinterpret_cast<float*>(&As[0][0][0]);
  if constexpr (SWIGLU) {
    static_assert(2 * RT * CG * 4 * 64 * 4 <= sizeof(As), "reduction buffer");
    const int slot = rh * (CS / 2) + wc;
    if (!xwave && upw) {
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < CG; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            red[(((slot * RT + i) * CG + j) * 4 + e) * 64 + lane] = acc[i][j][e];
    }
    __syncthreads();
    if (!xwave && !upw) {
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < CG; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[i][j][e] = silu(acc[i][j][e]) * red[(((slot * RT + i) * CG + j) * 4 + e) * 64 + lane];
    }
  }
  // D[n = 4g + e][m = col] of each 16 x 16 result goes to tile row
  // i * 16 + col, columns wc * NW + j * 16 + 4g .. + 3.
  constexpr int TP = NO + 4;
  static_assert(MT * TP * 4 <= sizeof(As), "output tile");
  float* tile = red;
  __syncthreads();
  if (!xwave && !upw) {
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int j = 0; j < CG; ++j)
        *reinterpret_cast<float4*>(&tile[(rh * MR + i * 16 + col) * TP + wc * NW + j * 16 + 4 * g]) =
            make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
  }
  __syncthreads();
  store_tile<MT, NO, THREADS>(tile, tid, m0, n0, M, N, residual, out);
}

template <int MT, int NW, int WR, int XW, bool SWIGLU, Fmt F, bool LDS_SCALES, int XR = MT / XW>
hipError_t launch_sp(const uint8_t* soa, const uint8_t* up, const float* x,
                     const float* residual, float* out, int64_t m, int64_t n, int64_t k,
                     hipStream_t stream) {
  constexpr int NO = (SWIGLU ? 2 : 4) / WR * NW;
  const int64_t tm = (m + MT - 1) / MT;
  const int64_t tn = (n + NO - 1) / NO;
  if (tm * tn > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid(unsigned(tm * tn));
  const size_t so = scales_offset(F, n, k);
  // Rows the x waves would not stage (only where XR * XW < MT).
  if (int64_t(XR) * XW < MT && m > int64_t(XR) * XW) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_sp_kernel<MT, NW, WR, XW, SWIGLU, F, LDS_SCALES, XR>), grid,
                     dim3(64 * (4 + XW)), 0, stream,
                     soa, soa + so, up, up ? up + so : nullptr, x, residual, out, int(m), int(n),
                     int(k), int(tm), int(tn));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// K-split variant for 16 < M <= 128 with x converted once per call (path 2,
// tq2_gemm_ws).  Each CU of gemm_sp_kernel streams all of x in f32 from L2,
// and a CU takes about 118 GB/s from L2 however the loads are spread over
// its waves (measured with contiguous 16-byte-per-lane loads): 1.64 MB of x
// at M = 100, K = 4096 is 14 us per block before any arithmetic.  Reading x
// in MFMA fragment order straight from its f32 rows is worse still (35 GB/s
// per CU: a 16-row fragment touches 16 lines one row pitch apart).  So a
// pre-pass writes x once per call as binary16 fragments into a workspace
// (half the bytes, each fragment a contiguous 1 KB), and the GEMM's waves
// load those fragments directly into operand registers: no x tile in LDS,
// no staging waves and no barrier inside the K loop.
//
// x16_fragments_kernel: fragment (rt, c, s), 1 KB, holds for lane
// l = 16 g + col the binary16 (RNE) values x[16 rt + col][256 c + 64 g +
// 8 s .. + 7], the B operand of MFMA step s of chunk c for row tile rt in the
// chunk bookkeeping above.  Rows past M and k past K are written as zeros.
// One block per (rt, c): thread t reads 16 consecutive k (64 bytes) of row
// t / 16 (whole 1 KB rows per 16 threads), puts its two 8-value groups in
// their fragment slots in LDS, and the block then writes its 8 fragments
// (8 KB, contiguous in the workspace) 32 bytes per thread.
__global__ __launch_bounds__(256) void x16_fragments_kernel(const float* __restrict__ x, int M,
                                                            int K, int nch,
                                                            u32x4_t* __restrict__ frag) {
  __shared__ u32x4_t sl[8 * 64];
  const int c = int(blockIdx.x) % nch;
  const int rt = int(blockIdx.x) / nch;
  const int t = threadIdx.x;
  const int r = t >> 4, seg = t & 15;          // row in the tile, 16-wide k segment
  const int m = 16 * rt + r;
  const int k0 = c * kChunk + 16 * seg;
  u32x4_t h0 = {0u, 0u, 0u, 0u}, h1 = {0u, 0u, 0u, 0u};
  if (m < M && k0 < K) {
    const float4* p = reinterpret_cast<const float4*>(x + size_t(m) * uint32_t(K) + k0);
    const float4 a = p[0], b = p[1], e = p[2], f = p[3];
    auto pk = [](float u, float v) { return __builtin_bit_cast(uint32_t, half2_t{_Float16(u), _Float16(v)}); };
    h0 = u32x4_t{pk(a.x, a.y), pk(a.z, a.w), pk(b.x, b.y), pk(b.z, b.w)};
    h1 = u32x4_t{pk(e.x, e.y), pk(e.z, e.w), pk(f.x, f.y), pk(f.z, f.w)};
  }
  // k = 64 g + 8 st + i inside the chunk: this thread's groups are
  // g = seg / 4, st = 2 (seg % 4) and st + 1, for lane 16 g + r.
  const int g = seg >> 2, st = 2 * (seg & 3);
  sl[st * 64 + 16 * g + r] = h0;
  sl[(st + 1) * 64 + 16 * g + r] = h1;
  __syncthreads();
  u32x4_t* dst = frag + (size_t(rt) * uint32_t(nch) + uint32_t(c)) * 512u;
  dst[2 * t] = sl[2 * t];
  dst[2 * t + 1] = sl[2 * t + 1];
}

// gemm_ks_kernel: block = all RT * 16 rows (one row block, 16 < M <= 128)
// x CT * 16 weight columns, 8 waves (two per SIMD).  Wave w owns the chunks
// [w nch / 8, (w + 1) nch / 8) of K: for each it takes the chunk's code words
// and scales of its CT column groups and streams the chunk's 8 x RT x
// fragments through RT x CT MFMAs per step, decoding each weight once for all
// rows.  Nothing is shared between the waves until their partial sums meet
// in LDS at the end, in a fixed order (waves w and w + 4, then the four
// sums), so results are deterministic.  Two waves per SIMD let one wave's
// decode overlap the other's MFMAs.
//
// LDS_W (TQ2, K <= kKsMaxK): the block first copies its whole weight slice
// (codes in MFMA lane order, and scales) into LDS, so that the K loop's only
// global loads are the x fragments.  Vector loads complete in issue order: a
// chunk's code words, fetched from HBM inside the loop, held back every x
// fragment issued after them (at M = 100, N = 11008, K = 4096 the kernel
// takes 15.3 us with the staged weights, 16.3 us with per-chunk loads).
// Otherwise each wave loads its chunks' weights from global memory a chunk
// ahead.
constexpr int kKsLdsBytes = 156 * 1024;
constexpr int64_t kKsMaxK = 12288;           // staged weights: 48 columns x K, plus scales

template <int RT, int CT, int RING, Fmt F, bool LDS_W>
__global__ __launch_bounds__(512) void gemm_ks_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const u32x4_t* __restrict__ frag, const float* __restrict__ residual,
    float* __restrict__ out, int M, int N, int K, int nch) {
  constexpr int NO = 16 * CT;
  constexpr int BITS = int(F);
  constexpr int QW = 2 * BITS;                 // code dwords per lane per chunk
  static_assert(!LDS_W || F == Fmt::kTq2, "staged weights use the TQ2 lane order");
  static_assert(4 * RT * CT * 64 * 16 <= kKsLdsBytes, "reduction buffer");
  static_assert(!LDS_W || (kKsMaxK / kChunk) * CT * 1024 + NO * (kKsMaxK / 128) * 2 <= kKsLdsBytes,
                "staged weights");
  __shared__ __attribute__((aligned(16))) uint8_t smem[kKsLdsBytes];

  const int n0 = blockIdx.x * NO;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int KB = K >> 7;
  const int c0 = (wave * nch) >> 3;
  const int c1 = ((wave + 1) * nch) >> 3;

  typedef uint32_t codes_t[QW];
  const uint32_t row_bytes = uint32_t(K / 8) * uint32_t(BITS);
  // One resource per row tile (its nch * 8 fragments), so that a step's RT
  // loads share one per-lane offset and the step's place inside its half
  // chunk goes into the instructions' immediate offsets.  Fragment loads past
  // the wave's (or the matrix's) last chunk are issued anyway: they read
  // another wave's data or, past the row tile's end, zeros (range check),
  // and keep every load unconditional.
  const uint32_t xrt = uint32_t(nch) * 8u * 1024u;     // bytes per row tile
  rsrc_t rx[RT];
#pragma unroll
  for (int i = 0; i < RT; ++i)
    rx[i] = make_rsrc(reinterpret_cast<const uint8_t*>(frag) + size_t(i) * xrt, xrt);
  auto load_x = [&](int c, int st, u32x4_t (&xf)[RT]) {
    const uint32_t off = uint32_t((c * 8 + (st & 4)) * 1024) + 16u * uint32_t(lane);
#pragma unroll
    for (int i = 0; i < RT; ++i)
      xf[i] = __builtin_amdgcn_raw_buffer_load_b128(rx[i], off + uint32_t((st & 3) * 1024), 0, 0);
  };

  // Staged weights: wl[(c * CT + j) * 64 + lane] holds the four code words
  // lane (col, g) of column group j uses in chunk c; sl[n * KB + kb] the
  // scales of the block's columns.
  const u32x4_t* wl = reinterpret_cast<const u32x4_t*>(smem);
  const uint16_t* sl = reinterpret_cast<const uint16_t*>(smem + size_t(nch) * CT * 1024);
  // Global weights (not LDS_W): column n0 + 16 j + col, k-group g.
  const uint32_t nl = uint32_t(n0 + col);
  const uint32_t code_voff = nl * row_bytes + 8u * BITS * uint32_t(g);
  const uint32_t scale_voff = (nl * uint32_t(KB) + uint32_t(g >> 1)) * 2u;
  const rsrc_t rc = make_rsrc(codes, uint32_t(N) * row_bytes);
  const rsrc_t rs = make_rsrc(scales, uint32_t(N) * uint32_t(KB) * 2u);
  auto load_w = [&](int c, codes_t (&cw)[CT], uint32_t (&dsc)[CT]) {
#pragma unroll
    for (int j = 0; j < CT; ++j) {
      if constexpr (LDS_W) {
        const u32x4_t v = wl[(c * CT + j) * 64 + lane];
        cw[j][0] = v[0]; cw[j][1] = v[1]; cw[j][2] = v[2]; cw[j][3] = v[3];
        dsc[j] = sl[(16 * j + col) * KB + 2 * c + (g >> 1)];
      } else {
        const uint32_t off = code_voff + uint32_t(j * 16) * row_bytes + uint32_t(c * 32 * BITS);
        if constexpr (QW == 4) {
          const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rc, off, 0, 0);
          cw[j][0] = v[0]; cw[j][1] = v[1]; cw[j][2] = v[2]; cw[j][3] = v[3];
        } else {
          const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rc, off, 0, 0);
          cw[j][0] = v[0]; cw[j][1] = v[1];
        }
        dsc[j] = __builtin_amdgcn_raw_buffer_load_b16(
            rs, scale_voff + uint32_t(j * 16 * KB * 2 + c * 4), 0, 0);
      }
    }
  };

  // A ring of RING (2 or 4, a divisor of 8) steps' fragments: step st of a
  // chunk reads slot st % RING and loads step st + RING - 1 into the slot
  // freed by step st - 1, so each load has RING - 1 steps' work to arrive.
  // The first RING - 1 steps go out before anything else.  Two slots are
  // used: with four, the loop was slower (M = 100, N = 11008, K = 4096:
  // 16.8 - 17.5 against 15.3 us per kernel; RT = 7 then spills).
  static_assert(RING == 2 || RING == 4, "ring depth");
  u32x4_t xr[RING][RT];
  if (c0 < c1) {
#pragma unroll
    for (int q = 0; q < RING - 1; ++q) load_x(c0, q, xr[q]);
  }

  if constexpr (LDS_W) {
    // The block's weight slice into LDS: 16-byte units u = (column jn, unit
    // t16 = 4 c + g of its row), 8 loads in flight per thread, columns past
    // N read as zeros.  The weight is read once per call: its loads carry
    // the streaming hint, so that they do not push the x fragments out of
    // the caches.
    const int live_cols = min(NO, N - n0);
    const rsrc_t rcb = make_rsrc(codes + size_t(n0) * row_bytes, uint32_t(live_cols) * row_bytes);
    const rsrc_t rsb = make_rsrc(scales + size_t(n0) * uint32_t(KB) * 2u,
                                 uint32_t(live_cols) * uint32_t(KB) * 2u);
    const int upc = K >> 6;                    // 16-byte units per column row
    const int units = NO * upc;
    u32x4_t* wls = reinterpret_cast<u32x4_t*>(smem);
    for (int base = 0; base < units; base += 8 * 512) {
      u32x4_t v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int u = base + q * 512 + tid;
        const int jn = u / upc, t16 = u - jn * upc;
        const uint32_t off = u < units ? uint32_t(jn) * row_bytes + 16u * uint32_t(t16) : 0xFFFFFFF0u;
        v[q] = __builtin_amdgcn_raw_buffer_load_b128(rcb, off, 0, kStreamOnce);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int u = base + q * 512 + tid;
        if (u < units) {
          const int jn = u / upc, t16 = u - jn * upc;
          wls[((t16 >> 2) * CT + (jn >> 4)) * 64 + 16 * (t16 & 3) + (jn & 15)] = v[q];
        }
      }
    }
    uint16_t* sls = reinterpret_cast<uint16_t*>(smem + size_t(nch) * CT * 1024);
    for (int u = tid; u < NO * KB; u += 512)
      sls[u] = __builtin_amdgcn_raw_buffer_load_b16(rsb, 2u * uint32_t(u), 0, kStreamOnce);
    lds_barrier();
  }

  floatx4_t acc[RT][CT];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < CT; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  const uint32_t magic = 0x64006400u;
  if (c0 < c1) {
    // Global weights: loaded a chunk ahead (cw / dsc for chunk c, cwn / dsn
    // for c + 1).  Staged weights: read from LDS at the start of each chunk.
    codes_t cw[CT];
    uint32_t dsc[CT];
    if constexpr (!LDS_W) load_w(c0, cw, dsc);
    for (int c = c0; c < c1; ++c) {
      codes_t cwn[CT];
      uint32_t dsn[CT];
      if constexpr (LDS_W)
        load_w(c, cw, dsc);
      else
        load_w(c + 1, cwn, dsn);
      __builtin_amdgcn_sched_barrier(0);
      // binary16 pair (d, d), or (0, 0) where k runs past K in the last
      // chunk (Q1: the |d| pair, and the words folded by the sign of d).
      const bool live = c * kChunk + 64 * g < K;
      half2_t dw[CT];
      codes_t cwd[CT];
#pragma unroll
      for (int j = 0; j < CT; ++j) {
        const uint32_t db = live ? dsc[j] & 0xFFFFu : 0u;
        if constexpr (F == Fmt::kQ1) {
          dw[j] = __builtin_bit_cast(half2_t, q1_dabs2(db));
          const uint32_t fold = q1_fold(db);
#pragma unroll
          for (int q = 0; q < QW; ++q) cwd[j][q] = cw[j][q] ^ fold;
        } else {
          const _Float16 d = __builtin_bit_cast(_Float16, uint16_t(db));
          dw[j] = half2_t{d, d};
#pragma unroll
          for (int q = 0; q < QW; ++q) cwd[j][q] = cw[j][q];
        }
      }
      auto step = [&](int st, const u32x4_t (&xc)[RT], u32x4_t (&xn)[RT]) {
        // Step st + RING - 1's fragments (past step 7: the next chunk's).
        if (st + RING - 1 < 8)
          load_x(c, st + RING - 1, xn);
        else
          load_x(c + 1, st + RING - 1 - 8, xn);
        // Keep these loads ahead of the step's arithmetic (the scheduler
        // would sink them to their registers' last use).
        __builtin_amdgcn_sched_barrier(0);
        half8_t b[CT];
#pragma unroll
        for (int j = 0; j < CT; ++j) {
          if constexpr (F == Fmt::kQ1) {
            b[j] = decode_step_q1(cwd[j][st >> 2], 4 * (st & 3),
                                  __builtin_bit_cast(uint32_t, dw[j]));
          } else {
            uint32_t w = cwd[j][st >> 1];
            if (st & 1) w >>= 8;
            b[j] = decode_step(w, dw[j], magic);
          }
        }
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
          for (int j = 0; j < CT; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                b[j], __builtin_bit_cast(half8_t, xc[i]), acc[i][j], 0, 0, 0);
      };
#pragma unroll
      for (int st = 0; st < 8; ++st) step(st, xr[st % RING], xr[(st + RING - 1) % RING]);
      if constexpr (!LDS_W) {
#pragma unroll
        for (int j = 0; j < CT; ++j) {
          dsc[j] = dsn[j];
#pragma unroll
          for (int q = 0; q < QW; ++q) cw[j][q] = cwn[j][q];
        }
      }
    }
  }

  // ---- the eight partial sums, in a fixed order: S_w = P_w + P_{w+4}, then
  // ((S_0 + S_1) + (S_2 + S_3)).  D[n = 4g + e][m = col] of each 16 x 16
  // result is out[16 i + col][n0 + 16 j + 4g + e].  The barriers wait for
  // LDS only: loads still in flight (fragments past the last chunk) are not
  // waited for here.
  float4 (*red)[RT * CT][64] = reinterpret_cast<float4 (*)[RT * CT][64]>(smem);
  if constexpr (LDS_W) lds_barrier();           // every wave is done with the staged weights
  if (wave >= 4) {
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int j = 0; j < CT; ++j)
        red[wave - 4][i * CT + j][lane] =
            make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
  }
  lds_barrier();
  if (wave < 4) {
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int j = 0; j < CT; ++j) {
        const float4 o = red[wave][i * CT + j][lane];
        acc[i][j] += floatx4_t{o.x, o.y, o.z, o.w};
      }
  }
  lds_barrier();
  if (wave < 4) {
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int j = 0; j < CT; ++j)
        red[wave][i * CT + j][lane] =
            make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
  }
  lds_barrier();
  const bool vec = (N & 3) == 0;
  for (int it = tid; it < RT * CT * 64; it += 512) {
    const int q = it >> 6, l = it & 63;
    const int i = q / CT, j = q - i * CT;
    const int m = 16 * i + (l & 15), n = n0 + 16 * j + 4 * (l >> 4);
    if (m >= M || n >= N) continue;
    const float4 a = red[0][q][l], b = red[1][q][l], cc = red[2][q][l], d = red[3][q][l];
    floatx4_t v = {(a.x + b.x) + (cc.x + d.x), (a.y + b.y) + (cc.y + d.y),
                   (a.z + b.z) + (cc.z + d.z), (a.w + b.w) + (cc.w + d.w)};
    const size_t o = size_t(m) * uint32_t(N) + uint32_t(n);
    if (vec && n + 3 < N) {
      if (residual) {
        const float4 rr = *reinterpret_cast<const float4*>(residual + o);
        v = floatx4_t{rr.x + v[0], rr.y + v[1], rr.z + v[2], rr.w + v[3]};
      }
      __builtin_nontemporal_store(v, reinterpret_cast<floatx4_t*>(out + o));
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (n + e < N) {
          float r = v[e];
          if (residual) r = residual[o + e] + r;
          out[o + e] = r;
        }
      }
    }
  }
}

// Workspace bytes of the binary16 x fragments for an M x K call (M <= 128).
inline size_t ks_workspace_bytes(int64_t m, int64_t k) {
  const int64_t rt = (m + 15) / 16;
  const int64_t nch = (k + kChunk - 1) / kChunk;
  return size_t(rt) * size_t(nch) * 8u * 1024u;
}

template <int RT, Fmt F>
hipError_t launch_ks(const uint8_t* soa, const float* x, const float* residual, float* out,
                     int64_t m, int64_t n, int64_t k, void* ws, hipStream_t stream) {
  constexpr int CT = 3;
  const int nch = int((k + kChunk - 1) / kChunk);
  hipLaunchKernelGGL(x16_fragments_kernel, dim3(unsigned(RT * nch)), dim3(256), 0, stream, x,
                     int(m), int(k), nch, static_cast<u32x4_t*>(ws));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t blocks = (n + 16 * CT - 1) / (16 * CT);
  const size_t so = scales_offset(F, n, k);
  constexpr int RING = 2;
  if (F == Fmt::kTq2 && k <= kKsMaxK)
    hipLaunchKernelGGL((gemm_ks_kernel<RT, CT, RING, F, F == Fmt::kTq2>), dim3(unsigned(blocks)),
                       dim3(512), 0, stream, soa, soa + so, static_cast<const u32x4_t*>(ws),
                       residual, out, int(m), int(n), int(k), nch);
  else
    hipLaunchKernelGGL((gemm_ks_kernel<RT, CT, RING, F, false>), dim3(unsigned(blocks)),
                       dim3(512), 0, stream, soa, soa + so, static_cast<const u32x4_t*>(ws),
                       residual, out, int(m), int(n), int(k), nch);
  return hipGetLastError();
}

template <Fmt F>
hipError_t dispatch_ks(const uint8_t* soa, const float* x, const float* residual, float* out,
                       int64_t m, int64_t n, int64_t k, void* ws, hipStream_t stream) {
  switch ((m + 15) / 16) {
    case 2: return launch_ks<2, F>(soa, x, residual, out, m, n, k, ws, stream);
    case 3: return launch_ks<3, F>(soa, x, residual, out, m, n, k, ws, stream);
    case 4: return launch_ks<4, F>(soa, x, residual, out, m, n, k, ws, stream);
    case 5: return launch_ks<5, F>(soa, x, residual, out, m, n, k, ws, stream);
    case 6: return launch_ks<6, F>(soa, x, residual, out, m, n, k, ws, stream);
    case 7: return launch_ks<7, F>(soa, x, residual, out, m, n, k, ws, stream);
    case 8: return launch_ks<8, F>(soa, x, residual, out, m, n, k, ws, stream);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------
// Skinny variant for M <= 16 with x split into two binary16 limbs (the
// f32-class path).  At this M the work per weight is tiny, so the kernel is
// laid out for the weight stream rather than for matrix-core reuse: the
// block's waves split K, not N.  In pass p wave w owns the slice
// k in [4096 p + SLICE w, +SLICE), SLICE = 4096 / WAVES.  It loads that slice
// of x once, one row per 16-byte-per-lane load (whole cache lines), converts
// it to the hi and lo binary16 limbs, and passes it through a per-wave LDS
// region into operand fragments that stay in registers.  Meanwhile the code
// words and scales of the block's 16-column tiles are already in flight
// (PF tiles ahead); the wave streams them through the fragments with no
// barrier inside the K loop.  The waves' partial sums of each output meet in
// LDS once, at the end.
//
// x is the MFMA's A operand and the weight its B operand, so lane (col, g)
// accumulates D[m = 4g + e][n = col].  Each MFMA step contracts 32 k's of one
// 128-weight block: steps 4b .. 4b + 3 of a 256-wide chunk cover its block b,
// and lane (col, g) holds for block b the two code words (TQ2; one word for
// Q1) of its column that cover k = kb .. kb + 31, with kb = 32 (2 (g & 1) +
// (g >> 1)) for b = 0 and 128 + 32 (2 (g & 1) + 1 - (g >> 1)) for b = 1;
// step 4b + s takes k = kb + 8s .. + 7 from both operands.  The weights enter as exact
// binary16 (c - 1) (Q1: +-1), each block's four steps accumulate into a fresh
// D, and acc += d * D applies the column's block scale in f32 (one FMA per
// output and block instead of one packed multiply per weight pair).
//
// PACK (M <= 8): the A operand's 16 rows hold the hi limbs of x rows 0..7
// and the lo limbs of the same rows, so one MFMA per step covers both limbs
// and output (m, n) is D[m][n] + D[m + 8][n].  Otherwise (M <= 16) the limbs
// take one MFMA each.
template <int TMAX, int WAVES, bool PACK, bool SWIGLU, Fmt F, bool SKIP>
__global__ __launch_bounds__(64 * WAVES) void gemm_skinny_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const uint8_t* __restrict__ ucodes, const uint8_t* __restrict__ uscales,
    const float* __restrict__ x, const float* __restrict__ residual, float* __restrict__ out,
    int M, int N, int K) {
  constexpr int THREADS = 64 * WAVES;
  constexpr int PASS_K = 4096;
  constexpr int SLICE = PASS_K / WAVES;  // k per wave per pass
  constexpr int CPW = SLICE / kChunk;    // 256-wide chunks per wave
  constexpr int BITS = int(F);
  constexpr int QW = 2 * BITS;           // code dwords per lane per chunk
  constexpr int NMAT = SWIGLU ? 2 : 1;   // weights read per tile (gate, up)
  constexpr int PF = SWIGLU ? 2 : TMAX;  // tiles whose loads are in flight
  constexpr int XR = PACK ? 8 : 16;      // x rows staged
  constexpr int LIMBS = PACK ? 1 : 2;    // MFMAs per step
  constexpr int LROWS = 2 * XR;          // LDS rows per wave: hi rows, then lo rows
  constexpr int XS_BYTES = WAVES * LROWS * kLdsRow * 2;
  constexpr int RED_BYTES = WAVES * TMAX * NMAT * 4 * 64 * 4;
  static_assert(CPW >= 1 && CPW * kChunk * WAVES == PASS_K, "slice split");
  typedef uint32_t codes_t[QW];
  __shared__ __attribute__((aligned(16))) unsigned char smem[XS_BYTES > RED_BYTES ? XS_BYTES : RED_BYTES];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int KB = K >> 7;
  const int tiles = (N + 15) >> 4;
  const int tile0 = blockIdx.x * TMAX;
  const int ntile = min(TMAX, tiles - tile0);
  _Float16* xs = reinterpret_cast<_Float16*>(smem) + wave * LROWS * kLdsRow;

  // x rows past M, columns past N read as zero.
  const rsrc_t rx = make_rsrc(x, uint32_t(M) * uint32_t(K) * 4u);
  const uint32_t row_bytes = uint32_t(K / 8) * uint32_t(BITS);
  const rsrc_t rc[2] = {make_rsrc(codes, uint32_t(N) * row_bytes),
                        make_rsrc(SWIGLU ? ucodes : codes, uint32_t(N) * row_bytes)};
  const rsrc_t rs[2] = {make_rsrc(scales, uint32_t(N) * uint32_t(KB) * 2u),
                        make_rsrc(SWIGLU ? uscales : scales, uint32_t(N) * uint32_t(KB) * 2u)};

  floatx4_t acc[TMAX][NMAT];             // [tile][gate/up]; both limbs accumulate here
#pragma unroll
  for (int t = 0; t < TMAX; ++t)
#pragma unroll
    for (int q = 0; q < NMAT; ++q) acc[t][q] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  const uint32_t magic = 0x64006400u;
  const int npass = (K + PASS_K - 1) / PASS_K;
  // acc holds the sums times 2^e_acc.  e_acc is a running exponent: the
  // prescale_exponent of the largest |x| the wave has seen so far (passes of
  // zeros leave it alone), so it only falls and acc is only ever scaled down.
  int e_acc = 1 << 20;
  for (int pass = 0; pass < npass; ++pass) {
    const int k0 = pass * PASS_K + wave * SLICE;
    if (k0 >= K) break;                  // wave-uniform: the rest of K is past the end
    const bool all_live = k0 + SLICE <= K;

    // ---- x slice: row r of chunk h is one 1 KB load (16 bytes per lane) ----
    float4 xq[CPW][XR];
#pragma unroll
    for (int h = 0; h < CPW; ++h)
#pragma unroll
      for (int r = 0; r < XR; ++r) {
        const uint32_t off = (uint32_t(r) * uint32_t(K) + uint32_t(k0 + 256 * h + 4 * lane)) * 4u;
        xq[h][r] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
      }
    __builtin_amdgcn_sched_barrier(0);

    // ---- weights: tile t's code words and scales, PF tiles in flight -------
    // The MFMA wants lane (col, g) to hold column col's codes for k-group g,
    // so a quarter-wave (fixed g) would touch 16 weight rows, 16 bytes each:
    // 64 cache-line accesses per load, about seven times the texture-unit
    // time of a contiguous 1 KB load.  So the loads use another lane order --
    // quarter-wave qq reads rows 4qq .. 4qq+3 in full (4 rows x 64 bytes) --
    // and the words are moved to the MFMA order with lane permutes when the
    // tile is computed.  Load lane (row r, piece p) holds words 4p .. 4p + 3
    // of the row's chunk (TQ2; Q1: words 2p, 2p + 1) and the scale of block
    // p >> 1.  Lane (col, g) takes the first half of its registers from piece
    // g and the second half from piece g ^ 2 of row col: for g < 2 that is
    // block 0's words, then block 1's; for g >= 2 the other way round, and a
    // select puts them in block order.  The two scales come from pieces 0
    // and 2.
    const int lrow = 4 * (lane >> 4) + ((lane >> 2) & 3);
    const int lpiece = lane & 3;
    const int perm_row = 4 * (16 * (col >> 2) + 4 * (col & 3));
    const int perm_a = perm_row + 4 * g;
    const int perm_b = perm_row + 4 * (g ^ 2);
    const bool swap_blocks = g >= 2;
    const int kbase[2] = {32 * (2 * (g & 1) + (g >> 1)), 128 + 32 * (2 * (g & 1) + 1 - (g >> 1))};
    codes_t cw[PF][NMAT][CPW];
    uint32_t dr[PF][NMAT][CPW];
    auto load_tile = [&](int t, codes_t (&c)[NMAT][CPW], uint32_t (&d)[NMAT][CPW]) {
      const uint32_t n = uint32_t(16 * (tile0 + min(t, ntile - 1)) + lrow);
#pragma unroll
      for (int q = 0; q < NMAT; ++q)
#pragma unroll
        for (int h = 0; h < CPW; ++h) {
          const uint32_t kk = uint32_t(k0 + 256 * h + 64 * lpiece);
          const uint32_t off = n * row_bytes + kk / 8u * uint32_t(BITS);
          if constexpr (QW == 4) {
            const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rc[q], off, 0, 0);
            c[q][h][0] = v[0]; c[q][h][1] = v[1]; c[q][h][2] = v[2]; c[q][h][3] = v[3];
          } else {
            const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rc[q], off, 0, 0);
            c[q][h][0] = v[0]; c[q][h][1] = v[1];
          }
          d[q][h] = __builtin_amdgcn_raw_buffer_load_b16(rs[q], (n * uint32_t(KB) + (kk >> 7)) * 2u,
                                                         0, 0);
        }
    };
#pragma unroll
    for (int t = 0; t < PF; ++t) load_tile(t, cw[t], dr[t]);
    __builtin_amdgcn_sched_barrier(0);   // weights in flight while x is converted

    // ---- x fragments: hi = binary16(x 2^e) (RNE), lo = binary16(x 2^e - hi) --
    // Positions past K are zeroed (a partial last slice).  One power of two
    // 2^e per wave and pass scales x before the split: e is the running
    // exponent, lowered to the prescale_exponent of this slice's largest |x|
    // (over all rows) when that is smaller; acc is brought down to it.
    // SKIP: rows past M are neither measured nor staged.  Their LDS rows
    // keep whatever they held, which reaches only rows of D that are not
    // stored.  The test is a bit mask over the rows past the instance's
    // smallest M, rather than r < M (which the compiler turns into a variable
    // trip count, keeping the loop rolled); without SKIP there is no test.
    const uint32_t xrows = SKIP ? (M >= XR ? ~0u : (1u << M) - 1u) | ((1u << (PACK ? 2 : 9)) - 1u) : ~0u;
    float mx = 0.f;
#pragma unroll
    for (int h = 0; h < CPW; ++h) {
      const bool live = all_live || k0 + 256 * h + 4 * lane < K;
      float mh = 0.f;
#pragma unroll
      for (int r = 0; r < XR; ++r) {
        if ((xrows >> r) & 1u) {         // wave-uniform
          const float4 v = xq[h][r];
          mh = max3_abs(mh, v.x, v.y);
          mh = max3_abs(mh, v.z, v.w);
        }
      }
      mx = max3_abs(mx, live ? mh : 0.f, 0.f);
    }
    const float mr = wave_max_nonneg_bits(mx);
    const int e = mr > 0.f ? min(e_acc, prescale_exponent(mr)) : e_acc;
    if (pass > 0 && e != e_acc) {        // wave-uniform; acc only ever scaled down (zero in pass 0)
#pragma unroll
      for (int t = 0; t < TMAX; ++t)
#pragma unroll
        for (int q = 0; q < NMAT; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[t][q][i] = __builtin_amdgcn_ldexpf(acc[t][q][i], e - e_acc);
    }
    e_acc = e;
    // Lane l converts k = 4l .. 4l+3 of each row into LDS row r (hi) and row
    // XR + r (lo); each lane then reads its fragments back.  A later chunk
    // reuses the region once the previous chunk's reads have completed.
    half8_t xf[CPW][8][LIMBS];
#pragma unroll
    for (int h = 0; h < CPW; ++h) {
      if (h > 0) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const bool live = all_live || k0 + 256 * h + 4 * lane < K;
      const uint32_t keep = live ? 0xFFFFFFFFu : 0u;
      auto stage_row = [&](int r) {
        float4 v = xq[h][r];
        if (!all_live) {                 // wave-uniform
          v.x = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v.x) & keep);
          v.y = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v.y) & keep);
          v.z = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v.z) & keep);
          v.w = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v.w) & keep);
        }
        uint32_t hi[2], lo[2];
        split_limbs(__builtin_amdgcn_ldexpf(v.x, e), __builtin_amdgcn_ldexpf(v.y, e), hi[0], lo[0]);
        split_limbs(__builtin_amdgcn_ldexpf(v.z, e), __builtin_amdgcn_ldexpf(v.w, e), hi[1], lo[1]);
        *reinterpret_cast<u32x2_t*>(&xs[r * kLdsRow + 4 * lane]) = u32x2_t{hi[0], hi[1]};
        *reinterpret_cast<u32x2_t*>(&xs[(XR + r) * kLdsRow + 4 * lane]) = u32x2_t{lo[0], lo[1]};
      };
#pragma unroll
      for (int r = 0; r < XR; ++r)
        if ((xrows >> r) & 1u) stage_row(r);   // wave-uniform
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int st = 0; st < 8; ++st)
#pragma unroll
        for (int l = 0; l < LIMBS; ++l)
          xf[h][st][l] = *reinterpret_cast<const half8_t*>(
              &xs[(16 * l + col) * kLdsRow + kbase[st >> 2] + 8 * (st & 3)]);
    }

    // ---- stream the tiles ----------------------------------------------------
    constexpr int BW = QW / 2;               // code words per lane and block
    auto compute = [&](int t, const codes_t (&c)[NMAT][CPW], const uint32_t (&d)[NMAT][CPW]) {
#pragma unroll
      for (int q = 0; q < NMAT; ++q)
#pragma unroll
        for (int h = 0; h < CPW; ++h) {
          // Block b of the chunk is past K as a whole or not at all (K is a
          // multiple of 128); its scale is then taken as 0 (its x is zero).
          float dv[2];
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            const bool live = all_live || k0 + 256 * h + 128 * b < K;
            const uint32_t draw = uint32_t(__builtin_amdgcn_ds_bpermute(perm_row + 8 * b, int(d[q][h])));
            dv[b] = live ? float(__builtin_bit_cast(_Float16, uint16_t(draw & 0xFFFFu))) : 0.f;
          }
          uint32_t raw[QW], cb[2][BW];
#pragma unroll
          for (int i = 0; i < QW; ++i)
            raw[i] = uint32_t(__builtin_amdgcn_ds_bpermute(i < BW ? perm_a : perm_b, int(c[q][h][i])));
#pragma unroll
          for (int i = 0; i < BW; ++i) {
            cb[0][i] = swap_blocks ? raw[BW + i] : raw[i];
            cb[1][i] = swap_blocks ? raw[i] : raw[BW + i];
          }
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            floatx4_t D = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              half8_t w8;
              if constexpr (F == Fmt::kQ1) {
                // +-1: the complemented word puts the sign on the weights whose bit is 0.
                w8 = decode_step_q1(~cb[b][0], 4 * s, 0x3C003C00u);
              } else {
                uint32_t w = cb[b][s >> 1];
                if (s & 1) w >>= 8;
                w8 = decode_step_unit(w, magic);
              }
#pragma unroll
              for (int l = 0; l < LIMBS; ++l)
                D = __builtin_amdgcn_mfma_f32_16x16x32_f16(xf[h][4 * b + s][l], w8, D, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[t][q][i] = __builtin_fmaf(dv[b], D[i], acc[t][q][i]);
          }
        }
    };
    // Every block computes TMAX tiles; in the last block the tiles past the
    // end repeat its last tile (results not stored), so that no branch
    // splits the load stream.
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      const int slot = t % PF;
      compute(t, cw[slot], dr[slot]);
      if (t + PF < TMAX) load_tile(t + PF, cw[slot], dr[slot]);
    }
  }

  // ---- the waves' partial sums meet in LDS -----------------------------------
  // acc holds D[m = 4g + e][n = col] of each tile (x is the MFMA's row
  // operand).  red[wave][tile][gate/up][e][lane].
  __syncthreads();                       // every wave is done with its x region
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int t = 0; t < TMAX; ++t)
#pragma unroll
    for (int q = 0; q < NMAT; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        red[(((wave * TMAX + t) * NMAT + q) * 4 + e) * 64 + lane] =
            __builtin_amdgcn_ldexpf(acc[t][q][e], -e_acc);
  __syncthreads();
  // Thread o of the block finishes output (m, tile t, column c): consecutive
  // threads take consecutive columns of one row, so the stores coalesce.
  const int cols = ntile * 16;
  const int rows = min(M, XR);
  for (int o = tid; o < rows * cols; o += THREADS) {
    const int m = o / cols;
    const int rem = o - m * cols;
    const int t = rem >> 4;
    const int c = rem & 15;
    const int n = 16 * (tile0 + t) + c;
    if (n >= N) continue;
    const int ln = c + 16 * (m >> 2);    // PACK: the lo limbs are rows m + 8, lanes ln + 32
    const int e = m & 3;
    float v[NMAT];
#pragma unroll
    for (int q = 0; q < NMAT; ++q) {
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        const float* rw = &red[(((w * TMAX + t) * NMAT + q) * 4 + e) * 64];
        sum += PACK ? rw[ln] + rw[ln + 32] : rw[ln];
      }
      v[q] = sum;
    }
    const size_t oi = size_t(m) * N + n;
    float r;
    if constexpr (SWIGLU) {
      r = silu(v[0]) * v[1];
    } else {
      r = v[0];
      if (residual) r = residual[oi] + r;
    }
    out[oi] = r;
  }
}

// ---------------------------------------------------------------------------
// Ping-pong variant for large M.  Eight waves, two groups of four; wave w and
// wave w + 4 share a SIMD.  Both groups own the same MT x 4NW output tile and
// the same columns per wave (wn = w & 3); group p takes MFMA steps 4p .. 4p+3
// of every 256-wide chunk.  The groups run half a chunk apart: while one group
// issues its chunk's 72 MFMAs (at raised wave priority, operands ready:
// weights decoded beforehand into registers, x fragments read from LDS one
// step ahead), the other group does the memory work -- decodes its weights
// for its next MFMA phase, converts and stores its half of the next x tile,
// and issues the global loads one chunk ahead.  A barrier separates the
// phases, so each SIMD's matrix core alternates between its two waves while
// the VALU, LDS and load path work for the other.
//
// Phase order (chunk c):  A: group 0 MFMA(c), group 1 MEM;  B: group 1
// MFMA(c), group 0 MEM.  x tile c + 1 is stored in two halves, by group 1 in
// phase A and by group 0 in phase B, into the buffer nobody reads during
// chunk c.
//
// SWIGLU: waves wn = 0, 1 of each group read gate-weight columns, waves 2, 3
// the same columns of the up weight; the output tile is MT x 2NW.
//
// Scales.  LDS_SCALES (K <= 12288): the block's scales for the whole K are
// loaded into LDS once, before the loop.  Otherwise group 0 loads each
// chunk's scales with its code words and hands group 1's copy over through
// LDS with them; the per-chunk gathers cost about 10% at K <= 12288, so they
// serve only the K the LDS copy cannot hold.
template <int MT, int NW, bool SWIGLU, Fmt F, bool LDS_SCALES>
__global__ __launch_bounds__(512) void gemm_pp_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const uint8_t* __restrict__ ucodes, const uint8_t* __restrict__ uscales,
    const float* __restrict__ x, const float* __restrict__ residual, float* __restrict__ out,
    int M, int N, int K, int tiles_m, int tiles_n) {
  constexpr int GT = 256;                // threads per group
  constexpr int RT = MT / 16;
  constexpr int CG = NW / 16;
  constexpr int NT = 4 * NW;             // weight rows per block
  constexpr int NO = SWIGLU ? 2 * NW : NT;   // output columns per block
  constexpr int STEPS = 4;               // MFMA steps per group per chunk
  constexpr int BITS = int(F);           // code bits per weight
  constexpr int QW = BITS;               // code dwords per lane per chunk
  constexpr int AV = MT * (kChunk / 4) / 2 / GT;   // float4 of x per thread per chunk
  static_assert(MT % 16 == 0 && NW % 16 == 0, "tile shape");
  static_assert((MT / 2) * (kChunk / 4) % GT == 0, "x staging split");

  __shared__ _Float16 As[2][MT][kLdsRow];
  // LDS_SCALES: the block's scales for the whole K (NT rows of the scales
  // plane, which are contiguous; with SWIGLU 2NW gate rows, then the same 2NW
  // up rows), loaded once.
  __shared__ __attribute__((aligned(16))) uint16_t Ls[LDS_SCALES ? NT * kPpMaxKB : 8];

  const int ntiles = tiles_m * tiles_n;
  int t = blockIdx.x;
  if ((ntiles & 7) == 0) t = (t & 7) * (ntiles >> 3) + (t >> 3);
  const int mt = t / tiles_n;
  const int nt = t - mt * tiles_n;
  const int m0 = mt * MT;
  const int n0 = nt * NO;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int grp = wave >> 2;
  const int wn = wave & 3;
  // Gate or up weight (wave-uniform), and the column share inside it.
  const bool upw = SWIGLU && __builtin_amdgcn_readfirstlane(wn) >= 2;
  const int wc = SWIGLU ? (wn & 1) : wn;
  const int lane = tid & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int gt = tid & (GT - 1);         // thread index inside the group
  const int KB = K >> 7;
  const int nchunks = (K + kChunk - 1) / kChunk;

  const rsrc_t rx = make_rsrc(x + size_t(m0) * K, uint32_t(min(MT, M - m0)) * uint32_t(K) * 4u);
  const uint32_t row_bytes = uint32_t(K / 8) * uint32_t(BITS);   // codes per weight row
  const rsrc_t rc = make_rsrc(upw ? ucodes : codes, uint32_t(N) * row_bytes);
  const rsrc_t rs = make_rsrc(upw ? uscales : scales, uint32_t(N) * uint32_t(KB) * 2u);

  // x staging: group p converts rows p*MT/2 .. p*MT/2 + MT/2 - 1 of a chunk;
  // its thread gt handles float4 f = gt + GT*i: row f / 64, float4 f % 64.
  constexpr int AROWS = GT / 64;
  const int arow0 = grp * (MT / 2) + (gt >> 6);
  const uint32_t aoff = uint32_t(arow0) * uint32_t(K) * 4u + 16u * uint32_t(gt & 63);
  float4 areg[AV];
  auto load_a = [&](int c, int lo, int hi) {
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      if (i < lo || i >= hi) continue;
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(
          rx, aoff + uint32_t(i * AROWS * K * 4 + c * kChunk * 4), 0, 0);
      areg[i] = __builtin_bit_cast(float4, v);
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const float4 v = areg[i];
      half4_t h = {_Float16(v.x), _Float16(v.y), _Float16(v.z), _Float16(v.w)};
      *reinterpret_cast<half4_t*>(&As[buf][arow0 + AROWS * i][4 * (gt & 63)]) = h;
    }
  };

  // Weights: lane's column and k-group g.  Group 0 loads the code words of
  // both groups' halves of the steps (one 2*QW-dword load per column group,
  // twice the bytes per instruction of a per-group load), without LDS_SCALES
  // also the raw binary16 scale of the block they fall in (block
  // 2c + (g >> 1), the same for both halves), and hands group 1's half (and
  // the scale) over through LDS one phase later; group 1 issues no weight
  // loads.  cw[j][0 .. QW) is the calling group's half.  Columns past N read
  // as zero codes and zero scales; chunks past the end read the next row's
  // bytes, which the caller masks (decode_all zeroes d where k runs past K).
  const uint32_t nl = uint32_t(n0 + wc * NW + col);
  const uint32_t code_voff = nl * row_bytes + 8u * BITS * uint32_t(g);
  const uint32_t scale_voff = (nl * uint32_t(KB) + uint32_t(g >> 1)) * 2u;
  uint32_t cw[CG][2 * QW];
  uint32_t dsc[CG];                            // raw binary16 scale bits
  __shared__ uint32_t Hw[4 * CG * 64 * QW];    // hand-over: [wn][j][lane][QW]
  __shared__ uint16_t Hd[LDS_SCALES ? 8 : 4 * CG * 64];   // scale hand-over: [wn][j][lane]
  auto load_w = [&](int c) {                   // group 0
#pragma unroll
    for (int j = 0; j < CG; ++j) {
      const uint32_t off = code_voff + uint32_t(j * 16) * row_bytes + uint32_t(c * 32 * BITS);
      if constexpr (QW == 2) {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rc, off, 0, 0);
        cw[j][0] = v[0]; cw[j][1] = v[1]; cw[j][2] = v[2]; cw[j][3] = v[3];
      } else {
        const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rc, off, 0, 0);
        cw[j][0] = v[0]; cw[j][1] = v[1];
      }
      if constexpr (!LDS_SCALES)
        dsc[j] = __builtin_amdgcn_raw_buffer_load_b16(
            rs, scale_voff + uint32_t(j * 16 * KB * 2 + c * 4), 0, 0);
    }
  };
  auto hand_over = [&]() {                     // group 0: group 1's half into LDS
#pragma unroll
    for (int j = 0; j < CG; ++j) {
      uint32_t* h = &Hw[((wn * CG + j) * 64 + lane) * QW];
      if constexpr (QW == 2)
        *reinterpret_cast<u32x2_t*>(h) = u32x2_t{cw[j][2], cw[j][3]};
      else
        *h = cw[j][1];
      if constexpr (!LDS_SCALES) Hd[(wn * CG + j) * 64 + lane] = uint16_t(dsc[j]);
    }
  };
  auto take_over = [&]() {                     // group 1: its half from LDS
#pragma unroll
    for (int j = 0; j < CG; ++j) {
      const uint32_t* h = &Hw[((wn * CG + j) * 64 + lane) * QW];
      if constexpr (QW == 2) {
        const u32x2_t v = *reinterpret_cast<const u32x2_t*>(h);
        cw[j][0] = v[0]; cw[j][1] = v[1];
      } else {
        cw[j][0] = *h;
      }
      if constexpr (!LDS_SCALES) dsc[j] = Hd[(wn * CG + j) * 64 + lane];
    }
  };
  // LDS_SCALES: scale of this lane's column j and chunk c, block 2c + (g >> 1).
  // The chunk is clamped so the read stays inside Ls for the pass past the
  // end; with an odd block count the last chunk's second block reads the
  // next row's first scale (still inside Ls, since KB < kPpMaxKB), and the
  // caller zeroes it.
  const int ls_base = (wn * NW + col) * KB + (g >> 1);
  auto scale_bits = [&](int j, int c) -> uint32_t {
    if constexpr (LDS_SCALES) return Ls[ls_base + j * 16 * KB + 2 * min(c, nchunks - 1)];
    return dsc[j];
  };

  // Decoded weight operands of one MFMA phase.  The memory phase decodes
  // steps 0 .. STEPS-2 and keeps the code word and scale pair of the last
  // step, which the MFMA phase decodes itself between its MFMAs (one column
  // group per step), so that the two phases carry similar VALU work.
  const uint32_t magic = 0x64006400u;
  half8_t bf[STEPS][CG];
  uint32_t wlast[CG];
  half2_t dlast[CG];
  auto decode_all = [&](int c) {
    const bool live = c * kChunk + 64 * g < K && c < nchunks;
#pragma unroll
    for (int j = 0; j < CG; ++j) {
      const _Float16 d =
          live ? __builtin_bit_cast(_Float16, uint16_t(scale_bits(j, c))) : _Float16(0.0f);
      if constexpr (F == Fmt::kQ1) {
        // One word holds the four steps; dlast carries the |d| pair's bits.
        const uint32_t db = __builtin_bit_cast(uint16_t, d);
        const uint32_t da = q1_dabs2(db);
        const uint32_t w = cw[j][0] ^ q1_fold(db);
#pragma unroll
        for (int ss = 0; ss < STEPS - 1; ++ss) bf[ss][j] = decode_step_q1(w, 4 * ss, da);
        wlast[j] = w;
        dlast[j] = __builtin_bit_cast(half2_t, da);
      } else {
        const half2_t d2 = {d, d};
#pragma unroll
        for (int ss = 0; ss < STEPS - 1; ++ss) {
          uint32_t w = cw[j][ss >> 1];
          if (ss & 1) w >>= 8;
          bf[ss][j] = decode_step(w, d2, magic);
        }
        wlast[j] = cw[j][(STEPS - 1) >> 1] >> 8;
        dlast[j] = d2;
      }
    }
  };

  floatx4_t acc[RT][CG];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < CG; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  auto load_afrags = [&](int buf, int s, half8_t (&a)[RT]) {
#pragma unroll
    for (int i = 0; i < RT; ++i)
      a[i] = *reinterpret_cast<const half8_t*>(&As[buf][i * 16 + col][64 * g + 8 * s]);
  };
  auto mfmas = [&](const half8_t (&a)[RT], const half8_t (&b)[CG]) {
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int j = 0; j < CG; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b[j], a[i], acc[i][j], 0, 0, 0);
  };
  // MFMA phase: x fragments of step ss + 1 are read while step ss's MFMAs
  // issue (one LDS read per CG MFMAs), so every read has a step to land.
  // The MFMA phase also issues the second half of the x loads for chunk
  // ca (the chunk this group stores in its next memory phase), spread over
  // its first steps, so the memory phase issues fewer loads in one burst.
  auto mfma_phase = [&](int c, int ca) {
    const int buf = c & 1;
    __builtin_amdgcn_s_setprio(1);
    half8_t a0[RT], a1[RT];
    load_afrags(buf, grp * STEPS, a0);
    load_a(ca, AV / 2, AV);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ss = 0; ss < STEPS; ++ss) {
      if ((ss & 1) == 0) {
        if (ss + 1 < STEPS) load_afrags(buf, grp * STEPS + ss + 1, a1);
        mfmas(a0, bf[ss]);
      } else {
        if (ss + 1 < STEPS) load_afrags(buf, grp * STEPS + ss + 1, a0);
        mfmas(a1, bf[ss]);
      }
      // Last step's operands, one column group per earlier step.
#pragma unroll
      for (int j = 0; j < CG; ++j)
        if (ss == (j * (STEPS - 1)) / CG) {
          if constexpr (F == Fmt::kQ1)
            bf[STEPS - 1][j] = decode_step_q1(wlast[j], 4 * (STEPS - 1),
                                              __builtin_bit_cast(uint32_t, dlast[j]));
          else
            bf[STEPS - 1][j] = decode_step(wlast[j], dlast[j], magic);
        }
#pragma unroll
      for (int q = 0; q < RT * CG; ++q) {
        if (q % CG == 0 && ss + 1 < STEPS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (ss + 1 < STEPS) __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // Pin the decoded operands (and so all decode arithmetic) before the
  // barrier that ends a memory phase; register-only work could otherwise
  // drift past it into the MFMA phase.
  auto pin_operands = [&]() {
#pragma unroll
    for (int ss = 0; ss < STEPS - 1; ++ss)
#pragma unroll
      for (int j = 0; j < CG; ++j) asm volatile("" ::"v"(bf[ss][j]));
#pragma unroll
    for (int j = 0; j < CG; ++j) asm volatile("" ::"v"(wlast[j]), "v"(dlast[j]));
  };
  // Memory phase of group 0: decode chunk cd's weights (loaded one chunk
  // ago), hand group 1's half of them over, store this group's half of x
  // chunk cs, then load x chunk cs + 1 and weight chunk cw_next.
  auto mem_phase0 = [&](int cd, int cs, int cw_next) {
    decode_all(cd);
    hand_over();
    store_a(cs & 1);
    load_a(cs + 1, 0, AV / 2);
    load_w(cw_next);
    pin_operands();
  };
  // Memory phase of group 1: take chunk cd's words over from LDS (written by
  // group 0 in the previous phase) and decode them, store x chunk cs, load
  // x chunk cs + 1.
  auto mem_phase1 = [&](int cd, int cs) {
    take_over();
    decode_all(cd);
    store_a(cs & 1);
    load_a(cs + 1, 0, AV / 2);
    pin_operands();
  };

  // Prologue: (LDS_SCALES) the block's scales into LDS; x tile 0 complete in
  // buffer 0; group 0's operands for chunk 0 decoded, group 1's half of
  // chunk 0 (and its scales) handed over, and weight chunk 1 in flight.  Both
  // groups hold their half of x chunk 1 in registers.
  if constexpr (LDS_SCALES) {
    // 16-byte loads for the whole granules (a load that straddles the end
    // of a buffer resource returns zeros in full), 2-byte loads for the tail.
    // Entries for columns past N are left unset: their outputs are never
    // stored.
    auto preload = [&](const uint8_t* plane, int rows, int dst) {
      const uint32_t valid = uint32_t(min(rows, N - n0)) * uint32_t(KB) * 2u;
      const uint32_t full = valid & ~15u;
      const rsrc_t rsb = make_rsrc(plane + size_t(n0) * KB * 2, valid);
      uint8_t* ls = reinterpret_cast<uint8_t*>(Ls + dst);
      for (uint32_t o = 16u * uint32_t(tid); o < full; o += 16u * 512u) {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rsb, o, 0, 0);
        *reinterpret_cast<u32x4_t*>(ls + o) = v;
      }
      const uint32_t o2 = full + 2u * uint32_t(tid);
      if (o2 < valid)
        *reinterpret_cast<uint16_t*>(ls + o2) = __builtin_amdgcn_raw_buffer_load_b16(rsb, o2, 0, 0);
    };
    if constexpr (SWIGLU) {
      // Gate rows at Ls row 0, up rows at Ls row 2NW: 2NW * KB * 2 bytes is a
      // multiple of 16 (NW is a multiple of 16), so both halves stay aligned.
      preload(scales, 2 * NW, 0);
      preload(uscales, 2 * NW, 2 * NW * KB);
    } else {
      preload(scales, NT, 0);
    }
  }
  load_a(0, 0, AV);
  if (grp == 0) load_w(0);
  store_a(0);
  load_a(1, 0, AV);
  lds_barrier();                         // LDS_SCALES: scales visible
  if (grp == 0) {
    decode_all(0);
    hand_over();
    load_w(1);
    pin_operands();
  }
  lds_barrier();
  if (grp == 0) {
    for (int c = 0; c < nchunks; ++c) {
      mfma_phase(c, c + 1);
      lds_barrier();
      mem_phase0(c + 1, c + 1, c + 2);
      lds_barrier();
    }
  } else {
    for (int c = 0; c < nchunks; ++c) {
      mem_phase1(c, c + 1);
      lds_barrier();
      mfma_phase(c, c + 2);
      lds_barrier();
    }
  }

  // ---- epilogue ----------------------------------------------------------------
  // Group 1 hands its partial sums to group 0 through LDS (and, for SwiGLU,
  // group 0's up waves hand theirs to the gate waves).  The finished MT x NO
  // tile is then laid out row-major in LDS, and all 512 threads store it in
  // whole rows, 16 bytes per lane, reading the residual the same way.
  float* red = reinterpret_cast<float*>(&As[0][0][0]);
  static_assert(4 * RT * CG * 4 * 64 * 4 <= sizeof(As), "reduction buffer");
  if (grp == 1) {
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int j = 0; j < CG; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          red[(((wn * RT + i) * CG + j) * 4 + e) * 64 + lane] = acc[i][j][e];
  }
  __syncthreads();
  if (grp == 0) {
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int j = 0; j < CG; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[i][j][e] += red[(((wn * RT + i) * CG + j) * 4 + e) * 64 + lane];
  }
  if constexpr (SWIGLU) {
    // Each up wave overwrites only the slots its own lanes have just read.
    if (grp == 0 && upw) {
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < CG; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            red[(((wn * RT + i) * CG + j) * 4 + e) * 64 + lane] = acc[i][j][e];
    }
    __syncthreads();
    if (grp == 0 && !upw) {
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < CG; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[i][j][e] =
                silu(acc[i][j][e]) * red[((((wn + 2) * RT + i) * CG + j) * 4 + e) * 64 + lane];
    }
  }

  // Row-major staging: D[n = 4g + e][m = col] of each 16 x 16 result goes to
  // tile row i * 16 + col, columns wc * NW + j * 16 + 4g .. + 3.
  constexpr int TP = NO + 4;             // tile row pitch in floats
  static_assert(MT * TP * 4 <= sizeof(As), "output tile");
  float* tile = red;
  __syncthreads();                       // every read of the reduction slots is done
  if (grp == 0 && !upw) {
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int j = 0; j < CG; ++j)
        *reinterpret_cast<float4*>(&tile[(i * 16 + col) * TP + wc * NW + j * 16 + 4 * g]) =
            make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
  }
  __syncthreads();
  store_tile<MT, NO, 512>(tile, tid, m0, n0, M, N, residual, out);
}

// `up` is null for the plain matmul; with SWIGLU, `soa` is the gate weight.
template <int MT, int NW, bool SWIGLU, Fmt F, bool LDS_SCALES>
hipError_t launch_pp(const uint8_t* soa, const uint8_t* up, const float* x,
                     const float* residual, float* out, int64_t m, int64_t n, int64_t k,
                     hipStream_t stream) {
  constexpr int NO = SWIGLU ? 2 * NW : 4 * NW;
  const int64_t tm = (m + MT - 1) / MT;
  const int64_t tn = (n + NO - 1) / NO;
  if (tm * tn > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid(unsigned(tm * tn));
  const size_t so = scales_offset(F, n, k);
  hipLaunchKernelGGL((gemm_pp_kernel<MT, NW, SWIGLU, F, LDS_SCALES>), grid, dim3(512), 0, stream, soa, soa + so,
                     up, up ? up + so : nullptr, x, residual, out, int(m), int(n), int(k), int(tm),
                     int(tn));
  return hipGetLastError();
}

template <int MT, int NW, int WN, int WK, int LIMBS, bool SWIGLU, Fmt F>
hipError_t launch_tile(const uint8_t* soa, const uint8_t* up, const float* x,
                       const float* residual, float* out, int64_t m, int64_t n, int64_t k,
                       hipStream_t stream) {
  constexpr int NO = SWIGLU ? WN / 2 * NW : WN * NW;
  const int64_t tm = (m + MT - 1) / MT;
  const int64_t tn = (n + NO - 1) / NO;
  if (tm * tn > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int tiles_m = int(tm), tiles_n = int(tn);
  const dim3 grid(unsigned(tm * tn));
  const size_t so = scales_offset(F, n, k);
  hipLaunchKernelGGL((gemm_kernel<MT, NW, WN, WK, LIMBS, SWIGLU, F>), grid, dim3(64 * WN * WK), 0,
                     stream, soa, soa + so, up, up ? up + so : nullptr, x, residual, out, int(m),
                     int(n), int(k), tiles_m, tiles_n);
  return hipGetLastError();
}

// Skinny kernel: TMAX 16-column tiles per block, so that about one block
// per CU covers N (at most 4 tiles per block; more blocks beyond that).
template <int TMAX, bool SWIGLU, Fmt F>
hipError_t launch_skinny(const uint8_t* soa, const uint8_t* up, const float* x,
                         const float* residual, float* out, int64_t m, int64_t n, int64_t k,
                         hipStream_t stream) {
  const int64_t tiles = (n + 15) / 16;
  const int64_t blocks = (tiles + TMAX - 1) / TMAX;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const size_t so = scales_offset(F, n, k);
  const dim3 grid(static_cast<unsigned>(blocks));
  // M <= 8 packs both limbs into one MFMA column set and stages 8 x rows per
  // wave, so 16 waves (one 256-wide chunk each) fit the LDS; M <= 16 uses 8.
  // Where at least a quarter of the staged rows would be padding (M <= 4 of
  // 8, M <= 12 of 16) the instance skips the rows past M; with fewer, the
  // per-row tests cost more than the rows they save (measured).
  if (m <= 4)
    hipLaunchKernelGGL((gemm_skinny_kernel<TMAX, 16, true, SWIGLU, F, true>), grid, dim3(1024), 0,
                       stream, soa, soa + so, up, up ? up + so : nullptr, x, residual, out, int(m),
                       int(n), int(k));
  else if (m <= 8)
    hipLaunchKernelGGL((gemm_skinny_kernel<TMAX, 16, true, SWIGLU, F, false>), grid, dim3(1024), 0,
                       stream, soa, soa + so, up, up ? up + so : nullptr, x, residual, out, int(m),
                       int(n), int(k));
  else if (m <= 12)
    hipLaunchKernelGGL((gemm_skinny_kernel<TMAX, 8, false, SWIGLU, F, true>), grid, dim3(512), 0,
                       stream, soa, soa + so, up, up ? up + so : nullptr, x, residual, out, int(m),
                       int(n), int(k));
  else
    hipLaunchKernelGGL((gemm_skinny_kernel<TMAX, 8, false, SWIGLU, F, false>), grid, dim3(512), 0,
                       stream, soa, soa + so, up, up ? up + so : nullptr, x, residual, out, int(m),
                       int(n), int(k));
  return hipGetLastError();
}

template <bool SWIGLU, Fmt F>
hipError_t dispatch_skinny(const uint8_t* soa, const uint8_t* up, const float* x,
                           const float* residual, float* out, int64_t m, int64_t n, int64_t k,
                           hipStream_t stream) {
  constexpr int64_t kCus = 256;
  const int64_t tiles = (n + 15) / 16;
  const int64_t want = (tiles + kCus - 1) / kCus;
  const int tpb = int(want < 4 ? want : 4);
  if (tpb <= 1) return launch_skinny<1, SWIGLU, F>(soa, up, x, residual, out, m, n, k, stream);
  if (tpb == 2) return launch_skinny<2, SWIGLU, F>(soa, up, x, residual, out, m, n, k, stream);
  if (tpb == 3) return launch_skinny<3, SWIGLU, F>(soa, up, x, residual, out, m, n, k, stream);
  return launch_skinny<4, SWIGLU, F>(soa, up, x, residual, out, m, n, k, stream);
}

// Kernel choice by path and M (shared by the plain and the SwiGLU forms).
template <bool SWIGLU, Fmt F>
hipError_t dispatch(int path, const uint8_t* soa, const uint8_t* up, const float* x,
                    const float* residual, float* out, int64_t m, int64_t n, int64_t k,
                    hipStream_t stream) {
  if (path == 1) {
    // Split-binary16 (f32-class) kernels: the skinny kernel up to M = 16,
    // 64-row tiles beyond (tq2_gemm_precise), so each weight is decoded once
    // per 64 rows of x.
    if (m <= 16) return dispatch_skinny<SWIGLU, F>(soa, up, x, residual, out, m, n, k, stream);
    return launch_tile<64, 16, 4, 2, 2, SWIGLU, F>(soa, up, x, residual, out, m, n, k, stream);
  }
  if (m <= 128) {
    // One row block of the smallest 32-row multiple that covers M, on the
    // warp-specialised kernel: x rows past M read zeros and their output
    // rows are not stored.
    if (k <= int64_t(kPpMaxKB) * kBlockWeights) {
      switch ((m + 31) / 32) {
        case 1: return launch_sp<32, 32, 2, 8, SWIGLU, F, true>(soa, up, x, residual, out, m, n, k, stream);
        case 2: return launch_sp<64, 32, 2, 8, SWIGLU, F, true>(soa, up, x, residual, out, m, n, k, stream);
        case 3: return launch_sp<96, 32, 2, 8, SWIGLU, F, true>(soa, up, x, residual, out, m, n, k, stream);
        default:
          // Up to M = 104, eight x waves of 13 rows cover M with fewer loads.
          if (m <= 104)
            return launch_sp<128, 32, 2, 8, SWIGLU, F, true, 13>(soa, up, x, residual, out, m, n, k, stream);
          return launch_sp<128, 32, 2, 8, SWIGLU, F, true>(soa, up, x, residual, out, m, n, k, stream);
      }
    }
    switch ((m + 31) / 32) {
      case 1: return launch_sp<32, 32, 2, 8, SWIGLU, F, false>(soa, up, x, residual, out, m, n, k, stream);
      case 2: return launch_sp<64, 32, 2, 8, SWIGLU, F, false>(soa, up, x, residual, out, m, n, k, stream);
      case 3: return launch_sp<96, 32, 2, 8, SWIGLU, F, false>(soa, up, x, residual, out, m, n, k, stream);
      default:
        if (m <= 104)
          return launch_sp<128, 32, 2, 8, SWIGLU, F, false, 13>(soa, up, x, residual, out, m, n, k, stream);
        return launch_sp<128, 32, 2, 8, SWIGLU, F, false>(soa, up, x, residual, out, m, n, k, stream);
    }
  }
  if (k <= int64_t(kPpMaxKB) * kBlockWeights)
    return launch_pp<96, 48, SWIGLU, F, true>(soa, up, x, residual, out, m, n, k, stream);
  return launch_pp<96, 48, SWIGLU, F, false>(soa, up, x, residual, out, m, n, k, stream);
}

}  // namespace

hipError_t launch_gemm(int path, const uint8_t* soa, const float* x, const float* residual,
                       float* out, int64_t m, int64_t n, int64_t k, hipStream_t stream) {
  return dispatch<false, Fmt::kTq2>(path, soa, nullptr, x, residual, out, m, n, k, stream);
}

hipError_t launch_gemm_swiglu(int path, const uint8_t* gate, const uint8_t* up, const float* x,
                              float* out, int64_t m, int64_t n, int64_t k, hipStream_t stream) {
  return dispatch<true, Fmt::kTq2>(path, gate, up, x, nullptr, out, m, n, k, stream);
}

hipError_t launch_gemm_q1(int path, const uint8_t* soa, const float* x, const float* residual,
                          float* out, int64_t m, int64_t n, int64_t k, hipStream_t stream) {
  return dispatch<false, Fmt::kQ1>(path, soa, nullptr, x, residual, out, m, n, k, stream);
}

hipError_t launch_gemm_swiglu_q1(int path, const uint8_t* gate, const uint8_t* up,
                                 const float* x, float* out, int64_t m, int64_t n, int64_t k,
                                 hipStream_t stream) {
  return dispatch<true, Fmt::kQ1>(path, gate, up, x, nullptr, out, m, n, k, stream);
}

size_t gemm_ws_bytes(int64_t m, int64_t n, int64_t k) {
  (void)n;
  if (m <= kSplitMaxM || m > kWsMaxM) return 0;
  return ks_workspace_bytes(m, k);
}

hipError_t launch_gemm_ws(const uint8_t* soa, const float* x, const float* residual, float* out,
                          int64_t m, int64_t n, int64_t k, void* ws, hipStream_t stream) {
  return dispatch_ks<Fmt::kTq2>(soa, x, residual, out, m, n, k, ws, stream);
}

}  // namespace tq2
