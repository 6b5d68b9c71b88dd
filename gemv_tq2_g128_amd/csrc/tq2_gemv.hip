// Decode GEMV (M = 1): out[n] = residual[n] + sum_k x[k] * w[n, k].
//
// The pages' decode kernel is `gemv_tq2_g128_v1` (oxibonsai-kernels 0.1.5,
// pipelines.rs, `MetalPipelines`, ternary section); its source is not on the
// pages.  The optional fused residual follows the `gemv_q1_g128_v7_residual`
// entry of the same table.  This kernel is designed for gfx950 on its own.
//
// Work split.  Lane t of a 256-thread block owns one 32-bit code word (16
// consecutive k) of each of ROWS rows; LPS lanes (a power of two >= K/16,
// at most 256) form a row slot, so a block covers 256/LPS slots x ROWS rows.
// For K > 4096 a slot walks K in 4096-wide segments.  A wave therefore reads
// 256 contiguous code bytes per row, and a lane keeps its 16 x values in
// registers for all ROWS rows.
//
// Latency.  The code words and scales of all ROWS rows are loaded with
// branch-free buffer loads before any arithmetic, so one block keeps ROWS
// loads per lane in flight instead of paying the HBM latency per row.  When
// a block is one row slot its rows are block-uniform: each row's offset is a
// scalar operand and the lane's offset is shared by all rows, so the loads
// cost no per-row vector address arithmetic.
// The lane's x values are loaded before them: loads complete in issue order,
// so row r's arithmetic starts as soon as row r's weights have arrived.
//
// Arithmetic (f32 products and sums, weights exact).  One AND-OR puts two
// codes of the word into the mantissas of a binary16 pair 1024 + 4^f c (the
// SoA stores codes k and k+1 at bits 2f and 2f+16, see tq2_internal.h); one
// packed FMA maps it to the exact pair (c - 1); each weight then costs one
// v_fma_mix_f32 (f32 x times binary16 weight, f32 accumulate).  Each lane's
// 16-term sum is scaled by its block's d once; the partial sums of a row are
// added in LDS and with cross-lane shuffles, and the residual is added last.
//
// Q1_g128 weights (the pages' `gemv_q1_g128_v7` / `_residual` decode kernels,
// same table) run the same kernels with F = Fmt::kQ1.  A lane still owns 16
// consecutive weights: half of a 32-bit word (two lanes read the same word;
// the odd one shifts it right by 8).  Each pair's two bits are shifted onto
// the binary16 sign positions and OR-ed with 1.0, giving the exact pair
// ((-1)^b, (-1)^b'), and the 16-term sum is scaled by -d.
#include "tq2_internal.h"
#include "tq2_device.h"

namespace tq2 {
namespace {

constexpr int kThreads = 256;
constexpr uint32_t kMagic = 0x64006400u;   // binary16 pair (1024, 1024)

// The 8 exact binary16 pairs (c_k - 1, c_{k+1} - 1) of one code word.
__device__ __forceinline__ void decode_word(uint32_t w, uint32_t magic, half2_t (&v)[8]) {
  const uint32_t w10 = w >> 10;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int f = p < 5 ? p : p - 5;          // field position inside the half-word
    const uint32_t src = p < 5 ? w : w10;
    const uint32_t mask = (3u << (2 * f)) | (3u << (2 * f + 16));
    const half2_t h = __builtin_bit_cast(half2_t, and_or(src, mask, magic));
    const _Float16 sc = _Float16(1.0f / float(1 << (2 * f)));
    const _Float16 off = _Float16(-(1024.0f / float(1 << (2 * f)) + 1.0f));
    const half2_t scv = {sc, sc};
    const half2_t offv = {off, off};
    v[p] = h * scv + offv;
  }
}

// Sum of v over aligned groups of G consecutive lanes (G a power of two, at
// most 64) with DPP lane moves: xor 1 and 2 (quad permutes), then the 8- and
// 16-lane mirrors, then the row broadcasts of lanes 15 and 31.  Afterwards
// lane G - 1 of each group holds the group's sum.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 2) v += dpp_move<0xB1, 0xF>(v);     // quad_perm [1, 0, 3, 2]
  if constexpr (G >= 4) v += dpp_move<0x4E, 0xF>(v);     // quad_perm [2, 3, 0, 1]
  if constexpr (G >= 8) v += dpp_move<0x141, 0xF>(v);    // row_half_mirror
  if constexpr (G >= 16) v += dpp_move<0x140, 0xF>(v);   // row_mirror
  if constexpr (G >= 32) v += dpp_move<0x142, 0xA>(v);   // row_bcast15 into rows 1 and 3
  if constexpr (G >= 64) v += dpp_move<0x143, 0xC>(v);   // row_bcast31 into rows 2 and 3
  return v;
}

// Code words per weight row, and the code word of lane unit u (16 weights):
// TQ2 word u; Q1 half (u & 1) of word u >> 1, moved to the low byte of each
// half-word so that pair r of the unit sits at bits r and r + 16.
template <Fmt F>
__device__ __forceinline__ int words_per_row(int k) { return F == Fmt::kQ1 ? k >> 5 : k >> 4; }


__device__ __forceinline__ float dot16(const half2_t (&v)[8], const float (&xv)[16]) {
  float s = 0.f;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    s = __builtin_fmaf(xv[2 * p], float(v[p][0]), s);
    s = __builtin_fmaf(xv[2 * p + 1], float(v[p][1]), s);
  }
  return s;
}

// Sum of x[t] * (2 b_t - 1) over the 16 weights of one Q1 unit (exact +-1
// pairs, f32 products and sums).
__device__ __forceinline__ float dot16_q1(uint32_t w, const float (&xv)[16]) {
  const uint32_t one = 0x3C003C00u;             // binary16 pair (1, 1)
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const half2_t v = __builtin_bit_cast(half2_t, and_or(w << (15 - p), 0x80008000u, one));
    s0 = __builtin_fmaf(xv[2 * p], float(v[0]), s0);
    s1 = __builtin_fmaf(xv[2 * p + 1], float(v[1]), s1);
  }
  return -(s0 + s1);                            // (-1)^b = -(2b - 1)
}

// The 16 x values of lane unit wc.
__device__ __forceinline__ void load_x16(const float* __restrict__ x, int wc, float (&xv)[16]) {
  const float4* xp = reinterpret_cast<const float4*>(x + 16 * wc);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 q = xp[i];
    xv[4 * i] = q.x;
    xv[4 * i + 1] = q.y;
    xv[4 * i + 2] = q.z;
    xv[4 * i + 3] = q.w;
  }
}

// The code word holding lane unit u of a row whose words start at byte
// `row_off` (scalar) + `lane_row_off` (per lane) of the resource.
template <Fmt F>
__device__ __forceinline__ uint32_t unit_word_at(rsrc_t rc, uint32_t lane_row_off,
                                                 uint32_t row_off, unsigned u) {
  if constexpr (F == Fmt::kQ1)
    return __builtin_amdgcn_raw_buffer_load_b32(rc, lane_row_off + (u >> 1) * 4u, row_off,
                                                kStreamOnce) >> (8 * (u & 1));
  return __builtin_amdgcn_raw_buffer_load_b32(rc, lane_row_off + u * 4u, row_off, kStreamOnce);
}

// Row `r` of a block whose first row is blk_row0, as an index into the
// block's resources: with one slot per block (SLOTS == 1) r is block-uniform
// and clamped to the last row, so every access stays inside the resource;
// otherwise r is per lane and rows past the end read zeros through the range
// check (their sums are never stored).
template <int SLOTS>
__device__ __forceinline__ uint32_t block_row(int blk_row0, int r, int n_rows) {
  if constexpr (SLOTS == 1) return uint32_t(min(blk_row0 + r, n_rows - 1) - blk_row0);
  return uint32_t(r);
}

// Code word and scale of lane unit u of block row `row`, loaded as a stream
// read once per launch (kStreamOnce).  SLOTS == 1: the
// row's offset is a scalar (the scalar offset operand) and the lane's offset
// is the same for every row, so a row costs no vector address arithmetic.
template <int SLOTS, Fmt F>
__device__ __forceinline__ void load_row(rsrc_t rc, rsrc_t rs, uint32_t row, uint32_t wrow,
                                         uint32_t kb_count, unsigned u, uint32_t& cw,
                                         uint32_t& db) {
  if constexpr (SLOTS == 1) {
    cw = unit_word_at<F>(rc, 0u, row * wrow * 4u, u);
    db = __builtin_amdgcn_raw_buffer_load_b16(rs, (u >> 3) * 2u, row * kb_count * 2u,
                                              kStreamOnce);
  } else {
    cw = unit_word_at<F>(rc, row * wrow * 4u, 0u, u);
    db = __builtin_amdgcn_raw_buffer_load_b16(rs, (row * kb_count + (u >> 3)) * 2u, 0,
                                              kStreamOnce);
  }
}

// Load the 16 x values of lane unit wc (16 weights), then ROWS code words
// and scales of it.  Vector loads return in issue order, so the x loads (L2
// hits) go first: the arithmetic of row 0 then waits only for row 0's
// weights, and each later row's arithmetic overlaps the arrival of the rest.
// The buffer resources start at the block's first row `blk_row0` and cover
// its rows that exist.
template <int ROWS, int SLOTS, Fmt F>
__device__ __forceinline__ void load_segment(const uint32_t* __restrict__ codes,
                                             const uint16_t* __restrict__ scales,
                                             const float* __restrict__ x, int blk_row0,
                                             int slot, int n_rows, int k, int kb_count, int wc,
                                             uint32_t (&cw)[ROWS], uint32_t (&db)[ROWS],
                                             float (&xv)[16]) {
  const unsigned uwc = unsigned(wc);
  const uint32_t wrow = uint32_t(words_per_row<F>(k));
  const uint32_t live_rows = uint32_t(min(SLOTS * ROWS, n_rows - blk_row0));
  const rsrc_t rc = make_rsrc(codes + size_t(blk_row0) * wrow, live_rows * wrow * 4u);
  const rsrc_t rs = make_rsrc(scales + size_t(blk_row0) * uint32_t(kb_count),
                              live_rows * uint32_t(kb_count) * 2u);
  load_x16(x, wc, xv);
  __builtin_amdgcn_sched_barrier(0);            // keep the x loads first
#pragma unroll
  for (int r = 0; r < ROWS; ++r)
    load_row<SLOTS, F>(rc, rs, block_row<SLOTS>(blk_row0, slot * ROWS + r, n_rows), wrow,
                       uint32_t(kb_count), uwc, cw[r], db[r]);
}

template <int ROWS, Fmt F>
__device__ __forceinline__ void accumulate_segment(const uint32_t (&cw)[ROWS],
                                                   const uint32_t (&db)[ROWS],
                                                   const float (&xv)[16], bool live,
                                                   float (&part)[ROWS]) {
  const uint32_t magic = kMagic;
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const float d = float(__builtin_bit_cast(_Float16, uint16_t(db[r])));
    float s;
    if constexpr (F == Fmt::kQ1) {
      s = dot16_q1(cw[r], xv) * d;
    } else {
      half2_t v[8];
      decode_word(cw[r], magic, v);
      s = dot16(v, xv) * d;
    }
    part[r] += live ? s : 0.f;
  }
}

// One block's rows: block `blk` covers rows blk * OUTS .. blk * OUTS + OUTS - 1
// of an [n_rows, k] weight.  ONE_SEG: K/16 <= LPS, the whole row fits one
// pass and every load of the thread is issued before the first use.
template <int ROWS, int LPS, bool ONE_SEG, Fmt F = Fmt::kTq2>
__device__ __forceinline__ void gemv_block(const uint32_t* __restrict__ codes,
                                           const uint16_t* __restrict__ scales,
                                           const float* __restrict__ x,
                                           const float* __restrict__ residual,
                                           float* __restrict__ out, int n_rows, int k, int blk) {
  constexpr int SLOTS = kThreads / LPS;
  constexpr int OUTS = SLOTS * ROWS;            // rows per block
  constexpr int G = kThreads / OUTS;            // threads that finish one row
  static_assert(LPS >= ROWS && G >= 1 && G <= 64, "reduction shape");
  const int t = threadIdx.x;
  // With one slot per block the row indices are block-uniform (scalar).
  const int slot = SLOTS == 1 ? 0 : t / LPS;
  const int lw = SLOTS == 1 ? t : t % LPS;      // word index inside a K segment
  const int wpr = k >> 4;                       // lane units (16 weights) per row
  const int kb_count = k >> 7;
  // The output row this thread finishes (if it is its group's last lane),
  // and its residual, loaded first so that its latency is hidden.
  const int g = t % G;
  const int orow = blk * OUTS + t / G;
  const bool writer = g == G - 1 && orow < n_rows;
  float rres = 0.f;
  if (residual && writer) rres = residual[orow];

  float part[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) part[r] = 0.f;

  uint32_t cw[ROWS];
  uint32_t db[ROWS];
  float xv[16];
  if constexpr (ONE_SEG) {
    if (wpr == LPS) {                           // every lane has a unit: no masking
      load_segment<ROWS, SLOTS, F>(codes, scales, x, blk * OUTS, slot, n_rows, k, kb_count, lw,
                                   cw, db, xv);
      accumulate_segment<ROWS, F>(cw, db, xv, true, part);
    } else {
      const bool live = lw < wpr;
      load_segment<ROWS, SLOTS, F>(codes, scales, x, blk * OUTS, slot, n_rows, k, kb_count,
                                   live ? lw : wpr - 1, cw, db, xv);
      accumulate_segment<ROWS, F>(cw, db, xv, live, part);
    }
  } else {
    for (int seg = 0; seg < wpr; seg += LPS) {
      const int w = seg + lw;
      const bool live = w < wpr;
      load_segment<ROWS, SLOTS, F>(codes, scales, x, blk * OUTS, slot, n_rows, k, kb_count,
                                   live ? w : wpr - 1, cw, db, xv);
      accumulate_segment<ROWS, F>(cw, db, xv, live, part);
    }
  }

  // Row sums: red[r][t] holds thread t's partial of its slot's row r.
  __shared__ float red[ROWS][kThreads];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) red[r][t] = part[r];
  __syncthreads();
  const int o = t / G;                          // block row finished by this thread
  const int os = o / ROWS;                      // its slot
  const int orr = o % ROWS;                     // its row inside the slot
  constexpr int PER = LPS / G;                  // partials summed by one thread
  float v = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) v += red[orr][os * LPS + g * PER + i];
  v = group_sum<G>(v);
  if (writer) {                                 // orow == blk * OUTS + os * ROWS + orr
    if (residual) v = rres + v;
    out[orow] = v;
  }
}

template <int ROWS, int LPS, bool ONE_SEG, Fmt F>
__global__ __launch_bounds__(kThreads) void gemv_kernel(const uint32_t* __restrict__ codes,
                                                        const uint16_t* __restrict__ scales,
                                                        const float* __restrict__ x,
                                                        const float* __restrict__ residual,
                                                        float* __restrict__ out, int n_rows,
                                                        int k) {
  gemv_block<ROWS, LPS, ONE_SEG, F>(codes, scales, x, residual, out, n_rows, k, blockIdx.x);
}

// Several independent GEMVs with the same k in one launch: block b belongs to
// the problem p with first_block[p] <= b < first_block[p + 1].
struct GemvBatchArgs {
  const uint32_t* codes[kGemvBatchMax];
  const uint16_t* scales[kGemvBatchMax];
  const float* x[kGemvBatchMax];
  const float* residual[kGemvBatchMax];
  float* out[kGemvBatchMax];
  int n[kGemvBatchMax];
  int first_block[kGemvBatchMax + 1];
  int count;
};

template <int ROWS, int LPS, bool ONE_SEG>
__global__ __launch_bounds__(kThreads) void gemv_batched_kernel(const GemvBatchArgs args, int k) {
  const int b = blockIdx.x;
  int p = 0;
  while (p + 1 < args.count && args.first_block[p + 1] <= b) ++p;   // uniform scan
  gemv_block<ROWS, LPS, ONE_SEG>(args.codes[p], args.scales[p], args.x[p], args.residual[p],
                                 args.out[p], args.n[p], k, b - args.first_block[p]);
}

// Fused gate/up projections + SwiGLU, decode (M = 1):
//     out[n] = silu(g[n]) * u[n],  g = W_gate x,  u = W_up x,
// silu(z) = z / (1 + e^-z) (oxibonsai-kernels 0.1.5, pipelines.rs,
// `MetalPipelines`: `fused_gate_up_swiglu_q1`, here for ternary weights).
// Lane t owns one code word of 8 rows, as in gemv_block: rows 0..3 of its
// slot's gate weight and the same 4 rows of the up weight, so a block streams
// both weights' rows for its outputs and the finishing thread of output n
// holds g[n] and u[n] together.  Neither projection leaves the chip.
__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

template <int LPS, bool ONE_SEG, Fmt F>
__global__ __launch_bounds__(kThreads) void gemv_swiglu_kernel(
    const uint32_t* __restrict__ gcodes, const uint16_t* __restrict__ gscales,
    const uint32_t* __restrict__ ucodes, const uint16_t* __restrict__ uscales,
    const float* __restrict__ x, float* __restrict__ out, int n_rows, int k) {
  constexpr int HALF = 4;                       // outputs per slot
  constexpr int ROWS = 2 * HALF;                // weight rows per lane
  constexpr int SLOTS = kThreads / LPS;
  constexpr int OUTS = SLOTS * HALF;            // outputs per block
  constexpr int G = kThreads / OUTS;            // threads that finish one output
  static_assert(LPS >= ROWS && G >= 1 && G <= 64, "reduction shape");
  const int t = threadIdx.x;
  const int slot = SLOTS == 1 ? 0 : t / LPS;
  const int lw = SLOTS == 1 ? t : t % LPS;
  const int wpr = k >> 4;                       // lane units (16 weights) per row
  const int wrow = words_per_row<F>(k);
  const int kb_count = k >> 7;

  float part[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) part[r] = 0.f;
  uint32_t cw[ROWS];
  uint32_t db[ROWS];
  float xv[16];
  // Rows 0..HALF-1 from the gate weight, HALF..ROWS-1 from the up weight.
  const int blk_row0 = blockIdx.x * OUTS;
  const uint32_t live_rows = uint32_t(min(OUTS, n_rows - blk_row0));
  const uint32_t uwrow = uint32_t(wrow), ukb = uint32_t(kb_count);
  const rsrc_t rc[2] = {make_rsrc(gcodes + size_t(blk_row0) * uwrow, live_rows * uwrow * 4u),
                        make_rsrc(ucodes + size_t(blk_row0) * uwrow, live_rows * uwrow * 4u)};
  const rsrc_t rs[2] = {make_rsrc(gscales + size_t(blk_row0) * ukb, live_rows * ukb * 2u),
                        make_rsrc(uscales + size_t(blk_row0) * ukb, live_rows * ukb * 2u)};
  auto load = [&](int wc) {
    load_x16(x, wc, xv);                        // x first, as in load_segment
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
      load_row<SLOTS, F>(rc[r / HALF], rs[r / HALF],
                         block_row<SLOTS>(blk_row0, slot * HALF + r % HALF, n_rows), uwrow, ukb,
                         unsigned(wc), cw[r], db[r]);
  };
  if constexpr (ONE_SEG) {
    const bool live = lw < wpr;
    load(live ? lw : wpr - 1);
    accumulate_segment<ROWS, F>(cw, db, xv, live, part);
  } else {
    for (int seg = 0; seg < wpr; seg += LPS) {
      const int w = seg + lw;
      const bool live = w < wpr;
      load(live ? w : wpr - 1);
      accumulate_segment<ROWS, F>(cw, db, xv, live, part);
    }
  }

  __shared__ float red[ROWS][kThreads];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) red[r][t] = part[r];
  __syncthreads();
  const int o = t / G;                          // block output finished by this thread
  const int os = o / HALF;
  const int orr = o % HALF;
  const int g = t % G;
  constexpr int PER = LPS / G;
  float vg = 0.f, vu = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    vg += red[orr][os * LPS + g * PER + i];
    vu += red[orr + HALF][os * LPS + g * PER + i];
  }
  vg = group_sum<G>(vg);
  vu = group_sum<G>(vu);
  const int row = blockIdx.x * OUTS + o;
  if (g == G - 1 && row < n_rows) out[row] = silu(vg) * vu;
}

template <int ROWS, Fmt F>
hipError_t launch_rows(int lps, const uint32_t* codes, const uint16_t* scales, const float* x,
                       const float* residual, float* out, int n, int k, hipStream_t stream) {
  const int outs = (kThreads / lps) * ROWS;
  const dim3 grid((n + outs - 1) / outs);
#define TQ2_GEMV_CASE(L)                                                                     \
  case L:                                                                                    \
    hipLaunchKernelGGL((gemv_kernel<ROWS, L, true, F>), grid, dim3(kThreads), 0, stream,      \
                       codes, scales, x, residual, out, n, k);                               \
    break;
  switch (lps) {
    TQ2_GEMV_CASE(8)
    TQ2_GEMV_CASE(16)
    TQ2_GEMV_CASE(32)
    TQ2_GEMV_CASE(64)
    TQ2_GEMV_CASE(128)
    default:
      if (k / 16 <= 256)
        hipLaunchKernelGGL((gemv_kernel<ROWS, 256, true, F>), grid, dim3(kThreads), 0, stream,
                           codes, scales, x, residual, out, n, k);
      else
        hipLaunchKernelGGL((gemv_kernel<ROWS, 256, false, F>), grid, dim3(kThreads), 0, stream,
                           codes, scales, x, residual, out, n, k);
      break;
  }
#undef TQ2_GEMV_CASE
  return hipGetLastError();
}

template <int ROWS>
hipError_t launch_batched_rows(int lps, const GemvBatchArgs& args, int blocks, int k,
                               hipStream_t stream) {
  const dim3 grid(blocks);
#define TQ2_GEMV_BCASE(L)                                                                    \
  case L:                                                                                    \
    hipLaunchKernelGGL((gemv_batched_kernel<ROWS, L, true>), grid, dim3(kThreads), 0, stream, \
                       args, k);                                                             \
    break;
  switch (lps) {
    TQ2_GEMV_BCASE(8)
    TQ2_GEMV_BCASE(16)
    TQ2_GEMV_BCASE(32)
    TQ2_GEMV_BCASE(64)
    TQ2_GEMV_BCASE(128)
    default:
      if (k / 16 <= 256)
        hipLaunchKernelGGL((gemv_batched_kernel<ROWS, 256, true>), grid, dim3(kThreads), 0,
                           stream, args, k);
      else
        hipLaunchKernelGGL((gemv_batched_kernel<ROWS, 256, false>), grid, dim3(kThreads), 0,
                           stream, args, k);
      break;
  }
#undef TQ2_GEMV_BCASE
  return hipGetLastError();
}

// Lanes per row slot for a given k: a power of two >= k/16, at most 256.
int lanes_per_slot(int64_t k) {
  const int64_t wpr = k / 16;
  int lps = 8;
  while (lps < wpr && lps < kThreads) lps <<= 1;
  return lps;
}

}  // namespace

namespace {

template <Fmt F>
hipError_t launch_swiglu_fmt(const uint8_t* gate, const uint8_t* up, const float* x, float* out,
                             int64_t n, int64_t k, hipStream_t stream) {
  const uint32_t* gc = reinterpret_cast<const uint32_t*>(gate);
  const uint16_t* gs = reinterpret_cast<const uint16_t*>(gate + scales_offset(F, n, k));
  const uint32_t* uc = reinterpret_cast<const uint32_t*>(up);
  const uint16_t* us = reinterpret_cast<const uint16_t*>(up + scales_offset(F, n, k));
  const int lps = lanes_per_slot(k);
  const int outs = (kThreads / lps) * 4;
  const int64_t blocks = (n + outs - 1) / outs;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks));
  const int ni = int(n), ki = int(k);
#define TQ2_SWIGLU_CASE(L)                                                                    \
  case L:                                                                                     \
    hipLaunchKernelGGL((gemv_swiglu_kernel<L, true, F>), grid, dim3(kThreads), 0, stream, gc,  \
                       gs, uc, us, x, out, ni, ki);                                           \
    break;
  switch (lps) {
    TQ2_SWIGLU_CASE(8)
    TQ2_SWIGLU_CASE(16)
    TQ2_SWIGLU_CASE(32)
    TQ2_SWIGLU_CASE(64)
    TQ2_SWIGLU_CASE(128)
    default:
      if (k / 16 <= 256)
        hipLaunchKernelGGL((gemv_swiglu_kernel<256, true, F>), grid, dim3(kThreads), 0, stream,
                           gc, gs, uc, us, x, out, ni, ki);
      else
        hipLaunchKernelGGL((gemv_swiglu_kernel<256, false, F>), grid, dim3(kThreads), 0, stream,
                           gc, gs, uc, us, x, out, ni, ki);
      break;
  }
#undef TQ2_SWIGLU_CASE
  return hipGetLastError();
}

template <Fmt F>
hipError_t launch_gemv_fmt(const uint8_t* soa, const float* x, const float* residual, float* out,
                           int64_t n, int64_t k, hipStream_t stream) {
  const uint32_t* codes = reinterpret_cast<const uint32_t*>(soa);
  const uint16_t* scales = reinterpret_cast<const uint16_t*>(soa + scales_offset(F, n, k));
  const int lps = lanes_per_slot(k);
  // Rows per thread: 8 when that still gives >= 2 blocks per CU, else fewer.
  const int slots = kThreads / lps;
  int rows = 8;
  while (rows > 4 && (n + int64_t(slots) * rows - 1) / (int64_t(slots) * rows) < 512) rows >>= 1;
  if (rows > lps) rows = lps;
  const int ni = int(n), ki = int(k);
  if (rows == 8) return launch_rows<8, F>(lps, codes, scales, x, residual, out, ni, ki, stream);
  return launch_rows<4, F>(lps, codes, scales, x, residual, out, ni, ki, stream);
}

}  // namespace

hipError_t launch_gemv_swiglu(const uint8_t* gate, const uint8_t* up, const float* x,
                              float* out, int64_t n, int64_t k, hipStream_t stream) {
  return launch_swiglu_fmt<Fmt::kTq2>(gate, up, x, out, n, k, stream);
}

hipError_t launch_gemv_swiglu_q1(const uint8_t* gate, const uint8_t* up, const float* x,
                                 float* out, int64_t n, int64_t k, hipStream_t stream) {
  return launch_swiglu_fmt<Fmt::kQ1>(gate, up, x, out, n, k, stream);
}

hipError_t launch_gemv_batched(const GemvProblem* probs, int count, int64_t k,
                               hipStream_t stream) {
  const int lps = lanes_per_slot(k);
  const int slots = kThreads / lps;
  int64_t rows_total = 0;
  for (int p = 0; p < count; ++p) rows_total += probs[p].n;
  // Rows per thread: 8 when that still gives >= 2 blocks per CU, else 4.
  int rows = 8;
  if ((rows_total + int64_t(slots) * 8 - 1) / (int64_t(slots) * 8) < 512) rows = 4;
  if (rows > lps) rows = lps;
  const int outs = slots * rows;
  GemvBatchArgs args;
  int64_t blocks = 0;
  for (int p = 0; p < count; ++p) {
    args.codes[p] = reinterpret_cast<const uint32_t*>(probs[p].soa);
    args.scales[p] = reinterpret_cast<const uint16_t*>(probs[p].soa + scales_offset(probs[p].n, k));
    args.x[p] = probs[p].x;
    args.residual[p] = probs[p].residual;
    args.out[p] = probs[p].out;
    args.n[p] = int(probs[p].n);
    args.first_block[p] = int(blocks);
    blocks += (probs[p].n + outs - 1) / outs;
  }
  args.first_block[count] = int(blocks);
  args.count = count;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (rows == 8) return launch_batched_rows<8>(lps, args, int(blocks), int(k), stream);
  return launch_batched_rows<4>(lps, args, int(blocks), int(k), stream);
}

hipError_t launch_gemv(const uint8_t* soa, const float* x, const float* residual, float* out,
                       int64_t n, int64_t k, hipStream_t stream) {
  return launch_gemv_fmt<Fmt::kTq2>(soa, x, residual, out, n, k, stream);
}

hipError_t launch_gemv_q1(const uint8_t* soa, const float* x, const float* residual, float* out,
                          int64_t n, int64_t k, hipStream_t stream) {
  return launch_gemv_fmt<Fmt::kQ1>(soa, x, residual, out, n, k, stream);
}

}  // namespace tq2
