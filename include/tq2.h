/*
 * tq2.h -- C ABI of libtq2, the MI355X (gfx950) TQ2_0_g128 ternary matmul.
 *
 * The operation (oxibonsai-image 0.2.2, src/gpu.rs: module doc "Correctness
 * contract" and the doc of `ternary_matmul_gpu`):
 *
 *     out[m, n] = residual[m, n] + sum_k x[m, k] * dequant(W)[n, k]
 *
 * with x row-major f32 [M, K], W out-major [N, K] (no transpose) and out
 * row-major f32 [M, N].  The residual term is optional; it mirrors the fused
 * `*_residual` kernels of oxibonsai-kernels 0.1.5 (pipelines.rs,
 * `MetalPipelines` fields `gemv_q1_g128_v7_residual`,
 * `gemm_q1_g128_v7_residual`) and is added once to the finished dot product.
 *
 * Weight format (gpu.rs, doc of `blocks_as_bytes`): N * (K / 128) blocks of
 * 34 bytes, `qs[32]` then a little-endian binary16 scale `d`; row n's blocks
 * are contiguous, block index increasing with k.  Recorded convention (the
 * pages give neither): weight j of a block has code
 * (qs[j / 4] >> (2 * (j % 4))) & 3, and codes 0, 1, 2 mean -1, 0, +1 times d;
 * code 3 is reserved and means 0.
 *
 * Like the pages' kernel, the library runs on a resident re-laid-out copy of
 * the weight (gpu.rs: `blocks_as_bytes` feeds `reformat_tq2_aos_to_soa`, and
 * `ternary_matmul_gpu` keeps the resulting buffer resident): callers convert
 * each weight once with tq2_reformat_aos_to_soa and pass the result to
 * tq2_gemv / tq2_gemm.  That "SoA" layout is private to the library and
 * versioned by tq2_soa_layout_version(); only its size is public.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers on the current HIP device, owned by the
 *     caller.  The library never allocates, frees or keeps them.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Every
 *     call only enqueues work on it and returns; nothing synchronises.  The
 *     returned status covers argument checks and the launch; faults during
 *     execution surface at the caller's next synchronisation.
 *   - Errors are returned as negative tq2_status values; nothing aborts.
 *     Nothing is enqueued when a call returns an error.
 *   - Calls are stateless and thread-safe; calls on different streams may run
 *     concurrently.
 */
#ifndef TQ2_H
#define TQ2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status of a call.  Error policy of the pages (oxibonsai-image 0.2.2,
 * src/gpu.rs: the module doc's last paragraph, the `GpuMatmulError` enum and
 * the "# Errors" section of `ternary_matmul_gpu`): every failure of the GPU
 * matmul -- device unavailable, weight upload / encode / dispatch failed,
 * k % 128 != 0, a length mismatch -- comes back to the caller as a value, and
 * nothing panics or aborts.  The codes split that enum's cases finer:
 * GraphUnavailable is TQ2_ERR_DEVICE; the `Metal` case (encode / dispatch)
 * is TQ2_ERR_LAUNCH; the argument errors its doc names are TQ2_ERR_SHAPE
 * (k % 128 != 0) and TQ2_ERR_INVALID (a length or size the call cannot
 * take).  TQ2_ERR_ALIGN and TQ2_ERR_ALIAS are this library's own checks of
 * raw device pointers, which the pages' slice-typed API cannot receive.  The
 * pages' caller turns any error into a CPU fallback; this library has none,
 * so the caller sees the status. */
typedef enum tq2_status {
  TQ2_OK = 0,
  TQ2_ERR_INVALID = -1, /* null pointer, negative size, K <= 0, size too large (gpu.rs,
                           `ternary_matmul_gpu` "# Errors": a length the call cannot take) */
  TQ2_ERR_SHAPE = -2,   /* K is not a multiple of 128 (gpu.rs, `ternary_matmul_gpu`
                           "# Errors": `k % 128 != 0`) */
  TQ2_ERR_ALIGN = -3,   /* soa not 256-byte aligned, or x / out / residual not 16-byte aligned */
  TQ2_ERR_ALIAS = -4,   /* out overlaps x or soa, residual partially overlaps out, aos overlaps soa */
  TQ2_ERR_DEVICE = -5,  /* current HIP device is not gfx950, or HIP could not be queried
                           (gpu.rs, `GpuMatmulError::GraphUnavailable`: no usable device) */
  TQ2_ERR_LAUNCH = -6   /* the kernel launch failed (gpu.rs, `GpuMatmulError::Metal`:
                           encode / dispatch failed) */
} tq2_status;

/* Bytes of an [n, k] weight in the 34-byte AoS block format: n * (k/128) * 34,
 * the byte length of the blocks' raw view that gpu.rs uploads (oxibonsai-image
 * 0.2.2, src/gpu.rs: doc of `blocks_as_bytes`, a `#[repr(C)]` 34-byte block
 * `qs[32]` then the binary16 `d`, and its test that the view is 34 bytes per
 * block; `ternary_matmul_gpu` takes n * (k / 128) blocks).
 * Returns 0 for n < 0, k <= 0 or k % 128 != 0.  Pure host function. */
size_t tq2_aos_bytes(int64_t n, int64_t k);

/* Bytes the library's resident SoA copy of an [n, k] weight occupies (a
 * multiple of 256): the buffer `reformat_tq2_aos_to_soa` fills from the AoS
 * bytes and the matmul keeps resident (gpu.rs: doc of `blocks_as_bytes`, and
 * `ternary_matmul_gpu`'s "resident SoA buffer").  2.125 bits per weight, as
 * the AoS.  Returns 0 for invalid n, k as above.  Pure host function. */
size_t tq2_soa_bytes(int64_t n, int64_t k);

/* Version number of the private SoA layout written by tq2_reformat_aos_to_soa
 * (the pages' kernels likewise share one private SoA weight buffer:
 * oxibonsai-kernels 0.1.5, pipelines.rs, fields `gemm_tq2_g128_v9_simdgroup`
 * and `gemm_tq2_g128_v10_simdgroup`, "same op / SoA weight buffer"). */
int tq2_soa_layout_version(void);

/* Convert an [n, k] weight from AoS blocks (`aos`, tq2_aos_bytes(n, k) bytes,
 * any alignment of 2 bytes or more) to the library's SoA layout (`soa`,
 * tq2_soa_bytes(n, k) bytes, 256-byte aligned).  The AoS->SoA step the pages
 * name `reformat_tq2_aos_to_soa` (gpu.rs, doc of `blocks_as_bytes`); this
 * library's layout is its own.  `aos` and `soa` must not overlap.
 * n == 0 is a no-op.  Errors: INVALID, SHAPE, ALIGN (aos odd or soa not
 * 256-aligned), ALIAS, DEVICE, LAUNCH. */
int tq2_reformat_aos_to_soa(const void* aos, void* soa, int64_t n, int64_t k, void* stream);

/* Decode GEMV (M = 1): out[n] = residual[n] + sum_k x[k] * w[n, k].
 * soa: tq2_soa_bytes(n, k) bytes from tq2_reformat_aos_to_soa.  x: f32 [k].
 * residual: f32 [n] or NULL.  out: f32 [n]; may be the same pointer as
 * residual (in-place add), must not overlap x or soa otherwise.
 * Arithmetic: f32 products and sums in short chains; error within
 * 1e-5 * (sum_k |x[k] w[n,k]| + |residual[n]|).  Kernel of the pages' decode
 * path: oxibonsai-kernels 0.1.5, pipelines.rs, field `gemv_tq2_g128_v1`.
 * n == 0 is a no-op.  Errors: INVALID, SHAPE, ALIGN, ALIAS, DEVICE, LAUNCH. */
int tq2_gemv(const void* soa, const float* x, const float* residual, float* out,
             int64_t n, int64_t k, void* stream);

/* One independent decode GEMV of a batch (see tq2_gemv_batched). */
typedef struct tq2_gemv_problem {
  const void* soa;        /* tq2_soa_bytes(n, k) bytes from tq2_reformat_aos_to_soa */
  const float* x;         /* f32 [k] */
  const float* residual;  /* f32 [n] or NULL */
  float* out;             /* f32 [n]; may equal residual */
  int64_t n;
  int64_t k;
} tq2_gemv_problem;

/* Most problems one tq2_gemv_batched call takes. */
#define TQ2_GEMV_BATCH_MAX 32

/* Several independent decode GEMVs, out_p = residual_p + W_p x_p, enqueued
 * together: one launch per distinct k, all of that k's problems' row blocks
 * in one grid, so the launch and ramp cost of a decode step with many
 * projections is paid once rather than per weight (the decode path runs one
 * TQ2 GEMV per projection: oxibonsai-kernels 0.1.5, pipelines.rs, field
 * `gemv_tq2_g128_v1`).  Each problem follows tq2_gemv's rules and arithmetic;
 * problems may share x, soa or residual buffers, but no problem's out may
 * overlap any buffer of another problem.  `problems` is a HOST array of
 * `count` entries, read during the call and not kept.  count == 0 and
 * problems with n == 0 are no-ops.  Every problem is checked before anything
 * is enqueued; a failed launch (TQ2_ERR_LAUNCH) may leave the launches for
 * smaller k already enqueued.  Errors: INVALID (null problems with count > 0,
 * count < 0 or count > TQ2_GEMV_BATCH_MAX, a problem's argument, or the
 * problems of one k with a sum of ceil(n / 4) above 2^31 - 1: their grid),
 * SHAPE, ALIGN, ALIAS, DEVICE, LAUNCH. */
int tq2_gemv_batched(const tq2_gemv_problem* problems, int count, void* stream);

/* Batched matmul for any M >= 1: out[m, n] = residual[m, n] + sum_k x[m, k] w[n, k].
 * x: f32 [m, k] row-major; residual: f32 [m, n] or NULL; out: f32 [m, n],
 * same aliasing rules as tq2_gemv.  The kernel is picked by tq2_gemm_path:
 *   0: M == 1, the GEMV above;
 *   1: 2 <= M <= 16: matrix-core GEMM with x split into two binary16 parts
 *      (x = hi + lo), error within 1e-5 * sum|x w| at any overall magnitude
 *      of x: each wave scales its slice of x (per 4096-wide pass over K) by
 *      a power of two before the split so that both parts stay normal
 *      binary16, and scales the sums back (exact); the power follows the
 *      largest |x| the wave has seen so far (over the rows it holds, in this
 *      and earlier passes), so it only falls and the sums never overflow.
 *      The bound assumes the elements that carry a row's sum are within
 *      2^17 of that largest |x|: a smaller element keeps an absolute error
 *      below 2^-39 of the largest |x|, which can exceed 1e-5 * sum|x w| when
 *      the largest |x| meets only zero weights;
 *   2: M > 16: matrix-core GEMM with x rounded to binary16 and weights staged
 *      as exact binary16 code * d (oxibonsai-kernels 0.1.5, pipelines.rs,
 *      fields `gemm_tq2_g128_v9_simdgroup` / `gemm_tq2_g128_v10_simdgroup`:
 *      f16-staged operands, f32 accumulation); error within
 *      2e-3 * sum|x w| for |x| <= 65504 whose rows do not average below
 *      about 1.5e-5 in |x| (under binary16's normal range, 2^-14, the
 *      rounding of x leaves an absolute error of 2^-25 |w| per element);
 *      tq2_gemm_precise holds its bound at any magnitude.
 * m == 0 or n == 0 is a no-op.  Errors: INVALID, SHAPE, ALIGN, ALIAS, DEVICE,
 * LAUNCH. */
int tq2_gemm(const void* soa, const float* x, const float* residual, float* out,
             int64_t m, int64_t n, int64_t k, void* stream);

/* Bytes of device workspace that tq2_gemm_ws uses for an (m, n, k) call, or 0
 * where it uses none (it then runs tq2_gemm's kernels); 0 also for invalid
 * shapes.  Nonzero for path 2 with M <= 128: about 2 * ceil(M/16) * 16 * K
 * bytes (x as binary16, rows padded to 16 and K to 256). */
size_t tq2_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k);

/* tq2_gemm with a device workspace from the caller, for path 2 at
 * 16 < M <= 128.  Same operation, arguments, aliasing rules, tolerance
 * (path 2's 2e-3 * sum|x w|: x rounded to binary16, weights exact binary16
 * code * d, f32 accumulation, as in the pages' f16-staged v9/v10 kernels,
 * oxibonsai-kernels 0.1.5, pipelines.rs, fields `gemm_tq2_g128_v9_simdgroup`
 * / `gemm_tq2_g128_v10_simdgroup`) and errors as tq2_gemm; the results may
 * differ from tq2_gemm's in the last bits (another summation order).
 * x is first written once into `workspace` as binary16 in the matrix cores'
 * operand order, so the GEMM's blocks read half the bytes of x and need no
 * staging; each block then splits K over its waves.
 * workspace: device memory of workspace_bytes >= tq2_gemm_workspace_bytes(
 * m, n, k), 256-byte aligned, not overlapping soa, x, residual or out; it is
 * overwritten (owned by the call until the stream reaches its end), so calls
 * that share one workspace must be ordered (one stream).  Where that size is
 * 0 the call is tq2_gemm and workspace may be NULL.  Errors: those of
 * tq2_gemm, and INVALID for a missing or too small workspace, ALIGN, ALIAS. */
int tq2_gemm_ws(const void* soa, const float* x, const float* residual, float* out,
                int64_t m, int64_t n, int64_t k, void* workspace, size_t workspace_bytes,
                void* stream);

/* Size of the device array behind tq2_gemm_noalloc (4 MiB per GPU). */
#define TQ2_NOALLOC_SCRATCH_BYTES (4u << 20)

/* tq2_gemm_ws without a workspace argument, for callers that cannot allocate
 * device memory at all: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The workspace is a fixed array of
 * TQ2_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held from the
 * library's load until the process ends; the call allocates and frees
 * nothing.  Same operation, arguments, rules, tolerance and errors as
 * tq2_gemm_ws, and the same results bit for bit.  Limit: a call whose
 * tq2_gemm_workspace_bytes(m, n, k) exceeds TQ2_NOALLOC_SCRATCH_BYTES
 * returns TQ2_ERR_INVALID and enqueues nothing (at M = 100 that is
 * K > 18688; at M = 128, K > 16384); where that size is 0 the call is
 * tq2_gemm.  Every call on one GPU shares that GPU's array, so calls that
 * overlap on one GPU (concurrent streams, or graph replays in flight
 * together) race and may return wrong results; order them on one stream. */
int tq2_gemm_noalloc(const void* soa, const float* x, const float* residual, float* out,
                     int64_t m, int64_t n, int64_t k, void* stream);

/* tq2_gemm with f32-class accuracy at every M: the split-binary16 matrix-core
 * kernel of path 1 (x = hi + lo, both parts against the same exact binary16
 * weight, f32 accumulation) for every M >= 2, and the GEMV for M == 1; error
 * within 1e-5 * sum|x w| at any overall magnitude of x, under the same
 * assumption as path 1 (for M > 16 the power of two is kept per group of x
 * rows and 256-wide K chunk, falling as larger values arrive, with the sums
 * rescaled to it), at about twice path 2's matrix-core
 * work for M > 16.  The pages stage both operands as binary16 for large M
 * (pipelines.rs, fields `gemm_tq2_g128_v9_simdgroup` /
 * `gemm_tq2_g128_v10_simdgroup`); this is the variant for callers that need
 * the f32 path's accuracy (their `gemm_tq2_g128_v7` / `_v8_tiled`).  Same
 * arguments, rules and errors as tq2_gemm. */
int tq2_gemm_precise(const void* soa, const float* x, const float* residual, float* out,
                     int64_t m, int64_t n, int64_t k, void* stream);

/* Fused gate/up projections with SwiGLU, for any M >= 1:
 *     out[m, n] = silu(g[m, n]) * u[m, n],  silu(z) = z / (1 + exp(-z)),
 *     g = x W_gate^T,  u = x W_up^T.
 * The ternary counterpart of the pages' `fused_gate_up_swiglu_q1` (decode)
 * and `fused_gate_up_swiglu_gemm_q1` (prefill) pipelines (oxibonsai-kernels
 * 0.1.5, pipelines.rs, `MetalPipelines`); the pages name the fusion, and the
 * arithmetic is the usual SwiGLU gate with SiLU as in their `silu_f32`.
 * gate_soa, up_soa: two [n, k] weights in this library's SoA layout (256-byte
 * aligned device buffers from tq2_reformat_aos_to_soa; they may be the same
 * buffer).  x: f32 [m, k] row-major; out: f32 [m, n] row-major, which must not
 * overlap x or either weight.  Both projections stay on chip: each output
 * tile reads x once for both weights.  The kernels follow tq2_gemm_path:
 * M == 1 runs a fused f32 GEMV, 2 <= M <= 16 the split-binary16 matrix-core
 * kernel, M > 16 the binary16 matrix-core kernel, with g and u each as
 * accurate as tq2_gemm's result on that path (tolerance tol = 1e-5 or
 * 2e-3 of sum|x w|); out is then within
 *     tol * (1.1 * Sg * (|u| + tol * Su) + |silu(g)| * Su)
 * plus a few f32 roundings of |out|, where Sg, Su are sum_k |x w| of each
 * projection (1.1 bounds silu's slope).  m == 0 or n == 0 is a no-op.
 * Errors: INVALID (null pointer or oversized shape), SHAPE, ALIGN, ALIAS,
 * DEVICE, LAUNCH. */
int tq2_gate_up_swiglu(const void* gate_soa, const void* up_soa, const float* x, float* out,
                       int64_t m, int64_t n, int64_t k, void* stream);

/* ---- Q1_g128: the 1-bit sibling format --------------------------------------
 * The pages' decode and prefill kernels for 1-bit weights (oxibonsai-kernels
 * 0.1.5, pipelines.rs, `MetalPipelines` fields `gemv_q1_g128_v7`,
 * `gemv_q1_g128_v7_residual`, `gemm_q1_g128_v7`, `gemm_q1_g128_v7_residual`,
 * `fused_gate_up_swiglu_q1`, `fused_gate_up_swiglu_gemm_q1`) run on a format
 * the pages name but do not lay out.  Recorded reading, mirroring the TQ2
 * block: 128 weights per block in 18 bytes, `qs[16]` then a little-endian
 * binary16 `d`; weight j has bit (qs[j / 8] >> (j % 8)) & 1, and a set bit is
 * +d, a clear bit -d.  The operations, arguments, path choice (tq2_gemm_path),
 * tolerances, aliasing rules and errors are those of the TQ2 entry points
 * above; only the weight buffers differ (sizes from tq2_q1_aos_bytes /
 * tq2_q1_soa_bytes, a private SoA layout of the same version number). */

/* Bytes of an [n, k] Q1_g128 weight in AoS blocks: n * (k/128) * 18, or 0 for
 * invalid n, k. */
size_t tq2_q1_aos_bytes(int64_t n, int64_t k);

/* Bytes of the library's resident Q1 SoA copy (a multiple of 256), or 0. */
size_t tq2_q1_soa_bytes(int64_t n, int64_t k);

/* Q1 AoS -> SoA, as tq2_reformat_aos_to_soa. */
int tq2_q1_reformat_aos_to_soa(const void* aos, void* soa, int64_t n, int64_t k, void* stream);

/* Q1 decode GEMV (M = 1) with optional residual, as tq2_gemv (the pages'
 * `gemv_q1_g128_v7` / `gemv_q1_g128_v7_residual`). */
int tq2_q1_gemv(const void* soa, const float* x, const float* residual, float* out,
                int64_t n, int64_t k, void* stream);

/* Q1 matmul for any M >= 1 with optional residual, as tq2_gemm (the pages'
 * `gemm_q1_g128_v7` / `gemm_q1_g128_v7_residual`, with no cap on M). */
int tq2_q1_gemm(const void* soa, const float* x, const float* residual, float* out,
                int64_t m, int64_t n, int64_t k, void* stream);

/* Q1 fused gate/up projections + SwiGLU, as tq2_gate_up_swiglu (the pages'
 * `fused_gate_up_swiglu_q1` / `fused_gate_up_swiglu_gemm_q1`). */
int tq2_q1_gate_up_swiglu(const void* gate_soa, const void* up_soa, const float* x, float* out,
                          int64_t m, int64_t n, int64_t k, void* stream);

/* The kernel tq2_gemm uses for this shape (0, 1 or 2 as listed above), or
 * TQ2_ERR_INVALID / TQ2_ERR_SHAPE for an invalid shape.  Pure host function.
 * The pages pick among their ternary kernels inside `encode_gemm_tq2`
 * (oxibonsai-kernels 0.1.5, pipelines.rs, `MetalPipelines` fields
 * `gemm_tq2_g128_v8_tiled`, `gemm_tq2_g128_v9_simdgroup` and
 * `gemm_tq2_g128_v10_simdgroup`: the large-M path dispatches the
 * matrix-unit kernel, and v10 only when it passes parity and is faster), and
 * gpu.rs reports only whether the GPU ran at all (`gpu_was_used`, the
 * `GPU_USED` flag used to prove the GPU path executed).  This query states the
 * choice before the call, as a pure function of the shape, so a caller (or a
 * test) knows which kernel -- and so which accuracy bound above -- applies. */
int tq2_gemm_path(int64_t m, int64_t n, int64_t k);

/* Static description of a status value ("ok", "invalid argument", ...): the
 * counterpart of the `#[error(...)]` messages of gpu.rs's `GpuMatmulError`
 * (oxibonsai-image 0.2.2, src/gpu.rs), for callers that log a failure
 * instead of panicking.  Unknown values give "unknown tq2 status"; the
 * returned string is static and must not be freed. */
const char* tq2_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* TQ2_H */
