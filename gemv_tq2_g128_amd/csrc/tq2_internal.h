// Internal declarations shared by the libtq2 translation units (not installed).
//
// Private SoA layout, version 1, of an [N, K] weight (KB = K / 128 blocks per
// row), written by tq2_reformat_aos_to_soa:
//
//   codes plane  at byte 0:            N * K/4 bytes, row n at n * K/4.
//                Row n is K/16 little-endian 32-bit words; word w holds the
//                codes of k = 16w .. 16w+15.  Code of k = 16w + t sits at bit
//                2*(t >> 1) + 16*(t & 1): even t in the low half-word, odd t
//                in the high half-word, each half in increasing t.  Codes are
//                stored canonical: 0 (-1), 1 (0), 2 (+1); a reserved code 3 is
//                stored as 1.
//   scales plane at byte align256(N*K/4):  binary16 d[n * KB + kb].
//   total size  align256(scales offset + N*KB*2).
//
// The half-word split lets one AND-OR with 0x64006400 place the codes of two
// neighbouring weights (k, k+1) into the mantissas of a binary16 pair, which
// is the operand order of both the dot2 and the MFMA kernels.
//
// Q1_g128 (1-bit) SoA of an [N, K] weight, same version, written by
// tq2_q1_reformat_aos_to_soa:
//
//   bits plane   at byte 0:            N * K/8 bytes, row n at n * K/8.
//                Row n is K/32 little-endian 32-bit words; word w holds the
//                bits of k = 32w .. 32w+31.  The bit of k = 32w + t sits at
//                bit (t >> 1) + 16*(t & 1): pair p = (32w+2p, 32w+2p+1) at bits
//                p and p + 16.  1 = +d, 0 = -d.
//   scales plane at byte align256(N*K/8):  binary16 d[n * KB + kb].
//   total size  align256(scales offset + N*KB*2).
//
// Shifting a word left by 15 - p puts pair p's bits on the two binary16 sign
// positions, so one AND-OR with |d| yields the pair (+-d, +-d).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tq2 {

constexpr int kBlockWeights = 128;
constexpr int kBlockBytes = 34;
constexpr int kLayoutVersion = 1;

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }
inline size_t codes_bytes(int64_t n, int64_t k) { return size_t(n) * size_t(k / 4); }
inline size_t scales_offset(int64_t n, int64_t k) { return align256(codes_bytes(n, k)); }
inline size_t soa_bytes(int64_t n, int64_t k) {
  return align256(scales_offset(n, k) + size_t(n) * size_t(k / kBlockWeights) * 2);
}

// Weight formats of the kernels: bits per weight in the SoA codes plane.
enum class Fmt : int { kTq2 = 2, kQ1 = 1 };

constexpr int kQ1BlockBytes = 18;
inline size_t codes_bytes(Fmt f, int64_t n, int64_t k) {
  return size_t(n) * size_t(k / 8) * size_t(int(f));
}
inline size_t scales_offset(Fmt f, int64_t n, int64_t k) { return align256(codes_bytes(f, n, k)); }
inline size_t soa_bytes(Fmt f, int64_t n, int64_t k) {
  return align256(scales_offset(f, n, k) + size_t(n) * size_t(k / kBlockWeights) * 2);
}

// Kernel launchers (one per translation unit).  Arguments are already
// validated by the C ABI; each returns the hipError_t of its launch.
hipError_t launch_reformat(const uint16_t* aos, uint8_t* soa, int64_t n, int64_t k,
                           hipStream_t stream);
hipError_t launch_reformat_q1(const uint16_t* aos, uint8_t* soa, int64_t n, int64_t k,
                              hipStream_t stream);
hipError_t launch_gemv(const uint8_t* soa, const float* x, const float* residual, float* out,
                       int64_t n, int64_t k, hipStream_t stream);
hipError_t launch_gemm(int path, const uint8_t* soa, const float* x, const float* residual,
                       float* out, int64_t m, int64_t n, int64_t k, hipStream_t stream);
// Q1_g128 weights: the same kernels with the 1-bit decode.
hipError_t launch_gemv_q1(const uint8_t* soa, const float* x, const float* residual, float* out,
                          int64_t n, int64_t k, hipStream_t stream);
hipError_t launch_gemm_q1(int path, const uint8_t* soa, const float* x, const float* residual,
                          float* out, int64_t m, int64_t n, int64_t k, hipStream_t stream);

// Fused gate/up projections + SwiGLU: out = silu(x W_gate^T) * (x W_up^T),
// both weights [n, k] in SoA v1.  The GEMV form serves M = 1; the matrix-core
// form takes `path` 1 or 2 as launch_gemm does.
hipError_t launch_gemv_swiglu(const uint8_t* gate, const uint8_t* up, const float* x,
                              float* out, int64_t n, int64_t k, hipStream_t stream);
hipError_t launch_gemm_swiglu(int path, const uint8_t* gate, const uint8_t* up, const float* x,
                              float* out, int64_t m, int64_t n, int64_t k, hipStream_t stream);
hipError_t launch_gemv_swiglu_q1(const uint8_t* gate, const uint8_t* up, const float* x,
                                 float* out, int64_t n, int64_t k, hipStream_t stream);
hipError_t launch_gemm_swiglu_q1(int path, const uint8_t* gate, const uint8_t* up,
                                 const float* x, float* out, int64_t m, int64_t n, int64_t k,
                                 hipStream_t stream);

// Batched decode GEMV: up to kGemvBatchMax independent problems with the same
// k in one launch (their descriptors travel in the kernel arguments).
constexpr int kGemvBatchMax = 32;
struct GemvProblem {
  const uint8_t* soa;
  const float* x;
  const float* residual;
  float* out;
  int64_t n;
};
hipError_t launch_gemv_batched(const GemvProblem* probs, int count, int64_t k, hipStream_t stream);

// Largest M served by the split-f16 (f32-class) matrix-core path.
constexpr int64_t kSplitMaxM = 16;

// The matrix-core kernels address x row blocks (up to 128 rows of K f32) and
// the weight planes through 32-bit buffer offsets: K <= 2^21 and
// N * K / 4 < 2^31 bytes of codes (the same bound on N * K serves Q1).
constexpr int64_t kGemmMaxK = int64_t(1) << 21;
constexpr int64_t kGemmMaxCodeBytes = int64_t(1) << 31;

// Path 2 with a caller workspace (tq2_gemm_ws) for kSplitMaxM < M <= kWsMaxM:
// x is written once per call as binary16 MFMA fragments into the workspace
// (gemm_ws_bytes of them), and a K-split kernel reads them.  gemm_ws_bytes
// is 0 where tq2_gemm_ws runs tq2_gemm's kernels instead.
constexpr int64_t kWsMaxM = 128;
size_t gemm_ws_bytes(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_ws(const uint8_t* soa, const float* x, const float* residual, float* out,
                          int64_t m, int64_t n, int64_t k, void* ws, hipStream_t stream);

}  // namespace tq2
