// C ABI of libtq2: argument checks, device check, kernel selection.
//
// Error policy after the pages (oxibonsai-image 0.2.2, src/gpu.rs: the
// `GpuMatmulError` enum and the doc of `ternary_matmul_gpu`): every failure,
// including k % 128 != 0 and size mismatches, is returned to the caller and
// nothing panics.  Unlike the pages there is no CPU fallback behind it.
#include <atomic>
#include <cstring>

#include "../../include/tq2.h"
#include "tq2_internal.h"

namespace {

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other architecture.
std::atomic<int> g_device_kind[kMaxDevices];

// Device memory of tq2_gemm_noalloc: one fixed array per GPU, held from the
// library's load until the process ends, so that call allocates nothing.
// In host code `scratch` is only the host-side stand-in of the symbol, not a
// device address: device_scratch() returns the address on the current
// device (hipGetSymbolAddress, once per device), and only that is passed on.
static __device__ __align__(256) uint8_t scratch[TQ2_NOALLOC_SCRATCH_BYTES];
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The scratch array's address on device `dev` (current), or nullptr.
void* device_scratch(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
  g_scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
}

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return TQ2_ERR_DEVICE;
  if (dev < kMaxDevices) {
    const int kind = g_device_kind[dev].load(std::memory_order_relaxed);
    if (kind == 1) return TQ2_OK;
    if (kind == 2) return TQ2_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return TQ2_ERR_DEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_device_kind[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? TQ2_OK : TQ2_ERR_DEVICE;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

constexpr int64_t kMaxDim = int64_t(1) << 30;   // keeps every 32-bit index in range

// Shape check shared by every entry point; m may be 0 (no-op) where allowed.
int check_shape(int64_t m, int64_t n, int64_t k) {
  if (m < 0 || n < 0 || k <= 0) return TQ2_ERR_INVALID;
  if (k % tq2::kBlockWeights) return TQ2_ERR_SHAPE;
  if (m > kMaxDim || n > kMaxDim || k > kMaxDim) return TQ2_ERR_INVALID;
  return TQ2_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? TQ2_OK : TQ2_ERR_LAUNCH; }

// Host-side checks common to the matmul entry points once the shape is valid
// and non-empty: pointers, alignment and aliasing.
int check_matmul_host(const void* soa, const float* x, const float* residual, const float* out,
                      int64_t m, int64_t n, int64_t k, tq2::Fmt f = tq2::Fmt::kTq2) {
  if (!soa || !x || !out) return TQ2_ERR_INVALID;
  if (!aligned(soa, 256) || !aligned(x, 16) || !aligned(out, 16) ||
      (residual && !aligned(residual, 16)))
    return TQ2_ERR_ALIGN;
  const size_t xb = size_t(m) * size_t(k) * 4, ob = size_t(m) * size_t(n) * 4;
  const size_t sb = tq2::soa_bytes(f, n, k);
  if (overlaps(out, ob, x, xb) || overlaps(out, ob, soa, sb)) return TQ2_ERR_ALIAS;
  if (residual && residual != out && overlaps(out, ob, residual, ob)) return TQ2_ERR_ALIAS;
  return TQ2_OK;
}

int check_matmul_args(const void* soa, const float* x, const float* residual, const float* out,
                      int64_t m, int64_t n, int64_t k, tq2::Fmt f = tq2::Fmt::kTq2) {
  const int st = check_matmul_host(soa, x, residual, out, m, n, k, f);
  return st != TQ2_OK ? st : check_device();
}

// The matrix-core kernels' 32-bit offsets (see tq2_internal.h).
bool gemm_shape_fits(int64_t n, int64_t k) {
  return k <= tq2::kGemmMaxK && n * (k / 4) < tq2::kGemmMaxCodeBytes;
}

int reformat_impl(tq2::Fmt f, const void* aos, void* soa, int64_t n, int64_t k, void* stream) {
  int st = check_shape(0, n, k);
  if (st != TQ2_OK) return st;
  if (n == 0) return TQ2_OK;
  if (!aos || !soa) return TQ2_ERR_INVALID;
  if (!aligned(aos, 2) || !aligned(soa, 256)) return TQ2_ERR_ALIGN;
  const size_t ab = size_t(n) * size_t(k / tq2::kBlockWeights) *
                    (f == tq2::Fmt::kQ1 ? tq2::kQ1BlockBytes : tq2::kBlockBytes);
  if (overlaps(aos, ab, soa, tq2::soa_bytes(f, n, k))) return TQ2_ERR_ALIAS;
  st = check_device();
  if (st != TQ2_OK) return st;
  const uint16_t* a = static_cast<const uint16_t*>(aos);
  uint8_t* o = static_cast<uint8_t*>(soa);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return launch_status(f == tq2::Fmt::kQ1 ? tq2::launch_reformat_q1(a, o, n, k, s)
                                          : tq2::launch_reformat(a, o, n, k, s));
}

int gemv_impl(tq2::Fmt f, const void* soa, const float* x, const float* residual, float* out,
              int64_t n, int64_t k, void* stream) {
  int st = check_shape(1, n, k);
  if (st != TQ2_OK) return st;
  if (n == 0) return TQ2_OK;
  st = check_matmul_args(soa, x, residual, out, 1, n, k, f);
  if (st != TQ2_OK) return st;
  const uint8_t* w = static_cast<const uint8_t*>(soa);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return launch_status(f == tq2::Fmt::kQ1 ? tq2::launch_gemv_q1(w, x, residual, out, n, k, s)
                                          : tq2::launch_gemv(w, x, residual, out, n, k, s));
}

// path: 0 = GEMV, 1 = split-binary16 matrix cores, 2 = binary16 matrix cores.
int gemm_impl(tq2::Fmt f, int path, const void* soa, const float* x, const float* residual,
              float* out, int64_t m, int64_t n, int64_t k, void* stream) {
  if (path == 0) return gemv_impl(f, soa, x, residual, out, n, k, stream);
  int st = check_matmul_host(soa, x, residual, out, m, n, k, f);
  if (st != TQ2_OK) return st;
  if (!gemm_shape_fits(n, k)) return TQ2_ERR_INVALID;
  st = check_device();
  if (st != TQ2_OK) return st;
  const uint8_t* w = static_cast<const uint8_t*>(soa);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return launch_status(f == tq2::Fmt::kQ1
                           ? tq2::launch_gemm_q1(path, w, x, residual, out, m, n, k, s)
                           : tq2::launch_gemm(path, w, x, residual, out, m, n, k, s));
}

int swiglu_impl(tq2::Fmt f, const void* gate_soa, const void* up_soa, const float* x,
                float* out, int64_t m, int64_t n, int64_t k, void* stream) {
  int st = check_shape(m, n, k);
  if (st != TQ2_OK) return st;
  if (m == 0 || n == 0) return TQ2_OK;
  if (!up_soa) return TQ2_ERR_INVALID;
  st = check_matmul_host(gate_soa, x, nullptr, out, m, n, k, f);
  if (st != TQ2_OK) return st;
  if (!aligned(up_soa, 256)) return TQ2_ERR_ALIGN;
  if (overlaps(out, size_t(m) * size_t(n) * 4, up_soa, tq2::soa_bytes(f, n, k)))
    return TQ2_ERR_ALIAS;
  const int path = m <= 1 ? 0 : (m <= tq2::kSplitMaxM ? 1 : 2);
  if (path != 0 && !gemm_shape_fits(n, k)) return TQ2_ERR_INVALID;
  st = check_device();
  if (st != TQ2_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* g = static_cast<const uint8_t*>(gate_soa);
  const uint8_t* u = static_cast<const uint8_t*>(up_soa);
  if (f == tq2::Fmt::kQ1)
    return launch_status(path == 0 ? tq2::launch_gemv_swiglu_q1(g, u, x, out, n, k, s)
                                   : tq2::launch_gemm_swiglu_q1(path, g, u, x, out, m, n, k, s));
  return launch_status(path == 0 ? tq2::launch_gemv_swiglu(g, u, x, out, n, k, s)
                                 : tq2::launch_gemm_swiglu(path, g, u, x, out, m, n, k, s));
}

}  // namespace

extern "C" {

size_t tq2_aos_bytes(int64_t n, int64_t k) {
  if (check_shape(0, n, k) != TQ2_OK) return 0;
  return size_t(n) * size_t(k / tq2::kBlockWeights) * tq2::kBlockBytes;
}

size_t tq2_soa_bytes(int64_t n, int64_t k) {
  if (check_shape(0, n, k) != TQ2_OK) return 0;
  return tq2::soa_bytes(n, k);
}

int tq2_soa_layout_version(void) { return tq2::kLayoutVersion; }

int tq2_reformat_aos_to_soa(const void* aos, void* soa, int64_t n, int64_t k, void* stream) {
  return reformat_impl(tq2::Fmt::kTq2, aos, soa, n, k, stream);
}

int tq2_gemm_path(int64_t m, int64_t n, int64_t k) {
  const int st = check_shape(m, n, k);
  if (st != TQ2_OK) return st;
  if (m <= 1) return 0;
  return m <= tq2::kSplitMaxM ? 1 : 2;
}

int tq2_gemv(const void* soa, const float* x, const float* residual, float* out, int64_t n,
             int64_t k, void* stream) {
  return gemv_impl(tq2::Fmt::kTq2, soa, x, residual, out, n, k, stream);
}

int tq2_gemv_batched(const tq2_gemv_problem* problems, int count, void* stream) {
  static_assert(TQ2_GEMV_BATCH_MAX == tq2::kGemvBatchMax, "batch limit");
  if (count == 0) return TQ2_OK;
  if (!problems || count < 0 || count > TQ2_GEMV_BATCH_MAX) return TQ2_ERR_INVALID;
  for (int i = 0; i < count; ++i) {
    const tq2_gemv_problem& p = problems[i];
    int st = check_shape(1, p.n, p.k);
    if (st != TQ2_OK) return st;
    if (p.n == 0) continue;
    st = check_matmul_host(p.soa, p.x, p.residual, p.out, 1, p.n, p.k);
    if (st != TQ2_OK) return st;
  }
  // No problem's out may touch another problem's buffers.
  for (int i = 0; i < count; ++i) {
    const tq2_gemv_problem& p = problems[i];
    if (p.n == 0) continue;
    const size_t ob = size_t(p.n) * 4;
    for (int j = 0; j < count; ++j) {
      const tq2_gemv_problem& q = problems[j];
      if (j == i || q.n == 0) continue;
      if (overlaps(p.out, ob, q.out, size_t(q.n) * 4) ||
          overlaps(p.out, ob, q.x, size_t(q.k) * 4) ||
          overlaps(p.out, ob, q.soa, tq2::soa_bytes(q.n, q.k)) ||
          overlaps(p.out, ob, q.residual, size_t(q.n) * 4))
        return TQ2_ERR_ALIAS;
    }
  }
  // Each k's launch is one grid of at most ceil(n / 4) row blocks per problem;
  // a grid that would not fit is rejected before anything is enqueued.
  bool any = false;
  for (int i = 0; i < count; ++i) {
    if (problems[i].n == 0) continue;
    any = true;
    int64_t blocks = 0;
    for (int j = 0; j < count; ++j)
      if (problems[j].n > 0 && problems[j].k == problems[i].k) blocks += (problems[j].n + 3) / 4;
    if (blocks > INT32_MAX) return TQ2_ERR_INVALID;
  }
  if (!any) return TQ2_OK;
  const int dst = check_device();
  if (dst != TQ2_OK) return dst;
  // One launch per distinct k, in increasing k.
  hipStream_t s = static_cast<hipStream_t>(stream);
  int64_t last_k = 0;
  for (;;) {
    int64_t k = 0;
    for (int i = 0; i < count; ++i)
      if (problems[i].n > 0 && problems[i].k > last_k && (k == 0 || problems[i].k < k))
        k = problems[i].k;
    if (k == 0) break;
    tq2::GemvProblem group[tq2::kGemvBatchMax];
    int ng = 0;
    for (int i = 0; i < count; ++i) {
      const tq2_gemv_problem& p = problems[i];
      if (p.n > 0 && p.k == k)
        group[ng++] = {static_cast<const uint8_t*>(p.soa), p.x, p.residual, p.out, p.n};
    }
    const int st = launch_status(tq2::launch_gemv_batched(group, ng, k, s));
    if (st != TQ2_OK) return st;
    last_k = k;
  }
  return TQ2_OK;
}

int tq2_gemm(const void* soa, const float* x, const float* residual, float* out, int64_t m,
             int64_t n, int64_t k, void* stream) {
  const int st = check_shape(m, n, k);
  if (st != TQ2_OK) return st;
  if (m == 0 || n == 0) return TQ2_OK;
  return gemm_impl(tq2::Fmt::kTq2, tq2_gemm_path(m, n, k), soa, x, residual, out, m, n, k, stream);
}

size_t tq2_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  if (check_shape(m, n, k) != TQ2_OK || m == 0 || n == 0) return 0;
  if (tq2_gemm_path(m, n, k) != 2 || !gemm_shape_fits(n, k)) return 0;
  return tq2::gemm_ws_bytes(m, n, k);
}

int tq2_gemm_ws(const void* soa, const float* x, const float* residual, float* out, int64_t m,
                int64_t n, int64_t k, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_shape(m, n, k);
  if (st != TQ2_OK) return st;
  if (m == 0 || n == 0) return TQ2_OK;
  const size_t need = tq2_gemm_workspace_bytes(m, n, k);
  if (need == 0) return tq2_gemm(soa, x, residual, out, m, n, k, stream);
  st = check_matmul_host(soa, x, residual, out, m, n, k);
  if (st != TQ2_OK) return st;
  if (!workspace || workspace_bytes < need) return TQ2_ERR_INVALID;
  if (!aligned(workspace, 256)) return TQ2_ERR_ALIGN;
  const size_t ob = size_t(m) * size_t(n) * 4;
  if (overlaps(workspace, need, x, size_t(m) * size_t(k) * 4) ||
      overlaps(workspace, need, out, ob) || overlaps(workspace, need, residual, ob) ||
      overlaps(workspace, need, soa, tq2::soa_bytes(n, k)))
    return TQ2_ERR_ALIAS;
  st = check_device();
  if (st != TQ2_OK) return st;
  return launch_status(tq2::launch_gemm_ws(static_cast<const uint8_t*>(soa), x, residual, out, m,
                                           n, k, workspace, static_cast<hipStream_t>(stream)));
}

int tq2_gemm_noalloc(const void* soa, const float* x, const float* residual, float* out,
                     int64_t m, int64_t n, int64_t k, void* stream) {
  int st = check_shape(m, n, k);
  if (st != TQ2_OK) return st;
  if (m == 0 || n == 0) return TQ2_OK;
  const size_t need = tq2_gemm_workspace_bytes(m, n, k);
  if (need == 0) return tq2_gemm(soa, x, residual, out, m, n, k, stream);
  if (need > size_t(TQ2_NOALLOC_SCRATCH_BYTES)) return TQ2_ERR_INVALID;
  st = check_matmul_host(soa, x, residual, out, m, n, k);
  if (st != TQ2_OK) return st;
  st = check_device();
  if (st != TQ2_OK) return st;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return TQ2_ERR_DEVICE;
  void* ws = device_scratch(dev);
  if (!ws) return TQ2_ERR_DEVICE;
  return launch_status(tq2::launch_gemm_ws(static_cast<const uint8_t*>(soa), x, residual, out, m,
                                           n, k, ws, static_cast<hipStream_t>(stream)));
}

int tq2_gemm_precise(const void* soa, const float* x, const float* residual, float* out,
                     int64_t m, int64_t n, int64_t k, void* stream) {
  const int st = check_shape(m, n, k);
  if (st != TQ2_OK) return st;
  if (m == 0 || n == 0) return TQ2_OK;
  return gemm_impl(tq2::Fmt::kTq2, m <= 1 ? 0 : 1, soa, x, residual, out, m, n, k, stream);
}

int tq2_gate_up_swiglu(const void* gate_soa, const void* up_soa, const float* x, float* out,
                       int64_t m, int64_t n, int64_t k, void* stream) {
  return swiglu_impl(tq2::Fmt::kTq2, gate_soa, up_soa, x, out, m, n, k, stream);
}

size_t tq2_q1_aos_bytes(int64_t n, int64_t k) {
  if (check_shape(0, n, k) != TQ2_OK) return 0;
  return size_t(n) * size_t(k / tq2::kBlockWeights) * tq2::kQ1BlockBytes;
}

size_t tq2_q1_soa_bytes(int64_t n, int64_t k) {
  if (check_shape(0, n, k) != TQ2_OK) return 0;
  return tq2::soa_bytes(tq2::Fmt::kQ1, n, k);
}

int tq2_q1_reformat_aos_to_soa(const void* aos, void* soa, int64_t n, int64_t k, void* stream) {
  return reformat_impl(tq2::Fmt::kQ1, aos, soa, n, k, stream);
}

int tq2_q1_gemv(const void* soa, const float* x, const float* residual, float* out, int64_t n,
                int64_t k, void* stream) {
  return gemv_impl(tq2::Fmt::kQ1, soa, x, residual, out, n, k, stream);
}

int tq2_q1_gemm(const void* soa, const float* x, const float* residual, float* out, int64_t m,
                int64_t n, int64_t k, void* stream) {
  const int st = check_shape(m, n, k);
  if (st != TQ2_OK) return st;
  if (m == 0 || n == 0) return TQ2_OK;
  return gemm_impl(tq2::Fmt::kQ1, tq2_gemm_path(m, n, k), soa, x, residual, out, m, n, k, stream);
}

int tq2_q1_gate_up_swiglu(const void* gate_soa, const void* up_soa, const float* x, float* out,
                          int64_t m, int64_t n, int64_t k, void* stream) {
  return swiglu_impl(tq2::Fmt::kQ1, gate_soa, up_soa, x, out, m, n, k, stream);
}

const char* tq2_status_string(int status) {
  switch (status) {
    case TQ2_OK: return "ok";
    case TQ2_ERR_INVALID: return "invalid argument (null pointer, negative or oversized dimension, k <= 0)";
    case TQ2_ERR_SHAPE: return "k is not a multiple of 128";
    case TQ2_ERR_ALIGN: return "misaligned pointer (soa needs 256 bytes, x/out/residual 16 bytes)";
    case TQ2_ERR_ALIAS: return "output overlaps an input (only out == residual is allowed)";
    case TQ2_ERR_DEVICE: return "current HIP device is not gfx950 or cannot be queried";
    case TQ2_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown tq2 status";
  }
}

}  // extern "C"
