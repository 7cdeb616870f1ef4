// extern "C" entry points of libnf4.so (declared and documented in nf4.h):
// argument validation, launch planning and path counters.  No entry point
// allocates, frees or synchronises.
#include <atomic>
#include <climits>
#include <mutex>

#include "../../include/nf4.h"
#include "nf4_internal.hpp"

namespace nf4 {

static std::atomic<int64_t> g_path_counts[NF4_PATH_COUNT];

// The fixed device buffer of nf4_matmul_fwd_noalloc (split-contraction
// partials).  In host code its name is only a stand-in for registration: the
// device address is obtained per device with hipGetSymbolAddress and only
// that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[NF4_NOALLOC_SCRATCH_BYTES];

void count_path(int path) {
  if (path >= 0 && path < NF4_PATH_COUNT) g_path_counts[path].fetch_add(1, std::memory_order_relaxed);
}

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Checks shared by every call that takes the W-args.
int check_w(const uint8_t* packed, const void* absmax, const float* nested_absmax,
            const float* nested_offset, const float* code16, const float* ncode, int64_t N,
            int64_t K, int bits = 4) {
  if (N < 0 || K < 0) return NF4_ERR_SHAPE;
  if (N > 0 && K > INT64_MAX / N) return NF4_ERR_SHAPE;
  // a weight with no elements has no packed bytes or scales to point at
  if (!code16 || ((!packed || !absmax) && N * K != 0)) return NF4_ERR_NULL;
  if (nested_absmax && (!nested_offset || !ncode)) return NF4_ERR_NULL;
  if (bits == 4 && (N * K) % 2) return NF4_ERR_SHAPE;
  if (!aligned16(packed)) return NF4_ERR_ALIGN;
  return NF4_OK;
}

int check_gemm_shape(int64_t M, int64_t N, int64_t K, bool bwd) {
  if (M < 0) return NF4_ERR_SHAPE;
  if (K % 64) return NF4_ERR_UNSUPPORTED;   // every 64-block must lie in one row of W
  if (bwd && (N % 8)) return NF4_ERR_UNSUPPORTED;
  if (M > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2) return NF4_ERR_UNSUPPORTED;
  return NF4_OK;
}

int to_status(hipError_t e) { return e == hipSuccess ? NF4_OK : NF4_ERR_HIP; }

// Zero fill of a bf16 output whose contraction is empty.  A kernel rather than
// hipMemsetAsync, so that a caller capturing the call into a HIP graph records
// a kernel node and never a memset node.  `out` is 16-byte aligned.
__global__ __launch_bounds__(256) void k_zero_bf16(uint16_t* __restrict__ out, int64_t n) {
  const int64_t n8 = n / 8;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n8; i += stride)
    reinterpret_cast<uint4*>(out)[i] = make_uint4(0u, 0u, 0u, 0u);
  if (blockIdx.x == 0 && threadIdx.x < n - 8 * n8) out[8 * n8 + threadIdx.x] = 0;
}

hipError_t zero_bf16(void* out, int64_t n, hipStream_t stream) {
  const int64_t blocks = (n / 8 + 255) / 256;
  const unsigned grid = static_cast<unsigned>(blocks < 1 ? 1 : (blocks > 2048 ? 2048 : blocks));
  k_zero_bf16<<<grid, 256, 0, stream>>>(static_cast<uint16_t*>(out), n);
  return hipGetLastError();
}

// Device address of the current device's copy of `scratch`, looked up once per
// device while it is current.  hipGetSymbolAddress allocates nothing.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return NF4_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return NF4_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return NF4_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return NF4_OK;
}

// fixed_scratch: ws is the library's own fixed buffer of ws_bytes; a plan
// that needs more is NF4_ERR_SCRATCH rather than a caller workspace error.
int matmul_common(GemmKind kind, const void* A, int64_t M, const uint8_t* packed,
                  const void* absmax, const float* nested_absmax, const float* nested_offset,
                  const float* code16, const float* ncode, int64_t N, int64_t K, void* C,
                  void* ws, size_t ws_bytes, void* stream, bool fixed_scratch = false,
                  int bits = 4) {
  const bool bwd = kind == GemmKind::kBwdInput;
  int st = check_w(packed, absmax, nested_absmax, nested_offset, code16, ncode, N, K, bits);
  if (st) return st;
  // an operand with no elements (empty batch, empty contraction, no output
  // columns) is never read or written and may be NULL, as torch gives for
  // empty tensors
  if (!A && M != 0 && (bwd ? N : K) != 0) return NF4_ERR_NULL;
  if (!C && M != 0 && (bwd ? K : N) != 0) return NF4_ERR_NULL;
  st = check_gemm_shape(M, N, K, bwd);
  if (st) return st;
  if (!aligned16(A) || !aligned16(C)) return NF4_ERR_ALIGN;
  if (M == 0 || N == 0 || K == 0) {
    if (M > 0 && (bwd ? K : N) > 0) {
      // an empty contraction: the product is all zeros
      return to_status(zero_bf16(C, M * (bwd ? K : N), static_cast<hipStream_t>(stream)));
    }
    return NF4_OK;
  }
  const GemmPlan plan = bits == 8 ? plan_gemm8(kind, M, N, K, device_cu_count())
                                  : plan_gemm(kind, M, N, K, device_cu_count());
  if (fixed_scratch) {
    if (plan.ws_bytes > ws_bytes) return NF4_ERR_SCRATCH;
    // set-up on the first call that reaches a launch on this device
    const int sst = scratch_for_current_device(&ws);
    if (sst) return sst;
  }
  if (plan.ws_bytes > 0 && (!ws || ws_bytes < plan.ws_bytes)) return NF4_ERR_WORKSPACE;
  if (plan.ws_bytes > 0 && !aligned16(ws)) return NF4_ERR_ALIGN;
  WArgs w{packed, absmax, nested_absmax, nested_offset, code16, ncode, N, K};
  w.bits = bits;
  if (bits == 8) return to_status(launch_gemm8(kind, plan, A, M, w, C, ws, static_cast<hipStream_t>(stream)));
  return to_status(launch_gemm(kind, plan, A, M, w, C, ws, static_cast<hipStream_t>(stream)));
}

int grouped_common(GemmKind kind, const void* A, const int32_t* offsets, int32_t E,
                   int64_t total_M, const uint8_t* packed, const void* absmax,
                   const float* nested_absmax, const float* nested_offset, const float* code16,
                   const float* ncode, int64_t N, int64_t K, void* C, void* ws, size_t ws_bytes,
                   void* stream, int bits = 4) {
  (void)ws;
  (void)ws_bytes;
  const bool bwd = kind == GemmKind::kBwdInput;
  if (E < 1) return NF4_ERR_SHAPE;
  if (N < 0 || K < 0 || (N > 0 && E > INT64_MAX / N)) return NF4_ERR_SHAPE;
  int st = check_w(packed, absmax, nested_absmax, nested_offset, code16, ncode,
                   static_cast<int64_t>(E) * N, K, bits);
  if (st) return st;
  if (!offsets) return NF4_ERR_NULL;
  if (!A && total_M != 0 && (bwd ? N : K) != 0) return NF4_ERR_NULL;
  if (!C && total_M != 0 && (bwd ? K : N) != 0) return NF4_ERR_NULL;
  st = check_gemm_shape(total_M, N, K, bwd);
  if (st) return st;
  if (!aligned16(A) || !aligned16(C)) return NF4_ERR_ALIGN;
  if (total_M == 0 || N == 0 || K == 0) {
    if (total_M > 0 && (bwd ? K : N) > 0) {
      return to_status(zero_bf16(C, total_M * (bwd ? K : N), static_cast<hipStream_t>(stream)));
    }
    return NF4_OK;
  }
  WArgs w{packed, absmax, nested_absmax, nested_offset, code16, ncode, N, K};
  w.bits = bits;
  if (bits == 8)
    return to_status(launch_grouped8(kind, A, offsets, E, total_M, w, C, static_cast<hipStream_t>(stream)));
  const GemmPlan plan = plan_grouped(kind, total_M, N, K, E);
  return to_status(launch_grouped(kind, plan, A, offsets, E, total_M, w, C,
                                  static_cast<hipStream_t>(stream)));
}

int quantize_common(const void* w, int w_dtype, int64_t N, int64_t K, const float* code16,
                    const float* nested_code256, uint8_t* packed, void* absmax,
                    float* nested_absmax, float* nested_offset, void* ws, size_t ws_bytes,
                    void* stream, int bits) {
  if (w_dtype != NF4_DTYPE_F32 && w_dtype != NF4_DTYPE_BF16) return NF4_ERR_DTYPE;
  if (!w || !code16 || !packed || !absmax) return NF4_ERR_NULL;
  const bool nested = nested_code256 != nullptr;
  if (nested && (!nested_absmax || !nested_offset)) return NF4_ERR_NULL;
  if (N < 0 || K < 0) return NF4_ERR_SHAPE;
  if (N > 0 && K > INT64_MAX / N) return NF4_ERR_SHAPE;
  const int64_t n = N * K;
  if (bits == 4 && n % 2) return NF4_ERR_SHAPE;
  if (n == 0) return NF4_OK;
  if (!aligned16(packed) || !aligned16(w)) return NF4_ERR_ALIGN;
  const size_t need = quantize_ws_bytes(n, nested);
  if (need > 0 && (!ws || ws_bytes < need)) return NF4_ERR_WORKSPACE;
  if (need > 0 && !aligned16(ws)) return NF4_ERR_ALIGN;
  const hipError_t e = launch_quantize(w, w_dtype == NF4_DTYPE_BF16, n, code16, nested_code256,
                                       packed, absmax, nested_absmax, nested_offset, ws,
                                       static_cast<hipStream_t>(stream), bits);
  if (e == hipSuccess) count_path(NF4_PATH_QUANTIZE);
  return e == hipSuccess ? NF4_OK : NF4_ERR_HIP;
}

int dequantize_common(const uint8_t* packed, const void* absmax, const float* nested_absmax,
                      const float* nested_offset, const float* code16,
                      const float* nested_code256, int64_t N, int64_t K, int out_dtype, void* out,
                      void* stream, int bits) {
  if (out_dtype != NF4_DTYPE_F32 && out_dtype != NF4_DTYPE_BF16) return NF4_ERR_DTYPE;
  int st = check_w(packed, absmax, nested_absmax, nested_offset, code16, nested_code256, N, K, bits);
  if (st) return st;
  if (!out) return NF4_ERR_NULL;
  if (!aligned16(out)) return NF4_ERR_ALIGN;
  const int64_t n = N * K;
  if (n == 0) return NF4_OK;
  WArgs w{packed, absmax, nested_absmax, nested_offset, code16, nested_code256, N, K};
  w.bits = bits;
  const hipError_t e = launch_dequantize(w, n, out_dtype == NF4_DTYPE_BF16, out,
                                         static_cast<hipStream_t>(stream));
  if (e == hipSuccess) count_path(NF4_PATH_DEQUANTIZE);
  return e == hipSuccess ? NF4_OK : NF4_ERR_HIP;
}

}  // namespace
}  // namespace nf4

using namespace nf4;

extern "C" {

int nf4_quantize(const void* w, int w_dtype, int64_t N, int64_t K, const float* code16,
                 const float* nested_code256, uint8_t* packed, void* absmax, float* nested_absmax,
                 float* nested_offset, void* ws, size_t ws_bytes, void* stream) {
  return quantize_common(w, w_dtype, N, K, code16, nested_code256, packed, absmax, nested_absmax,
                         nested_offset, ws, ws_bytes, stream, 4);
}

int nf4_quantize_8bit(const void* w, int w_dtype, int64_t N, int64_t K, const float* code256,
                      const float* nested_code256, uint8_t* packed, void* absmax,
                      float* nested_absmax, float* nested_offset, void* ws, size_t ws_bytes,
                      void* stream) {
  return quantize_common(w, w_dtype, N, K, code256, nested_code256, packed, absmax, nested_absmax,
                         nested_offset, ws, ws_bytes, stream, 8);
}

int nf4_dequantize(const uint8_t* packed, const void* absmax, const float* nested_absmax,
                   const float* nested_offset, const float* code16, const float* nested_code256,
                   int64_t N, int64_t K, int out_dtype, void* out, void* stream) {
  return dequantize_common(packed, absmax, nested_absmax, nested_offset, code16, nested_code256, N,
                           K, out_dtype, out, stream, 4);
}

int nf4_dequantize_8bit(const uint8_t* packed, const void* absmax, const float* nested_absmax,
                        const float* nested_offset, const float* code256,
                        const float* nested_code256, int64_t N, int64_t K, int out_dtype,
                        void* out, void* stream) {
  return dequantize_common(packed, absmax, nested_absmax, nested_offset, code256, nested_code256, N,
                           K, out_dtype, out, stream, 8);
}

int nf4_matmul_fwd_8bit(const void* x, int64_t M, const uint8_t* packed, const void* absmax,
                        const float* nested_absmax, const float* nested_offset,
                        const float* code256, const float* nested_code256, int64_t N, int64_t K,
                        void* y, void* ws, size_t ws_bytes, void* stream) {
  return matmul_common(GemmKind::kFwd, x, M, packed, absmax, nested_absmax, nested_offset, code256,
                       nested_code256, N, K, y, ws, ws_bytes, stream, false, 8);
}

int nf4_matmul_bwd_input_8bit(const void* grad_y, int64_t M, const uint8_t* packed,
                              const void* absmax, const float* nested_absmax,
                              const float* nested_offset, const float* code256,
                              const float* nested_code256, int64_t N, int64_t K, void* grad_x,
                              void* ws, size_t ws_bytes, void* stream) {
  return matmul_common(GemmKind::kBwdInput, grad_y, M, packed, absmax, nested_absmax,
                       nested_offset, code256, nested_code256, N, K, grad_x, ws, ws_bytes, stream,
                       false, 8);
}

int nf4_grouped_matmul_fwd_8bit(const void* x, const int32_t* offsets, int32_t E, int64_t total_M,
                                const uint8_t* packed, const void* absmax,
                                const float* nested_absmax, const float* nested_offset,
                                const float* code256, const float* nested_code256, int64_t N,
                                int64_t K, void* y, void* ws, size_t ws_bytes, void* stream) {
  return grouped_common(GemmKind::kFwd, x, offsets, E, total_M, packed, absmax, nested_absmax,
                        nested_offset, code256, nested_code256, N, K, y, ws, ws_bytes, stream, 8);
}

int nf4_grouped_matmul_bwd_input_8bit(const void* grad_y, const int32_t* offsets, int32_t E,
                                      int64_t total_M, const uint8_t* packed, const void* absmax,
                                      const float* nested_absmax, const float* nested_offset,
                                      const float* code256, const float* nested_code256,
                                      int64_t N, int64_t K, void* grad_x, void* ws,
                                      size_t ws_bytes, void* stream) {
  return grouped_common(GemmKind::kBwdInput, grad_y, offsets, E, total_M, packed, absmax,
                        nested_absmax, nested_offset, code256, nested_code256, N, K, grad_x, ws,
                        ws_bytes, stream, 8);
}

int nf4_matmul_fwd(const void* x, int64_t M, const uint8_t* packed, const void* absmax,
                   const float* nested_absmax, const float* nested_offset, const float* code16,
                   const float* nested_code256, int64_t N, int64_t K, void* y, void* ws,
                   size_t ws_bytes, void* stream) {
  return matmul_common(GemmKind::kFwd, x, M, packed, absmax, nested_absmax, nested_offset,
                       code16, nested_code256, N, K, y, ws, ws_bytes, stream);
}

int nf4_matmul_fwd_noalloc(const void* x, int64_t M, const uint8_t* packed, const void* absmax,
                           const float* nested_absmax, const float* nested_offset,
                           const float* code16, const float* nested_code256, int64_t N, int64_t K,
                           void* y, void* stream) {
  return matmul_common(GemmKind::kFwd, x, M, packed, absmax, nested_absmax, nested_offset, code16,
                       nested_code256, N, K, y, nullptr, NF4_NOALLOC_SCRATCH_BYTES, stream,
                       /*fixed_scratch=*/true);
}

int nf4_matmul_bwd_input(const void* grad_y, int64_t M, const uint8_t* packed,
                         const void* absmax, const float* nested_absmax,
                         const float* nested_offset, const float* code16,
                         const float* nested_code256, int64_t N, int64_t K, void* grad_x,
                         void* ws, size_t ws_bytes, void* stream) {
  return matmul_common(GemmKind::kBwdInput, grad_y, M, packed, absmax, nested_absmax,
                       nested_offset, code16, nested_code256, N, K, grad_x, ws, ws_bytes,
                       stream);
}

int nf4_grouped_matmul_fwd(const void* x, const int32_t* offsets, int32_t E, int64_t total_M,
                           const uint8_t* packed, const void* absmax, const float* nested_absmax,
                           const float* nested_offset, const float* code16,
                           const float* nested_code256, int64_t N, int64_t K, void* y, void* ws,
                           size_t ws_bytes, void* stream) {
  return grouped_common(GemmKind::kFwd, x, offsets, E, total_M, packed, absmax, nested_absmax,
                        nested_offset, code16, nested_code256, N, K, y, ws, ws_bytes, stream);
}

int nf4_grouped_matmul_bwd_input(const void* grad_y, const int32_t* offsets, int32_t E,
                                 int64_t total_M, const uint8_t* packed, const void* absmax,
                                 const float* nested_absmax, const float* nested_offset,
                                 const float* code16, const float* nested_code256, int64_t N,
                                 int64_t K, void* grad_x, void* ws, size_t ws_bytes,
                                 void* stream) {
  return grouped_common(GemmKind::kBwdInput, grad_y, offsets, E, total_M, packed, absmax,
                        nested_absmax, nested_offset, code16, nested_code256, N, K, grad_x, ws,
                        ws_bytes, stream);
}

size_t nf4_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int32_t E) {
  if (M < 0 || N < 0 || K < 0) return SIZE_MAX;
  if (N > 0 && K > INT64_MAX / N) return SIZE_MAX;
  switch (op) {
    case NF4_OP_QUANTIZE:
      return quantize_ws_bytes(N * K, true);
    case NF4_OP_MATMUL_FWD:
    case NF4_OP_MATMUL_BWD_INPUT: {
      if (M == 0 || N == 0 || K == 0) return 0;
      const GemmKind kind = op == NF4_OP_MATMUL_FWD ? GemmKind::kFwd : GemmKind::kBwdInput;
      return plan_gemm(kind, M, N, K, device_cu_count()).ws_bytes;
    }
    case NF4_OP_GROUPED_FWD:
    case NF4_OP_GROUPED_BWD_INPUT:
      if (E < 1) return SIZE_MAX;
      return 0;
    case NF4_OP_MATMUL_FWD_8BIT:
    case NF4_OP_MATMUL_BWD_INPUT_8BIT: {
      if (M == 0 || N == 0 || K == 0) return 0;
      const GemmKind kind = op == NF4_OP_MATMUL_FWD_8BIT ? GemmKind::kFwd : GemmKind::kBwdInput;
      return plan_gemm8(kind, M, N, K, device_cu_count()).ws_bytes;
    }
    default:
      return SIZE_MAX;
  }
}

int64_t nf4_packed_bytes(int64_t N, int64_t K) {
  if (N < 0 || K < 0 || (N > 0 && K > INT64_MAX / N)) return -1;
  return N * K / 2;
}

int64_t nf4_absmax_count(int64_t N, int64_t K) {
  if (N < 0 || K < 0 || (N > 0 && K > INT64_MAX / N)) return -1;
  return ceil_div(N * K, 64);
}

int64_t nf4_nested_count(int64_t N, int64_t K) {
  const int64_t nb = nf4_absmax_count(N, K);
  return nb < 0 ? -1 : ceil_div(nb, 256);
}

int64_t nf4_path_count(int path) {
  if (path < 0 || path >= NF4_PATH_COUNT) return -1;
  return g_path_counts[path].load(std::memory_order_relaxed);
}

void nf4_reset_path_counts(void) {
  for (auto& c : g_path_counts) c.store(0, std::memory_order_relaxed);
}

const char* nf4_status_str(int status) {
  switch (status) {
    case NF4_OK: return "NF4_OK: success";
    case NF4_ERR_NULL: return "NF4_ERR_NULL: a required pointer is NULL";
    case NF4_ERR_SHAPE: return "NF4_ERR_SHAPE: invalid sizes";
    case NF4_ERR_UNSUPPORTED: return "NF4_ERR_UNSUPPORTED: unsupported shape (K % 64, N % 8 or size limit)";
    case NF4_ERR_ALIGN: return "NF4_ERR_ALIGN: a pointer is not 16-byte aligned";
    case NF4_ERR_WORKSPACE: return "NF4_ERR_WORKSPACE: workspace missing or too small";
    case NF4_ERR_HIP: return "NF4_ERR_HIP: the HIP runtime reported an error";
    case NF4_ERR_DTYPE: return "NF4_ERR_DTYPE: unknown dtype selector";
    case NF4_ERR_SCRATCH:
      return "NF4_ERR_SCRATCH: the product needs more split partials than the fixed scratch buffer "
             "of nf4_matmul_fwd_noalloc holds (NF4_NOALLOC_SCRATCH_BYTES); use nf4_matmul_fwd with a workspace";
    default: return "unknown NF4 status";
  }
}

const char* nf4_version(void) { return "nf4-mi355x 0.1 (gfx950)"; }

}  // extern "C"
