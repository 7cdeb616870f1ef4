// Internal launch interface between the C ABI (nf4_abi.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nf4 {

// The W-args of the ABI: one quantised tensor of N rows x K columns (for the
// grouped calls, E*N rows; N and K are per expert).
struct WArgs {
  const uint8_t* packed;
  const void* absmax;
  const float* nested_absmax;  // NULL -> plain fp32 absmax
  const float* nested_offset;
  const float* code;           // 16 fp32
  const float* ncode;          // 256 fp32 (nested only)
  int64_t N, K;
  int32_t bits = 4;            // 4: NF4-style packed nibbles, 16-entry code;
                               // 8: one index per byte, 256-entry code
  bool nested() const { return nested_absmax != nullptr; }
};

// ---- codec -----------------------------------------------------------------
size_t quantize_ws_bytes(int64_t n_elems, bool nested);
hipError_t launch_quantize(const void* w, bool w_is_bf16, int64_t n_elems, const float* code,
                           const float* ncode, uint8_t* packed, void* absmax,
                           float* nested_absmax, float* nested_offset, void* ws,
                           hipStream_t stream, int bits = 4);
hipError_t launch_dequantize(const WArgs& w, int64_t n_elems, bool out_bf16, void* out,
                             hipStream_t stream);

// ---- fused matmuls ---------------------------------------------------------
enum class GemmKind { kFwd, kBwdInput };

// How one dense (non-grouped) call is split into launches.  A pure function
// of (M, N, K, kind, compute units).
struct GemmPlan {
  int bm;          // rows of the activation tile
  int bn;          // output columns per tile (256 or 128)
  int consumers;   // MFMA waves per SIMD (1 or 2) beside one expanding wave;
                   // 0 = the 256 x 256 ping-pong kernel, 3 = the
                   // register-operand forward, kStagedTile = the
                   // register-staged tile kernel (bn = 128, bm = 32/64/128),
                   // kStagedTile8 the same with 8 waves (bm = 64/128)
  int splits;      // contraction split count (1 = none)
  bool small_m;    // weight-streaming forward (bm = MFMA rows 16 / 32)
  int kc;          // weight-streaming forward: contraction per split
  size_t ws_bytes; // fp32 partials when splits > 1
};
constexpr int kStagedTile = 5;    // 4 waves
constexpr int kStagedTile8 = 6;   // 8 waves (NF4, 64 or 128 rows; 128 x 256)
int device_cu_count();
GemmPlan plan_gemm(GemmKind kind, int64_t M, int64_t N, int64_t K, int cus);
GemmPlan plan_grouped(GemmKind kind, int64_t total_M, int64_t N, int64_t K, int32_t E);

// small-M forward (nf4_gemv.hip)
void plan_small_m(GemmPlan& pl, int64_t M, int64_t N, int64_t K, int cus);
hipError_t launch_gemv(const GemmPlan& plan, const void* x, int64_t M, const WArgs& w, void* y,
                       void* ws, hipStream_t stream);

hipError_t launch_gemm(GemmKind kind, const GemmPlan& plan, const void* A, int64_t M,
                       const WArgs& w, void* C, void* ws, hipStream_t stream);
hipError_t launch_grouped(GemmKind kind, const GemmPlan& plan, const void* A,
                          const int32_t* offsets, int32_t E, int64_t total_M, const WArgs& w,
                          void* C, hipStream_t stream);

// 8-bit blockwise matmuls (one index per byte, 256-entry table): their own
// tiled kernel (nf4_gemm.hip), 128 or 32 activation rows per tile
GemmPlan plan_gemm8(GemmKind kind, int64_t M, int64_t N, int64_t K, int cus);
hipError_t launch_gemm8(GemmKind kind, const GemmPlan& plan, const void* A, int64_t M,
                        const WArgs& w, void* C, void* ws, hipStream_t stream);
hipError_t launch_grouped8(GemmKind kind, const void* A, const int32_t* offsets, int32_t E,
                           int64_t total_M, const WArgs& w, void* C, hipStream_t stream);

// path counters (defined in nf4_abi.hip)
void count_path(int path);

}  // namespace nf4
