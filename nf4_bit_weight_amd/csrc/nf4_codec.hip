// NF4 codec kernels: blockwise quantisation (with the nested 8-bit form) and
// dequantisation to bf16 / fp32.  Off the matmul hot path; HBM-bound.
//
// Quantisation follows quantize_4bit(w, blocksize=64, quant_type="nf4",
// compress_statistics=...) as called in bitsandbytes #2034 ("Minimal
// reproducer"), with the readings of the encoding documented in nf4.h:
// midpoint thresholds with strict '>', correctly rounded fp32 division,
// high nibble first, nested mean offset summed in a fixed fp64 order.
#include "nf4_device.hpp"
#include "nf4_internal.hpp"

namespace nf4 {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float load_w(const float* w, int64_t i) { return w[i]; }
__device__ __forceinline__ float load_w(const uint16_t* w, int64_t i) {
  return __uint_as_float(static_cast<uint32_t>(w[i]) << 16);   // exact widening
}

// Number of midpoints strictly below t (the nearest-code index).
__device__ __forceinline__ uint32_t nf4_index(float t, const float (&mid)[15]) {
  uint32_t q = 0;
#pragma unroll
  for (int j = 0; j < 15; ++j) q += (t > mid[j]) ? 1u : 0u;
  return q;
}

// One thread per 8 consecutive elements, 8 threads per 64-block.  Writes the
// packed bytes and the fp32 block absmax (to `absmax_out`: the output in the
// plain form, the workspace in the nested form).
template <typename T>
__global__ __launch_bounds__(kThreads) void k_quant_blocks(const T* __restrict__ w, int64_t n,
                                                           const float* __restrict__ code,
                                                           uint8_t* __restrict__ packed,
                                                           float* __restrict__ absmax_out) {
  float mid[15];
#pragma unroll
  for (int j = 0; j < 15; ++j) mid[j] = __fmul_rn(__fadd_rn(code[j], code[j + 1]), 0.5f);

  const int64_t g = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;  // 8-group
  const int64_t e0 = g * 8;
  float v[8];
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = (e0 + i < n) ? load_w(w, e0 + i) : 0.f;
    m = fmaxf(m, fabsf(v[i]));
  }
  // max over the 8 threads of the block (lanes aligned to 8 inside the wave)
  m = fmaxf(m, __shfl_xor(m, 1, 8));
  m = fmaxf(m, __shfl_xor(m, 2, 8));
  m = fmaxf(m, __shfl_xor(m, 4, 8));
  if (e0 >= n) return;

  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float t = (m == 0.f) ? 0.f : v[i] / m;   // correctly rounded division
    const uint32_t q = nf4_index(t, mid);
    const int byte = i >> 1;
    word |= q << (8 * byte + ((i & 1) ? 0 : 4));
  }
  if (e0 + 8 <= n) {
    reinterpret_cast<uint32_t*>(packed)[g] = word;
  } else {
    for (int64_t i = e0; i < n; i += 2) packed[i / 2] = static_cast<uint8_t>(word >> (8 * ((i - e0) / 2)));
  }
  if ((g & 7) == 0) absmax_out[g >> 3] = m;
}

// Nested step 1: fp64 sequential sum of each chunk of 256 absmax values.  One
// wave per chunk: the wave reads the chunk with coalesced 16-byte loads into
// its LDS slice, then lane 0 adds the 256 values in index order (the order the
// mean offset is defined with, so it is reproduced bit for bit).
constexpr int kSumWaves = kThreads / 64;
__global__ __launch_bounds__(kThreads) void k_chunk_sums(const float* __restrict__ absmax,
                                                         int64_t nb, double* __restrict__ sums) {
  __shared__ float chunk[kSumWaves][kNestedBlock];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t g = static_cast<int64_t>(blockIdx.x) * kSumWaves + wave;
  const int64_t b0 = g * kNestedBlock;
  if (b0 >= nb) return;                                   // whole wave leaves together
  const int64_t len = (b0 + kNestedBlock < nb) ? kNestedBlock : nb - b0;
  if (len == kNestedBlock && (reinterpret_cast<uintptr_t>(absmax) & 15u) == 0) {
    reinterpret_cast<f32x4_t*>(chunk[wave])[lane] = reinterpret_cast<const f32x4_t*>(absmax + b0)[lane];
  } else {
    for (int i = lane; i < len; i += 64) chunk[wave][i] = absmax[b0 + i];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lane != 0) return;
  double s = 0.0;
  for (int i = 0; i < len; ++i) s += static_cast<double>(chunk[wave][i]);
  sums[g] = s;
}

// Nested step 2: the chunk sums are added in order g = 0, 1, ... by one thread;
// the workgroup stages them through LDS in coalesced pieces so the serial
// chain waits on LDS, not on a global load per term.
constexpr int kOffPiece = 2048;
__global__ __launch_bounds__(kThreads) void k_offset(const double* __restrict__ sums, int64_t ng,
                                                     int64_t nb, float* __restrict__ offset) {
  __shared__ double piece[kOffPiece];
  double s = 0.0;
  for (int64_t g0 = 0; g0 < ng; g0 += kOffPiece) {
    const int len = static_cast<int>(ng - g0 < kOffPiece ? ng - g0 : kOffPiece);
    for (int i = threadIdx.x; i < len; i += kThreads) piece[i] = sums[g0 + i];
    __syncthreads();
    if (threadIdx.x == 0)
      for (int i = 0; i < len; ++i) s += piece[i];
    __syncthreads();
  }
  if (threadIdx.x == 0) offset[0] = static_cast<float>(s / static_cast<double>(nb));
}

// Nested step 3: one workgroup per group of 256 absmax values.
__global__ __launch_bounds__(kThreads) void k_nested(const float* __restrict__ absmax, int64_t nb,
                                                     const float* __restrict__ ncode,
                                                     const float* __restrict__ offset_p,
                                                     uint8_t* __restrict__ q2_out,
                                                     float* __restrict__ s2_out) {
  __shared__ float mid2[256];
  __shared__ float wmax[kThreads / 64];
  const int tid = threadIdx.x;
  if (tid < 255) mid2[tid] = __fmul_rn(__fadd_rn(ncode[tid], ncode[tid + 1]), 0.5f);
  const float off = offset_p[0];
  const int64_t b = static_cast<int64_t>(blockIdx.x) * kNestedBlock + tid;
  const float c = (b < nb) ? __fsub_rn(absmax[b], off) : 0.f;
  float m = fabsf(c);
  for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
  if ((tid & 63) == 0) wmax[tid >> 6] = m;
  __syncthreads();
  float s2 = wmax[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) s2 = fmaxf(s2, wmax[i]);
  if (b >= nb) return;
  const float t = (s2 == 0.f) ? 0.f : c / s2;
  int lo = 0, hi = 255;                           // first j with !(t > mid2[j])
  while (lo < hi) {
    const int md = (lo + hi) >> 1;
    if (t > mid2[md]) lo = md + 1; else hi = md;
  }
  q2_out[b] = static_cast<uint8_t>(lo);
  if (tid == 0) s2_out[blockIdx.x] = s2;
}

// Dequantisation to bf16: one thread per packed dword (8 elements).
template <bool NESTED>
__global__ __launch_bounds__(kThreads) void k_dequant_bf16(WArgs w, int64_t n,
                                                           uint16_t* __restrict__ out) {
  __shared__ float sncode[256];
  float code[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) code[i] = w.code[i];
  float off = 0.f;
  if constexpr (NESTED) {
    sncode[threadIdx.x] = w.ncode[threadIdx.x];
    off = w.nested_offset[0];
    __syncthreads();
  }
  const int64_t g = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t e0 = g * 8;
  if (e0 >= n) return;
  const float a = block_scale<NESTED>(w.absmax, w.nested_absmax, off, sncode, e0 / kBlock);
  const Lut t = make_lut(code, a);
  if (e0 + 8 <= n) {
    const uint32_t p = reinterpret_cast<const uint32_t*>(w.packed)[g];
    uint32_t o[4];
    expand8(p, t, o);
    u32x4_t v = {o[0], o[1], o[2], o[3]};
    reinterpret_cast<u32x4_t*>(out)[g] = v;
  } else {
    for (int64_t i = e0; i < n; ++i) {
      const uint32_t byte = w.packed[i / 2];
      const uint32_t q = (i & 1) ? (byte & 15u) : (byte >> 4);
      out[i] = to_bf16(__fmul_rn(code[q], a));
    }
  }
}

// Dequantisation to fp32 (no bf16 rounding): fp32(code[q] * absmax_hat).
template <bool NESTED>
__global__ __launch_bounds__(kThreads) void k_dequant_f32(WArgs w, int64_t n,
                                                          float* __restrict__ out) {
  __shared__ float sncode[256];
  __shared__ float scode[16];
  if (threadIdx.x < 16) scode[threadIdx.x] = w.code[threadIdx.x];
  float off = 0.f;
  if constexpr (NESTED) {
    sncode[threadIdx.x] = w.ncode[threadIdx.x];
    off = w.nested_offset[0];
  }
  __syncthreads();
  const int64_t g = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t e0 = g * 8;
  if (e0 >= n) return;
  const float a = block_scale<NESTED>(w.absmax, w.nested_absmax, off, sncode, e0 / kBlock);
  if (e0 + 8 <= n) {
    const uint32_t p = reinterpret_cast<const uint32_t*>(w.packed)[g];
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t q = (p >> (8 * (i >> 1) + ((i & 1) ? 0 : 4))) & 15u;
      v[i] = __fmul_rn(scode[q], a);
    }
    f32x4_t lo = {v[0], v[1], v[2], v[3]};
    f32x4_t hi = {v[4], v[5], v[6], v[7]};
    reinterpret_cast<f32x4_t*>(out)[2 * g] = lo;
    reinterpret_cast<f32x4_t*>(out)[2 * g + 1] = hi;
  } else {
    for (int64_t i = e0; i < n; ++i) {
      const uint32_t byte = w.packed[i / 2];
      const uint32_t q = (i & 1) ? (byte & 15u) : (byte >> 4);
      out[i] = __fmul_rn(scode[q], a);
    }
  }
}

// ---- 8-bit blockwise variants (one index per byte, 256-entry table) --------------
// The bitsandbytes fork PR "Experts trainability ... ExpertsNbit", "Commit 1"
// table lists 8-bit blockwise formats (int8 map, fp8 e4m3 codebook) with the
// same 64-element blocks; the 256-entry table is an argument, the index is
// the number of table midpoints strictly below t (binary search in LDS).

// One thread per 8 consecutive elements, 8 threads per 64-block.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_quant_blocks8(const T* __restrict__ w, int64_t n,
                                                            const float* __restrict__ code,
                                                            uint8_t* __restrict__ packed,
                                                            float* __restrict__ absmax_out) {
  __shared__ float mid[256];
  if (threadIdx.x < 255) mid[threadIdx.x] = __fmul_rn(__fadd_rn(code[threadIdx.x], code[threadIdx.x + 1]), 0.5f);
  __syncthreads();
  const int64_t g = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;  // 8-group
  const int64_t e0 = g * 8;
  float v[8];
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = (e0 + i < n) ? load_w(w, e0 + i) : 0.f;
    m = fmaxf(m, fabsf(v[i]));
  }
  m = fmaxf(m, __shfl_xor(m, 1, 8));
  m = fmaxf(m, __shfl_xor(m, 2, 8));
  m = fmaxf(m, __shfl_xor(m, 4, 8));
  if (e0 >= n) return;
  uint32_t word[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float t = (m == 0.f) ? 0.f : v[i] / m;   // correctly rounded division
    int lo = 0, hi = 255;                           // first j with !(t > mid[j])
    while (lo < hi) {
      const int md = (lo + hi) >> 1;
      if (t > mid[md]) lo = md + 1; else hi = md;
    }
    word[i >> 2] |= static_cast<uint32_t>(lo) << (8 * (i & 3));
  }
  if (e0 + 8 <= n) {
    reinterpret_cast<u32x2_t*>(packed)[g] = u32x2_t{word[0], word[1]};
  } else {
    for (int64_t i = e0; i < n; ++i) packed[i] = static_cast<uint8_t>(word[(i - e0) >> 2] >> (8 * ((i - e0) & 3)));
  }
  if ((g & 7) == 0) absmax_out[g >> 3] = m;
}

// Dequantisation: one thread per 8 elements, the table in LDS.
template <bool NESTED, bool BF16>
__global__ __launch_bounds__(kThreads) void k_dequant8(WArgs w, int64_t n, void* __restrict__ out) {
  __shared__ float sncode[256];
  __shared__ float scode[256];
  scode[threadIdx.x] = w.code[threadIdx.x];
  float off = 0.f;
  if constexpr (NESTED) {
    sncode[threadIdx.x] = w.ncode[threadIdx.x];
    off = w.nested_offset[0];
  }
  __syncthreads();
  const int64_t g = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t e0 = g * 8;
  if (e0 >= n) return;
  const float a = block_scale<NESTED>(w.absmax, w.nested_absmax, off, sncode, e0 / kBlock);
  float v[8];
  if (e0 + 8 <= n) {
    const u32x2_t p = reinterpret_cast<const u32x2_t*>(w.packed)[g];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __fmul_rn(scode[(p[i >> 2] >> (8 * (i & 3))) & 0xFFu], a);
    if constexpr (BF16) {
      reinterpret_cast<u32x4_t*>(out)[g] = u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                   pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
    } else {
      reinterpret_cast<f32x4_t*>(out)[2 * g] = f32x4_t{v[0], v[1], v[2], v[3]};
      reinterpret_cast<f32x4_t*>(out)[2 * g + 1] = f32x4_t{v[4], v[5], v[6], v[7]};
    }
  } else {
    for (int64_t i = e0; i < n; ++i) {
      const float x = __fmul_rn(scode[w.packed[i]], a);
      if constexpr (BF16) static_cast<uint16_t*>(out)[i] = to_bf16(x);
      else static_cast<float*>(out)[i] = x;
    }
  }
}

inline unsigned grid_for(int64_t items) {
  return static_cast<unsigned>((items + kThreads - 1) / kThreads);
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace

size_t quantize_ws_bytes(int64_t n_elems, bool nested) {
  if (!nested) return 0;
  const int64_t nb = (n_elems + kBlock - 1) / kBlock;
  const int64_t ng = (nb + kNestedBlock - 1) / kNestedBlock;
  return align_up(static_cast<size_t>(nb) * 4, 256) + static_cast<size_t>(ng) * 8;
}

hipError_t launch_quantize(const void* w, bool w_is_bf16, int64_t n, const float* code,
                           const float* ncode, uint8_t* packed, void* absmax,
                           float* nested_absmax, float* nested_offset, void* ws,
                           hipStream_t stream, int bits) {
  const bool nested = ncode != nullptr;
  const int64_t nb = (n + kBlock - 1) / kBlock;
  const int64_t ng = (nb + kNestedBlock - 1) / kNestedBlock;
  float* am32 = nested ? static_cast<float*>(ws) : static_cast<float*>(absmax);
  const int64_t groups8 = (n + 7) / 8;
  if (bits == 8) {
    if (w_is_bf16) {
      k_quant_blocks8<uint16_t><<<grid_for(groups8), kThreads, 0, stream>>>(
          static_cast<const uint16_t*>(w), n, code, packed, am32);
    } else {
      k_quant_blocks8<float><<<grid_for(groups8), kThreads, 0, stream>>>(
          static_cast<const float*>(w), n, code, packed, am32);
    }
  } else if (w_is_bf16) {
    k_quant_blocks<uint16_t><<<grid_for(groups8), kThreads, 0, stream>>>(
        static_cast<const uint16_t*>(w), n, code, packed, am32);
  } else {
    k_quant_blocks<float><<<grid_for(groups8), kThreads, 0, stream>>>(
        static_cast<const float*>(w), n, code, packed, am32);
  }
  if (!nested) return hipGetLastError();
  double* sums = reinterpret_cast<double*>(static_cast<char*>(ws) +
                                           align_up(static_cast<size_t>(nb) * 4, 256));
  k_chunk_sums<<<static_cast<unsigned>((ng + kSumWaves - 1) / kSumWaves), kThreads, 0, stream>>>(
      am32, nb, sums);
  k_offset<<<1, kThreads, 0, stream>>>(sums, ng, nb, nested_offset);
  k_nested<<<static_cast<unsigned>(ng), kThreads, 0, stream>>>(
      am32, nb, ncode, nested_offset, static_cast<uint8_t*>(absmax), nested_absmax);
  return hipGetLastError();
}

hipError_t launch_dequantize(const WArgs& w, int64_t n, bool out_bf16, void* out,
                             hipStream_t stream) {
  const unsigned grid = grid_for((n + 7) / 8);
  if (w.bits == 8) {
    if (w.nested()) {
      if (out_bf16) k_dequant8<true, true><<<grid, kThreads, 0, stream>>>(w, n, out);
      else k_dequant8<true, false><<<grid, kThreads, 0, stream>>>(w, n, out);
    } else {
      if (out_bf16) k_dequant8<false, true><<<grid, kThreads, 0, stream>>>(w, n, out);
      else k_dequant8<false, false><<<grid, kThreads, 0, stream>>>(w, n, out);
    }
    return hipGetLastError();
  }
  if (out_bf16) {
    if (w.nested())
      k_dequant_bf16<true><<<grid, kThreads, 0, stream>>>(w, n, static_cast<uint16_t*>(out));
    else
      k_dequant_bf16<false><<<grid, kThreads, 0, stream>>>(w, n, static_cast<uint16_t*>(out));
  } else {
    if (w.nested())
      k_dequant_f32<true><<<grid, kThreads, 0, stream>>>(w, n, static_cast<float*>(out));
    else
      k_dequant_f32<false><<<grid, kThreads, 0, stream>>>(w, n, static_cast<float*>(out));
  }
  return hipGetLastError();
}

}  // namespace nf4
