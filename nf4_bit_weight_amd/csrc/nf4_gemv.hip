// Small-M forward y = x . W_hat^T (M <= 32): weight-streaming kernel.
//
// At decode sizes the product is bound by HBM: every packed byte of W is used
// by at most 32 rows of x (Soup issue #842, "Nuance", on the small-batch regime
// where a fused 4-bit GEMV is the fast path).  The kernel therefore streams W
// once, with each lane expanding whole 64-blocks, and keeps x on chip.
//
//   * A wave owns MP rows of W (MP = 16 for M <= 16, 32 otherwise) and one
//     contraction chunk.  The MFMA is v_mfma_f32_16x16x32_bf16 (MP = 16) or
//     v_mfma_f32_32x32x16_bf16 (MP = 32); its A operand is x (rows >= M are
//     zero), its B operand the expanded weights.
//   * The contraction is permuted inside each step so that a lane's k-group
//     is one whole NF4 block: lane (n = l % MP, g = l / MP) of MFMA t reads
//     k = 64 * (G * s + g) + 8 t .. + 7 of step s (G = 64 / MP groups).  A
//     lane thus loads its block's 32 packed bytes with two 16-byte loads (the
//     G lanes of one row read G consecutive blocks: whole 128-byte lines),
//     builds one 16-entry byte table per block and expands one dword per MFMA.
//   * Within each 8-element group the expansion emits the order
//     (0, 2, 4, 6, 1, 3, 5, 7), which saves the final interleave; x is staged
//     into LDS in the same order, so every product pairs the right elements.
//   * Packed loads run PD steps ahead in registers.  The contraction is split
//     into chunks so that enough workgroups exist; chunk partials (fp32) are
//     added by the fixed-order split-K reduction, as in the tiled kernel.
#include <type_traits>

#include "nf4_device.hpp"
#include "nf4_internal.hpp"

namespace nf4 {
namespace {

constexpr int kGemvThreads = 256;   // 4 waves
constexpr int kPD = 4;              // packed-weight prefetch distance (steps)

struct GemvParams {
  const uint16_t* x;     // [M, K] bf16
  uint16_t* y;           // [M, N] bf16 (splits == 1)
  float* partial;        // [splits, M, N] fp32 (splits > 1)
  WArgs w;
  int32_t M;
  int32_t splits;
  int32_t kc;            // contraction per chunk (multiple of the step)
};

template <int MP>
struct Gv {
  static constexpr int G = 64 / MP;               // blocks per step
  static constexpr int kStepK = 64 * G;           // 256 or 128
  static constexpr int kRowsWG = 4 * MP;          // W rows per workgroup
  static constexpr int kMaxKC = MP == 16 ? 2048 : 1024;
  static constexpr int kAccRegs = MP == 16 ? 4 : 16;
};

template <int MP>
using acc_t = typename std::conditional<MP == 16, f32x4_t, f32x16_t>::type;

// Expand 8 nibbles in the order (0, 2, 4, 6, 1, 3, 5, 7): out[0] = (w0, w2),
// out[1] = (w4, w6), out[2] = (w1, w3), out[3] = (w5, w7).
__device__ __forceinline__ void expand8_eo(uint32_t p, const Lut& t, uint32_t (&out)[4]) {
  const uint32_t se = (p >> 4) & 0x07070707u;
  const uint32_t so = p & 0x07070707u;
  const uint32_t me = perm(p, p << 8, 0x0B090A08u);
  const uint32_t p4 = p << 4;
  const uint32_t mo = perm(p4, p4 << 8, 0x0B090A08u);
  const uint32_t he = bitsel(me, perm(t.h[3], t.h[2], se), perm(t.h[1], t.h[0], se));
  const uint32_t le = bitsel(me, perm(t.l[3], t.l[2], se), perm(t.l[1], t.l[0], se));
  const uint32_t ho = bitsel(mo, perm(t.h[3], t.h[2], so), perm(t.h[1], t.h[0], so));
  const uint32_t lo = bitsel(mo, perm(t.l[3], t.l[2], so), perm(t.l[1], t.l[0], so));
  out[0] = perm(he, le, 0x05010400u);
  out[1] = perm(he, le, 0x07030602u);
  out[2] = perm(ho, lo, 0x05010400u);
  out[3] = perm(ho, lo, 0x07030602u);
}

template <int MP, bool NESTED>
__global__ __launch_bounds__(kGemvThreads) void k_gemv(GemvParams p) {
  using S = Gv<MP>;
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];   // [MP][kc + 8]
  __shared__ float sncode[256];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int64_t N = p.w.N, K = p.w.K;
  const int M = p.M;
  const int z = blockIdx.y;
  const int64_t k0 = static_cast<int64_t>(z) * p.kc;
  const int64_t k1 = (k0 + p.kc < K) ? k0 + p.kc : K;
  const int kc = p.kc;
  const int pitch = kc + 8;                      // elements; rows land on distinct banks

  if constexpr (NESTED) sncode[tid] = p.w.ncode[tid];

  // ---- stage x[:, k0:k0+kc] into LDS, each 8-group as (0,2,4,6,1,3,5,7) ----
  // rows >= M and columns >= K are zero
  for (int c = tid; c < MP * (kc / 8); c += kGemvThreads) {
    const int m = c / (kc / 8), c8 = c % (kc / 8);
    const int64_t k = k0 + 8 * c8;
    u32x4_t d = {0u, 0u, 0u, 0u};
    if (m < M && k < K) d = *reinterpret_cast<const u32x4_t*>(p.x + static_cast<int64_t>(m) * K + k);
    const u32x4_t o = {perm(d[1], d[0], 0x05040100u), perm(d[3], d[2], 0x05040100u),
                       perm(d[1], d[0], 0x07060302u), perm(d[3], d[2], 0x07060302u)};
    *reinterpret_cast<u32x4_t*>(xs + m * pitch + 8 * c8) = o;
  }
  __syncthreads();

  float code[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) code[i] = p.w.code[i];
  const float off = NESTED ? p.w.nested_offset[0] : 0.f;

  // ---- this lane's row and block group -----------------------------------------
  const int r = lane % MP, g = lane / MP;
  const int64_t n = static_cast<int64_t>(blockIdx.x) * S::kRowsWG + wave * MP + r;
  const bool row_ok = n < N;
  const int64_t row_base = (row_ok ? n : 0) * K;             // element offset of the row
  const int nsteps = static_cast<int>((k1 - k0 + S::kStepK - 1) / S::kStepK);

  struct Raw {
    u32x4_t pk0, pk1;
    uint32_t sc;      // u8 nested index or fp32 bits of the plain absmax
    float s2;
    bool valid;
  };
  auto load = [&](int s, Raw& q) {
    const int sc_ = s < nsteps ? s : nsteps - 1;
    const int64_t koff = k0 + 64 * (S::G * sc_ + g);
    q.valid = row_ok & (koff < k1);
    const uint64_t flat = q.valid ? static_cast<uint64_t>(row_base + koff) : 0;   // multiple of 64
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(p.w.packed + (flat >> 1));
    q.pk0 = src[0];
    q.pk1 = src[1];
    const uint64_t b = flat >> 6;
    if constexpr (NESTED) {
      q.sc = static_cast<const uint8_t*>(p.w.absmax)[b];
      q.s2 = p.w.nested_absmax[b >> 8];
    } else {
      q.sc = __float_as_uint(static_cast<const float*>(p.w.absmax)[b]);
      q.s2 = 0.f;
    }
  };

  acc_t<MP> acc;
#pragma unroll
  for (int i = 0; i < S::kAccRegs; ++i) acc[i] = 0.f;

  // A fragment of MFMA t in step s: x row r (as the MFMA row), k-group g
  const uint16_t* xrow = xs + r * pitch + 64 * g;
  auto step = [&](int s, const Raw& q) {
    float a;
    if constexpr (NESTED) a = __fadd_rn(__fmul_rn(sncode[q.sc], q.s2), off);
    else a = __uint_as_float(q.sc);
    const Lut lt = make_lut(code, q.valid ? a : 0.f);
    const uint16_t* xa = xrow + 64 * S::G * s;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      uint32_t o[4];
      expand8_eo(t < 4 ? q.pk0[t] : q.pk1[t - 4], lt, o);
      const bf16x8_t bfr = __builtin_bit_cast(bf16x8_t, u32x4_t{o[0], o[1], o[2], o[3]});
      const bf16x8_t afr = *reinterpret_cast<const bf16x8_t*>(xa + 8 * t);
      if constexpr (MP == 16) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr, acc, 0, 0, 0);
      } else {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr, bfr, acc, 0, 0, 0);
      }
    }
  };

  // The fences keep every prefetch where it is written: without them the
  // compiler sinks each load next to its use one iteration later.
  auto fence = [] { asm volatile("" ::: "memory"); };
  Raw q0, q1, q2, q3;
  load(0, q0);
  load(1, q1);
  load(2, q2);
  load(3, q3);
  fence();
  int s = 0;
  for (; s + kPD <= nsteps; s += kPD) {
    step(s, q0);
    fence();
    load(s + 4, q0);
    fence();
    step(s + 1, q1);
    fence();
    load(s + 5, q1);
    fence();
    step(s + 2, q2);
    fence();
    load(s + 6, q2);
    fence();
    step(s + 3, q3);
    fence();
    load(s + 7, q3);
    fence();
  }
  if (s < nsteps) step(s, q0);
  if (s + 1 < nsteps) step(s + 1, q1);
  if (s + 2 < nsteps) step(s + 2, q2);

  // ---- epilogue: lane holds output column n; rows as laid out by the MFMA ----
  if (!row_ok) return;
#pragma unroll
  for (int i = 0; i < S::kAccRegs; ++i) {
    const int m = MP == 16 ? 4 * (lane / 16) + i : 8 * (i / 4) + 4 * (lane / 32) + (i % 4);
    if (m >= M) continue;
    if (p.splits == 1) {
      p.y[static_cast<int64_t>(m) * N + n] = to_bf16(acc[i]);
    } else {
      p.partial[(static_cast<int64_t>(z) * M + m) * N + n] = acc[i];
    }
  }
}

template <int MP, bool NESTED>
hipError_t launch_gemv_t(const GemvParams& p, hipStream_t stream) {
  using S = Gv<MP>;
  auto kern = k_gemv<MP, NESTED>;
  const size_t lds = static_cast<size_t>(MP) * (S::kMaxKC + 8) * 2;
  static const bool attr_done = [&] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    (void)hipGetLastError();
    return true;
  }();
  (void)attr_done;
  const size_t need = static_cast<size_t>(MP) * (p.kc + 8) * 2;
  const dim3 grid(static_cast<unsigned>((p.w.N + S::kRowsWG - 1) / S::kRowsWG),
                  static_cast<unsigned>(p.splits));
  kern<<<grid, kGemvThreads, need, stream>>>(p);
  return hipGetLastError();
}

}  // namespace

void plan_small_m(GemmPlan& pl, int64_t M, int64_t N, int64_t K, int cus) {
  pl.small_m = true;
  pl.bm = M <= 16 ? 16 : 32;                  // MFMA rows
  pl.bn = 0;
  pl.consumers = 0;
  const int step = pl.bm == 16 ? 256 : 128;
  const int max_kc = pl.bm == 16 ? 2048 : 1024;
  const int64_t row_wgs = (N + 4 * pl.bm - 1) / (4 * pl.bm);
  // aim for two workgroups per compute unit, each chunk a whole number of steps
  int64_t want = (2 * static_cast<int64_t>(cus) + row_wgs - 1) / row_wgs;
  const int64_t max_split = (K + step - 1) / step;
  if (want < 1) want = 1;
  if (want > max_split) want = max_split;
  int64_t kc = (K + want - 1) / want;
  kc = (kc + step - 1) / step * step;
  if (kc > max_kc) kc = max_kc;
  pl.kc = static_cast<int>(kc);
  pl.splits = static_cast<int>((K + kc - 1) / kc);
  pl.ws_bytes = pl.splits > 1
                    ? static_cast<size_t>(pl.splits) * static_cast<size_t>(M) * static_cast<size_t>(N) * 4
                    : 0;
}

hipError_t launch_gemv(const GemmPlan& plan, const void* x, int64_t M, const WArgs& w, void* y,
                       void* ws, hipStream_t stream) {
  GemvParams p{};
  p.x = static_cast<const uint16_t*>(x);
  p.y = static_cast<uint16_t*>(y);
  p.partial = static_cast<float*>(ws);
  p.w = w;
  p.M = static_cast<int32_t>(M);
  p.splits = plan.splits;
  p.kc = plan.kc;
  const bool nested = w.nested();
  if (plan.bm == 16) {
    return nested ? launch_gemv_t<16, true>(p, stream) : launch_gemv_t<16, false>(p, stream);
  }
  return nested ? launch_gemv_t<32, true>(p, stream) : launch_gemv_t<32, false>(p, stream);
}

}  // namespace nf4
