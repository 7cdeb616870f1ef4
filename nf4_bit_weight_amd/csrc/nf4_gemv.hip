// Small-M forward y = x . W_hat^T (M <= 32): weight-streaming kernels.
//
// At decode sizes the product is bound by HBM and by the expansion: every
// packed byte of W is used by at most 32 rows of x (Soup issue #842, "Nuance",
// on the small-batch regime where a fused 4-bit GEMV is the fast path).  The
// kernels therefore stream W once, with each lane expanding whole 64-blocks,
// and keep x on chip.  Two kernels share that plan:
//
//   * k_gemv_ln (below; up to M = 24, and small products to M = 32): 16-row
//     W groups, whole 128-byte lines copied global -> LDS per wave.
//   * k_gemv (large products above M = 24): 32-row W groups, each lane loads
//     its own block with two 16-byte loads.
//
// Common to both:
//   * A workgroup owns RW row groups of W and one contraction chunk.  Its
//     RW * KW waves are arranged as RW row groups times KW contraction
//     slices: the KW waves of a row group split the chunk's steps between
//     them, and their fp32 results are added through LDS in the fixed order
//     0 .. KW-1.  Splitting the contraction inside the workgroup gives enough
//     waves to cover HBM latency without partial sums in HBM; chunks across
//     workgroups (summed by the fixed-order split reduction) are only used
//     when the x chunk would not fit in LDS.
//   * The MFMA's A operand is x (rows >= M read a zero row), its B operand
//     the expanded weights.
//   * The contraction is permuted inside each step so that a lane's k-group
//     is one whole NF4 block: lane (n = l % R, g = l / R) of MFMA t reads
//     k = 64 * (G * s + g) + 8 t .. + 7 of step s (R rows per group, G = 64 / R
//     blocks per step).  A lane builds one 16-entry byte table per block and
//     expands one dword of its block's 32 packed bytes per MFMA.
//   * Within each 8-element group the expansion emits the order
//     (0, 2, 4, 6, 1, 3, 5, 7), which saves the final interleave; x is staged
//     into LDS in the same order, so every product pairs the right elements.
#include <stdlib.h>

#include <type_traits>

#include "nf4_device.hpp"
#include "nf4_internal.hpp"

namespace nf4 {
namespace {

constexpr int kPD = 4;                    // packed-weight prefetch distance (steps)
constexpr int kXBudgetBytes = 64 * 1024;  // LDS for a staged x chunk (M + 1 rows) ...
constexpr int kXWholeBytes = 96 * 1024;   // ... or for the whole of x in one chunk
constexpr int kMaxWaves = 16;

struct GemvParams {
  const uint16_t* x;     // [M, K] bf16
  uint16_t* y;           // [M, N] bf16 (splits == 1)
  float* partial;        // [splits, M, N] fp32 (splits > 1)
  WArgs w;
  int32_t M;
  int32_t splits;
  int32_t kc;            // contraction per chunk (multiple of the step)
  int32_t tb_off;        // line-staged kernel: byte offset of the per-wave staging slots in dynamic LDS
};

typedef __attribute__((address_space(3))) void lds_void_t;
template <int N>
using ic = std::integral_constant<int, N>;

// 32-row groups: one step is 128 columns (two 64-blocks per row), MFMA
// v_mfma_f32_32x32x16_bf16, 16 accumulator registers per lane.  Packed loads
// run kPD steps ahead in registers, the first kPD in flight while x is
// staged; block scales are loaded a batch of kPD steps ahead of that batch's
// packed bytes and decoded at the batch start.
template <int RW, int KW, bool NESTED>
__global__ __launch_bounds__(64 * RW * KW) void k_gemv(GemvParams p) {
  constexpr int MP = 32, kStepK = 128, kAccRegs = 16;
  constexpr int kThr = 64 * RW * KW;
  // [M + 1][kc + 8] bf16 (row M is zero), reused for the cross-wave sums
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
  __shared__ float sncode[256];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int rw = wave % RW, kw = wave / RW;
  const int64_t N = p.w.N, K = p.w.K;
  const int M = p.M;
  const int z = blockIdx.y;
  const int64_t k0 = static_cast<int64_t>(z) * p.kc;
  const int64_t k1 = (k0 + p.kc < K) ? k0 + p.kc : K;
  const int kc = p.kc;
  const int pitch = kc + 8;                      // elements; rows land on distinct banks

  // ---- this wave's steps of the chunk: a contiguous run ------------------------
  const int nsteps = static_cast<int>((k1 - k0 + kStepK - 1) / kStepK);
  const int per = (nsteps + KW - 1) / KW;
  const int s_begin = kw * per < nsteps ? kw * per : nsteps;
  const int s_end = s_begin + per < nsteps ? s_begin + per : nsteps;
  const int nw = s_end - s_begin;

  // ---- this lane's row and block group -----------------------------------------
  const int r = lane % MP, g = lane / MP;
  const int64_t n = (static_cast<int64_t>(blockIdx.x) * RW + rw) * MP + r;
  const bool row_ok = n < N;
  const int64_t row_base = (row_ok ? n : 0) * K;             // element offset of the row

  struct Raw {
    u32x4_t pk0, pk1;
  };
  // The block scales of a batch of kPD steps are loaded one batch ahead and
  // before that batch's packed bytes, and decoded at the batch's start: a
  // wait for them then leaves the packed prefetch in flight.  (Carried per
  // step instead, the compiler narrows the loop-carried absmax byte and
  // widens it at the loop top, which waits for the newest loads.)
  struct Scales {
    uint32_t sc[kPD];  // u8 nested index or fp32 bits of the plain absmax
    float s2[kPD];
  };
  // local step ls of this wave, clamped: past the end it reloads the last
  // step (an address already read), so every load stays inside the tensor
  auto clamp_step = [&](int ls) { return s_begin + (ls < nw ? ls : (nw > 0 ? nw - 1 : 0)); };
  auto step_valid = [&](int ls) {
    const int64_t koff = k0 + static_cast<int64_t>(kStepK) * clamp_step(ls) + 64 * g;
    return row_ok & (koff < k1) & (nw > 0);
  };
  auto load_scales = [&](int ls0, Scales& sq) {
#pragma unroll
    for (int j = 0; j < kPD; ++j) {
      const int64_t koff = k0 + static_cast<int64_t>(kStepK) * clamp_step(ls0 + j) + 64 * g;
      const bool v = row_ok & (koff < k1) & (nw > 0);
      const uint64_t bb = v ? static_cast<uint64_t>(row_base + koff) >> 6 : 0;
      if constexpr (NESTED) {
        sq.sc[j] = static_cast<const uint8_t*>(p.w.absmax)[bb];
        sq.s2[j] = p.w.nested_absmax[bb >> 8];
      } else {
        sq.sc[j] = __float_as_uint(static_cast<const float*>(p.w.absmax)[bb]);
        sq.s2[j] = 0.f;
      }
    }
  };
  // the lane's block of step ls (blocks past the end, or rows past N, read
  // the tensor's first bytes; their consumers see a zero scale)
  auto load = [&](int ls, Raw& q) {
    const int64_t koff = k0 + static_cast<int64_t>(kStepK) * clamp_step(ls) + 64 * g;
    const bool v = row_ok & (koff < k1) & (nw > 0);
    const uint64_t flat = v ? static_cast<uint64_t>(row_base + koff) : 0;   // multiple of 64
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(p.w.packed + (flat >> 1));
    q.pk0 = src[0];
    q.pk1 = src[1];
  };

  // The fences keep every prefetch where it is written: without them the
  // compiler sinks each load next to its use one iteration later; the
  // scheduling barrier keeps any arithmetic on a prefetched register from
  // moving ahead of its own step (a hoisted use waits for that load).
  auto fence = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- prologue: every load that the first step needs is issued before the
  // first wait, in the order it is consumed (loads complete in order) --------
  float code[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) code[i] = p.w.code[i];
  const float off = NESTED ? p.w.nested_offset[0] : 0.f;
  // the 256-entry nested table: kNC entries per thread
  constexpr int kNC = (256 + kThr - 1) / kThr;
  float nc_reg[kNC];
  if constexpr (NESTED) {
#pragma unroll
    for (int j = 0; j < kNC; ++j) {
      const int i = tid + j * kThr;
      nc_reg[j] = i < 256 ? p.w.ncode[i] : 0.f;
    }
  }
  // x[:, k0:k0+kc] is staged in batches of kXB 16-byte chunks per thread; each
  // 8-group is stored as (0,2,4,6,1,3,5,7); row M and columns >= K are zero
  constexpr int kXB = RW == 1 ? 4 : 8;       // more rows per workgroup: larger batches
  const int c8n = kc / 8;
  const int nchunks = (M + 1) * c8n;
  u32x4_t xd[kXB];
  int xm[kXB], x8[kXB];
  // chunk c -> (row c / c8n, column group c % c8n) without an integer divide:
  // a float reciprocal, then one correction each way (c < 2^24)
  const float inv_c8n = 1.0f / static_cast<float>(c8n);
  auto xload = [&](int base) {
#pragma unroll
    for (int j = 0; j < kXB; ++j) {
      const int c = base + tid + j * kThr;
      int m = static_cast<int>(static_cast<float>(c) * inv_c8n);
      m -= (m * c8n > c) ? 1 : 0;
      m += ((m + 1) * c8n <= c) ? 1 : 0;
      xm[j] = c < nchunks ? m : M + 1;               // M + 1: no chunk
      x8[j] = c - m * c8n;
      xd[j] = u32x4_t{0u, 0u, 0u, 0u};
      const int64_t k = k0 + 8 * x8[j];
      if (xm[j] < M && k < K)
        xd[j] = *reinterpret_cast<const u32x4_t*>(p.x + static_cast<int64_t>(xm[j]) * K + k);
    }
  };
  auto xstore = [&](int base) {
    (void)base;
#pragma unroll
    for (int j = 0; j < kXB; ++j) {
      if (xm[j] <= M) {
        const u32x4_t d = xd[j];
        const u32x4_t o = {perm(d[1], d[0], 0x05040100u), perm(d[3], d[2], 0x05040100u),
                           perm(d[1], d[0], 0x07060302u), perm(d[3], d[2], 0x07060302u)};
        *reinterpret_cast<u32x4_t*>(xs + xm[j] * pitch + 8 * x8[j]) = o;
      }
    }
  };
  xload(0);
  fence();
  Scales sc_cur, sc_next;
  load_scales(0, sc_cur);
  Raw q0, q1, q2, q3;
  load(0, q0);
  load(1, q1);
  load(2, q2);
  load(3, q3);
  fence();
  if constexpr (NESTED) {
#pragma unroll
    for (int j = 0; j < kNC; ++j) {
      const int i = tid + j * kThr;
      if (i < 256) sncode[i] = nc_reg[j];
    }
  }
  xstore(0);
  for (int base = kXB * kThr; base < nchunks; base += kXB * kThr) {
    xload(base);
    xstore(base);
  }
  __syncthreads();

  f32x16_t acc;
#pragma unroll
  for (int i = 0; i < kAccRegs; ++i) acc[i] = 0.f;

  // A fragments of MFMA t: x row r (rows >= M read the zero row M)
  const uint16_t* const xrow = xs + (r < M ? r : M) * pitch + 64 * g;
  // decoded scale of each step of the current batch (zero for blocks past the ends)
  float a_dec[kPD];
  auto decode = [&](int ls0, const Scales& sq) {
#pragma unroll
    for (int j = 0; j < kPD; ++j) {
      float a;
      if constexpr (NESTED) a = __fadd_rn(__fmul_rn(sncode[sq.sc[j]], sq.s2[j]), off);
      else a = __uint_as_float(sq.sc[j]);
      a_dec[j] = step_valid(ls0 + j) ? a : 0.f;
    }
  };
  auto step = [&](int ls, int j, const Raw& q) {
    // all eight A fragments first, so their LDS latency overlaps the table build
    const int xo = kStepK * (s_begin + ls);
    bf16x8_t afr[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) afr[t] = *reinterpret_cast<const bf16x8_t*>(xrow + xo + 8 * t);
    // the packed registers are redefined at the step's start, so no
    // arithmetic on them is scheduled (and waited for) earlier
    u32x4_t d0 = q.pk0, d1 = q.pk1;
    asm volatile("" : "+v"(d0), "+v"(d1));
    const Lut lt = make_lut(code, a_dec[j]);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      uint32_t o[4];
      expand8_eo(t < 4 ? d0[t] : d1[t - 4], lt, o);
      const bf16x8_t bfr = __builtin_bit_cast(bf16x8_t, u32x4_t{o[0], o[1], o[2], o[3]});
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr[t], bfr, acc, 0, 0, 0);
    }
  };

  int s = 0;
  for (; s + kPD <= nw; s += kPD) {
    decode(s, sc_cur);
    fence();
    load_scales(s + kPD, sc_next);
    fence();
    step(s, 0, q0);
    fence();
    load(s + 4, q0);
    fence();
    step(s + 1, 1, q1);
    fence();
    load(s + 5, q1);
    fence();
    step(s + 2, 2, q2);
    fence();
    load(s + 6, q2);
    fence();
    step(s + 3, 3, q3);
    fence();
    load(s + 7, q3);
    fence();
    sc_cur = sc_next;
  }
  if (s < nw) {
    decode(s, sc_cur);
    step(s, 0, q0);
    if (s + 1 < nw) step(s + 1, 1, q1);
    if (s + 2 < nw) step(s + 2, 2, q2);
  }

  // ---- fixed-order sum over the KW contraction slices of each row group ------
  if constexpr (KW > 1) {
    __syncthreads();                                   // x is no longer read
    float* red = reinterpret_cast<float*>(xs);         // [KW-1][RW][regs][64]
    if (kw > 0) {
#pragma unroll
      for (int i = 0; i < kAccRegs; ++i) red[(((kw - 1) * RW + rw) * kAccRegs + i) * 64 + lane] = acc[i];
    }
    __syncthreads();
    if (kw > 0) return;
    for (int v = 1; v < KW; ++v) {
#pragma unroll
      for (int i = 0; i < kAccRegs; ++i)
        acc[i] = __fadd_rn(acc[i], red[(((v - 1) * RW + rw) * kAccRegs + i) * 64 + lane]);
    }
  }

  // ---- epilogue: lane holds output column n; rows as laid out by the MFMA ----
  if (!row_ok) return;
#pragma unroll
  for (int i = 0; i < kAccRegs; ++i) {
    const int m = 8 * (i / 4) + 4 * (lane / 32) + (i % 4);
    if (m >= M) continue;
    if (p.splits == 1) {
      p.y[static_cast<int64_t>(m) * N + n] = to_bf16(acc[i]);
    } else {
      p.partial[(static_cast<int64_t>(z) * M + m) * N + n] = acc[i];
    }
  }
}

// ===========================================================================
// Line-staged streaming kernel: 16-row W groups, x as one (M <= 16) or two
// (M <= 32) 16-row halves.
//
// A wave owns one 16-row group of W and a contiguous run of 256-column steps
// of the contraction chunk; lane (r = l % 16, g = l / 16) expands block g of
// W row r in every step (one byte table, eight 8-nibble expansions) into the
// B operand of eight v_mfma_f32_16x16x32_bf16 whose A operand is x.
//
// The packed bytes of a step (16 rows x 128 B) are copied global -> LDS by
// two buffer_load_dwordx4 ... lds instructions, each covering 8 whole 128-byte
// lines, into one of kSD private staging slots of the wave.  The 16-byte
// pieces of row rr are stored at piece ^ ((rr >> 1) & 7), so the two 16-byte
// reads of a lane's block hit distinct banks across each 16-lane group.  The
// step's block scales (one per lane) arrive the same way, a byte or a dword
// per lane.  Every load of the loop is such a copy, issued kSD steps ahead;
// one explicit vmcnt per step is the only wait on memory, and a slot is only
// refilled by the wave that reads it, so the loop has no barrier.  No two
// copies in flight read the same bytes: a repeated copy of the same address
// let a counted wait pass before the older copy had landed (below).  So the
// nested scales, which consecutive steps share (one per 256 blocks), are not
// copied per step: a chunk holds at most 64 steps, so a lane's blocks span
// fewer than 256 and meet at most two nested groups, whose two scales the
// lane loads into registers once, before its first copy.  Two slots
// per wave keep a workgroup's LDS small (three or four were measured
// slower, see kSD).  The buffer resources carry the tensor bounds (reads past the end
// return zero) and move with the step in scalar registers: the loop computes
// no vector addresses.
// Staging slots per wave = copy distance in steps (2 to 4 supported).
// Measured on the Llama-3.1-8B decode passes: three slots made the forward
// of gate 15.0 us instead of 13.2-14.1 at M = 1 and 21.4 instead of 17.3 at
// M = 8, four slots 17.0 and 22.4 (the larger workgroups fit fewer per CU).
constexpr int kSD = 2;
constexpr int kSlotBytes = 2048 + 256;          // packed lines, block scales
constexpr int kLnMaxChunkSteps = 64;            // chunk length bound the nested-scale pair relies on
constexpr int kLnMaxWaves = 8;
constexpr int kRsrcWord3 = 0x00020000;          // raw buffer, 32-bit data format (gfx9 family)

// `bytes` > 0 (every copy starts inside its tensor); sizes from 2 GiB up are
// clamped (the offsets a wave uses stay far below).  The test is on the high
// bits so that it stays a scalar instruction.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  const uint64_t b = static_cast<uint64_t>(bytes);
  const uint32_t hi = static_cast<uint32_t>(b >> 32), lo = static_cast<uint32_t>(b);
  const int32_t n = (hi | (lo >> 31)) != 0 ? 0x7FFFFFFF : static_cast<int32_t>(lo);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), n,
                                           kRsrcWord3);
}

// s_waitcnt vmcnt(V), lgkmcnt and expcnt left open (gfx9 field layout)
template <int V>
__device__ __forceinline__ void vm_wait_open() {
  static_assert(V >= 0 && V < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((V & 15) | ((V >> 4) << 14) | (15 << 8) | (7 << 4));
}

template <int RW, int KW, bool NESTED, int MH>
__global__ __launch_bounds__(64 * RW * KW) void k_gemv_ln(GemvParams p) {
  constexpr int kThr = 64 * RW * KW;
  constexpr int C = 3;                          // copy instructions per step
  // [M + 1][kc + 8] bf16 (row M is zero), reused for the cross-wave sums;
  // the waves' staging slots follow at byte p.tb_off
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
  __shared__ float sncode[256];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int rw = wave % RW, kw = wave / RW;
  const int64_t N = p.w.N, K = p.w.K;
  const int M = p.M;
  const int z = blockIdx.y;
  const int64_t k0 = static_cast<int64_t>(z) * p.kc;
  const int64_t k1 = (k0 + p.kc < K) ? k0 + p.kc : K;
  const int kc = p.kc;
  const int pitch = kc + 8;

  const int r = lane & 15, g = lane >> 4;
  const int64_t rg0 = (static_cast<int64_t>(blockIdx.x) * RW + rw) * 16;   // first W row of the group

  // this wave's steps of the chunk: a contiguous run (none for a row group
  // past N, which the last workgroup of a launch with RW > 1 may hold: it
  // copies and computes nothing, and stores nothing)
  const int nsteps = static_cast<int>((k1 - k0 + 255) / 256);
  const int per = (nsteps + KW - 1) / KW;
  const int s_begin = kw * per < nsteps ? kw * per : nsteps;
  const int s_end = s_begin + per < nsteps ? s_begin + per : nsteps;
  const int nw = rg0 < N ? s_end - s_begin : 0;
  const int64_t kb = K >> 6;                       // blocks per W row
  const int64_t nb = N * kb;
  const int64_t ng = (nb + kNestedBlock - 1) / kNestedBlock;

  // ---- copy addressing (fixed per lane) --------------------------------------
  const int lr = lane >> 3;                        // row within the 8 rows of one copy
  auto piece = [](int row, int phys) { return phys ^ ((row >> 1) & 7); };
  const uint32_t voff_w0 = static_cast<uint32_t>(lr * (K >> 1)) + 16u * piece(lr, lane & 7);
  const uint32_t voff_w1 = static_cast<uint32_t>((8 + lr) * (K >> 1)) + 16u * piece(8 + lr, lane & 7);
  const uint32_t lane_b = static_cast<uint32_t>(r * kb + g);      // block of the lane within the step
  uint8_t* const slots = reinterpret_cast<uint8_t*>(xs) + p.tb_off + wave * (kSD * kSlotBytes);

  // Every copy lies inside the wave's own rows and steps: the host launches
  // this kernel only when K is a multiple of 256 and N of 16, so a step never
  // runs past the end of a row into the next one (which another wave of the
  // workgroup copies: two copies of the same bytes in flight must not
  // happen, see above) and a row group is either whole or, past N, idle.
  auto issue = [&](int ls, int slot) {
    const int st = s_begin + ls;                             // 0 <= st < nsteps
    const int64_t kstep = k0 + 256 * static_cast<int64_t>(st);
    uint8_t* const sl = slots + slot * kSlotBytes;
    const int64_t wb = (rg0 * K + kstep) >> 1;               // first byte of the step's lines
    const auto rw_ = rsrc(p.w.packed + wb, ((N * K) >> 1) - wb);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rw_, (lds_void_t*)sl, 16, voff_w0, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rw_, (lds_void_t*)(sl + 1024), 16, voff_w1, 0, 0, 0);
    const int64_t bb = rg0 * kb + (kstep >> 6);              // block of lane 0
    if constexpr (NESTED) {
      const auto ra = rsrc(static_cast<const uint8_t*>(p.w.absmax) + bb, nb - bb);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(sl + 2048), 1, lane_b, 0, 0, 0);
    } else {
      const auto ra = rsrc(static_cast<const float*>(p.w.absmax) + bb, 4 * (nb - bb));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(sl + 2048), 4, 4u * lane_b, 0, 0, 0);
    }
  };
  // Wait until at most the copies of `later` steps (C instructions each) are
  // in flight: vmcnt(C * later) with lgkmcnt and expcnt left open.
  static_assert(kSD >= 2 && kSD <= 4, "wait counts and step loop below");
  auto wait_later = [&](int later) {
    switch (later) {
      case 0: vm_wait_open<0>(); break;
      case 1: vm_wait_open<C>(); break;
      case 2: vm_wait_open<2 * C>(); break;
      case 3: vm_wait_open<3 * C>(); break;
      default: vm_wait_open<4 * C>(); break;
    }
  };
  // Before step ls: the copies of step ls have landed once at most those of
  // the later steps already issued (ls + 1 .. ls + kSD - 1, within the run)
  // are in flight.
  auto wait_copies = [&](int ls) {
    const int later = nw - 1 - ls < kSD - 1 ? nw - 1 - ls : kSD - 1;
    wait_later(later);
  };
  auto fence = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- prologue ---------------------------------------------------------------
  float code[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) code[i] = p.w.code[i];
  const float off = NESTED ? p.w.nested_offset[0] : 0.f;
  // x[:, k0 : k0 + kc) in batches of kXB 16-byte chunks per thread, each
  // 8-group stored as (0,2,4,6,1,3,5,7); row M and columns >= K are zero.
  // Chunk c -> (row c / c8n, group c % c8n) by a float reciprocal with one
  // correction each way (c < 2^24).  The first batch of x is loaded, then the
  // copies of the first two steps are issued, then that batch is stored: the
  // latencies of x and of the first weights overlap, and the wait for x
  // (the older loads) leaves the copies in flight.
  constexpr int kXB = 4;
  const int c8n = kc / 8;
  const int nchunks = (M + 1) * c8n;
  const float inv_c8n = 1.0f / static_cast<float>(c8n);
  u32x4_t xd[kXB];
  int xoff[kXB];
  auto x_load = [&](int base) {
#pragma unroll
    for (int j = 0; j < kXB; ++j) {
      const int c = base + tid + j * kThr;
      int m = static_cast<int>(static_cast<float>(c) * inv_c8n);
      m -= (m * c8n > c) ? 1 : 0;
      m += ((m + 1) * c8n <= c) ? 1 : 0;
      const int c8 = c - m * c8n;
      xoff[j] = c < nchunks ? m * pitch + 8 * c8 : -1;
      xd[j] = u32x4_t{0u, 0u, 0u, 0u};
      const int64_t k = k0 + 8 * c8;
      if (c < nchunks && m < M && k < K)
        xd[j] = *reinterpret_cast<const u32x4_t*>(p.x + static_cast<int64_t>(m) * K + k);
    }
  };
  auto x_store = [&] {
#pragma unroll
    for (int j = 0; j < kXB; ++j) {
      if (xoff[j] >= 0) {
        const u32x4_t d = xd[j];
        const u32x4_t o = {perm(d[1], d[0], 0x05040100u), perm(d[3], d[2], 0x05040100u),
                           perm(d[1], d[0], 0x07060302u), perm(d[3], d[2], 0x07060302u)};
        *reinterpret_cast<u32x4_t*>(xs + xoff[j]) = o;
      }
    }
  };
  // the nested table (256 entries over the workgroup's threads), and the
  // lane's nested scales: groups g0 (its block of its first step) and g0 + 1
  // (blocks of its later steps: 4 per step, at most 64 steps, so fewer than
  // 256 further on); indices clamped into the tensor (rows past N are never
  // stored, blocks past K meet zero x)
  constexpr int kNC = (256 + kThr - 1) / kThr;
  float nc_reg[kNC];
  const int64_t blk0 = (rg0 + r) * kb + (k0 >> 6) + 4 * static_cast<int64_t>(s_begin) + g;
  const int64_t g0 = blk0 >> 8;
  float s2a = 0.f, s2b = 0.f;
  x_load(0);
  if constexpr (NESTED) {
#pragma unroll
    for (int j = 0; j < kNC; ++j) nc_reg[j] = tid + j * kThr < 256 ? p.w.ncode[tid + j * kThr] : 0.f;
    s2a = p.w.nested_absmax[g0 < ng ? g0 : ng - 1];
    s2b = p.w.nested_absmax[g0 + 1 < ng ? g0 + 1 : ng - 1];
  }
  fence();
  // Only copies that will be read are issued.  (Measured: a wave of one step
  // that also issued a repeat copy of the same lines into its spare slot, to
  // keep the count behind every step uniform, read stale data in 2-22% of
  // runs after its counted wait; with exact counts and no repeated copy in
  // flight, 0 of 200.)
#pragma unroll
  for (int j = 0; j < kSD; ++j)
    if (j < nw) issue(j, j);
  fence();
  // the x and table loads have returned once at most this wave's copies are in flight
  wait_later(nw < kSD ? nw : kSD);
  if constexpr (NESTED) {
#pragma unroll
    for (int j = 0; j < kNC; ++j)
      if (tid + j * kThr < 256) sncode[tid + j * kThr] = nc_reg[j];
  }
  x_store();
  for (int base = kXB * kThr; base < nchunks; base += kXB * kThr) {
    x_load(base);
    x_store();
  }
  fence();
  // x and the table are visible to every wave once their LDS writes are done;
  // the weight copies go to each wave's own slots and are waited for per step
  __builtin_amdgcn_s_waitcnt((7 << 4) | 0xC00F);           // lgkmcnt(0), vmcnt and expcnt open
  __builtin_amdgcn_s_barrier();
  fence();

  f32x4_t acc[MH];
#pragma unroll
  for (int h = 0; h < MH; ++h)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[h][i] = 0.f;

  // A fragments: x row r (and r + 16), columns 64 g + 8 t of the step (rows >= M read the zero row)
  const uint16_t* xrow[MH];
#pragma unroll
  for (int h = 0; h < MH; ++h) xrow[h] = xs + (r + 16 * h < M ? r + 16 * h : M) * pitch + 64 * g;
  // LDS byte addresses of this lane's block pieces and scales in slot 0
  const uint32_t sl0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)slots));
  const uint32_t a_lo = sl0 + 16u * (8 * r + piece(r, 2 * g));
  const uint32_t a_hi = sl0 + 16u * (8 * r + piece(r, 2 * g + 1));
  const uint32_t a_sc = sl0 + 2048u + 4u * lane;

  struct Staged {
    u32x4_t lo, hi;
    uint32_t sc;
  };
#define NF4_LN_READ(OFF)                                                                   \
  asm volatile("ds_read_b128 %0, %3 offset:" #OFF "\n\t"                                   \
               "ds_read_b128 %1, %4 offset:" #OFF "\n\t"                                   \
               "ds_read_b32 %2, %5 offset:" #OFF "\n\t"                                    \
               "s_waitcnt lgkmcnt(0)"                                                      \
               : "=&v"(u.lo), "=&v"(u.hi), "=&v"(u.sc)                                     \
               : "v"(a_lo), "v"(a_hi), "v"(a_sc)                                           \
               : "memory")
  auto read_slot = [&](auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    static_assert(kSlotBytes == 2304 && kSD <= 4, "slot offsets below");
    Staged u;
    if constexpr (slot == 0) NF4_LN_READ(0);
    else if constexpr (slot == 1) NF4_LN_READ(2304);
    else if constexpr (slot == 2) NF4_LN_READ(4608);
    else NF4_LN_READ(6912);
    return u;
  };
#undef NF4_LN_READ

  auto compute = [&](int ls, auto slot_c) {
    const int xo = 256 * (s_begin + ls);
    bf16x8_t afr[MH][8];
#pragma unroll
    for (int h = 0; h < MH; ++h)
#pragma unroll
      for (int t = 0; t < 8; ++t) afr[h][t] = *reinterpret_cast<const bf16x8_t*>(xrow[h] + xo + 8 * t);
    const Staged u = read_slot(slot_c);
    float a;
    if constexpr (NESTED) {
      const float s2 = ((blk0 + 4 * ls) >> 8) == g0 ? s2a : s2b;
      a = __fadd_rn(__fmul_rn(sncode[u.sc & 0xFF], s2), off);
    } else {
      a = __uint_as_float(u.sc);
    }
    const Lut lt = make_lut(code, a);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      uint32_t o[4];
      expand8_eo(t < 4 ? u.lo[t] : u.hi[t - 4], lt, o);
      const bf16x8_t bfr = __builtin_bit_cast(bf16x8_t, u32x4_t{o[0], o[1], o[2], o[3]});
#pragma unroll
      for (int h = 0; h < MH; ++h)
        acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[h][t], bfr, acc[h], 0, 0, 0);
    }
  };
  // Step ls reads slot ls % kSD; then the copy of step ls + kSD, if there is
  // one, refills that slot.
  auto one = [&](int ls, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    wait_copies(ls);
    fence();
    compute(ls, slot_c);
    fence();
    if (ls + kSD < nw) issue(ls + kSD, slot);
    fence();
  };
  int s = 0;
  for (; s + kSD <= nw; s += kSD) {
    one(s, ic<0>{});
    one(s + 1, ic<1>{});
    if constexpr (kSD > 2) one(s + 2, ic<2>{});
    if constexpr (kSD > 3) one(s + 3, ic<3>{});
  }
  if (s < nw) one(s, ic<0>{});
  if constexpr (kSD > 2) {
    if (s + 1 < nw) one(s + 1, ic<1>{});
  }
  if constexpr (kSD > 3) {
    if (s + 2 < nw) one(s + 2, ic<2>{});
  }

  // ---- fixed-order sum over the KW contraction slices of each row group ------
  constexpr int kRegs = 4 * MH;
  if constexpr (KW > 1) {
    __syncthreads();                                   // x is no longer read
    float* red = reinterpret_cast<float*>(xs);         // [KW-1][RW][regs][64]
    if (kw > 0) {
#pragma unroll
      for (int h = 0; h < MH; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          red[(((kw - 1) * RW + rw) * kRegs + h * 4 + i) * 64 + lane] = acc[h][i];
    }
    __syncthreads();
    if (kw > 0) return;
    for (int v = 1; v < KW; ++v) {
#pragma unroll
      for (int h = 0; h < MH; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[h][i] = __fadd_rn(acc[h][i], red[(((v - 1) * RW + rw) * kRegs + h * 4 + i) * 64 + lane]);
    }
  }

  // ---- epilogue: lane holds output column n, rows 16 h + 4 (lane / 16) + i ---
  const int64_t n = rg0 + r;
  if (n >= N) return;
#pragma unroll
  for (int h = 0; h < MH; ++h) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 16 * h + 4 * g + i;
      if (m >= M) continue;
      if (p.splits == 1) {
        p.y[static_cast<int64_t>(m) * N + n] = to_bf16(acc[h][i]);
      } else {
        p.partial[(static_cast<int64_t>(z) * M + m) * N + n] = acc[h][i];
      }
    }
  }
}

// LDS of one launch: the x chunk (M + 1 rows) or the cross-wave sums, whichever is larger
size_t gemv_region_bytes(int mp, int rw, int kw, int64_t M, int kc) {
  const size_t xb = static_cast<size_t>(M + 1) * static_cast<size_t>(kc + 8) * 2;
  const int regs = mp == 32 ? 16 : (M > 16 ? 8 : 4);      // x halves at M > 16 (MP = 16)
  const size_t rb = static_cast<size_t>(kw - 1) * rw * regs * 64 * 4;
  return ((xb > rb ? xb : rb) + 15) / 16 * 16;
}
constexpr size_t kGemvLdsMax = kXWholeBytes + 4096;

template <int RW, int KW, bool NESTED>
hipError_t launch_gemv_t(const GemvParams& p, hipStream_t stream) {
  auto kern = k_gemv<RW, KW, NESTED>;
  static const bool attr_done = [&] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kGemvLdsMax);
    (void)hipGetLastError();
    return true;
  }();
  (void)attr_done;
  const size_t need = gemv_region_bytes(32, RW, KW, p.M, p.kc);
  const dim3 grid(static_cast<unsigned>((p.w.N + RW * 32 - 1) / (RW * 32)),
                  static_cast<unsigned>(p.splits));
  kern<<<grid, 64 * RW * KW, need, stream>>>(p);
  return hipGetLastError();
}

// the line-staged kernel: x region plus kSD staging slots per wave
size_t gemv_ln_lds_bytes(int rw, int kw, int64_t M, int kc) {
  return gemv_region_bytes(16, rw, kw, M, kc) + static_cast<size_t>(rw) * kw * kSD * kSlotBytes;
}
constexpr size_t kLnLdsMax = kXWholeBytes + 4096 + kLnMaxWaves * kSD * kSlotBytes;

template <int RW, int KW, bool NESTED, int MH>
hipError_t launch_ln_t(const GemvParams& p, hipStream_t stream) {
  auto kern = k_gemv_ln<RW, KW, NESTED, MH>;
  static const bool attr_done = [&] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kLnLdsMax);
    (void)hipGetLastError();
    return true;
  }();
  (void)attr_done;
  const size_t need = gemv_ln_lds_bytes(RW, KW, p.M, p.kc);
  const dim3 grid(static_cast<unsigned>((p.w.N + RW * 16 - 1) / (RW * 16)),
                  static_cast<unsigned>(p.splits));
  kern<<<grid, 64 * RW * KW, need, stream>>>(p);
  return hipGetLastError();
}

template <int RW, bool NESTED, int MH>
hipError_t launch_ln_kw(int kw, const GemvParams& p, hipStream_t stream) {
  switch (kw) {
    case 1: return launch_ln_t<RW, 1, NESTED, MH>(p, stream);
    case 2: return launch_ln_t<RW, 2, NESTED, MH>(p, stream);
    case 4: if constexpr (RW <= 2) return launch_ln_t<RW, 4, NESTED, MH>(p, stream); break;
    case 8: if constexpr (RW == 1) return launch_ln_t<RW, 8, NESTED, MH>(p, stream); break;
    default: break;
  }
  return hipErrorInvalidValue;
}

// 32-row groups: four per workgroup, 1, 2 or 4 contraction slices
template <bool NESTED>
hipError_t launch_kw32(int kw, const GemvParams& p, hipStream_t stream) {
  switch (kw) {
    case 1: return launch_gemv_t<4, 1, NESTED>(p, stream);
    case 2: return launch_gemv_t<4, 2, NESTED>(p, stream);
    case 4: return launch_gemv_t<4, 4, NESTED>(p, stream);
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace

// plan fields for the streaming forward: bm = MFMA rows (16 / 32), bn = row
// groups per workgroup (RW), consumers = contraction slices per row group (KW)
void plan_small_m(GemmPlan& pl, int64_t M, int64_t N, int64_t K, int cus) {
  pl.small_m = true;
  // MFMA rows: 16-row W groups up to M = 24 (two halves of x above 16), 32-row
  // groups from M = 25 (measured over the Llama-3.1-8B projections: per layer
  // 109 vs 130 us at M = 17, 119 vs 130 us at M = 24, but 143 vs 136 us at
  // M = 32, where the halves' smaller x chunks cost more partial traffic);
  // tuning override (documented): NF4_GEMV_MP32=0/1 picks either above M = 16
  // (above M = 16 the 32-row groups win on the large projections: at M = 24
  // the forward of gate 21.9 vs 31.4 us, at M = 32 q 14.6 vs 16.5 us, while
  // the 16-row kernel keeps k / v at 9.0 vs 12.9 us at M = 24)
  const char* o32 = getenv("NF4_GEMV_MP32");
  bool mp32 = M > 24 || (M > 16 && N * K >= (int64_t{32} << 20));
  if (o32 && (o32[0] == '0' || o32[0] == '1')) mp32 = o32[0] == '1';
  pl.bm = (M > 16 && mp32) ? 32 : 16;
  // The line-staged kernel (16-row groups) copies whole 256-column steps of
  // whole 16-row groups with LDS-direct loads under counted waits; it takes
  // only shapes where each such copy lies inside its own rows (K a multiple
  // of 256, N of 16: every Llama, Qwen and OLMoE projection).  Others run the
  // 32-row kernel, whose ordinary loads need no such care.  (Two wrong
  // results, once each in many runs, came from the ragged cases: a last
  // step that copied the head of the next row, which another wave copied,
  // and once, after that was fixed, at M = 7, N = 520, K = 1088 with no
  // cause found.)
  if (K % 256 != 0 || N % 16 != 0) pl.bm = 32;
  const int step = pl.bm == 16 ? 256 : 128;
  // largest chunk whose x (M + 1 rows, padded) fits the LDS budget
  // Chunks of x within 64 KB of LDS, or all of x in one chunk (no split of
  // the contraction, no partials) when it fits in 96 KB.  Measured over the
  // Llama-3.1-8B decode projections: the single chunk takes q / gate at M = 8
  // from 10.4 / 17.5 to 8.3 / 15.7 us and down at M = 2 from 16.0 to 14.0,
  // while chunks of up to 96 KB where x is larger made down at M = 4 24.3
  // instead of 18.3 us and q at M = 32 17.6 instead of 14.6.
  const int64_t k_all = (K + step - 1) / step * step;
  int64_t kx = (kXBudgetBytes / 2 / (M + 1) - 8) / step * step;
  if ((M + 1) * (k_all + 8) * 2 <= kXWholeBytes) kx = k_all;
  if (kx < step) kx = step;
  // the line-staged kernel's chunks hold at most kLnMaxChunkSteps steps
  if (pl.bm == 16 && kx > 256 * kLnMaxChunkSteps) kx = 256 * kLnMaxChunkSteps;
  int64_t z = (K + kx - 1) / kx;
  // tuning override (documented): NF4_GEMV_Z raises the chunk count
  const char* oz = getenv("NF4_GEMV_Z");
  if (oz && atoi(oz) > z) z = atoi(oz);
  if (z > (K + step - 1) / step) z = (K + step - 1) / step;
  int64_t kc = (K + z - 1) / z;
  kc = (kc + step - 1) / step * step;
  z = (K + kc - 1) / kc;
  const int64_t steps = kc / step;
  // Row groups per workgroup: each shares one staged x chunk.  32-row groups:
  // 4.  16-row groups (line-staged kernel): 4 above M = 4 when there are
  // still as many such workgroups as compute units (half as many above
  // M = 8), else 1; contraction
  // slices per row group: 2 with four row groups (8 waves), otherwise the
  // power of two (at most 8) that brings the launch to about 2048 waves.
  // Measured over the Llama-3.1-8B projections: at M = 8 four row groups take
  // the forward of gate / down from 18.2 / 24.1 to 16.9 / 16.5 us, while q and
  // k are best with one row group and 8 slices (9.9 / 7.4 us); at M = 1 the
  // slices give gate 13.1 (4 slices), q 7.1 and k 5.9 us (8 slices).
  int rw = 1;
  int kw = 1;
  const int64_t rg16 = (N + 15) / 16;
  if (pl.bm == 32) {
    rw = 4;
    // 32-row groups (streaming kernel with per-lane block loads): 2 slices,
    // doubled while a slice would hold more than 16 steps
    kw = 2;
    while (kw < 8 && steps > 16 * kw) kw *= 2;
  } else {
    // (at M = 16 the forward of q takes 11.2 us with four row groups, 15.3
    // with one; at M = 8 one row group and 8 slices are best for it, 9.9 us;
    // from M = 2 four row groups pay once their workgroups cover three
    // quarters of the compute units: gate at M = 2 / 4 13.9 / 14.6 us
    // against 16.4 / 19.5 with one, while down at M = 2, 128 such
    // workgroups, takes 23.0 against 16.3)
    const int64_t wgs4 = (rg16 + 3) / 4 * z;
    if (M > 1 && (4 * wgs4 >= 3 * static_cast<int64_t>(cus) || (M > 8 && 2 * wgs4 >= cus))) rw = 4;
    if (rw == 4) {
      kw = 2;
    } else {
      const int64_t wgs = rg16 * z;
      while (kw < 8 && wgs * kw < 2048) kw *= 2;
    }
  }
  // tuning override (documented): NF4_GEMV_RW (row groups per workgroup: 1 / 2 / 4 at M <= 16)
  const char* orw = getenv("NF4_GEMV_RW");
  if (orw && pl.bm == 16 && (atoi(orw) == 1 || atoi(orw) == 2 || atoi(orw) == 4)) rw = atoi(orw);
  pl.bn = rw;
  // the line-staged kernel holds two staging slots per wave: at most
  // kLnMaxWaves waves per workgroup; 32-row groups: 16
  const int kw_max = (pl.bm == 16 ? kLnMaxWaves : kMaxWaves) / rw;
  if (kw > kw_max) kw = kw_max;
  while (kw > 1 && kw > steps) kw /= 2;         // no idle slices on short contractions
  // tuning override (documented): NF4_GEMV_KW (1, 2, 4, 8 (16 with 32-row groups) within the waves cap / RW)
  const char* okw = getenv("NF4_GEMV_KW");
  if (okw) {
    const int v = atoi(okw);
    if ((v == 1 || v == 2 || v == 4 || v == 8 || v == 16) && v <= kw_max) kw = v;
  }
  pl.consumers = kw;
  pl.kc = static_cast<int>(kc);
  pl.splits = static_cast<int>(z);
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
  const int kw = plan.consumers;
  if (plan.bm == 16) {
    if (w.K % 256 != 0 || w.N % 16 != 0) return hipErrorInvalidValue;   // whole steps and row groups only
    // line-staged kernel; two halves of x per expanded fragment above M = 16.
    // A chunk of at most kLnMaxChunkSteps steps keeps each lane within two
    // nested groups (plan_small_m caps the chunk there).
    if (plan.bn * kw > kLnMaxWaves || gemv_ln_lds_bytes(plan.bn, kw, M, plan.kc) > kLnLdsMax ||
        plan.kc > 256 * kLnMaxChunkSteps)
      return hipErrorInvalidValue;
    p.tb_off = static_cast<int32_t>(gemv_region_bytes(16, plan.bn, kw, M, plan.kc));
    if (M > 16) {
      if (plan.bn == 1) return nested ? launch_ln_kw<1, true, 2>(kw, p, stream) : launch_ln_kw<1, false, 2>(kw, p, stream);
      if (plan.bn == 2) return nested ? launch_ln_kw<2, true, 2>(kw, p, stream) : launch_ln_kw<2, false, 2>(kw, p, stream);
      if (plan.bn == 4) return nested ? launch_ln_kw<4, true, 2>(kw, p, stream) : launch_ln_kw<4, false, 2>(kw, p, stream);
      return hipErrorInvalidValue;
    }
    if (plan.bn == 1) return nested ? launch_ln_kw<1, true, 1>(kw, p, stream) : launch_ln_kw<1, false, 1>(kw, p, stream);
    if (plan.bn == 2) return nested ? launch_ln_kw<2, true, 1>(kw, p, stream) : launch_ln_kw<2, false, 1>(kw, p, stream);
    if (plan.bn == 4) return nested ? launch_ln_kw<4, true, 1>(kw, p, stream) : launch_ln_kw<4, false, 1>(kw, p, stream);
    return hipErrorInvalidValue;
  }
  // 32-row groups
  if (plan.bm != 32 || plan.bn != 4 || gemv_region_bytes(32, 4, kw, M, plan.kc) > kGemvLdsMax)
    return hipErrorInvalidValue;
  p.tb_off = 0;
  return nested ? launch_kw32<true>(kw, p, stream) : launch_kw32<false>(kw, p, stream);
}

}  // namespace nf4
