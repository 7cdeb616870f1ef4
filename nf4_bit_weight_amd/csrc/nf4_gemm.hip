// Fused NF4 dequantise-and-multiply kernels for gfx950.
//
//   forward       y      = x      . W_hat^T   (bitsandbytes #2034, "Minimal
//                                              reproducer": matmul_4bit(h, w.t()))
//   input grad    grad_x = grad_y . W_hat     (Soup #842, "Design sketch": the
//                                              transposed fused backward)
//   grouped       the same per expert over expert-sorted rows (Experts PR,
//                 "Commit 2")
//
// Both directions are one contraction C[m, j] = sum_c A[m, c] * B(c, j):
//   forward : A = x [M, K],       j = n, c = k, B(c, j) = W_hat[j, c]
//   backward: A = grad_y [M, N],  j = k, c = n, B(c, j) = W_hat[c, j]
//
// One workgroup owns a BM x BN output tile and walks the contraction in steps
// of BK (BK * BN = 16384: one step's weight tile is 256 (row, 64-block)
// units).  Waves are specialised (see Tile below): per SIMD one producer wave
// copies the activation tile global -> LDS with global_load_lds_dwordx4 (no
// VGPR staging; 16-byte units of each row XOR-swizzled, swz below) and
// expands one (row, 64-block) weight unit per thread -- one byte table, eight
// 8-nibble expansions (nf4_device.hpp) -- straight into the LDS tile the MFMA
// operand is read from; C consumer waves per SIMD read fragments from LDS and
// run v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  Each weight is
// expanded once per workgroup and never written to HBM.  LDS is double
// buffered: the producers fill step s+1 while the consumers multiply step s.
// Weight tile layout in LDS:
//   forward : [BN rows n][BK k], same 16-byte XOR swizzle as A; the B
//             fragment (8 consecutive k of one n) is one 16-byte read;
//   backward: [BK rows n][BN k + 16 pad]; the B fragment (8 consecutive n at
//             one k) comes from two ds_read_b64_tr_b16 transposing reads
//             (each gives a lane 4 consecutive rows of its column).
// Output is rounded once to bf16 (RNE).  When too few tiles exist to fill the
// GPU the contraction is split S ways; each split writes fp32 partials and a
// second kernel adds them in the fixed order s = 0..S-1.  No atomics:
// repeated runs are bitwise identical.
#include <cstdlib>
#include <type_traits>

#include "nf4_device.hpp"
#include "nf4_internal.hpp"

namespace nf4 {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxBN = 256;            // widest output tile

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

struct GemmParams {
  const uint16_t* A;        // [rows, Kc] bf16
  uint16_t* C;              // [rows, Nc] bf16
  float* partial;           // [splits, M, Nc] fp32 when splits > 1
  WArgs w;
  const int32_t* offsets;   // grouped only: [E + 1]
  int64_t M;                // rows of A and C
  int32_t E;
  int32_t splits;
  int32_t m_tiles;          // row tiles (grouped: an upper bound)
};

// BM x BN output tile, contraction step BK chosen so the weight tile holds
// exactly 256 (row, 64-block) units.  The workgroup has 4 producer waves and
// 4*C consumer waves (C = 1 or 2), i.e. per SIMD one producer and C
// consumers:
//   producer : copies the activation tile (global -> LDS), fetches the packed
//              weights kPD steps ahead and expands one (row, 64-block) unit
//              per thread into the LDS weight tile -- pure VALU / memory work;
//   consumer : reads MFMA fragments from LDS and issues the MFMAs of its
//              (BM / CW_M) x (BN / CW_N) part of the tile.
// A wave cannot issue VALU work while its own MFMA runs (measured: MFMA + 8
// VALU ops cost ~54 cycles instead of 32), but the SIMD issues one wave's
// VALU and another wave's MFMA in the same cycles, so splitting the roles
// makes a step cost ~max(expansion, MFMA) instead of their sum.
// Global-memory latency (several steps' worth under load) is hidden by
// prefetch depth: the activation tile lives in an NA-stage LDS ring (copy
// issued NA-1 steps ahead) and the packed weights in kPD register sets.
template <int BM, int BN_, bool TRANS, int C_>
struct Tile {
  static constexpr int BN = BN_;
  static constexpr int C = C_;
  static constexpr int kThreads = 64 * (4 + 4 * C);
  static constexpr int BK = 16384 / BN;             // 64 (BN 256) or 128 (BN 128)
  static constexpr int CW_M = 2;                    // consumer waves: 2 x (2C)
  static constexpr int CW_N = 2 * C;
  static constexpr int WM = BM / CW_M;
  static constexpr int WN = BN / CW_N;
  static constexpr int MI = WM / 32;
  static constexpr int NI = WN / 32;
  static constexpr int KK = BK / 16;                // MFMA k-steps per step
  static constexpr int kUnits = BK / 8;             // 16-byte units per tile row
  static constexpr int kARowsPerInstr = 64 / kUnits;
  static constexpr int kARowsPerWave = BM / 4;      // activation rows per producer wave
  static constexpr int kAInstr = kARowsPerWave / kARowsPerInstr;
  static constexpr int kBTPitch = BN + 16;          // backward weight tile pitch (elements)
  static constexpr int kAElems = BM * BK;
  static constexpr int kBElems = TRANS ? BK * kBTPitch : BN * BK;
  // LDS: NA activation stages, 2 expanded weight buffers and PD staging
  // slots of packed weights (kWSlot bytes each: 256 units x 32 B, then
  // 256 x 4 B block scales, then 256 x 4 B nested scales), within 159 KB
  // (1 KB is the static nested table).  Deepest prefetch that fits, in the
  // order (4, 4), (2, 4), (2, 2).
  static constexpr int kWSlot = 10240;
  static constexpr int kFixed = 2 * kBElems * 2;
  static constexpr int kBudget = 159 * 1024;
  static constexpr bool kFit44 = kFixed + 4 * kAElems * 2 + 4 * kWSlot <= kBudget;
  static constexpr bool kFit24 = kFixed + 2 * kAElems * 2 + 4 * kWSlot <= kBudget;
  static constexpr int NA = kFit44 ? 4 : 2;         // activation stages
  static constexpr int kPD = (kFit44 || kFit24) ? 4 : 2;   // weight slots = prefetch distance
  static constexpr int kAOff = 0;
  static constexpr int kBOff = NA * kAElems * 2;
  static constexpr int kWOff = kBOff + kFixed;
  static constexpr int kLdsBytes = kWOff + kPD * kWSlot;
  // Consumers double-buffer their fragments when the registers allow it
  // (every wave of the kernel gets 512 / waves-per-SIMD registers).
  static constexpr int kRegs = (512 / (1 + C)) & ~7;
  static constexpr bool kFragDB = MI * NI * 16 + 2 * (MI + NI) * 4 + 32 <= kRegs;
  static_assert(MI >= 1 && NI >= 1, "tile too small");
  static_assert(kARowsPerWave % kARowsPerInstr == 0, "A copy split");
  static_assert(kLdsBytes <= kBudget, "LDS budget of one workgroup");
};

// 16-byte unit u of row r of a [rows][BK] tile is stored at unit u ^ ((r >> 1) & 7):
// for the MFMA fragment reads (32 rows x 2 units per wave instruction) this
// measured ~1.4x the LDS throughput of u ^ (r & 7) on gfx950.
__device__ __forceinline__ int swz(int r, int u) { return u ^ ((r >> 1) & 7); }

// Workgroups are dispatched to the 8 XCDs round-robin by linear id, and each
// XCD has its own L2.  Linear id L is mapped to tile t so that XCD j runs the
// contiguous tile range [j*q + min(j, r), ...) (q = T/8, r = T%8); tiles are
// ordered (column tile, split, row tile) with the row tile fastest, so the
// row tiles sharing one weight tile run together on one XCD and the weight
// tile is fetched from HBM into that L2 once.
__device__ __forceinline__ int xcd_tile(int L, int T) {
  const int xcd = L & 7, idx = L >> 3;
  const int q = T >> 3, r = T & 7;
  return xcd * q + (xcd < r ? xcd : r) + idx;
}

// Tile id (after xcd_tile) -> row tile mt, column tile ct, split z, for a grid
// of exactly T = m_tiles x column tiles x splits workgroups.  The split is the
// outermost index, so the run of ids one XCD serves shares one contraction
// slice: each XCD then fetches 1/splits of the activations into its L2 and the
// same weight bytes as with the split innermost (splits times the column
// tiles, each over a slice splits times shorter).  Measured on MI355X at
// M = 512 over the Llama-3.1-8B projections, same box: input gradients of
// down / gate 94.2 / 90.6 -> 92.1 / 88.3 us, forward of down 85.7 -> 82.7 us.
// The small-tile producer/consumer kernel keeps the split innermost (forward
// of k, 64 x 128 tiles, four splits: 20.7 against 22.6 us).
template <bool kSplitOuter = true>
__device__ __forceinline__ void tile_coords(int tt, int T, int m_tiles, int splits, int& mt, int& ct, int& z) {
  if constexpr (kSplitOuter) {
    const int per_split = T / splits;
    z = tt / per_split;
    const int r = tt - z * per_split;
    mt = r % m_tiles;
    ct = r / m_tiles;
  } else {
    mt = tt % m_tiles;
    const int cz = tt / m_tiles;
    z = cz % splits;
    ct = cz / splits;
  }
}

template <int N>
using ic = std::integral_constant<int, N>;

// LDS-direct copies written as inline assembly.  The compiler's own wait
// insertion treats every LDS access that may alias a pending LDS-direct copy
// as needing vmcnt(0); with the copies issued through the builtins it put
// about five such waits into each step of the ping-pong kernel (before the
// expanded-tile stores and the fragment reads), so every copy was waited for
// right after it was issued.  Copies issued here are invisible to it; the
// kernel's explicit waits (also assembly, vm_wait below) are then the only
// waits on them.  The wave-uniform LDS address is passed in M0; one wait
// state separates the M0 write from the copy.
__device__ __forceinline__ void dma_b128(const void* src, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(src), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma_b32(const void* src, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" :: "v"(src), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma_u8(const void* src, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_ubyte %0, off" :: "v"(src), "{m0}"(lds) : "memory");
}
template <int C>
__device__ __forceinline__ void vm_wait() {
  static_assert(C >= 0 && C < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(C) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void_t*)p));
}

// Rows of row tile mt: [row0, row_end) of A and C, and the first row of the
// weight tensor it multiplies.  Dense: tile mt of BM rows.  Grouped: the row
// tiles are numbered expert by expert (ceil(rows_e / BM) tiles each, from the
// expert-sorted offsets[E + 1], every entry clamped into [0, M] so a malformed
// array cannot index out of range); the tile stops at its expert's last row
// and meets that expert's slice of the [E * N, K] stack.  Returns false for a
// tile id past the last expert's tiles (m_tiles is an upper bound).
//
// Grouped search: 64 experts per round, one per lane of the wave: the lanes
// load their offsets together, an inclusive prefix sum of the tile counts
// runs across the wave, and a ballot names the expert whose tiles contain
// mt.  Every wave of the workgroup reaches the same answer on its own (no
// LDS, no barrier); called by whole waves.
template <int BM, bool GROUPED>
__device__ __forceinline__ bool row_tile(const GemmParams& p, int mt, int64_t N, int64_t& row0,
                                         int64_t& row_end, int64_t& wrow_base) {
  if constexpr (GROUPED) {
    const int lane = static_cast<int>(threadIdx.x & 63);
    int acc = 0;                                   // tiles of the experts before this round
    for (int e0 = 0; e0 < p.E; e0 += 64) {
      const int e = e0 + lane;
      int64_t a = 0, b = 0;
      if (e < p.E) {
        a = p.offsets[e];
        b = p.offsets[e + 1];
        a = a < 0 ? 0 : (a > p.M ? p.M : a);
        b = b < a ? a : (b > p.M ? p.M : b);
      }
      const int cnt = static_cast<int>((b - a + BM - 1) / BM);
      int incl = cnt;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(incl, d, 64);
        if (lane >= d) incl += t;
      }
      const int lo = acc + incl - cnt;             // first tile of expert e
      const unsigned long long hit = __ballot(mt >= lo && mt < acc + incl);
      if (hit != 0) {
        const int l = __ffsll(static_cast<long long>(hit)) - 1;
        const int first = __shfl(lo, l, 64);
        row0 = __shfl(a, l, 64) + static_cast<int64_t>(mt - first) * BM;
        row_end = __shfl(b, l, 64);
        wrow_base = static_cast<int64_t>(e0 + l) * N;
        return true;
      }
      acc += __shfl(incl, 63, 64);
    }
    return false;
  } else {
    row0 = static_cast<int64_t>(mt) * BM;
    row_end = p.M;
    wrow_base = 0;
    return true;
  }
}

template <int BM, int BN, bool TRANS, bool NESTED, bool GROUPED, int C>
__global__ __launch_bounds__(64 * (4 + 4 * C), 1) void k_gemm(GemmParams p) {
  using T = Tile<BM, BN, TRANS, C>;
  constexpr int BK = T::BK;
  constexpr int NA = T::NA;
  constexpr int PD = T::kPD;
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  __shared__ float sncode[256];

  const int tid = threadIdx.x;
  // the wave index is uniform across the wave; saying so keeps M0 (the LDS
  // destination of global_load_lds) and the role branch scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int64_t N = p.w.N, K = p.w.K;
  const int64_t Nc = TRANS ? K : N;        // output columns
  const int64_t Kc = TRANS ? N : K;        // contraction length
  const int ktiles = static_cast<int>((Kc + BK - 1) / BK);

  // ---- tile owned by this workgroup -----------------------------------------
  int mt, ct, z;
  tile_coords<false>(xcd_tile(blockIdx.x, gridDim.x), gridDim.x, p.m_tiles, p.splits, mt, ct, z);
  const int64_t col0 = static_cast<int64_t>(ct) * BN;
  int64_t row0, row_end, wrow_base;
  if (!row_tile<BM, GROUPED>(p, mt, N, row0, row_end, wrow_base)) return;
  const int kb = static_cast<int>(static_cast<int64_t>(z) * ktiles / p.splits);
  const int ke = static_cast<int>(static_cast<int64_t>(z + 1) * ktiles / p.splits);
  const int n = ke - kb;                   // steps of this workgroup

  auto a_tile = [&](int stage) { return lds + stage * T::kAElems; };
  auto b_tile = [&](int buf) { return lds + NA * T::kAElems + buf * T::kBElems; };
  char* const w_area = reinterpret_cast<char*>(lds) + T::kWOff;

  // Step i (0 <= i < n) of the contraction uses activation stage i % NA and
  // weight buffer i % 2.  During step i the consumers multiply step i while
  // the producers (a) issue the activation copy of step i+NA-1 into the stage
  // step i-1 used, (b) issue the packed-weight copy of step i+PD into the
  // staging slot step i used, (c) expand the weights of step i+1 into the
  // buffer step i-1 used.  One workgroup barrier ends each step.  Indices
  // past the last step are clamped to it: the copies and expansions they
  // cause land in buffers no later step reads.
  //
  // Every global load of the loop is an LDS-direct copy and the staging
  // reads are inline assembly, so the only waits on vector memory are the
  // explicit per-step vmcnt below (the compiler's own wait insertion falls
  // back to vmcnt(0) once a loop mixes LDS-direct copies with loads into
  // registers that are carried across iterations, which would drain the
  // whole prefetch pipeline every iteration).
  if (wave < 4) {
    // =================== producer waves (threads 0..255) ======================
    float code[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) code[i] = p.w.code[i];
    float off = 0.f;
    if constexpr (NESTED) {
      sncode[tid] = p.w.ncode[tid];
      off = p.w.nested_offset[0];
    }

    // Activation tile: global -> LDS directly.  Producer wave w copies rows
    // [w*BM/4, (w+1)*BM/4), 1 KB per instruction; lane l fills physical unit
    // l%U of row l/U (U = BK/8 units per row) with logical unit swz(row, l%U).
    // Rows past the end are clamped to the last valid row (their products
    // are never stored); contraction columns past Kc are clamped inside the
    // row and meet zero weights.
    const int a_r_in = lane / T::kUnits;
    const int a_unit = lane % T::kUnits;
    auto issue_a = [&](int i, int stage) {
      const int kt = kb + (i < n ? i : n - 1);
      const int64_t c0 = static_cast<int64_t>(kt) * BK;
#pragma unroll
      for (int j = 0; j < T::kAInstr; ++j) {
        const int r = wave * T::kARowsPerWave + j * T::kARowsPerInstr + a_r_in;
        int64_t row = row0 + r;
        row = row < row_end ? row : row_end - 1;
        int64_t col = c0 + 8 * swz(r, a_unit);
        col = col < Kc ? col : Kc - 8;
        const uint16_t* src = p.A + row * Kc + col;
        uint16_t* dst = a_tile(stage) + (wave * T::kARowsPerWave + j * T::kARowsPerInstr) * BK;
        __builtin_amdgcn_global_load_lds(src, (lds_void_t*)dst, 16, 0, 0);
      }
    };

    // Weight units.  Unit u of a step covers
    //   forward : W row (col0 + u % BN), block (kt*BK/64 + u / BN)
    //   backward: W row (kt*BK + u % BK), block (col0/64 + u / BK)
    // and its element offset is off0 + kt * dstep.  Producer thread t expands
    // unit t; the copy of unit u's 32 packed bytes is done by lanes 2u, 2u+1
    // (mod 64) of the same wave, the copy of its scale by lane u of the same
    // wave, so each wave reads only what its own copies wrote.  Units past
    // the matrix copy unit 0 of the tensor and are replaced by zero weights.
    struct Unit {
      int64_t off0;
      int var_in;
      bool fixed_ok;
    };
    const int64_t dstep = TRANS ? static_cast<int64_t>(BK) * K : BK;
    const int64_t var_lim = TRANS ? N : K;
    auto unit_of = [&](int u) {
      Unit g;
      if constexpr (TRANS) {
        const int64_t wcol = col0 + 64 * (u / BK);
        g.fixed_ok = wcol < K;
        g.off0 = (wrow_base + u % BK) * K + wcol;
        g.var_in = u % BK;
      } else {
        const int64_t wrow = col0 + (u % BN);
        g.fixed_ok = wrow < N;
        g.off0 = (wrow_base + wrow) * K + 64 * (u / BN);
        g.var_in = 64 * (u / BN);
      }
      return g;
    };
    auto unit_valid = [&](const Unit& g, int kt) {
      return g.fixed_ok & (static_cast<int64_t>(kt) * BK + g.var_in < var_lim);
    };
    auto unit_flat = [&](const Unit& g, int kt) -> uint64_t {
      return unit_valid(g, kt) ? static_cast<uint64_t>(g.off0 + kt * dstep) : 0;   // multiple of 64
    };
    const Unit own = unit_of(tid);
    const Unit cp0 = unit_of(64 * wave + (lane >> 1));
    const Unit cp1 = unit_of(64 * wave + 32 + (lane >> 1));
    auto issue_w = [&](int i, int slot) {
      const int kt = kb + (i < n ? i : n - 1);
      char* sl = w_area + slot * T::kWSlot;
      const uint8_t* s0 = p.w.packed + (unit_flat(cp0, kt) >> 1) + 16 * (lane & 1);
      const uint8_t* s1 = p.w.packed + (unit_flat(cp1, kt) >> 1) + 16 * (lane & 1);
      __builtin_amdgcn_global_load_lds(s0, (lds_void_t*)(sl + 2048 * wave), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(s1, (lds_void_t*)(sl + 2048 * wave + 1024), 16, 0, 0);
      const uint64_t b = unit_flat(own, kt) >> 6;
      if constexpr (NESTED) {
        // one byte per lane, written zero-extended to the lane's dword
        __builtin_amdgcn_global_load_lds(static_cast<const uint8_t*>(p.w.absmax) + b,
                                         (lds_void_t*)(sl + 8192 + 256 * wave), 1, 0, 0);
        __builtin_amdgcn_global_load_lds(p.w.nested_absmax + (b >> 8),
                                         (lds_void_t*)(sl + 9216 + 256 * wave), 4, 0, 0);
      } else {
        __builtin_amdgcn_global_load_lds(static_cast<const float*>(p.w.absmax) + b,
                                         (lds_void_t*)(sl + 8192 + 256 * wave), 4, 0, 0);
      }
    };
    // LDS byte addresses of this thread's staged unit and scale in slot 0
    const uint32_t st_unit = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)w_area)) + 32 * tid;
    const uint32_t st_scale = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)w_area)) + 8192 + 4 * tid;
    const uint32_t st_ncode = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)sncode));
    struct Staged {
      u32x4_t pk0, pk1;
      uint32_t sc, s2;
    };
#define NF4_READ_UNIT(OFF)                                                                 \
  asm volatile("ds_read_b128 %0, %4 offset:" #OFF "\n\t"                                   \
               "ds_read_b128 %1, %4 offset:" #OFF "+16\n\t"                                \
               "ds_read_b32 %2, %5 offset:" #OFF "\n\t"                                    \
               "ds_read_b32 %3, %5 offset:" #OFF "+1024\n\t"                               \
               "s_waitcnt lgkmcnt(0)"                                                      \
               : "=&v"(r.pk0), "=&v"(r.pk1), "=&v"(r.sc), "=&v"(r.s2)                      \
               : "v"(st_unit), "v"(st_scale)                                               \
               : "memory")
    auto read_unit = [&](int slot) {
      Staged r;
      static_assert(T::kWSlot == 10240, "slot offsets below");
      switch (slot) {
        case 0: NF4_READ_UNIT(0); break;
        case 1: NF4_READ_UNIT(10240); break;
        case 2: NF4_READ_UNIT(20480); break;
        default: NF4_READ_UNIT(30720); break;
      }
      return r;
    };
#undef NF4_READ_UNIT
    auto b_dst = [&](int buf, int d) -> uint16_t* {
      if constexpr (TRANS) {
        return b_tile(buf) + (tid % BK) * T::kBTPitch + 64 * (tid / BK) + 8 * d;
      } else {
        const int row = tid % BN;
        return b_tile(buf) + row * BK + 8 * swz(row, 8 * (tid / BN) + d);
      }
    };
    // expand the staged unit of step i (slot `slot`) into weight buffer `buf`
    auto expand_into = [&](int i, int slot, int buf) {
      const int kt = kb + (i < n ? i : n - 1);
      const bool valid = unit_valid(own, kt);
      const Staged r = read_unit(slot);
      float a;
      if constexpr (NESTED) {
        float nc;
        asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                     : "=v"(nc) : "v"(st_ncode + 4 * (r.sc & 0xFF)) : "memory");
        a = __fadd_rn(__fmul_rn(nc, __uint_as_float(r.s2)), off);
      } else {
        a = __uint_as_float(r.sc);
      }
      const u32x4_t zero_codes = {0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u};
      const u32x4_t pk0 = valid ? r.pk0 : zero_codes;
      const u32x4_t pk1 = valid ? r.pk1 : zero_codes;
      const Lut lt = make_lut(code, valid ? a : 0.f);
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        uint32_t o[4];
        // input gradient: the unit's 8 weights are 8 output columns, so the
        // cheaper (0,2,4,6,1,3,5,7) order is undone in the epilogue
        if constexpr (TRANS) expand8_eo(d < 4 ? pk0[d] : pk1[d - 4], lt, o);
        else expand8(d < 4 ? pk0[d] : pk1[d - 4], lt, o);
        *reinterpret_cast<u32x4_t*>(b_dst(buf, d)) = u32x4_t{o[0], o[1], o[2], o[3]};
      }
    };
    // Vector-memory operations complete in issue order; step i issues the
    // activation copy of step i+NA-1 (kA operations), then the weight copy
    // of step i+PD (kW).  At the end of step i the activation copy of step
    // i+1 (multiplied in step i+1) and the weight copy of step i+2 (expanded
    // in step i+1) must have landed, i.e. at most kWait later operations may
    // still be in flight.
    constexpr int kA = T::kAInstr;
    constexpr int kW = NESTED ? 4 : 3;
    constexpr int kAfterA = kW + (NA - 2) * (kA + kW);
    constexpr int kAfterW = (PD - 2) * (kA + kW);
    constexpr int kWait = kAfterA < kAfterW ? kAfterA : kAfterW;
    static_assert(kWait < 64, "vmcnt range");
    auto wait_vm = [](auto cnt) {
      constexpr int c = decltype(cnt)::value;
      // vmcnt(c) lgkmcnt(0); vmcnt is split over bits 3:0 and 15:14
      __builtin_amdgcn_s_waitcnt((c & 15) | ((c >> 4) << 14) | (7 << 4));
    };
    auto end_step = [&]() {
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
      wait_vm(ic<kWait>{});
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };

    if (n > 0) {
      if constexpr (NESTED) __syncthreads();      // sncode filled (matched by consumers)
#pragma unroll
      for (int j = 0; j < NA - 1; ++j) issue_a(j, j);
#pragma unroll
      for (int j = 0; j < PD; ++j) issue_w(j, j);
      wait_vm(ic<(PD - 1) * kW>{});                // every activation copy, weights of step 0
      expand_into(0, 0, 0);
      // Weights of step 1, and of step 2 when the prologue issued them: kWait
      // assumes each step's weight copy is followed by the copies of later
      // steps in the steady order (activation, weights), but the prologue put
      // every activation copy first, so at the end of step 0 fewer operations
      // follow the weights of step 2 than kWait allows in flight (with four
      // activation stages and four weight slots).
      wait_vm(ic<(PD > 2 ? PD - 3 : 0) * kW>{});
      __syncthreads();
      auto step = [&](int i, auto ph) {
        constexpr int P = decltype(ph)::value;
        issue_a(i + NA - 1, (P + NA - 1) % NA);
        issue_w(i + PD, P % PD);
        __builtin_amdgcn_sched_barrier(0);
        expand_into(i + 1, (P + 1) % PD, (P + 1) % 2);
        end_step();
      };
      int i = 0;
      for (; i + 4 <= n; i += 4) {
        step(i, ic<0>{});
        step(i + 1, ic<1>{});
        step(i + 2, ic<2>{});
        step(i + 3, ic<3>{});
      }
      if (i < n) step(i, ic<0>{});
      if (i + 1 < n) step(i + 1, ic<1>{});
      if (i + 2 < n) step(i + 2, ic<2>{});
      __builtin_amdgcn_s_waitcnt(0);               // no copy into LDS outlives the workgroup
    }
    return;
  }

  // ===================== consumer waves ========================================
  const int cw = wave - 4;
  const int wm = cw / T::CW_N, wn = cw % T::CW_N;
  const int r32 = lane & 31, h = lane >> 5;
  f32x16_t acc[T::MI][T::NI];
#pragma unroll
  for (int i = 0; i < T::MI; ++i)
#pragma unroll
    for (int j = 0; j < T::NI; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // Fragment addresses.  Fragment i of k-step kk reads A row
  // wm*WM + 32i + r32, 16-byte unit 2kk + h, stored at unit
  // (2kk + h) ^ ((row >> 1) & 7) = 2kk ^ y with y = h ^ ((r32 >> 1) & 7)
  // (WM and WN are multiples of 32, and 2kk and h use disjoint bits).  So a
  // lane needs one address per (kk mod 4) for A and one for B; stage, buffer,
  // fragment index and kk >= 4 (unit + 8) are compile-time offsets that fit
  // the instruction's immediate field.
  const int y = h ^ ((r32 >> 1) & 7);
  const char* pa[4];
  const char* pb[4];
  {
    const char* a0 = reinterpret_cast<const char*>(lds) + (wm * T::WM + r32) * BK * 2;
    const char* b0 = reinterpret_cast<const char*>(lds + NA * T::kAElems);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      pa[q] = a0 + 16 * ((2 * q) ^ y);
      if constexpr (TRANS) {
        // backward transposing read: lane l of 16-lane group g, index s = l%16
        const int tg = lane >> 4, ts = lane & 15;
        const int tr_row = 8 * (tg >> 1) + (ts >> 2);                 // + 16*kk + 4*half
        const int tr_col = wn * T::WN + 16 * (tg & 1) + 4 * (ts & 3); // + 32*j
        pb[q] = b0 + (tr_row * T::kBTPitch + tr_col) * 2;
      } else {
        pb[q] = b0 + (wn * T::WN + r32) * BK * 2 + 16 * ((2 * q) ^ y);
      }
    }
  }

  struct Frags {
    bf16x8_t a[T::MI];
    bf16x8_t b[T::NI];
  };
  // stage, buf and kk are compile-time constants at every call
  auto load_frags = [&](int stage, int buf, int kk, Frags& f) {
#pragma unroll
    for (int i = 0; i < T::MI; ++i)
      f.a[i] = *reinterpret_cast<const bf16x8_t*>(pa[kk & 3] + stage * T::kAElems * 2 +
                                                  (kk >> 2) * 128 + i * 32 * BK * 2);
#pragma unroll
    for (int j = 0; j < T::NI; ++j) {
      if constexpr (TRANS) {
        const char* src = pb[0] + buf * T::kBElems * 2 + (16 * kk * T::kBTPitch + 32 * j) * 2;
        s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(src));
        s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(src + 4 * T::kBTPitch * 2));
        u32x2_t ul = __builtin_bit_cast(u32x2_t, lo), uh = __builtin_bit_cast(u32x2_t, hi);
        f.b[j] = __builtin_bit_cast(bf16x8_t, u32x4_t{ul[0], ul[1], uh[0], uh[1]});
      } else {
        f.b[j] = *reinterpret_cast<const bf16x8_t*>(pb[kk & 3] + buf * T::kBElems * 2 +
                                                    (kk >> 2) * 128 + j * 32 * BK * 2);
      }
    }
  };
  auto mfmas = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < T::MI; ++i)
#pragma unroll
      for (int j = 0; j < T::NI; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
  };
  // With double-buffered fragments the reads of k-step kk+1 are issued
  // while the MFMAs of kk run (a scheduling fence per k-step keeps at most
  // two sets live); otherwise the other consumer wave of the SIMD covers
  // the read latency.
  auto compute = [&](int stage, int buf) {
    if constexpr (T::kFragDB) {
      Frags f0, f1;
      load_frags(stage, buf, 0, f0);
#pragma unroll
      for (int kk = 0; kk < T::KK; ++kk) {
        Frags& fc = (kk & 1) ? f1 : f0;
        Frags& fn = (kk & 1) ? f0 : f1;
        if (kk + 1 < T::KK) load_frags(stage, buf, kk + 1, fn);
        mfmas(fc);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < T::KK; ++kk) {
        Frags f;
        load_frags(stage, buf, kk, f);
        mfmas(f);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  auto end_step = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);                         // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  if (n > 0) {
    if constexpr (NESTED) __syncthreads();        // matches the producers' sncode barrier
    __syncthreads();                              // step 0 is in stage 0 / buffer 0
    auto step = [&](auto ph) {
      constexpr int P = decltype(ph)::value;
      compute(P % NA, P % 2);
      end_step();
    };
    int i = 0;
    for (; i + 4 <= n; i += 4) {
      step(ic<0>{});
      step(ic<1>{});
      step(ic<2>{});
      step(ic<3>{});
    }
    if (i < n) step(ic<0>{});
    if (i + 1 < n) step(ic<1>{});
    if (i + 2 < n) step(ic<2>{});
  }

  // ---- epilogue ----------------------------------------------------------------
  // acc[i][j][v] holds C[32i + 8(v/4) + 4h + v%4][32j + r32] of the wave tile
  // (input gradient: tile column c is output column 8 (c / 8) + pi(c % 8), the
  // order of expand8_eo).
#pragma unroll
  for (int i = 0; i < T::MI; ++i) {
#pragma unroll
    for (int j = 0; j < T::NI; ++j) {
      int64_t col = col0 + wn * T::WN + 32 * j + r32;
      if constexpr (TRANS) col = (col & ~int64_t{7}) | (((col & 3) << 1) | ((col >> 2) & 1));
      if (col >= Nc) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = row0 + wm * T::WM + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
        if (row >= row_end) continue;
        if (p.splits == 1) {
          p.C[row * Nc + col] = to_bf16(acc[i][j][v]);
        } else {
          p.partial[(static_cast<int64_t>(z) * p.M + row) * Nc + col] = acc[i][j][v];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 256 x 256 "ping-pong" kernel.  Eight identical waves, two per SIMD, no
// dedicated roles.  Wave w owns the 128 x 64 output block (w / 4, w % 4)
// with double-buffered MFMA fragments (at two waves per SIMD every wave has
// 256 VGPRs, room the three-waves-per-SIMD producer/consumer layout lacks),
// and every thread also expands half a weight unit (32 weights) per step.
// Two schedules for a step, picked per direction by measurement:
//   forward: each k-step's 8 MFMAs are interleaved with one piece of the
//            next step's expansion (scheduling groups of one MFMA and a few
//            VALU operations), so every wave mixes both;
//   input gradient: the waves sharing a SIMD (w and w + 4; measured: this is
//            how the CU places them) take the multiply and expand halves in
//            opposite order, one wave's expansion under the other's MFMAs
//            (measured: another wave's VALU leaves MFMA throughput intact).
// Staging as in k_gemm: LDS-direct copies of the activation tile (2 stages)
// and of the packed weights and scales (2 slots), one explicit vmcnt per
// step, one barrier per step.  A wave's six copy instructions of a step are
// spread over the first half of its step (between MFMA groups or between
// expansion groups) rather than issued in one burst: 48 copies issued at once
// back up the CU's vector-memory queue and hold every wave at the issue.
struct PP {
  static constexpr int BM = 256, BN = 256, BK = 64;
  static constexpr int kThreads = 512;
  static constexpr int MI = 4, NI = 2, WM = 128, WN = 64, KK = 4;
  static constexpr int kAElems = BM * BK;
  // Input gradient: the expanded tile is [k-row][n] with 256-element rows
  // and its 16-byte units XOR-swizzled by the row: unit c of row r is stored
  // at unit c ^ swz_t(r).  Both the expansion's 16-byte writes (16 lanes: 8
  // rows x 2 halves) and the transposed 8-byte fragment reads (32 lanes: 4
  // rows x 8 columns) then hit 64 distinct banks; a padded pitch (BN + 16)
  // left both 2-way conflicted (measured: conflict cycles were a third of the
  // kernel's LDS cycles).
  static constexpr int kBTPitch = BN;
  static constexpr int kWSlot = 10240;          // 8 KB packed, 1 KB scales, 1 KB nested scales
  static constexpr int kWSlots = 3;             // weight slots: each copy has two steps to land
  // unit swizzle of row r: rows r & 3 = 0..3 take distinct bits 2-3 (reads
  // of four rows), and over r & 7 the values with bit 2 cleared are distinct
  // (writes of eight rows, two halves 4 units apart)
  static __device__ __forceinline__ int swz_t(int r) { return (5 * (r & 3)) ^ (2 * ((r >> 2) & 1)); }
  template <bool TRANS>
  static constexpr int b_elems() { return TRANS ? BK * kBTPitch : BN * BK; }
  template <bool TRANS>
  static constexpr int lds_bytes() { return 2 * kAElems * 2 + 2 * b_elems<TRANS>() * 2 + kWSlots * kWSlot; }
};
static_assert(PP::lds_bytes<true>() + 1024 <= 160 * 1024, "LDS budget of one workgroup");

template <bool TRANS, bool NESTED, bool GROUPED>
__global__ __launch_bounds__(512, 1) void k_pp(GemmParams p) {
  constexpr int BM = PP::BM, BN = PP::BN, BK = PP::BK;
  constexpr int kBElems = PP::b_elems<TRANS>();
  constexpr int kBOff = 2 * PP::kAElems * 2;
  constexpr int kWOff = kBOff + 2 * kBElems * 2;
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  __shared__ float sncode[256];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int64_t N = p.w.N, K = p.w.K;
  const int64_t Nc = TRANS ? K : N;
  const int64_t Kc = TRANS ? N : K;
  const int ktiles = static_cast<int>((Kc + BK - 1) / BK);

  // ---- tile owned by this workgroup (as k_gemm) ----------------------------------
  int mt, ct, z;
  tile_coords(xcd_tile(blockIdx.x, gridDim.x), gridDim.x, p.m_tiles, p.splits, mt, ct, z);
  const int64_t col0 = static_cast<int64_t>(ct) * BN;
  int64_t row0, row_end, wrow_base;
  if (!row_tile<BM, GROUPED>(p, mt, N, row0, row_end, wrow_base)) return;
  const int kb = static_cast<int>(static_cast<int64_t>(z) * ktiles / p.splits);
  const int ke = static_cast<int>(static_cast<int64_t>(z + 1) * ktiles / p.splits);
  const int n = ke - kb;

  auto a_tile = [&](int stage) { return lds + stage * PP::kAElems; };
  auto b_tile = [&](int buf) { return lds + 2 * PP::kAElems + buf * kBElems; };
  char* const w_area = reinterpret_cast<char*>(lds) + kWOff;

  if constexpr (NESTED) {
    if (tid < 256) sncode[tid] = p.w.ncode[tid];
  }
  float code[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) code[i] = p.w.code[i];
  const float off = NESTED ? p.w.nested_offset[0] : 0.f;

  // ---- copies (every wave issues its share) ---------------------------------------
  // activation: wave w copies rows [32w, 32w + 32), 8 rows per instruction
  const int a_r_in = lane >> 3, a_unit = lane & 7;
  // j-th of the wave's four activation copy instructions of step i.  The
  // row part of each lane's address is fixed for the workgroup (rows past the
  // end clamped); per step only the column moves.
  const uint16_t* a_row_ptr[4];
  int a_colofs[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 32 * wave + 8 * j + a_r_in;
    int64_t row = row0 + r;
    row = row < row_end ? row : row_end - 1;
    a_row_ptr[j] = p.A + row * Kc;
    a_colofs[j] = 8 * swz(r, a_unit);
  }
  auto issue_a = [&](int i, int stage, int j) __attribute__((always_inline)) {
    const int kt = kb + (i < n ? i : n - 1);
    const int64_t c0 = static_cast<int64_t>(kt) * BK;
    int64_t col = c0 + a_colofs[j];
    col = col < Kc ? col : Kc - 8;
    const uint16_t* src = a_row_ptr[j] + col;
    dma_b128(src, __builtin_amdgcn_readfirstlane(lds_addr(a_tile(stage) + (32 * wave + 8 * j) * BK)));
  };
  // weights: thread t expands half h = t & 1 of unit u = t >> 1 of the step
  // (fwd: W row col0 + u, block kt; bwd: W row kt*64 + u % 64, block
  // col0/64 + u / 64).  Lane t of the packed copy fetches exactly those 16
  // bytes.  The scales of units 64v .. 64v+63 are copied by wave v (v < 4),
  // their nested scales by wave v + 4, one unit per lane.
  struct UnitG {
    int64_t off0;
    int var_in;
    bool fixed_ok;
  };
  const int64_t dstep = TRANS ? static_cast<int64_t>(BK) * K : BK;
  const int64_t var_lim = TRANS ? N : K;
  auto unit_of = [&](int uu) {
    UnitG g;
    if constexpr (TRANS) {
      const int64_t wcol = col0 + 64 * (uu / 64);
      g.fixed_ok = wcol < K;
      g.off0 = (wrow_base + uu % 64) * K + wcol;
      g.var_in = uu % 64;
    } else {
      const int64_t wrow = col0 + uu;
      g.fixed_ok = wrow < N;
      g.off0 = (wrow_base + wrow) * K;
      g.var_in = 0;
    }
    return g;
  };
  const int u = tid >> 1, hh = tid & 1;
  const UnitG own = unit_of(u);
  const UnitG scu = unit_of(64 * (wave & 3) + lane);     // unit whose scale this lane copies
  auto unit_valid = [&](const UnitG& g, int kt) {
    return g.fixed_ok & (static_cast<int64_t>(kt) * BK + g.var_in < var_lim);
  };
  auto unit_flat = [&](const UnitG& g, int kt) -> uint64_t {
    return unit_valid(g, kt) ? static_cast<uint64_t>(g.off0 + kt * dstep) : 0;   // multiple of 64
  };
  // packed bytes of this thread's half unit: a fixed lane base plus the
  // uniform step offset kt * dstep / 2; invalid units read unit 0
  const uint8_t* const pk_base = p.w.packed + (own.off0 >> 1) + 16 * hh;
  auto issue_wpk = [&](int i, int slot) __attribute__((always_inline)) {
    const int kt = kb + (i < n ? i : n - 1);
    char* sl = w_area + slot * PP::kWSlot;
    const uint8_t* src = unit_valid(own, kt) ? pk_base + ((static_cast<int64_t>(kt) * dstep) >> 1) : p.w.packed;
    dma_b128(src, __builtin_amdgcn_readfirstlane(lds_addr(sl + 1024 * wave)));
  };
  auto issue_ws = [&](int i, int slot) __attribute__((always_inline)) {
    const int kt = kb + (i < n ? i : n - 1);
    char* sl = w_area + slot * PP::kWSlot;
    const uint64_t b = unit_flat(scu, kt) >> 6;
    if (wave < 4) {
      if constexpr (NESTED) {
        // one byte per lane, written zero-extended to the lane's dword
        dma_u8(static_cast<const uint8_t*>(p.w.absmax) + b,
               __builtin_amdgcn_readfirstlane(lds_addr(sl + 8192 + 256 * wave)));
      } else {
        dma_b32(static_cast<const float*>(p.w.absmax) + b,
                __builtin_amdgcn_readfirstlane(lds_addr(sl + 8192 + 256 * wave)));
      }
    } else if constexpr (NESTED) {
      dma_b32(p.w.nested_absmax + (b >> 8),
              __builtin_amdgcn_readfirstlane(lds_addr(sl + 9216 + 256 * (wave - 4))));
    }
  };
  const uint32_t st_pk = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)w_area)) + 16 * tid;
  const uint32_t st_sc = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)w_area)) + 8192 + 4 * u;
  const uint32_t st_ncode = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)sncode));
  struct Staged {
    u32x4_t pk;
    uint32_t sc, s2;
  };
#define NF4_PP_READ(OFF)                                                                   \
  asm volatile("ds_read_b128 %0, %3 offset:" #OFF "\n\t"                                   \
               "ds_read_b32 %1, %4 offset:" #OFF "\n\t"                                    \
               "ds_read_b32 %2, %4 offset:" #OFF "+1024\n\t"                               \
               "s_waitcnt lgkmcnt(0)"                                                      \
               : "=&v"(r.pk), "=&v"(r.sc), "=&v"(r.s2)                                     \
               : "v"(st_pk), "v"(st_sc)                                                    \
               : "memory")
  auto read_unit = [&](int slot) __attribute__((always_inline)) {
    Staged r;
    static_assert(PP::kWSlot == 10240 && PP::kWSlots == 3, "slot offsets below");
    if (slot == 0) NF4_PP_READ(0);
    else if (slot == 1) NF4_PP_READ(10240);
    else NF4_PP_READ(20480);
    return r;
  };
#undef NF4_PP_READ
  auto b_dst = [&](int buf, int d) -> uint16_t* {
    if constexpr (TRANS) {
      const int row = u % 64, unit = 8 * (u / 64) + 4 * hh + d;
      return b_tile(buf) + row * PP::kBTPitch + 8 * (unit ^ PP::swz_t(row));
    } else {
      return b_tile(buf) + u * BK + 8 * swz(u, 4 * hh + d);
    }
  };
  // The copies issued from inside the first phase of step ci: group g issues
  // activation copy g of step ci + 1, and after the last one (g == 3) the
  // packed-weight and scale copies of step ci + 3 into slot ci % 3 (the
  // slot of step ci, expanded in step ci - 1).  Copies of steps past the end
  // are not issued: a second copy of lines already in flight could let the
  // counted wait below pass before the first one has landed.
  int ci = 0;
  auto dma = [&](int g) __attribute__((always_inline)) {
    if (ci + 1 < n) issue_a(ci + 1, (ci + 1) & 1, g);
    if (g == 3 && ci + 3 < n) {
      issue_wpk(ci + 3, ci % 3);
      issue_ws(ci + 3, ci % 3);
    }
  };
  auto expand = [&](int i, int slot, int buf, bool with_dma) __attribute__((always_inline)) {
    const int kt = kb + (i < n ? i : n - 1);
    const bool valid = unit_valid(own, kt);
    const Staged r = read_unit(slot);
    float a;
    if constexpr (NESTED) {
      float nc;
      asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                   : "=v"(nc) : "v"(st_ncode + 4 * (r.sc & 0xFF)) : "memory");
      a = __fadd_rn(__fmul_rn(nc, __uint_as_float(r.s2)), off);
    } else {
      a = __uint_as_float(r.sc);
    }
    // an invalid unit copied unit 0 of the tensor; a zero scale makes every
    // one of its weights zero
    const Lut lt = make_lut(code, valid ? a : 0.f);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t o[4];
      // input gradient: 8 output columns per dword, in the (0,2,4,6,1,3,5,7)
      // order that the epilogue undoes
      if constexpr (TRANS) expand8_eo(r.pk[d], lt, o);
      else expand8(r.pk[d], lt, o);
      *reinterpret_cast<u32x4_t*>(b_dst(buf, d)) = u32x4_t{o[0], o[1], o[2], o[3]};
      if (with_dma) dma(d);
    }
  };

  // ---- MFMA part ------------------------------------------------------------------
  const int wm = wave >> 2, wn = wave & 3;
  const int r32 = lane & 31, h = lane >> 5;
  f32x16_t acc[PP::MI][PP::NI];
#pragma unroll
  for (int i = 0; i < PP::MI; ++i)
#pragma unroll
    for (int j = 0; j < PP::NI; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  const int y = h ^ ((r32 >> 1) & 7);
  const char* pa[4];
  const char* pb[4];
  const char* pbt[PP::NI][2];     // input gradient: fragment j, rows +0 / +4
  {
    const char* a0 = reinterpret_cast<const char*>(lds) + (wm * PP::WM + r32) * BK * 2;
    const char* b0 = reinterpret_cast<const char*>(lds) + kBOff;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      pa[q] = a0 + 16 * ((2 * q) ^ y);
      if constexpr (!TRANS) pb[q] = b0 + (wn * PP::WN + r32) * BK * 2 + 16 * ((2 * q) ^ y);
    }
    if constexpr (TRANS) {
      // lane: row 8*(tg/2) + ts/4 (+4 for the upper half, +16 per k-slice,
      // which keeps row & 7), columns 16*(tg&1) + 4*(ts&3) of fragment j
      const int tg = lane >> 4, ts = lane & 15;
      const int tr_row = 8 * (tg >> 1) + (ts >> 2);
      const int tr_col = wn * PP::WN + 16 * (tg & 1) + 4 * (ts & 3);
#pragma unroll
      for (int j = 0; j < PP::NI; ++j)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int row = tr_row + 4 * hf, col = tr_col + 32 * j;
          pbt[j][hf] = b0 + (row * PP::kBTPitch + 8 * ((col >> 3) ^ PP::swz_t(row)) + (col & 7)) * 2;
        }
    }
    (void)pb;
  }
  struct Frags {
    bf16x8_t a[PP::MI];
    bf16x8_t b[PP::NI];
  };
  // The transposed reads are one assembly block that waits for its own data:
  // issued through the builtin, each one was preceded by a compiler-inserted
  // vmcnt(0), which waited for the step's copies right after their issue.
  static_assert(!TRANS || PP::NI == 2, "four transposed reads per slice");
  uint32_t tr_addr[2][2];
  if constexpr (TRANS) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) tr_addr[j][hf] = lds_addr(pbt[j][hf]);
  }
  auto load_frags = [&](int stage, int buf, int kk, Frags& f) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PP::MI; ++i)
      f.a[i] = *reinterpret_cast<const bf16x8_t*>(pa[kk & 3] + stage * PP::kAElems * 2 + i * 32 * BK * 2);
    if constexpr (TRANS) {
      const uint32_t off = static_cast<uint32_t>((buf * kBElems + 16 * kk * PP::kBTPitch) * 2);
      u32x2_t l0, h0, l1, h1;
      asm volatile("ds_read_b64_tr_b16 %0, %4\n\t"
                   "ds_read_b64_tr_b16 %1, %5\n\t"
                   "ds_read_b64_tr_b16 %2, %6\n\t"
                   "ds_read_b64_tr_b16 %3, %7\n\t"
                   "s_waitcnt lgkmcnt(0)"
                   : "=&v"(l0), "=&v"(h0), "=&v"(l1), "=&v"(h1)
                   : "v"(tr_addr[0][0] + off), "v"(tr_addr[0][1] + off), "v"(tr_addr[1][0] + off),
                     "v"(tr_addr[1][1] + off)
                   : "memory");
      f.b[0] = __builtin_bit_cast(bf16x8_t, u32x4_t{l0[0], l0[1], h0[0], h0[1]});
      f.b[1] = __builtin_bit_cast(bf16x8_t, u32x4_t{l1[0], l1[1], h1[0], h1[1]});
    } else {
#pragma unroll
      for (int j = 0; j < PP::NI; ++j)
        f.b[j] = *reinterpret_cast<const bf16x8_t*>(pb[kk & 3] + buf * kBElems * 2 + j * 32 * BK * 2);
    }
  };
  // slice 0 of a step's fragments is read ahead, right after the barrier
  // that ends the previous step (fpre)
  Frags fpre;
  auto compute = [&](int stage, int buf, bool with_dma) __attribute__((always_inline)) {
    Frags f0 = fpre, f1;
#pragma unroll
    for (int kk = 0; kk < PP::KK; ++kk) {
      Frags& fc = (kk & 1) ? f1 : f0;
      Frags& fn = (kk & 1) ? f0 : f1;
      if (kk + 1 < PP::KK) load_frags(stage, buf, kk + 1, fn);
#pragma unroll
      for (int i = 0; i < PP::MI; ++i)
#pragma unroll
        for (int j = 0; j < PP::NI; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fc.a[i], fc.b[j], acc[i][j], 0, 0, 0);
      if (with_dma) dma(kk);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // One step in a single pass: k-step kk's 8 MFMAs are interleaved with one
  // piece of the next step's expansion (kk = 0: the byte table; kk > 0: one
  // 8-weight group), and with one of the wave's copy instructions, so that
  // every wave keeps both the MFMA pipe and the VALU busy; the scheduling
  // groups ask for one MFMA followed by a few VALU operations.
  auto mixed = [&](int i, int stage, int buf_r, int slot_w, int buf_w) __attribute__((always_inline)) {
    const int kt = kb + (i + 1 < n ? i + 1 : n - 1);
    const bool valid = unit_valid(own, kt);
    Frags f0, f1;
    load_frags(stage, buf_r, 0, f0);
    const Staged r = read_unit(slot_w);
    float a;
    if constexpr (NESTED) {
      float nc;
      asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                   : "=v"(nc) : "v"(st_ncode + 4 * (r.sc & 0xFF)) : "memory");
      a = __fadd_rn(__fmul_rn(nc, __uint_as_float(r.s2)), off);
    } else {
      a = __uint_as_float(r.sc);
    }
    Lut lt;
#pragma unroll
    for (int kk = 0; kk < PP::KK; ++kk) {
      Frags& fc = (kk & 1) ? f1 : f0;
      Frags& fn = (kk & 1) ? f0 : f1;
      if (kk + 1 < PP::KK) load_frags(stage, buf_r, kk + 1, fn);
#pragma unroll
      for (int ii = 0; ii < PP::MI; ++ii)
#pragma unroll
        for (int j = 0; j < PP::NI; ++j)
          acc[ii][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fc.a[ii], fc.b[j], acc[ii][j], 0, 0, 0);
      if (kk == 0) {
        lt = make_lut(code, valid ? a : 0.f);
      } else {
        uint32_t o[4];
        expand8(r.pk[kk - 1], lt, o);
        *reinterpret_cast<u32x4_t*>(b_dst(buf_w, kk - 1)) = u32x4_t{o[0], o[1], o[2], o[3]};
      }
      dma(kk);
#pragma unroll
      for (int m = 0; m < PP::MI * PP::NI; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // then up to four VALU
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    uint32_t o[4];
    expand8(r.pk[3], lt, o);
    *reinterpret_cast<u32x4_t*>(b_dst(buf_w, 3)) = u32x4_t{o[0], o[1], o[2], o[3]};
  };

  // ---- pipeline -------------------------------------------------------------------
  // Step i multiplies stage/buffer i % 2 and expands step i+1 (slot
  // (i+1) % 3) into the other buffer.  During its first phase every wave
  // issues the activation copy of step i+1, then the weight copies of step
  // i+3.  By the end of the step the activation copy must have landed, and
  // so have the weights of step i+2 (issued one step earlier, so older than
  // that activation copy); the weight copies of step i+3 (kWc per wave, the
  // newest) may stay in flight.  Then one barrier.
  // (assembly: the copies are invisible to the compiler's wait bookkeeping)
  auto wait_vm = [](auto cnt) {
    vm_wait<decltype(cnt)::value>();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  // weight copies per wave and step: packed bytes, plus a scale (waves 0-3)
  // or a nested scale (waves 4-7, nested form only)
  const bool two_w = wave < 4 || NESTED;
  auto end_step = [&](int i) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    if (i + 3 < n) {
      if (two_w) wait_vm(ic<2>{});
      else wait_vm(ic<1>{});
    } else {
      wait_vm(ic<0>{});
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  const bool mfma_first = wave < 4;
  if (n > 0) {
    if constexpr (NESTED) __syncthreads();         // sncode filled
#pragma unroll
    for (int j = 0; j < 4; ++j) issue_a(0, 0, j);
    issue_wpk(0, 0);
    issue_ws(0, 0);
    if (n > 1) {
      issue_wpk(1, 1);
      issue_ws(1, 1);
    }
    if (n > 2) {
      issue_wpk(2, 2);
      issue_ws(2, 2);
      if (two_w) wait_vm(ic<2>{});                // all but the weights of step 2
      else wait_vm(ic<1>{});
    } else {
      wait_vm(ic<0>{});
    }
    __syncthreads();                               // every wave's copies of steps 0 and 1 landed
    expand(0, 0, 0, false);
    __syncthreads();
    if constexpr (TRANS) load_frags(0, 0, 0, fpre);
    auto step = [&](int i, auto ph) __attribute__((always_inline)) {
      constexpr int P = decltype(ph)::value;
      ci = i;
      if constexpr (!TRANS) {
        mixed(i, P & 1, P & 1, (i + 1) % 3, (P + 1) & 1);
      } else {
        // the input gradient measured faster with the two halves of a step
        // run as separate phases, in opposite order on the two waves of a
        // SIMD (w and w + 4): one wave's expansion under the other's MFMAs
        if (!mfma_first) expand(i + 1, (i + 1) % 3, (P + 1) & 1, true);
        __builtin_amdgcn_sched_barrier(0);
        compute(P & 1, P & 1, mfma_first);
        __builtin_amdgcn_sched_barrier(0);
        if (mfma_first) expand(i + 1, (i + 1) % 3, (P + 1) & 1, false);
      }
      end_step(i);
      // slice 0 of step i+1 (a harmless re-read of landed data after the last step)
      if constexpr (TRANS) load_frags((P + 1) & 1, (P + 1) & 1, 0, fpre);
    };
    int i = 0;
    for (; i + 2 <= n; i += 2) {
      step(i, ic<0>{});
      step(i + 1, ic<1>{});
    }
    if (i < n) step(i, ic<0>{});
  }

  // ---- epilogue -------------------------------------------------------------------
#pragma unroll
  for (int i = 0; i < PP::MI; ++i) {
#pragma unroll
    for (int j = 0; j < PP::NI; ++j) {
      int64_t col = col0 + wn * PP::WN + 32 * j + r32;
      // input gradient: tile column c is output column 8 (c / 8) + pi(c % 8)
      if constexpr (TRANS) col = (col & ~int64_t{7}) | (((col & 3) << 1) | ((col >> 2) & 1));
      if (col >= Nc) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = row0 + wm * PP::WM + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
        if (row >= row_end) continue;
        if (p.splits == 1) {
          p.C[row * Nc + col] = to_bf16(acc[i][j][v]);
        } else {
          p.partial[(static_cast<int64_t>(z) * p.M + row) * Nc + col] = acc[i][j][v];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// Forward, 256 x 256, with the expanded weights kept in registers.
//
// The eight waves split the tile by columns only: wave w owns output columns
// (W rows) 32w .. 32w+31 for all 256 rows, 8 accumulators of 32x32.  Lane l
// expands W row 32w + l%32, half h = l/32 of the step's 64-block, i.e. 32
// consecutive weights = one 16-byte load = the MFMA B operands of all four
// 16-deep k slices of the step: slice kk pairs lane half h with contraction
// indices 32h + 8kk .. +7, and the activation fragments are read with the
// same pairing (any fixed assignment of contraction indices to the two lane
// halves gives the same sum).  No weight tile goes through LDS, so LDS holds
// a 3-deep activation ring (each copy has two steps to land) and a 3-deep
// ring of per-wave weight slots, which only the wave that copied them reads.
// One barrier per step: every wave's activation copy of step i has landed
// (own vmcnt, then the barrier) and every wave has finished reading the
// stage that the step's new copy overwrites.
template <int WAVES>
struct RB {
  static constexpr int BM = 256, BN = 32 * WAVES, BK = 64;
  static constexpr int kThreads = 64 * WAVES;
  static constexpr int kStages = 3;
  static constexpr int kAElems = BM * BK;              // bf16 per activation stage (32 KB)
  static constexpr int kARows = BM / WAVES;            // activation rows each wave copies
  static constexpr int kWWave = 1536;                  // per wave: 1 KB packed, 256 B scale, 256 B nested
  static constexpr int kWSlot = WAVES * kWWave;
  static constexpr int kWOff = kStages * kAElems * 2;  // 96 KB
  static constexpr int kLds = kWOff + kStages * kWSlot;
};
static_assert(RB<8>::kLds + 1024 <= 160 * 1024, "LDS budget of one workgroup");

template <int WAVES, bool NESTED, bool GROUPED>
__global__ __launch_bounds__(64 * WAVES, 1) void k_rb(GemmParams p) {
  using R = RB<WAVES>;
  constexpr int BM = R::BM, BN = R::BN, BK = R::BK;
  constexpr int kAJ = R::kARows / 8;               // activation copy instructions per wave
  // per-wave copy instructions of one step: activation, packed, scale (+ nested)
  constexpr int kWCopies = NESTED ? 3 : 2;          // packed, scale (+ nested)
  constexpr int kCopies = kAJ + kWCopies;
  static_assert(2 * kCopies <= 63, "outstanding copies fit the vmcnt field");
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  __shared__ float sncode[256];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int64_t N = p.w.N, K = p.w.K;
  const int ktiles = static_cast<int>((K + BK - 1) / BK);

  int mt, ct, z;
  tile_coords(xcd_tile(blockIdx.x, gridDim.x), gridDim.x, p.m_tiles, p.splits, mt, ct, z);
  const int64_t col0 = static_cast<int64_t>(ct) * BN;
  int64_t row0, row_end, wrow_base;
  if (!row_tile<BM, GROUPED>(p, mt, N, row0, row_end, wrow_base)) return;
  const int kb = static_cast<int>(static_cast<int64_t>(z) * ktiles / p.splits);
  const int ke = static_cast<int>(static_cast<int64_t>(z + 1) * ktiles / p.splits);
  const int n = ke - kb;

  if constexpr (NESTED) {
    if (tid < 256) sncode[tid] = p.w.ncode[tid];
  }
  float code[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) code[i] = p.w.code[i];
  const float off = NESTED ? p.w.nested_offset[0] : 0.f;

  // ---- activation copies: wave w copies rows kARows*w .. +kARows-1, 8 rows
  // per instruction, 16-byte units swizzled (swz) as the fragment reads expect
  const int a_r_in = lane >> 3, a_unit = lane & 7;
  const uint16_t* a_row_ptr[kAJ];
  int a_colofs[kAJ];
#pragma unroll
  for (int j = 0; j < kAJ; ++j) {
    const int r = R::kARows * wave + 8 * j + a_r_in;
    int64_t row = row0 + r;
    row = row < row_end ? row : row_end - 1;
    a_row_ptr[j] = p.A + row * K;
    a_colofs[j] = 8 * swz(r, a_unit);
  }
  auto stage_ptr = [&](int stage) { return lds + stage * R::kAElems; };
  // copy j (8 rows) of the wave's part of the activation tile of step i < n
  auto issue_a_one = [&](int i, int stage, int j) __attribute__((always_inline)) {
    const int64_t c0 = static_cast<int64_t>(kb + i) * BK;
    int64_t col = c0 + a_colofs[j];
    col = col < K ? col : K - 8;
    const uint16_t* src = a_row_ptr[j] + col;
    __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(stage_ptr(stage) + (R::kARows * wave + 8 * j) * BK), 16, 0, 0);
  };
  auto issue_a = [&](int i, int stage) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kAJ; ++j) issue_a_one(i, stage, j);
  };

  // ---- weight copies: lane l fetches the 16 bytes it expands (W row
  // col0 + 32w + l%32, half l/32 of block kt), that row's block scale and, when
  // nested, the scale's nested scale, into the wave's part of a slot
  const int r32 = lane & 31, h = lane >> 5;
  const int64_t wrow = col0 + 32 * wave + r32;
  const bool row_ok = wrow < N;
  const int64_t wrow_g = wrow_base + wrow;
  const uint8_t* const pk_base = p.w.packed + ((wrow_g * K) >> 1) + 16 * h;
  const int64_t blocks_per_row = K / BK;
  char* const w_area = reinterpret_cast<char*>(lds) + R::kWOff;
  auto issue_w = [&](int i, int slot) __attribute__((always_inline)) {   // step i < n
    const int kt = kb + i;
    char* sl = w_area + slot * R::kWSlot + wave * R::kWWave;
    const uint8_t* src = row_ok ? pk_base + static_cast<int64_t>(kt) * (BK / 2) : p.w.packed;
    __builtin_amdgcn_global_load_lds(src, (lds_void_t*)sl, 16, 0, 0);
    const int64_t b = row_ok ? wrow_g * blocks_per_row + kt : 0;
    if constexpr (NESTED) {
      const uint8_t* sa = static_cast<const uint8_t*>(p.w.absmax) + b;
      __builtin_amdgcn_global_load_lds(sa, (lds_void_t*)(sl + 1024), 1, 0, 0);
      const float* sn = p.w.nested_absmax + (b >> 8);
      __builtin_amdgcn_global_load_lds(sn, (lds_void_t*)(sl + 1280), 4, 0, 0);
    } else {
      const float* sa = static_cast<const float*>(p.w.absmax) + b;
      __builtin_amdgcn_global_load_lds(sa, (lds_void_t*)(sl + 1024), 4, 0, 0);
    }
  };
  const uint32_t st_pk = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)w_area)) +
                         wave * R::kWWave + 16 * lane;
  const uint32_t st_sc = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)w_area)) +
                         wave * R::kWWave + 1024 + 4 * lane;
  const uint32_t st_ncode = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)sncode));
  struct Staged {
    u32x4_t pk;
    uint32_t sc, s2;
  };
  auto read_unit = [&](auto slot_c) __attribute__((always_inline)) {
    constexpr int off = decltype(slot_c)::value * R::kWSlot;
    static_assert(2 * R::kWSlot + 256 < 65536, "slot offsets fit the ds immediate");
    Staged r;
    asm volatile("ds_read_b128 %0, %3 offset:%5\n\t"
                 "ds_read_b32 %1, %4 offset:%5\n\t"
                 "ds_read_b32 %2, %4 offset:%6\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r.pk), "=&v"(r.sc), "=&v"(r.s2)
                 : "v"(st_pk), "v"(st_sc), "i"(off), "i"(off + 256)
                 : "memory");
    if constexpr (!NESTED) r.s2 = 0;
    return r;
  };
  auto unit_scale = [&](const Staged& r) __attribute__((always_inline)) {
    float a;
    if constexpr (NESTED) {
      float nc;
      asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                   : "=v"(nc) : "v"(st_ncode + 4 * (r.sc & 0xFF)) : "memory");
      a = __fadd_rn(__fmul_rn(nc, __uint_as_float(r.s2)), off);
    } else {
      a = __uint_as_float(r.sc);
    }
    return row_ok ? a : 0.f;     // rows past N expand to zero
  };

  // ---- MFMA operands ---------------------------------------------------------------
  f32x16_t acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;
  // activation fragment of slice kk, row block mi: row 32mi + r32, logical
  // 16-byte unit 4h + kk (contraction 32h + 8kk .. +7), stored at unit ^ swz
  int a_ofs[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) a_ofs[kk] = r32 * BK * 2 + 16 * swz(r32, 4 * h + kk);
  auto load_a = [&](int stage, int kk, bf16x8_t (&f)[8]) __attribute__((always_inline)) {
    const char* base = reinterpret_cast<const char*>(stage_ptr(stage)) + a_ofs[kk];
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) f[mi] = *reinterpret_cast<const bf16x8_t*>(base + mi * 32 * BK * 2);
  };
  bf16x8_t bw[4];      // B operands of the step being multiplied, slice kk in bw[kk]

  // s_waitcnt on vmcnt only (expcnt and lgkmcnt fields at their maximum)
  auto wait_vm = [](auto cnt) {
    constexpr int c = decltype(cnt)::value;
    __builtin_amdgcn_s_waitcnt((c & 15) | ((c >> 4) << 14) | (7 << 4) | (15 << 8));
  };

  // ---- pipeline ---------------------------------------------------------------------
  // Copies of step j: the activation tile during step j-2, the weights during
  // step j-3 (the prologue issues W0 A0 W1 A1 W2).  Only copies of steps that
  // exist are issued: a second copy of bytes already in flight could let a
  // counted wait pass before the first one has landed, so every wait below
  // counts exactly the copies issued after the one it needs.  Within a step
  // the copies go out between the MFMA groups of its slices (activation
  // copies in slices 0-2, the weights in slice 3): issued in one burst at the
  // step's start they held the wave at the issue for ~800 of ~3000 cycles
  // per step (per-phase timestamps), with no MFMA in flight.
  if (n > 0) {
    if constexpr (NESTED) __syncthreads();         // sncode filled, before any copy is in flight
    issue_w(0, 0);
    issue_a(0, 0);
    if (n > 1) {
      issue_w(1, 1);
      issue_a(1, 1);
    }
    if (n > 2) issue_w(2, 2);
    // weights of step 0 landed (issued after them: A0, and W1 A1 W2 where they exist)
    if (n > 2) wait_vm(ic<2 * kCopies>{});
    else if (n > 1) wait_vm(ic<kAJ + kCopies>{});
    else wait_vm(ic<kAJ>{});
    {
      const Staged r = read_unit(ic<0>{});
      const Lut lt = make_lut(code, unit_scale(r));
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t o[4];
        expand8(r.pk[d], lt, o);
        bw[d] = __builtin_bit_cast(bf16x8_t, u32x4_t{o[0], o[1], o[2], o[3]});
      }
    }

    // Step i: the activation fragments of slice 0 were read at the end of
    // step i-1; slice kk's 8 MFMAs run with the reads of slice kk+1 in flight
    // and, interleaved, one piece of step i+1's expansion.  After the last
    // MFMAs are issued the wave waits for its part of A(i+1), joins the
    // barrier and reads slice 0 of step i+1 while those MFMAs still run.
    bf16x8_t f0[8], f1[8];
    // own part of A(0) landed (W1 A1 W2 may fly)
    if (n > 2) wait_vm(ic<kAJ + 2 * kWCopies>{});
    else if (n > 1) wait_vm(ic<kCopies>{});
    else wait_vm(ic<0>{});
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    load_a(0, 0, f0);
    // FULL: a step with three more after it (every copy below exists; no
    // branch splits its slices)
    auto step = [&](int i, auto ph, auto full_c) __attribute__((always_inline)) {
      constexpr int P = decltype(ph)::value;       // i % 3
      constexpr bool FULL = decltype(full_c)::value;
      __builtin_amdgcn_sched_barrier(0);
      // weights of step i+1 landed (issued after them: A(i+1), W(i+2) where it exists)
      if (FULL || i + 2 < n) wait_vm(ic<kCopies>{});
      else if (i + 1 < n) wait_vm(ic<kAJ>{});
      asm volatile("" ::: "memory");
      const Staged r = read_unit(ic<(P + 1) % 3>{});
      // the nested-scale lookup waits on LDS: do it before the slice-1
      // fragment reads are in flight
      const float a_next = unit_scale(r);
      Lut lt;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        bf16x8_t (&fc)[8] = (kk & 1) ? f1 : f0;
        bf16x8_t (&fn)[8] = (kk & 1) ? f0 : f1;
        if (kk + 1 < 4) load_a(P, kk + 1, fn);
#pragma unroll
        for (int mi = 0; mi < 8; ++mi)
          acc[mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bw[kk], fc[mi], acc[mi], 0, 0, 0);
        if (kk == 0) {
          lt = make_lut(code, a_next);
        } else {
          uint32_t o[4];
          expand8(r.pk[kk - 1], lt, o);
          bw[kk - 1] = __builtin_bit_cast(bf16x8_t, u32x4_t{o[0], o[1], o[2], o[3]});
        }
        // this slice's share of the copies of step i: activation copies j
        // with 3 j / kAJ == kk of A(i+2), in slice 3 the weights of step i+3
        if (kk < 3 && (FULL || i + 2 < n)) {
#pragma unroll
          for (int j = 0; j < kAJ; ++j)
            if ((3 * j) / kAJ == kk) issue_a_one(i + 2, (P + 2) % 3, j);
        }
        if (kk == 3 && (FULL || i + 3 < n)) issue_w(i + 3, P);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // a copy, while there are any
          __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // then up to five VALU
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      {
        uint32_t o[4];
        expand8(r.pk[3], lt, o);
        bw[3] = __builtin_bit_cast(bf16x8_t, u32x4_t{o[0], o[1], o[2], o[3]});
      }
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
      // own part of A(i+1) landed: issued after it, W(i+2), A(i+2) and W(i+3)
      // where they exist
      if (FULL || i + 3 < n) wait_vm(ic<kCopies + kWCopies>{});
      else if (i + 2 < n) wait_vm(ic<kCopies>{});
      else wait_vm(ic<0>{});
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      load_a((P + 1) % 3, 0, f0);                  // slice 0 of step i+1 (a re-read on the last step)
    };
    int i = 0;
    for (; i + 6 <= n; i += 3) {                   // steps i .. i+2 each have three more after them
      step(i, ic<0>{}, std::true_type{});
      step(i + 1, ic<1>{}, std::true_type{});
      step(i + 2, ic<2>{}, std::true_type{});
    }
    for (; i + 3 <= n; i += 3) {
      step(i, ic<0>{}, std::false_type{});
      step(i + 1, ic<1>{}, std::false_type{});
      step(i + 2, ic<2>{}, std::false_type{});
    }
    if (i < n) step(i, ic<0>{}, std::false_type{});
    if (i + 1 < n) step(i + 1, ic<1>{}, std::false_type{});
    wait_vm(ic<0>{});                              // no copy outlives the workgroup
  }

  // ---- epilogue -----------------------------------------------------------------------
  // The MFMAs take the weights as the first operand, so accumulator mi holds
  // the transposed 32 x 32 block: lane l has output row 32mi + l%32 and, for
  // register v, column 32w + 8(v/4) + 4h + v%4 -- four consecutive columns
  // per register group, stored as one 8-byte (bf16) or 16-byte (fp32) write.
  const int64_t ncol0 = col0 + 32 * wave + 4 * h;
  const bool vec_ok = (N & 3) == 0 &&
                      (reinterpret_cast<uintptr_t>(p.splits == 1 ? static_cast<void*>(p.C)
                                                                 : static_cast<void*>(p.partial)) &
                       15) == 0;
#pragma unroll
  for (int mi = 0; mi < 8; ++mi) {
    const int64_t row = row0 + 32 * mi + r32;
    if (row >= row_end) continue;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t col = ncol0 + 8 * g;
      if (col >= N) continue;
      const float v0 = acc[mi][4 * g], v1 = acc[mi][4 * g + 1], v2 = acc[mi][4 * g + 2], v3 = acc[mi][4 * g + 3];
      if (p.splits == 1) {
        uint16_t* dst = p.C + row * N + col;
        if (vec_ok && col + 3 < N) {
          *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
        } else {
          const float vv[4] = {v0, v1, v2, v3};
          for (int c = 0; c < 4 && col + c < N; ++c) dst[c] = to_bf16(vv[c]);
        }
      } else {
        float* dst = p.partial + (static_cast<int64_t>(z) * p.M + row) * N + col;
        if (vec_ok && col + 3 < N) {
          *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{v0, v1, v2, v3};
        } else {
          const float vv[4] = {v0, v1, v2, v3};
          for (int c = 0; c < 4 && col + c < N; ++c) dst[c] = vv[c];
        }
      }
    }
  }
}

// Fixed-order sum of split partials: out = bf16(sum_{s=0}^{S-1} part[s]).
// Four outputs per thread; n % 4 tails handled one by one.
__global__ __launch_bounds__(kThreads) void k_splitk_reduce(const float* __restrict__ part,
                                                            int splits, int64_t n,
                                                            uint16_t* __restrict__ out) {
  const int64_t i4 = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) * 4;
  if (i4 >= n) return;
  // All S partials are loaded before the first add (one memory round trip
  // instead of S dependent ones), then summed in the order s = 0 .. S-1.
  auto sum_all = [&](auto s_c) __attribute__((always_inline)) {
    constexpr int S = decltype(s_c)::value;
    f32x4_t v[S];
#pragma unroll
    for (int z = 0; z < S; ++z) v[z] = *reinterpret_cast<const f32x4_t*>(part + static_cast<int64_t>(z) * n + i4);
    f32x4_t s = v[0];
#pragma unroll
    for (int z = 1; z < S; ++z)
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] = __fadd_rn(s[e], v[z][e]);
    const uint32_t lo = pack_bf16x2(s[0], s[1]), hi = pack_bf16x2(s[2], s[3]);
    *reinterpret_cast<u32x2_t*>(out + i4) = u32x2_t{lo, hi};
  };
  if (i4 + 4 <= n && (n & 3) == 0 && splits >= 2 && splits <= 8) {
    switch (splits) {
      case 2: sum_all(std::integral_constant<int, 2>{}); break;
      case 3: sum_all(std::integral_constant<int, 3>{}); break;
      case 4: sum_all(std::integral_constant<int, 4>{}); break;
      case 5: sum_all(std::integral_constant<int, 5>{}); break;
      case 6: sum_all(std::integral_constant<int, 6>{}); break;
      case 7: sum_all(std::integral_constant<int, 7>{}); break;
      default: sum_all(std::integral_constant<int, 8>{}); break;
    }
  } else if (i4 + 4 <= n && (n & 3) == 0) {
    f32x4_t s = *reinterpret_cast<const f32x4_t*>(part + i4);
    for (int z = 1; z < splits; ++z) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(part + static_cast<int64_t>(z) * n + i4);
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] = __fadd_rn(s[e], v[e]);
    }
    const uint32_t lo = pack_bf16x2(s[0], s[1]), hi = pack_bf16x2(s[2], s[3]);
    *reinterpret_cast<u32x2_t*>(out + i4) = u32x2_t{lo, hi};
  } else {
    for (int64_t i = i4; i < n && i < i4 + 4; ++i) {
      float s = part[i];
      for (int z = 1; z < splits; ++z) s = __fadd_rn(s, part[static_cast<int64_t>(z) * n + i]);
      out[i] = to_bf16(s);
    }
  }
}

// ---------------------------------------------------------------------------------
// Register-staged tile kernel: the 8-bit blockwise formats, and NF4 tiles of
// 32 to 128 rows (grouped experts, small products).
//
// 8-bit: the weight is one index per byte into a 256-entry table
// (bitsandbytes fork PR "Experts trainability ... ExpertsNbit", "Commit 1":
// int8 and fp8 e4m3 blockwise beside nf4 / fp4), w_hat =
// bf16(fp32(code[q] * absmax_hat)) with the same 64-element blocks and
// (nested) scales.  A 256-entry table per (row, block) does not fit the
// register byte tables, so the table (256 fp32) sits in LDS and each weight
// costs one LDS lookup, one fp32 multiply and half a packed conversion.
// NF4: each thread expands one whole (row, 64-block) per step through the
// register byte tables (one table per block), in the (0,2,4,6,1,3,5,7) order
// of expand8_eo; the forward stores its activation tile in the same order,
// the input gradient maps the output column back in the epilogue.
//
// Tile BM x 128 (BM = 128, 64 or 32), BK = 64 (8-bit) or 128 (NF4): every
// thread owns 32 weight bytes of a step.  Four waves (2 x 2 of 64 x 64, or
// 1 x 4 of BM x 32), or eight (NF4: 2 x 4 of 64 x 32 or 32 x 32), with
// v_mfma_f32_32x32x16_bf16.  NF4 also as 128 x 256 with eight waves of
// 64 x 64 and BK = 64: per MFMA two thirds of the fragment reads of the
// 128 x 128 eight-wave tile, whose LDS reads bound its multiply part; its
// grouped form serves experts of up to 128 rows.  Every step the threads load
// the next step's activation vectors and weight bytes into registers, the
// waves multiply the current LDS buffers, and the threads then store the
// activations and expand their weights into the other buffer; one barrier
// per step.  A tile and the forward's weight tile are stored [row][BK + 8],
// so every MFMA fragment is one 16-byte read; the 8-bit input gradient
// stores its weights one element per output-column row, the NF4 input
// gradient [contraction][128 + 16] (whole 16-byte stores), read with
// ds_read_b64_tr_b16 as in the producer/consumer kernel.
template <int BITS, int BM, int NW, int BN_ = 128>
struct GT {
  static_assert(NW == 4 || (NW == 8 && BITS == 4 && BM >= 64), "8 waves: NF4, 64 or 128 rows");
  static_assert(BN_ == 128 || (BN_ == 256 && BITS == 4 && NW == 8 && BM == 128),
                "256 columns: NF4, 8 waves, 128 rows");
  static constexpr int kThreads = 64 * NW;
  // 256 columns take 64-deep steps: two buffers of 128 x 128 and 256 x 128
  // would not fit the LDS
  static constexpr int BN = BN_, BK = (BITS == 8 || BN_ == 256) ? 64 : 128, kPitch = BK + 8, kPitchT = BN + 16;
  static constexpr int WAVES_M = (BM == 128 || NW == 8) ? 2 : 1, WAVES_N = NW / WAVES_M;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int MI = WM / 32, NI = WN / 32;
  // weights per thread piece: 32 bytes (4 waves), 16 bytes of NF4 (8 waves)
  static constexpr int PW = BITS == 8 ? 32 : (NW == 8 ? 32 : 64);
  static constexpr int kUnits = PW * BITS / 32;                // packed dwords per piece
  static constexpr int kVR = BK / 8;                           // 16-byte activation vectors per row
  static constexpr int kA = BM * kPitch;                       // elements per buffer
  static constexpr int kAVec = BM * BK / 8 / kThreads;         // activation vectors per thread
  static constexpr int kDepth = 4;                             // steps held in registers
  static constexpr bool kTrRead(bool trans) { return trans; }
  // Eight waves: the transposed tile has unpadded rows whose 16-byte units
  // are XOR-swizzled by the row (256 columns: as in the ping-pong kernel; 128
  // columns: unit ^ 5 (row & 3)), so that the expansion's 16-byte writes (16
  // lanes) and the transposed 8-byte reads (32 lanes) each hit 64 distinct
  // banks.  Measured on the padded pitch (BN + 16): both were 2-way
  // conflicted, and the conflicts were more than half of the 128 x 256 input
  // gradient's LDS cycles.
  static constexpr bool kSwzT = NW == 8;
  static __device__ __forceinline__ int swz(int r) {
    if constexpr (BN_ == 256) return PP::swz_t(r);
    else return 5 * (r & 3);
  }
  static constexpr int kB(bool trans) {
    return kTrRead(trans) ? BK * (kSwzT ? BN : kPitchT) : BN * kPitch;
  }
  static constexpr int kLds(bool trans) { return 2 * (kA + kB(trans)) * 2; }
};

template <int BITS, int BM, int NW, int BN_, bool TRANS, bool NESTED, bool GROUPED>
__global__ __launch_bounds__(64 * NW) void k_gemmt(GemmParams p) {
  using G = GT<BITS, BM, NW, BN_>;
  constexpr int BN = G::BN, BK = G::BK, P = G::kPitch;
  constexpr bool TR = G::kTrRead(TRANS);
  constexpr bool SWZ = TR && G::kSwzT;
  constexpr int PT = SWZ ? BN : G::kPitchT;             // row pitch of the transposed tile
  constexpr int KB = G::kB(TRANS);
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  __shared__ float scode[BITS == 8 ? 256 : 1];
  __shared__ float sncode[256];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int64_t N = p.w.N, K = p.w.K;
  const int64_t Nc = TRANS ? K : N;
  const int64_t Kc = TRANS ? N : K;
  const int ktiles = static_cast<int>((Kc + BK - 1) / BK);

  int mt, ct, z;
  if constexpr (GROUPED) {
    // An expert's weight tiles serve only its own rows, while its activation
    // rows are shared by all of its column tiles: XCD x (workgroups are
    // dealt to the 8 XCDs in turn) serves row tiles x, x + 8, ..., each
    // with all its column tiles in a row, so those activations are fetched
    // into one L2.  m_tiles is a multiple of 8 here and splits = 1.
    const int idx = static_cast<int>(blockIdx.x >> 3), nct = static_cast<int>(gridDim.x) / p.m_tiles;
    mt = 8 * (idx / nct) + static_cast<int>(blockIdx.x & 7);
    const int cz = idx % nct;
    z = cz % p.splits;
    ct = cz / p.splits;
  } else {
    tile_coords(xcd_tile(blockIdx.x, gridDim.x), gridDim.x, p.m_tiles, p.splits, mt, ct, z);
  }
  const int64_t col0 = static_cast<int64_t>(ct) * BN;
  int64_t row0, row_end, wrow_base;
  if (!row_tile<BM, GROUPED>(p, mt, N, row0, row_end, wrow_base)) return;
  const int kb = static_cast<int>(static_cast<int64_t>(z) * ktiles / p.splits);
  const int ke = static_cast<int>(static_cast<int64_t>(z + 1) * ktiles / p.splits);
  const int n = ke - kb;

  float code[BITS == 4 ? 16 : 1];
  if constexpr (BITS == 8) {
    if (tid < 256) scode[tid] = p.w.code[tid];
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) code[i] = p.w.code[i];
  }
  if constexpr (NESTED) {
    if (tid < 256) sncode[tid] = p.w.ncode[tid];
  }
  const float off = NESTED ? p.w.nested_offset[0] : 0.f;

  auto a_buf = [&](int b) { return lds + b * G::kA; };
  auto b_buf = [&](int b) { return lds + 2 * G::kA + b * KB; };

  // ---- this thread's loads ---------------------------------------------------------
  // activation vector j: row (tid + T j) / kVR, 16-byte unit (tid + T j) %
  // kVR (T threads); rows past the end repeat the last row, columns past Kc
  // repeat the last vector (they meet zero weights or are never stored)
  const uint16_t* a_row[G::kAVec];
  int a_c8[G::kAVec], a_dst[G::kAVec];
#pragma unroll
  for (int j = 0; j < G::kAVec; ++j) {
    const int u = tid + G::kThreads * j;
    const int r = u / G::kVR;
    int64_t row = row0 + r;
    row = row < row_end ? row : row_end - 1;
    a_row[j] = p.A + row * Kc;
    a_c8[j] = 8 * (u % G::kVR);
    a_dst[j] = r * P + a_c8[j];
  }
  // weights: thread piece = PW weights of one W row (kUnits packed dwords).
  // Forward: W row col0 + tid / kTpr, contraction PW (tid % kTpr) .. of the
  // step.  Input gradient: W row (contraction) of the step tid / kTpr, output
  // columns col0 + PW (tid % kTpr) ..  Invalid pieces read byte 0 of the
  // tensor and get a zero scale.
  constexpr int kTpr = (TRANS ? BN : BK) / G::PW;       // threads per W row of the step
  static_assert(kTpr * (TRANS ? BK : BN) == G::kThreads, "one piece per thread");
  // (swizzled 256-column transposed tile: thread t takes half t & 1 of unit
  // t >> 1, W row (t >> 1) % 64 of the step, columns 64 ((t >> 1) / 64) +
  // 32 (t & 1), the write pattern its swizzle spreads over distinct banks;
  // 128 columns keep the mapping below, four threads per W row)
  constexpr bool kPPMap = SWZ && BN == 256;
  static_assert(!kPPMap || (kTpr == 8 && BK == 64 && G::kThreads == 512), "swizzled mapping below");
  static_assert(!SWZ || kPPMap || kTpr == 4, "128-column swizzle: four threads per W row");
  const int wl = kPPMap ? ((tid >> 1) & 63) : tid / kTpr;
  const int wq = kPPMap ? (((tid >> 7) << 1) | (tid & 1)) : tid % kTpr;
  const int64_t kblocks = K / 64;
  struct Regs {
    u32x4_t a[G::kAVec];
    u32x4_t w0, w1;
    uint32_t sc, s2;
    bool ok;
  };
  auto load = [&](int i, Regs& r) __attribute__((always_inline)) {
    const int kt = kb + i;
    const int64_t c = static_cast<int64_t>(kt) * BK;
#pragma unroll
    for (int j = 0; j < G::kAVec; ++j) {
      const int64_t cc = c + a_c8[j];
      r.a[j] = *reinterpret_cast<const u32x4_t*>(a_row[j] + (cc + 8 <= Kc ? cc : Kc - 8));
    }
    int64_t wrow, wcol;
    if constexpr (TRANS) {
      wrow = static_cast<int64_t>(kt) * BK + wl;
      wcol = col0 + G::PW * wq;
    } else {
      wrow = col0 + wl;
      wcol = static_cast<int64_t>(kt) * BK + G::PW * wq;
    }
    r.ok = wrow < N && wcol < K;
    const int64_t grow = wrow_base + (r.ok ? wrow : 0);
    const int64_t e0 = r.ok ? grow * K + wcol : 0;
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(p.w.packed + (BITS == 8 ? e0 : e0 / 2));
    r.w0 = src[0];
    if constexpr (G::kUnits == 8) r.w1 = src[1];
    const int64_t b = r.ok ? grow * kblocks + (wcol >> 6) : 0;
    if constexpr (NESTED) {
      r.sc = static_cast<const uint8_t*>(p.w.absmax)[b];
      r.s2 = __float_as_uint(p.w.nested_absmax[b >> 8]);
    } else {
      r.sc = __float_as_uint(static_cast<const float*>(p.w.absmax)[b]);
      r.s2 = 0;
    }
  };
  // The staging of one step is split into units so that it can run between
  // the MFMAs of the step before: activation vector j, and weight unit d
  // (packed dword d of the piece: 8 NF4 weights or 4 8-bit weights).
  auto store_a = [&](int buf, const Regs& r, int j) __attribute__((always_inline)) {
    u32x4_t v = r.a[j];
    if constexpr (BITS == 4 && !TRANS)    // the contraction order of expand8_eo
      v = u32x4_t{perm(v[1], v[0], 0x05040100u), perm(v[3], v[2], 0x05040100u),
                  perm(v[1], v[0], 0x07060302u), perm(v[3], v[2], 0x07060302u)};
    *reinterpret_cast<u32x4_t*>(a_buf(buf) + a_dst[j]) = v;
  };
  auto wscale = [&](const Regs& r) __attribute__((always_inline)) {
    float a;
    // r.sc is a zero-extended byte here (loaded as uint8_t above)
    if constexpr (NESTED) a = __fadd_rn(__fmul_rn(sncode[r.sc], __uint_as_float(r.s2)), off);
    else a = __uint_as_float(r.sc);
    return r.ok ? a : 0.f;
  };
  auto store_w = [&](int buf, const Regs& r, const Lut& lt, float a, int d) __attribute__((always_inline)) {
    uint16_t* bb = b_buf(buf);
    const uint32_t wd = d < 4 ? r.w0[d] : r.w1[d - 4];
    if constexpr (BITS == 8) {
      const uint32_t o0 = pack_bf16x2(__fmul_rn(scode[wd & 0xFFu], a), __fmul_rn(scode[(wd >> 8) & 0xFFu], a));
      const uint32_t o1 = pack_bf16x2(__fmul_rn(scode[(wd >> 16) & 0xFFu], a), __fmul_rn(scode[wd >> 24], a));
      if constexpr (TRANS) {
        // element 4 d + e of the piece is W_hat[row wl, column PW wq + 4 d + e]:
        // four consecutive columns of contraction row wl of the [k][n] tile,
        // which the transposed fragment reads take apart (as for NF4)
        static_assert(TR && !SWZ, "8-bit input gradient: padded [k][n] tile");
        *reinterpret_cast<u32x2_t*>(bb + wl * PT + G::PW * wq + 4 * d) = u32x2_t{o0, o1};
      } else {
        *reinterpret_cast<u32x2_t*>(bb + wl * P + 32 * wq + 4 * d) = u32x2_t{o0, o1};
      }
    } else {
      uint32_t o[4];
      expand8_eo(wd, lt, o);
      uint16_t* dst;
      if constexpr (SWZ) dst = bb + wl * PT + 8 * ((4 * wq + d) ^ G::swz(wl));
      else dst = (TRANS ? bb + wl * PT + G::PW * wq : bb + wl * P + G::PW * wq) + 8 * d;
      *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{o[0], o[1], o[2], o[3]};
    }
  };
  auto make_table = [&](float a) __attribute__((always_inline)) {
    if constexpr (BITS == 4) return make_lut(code, a);
    else return Lut{};
  };
  auto store = [&](int buf, const Regs& r) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < G::kAVec; ++j) store_a(buf, r, j);
    const float a = wscale(r);
    const Lut lt = make_table(a);
#pragma unroll
    for (int d = 0; d < G::kUnits; ++d) store_w(buf, r, lt, a, d);
  };

  // ---- MFMA part ------------------------------------------------------------------
  const int wm = wave / G::WAVES_N, wn = wave % G::WAVES_N;
  const int r32 = lane & 31, h = lane >> 5;
  f32x16_t acc[G::MI][G::NI];
#pragma unroll
  for (int i = 0; i < G::MI; ++i)
#pragma unroll
    for (int j = 0; j < G::NI; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  // transposed-read lane offsets: rows 8 (g >> 1) + (s >> 2) (+ 4 for the
  // upper half; + 16 per slice, which keeps row & 7 and so the swizzle),
  // columns 16 (g & 1) + 4 (s & 3) of 32-column fragment j (g = lane / 16,
  // s = lane % 16)
  int tr_o[G::NI][2];
#pragma unroll
  for (int j = 0; j < G::NI; ++j)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int row = 8 * ((lane >> 4) >> 1) + ((lane & 15) >> 2) + 4 * hf;
      const int col = wn * G::WN + 16 * ((lane >> 4) & 1) + 4 * (lane & 3) + 32 * j;
      tr_o[j][hf] = SWZ ? row * PT + 8 * ((col >> 3) ^ G::swz(row)) + (col & 7) : row * PT + col;
    }
  // a wave whose rows all lie past the tile's last row skips its MFMAs
  const bool active = row0 + wm * G::WM < row_end;
  struct Frags {
    bf16x8_t a[G::MI], b[G::NI];
  };
  auto read_frags = [&](int buf, int kk, Frags& f) __attribute__((always_inline)) {
    const uint16_t* ab = a_buf(buf) + (wm * G::WM + r32) * P + 8 * h;
    const uint16_t* bb = b_buf(buf) + (wn * G::WN + r32) * P + 8 * h;
#pragma unroll
    for (int i = 0; i < G::MI; ++i) f.a[i] = *reinterpret_cast<const bf16x8_t*>(ab + 32 * i * P + 16 * kk);
#pragma unroll
    for (int j = 0; j < G::NI; ++j) {
      if constexpr (TR) {
        const uint16_t* src = b_buf(buf) + 16 * kk * PT;
        s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(src + tr_o[j][0]));
        s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(src + tr_o[j][1]));
        const u32x2_t ul = __builtin_bit_cast(u32x2_t, lo), uh = __builtin_bit_cast(u32x2_t, hi);
        f.b[j] = __builtin_bit_cast(bf16x8_t, u32x4_t{ul[0], ul[1], uh[0], uh[1]});
      } else {
        f.b[j] = *reinterpret_cast<const bf16x8_t*>(bb + 32 * j * P + 16 * kk);
      }
    }
  };
  constexpr int KK = BK / 16;                          // 16-deep MFMA slices per step
  // One step: the MFMAs of buffer `buf` (fragments read two slices ahead;
  // none for a wave with no rows in the tile), and, between them, the staging
  // of the next step's registers `rn` into the other buffer: slice kk stages
  // weight units 8 kk / KK .. and the activation vectors j with
  // j KK / kAVec == kk.  ACT and STAGE are compile-time, so each slice is one
  // basic block the scheduler can interleave.
  auto step = [&](auto act_c, auto stage_c, int buf, const Regs& rn) __attribute__((always_inline)) {
    constexpr bool ACT = decltype(act_c)::value, STAGE = decltype(stage_c)::value;
    float a = 0.f;
    Lut lt{};
    if constexpr (STAGE) {
      a = wscale(rn);
      lt = make_table(a);
    }
    // fragments are read two slices ahead (a ring of three): with two MFMAs
    // per slice and wave (8 waves), one slice ahead left the reads' LDS
    // latency in front of every MFMA pair
    Frags f[3];
    if constexpr (ACT) {
      read_frags(buf, 0, f[0]);
      if (KK > 1) read_frags(buf, 1, f[1]);
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if constexpr (ACT) {
        if (kk + 2 < KK) read_frags(buf, kk + 2, f[(kk + 2) % 3]);
        const Frags& fc = f[kk % 3];
#pragma unroll
        for (int i = 0; i < G::MI; ++i)
#pragma unroll
          for (int j = 0; j < G::NI; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fc.a[i], fc.b[j], acc[i][j], 0, 0, 0);
      }
      if constexpr (STAGE) {
#pragma unroll
        for (int d = G::kUnits * kk / KK; d < G::kUnits * (kk + 1) / KK; ++d) store_w(buf ^ 1, rn, lt, a, d);
#pragma unroll
        for (int j = 0; j < G::kAVec; ++j)
          if (j * KK / G::kAVec == kk) store_a(buf ^ 1, rn, j);
      }
      // keep each slice's reads, MFMAs and staging together: without the
      // fence the scheduler moves MFMAs up next to their own reads
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Registers hold D = kDepth steps: step i multiplies buffer i % 2 and
  // stages step i + 1 (loaded during step i + 1 - D) into the other buffer,
  // after the loads of step i + D were issued into the registers step i came
  // from (staged during step i - 1).  The loop is unrolled by 4 so that the
  // register set and the buffer of every step are compile-time.
  constexpr int D = G::kDepth;
  static_assert(D == 2 || D == 4, "ring of 2 or 4 register sets, unrolled by 4");
  // Every load is issued, also for steps past the last one, with the step
  // index clamped to the last step (registers no step reads; load() clamps
  // its addresses into the tensors anyway): with the loads under a branch
  // the compiler could not count the loads issued after the ones a step
  // needs and waited for all of them (vmcnt(0)) once every four steps,
  // including the loads just issued for three steps ahead.
  const int last = n > 0 ? n - 1 : 0;
  auto run = [&](auto act_c) __attribute__((always_inline)) {
    Regs R[D];
#pragma unroll
    for (int j = 0; j < D; ++j) load(j < last ? j : last, R[j]);
    store(0, R[0]);
    __syncthreads();
    // step i = i0 + U of the unrolled body (i0 % 4 == 0)
    auto body = [&](auto u_c, int i) __attribute__((always_inline)) {
      constexpr int U = decltype(u_c)::value;
      load(i + D < last ? i + D : last, R[U % D]);
      step(act_c, std::true_type{}, U & 1, R[(U + 1) % D]);
      __syncthreads();
    };
    int i = 0;
    for (; i + 4 < n; i += 4) {                        // four steps that each stage a next step
      body(ic<0>{}, i);
      body(ic<1>{}, i + 1);
      body(ic<2>{}, i + 2);
      body(ic<3>{}, i + 3);
    }
    // the last 1..4 steps: no loads are left, the final step stages nothing
    const int rem = n - i;
    if (rem >= 2) body(ic<0>{}, i);
    if (rem >= 3) body(ic<1>{}, i + 1);
    if (rem >= 4) body(ic<2>{}, i + 2);
    if (rem == 1) step(act_c, std::false_type{}, 0, R[1 % D]);
    else if (rem == 2) step(act_c, std::false_type{}, 1, R[2 % D]);
    else if (rem == 3) step(act_c, std::false_type{}, 0, R[3 % D]);
    else step(act_c, std::false_type{}, 1, R[0]);
  };

  __syncthreads();                                     // tables in LDS
  if (n > 0) {
    if (active) run(std::true_type{});
    else run(std::false_type{});
  }

  // ---- epilogue -------------------------------------------------------------------
  if (!active) return;
#pragma unroll
  for (int i = 0; i < G::MI; ++i) {
#pragma unroll
    for (int j = 0; j < G::NI; ++j) {
      int64_t col = col0 + wn * G::WN + 32 * j + r32;
      // NF4 input gradient: tile column c holds output column 8 (c / 8) + pi(c % 8)
      // (the 8-bit expansion keeps the column order)
      if constexpr (TR && BITS == 4) col = (col & ~int64_t{7}) | (((col & 3) << 1) | ((col >> 2) & 1));
      if (col >= Nc) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = row0 + wm * G::WM + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
        if (row >= row_end) continue;
        if (p.splits == 1) {
          p.C[row * Nc + col] = to_bf16(acc[i][j][v]);
        } else {
          p.partial[(static_cast<int64_t>(z) * p.M + row) * Nc + col] = acc[i][j][v];
        }
      }
    }
  }
}

template <int BITS, int BM, int NW, int BN_, bool TRANS, bool NESTED, bool GROUPED>
hipError_t launch_gt(const GemmParams& p, int64_t m_tiles, int64_t n_cols, hipStream_t stream) {
  using G = GT<BITS, BM, NW, BN_>;
  auto kern = k_gemmt<BITS, BM, NW, BN_, TRANS, NESTED, GROUPED>;
  constexpr int lds = G::kLds(TRANS);
  static const bool attr_done = [&] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    (void)hipGetLastError();
    return true;
  }();
  (void)attr_done;
  GemmParams q = p;
  // grouped: row tiles dealt to the XCDs in turn (a multiple of 8; the
  // extra ids past the real tiles exit at once)
  if constexpr (GROUPED) m_tiles = (m_tiles + 7) / 8 * 8;
  q.m_tiles = static_cast<int32_t>(m_tiles);
  const int64_t tiles = ((n_cols + G::BN - 1) / G::BN) * m_tiles * p.splits;
  if (tiles <= 0 || tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  kern<<<dim3(static_cast<unsigned>(tiles)), G::kThreads, lds, stream>>>(q);
  return hipGetLastError();
}

// Register-staged tiles: BM = 32, 64 or 128 (8-bit: 32 or 128) by 128
// columns; NF4 with 4 waves, or 8 waves at 64 and 128 rows; NF4 128 x 256
// with 8 waves.
template <int BITS, bool TRANS, bool GROUPED>
hipError_t dispatch_gt(int bm, int nw, int bn, const GemmParams& p, int64_t m_tiles, int64_t n_cols,
                       hipStream_t stream) {
  const bool nested = p.w.nested();
#define NF4_GT(BMV, NWV, BNV)                                                                        \
  if (bm == BMV && nw == NWV && bn == BNV)                                                           \
    return nested ? launch_gt<BITS, BMV, NWV, BNV, TRANS, true, GROUPED>(p, m_tiles, n_cols, stream) \
                  : launch_gt<BITS, BMV, NWV, BNV, TRANS, false, GROUPED>(p, m_tiles, n_cols, stream);
  NF4_GT(32, 4, 128)
  NF4_GT(128, 4, 128)
  if constexpr (BITS == 4) {
    NF4_GT(64, 4, 128)
    NF4_GT(64, 8, 128)
    NF4_GT(128, 8, 128)
    NF4_GT(128, 8, 256)
  }
#undef NF4_GT
  return hipErrorInvalidValue;
}

template <int BM, int BN, bool TRANS, bool NESTED, bool GROUPED, int C>
hipError_t launch_tiled(const GemmParams& p, int64_t m_tiles, int64_t n_cols, hipStream_t stream) {
  using T = Tile<BM, BN, TRANS, C>;
  auto kern = k_gemm<BM, BN, TRANS, NESTED, GROUPED, C>;
  // raise the dynamic-LDS limit once per template instance (thread-safe
  // static initialisation); a failure here surfaces at the launch below
  static const bool attr_done = [&] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                              hipFuncAttributeMaxDynamicSharedMemorySize, T::kLdsBytes);
    (void)hipGetLastError();
    return true;
  }();
  (void)attr_done;
  GemmParams q = p;
  q.m_tiles = static_cast<int32_t>(m_tiles);
  const int64_t tiles = ((n_cols + BN - 1) / BN) * m_tiles * p.splits;
  if (tiles <= 0 || tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  kern<<<dim3(static_cast<unsigned>(tiles)), T::kThreads, T::kLdsBytes, stream>>>(q);
  return hipGetLastError();
}

template <bool TRANS, bool NESTED, bool GROUPED>
hipError_t launch_pp(const GemmParams& p, int64_t m_tiles, int64_t n_cols, hipStream_t stream) {
  auto kern = k_pp<TRANS, NESTED, GROUPED>;
  constexpr int lds = PP::lds_bytes<TRANS>();
  static const bool attr_done = [&] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    (void)hipGetLastError();
    return true;
  }();
  (void)attr_done;
  GemmParams q = p;
  q.m_tiles = static_cast<int32_t>(m_tiles);
  const int64_t tiles = ((n_cols + PP::BN - 1) / PP::BN) * m_tiles * p.splits;
  if (tiles <= 0 || tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  kern<<<dim3(static_cast<unsigned>(tiles)), PP::kThreads, lds, stream>>>(q);
  return hipGetLastError();
}

template <int WAVES, bool NESTED, bool GROUPED>
hipError_t launch_rb(const GemmParams& p, int64_t m_tiles, int64_t n_cols, hipStream_t stream) {
  using R = RB<WAVES>;
  auto kern = k_rb<WAVES, NESTED, GROUPED>;
  static const bool attr_done = [&] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                              hipFuncAttributeMaxDynamicSharedMemorySize, R::kLds);
    (void)hipGetLastError();
    return true;
  }();
  (void)attr_done;
  GemmParams q = p;
  q.m_tiles = static_cast<int32_t>(m_tiles);
  const int64_t tiles = ((n_cols + R::BN - 1) / R::BN) * m_tiles * p.splits;
  if (tiles <= 0 || tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  kern<<<dim3(static_cast<unsigned>(tiles)), R::kThreads, R::kLds, stream>>>(q);
  return hipGetLastError();
}

template <bool TRANS, bool GROUPED>
hipError_t dispatch_tile(int bm, int bn, int c, const GemmParams& p, int64_t m_tiles,
                         int64_t n_cols, hipStream_t stream) {
  const bool nested = p.w.nested();
#define NF4_CASE(BMV, BNV, CV)                                                                       \
  if (bm == BMV && bn == BNV && c == CV) {                                                           \
    return nested ? launch_tiled<BMV, BNV, TRANS, true, GROUPED, CV>(p, m_tiles, n_cols, stream)     \
                  : launch_tiled<BMV, BNV, TRANS, false, GROUPED, CV>(p, m_tiles, n_cols, stream);   \
  }
  if (c == kStagedTile || c == kStagedTile8) {
    return dispatch_gt<4, TRANS, GROUPED>(bm, c == kStagedTile8 ? 8 : 4, bn, p, m_tiles, n_cols, stream);
  }
  if (bm == 256 && bn == 256 && c == 0) {
    return nested ? launch_pp<TRANS, true, GROUPED>(p, m_tiles, n_cols, stream)
                  : launch_pp<TRANS, false, GROUPED>(p, m_tiles, n_cols, stream);
  }
  if constexpr (!TRANS) {
    if (bm == 256 && bn == 256 && c == 3) {
      return nested ? launch_rb<8, true, GROUPED>(p, m_tiles, n_cols, stream)
                    : launch_rb<8, false, GROUPED>(p, m_tiles, n_cols, stream);
    }
    if (bm == 256 && bn == 128 && c == 3) {
      return nested ? launch_rb<4, true, GROUPED>(p, m_tiles, n_cols, stream)
                    : launch_rb<4, false, GROUPED>(p, m_tiles, n_cols, stream);
    }
  }
  NF4_CASE(256, 256, 2)
  NF4_CASE(128, 256, 1)
  NF4_CASE(128, 256, 2)
  NF4_CASE(64, 256, 1)
  NF4_CASE(128, 128, 1)
  NF4_CASE(64, 128, 1)
#undef NF4_CASE
  return hipErrorInvalidValue;
}

int env_int(const char* name) {
  const char* v = getenv(name);
  return v ? atoi(v) : 0;
}

}  // namespace

int device_cu_count() {
  static int cached = 0;
  if (cached > 0) return cached;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      cus > 0) {
    cached = cus;
    return cus;
  }
  (void)hipGetLastError();
  return 256;   // MI355X
}

GemmPlan plan_gemm(GemmKind kind, int64_t M, int64_t N, int64_t K, int cus) {
  GemmPlan pl{};
  const int64_t nc = (kind == GemmKind::kFwd) ? N : K;
  const int64_t kc = (kind == GemmKind::kFwd) ? K : N;
  // Forward at M <= 32 streams the weights (nf4_gemv.hip) unless NF4_SMALL_M=0.
  // The streaming kernel addresses a 16-row group of W with 32-bit offsets:
  // rows of up to 2^26 elements.
  const char* sm = getenv("NF4_SMALL_M");
  // Above M = 16 the large products take the 8-wave 64-row register-staged
  // tile instead (measured on MI355X over the Llama-3.1-8B projections,
  // gate / down: at M = 32 24.1 / 23.4 against 26.6 / 25.5 us, at M = 20
  // 23.3 / 23.4 against 24.3 / 28.2, at M = 24 23.6 / 23.2 against
  // 22.9 / 27.7; q and k, 15.8 / 14.2 against 14.7 / 13.0 us at M = 32, stay
  // with the streaming kernels, as does every product up to M = 12)
  const bool staged_small = kind == GemmKind::kFwd && M > 16 && M <= 32 &&
                            static_cast<double>(N) * static_cast<double>(K) >= 33554432.0;
  if (kind == GemmKind::kFwd && M <= 32 && K <= (int64_t{1} << 26) && !(sm && sm[0] == '0') &&
      !staged_small) {
    plan_small_m(pl, M, N, K, cus);
    return pl;
  }
  pl.small_m = false;
  pl.kc = 0;
  // Tile choice by the size of the product (measured on MI355X over the
  // Llama-3.1-8B projections at M = 512 and the Qwen2.5-32B ones at
  // M = 2048): large products take 256 x 256 (each expanded weight serves 256
  // rows), mid-size ones 128 x 128 (4x the tiles), small ones 64 x 128.
  const double macs = static_cast<double>(M) * static_cast<double>(nc) * static_cast<double>(kc);
  // The forward takes the register-operand kernel from 4e9 MACs at M > 128
  // (tile width and split chosen by the cost model below); so does the input
  // gradient (ping-pong kernel) once its 256 x 256 tiles alone fill half the
  // compute units (Qwen k/v at M = 2048: 160 tiles, 43 vs 57 us with
  // 128 x 128; the M = 512 q/o input gradients, 32 tiles, stay at 128 x 128).
  const int64_t tiles256 = ((M + 255) / 256) * ((nc + 255) / 256);
  // Mid-size products at moderate M take the 8-wave register-staged tiles
  // (128 x 128, split by the model below): Llama q/o at M = 512, 36.5 us
  // against 39-40 us with 256-row tiles in either direction (k/v and the
  // larger gate/down keep the kernels below).
  const bool staged_mid = M >= 256 && M <= 1024 && macs >= 6e9 && macs < 1.6e10;
  if (staged_mid) {
    pl.bm = 128; pl.bn = 128;
  } else if (staged_small) {
    pl.bm = 64; pl.bn = 128;
  } else if ((macs >= 2e10 || (macs >= 4e9 && (kind == GemmKind::kFwd || 2 * tiles256 >= cus))) && M > 128) {
    pl.bm = 256; pl.bn = 256;
  } else if (macs >= 4e9 && M > 64) {
    pl.bm = 128; pl.bn = 128;
  } else {
    pl.bm = 64; pl.bn = 128;
  }
  // Tuning overrides (documented): NF4_BM, NF4_BN, NF4_CONSUMERS, NF4_SPLITS
  // (tiled kernel); NF4_SMALL_M=0 sends M <= 32 forwards to the tiled kernel.
  const int o_bm = env_int("NF4_BM"), o_bn = env_int("NF4_BN"), o_s = env_int("NF4_SPLITS");
  const int o_c = env_int("NF4_CONSUMERS");
  if (o_bm == 64 || o_bm == 128 || o_bm == 256) pl.bm = o_bm;
  if (o_bn == 128 || o_bn == 256) pl.bn = o_bn;
  // 256 x 128 exists only as the register-operand forward (NF4_BN=128)
  if (pl.bm == 256 && !(kind == GemmKind::kFwd && o_bn == 128 && o_c != 2 && o_c != 4)) pl.bn = 256;
  // 256 x 256: the forward runs the register-operand kernel (consumers = 3),
  // the input gradient the ping-pong kernel (consumers = 0); NF4_CONSUMERS=2
  // selects the producer/consumer kernel with 8 MFMA waves, NF4_CONSUMERS=4
  // the ping-pong kernel for the forward too
  pl.consumers = (pl.bm == 256) ? (o_c == 2 ? 2 : (kind == GemmKind::kFwd && o_c != 4 ? 3 : 0)) : 1;
  if (o_c == 2 && pl.bm == 128 && pl.bn == 256) pl.consumers = 2;
  if ((staged_mid || staged_small) && o_bm == 0 && o_bn == 0 && o_c == 0) pl.consumers = kStagedTile8;
  // NF4_CONSUMERS=5/6: the register-staged tile kernel with 4 / 8 waves, 128
  // columns, NF4_BM rows (32, 64 or 128; default 128); 6 with NF4_BN=256:
  // 128 x 256
  if (o_c == kStagedTile || o_c == kStagedTile8) {
    pl.consumers = o_c;
    pl.bn = 128;
    pl.bm = (o_bm == 64 || (o_bm == 32 && o_c == kStagedTile)) ? o_bm : 128;
    if (o_c == kStagedTile8 && o_bn == 256) { pl.bn = 256; pl.bm = 128; }
  }
  const bool staged = pl.consumers == kStagedTile || pl.consumers == kStagedTile8;
  const int bk = (pl.consumers == 3) ? 64 : (staged ? (pl.bn == 256 ? 64 : 128) : 16384 / pl.bn);
  const int64_t tiles = ((M + pl.bm - 1) / pl.bm) * ((nc + pl.bn - 1) / pl.bn);
  const int64_t ksteps = (kc + bk - 1) / bk;
  // Split count: minimise (rounds of workgroups over the compute units) x
  // (steps per workgroup) x step time + the fixed-order reduction, which
  // moves (4 S + 2) M Nc bytes.  Step time is modelled at ~3.8 TFLOP/s per
  // compute unit and the reduction at ~5 TB/s; each split keeps >= 8 steps.
  int s = 1;
  // Split count (and, for the register-operand forward, the tile width):
  // minimise rounds of workgroups over the compute units x (steps per
  // workgroup x step time + ~4 us of prologue and epilogue) + the split
  // traffic (the partials written and read back and the bf16 result).  Step
  // times measured on MI355X: 256 x 256 register-operand ~1.75 us, 256 x 128
  // ~1.25 us; the other kernels are modelled at ~3.8 TFLOP/s per compute
  // unit.  Each split keeps >= 8 steps.
  {
    const bool rb = pl.consumers == 3;
    // measured per kernel family: the register-operand forward's split
    // traffic is charged at (8 S + 2) M Nc bytes / 2.5 TB/s, the other
    // kernels' at (4 S + 2) M Nc bytes / 5 TB/s
    auto split_cost = [&](int c) {
      const double mn = static_cast<double>(M) * static_cast<double>(nc);
      return rb ? (8.0 * c + 2.0) * mn / 2.5e6 : (4.0 * c + 2.0) * mn / 5.0e6;
    };
    auto cost = [&](int bn_c, int bk_c, double t_step, int c) {
      const int64_t tl = ((M + pl.bm - 1) / pl.bm) * ((nc + bn_c - 1) / bn_c);
      const int64_t ks = (kc + bk_c - 1) / bk_c;
      const int64_t rounds = (tl * c + cus - 1) / cus;
      const int64_t steps = (ks + c - 1) / c;
      double t = static_cast<double>(rounds) * (static_cast<double>(steps) * t_step + 4.0);
      if (c > 1) t += split_cost(c);
      return t;
    };
    const double t_step = rb ? (pl.bn == 256 ? 1.75 : 1.25) : 2.0 * pl.bm * pl.bn * bk / 3.8e6;
    double best = 0;
    for (int c = 1; c <= 8; ++c) {
      if (c > 1 && ksteps < 8 * c) break;
      const double t = cost(pl.bn, bk, t_step, c);
      if (c == 1 || t < best) { best = t; s = c; }
    }
    // the 4-wave 256 x 128 register-operand forward, unless a width was forced
    if (rb && pl.bn == 256 && o_bn == 0) {
      for (int c = 1; c <= 8; ++c) {
        if (c > 1 && ksteps < 8 * c) break;
        const double t = cost(128, 64, 1.25, c);
        if (t < best) { best = t; s = c; pl.bn = 128; }
      }
    }
  }
  if (o_s >= 1 && o_s <= 16) s = o_s;
  pl.splits = s;
  pl.ws_bytes = (s > 1) ? static_cast<size_t>(s) * static_cast<size_t>(M) * static_cast<size_t>(nc) * 4 : 0;
  return pl;
}

GemmPlan plan_grouped(GemmKind kind, int64_t total_M, int64_t N, int64_t K, int32_t E) {
  GemmPlan pl{};
  pl.small_m = false;
  pl.splits = 1;
  pl.ws_bytes = 0;
  pl.bn = 256;
  // rows per expert are only known on the device; size the tile by the mean
  const int64_t mean = (E > 0) ? (total_M + E - 1) / E : total_M;
  if (mean <= 128) {
    // Few rows per expert: the 8-wave register-staged 128 x 256 tile, one row
    // tile per expert of up to 128 rows, each weight expanded once per
    // expert.  Measured on MI355X with 64 experts of 46-86 rows (OLMoE
    // shapes): gate/up 52.7 / 64.0 us forward / input gradient, down
    // 55.7 / 54.3 us, against 63.0 / 75.5 and 65.8 / 59.9 us with 128 x 128
    // (64 x 32 per wave: a third more LDS fragment reads per MFMA) and
    // 98 / 100 and 76 / 95 us with 256-row register-operand and ping-pong
    // tiles.
    pl.bm = 128;
    pl.bn = 256;
    pl.consumers = kStagedTile8;
  } else {
    pl.bm = mean <= 192 ? 128 : 256;
    pl.consumers = (pl.bm == 256) ? 0 : 1;
  }
  // Tuning overrides (documented): NF4_BM, NF4_BN, NF4_CONSUMERS select the
  // tile as for a single product; there is no split of the contraction here.
  const int o_bm = env_int("NF4_BM"), o_bn = env_int("NF4_BN"), o_c = env_int("NF4_CONSUMERS");
  if (o_bm != 0 || o_bn != 0 || o_c != 0) {
    if (o_bm == 64 || o_bm == 128 || o_bm == 256) pl.bm = o_bm;
    if (o_bn == 128 || o_bn == 256) pl.bn = o_bn;
    if (pl.bm == 256 && !(kind == GemmKind::kFwd && o_bn == 128 && o_c != 2 && o_c != 4)) pl.bn = 256;
    pl.consumers = (pl.bm == 256) ? (o_c == 2 ? 2 : (kind == GemmKind::kFwd && o_c != 4 ? 3 : 0)) : 1;
    if (o_c == 2 && pl.bm == 128 && pl.bn == 256) pl.consumers = 2;
    if (o_c == kStagedTile || o_c == kStagedTile8) {
      pl.consumers = o_c;
      pl.bn = 128;
      pl.bm = (o_bm == 64 || (o_bm == 32 && o_c == kStagedTile)) ? o_bm : 128;
      if (o_c == kStagedTile8 && o_bn == 256) { pl.bn = 256; pl.bm = 128; }
    }
  }
  return pl;
}

hipError_t launch_gemm(GemmKind kind, const GemmPlan& plan, const void* A, int64_t M,
                       const WArgs& w, void* C, void* ws, hipStream_t stream) {
  const bool trans = kind == GemmKind::kBwdInput;
  const int64_t nc = trans ? w.K : w.N;
  if (plan.small_m) {
    hipError_t e = launch_gemv(plan, A, M, w, C, ws, stream);
    if (e != hipSuccess) return e;
    count_path(3);
    if (plan.splits > 1) {
      const int64_t n = M * nc;
      const int64_t threads = (n + 3) / 4;
      k_splitk_reduce<<<static_cast<unsigned>((threads + kThreads - 1) / kThreads), kThreads, 0, stream>>>(
          static_cast<const float*>(ws), plan.splits, n, static_cast<uint16_t*>(C));
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      count_path(5);
    }
    return hipSuccess;
  }
  GemmParams p{};
  p.A = static_cast<const uint16_t*>(A);
  p.C = static_cast<uint16_t*>(C);
  p.partial = static_cast<float*>(ws);
  p.w = w;
  p.offsets = nullptr;
  p.M = M;
  p.E = 1;
  p.splits = plan.splits;
  const int64_t m_tiles = (M + plan.bm - 1) / plan.bm;
  hipError_t e = trans ? dispatch_tile<true, false>(plan.bm, plan.bn, plan.consumers, p, m_tiles, nc, stream)
                       : dispatch_tile<false, false>(plan.bm, plan.bn, plan.consumers, p, m_tiles, nc, stream);
  if (e != hipSuccess) return e;
  count_path(trans ? 4 : 2);
  if (plan.splits > 1) {
    const int64_t n = M * nc;
    const int64_t threads = (n + 3) / 4;
    k_splitk_reduce<<<static_cast<unsigned>((threads + kThreads - 1) / kThreads), kThreads, 0, stream>>>(
        static_cast<const float*>(ws), plan.splits, n, static_cast<uint16_t*>(C));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    count_path(5);
  }
  return hipSuccess;
}

hipError_t launch_grouped(GemmKind kind, const GemmPlan& plan, const void* A,
                          const int32_t* offsets, int32_t E, int64_t total_M, const WArgs& w,
                          void* C, hipStream_t stream) {
  const bool trans = kind == GemmKind::kBwdInput;
  const int64_t nc = trans ? w.K : w.N;
  GemmParams p{};
  p.A = static_cast<const uint16_t*>(A);
  p.C = static_cast<uint16_t*>(C);
  p.partial = nullptr;
  p.w = w;
  p.offsets = offsets;
  p.M = total_M;
  p.E = E;
  p.splits = 1;
  // upper bound on sum_e ceil(M_e / bm); workgroups past the real count exit
  const int64_t m_tiles = (total_M + plan.bm - 1) / plan.bm + E;
  hipError_t e = trans ? dispatch_tile<true, true>(plan.bm, plan.bn, plan.consumers, p, m_tiles, nc, stream)
                       : dispatch_tile<false, true>(plan.bm, plan.bn, plan.consumers, p, m_tiles, nc, stream);
  if (e != hipSuccess) return e;
  count_path(trans ? 7 : 6);
  return hipSuccess;
}

}  // namespace nf4

// ---- 8-bit blockwise matmuls ------------------------------------------------------
namespace nf4 {

// 128-row tiles, or 32 at M <= 32; the contraction is split (powers of two up
// to 16) while the tiles alone leave compute units idle and every split keeps
// at least two 64-deep steps.
GemmPlan plan_gemm8(GemmKind kind, int64_t M, int64_t N, int64_t K, int cus) {
  GemmPlan pl{};
  const int64_t nc = (kind == GemmKind::kFwd) ? N : K;
  const int64_t kc = (kind == GemmKind::kFwd) ? K : N;
  pl.bm = M <= 32 ? 32 : 128;
  pl.bn = 128;
  pl.consumers = 0;
  pl.small_m = false;
  pl.kc = 0;
  const int64_t tiles = (M + pl.bm - 1) / pl.bm * ((nc + 127) / 128);
  const int64_t ktiles = (kc + 63) / 64;
  int s = 1;
  while (s < 16 && tiles * s < cus && ktiles / (2 * s) >= 2) s *= 2;
  pl.splits = s;
  pl.ws_bytes = s > 1 ? static_cast<size_t>(s) * static_cast<size_t>(M) * static_cast<size_t>(nc) * 4 : 0;
  return pl;
}

hipError_t launch_gemm8(GemmKind kind, const GemmPlan& plan, const void* A, int64_t M,
                        const WArgs& w, void* C, void* ws, hipStream_t stream) {
  const bool trans = kind == GemmKind::kBwdInput;
  const int64_t nc = trans ? w.K : w.N;
  GemmParams p{};
  p.A = static_cast<const uint16_t*>(A);
  p.C = static_cast<uint16_t*>(C);
  p.partial = static_cast<float*>(ws);
  p.w = w;
  p.offsets = nullptr;
  p.M = M;
  p.E = 1;
  p.splits = plan.splits;
  const int64_t m_tiles = (M + plan.bm - 1) / plan.bm;
  hipError_t e = trans ? dispatch_gt<8, true, false>(plan.bm, 4, 128, p, m_tiles, nc, stream)
                       : dispatch_gt<8, false, false>(plan.bm, 4, 128, p, m_tiles, nc, stream);
  if (e != hipSuccess) return e;
  count_path(trans ? 9 : 8);
  if (plan.splits > 1) {
    const int64_t n = M * nc;
    const int64_t threads = (n + 3) / 4;
    k_splitk_reduce<<<static_cast<unsigned>((threads + kThreads - 1) / kThreads), kThreads, 0, stream>>>(
        static_cast<const float*>(ws), plan.splits, n, static_cast<uint16_t*>(C));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    count_path(5);
  }
  return hipSuccess;
}

// Grouped: 32-row tiles when experts hold 48 rows or fewer on average, else
// 128; no split.
hipError_t launch_grouped8(GemmKind kind, const void* A, const int32_t* offsets, int32_t E,
                           int64_t total_M, const WArgs& w, void* C, hipStream_t stream) {
  const bool trans = kind == GemmKind::kBwdInput;
  const int64_t nc = trans ? w.K : w.N;
  const int bm = total_M <= 48 * static_cast<int64_t>(E) ? 32 : 128;
  GemmParams p{};
  p.A = static_cast<const uint16_t*>(A);
  p.C = static_cast<uint16_t*>(C);
  p.partial = nullptr;
  p.w = w;
  p.offsets = offsets;
  p.M = total_M;
  p.E = E;
  p.splits = 1;
  const int64_t m_tiles = (total_M + bm - 1) / bm + E;
  hipError_t e = trans ? dispatch_gt<8, true, true>(bm, 4, 128, p, m_tiles, nc, stream)
                       : dispatch_gt<8, false, true>(bm, 4, 128, p, m_tiles, nc, stream);
  if (e != hipSuccess) return e;
  count_path(trans ? 9 : 8);
  return hipSuccess;
}

}  // namespace nf4
