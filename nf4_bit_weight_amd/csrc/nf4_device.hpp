// Device building blocks shared by the NF4 kernels (gfx950 / CDNA4).
//
// Decode of one NF4 weight (the QuantState fields of bitsandbytes #2034,
// "Root cause" / "Why save_for_backward fixes it"):
//   absmax_hat = fp32(fp32(nested_code[q2] * s2[b/256]) + offset)   (nested)
//              | absmax[b]                                          (plain)
//   w_hat      = bf16_rne(fp32(code[q] * absmax_hat))
//
// The expansion never computes a product per weight.  For each (row, 64-block)
// the 16 possible bf16 results are built once (16 fp32 multiplies, 8 packed
// bf16 conversions) and split into a high-byte table and a low-byte table of
// 16 bytes each (4 dwords each).  One packed dword (8 nibbles) is then
// expanded with v_perm_b32 byte selects: the low 3 bits of a nibble pick a
// byte from an 8-byte half-table, bit 3 picks the half through a byte mask
// built with v_perm_b32's sign-replicate selectors.  ~28 VALU ops per 8
// weights plus 32 per table, and the products are exactly those of the
// per-element definition.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nf4 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kBlock = 64;         // NF4 block (elements per absmax)
constexpr int kNestedBlock = 256;  // absmax values per nested scale

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  // v_perm_b32: bytes 0-3 of the 8-byte source are `lo`, bytes 4-7 are `hi`;
  // selector 8/9/10/11 replicates the MSB of byte 1/3/5/7, 12 gives 0x00.
  return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ uint32_t bitsel(uint32_t mask, uint32_t a, uint32_t b) {
  return (mask & a) | (~mask & b);  // v_bfi_b32
}

// Two fp32 -> one dword of two bf16 (x in the low half), round-to-nearest-even
// (v_cvt_pk_bf16_f32 under the default rounding mode).
__device__ __forceinline__ uint32_t pack_bf16x2(float x, float y) {
  f32x2_t v = {x, y};
  bf16x2_t r = __builtin_convertvector(v, bf16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Byte tables of the 16 bf16 values of one (row, block).
struct Lut {
  uint32_t h[4];  // h[j] byte i = high byte of value 4j+i
  uint32_t l[4];  // l[j] byte i = low byte of value 4j+i
};

// code[] in registers (uniform), a = decoded block scale.
__device__ __forceinline__ Lut make_lut(const float (&code)[16], float a) {
  uint32_t p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // separate fp32 multiplies: exactly fp32(code[q] * a) per entry
    float v0 = __fmul_rn(code[2 * i], a);
    float v1 = __fmul_rn(code[2 * i + 1], a);
    p[i] = pack_bf16x2(v0, v1);
  }
  Lut t;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    t.h[j] = perm(p[2 * j + 1], p[2 * j], 0x07050301u);
    t.l[j] = perm(p[2 * j + 1], p[2 * j], 0x06040200u);
  }
  return t;
}

// Expand one packed dword (element 2i in the high nibble of byte i) into 4
// dwords of bf16 pairs in element order: out[j] = (w[2j] low half, w[2j+1]
// high half).
__device__ __forceinline__ void expand8(uint32_t p, const Lut& t, uint32_t (&out)[4]) {
  const uint32_t se = (p >> 4) & 0x07070707u;          // even elements, index & 7
  const uint32_t so = p & 0x07070707u;                 // odd elements,  index & 7
  const uint32_t me = perm(p, p << 8, 0x0B090A08u);    // 0xFF where even index >= 8
  const uint32_t p4 = p << 4;
  const uint32_t mo = perm(p4, p4 << 8, 0x0B090A08u);  // 0xFF where odd index >= 8
  const uint32_t he = bitsel(me, perm(t.h[3], t.h[2], se), perm(t.h[1], t.h[0], se));
  const uint32_t le = bitsel(me, perm(t.l[3], t.l[2], se), perm(t.l[1], t.l[0], se));
  const uint32_t ho = bitsel(mo, perm(t.h[3], t.h[2], so), perm(t.h[1], t.h[0], so));
  const uint32_t lo = bitsel(mo, perm(t.l[3], t.l[2], so), perm(t.l[1], t.l[0], so));
  const uint32_t e01 = perm(he, le, 0x05010400u);      // (w0, w2)
  const uint32_t e23 = perm(he, le, 0x07030602u);      // (w4, w6)
  const uint32_t o01 = perm(ho, lo, 0x05010400u);      // (w1, w3)
  const uint32_t o23 = perm(ho, lo, 0x07030602u);      // (w5, w7)
  out[0] = perm(o01, e01, 0x05040100u);                // (w0, w1)
  out[1] = perm(o01, e01, 0x07060302u);                // (w2, w3)
  out[2] = perm(o23, e23, 0x05040100u);                // (w4, w5)
  out[3] = perm(o23, e23, 0x07060302u);                // (w6, w7)
}

// Expand 8 nibbles in the order (0, 2, 4, 6, 1, 3, 5, 7): out[0] = (w0, w2),
// out[1] = (w4, w6), out[2] = (w1, w3), out[3] = (w5, w7).  Four byte
// permutations fewer than expand8; the other operand of the product is read
// in the same order (both sides of a dot product may permute their terms
// alike), or, where the expanded index is an output column, the column is
// mapped back when the result is written.
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

// Decoded scale of block b.  `ncode` is the 256-entry nested table (LDS or
// global), `absmax` is u8 in the nested form and f32 otherwise.
template <bool NESTED>
__device__ __forceinline__ float block_scale(const void* absmax, const float* nested_absmax,
                                             float offset, const float* ncode, int64_t b) {
  if constexpr (NESTED) {
    const uint32_t q2 = static_cast<const uint8_t*>(absmax)[b];
    const float s2 = nested_absmax[b / kNestedBlock];
    return __fadd_rn(__fmul_rn(ncode[q2], s2), offset);   // two roundings, no FMA
  } else {
    return static_cast<const float*>(absmax)[b];
  }
}

}  // namespace nf4
