// common.hpp -- shared device helpers of the gfx950 W4A16 kernels: vector
// types, weight-code decoders and scale decoders.
//
// Weight formats (page titles):
//   int4 asymmetric, group 128 ("megakernel_int4_weight_decode.py", "The
//     weight format"): value = (code - zero) * scale, bf16 scale and uint8
//     zero per 128 contiguous k; byte (n, i) holds k = 2i in its LOW nibble.
//   NVFP4 ("Matmul2dFp4", run / run_smem_decode): e2m1 code times the
//     magnitude of an e4m3 scale per 16 k.
//   MXFP4: e2m1 code times 2^(E - 127), one e8m0 byte E per 32 k.
//
// Every decoder below produces exact values: an int4 weight has at most 12
// significant bits and an fp4 weight at most 6, so fp32 holds them exactly and
// one final round-to-nearest-even gives the bf16 weight.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// kInt4: int4 with groups of 128 (one group per 128-code k-block);
// kInt4G32 / kInt4G64: the same with groups of 32 / 64 codes;
// kInt4Sym: groups of 128 with the fixed zero point 8 (no zero array).
enum Format : int { kInt4 = 0, kNvfp4 = 1, kMxfp4 = 2, kInt4G32 = 3, kInt4G64 = 4, kInt4Sym = 5 };
constexpr int kFormats = 6;

// int4 formats: (code - zero) * scale with a bf16 scale per group; the zero
// is a u8 per group, or 8 for the symmetric format
constexpr bool is_int4(int fmt) {
  return fmt == kInt4 || fmt == kInt4G32 || fmt == kInt4G64 || fmt == kInt4Sym;
}
// int4 formats that come with a zero array
constexpr bool has_zeros(int fmt) { return fmt == kInt4 || fmt == kInt4G32 || fmt == kInt4G64; }
// int4 formats whose group is the 128-code k-block
constexpr bool is_int4_g128(int fmt) { return fmt == kInt4 || fmt == kInt4Sym; }
constexpr uint32_t kSymZero = 8;  // the symmetric format's zero point

template <int FMT>
struct FormatTraits;
template <>
struct FormatTraits<kInt4> {
  static constexpr int kGroup = 128;
};
template <>
struct FormatTraits<kNvfp4> {
  static constexpr int kGroup = 16;
};
template <>
struct FormatTraits<kMxfp4> {
  static constexpr int kGroup = 32;
};
template <>
struct FormatTraits<kInt4G32> {
  static constexpr int kGroup = 32;
};
template <>
struct FormatTraits<kInt4G64> {
  static constexpr int kGroup = 64;
};
template <>
struct FormatTraits<kInt4Sym> {
  static constexpr int kGroup = 128;
};

// ---- bit helpers ------------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// byte permute: result byte i = byte sel_i of the 8-byte value {hi:lo}
// (selector 0x0c gives 0x00).
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// two fp32 -> two bf16 packed in one dword, round to nearest even
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t r = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

// ---- buffer loads -------------------------------------------------------------
// A raw buffer resource over [base, base + bytes): loads at an offset past
// `bytes` return 0 without touching memory, so tails and padding need no
// branches (and no branch-induced waits between independent loads).  The
// base must be wave-uniform.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kBufferOOB = 0x80000000u;  // an offset past every buffer used here

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// ---- weight layouts ------------------------------------------------------------
// Byte offset of 16-byte chunk c (codes 32c .. 32c+31) of weight row r, counted
// from a row that is a multiple of 16, in one of the two layouts of the packed
// weights:
//   row-major (as given): rowb = K/2 bytes per row;
//   prepacked: 16-row tiles, and in a tile one 1-KB block per 128 codes
//     (4 chunks of each of the 16 rows), chunk c of row r at slot
//     (r % 16) + 16 (c % 4) of block c / 4 -- the order in which the lanes of
//     an MFMA 16x16x32 weight fragment read them, so that a wave's 16-byte
//     loads of one block are one contiguous kilobyte.
__device__ __forceinline__ uint32_t wchunk(uint32_t r, uint32_t c, uint32_t rowb, bool pre) {
  return pre ? (r >> 4) * (rowb << 4) + (c >> 2) * 1024u + ((r & 15u) + 16u * (c & 3u)) * 16u
             : r * rowb + c * 16u;
}
__device__ __forceinline__ u32x4_t buf_load_b128(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load_b32(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load_b16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load_b8(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}

// Asynchronous global -> LDS copy (gfx950 "buffer_load ... lds"): lane l of
// the wave reads `size` bytes at voff of the buffer and writes them to LDS
// dword slot l (16-byte slot l for the 16-byte form) after the wave-uniform
// LDS base `lds_addr`; 1- and 2-byte loads are zero-extended to the slot.
// Out-of-range lanes write zeros.  Issued through inline assembly so that
// the compiler neither waits for the copy nor knows of it: the caller owns the
// vmcnt accounting (s_waitcnt vmcnt(n) then s_barrier before any wave reads
// the slots).  m0 carries the LDS base and is restored afterwards.
__device__ __forceinline__ void lds_dma_b128(rsrc_t r, uint32_t lds_addr, uint32_t voff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(voff), "s"(r)
      : "memory");
}
__device__ __forceinline__ void lds_dma_b32(rsrc_t r, uint32_t lds_addr, uint32_t voff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(voff), "s"(r)
      : "memory");
}
__device__ __forceinline__ void lds_dma_b16(rsrc_t r, uint32_t lds_addr, uint32_t voff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_ushort %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(voff), "s"(r)
      : "memory");
}
__device__ __forceinline__ void lds_dma_b8(rsrc_t r, uint32_t lds_addr, uint32_t voff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_ubyte %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(voff), "s"(r)
      : "memory");
}
// 32-bit LDS address of a __shared__ object (the value m0 takes above)
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// ---- scale decoders -----------------------------------------------------------

// e4m3 ("fn" variant: bias 7, no infinities, S.1111.111 = NaN) -> |value| as
// fp32.  The 7 magnitude bits placed at fp32 bits 26:20 read as
// 2^(e-127) (1 + m/8) for e >= 1 and as the fp32 subnormal m 2^-129 for e = 0;
// multiplying by 2^120 (exact) gives 2^(e-7) (1 + m/8) and m 2^-9, the e4m3
// values.  The magnitude is used, the sign dropped.
__device__ __forceinline__ float e4m3_magnitude(uint32_t byte) {
  uint32_t mag = byte & 0x7Fu;
  float v = __uint_as_float(mag << 20) * 0x1p120f;
  return mag == 0x7Fu ? __uint_as_float(0x7FC00000u) : v;
}

// e8m0 byte E -> 2^(E - 127) as the fp32 bit pattern E << 23.  The scaled
// fp4 conversion instructions read only this exponent field, map a field of
// 0 to 2^-127, which is exactly the e8m0 meaning of E = 0, and a field of
// 255 to NaN for every code, zero included (measured on gfx950 over all 256
// code bytes), which is the e8m0 meaning of E = 0xFF: the NaN weights then
// make every output of their row NaN through the MFMA.
__device__ __forceinline__ float e8m0_as_exponent_scale(uint32_t E) {
  return __uint_as_float(E << 23);
}

// e8m0 byte E -> 2^(E - 127) as an ordinary fp32 value (E = 0 is the fp32
// subnormal 2^-127, E = 255 is NaN).
__device__ __forceinline__ float e8m0_value(uint32_t E) {
  uint32_t bits = (E == 0) ? 0x00400000u : (E << 23);
  return E == 255 ? __uint_as_float(0x7FC00000u) : __uint_as_float(bits);
}

// ---- fp4 decoders -------------------------------------------------------------

// 8 e2m1 codes (one dword, code k in nibble k) times 2^(E-127), E the
// exponent field of `escale`, to 8 bf16 in k order.  Exact for every code and
// E in 0..254 (hardware scaled conversion, two codes per instruction).
__device__ __forceinline__ u32x4_t fp4x8_to_bf16_escale(uint32_t q, float escale) {
  u32x4_t r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, escale, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, escale, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, escale, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, escale, 3));
  return r;
}

// 8 e2m1 codes times an arbitrary fp32 scale (exact e2m1 -> fp32 with unit
// scale, one exact fp32 multiply, one RNE to bf16 -- exact whenever the
// product is a bf16 value, e.g. for every e4m3 scale).
__device__ __forceinline__ u32x4_t fp4x8_to_bf16_fscale(uint32_t q, float scale) {
  const f32x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 0);
  const f32x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 1);
  const f32x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 2);
  const f32x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 3);
  u32x4_t r;
  r[0] = pack_bf16x2(v0[0] * scale, v0[1] * scale);
  r[1] = pack_bf16x2(v1[0] * scale, v1[1] * scale);
  r[2] = pack_bf16x2(v2[0] * scale, v2[1] * scale);
  r[3] = pack_bf16x2(v3[0] * scale, v3[1] * scale);
  return r;
}

// ---- int4 decoders -------------------------------------------------------------

// 8 consecutive bf16 values (k order 0..7, two per dword) reordered to the k
// order (0, 2, 4, 6, 1, 3, 5, 7) of int4x8_minus_zero_even_odd.
__device__ __forceinline__ u32x4_t bf16x8_even_odd(u32x4_t a) {
  u32x4_t r;
  r[0] = perm_b32(a[1], a[0], 0x05040100u);  // (a0, a2)
  r[1] = perm_b32(a[3], a[2], 0x05040100u);  // (a4, a6)
  r[2] = perm_b32(a[1], a[0], 0x07060302u);  // (a1, a3)
  r[3] = perm_b32(a[3], a[2], 0x07060302u);  // (a5, a7)
  return r;
}

// 8 int4 codes to bf16 weights (code - zero) * scale, each rounded once to
// nearest even.  The subtraction comes first, as the format defines it (so a
// zero weight takes the sign of the scale); both steps are exact in fp32 (at
// most 17 significant bits), so the only rounding is the final bf16 one.  The
// codes reach fp32 through the scaled fp8 converter (each masked byte read as
// the e4m3 value code * 2^-9, scaled by 2^9: exact, two per instruction).
__device__ __forceinline__ u32x4_t int4x8_to_bf16_weights(uint32_t q, float s, float zf) {
  const uint32_t lo = q & 0x0F0F0F0Fu;         // codes k = 0, 2, 4, 6
  const uint32_t hi = (q >> 4) & 0x0F0F0F0Fu;  // codes k = 1, 3, 5, 7
  const f32x2_t e0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(lo, 512.0f, false);  // k0, k2
  const f32x2_t e1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(lo, 512.0f, true);   // k4, k6
  const f32x2_t o0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, 512.0f, false);  // k1, k3
  const f32x2_t o1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, 512.0f, true);   // k5, k7
  u32x4_t r;
  r[0] = pack_bf16x2((e0[0] - zf) * s, (o0[0] - zf) * s);
  r[1] = pack_bf16x2((e0[1] - zf) * s, (o0[1] - zf) * s);
  r[2] = pack_bf16x2((e1[0] - zf) * s, (o1[0] - zf) * s);
  r[3] = pack_bf16x2((e1[1] - zf) * s, (o1[1] - zf) * s);
  return r;
}

// 8 int4 codes to their exact weights (code - zero) * scale (at most 16
// significant bits, exact in fp32) as the sum of two bf16 fragments hi + lo,
// both exact: hi is the weight rounded to nearest even, lo = weight - hi has
// at most 8 significant bits.  Two MFMAs over hi and lo then accumulate the
// exact weights (natural k order).
__device__ __forceinline__ void int4x8_to_bf16_hilo(uint32_t q, float s, float zf, u32x4_t& hi,
                                                    u32x4_t& lo) {
  const uint32_t l = q & 0x0F0F0F0Fu;         // codes k = 0, 2, 4, 6
  const uint32_t h = (q >> 4) & 0x0F0F0F0Fu;  // codes k = 1, 3, 5, 7
  const f32x2_t e0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(l, 512.0f, false);  // k0, k2
  const f32x2_t e1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(l, 512.0f, true);   // k4, k6
  const f32x2_t o0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(h, 512.0f, false);  // k1, k3
  const f32x2_t o1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(h, 512.0f, true);   // k5, k7
  const float w[8] = {(e0[0] - zf) * s, (o0[0] - zf) * s, (e0[1] - zf) * s, (o0[1] - zf) * s,
                      (e1[0] - zf) * s, (o1[0] - zf) * s, (e1[1] - zf) * s, (o1[1] - zf) * s};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t p = pack_bf16x2(w[2 * i], w[2 * i + 1]);
    hi[i] = p;
    lo[i] = pack_bf16x2(w[2 * i] - __uint_as_float(p << 16), w[2 * i + 1] - __uint_as_float(p & 0xFFFF0000u));
  }
}

// 8 int4 codes to code - zero, exact in bf16 (an integer in -255 .. 15),
// natural k order; the group scale is applied to the fp32 sum afterwards.
__device__ __forceinline__ u32x4_t int4x8_minus_zero(uint32_t q, float zf) {
  const uint32_t l = q & 0x0F0F0F0Fu;         // codes k = 0, 2, 4, 6
  const uint32_t h = (q >> 4) & 0x0F0F0F0Fu;  // codes k = 1, 3, 5, 7
  const f32x2_t e0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(l, 512.0f, false);  // k0, k2
  const f32x2_t e1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(l, 512.0f, true);   // k4, k6
  const f32x2_t o0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(h, 512.0f, false);  // k1, k3
  const f32x2_t o1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(h, 512.0f, true);   // k5, k7
  u32x4_t r;
  r[0] = pack_bf16x2(e0[0] - zf, o0[0] - zf);
  r[1] = pack_bf16x2(e0[1] - zf, o0[1] - zf);
  r[2] = pack_bf16x2(e1[0] - zf, o1[0] - zf);
  r[3] = pack_bf16x2(e1[1] - zf, o1[1] - zf);
  return r;
}

// ---- int4 through fp16 ---------------------------------------------------------
// An integer code - zero in -255 .. 15 is exact in fp16 as well, and fp16
// has packed arithmetic: with the code in the low mantissa bits of 0x6400
// (1024.0) the fp16 value is 1024 + code, and one packed fp16 subtraction of
// 1024 + zero (both in [1024, 1280), exact) leaves code - zero exactly.  That
// is 11 VALU instructions per 8 codes (3 shifts, 4 bit-field inserts, 4 packed
// subtractions) against the 19 of the fp32 route above.  The A operand is
// then fp16 too, exact for a bf16 value that is 0, inf, or of magnitude in
// [2^-17, 65504] (8 significant bits; fp16 subnormals keep 8 bits down to
// 2^-17).  The products equal those of the bf16 route, and gfx950's MFMA
// sums the 32 products of a step and the accumulator to the same bits
// whatever the slot order and operand type (measured over 2^20 outputs of
// four chained steps with exact products, slots permuted within each 8).
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// mask and bias of the bit-field inserts, held in VGPRs (register operands)
struct F16Consts {
  uint32_t mask, bias;
};
__device__ __forceinline__ F16Consts f16_consts() {
  F16Consts c{0x000F000Fu, 0x64006400u};
  asm volatile("" : "+v"(c.mask), "+v"(c.bias));
  return c;
}
// the fp16 pair (1024 + zero, 1024 + zero), zero a byte 0 .. 255
__device__ __forceinline__ uint32_t f16_zero_pair(uint32_t zero) {
  const uint32_t h = 0x6400u | zero;
  return h | (h << 16);
}
__device__ __forceinline__ uint32_t f16x2_minus(uint32_t x, f16x2_t z) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, x) - z);
}
// 8 int4 codes (k = 0 .. 7, low nibble first) to code - zero in fp16, exact,
// in the k order (0, 4, 1, 5, 2, 6, 3, 7): the dword of codes k, k + 4 takes
// the nibbles at bits 4k and 4k + 16.
__device__ __forceinline__ u32x4_t int4x8_minus_zero_f16(uint32_t q, F16Consts c, uint32_t zpair) {
  const f16x2_t z = __builtin_bit_cast(f16x2_t, zpair);
  const uint32_t bias = c.bias & ~c.mask;
  const uint32_t r0 = f16x2_minus((q & c.mask) | bias, z);
  const uint32_t r1 = f16x2_minus(((q >> 4) & c.mask) | bias, z);
  const uint32_t r2 = f16x2_minus(((q >> 8) & c.mask) | bias, z);
  const uint32_t r3 = f16x2_minus(((q >> 12) & c.mask) | bias, z);
  return u32x4_t{r0, r1, r2, r3};
}
// 8 bf16 values (k = 0 .. 7) to fp16 in the k order of int4x8_minus_zero_f16;
// `exact` is cleared unless every value converts exactly (a NaN clears it)
__device__ __forceinline__ u32x4_t bf16x8_to_f16_k04(u32x4_t a, bool& exact) {
  float f[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) f[k] = __uint_as_float(k & 1 ? a[k >> 1] & 0xFFFF0000u : a[k >> 1] << 16);
  uint32_t r[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const auto h = __builtin_amdgcn_cvt_pkrtz(f[k], f[k + 4]);
    exact = exact && (float)h[0] == f[k] && (float)h[1] == f[k + 4];
    r[k] = __builtin_bit_cast(uint32_t, h);
  }
  return u32x4_t{r[0], r[1], r[2], r[3]};
}

// The same in the k order (0, 2, 4, 6, 1, 3, 5, 7) of an A copy stored in
// even / odd order: the converter's pairs are used as they come.
__device__ __forceinline__ u32x4_t int4x8_minus_zero_even_odd(uint32_t q, float zf) {
  const uint32_t l = q & 0x0F0F0F0Fu;         // codes k = 0, 2, 4, 6
  const uint32_t h = (q >> 4) & 0x0F0F0F0Fu;  // codes k = 1, 3, 5, 7
  const f32x2_t e0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(l, 512.0f, false);  // k0, k2
  const f32x2_t e1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(l, 512.0f, true);   // k4, k6
  const f32x2_t o0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(h, 512.0f, false);  // k1, k3
  const f32x2_t o1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(h, 512.0f, true);   // k5, k7
  u32x4_t r;
  r[0] = pack_bf16x2(e0[0] - zf, e0[1] - zf);
  r[1] = pack_bf16x2(e1[0] - zf, e1[1] - zf);
  r[2] = pack_bf16x2(o0[0] - zf, o0[1] - zf);
  r[3] = pack_bf16x2(o1[0] - zf, o1[1] - zf);
  return r;
}

// Workgroup barrier that orders LDS accesses only: unlike __syncthreads() it
// does not wait for this wave's outstanding global loads (the fences carry
// the local address space alone, so only lgkmcnt is drained).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---- fused epilogue -------------------------------------------------------------

// Activations in fp32, branch-free, from the hardware base-2 exponential and
// reciprocal (each about 1 ulp): with sigma(x) = 1 / (1 + 2^(-x log2 e)),
//   SiLU(x) = x sigma(x);
//   GELU, tanh form: 0.5 x (1 + tanh(u)) = x sigma(2u), u = sqrt(2/pi) (x + 0.044715 x^3)
// (since 1 + tanh(u) = 2 sigma(2u)).  Saturation is exact: 2^(+large) = inf
// gives sigma = 0, 2^(-large) = 0 gives sigma = 1.
__device__ __forceinline__ float sigmoid_fast(float x) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}
__device__ __forceinline__ float act_silu(float v) { return v * sigmoid_fast(v); }
__device__ __forceinline__ float act_gelu_tanh(float v) {
  const float u = 0.7978845608028654f * __builtin_fmaf(0.044715f * v, v * v, v);
  return v * sigmoid_fast(2.f * u);
}
__device__ __forceinline__ float act_relu(float v) { return v > 0.f ? v : 0.f; }

// C[m, n] = act(alpha * c + bias[n]) + beta * R[m, n] on the fp32 accumulator
// c, given the operands already loaded (b = bias[n] or 0, r = R[m, n] or
// unused); the caller stores the result once (fp32, or bf16 RNE).
template <class E>
__device__ __forceinline__ float epilogue_value(const E& e, float c, float b, float r) {
  float v = __builtin_fmaf(e.alpha, c, b);
  if (e.act == 1) {
    v = act_relu(v);
  } else if (e.act == 2) {
    v = act_silu(v);
  } else if (e.act == 3) {
    v = act_gelu_tanh(v);
  }
  return e.res ? __builtin_fmaf(e.beta, r, v) : v;
}

// one residual element (C's dtype) as fp32
template <bool OUT_F32>
__device__ __forceinline__ float residual_at(const void* res, int64_t mn) {
  return OUT_F32 ? reinterpret_cast<const float*>(res)[mn]
                 : bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(res)[mn]);
}

// ---- MFMA ---------------------------------------------------------------------

// D(16x16 fp32) += A(16x32 bf16) B(32x16 bf16).  Lane l supplies row l%16 of A
// and column l%16 of B over the 8 k-slots 8*(l/16) .. +7, and holds D rows
// 4*(l/16) .. +3 of column l%16.  The k-slot order is immaterial as long as A
// and B use the same one.
__device__ __forceinline__ f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t d) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), d, 0, 0, 0);
}
// the same with fp16 operands
__device__ __forceinline__ f32x4_t mfma16x16x32_f16(u32x4_t a, u32x4_t b, f32x4_t d) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), d,
                                                0, 0, 0);
}

}  // namespace w4a16
