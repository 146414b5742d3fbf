/*
 * w4a16_oracle.c -- plain, slow CPU reference for the W4A16 dequantise-GEMM
 *
 *     C = A . dequant(B)^T
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test-suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or constant with the
 * HIP library under weight_only_bit_w4a16_amd/csrc.
 *
 * Every quantity is computed in IEEE binary64 from the definitions, one
 * element at a time, with no blocking or reordering:
 *   - a weight is the EXACT real value of its 4-bit code times its scale
 *     (binary64 holds it exactly: at most 12 significant bits);
 *   - a GEMM output is the fp64 sum over k ascending of a[m,k] * w[n,k];
 *   - the bf16 copy of a weight is that exact value rounded once, to nearest,
 *     ties to even.
 *
 * Sources (page titles; the pages are the four documents this library follows):
 *   [KB]  "megakernel_int4_weight_decode.py" task spec, section "The weight
 *         format" and the nibble-order paragraph of the contract: packed
 *         (out, in/2) bytes, LOW nibble = even input index; scale bf16 and
 *         zero uint8 per 128 contiguous inputs; value = (code - zero) * scale,
 *         subtraction first.  Its "Precision" section: fp32-or-better
 *         accumulation; the bf16 copy of a weight is a rounding of the exact
 *         value.
 *   [MJ]  "Matmul2dFp4" (Mojo, Apple GPU) struct reference, methods "run" /
 *         "run_smem_decode": NVFP4 operands packed (N, K/2) uint8 and scales
 *         (N, K/16) float8_e4m3fn; weight = decode_e2m1(code) * |scale|.
 *   [TL]  "example_dequant_gemm_bf16_fp4_hopper.py", helper
 *         _tir_u8_to_f4_to_bf16: fp4 is sign / 2 exponent bits / 1 mantissa
 *         bit with exponent bias 1 (its bf16 exponent offset of 126 is
 *         127 - 1); the kernel computes C = A @ B^T with B (N, K/2) uint8.
 *   The e4m3 (bias 7, no infinities, S.1111.111 = NaN) and e8m0 (2^(E-127),
 *   0xFF = NaN) element encodings are the OCP 8-bit floating-point and
 *   microscaling formats, the public definitions the formats above name.
 *
 * Readings where the pages are silent or disagree:
 *   - e2m1 codes with a zero exponent field are subnormal: 0 and 0.5 (and
 *     their negatives).  [TL]'s bit assembly would give 0.5 and 0.75 for
 *     them; it is only right for exponent fields 1..3.
 *   - the NVFP4 scale enters by magnitude, as [MJ] writes |scale|.
 *   - the int4 zero byte is used as the integer it holds (0..15 for valid
 *     data), with no masking.
 *   - the int4 group is a parameter of the format ([KB]'s configuration
 *     carries it as `group`, 128 in its fixture): formats 3 and 4 are the
 *     same asymmetric int4 with groups of 32 and 64 contiguous inputs.
 *   - groups start at k = 0 and run along K ([KB]'s group index i // 128);
 *     when K is not a multiple of the group, the last group of a row is the
 *     shorter rest with its own scale (and zero): ceil(K/G) per row.
 *   - format 5, symmetric int4: [KB] names only the cost of ignoring its
 *     weights' zero point; the symmetric encoding read here is the usual one
 *     for unsigned 4-bit codes -- no zero array, the zero point of every
 *     group is the code midpoint 8, value = (code - 8) * scale, bf16 scale
 *     per 128 contiguous inputs.
 *   - NaN inputs produce a NaN weight; the rounded bf16 NaN is 0x7FC0 (sign
 *     kept).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_INT4_G128 0
#define ORC_NVFP4 1
#define ORC_MXFP4 2
#define ORC_INT4_G32 3
#define ORC_INT4_G64 4
#define ORC_INT4_SYM 5
#define ORC_NFORMATS 6

static int is_int4(int fmt) {
  return fmt == ORC_INT4_G128 || fmt == ORC_INT4_G32 || fmt == ORC_INT4_G64 ||
         fmt == ORC_INT4_SYM;
}

/* ---- element decoders ---------------------------------------------------- */

/* bfloat16 bits -> real value: sign, 8-bit exponent (bias 127), 7-bit
 * mantissa; exponent 0 is subnormal (m * 2^-133), exponent 255 is inf/NaN. */
double orc_bf16_value(uint16_t h) {
  int s = h >> 15, e = (h >> 7) & 0xFF, m = h & 0x7F;
  double mag;
  if (e == 0xFF)
    mag = m ? NAN : INFINITY;
  else if (e == 0)
    mag = ldexp((double)m, -133);
  else
    mag = ldexp(1.0 + m / 128.0, e - 127);
  return s ? -mag : mag;
}

/* e2m1 code (low 4 bits of c) -> real value: sign bit 3, exponent bits 2:1
 * with bias 1, mantissa bit 0.  Exponent 0 is subnormal: 0.5 * m. */
double orc_e2m1_value(unsigned c) {
  int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -mag : mag;
}

/* float8 e4m3 ("fn": finite-only) byte -> real value: sign bit 7, exponent
 * bits 6:3 with bias 7, mantissa bits 2:0; exponent 0 is subnormal
 * (m/8 * 2^-6); exponent 15 with mantissa 7 is NaN (no infinities). */
double orc_e4m3_value(uint8_t b) {
  int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
  double mag;
  if (e == 15 && m == 7)
    mag = NAN;
  else if (e == 0)
    mag = ldexp(m / 8.0, -6);
  else
    mag = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* e8m0 byte -> 2^(E - 127); 0xFF is NaN. */
double orc_e8m0_value(uint8_t E) {
  if (E == 0xFF) return NAN;
  return ldexp(1.0, (int)E - 127);
}

/* Round a real value (held exactly in binary64) to bfloat16: to nearest,
 * ties to even, with bf16's subnormals (quantum 2^-133 below 2^-126) and
 * overflow to infinity.  Written out from the definition of the format. */
uint16_t orc_round_bf16(double x) {
  if (isnan(x)) return (uint16_t)(signbit(x) ? 0xFFC0 : 0x7FC0);
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | 0x7F80);
  int ex;
  frexp(a, &ex);            /* a = f * 2^ex with f in [0.5, 1) */
  int E = ex - 1;           /* a in [2^E, 2^(E+1)) */
  int qexp = (E < -126) ? -133 : E - 7; /* quantum: 8 significant bits */
  double n = ldexp(a, -qexp);            /* exact: a scaled by a power of 2 */
  double fl = floor(n), frac = n - fl;
  double r = fl;
  if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) == 1.0)) r = fl + 1.0;
  if (E < -126) {
    /* subnormal range: the encoding is the multiple of 2^-133 itself; r = 128
       is exactly the smallest normal, whose encoding is also 128 (0x0080). */
    return (uint16_t)(sign | (uint16_t)r);
  }
  if (r == 256.0) { /* rounded up into the next binade */
    r = 128.0;
    E += 1;
  }
  if (E > 127) return (uint16_t)(sign | 0x7F80);
  return (uint16_t)(sign | (uint16_t)((E + 127) << 7) | (uint16_t)(r - 128.0));
}

/* ---- weights --------------------------------------------------------------- */

static int64_t group_of(int fmt) {
  switch (fmt) {
    case ORC_INT4_G128: return 128;
    case ORC_NVFP4: return 16;
    case ORC_MXFP4: return 32;
    case ORC_INT4_G32: return 32;
    case ORC_INT4_SYM: return 128;
    default: return 64; /* ORC_INT4_G64 */
  }
}

/* The 4-bit code of element (n, k): byte (n, k/2), low nibble for even k,
 * high nibble for odd k ([KB] nibble order). */
static unsigned code_at(const uint8_t* packed, int64_t K, int64_t n, int64_t k) {
  uint8_t b = packed[n * (K / 2) + k / 2];
  return (k % 2 == 0) ? (b & 0xF) : (b >> 4);
}

/* Exact real weight w[n, k]. */
double orc_weight(int fmt, const uint8_t* packed, const void* scales,
                  const uint8_t* zeros, int64_t N, int64_t K, int64_t n,
                  int64_t k) {
  (void)N;
  int64_t G = group_of(fmt);
  int64_t g = k / G, groups = (K + G - 1) / G; /* the last group may be shorter */
  unsigned code = code_at(packed, K, n, k);
  if (is_int4(fmt)) {
    double s = orc_bf16_value(((const uint16_t*)scales)[n * groups + g]);
    int z = (fmt == ORC_INT4_SYM) ? 8 : zeros[n * groups + g];
    return (double)((int)code - z) * s; /* subtraction first, then scale */
  }
  double v = orc_e2m1_value(code);
  uint8_t sb = ((const uint8_t*)scales)[n * groups + g];
  double s = (fmt == ORC_NVFP4) ? fabs(orc_e4m3_value(sb)) : orc_e8m0_value(sb);
  return v * s;
}

/* Dequantise the whole (N, K) weight: exact values into w_exact (may be NULL)
 * and their bf16 roundings into w_bf16 (may be NULL).  Returns 0, or -1 on a
 * bad format / shape. */
int orc_dequant(int fmt, const uint8_t* packed, const void* scales,
                const uint8_t* zeros, int64_t N, int64_t K, double* w_exact,
                uint16_t* w_bf16) {
  if (fmt < 0 || fmt >= ORC_NFORMATS || N < 0 || K <= 0 || K % 2 != 0) return -1;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      double w = orc_weight(fmt, packed, scales, zeros, N, K, n, k);
      if (w_exact) w_exact[n * K + k] = w;
      if (w_bf16) w_bf16[n * K + k] = orc_round_bf16(w);
    }
  return 0;
}

/* ---- GEMM ------------------------------------------------------------------ */

/* One output element: C[m,n] = sum_k a[m,k] * w[n,k] in fp64, k ascending,
 * and S[m,n] = sum_k |a[m,k] * w[n,k]| (the scale of the error gate).
 * wrow holds the K weights of row n.  */
static void dot_row(const uint16_t* A, int64_t K, int64_t m, const double* wrow,
                    double* c, double* s) {
  double acc = 0.0, mag = 0.0;
  for (int64_t k = 0; k < K; ++k) {
    double p = orc_bf16_value(A[m * K + k]) * wrow[k];
    acc += p;
    mag += fabs(p);
  }
  *c = acc;
  *s = mag;
}

/* Full reference GEMM.  C and S are (M, N) row-major fp64.  With
 * weights_bf16 != 0 the weights are first rounded to bf16 (a diagnostic that
 * separates weight rounding from accumulation error).  Rows of the weight are
 * decoded one at a time; the loop over n may run on several threads, which
 * changes no result.  Returns 0, or -1 on a bad format / shape. */
int orc_gemm(int fmt, const uint16_t* A, const uint8_t* packed,
             const void* scales, const uint8_t* zeros, int64_t M, int64_t N,
             int64_t K, int weights_bf16, double* C, double* S) {
  if (fmt < 0 || fmt >= ORC_NFORMATS || M < 0 || N < 0 || K <= 0 || K % 2 != 0)
    return -1;
  int err = 0;
#pragma omp parallel
  {
    double* wrow = (double*)malloc(sizeof(double) * (size_t)K);
    if (!wrow) {
#pragma omp atomic write
      err = -1;
    } else {
#pragma omp for schedule(static)
      for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
          double w = orc_weight(fmt, packed, scales, zeros, N, K, n, k);
          wrow[k] = weights_bf16 ? orc_bf16_value(orc_round_bf16(w)) : w;
        }
        for (int64_t m = 0; m < M; ++m)
          dot_row(A, K, m, wrow, &C[m * N + n], &S[m * N + n]);
      }
      free(wrow);
    }
  }
  return err;
}

/* Sampled reference: the same per-element definition at `count` (m, n)
 * positions, for shapes whose full product is too large for this oracle. */
int orc_gemm_at(int fmt, const uint16_t* A, const uint8_t* packed,
                const void* scales, const uint8_t* zeros, int64_t M, int64_t N,
                int64_t K, int64_t count, const int64_t* m_idx,
                const int64_t* n_idx, double* C, double* S) {
  if (fmt < 0 || fmt >= ORC_NFORMATS || K <= 0 || K % 2 != 0) return -1;
  for (int64_t i = 0; i < count; ++i)
    if (m_idx[i] < 0 || m_idx[i] >= M || n_idx[i] < 0 || n_idx[i] >= N) return -1;
  int err = 0;
#pragma omp parallel
  {
    double* wrow = (double*)malloc(sizeof(double) * (size_t)K);
    if (!wrow) {
#pragma omp atomic write
      err = -1;
    } else {
#pragma omp for schedule(dynamic, 16)
      for (int64_t i = 0; i < count; ++i) {
        for (int64_t k = 0; k < K; ++k)
          wrow[k] = orc_weight(fmt, packed, scales, zeros, N, K, n_idx[i], k);
        dot_row(A, K, m_idx[i], wrow, &C[i], &S[i]);
      }
      free(wrow);
    }
  }
  return err;
}

/* ---- fused epilogue ----------------------------------------------------------
 *
 *     y[m, n] = act(alpha * c[m, n] + bias[n]) + beta * R[m, n]
 *
 * on the exact (binary64) GEMM value c.  Sources: [TX] "gemm.rst", the
 * alpha / beta parameters -- D = alpha * A@B + beta * C, and C is not read
 * when beta is 0 (D starts from C only when beta is 1, else from 0); [MJ]
 * "Matmul2dFp4", the optional fused per-element (row, col) epilogue; [KB]
 * "Precision" -- residual adds in fp32 or better.  The pages name no
 * activation; the ones offered are ReLU, SiLU (x times the logistic
 * function) and GELU in its tanh form.  Reading: bias is added before the
 * activation, the residual after it (a transformer's residual stream); R is
 * read only when present and beta != 0.
 */
#define ORC_ACT_NONE 0
#define ORC_ACT_RELU 1
#define ORC_ACT_SILU 2
#define ORC_ACT_GELU_TANH 3

double orc_activation(int act, double x) {
  switch (act) {
    case ORC_ACT_NONE: return x;
    case ORC_ACT_RELU: return x > 0.0 ? x : 0.0;
    case ORC_ACT_SILU: return x / (1.0 + exp(-x));
    case ORC_ACT_GELU_TANH: {
      const double u = sqrt(2.0 / 3.14159265358979323846) * (x + 0.044715 * x * x * x);
      return 0.5 * x * (1.0 + tanh(u));
    }
    default: return NAN;
  }
}

/* In place on y (M x N, row-major): y holds c on entry.  bias: bf16 bits (N)
 * or NULL; R: binary64 (M x N) or NULL.  Returns 0, or -1 on a bad
 * activation code. */
int orc_epilogue(int64_t M, int64_t N, double* y, double alpha, const uint16_t* bias,
                 int act, double beta, const double* R) {
  if (act < ORC_ACT_NONE || act > ORC_ACT_GELU_TANH) return -1;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      double v = alpha * y[m * N + n];
      if (bias) v += orc_bf16_value(bias[n]);
      v = orc_activation(act, v);
      if (R && beta != 0.0) v += beta * R[m * N + n];
      y[m * N + n] = v;
    }
  return 0;
}

/* Number of threads the parallel loops above use (1 without OpenMP). */
int orc_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Set the number of threads of later parallel loops (timing only; the
 * results do not depend on it: each output element is one thread's sum). */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
  extern void omp_set_num_threads(int);
  omp_set_num_threads(n > 0 ? n : 1);
#else
  (void)n;
#endif
}
