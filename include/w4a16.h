/*
 * w4a16.h -- C ABI of the MI355X (gfx950) W4A16 dequantise-GEMM library
 *
 *     C[m, n] = sum_k A[m, k] * W[n, k],   W = dequant(packed, scales, zeros)
 *
 * i.e. C = A . W^T with bf16 activations and 4-bit weights, fp32
 * accumulation.  Plain C: pointers, 64-bit sizes and int status codes; no
 * C++ or framework types cross this boundary.
 *
 * Operations and their sources (page titles):
 *   - The GEMM "C = A @ B^T" with B packed two 4-bit values per byte, shape
 *     (N, K/2): "example_dequant_gemm_bf16_fp4_hopper.py", kernel factory
 *     matmul and its prim_func main.
 *   - Asymmetric int4, group 128: "megakernel_int4_weight_decode.py", section
 *     "The weight format" -- scale bf16 and zero uint8 per 128 contiguous
 *     input elements, value = (code - zero) * scale; the contract's nibble
 *     paragraph -- LOW nibble of byte (n, i) is input 2i, HIGH nibble 2i+1.
 *     The group is a configuration value there (`group`, 128 in its
 *     fixture); W4A16_INT4_G32 / _G64 are the same format with groups of 32
 *     and 64.  W4A16_INT4_SYM is its symmetric form: no zero array, every
 *     group's zero point is the midpoint 8 of the codes 0..15, value =
 *     (code - 8) * scale, groups of 128 (the page measures only what ignoring
 *     the zero point of ITS asymmetric weights costs, in its tolerance table;
 *     the symmetric encoding itself is the usual reading, not the page's).
 *   - NVFP4: "Matmul2dFp4" (Mojo), methods run / run_smem_decode -- packed
 *     (N, K/2) uint8, scales (N, K/16) float8_e4m3fn, value =
 *     e2m1(code) * |scale|.
 *   - MXFP4: e2m1 codes with one e8m0 scale byte E per 32 contiguous inputs,
 *     value = e2m1(code) * 2^(E - 127); same packed layout.
 *   e2m1: sign bit 3, exponent bits 2:1 (bias 1), mantissa bit 0; exponent 0
 *   is subnormal, so the magnitudes are {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
 *
 * Memory: every pointer is a DEVICE pointer owned by the caller; the library
 * never allocates, frees or keeps them.  All arrays are row-major and dense:
 *   A       bf16  (M, K)                    16-byte aligned
 *   packed  uint8 (N, K/2)                  16-byte aligned (or prepacked:
 *           see w4a16_prepack)
 *   scales  int4: bf16 (N, ceil(K/G)), G = 128 / 32 / 64 (128 for INT4_SYM)   2-byte aligned
 *           NVFP4: e4m3 bytes (N, K/16)     2-byte aligned
 *           MXFP4: e8m0 bytes (N, K/32)
 *   zeros   int4 G128 / G32 / G64: uint8 (N, ceil(K/G)); must be NULL for
 *           INT4_SYM, NVFP4 and MXFP4
 *   C       bf16 or fp32 (M, N)             aligned to its element size
 *   W       bf16 (N, K)                     16-byte aligned (dequant output)
 * Shapes: M, N >= 0 (a zero extent is a valid call that enqueues nothing and
 * checks no pointer);
 * 0 < K <= 2^22, K % 16 == 0; M, N < 2^31.  K an odd multiple of 16 (rows of
 * K/2 bytes only 8-byte aligned: the NVFP4 layout of page "Matmul2dFp4" with
 * its (N, ceil(K/16)) scales) runs a separate, simpler kernel
 * (W4A16_PATH_RAGGED) for every format, M and entry point.  Groups
 * start at k = 0 and run along K; when K is not a multiple of the group (int4
 * with groups of 128 or 64), the last group of each row is the shorter rest
 * and has its own scale (and zero), hence ceil(K/G) of them per row.
 * Zero points: the GEMM and the dequantisation take any zero byte 0..255
 * (the format stores 0..15).
 *
 * Streams: `stream` is a hipStream_t (NULL = the default stream).  Calls only
 * enqueue kernels and return; they never synchronise, allocate or read
 * device memory from the host, so they may be captured into a HIP graph.
 * Results are deterministic: the same inputs give bit-identical outputs.
 *
 * Errors: every argument is checked on the host BEFORE anything is enqueued;
 * a failed check returns its code and enqueues nothing.  A launch failure
 * reported by the HIP runtime for the call's own launch returns W4A16_ERR_HIP
 * (an earlier error of the calling thread is neither reported nor cleared);
 * so does a launch whose grid would exceed 2^32 - 1 work-items along one
 * dimension (refused before it is enqueued): only weight matrices of more
 * than 2^26 rows (output columns) can reach that, on the kernels that give
 * every 16 to 64 rows a workgroup of their own (K % 128 != 0, int4 groups of
 * 32 / 64, or more than 16 rows of A).
 *
 * Threads: the library's only global state is a cache of device properties
 * (compute units per device, resident workgroups per kernel), filled on first
 * use through atomics and a mutex; calls are safe from several host threads.
 * The kernel choice and the summation order depend only on the format, the
 * flags and M, N, K: nothing read at run time (environment, device state)
 * changes the output bits.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- `format` argument: weight format, OR-ed with option flags ---------- */
#define W4A16_INT4_G128 0   /* asymmetric int4, bf16 scale + u8 zero per 128 */
#define W4A16_NVFP4 1       /* e2m1 codes, e4m3 scale per 16                  */
#define W4A16_MXFP4 2       /* e2m1 codes, e8m0 scale per 32                  */
#define W4A16_INT4_G32 3    /* the int4 format with groups of 32 inputs       */
#define W4A16_INT4_G64 4    /* the int4 format with groups of 64 inputs       */
#define W4A16_INT4_SYM 5    /* symmetric int4: bf16 scale per 128, zero 8     */
#define W4A16_FORMAT_MASK 0xFF

#define W4A16_OUT_BF16 0x000 /* C is bf16, rounded to nearest even (default) */
#define W4A16_OUT_F32 0x100  /* C is fp32                                    */
/* `packed` is in the prepacked layout (see w4a16_prepack), K % 128 == 0; taken
 * by every GEMM entry point, w4a16_dequant and w4a16_gemm_path */
#define W4A16_PREPACKED 0x400

/* Kernel choice for w4a16_gemm.  AUTO picks the skinny (split-K, register
 * decode) kernel for M <= 16.  Above that, while the LDS-tiled MFMA kernel
 * would have fewer than 256 tiles of 256 x 256: the mid kernel (tiles of 32
 * columns x up to 64 rows, split-K, each weight decoded once per tile) when it
 * has at least 160 and at most 896 workgroups (3.5 rounds of 256), the
 * skinny kernel (M <= 384) when it would have fewer, else the tiled kernel
 * (128 x 128 tiles below 192 large ones); with 256 or more large tiles, the
 * mid kernel for M <= 64 and the tiled kernel above.  The others force one
 * kernel at any M (the skinny kernel then walks M in slices of 16 rows, the
 * mid kernel in tiles of 32 to 64). */
#define W4A16_PATH_AUTO 0x0000
#define W4A16_PATH_SKINNY 0x1000
#define W4A16_PATH_TILED 0x2000
#define W4A16_PATH_MID 0x3000
#define W4A16_PATH_MASK 0x3000
/* returned by w4a16_gemm_path (never a flag): the kernel for K % 32 == 16,
 * which runs whatever PATH flag is given */
#define W4A16_PATH_RAGGED 0x4000

/* ---- status codes --------------------------------------------------------- */
#define W4A16_OK 0
#define W4A16_ERR_FORMAT (-1) /* unknown format or flag bits                 */
#define W4A16_ERR_SHAPE (-2)  /* negative M/N, K <= 0, K % 16 != 0 (K % 128
                                 != 0 with W4A16_PREPACKED), M or N >= 2^31,
                                 or K > 2^22                                */
#define W4A16_ERR_NULL (-3)   /* a required pointer is NULL, or zeros is
                                 non-NULL for a format without zeros
                                 (INT4_SYM, NVFP4, MXFP4)                   */
#define W4A16_ERR_ALIGN (-4)  /* a pointer violates its alignment           */
#define W4A16_ERR_HIP (-5)    /* the HIP runtime rejected a launch, or its
                                 grid would exceed 2^32 - 1 work-items along
                                 a dimension                                */
#define W4A16_ERR_EPILOGUE (-6) /* unknown activation, nonzero reserved field,
                                   or a residual that overlaps C without
                                   being C                                  */
#define W4A16_ERR_OVERLAP (-7)  /* w4a16_prepack's output overlaps its input */

/* C = A . dequant(packed, scales, zeros)^T, accumulated in fp32.
 * format = W4A16_INT4_G128 | W4A16_NVFP4 | W4A16_MXFP4, optionally OR-ed with
 * W4A16_OUT_F32, W4A16_PREPACKED and one W4A16_PATH_* flag.  C is fully overwritten.
 * Accuracy: |C - C_exact| <= 2e-3 * sum_k |A[m,k] W[n,k]| + 1e-6 per element,
 * plus 2^-8 |C_exact| when C is bf16 (C_exact: exact weights, exact sum). */
int w4a16_gemm(int format, const void* A, const void* packed, const void* scales,
               const void* zeros, void* C, int64_t M, int64_t N, int64_t K,
               void* stream);

/* ---- fused epilogue ---------------------------------------------------------
 * w4a16_gemm_ex applies, per output element, on the fp32 accumulator c:
 *     C[m,n] = act(alpha * c + bias[n]) + beta * R[m,n]
 * and rounds once to C's dtype.  The alpha / beta pair is the one of the
 * gemm primitive on page "gemm.rst" (D = alpha * A@B + beta * C, and C is not
 * read when beta is 0); the per-element form is the optional (row, col)
 * epilogue of page "Matmul2dFp4".  The pages name no activation; these are
 * offered: */
#define W4A16_ACT_NONE 0
#define W4A16_ACT_RELU 1      /* max(x, 0)                                   */
#define W4A16_ACT_SILU 2      /* x / (1 + exp(-x))                           */
#define W4A16_ACT_GELU_TANH 3 /* 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) */
typedef struct w4a16_epilogue {
  const void* bias;     /* bf16 (N) device array, or NULL (no bias); 2-byte aligned   */
  const void* residual; /* (M, N) device array in C's dtype, row-major, or NULL; it
                           may be C itself (in place), else must not overlap C;
                           read only when beta != 0; aligned like C              */
  float alpha;          /* multiplies A . W^T (1 for none)                         */
  float beta;           /* multiplies the residual                                 */
  int activation;       /* W4A16_ACT_*                                             */
  int reserved;         /* must be 0                                               */
} w4a16_epilogue;

/* w4a16_gemm with the fused epilogue `ep` (NULL: exactly w4a16_gemm).  The
 * epilogue runs in fp32 in the kernel's store (the tiled and both skinny
 * kernels), so it adds only the bias / residual reads.  Accuracy: the GEMM
 * bound above times |alpha| and the activation's Lipschitz constant (1, 1.1
 * for SiLU, 1.13 for GELU), plus 2^-20 of the magnitudes involved and, for
 * bf16 C, 2^-8 |C_exact|.  Errors as w4a16_gemm, plus W4A16_ERR_EPILOGUE, and
 * W4A16_ERR_ALIGN for a misaligned bias or residual; `ep` is read during the
 * call only. */
int w4a16_gemm_ex(int format, const void* A, const void* packed, const void* scales,
                  const void* zeros, void* C, int64_t M, int64_t N, int64_t K,
                  const w4a16_epilogue* ep, void* stream);

/* Several weight matrices that share one activation matrix A and one K --
 * e.g. the q, k and v projections of a decoder layer, or its gate and up
 * projections, which all multiply the same layer input (page
 * "megakernel_int4_weight_decode.py": the contract table's seven int4 triples
 * per layer, each applied as h . W^T; its spec fuses the decode step to cut
 * the per-kernel overhead its performance section measures, eager vs graph).
 * For i < count:
 *     C[i] = A . dequant(packed[i], scales[i], zeros[i])^T,  C[i] (M, N[i]).
 * `packed`, `scales`, `C` and `N` are HOST arrays of `count` entries (device
 * pointers / sizes), read during the call only; `zeros` is such an array for
 * the int4 formats with zeros and must be NULL for INT4_SYM, NVFP4 and MXFP4.  Each member follows the layout,
 * alignment and accuracy rules of w4a16_gemm.  1 <= count <= W4A16_MAX_GROUP
 * (else W4A16_ERR_SHAPE); members with N[i] == 0 are skipped and their
 * pointers not checked.  The skinny path computes all members in ONE launch;
 * the tiled path launches once per member.  Same error, stream and
 * determinism behaviour as w4a16_gemm. */
#define W4A16_MAX_GROUP 8
int w4a16_gemm_grouped(int format, const void* A, int count, const void* const* packed,
                       const void* const* scales, const void* const* zeros, void* const* C,
                       const int64_t* N, int64_t M, int64_t K, void* stream);

/* ---- batched independent GEMMs -----------------------------------------------
 * Item i computes C_i = A_i . dequant(packed_i, scales_i, zeros_i)^T with its
 * own activations A_i (M, K_i), weights (N_i rows) and output C_i (M, N_i);
 * the items share only the format, the output type and M.  In the decode
 * regime (M <= 16) the items of one (K, N) run in ONE launch (up to 32 items
 * per launch), so the weight matrices of a decoder step (page
 * "megakernel_int4_weight_decode.py": seven int4 projections per layer plus
 * the LM head, and its performance section's per-kernel overhead, eager vs
 * graph) take a handful of launches instead of one each.  Larger M: one
 * launch per item.  Each item's C equals, bit for bit, what w4a16_gemm gives
 * for that item alone.
 * The items must be independent: no item's C may overlap another item's C or
 * any item's input, since items run concurrently and in no fixed order.
 * `items` is a HOST array of `count` entries (device pointers and sizes),
 * read during the call only; every entry follows w4a16_gemm's layout,
 * alignment and zeros rules; entries with N == 0 are skipped and their
 * pointers not checked.  `format`: a weight format, optionally OR-ed with
 * W4A16_OUT_F32 and W4A16_PREPACKED (no W4A16_PATH_* flag).  count == 0 or M == 0 enqueues
 * nothing.  Errors: as w4a16_gemm, every item is checked before anything is
 * enqueued (W4A16_ERR_SHAPE also for count < 0); a launch failure
 * (W4A16_ERR_HIP) may leave the call's earlier launches enqueued. */
typedef struct w4a16_batch_item {
  const void* A;      /* bf16 (M, K) device array, 16-byte aligned            */
  const void* packed; /* uint8 (N, K/2) device array (or prepacked), 16-byte aligned */
  const void* scales; /* per the format, as for w4a16_gemm                    */
  const void* zeros;  /* uint8 zeros for the int4 formats with zeros, else NULL */
  void* C;            /* (M, N) device array, bf16 or fp32                    */
  int64_t N;          /* output columns (weight rows), 0 <= N < 2^31          */
  int64_t K;          /* inputs, 0 < K <= 2^22, K % 16 == 0                   */
} w4a16_batch_item;
int w4a16_gemm_batched(int format, int64_t M, int count, const w4a16_batch_item* items,
                       void* stream);

/* W = dequant(packed, scales, zeros) as bf16 (N, K): each weight's exact value
 * rounded once to nearest even (bit-exact; fp4 weights are exact in bf16 at
 * normal scale ranges).  `format` takes the format bits and W4A16_PREPACKED.
 * A checking path: the GEMM never materialises W. */
int w4a16_dequant(int format, const void* packed, const void* scales,
                  const void* zeros, void* W, int64_t N, int64_t K, void* stream);

/* ---- prepacked weights ------------------------------------------------------
 * Page "megakernel_int4_weight_decode.py", contract section: weights may be
 * repacked once, untimed, when the model is built -- interleaved, pre-ordered
 * for the matrix instruction's fragments, with the scales in a stream of their
 * own -- as long as no bf16 copy of the weights is materialised.  This
 * library's repacking moves whole 16-byte pieces of a packed row (32 codes,
 * nibble order unchanged) into the order in which the lanes of an MFMA
 * 16x16x32 weight fragment read them; scales and zeros keep their layout (they
 * already are arrays of their own, read once per group).  The prepacked array,
 * of w4a16_prepacked_bytes(N, K) = ceil(N/16) * 16 * K/2 bytes, holds for
 * t < ceil(N/16), b < K/128, l < 64, i < 16:
 *     out[((t * (K/128) + b) * 64 + l) * 16 + i]
 *         = packed[(16t + l % 16) * K/2 + 64 b + 16 (l / 16) + i]
 * (zero for rows 16t + l % 16 >= N): tiles of 16 rows, and in a tile one
 * 1-KB block per 128 codes, which a wave of the decode kernels loads as one
 * contiguous kilobyte (the row-major layout spreads it over 16 rows).  Every
 * entry point taking `packed` accepts this layout with W4A16_PREPACKED in
 * `format` and gives bit-identical results to the row-major layout.
 * Requires K % 128 == 0 (else W4A16_ERR_SHAPE); the prepacked array is
 * 16-byte aligned like `packed`.
 * w4a16_prepacked_bytes returns the size, or a negative status for a bad
 * shape.  w4a16_prepack enqueues the reordering on `stream` (host-side
 * checks as w4a16_gemm; `out` must not overlap `packed`: W4A16_ERR_OVERLAP). */
int64_t w4a16_prepacked_bytes(int64_t N, int64_t K);
int w4a16_prepack(const void* packed, void* out, int64_t N, int64_t K, void* stream);

/* Which kernel w4a16_gemm would launch for these arguments, without launching:
 * returns W4A16_PATH_SKINNY, W4A16_PATH_MID, W4A16_PATH_TILED or
 * W4A16_PATH_RAGGED, or a negative status if the format / shape would be
 * rejected.  Host-only. */
int w4a16_gemm_path(int format, int64_t M, int64_t N, int64_t K);

/* Static, NUL-terminated description of a status code. */
const char* w4a16_strerror(int status);

/* Library ABI version (major * 100 + minor). */
int w4a16_version(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
