// ragged.hip -- W4A16 GEMM for K an odd multiple of 16 (K % 32 == 16):
// C = A . dequant(B)^T, any M and N, every weight format, fp32 accumulation.
//
// Page "Matmul2dFp4" (Mojo) sizes the NVFP4 scales (N, ceil(K/16)): K needs
// only to be a multiple of the 16-code scale block.  A packed row of K/2
// bytes is then 8-byte aligned but not 16-byte aligned, so the 16-byte weight
// loads and global -> LDS copies of the other kernels do not apply.  This
// kernel reads each lane's 8 codes of an MFMA step with one 4-byte load
// (K/2 - byte rows at 8-byte alignment, 4-byte offsets inside them) and its 8
// activations with one 16-byte load (an A row is K * 2 = 32 * odd bytes, so
// every 8-value piece is 16-byte aligned); the last step's upper 16 codes
// lie past K and read as zero.  It is the correct, simple path for a rare
// shape: no LDS staging, no split of K.
//
// Workgroup: 4 waves, 64 output columns x 16 rows; wave w owns columns
// 16w .. 16w+15.  MFMA 16x16x32 with A as the first operand: lane l supplies
// A row m0 + l%16 and weight row n0 + l%16 over k-slots 8 (l/16) .. +7 of each
// 32-code step, and ends holding output rows m0 + 4 (l/16) .. +3 of column
// n0 + l%16.  Decode per step:
//   * int4 (groups of 32, 64, 128 and symmetric): code - zero exact in bf16,
//     the step's 32 codes lie in one group, whose scale (the lane's own
//     column's) multiplies the step's sum: exact weights;
//   * NVFP4 / MXFP4: the scale applied in the decode (exact in bf16).
#include "common.hpp"
#include "kernels.hpp"

namespace w4a16 {

namespace {

constexpr int kRaggedCols = 64;

template <int FMT, bool OUT_F32>
__global__ __launch_bounds__(256) void ragged_kernel(const uint16_t* __restrict__ A,
                                                     const uint8_t* __restrict__ packed,
                                                     const void* __restrict__ scales,
                                                     const uint8_t* __restrict__ zeros,
                                                     void* __restrict__ C, int M, int N, int K,
                                                     Epilogue epi) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nl = lane & 15;
  const int g = lane >> 4;
  const int n0 = (int)blockIdx.x * kRaggedCols + 16 * wave;
  const int m0 = (int)blockIdx.y * 16;
  const int n = n0 + nl;       // weight row supplied, output column held
  const int ma = m0 + nl;      // A row supplied
  constexpr int G = FormatTraits<FMT>::kGroup;
  const int groups = (K + G - 1) / G;
  const uint32_t rowb = (uint32_t)K >> 1;
  const bool nok = n < N, mok = ma < M;
  // descriptors over exactly the valid rows: anything else reads as 0
  const rsrc_t wr = make_rsrc(packed + (int64_t)n0 * rowb, (uint32_t)max(0, min(16, N - n0)) * rowb);
  const rsrc_t ar = make_rsrc(A + (int64_t)m0 * K, (uint32_t)max(0, min(16, M - m0)) * (uint32_t)K * 2u);

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  const int steps = (K + 31) / 32;
  for (int s = 0; s < steps; ++s) {
    const int k0 = 32 * s + 8 * g;   // the lane's first k (K % 8 == 0: all 8 valid or none)
    const bool kok = k0 < K;
    const u32x4_t a = buf_load_b128(ar, kok ? ((uint32_t)nl * (uint32_t)K + (uint32_t)k0) * 2u : kBufferOOB);
    const uint32_t q = buf_load_b32(wr, kok ? (uint32_t)nl * rowb + (uint32_t)(k0 >> 1) : kBufferOOB);
    if constexpr (is_int4(FMT)) {
      // the step (32 codes from k = 32 s) lies in one group; its scale and zero
      const int gi = (32 * s) / G;
      const float sc = nok ? bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(scales)[(int64_t)n * groups + gi]) : 0.f;
      const float zf = has_zeros(FMT) ? (nok ? (float)zeros[(int64_t)n * groups + gi] : 0.f) : (float)kSymZero;
      const f32x4_t p = mfma16x16x32(a, int4x8_minus_zero(q, zf), f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(sc, p[r], acc[r]);
    } else if constexpr (FMT == kNvfp4) {
      const uint32_t sb = (nok && kok) ? reinterpret_cast<const uint8_t*>(scales)[(int64_t)n * groups + k0 / 16] : 0u;
      acc = mfma16x16x32(a, fp4x8_to_bf16_fscale(q, e4m3_magnitude(sb)), acc);
    } else {
      const uint32_t E = (nok && kok) ? reinterpret_cast<const uint8_t*>(scales)[(int64_t)n * groups + k0 / 32] : 0u;
      acc = mfma16x16x32(a, fp4x8_to_bf16_escale(q, e8m0_as_exponent_scale(E)), acc);
    }
  }
  (void)mok;

  // lane holds rows m0 + 4g .. +3 of column n
  if (!nok) return;
  float b = 0.f;
  if (epi.on && epi.bias) b = bf16_bits_to_f32(epi.bias[n]);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = m0 + 4 * g + r;
    if (m >= M) continue;
    const int64_t mn = (int64_t)m * N + n;
    float v = acc[r];
    if (epi.on) v = epilogue_value(epi, v, b, epi.res ? residual_at<OUT_F32>(epi.res, mn) : 0.f);
    if constexpr (OUT_F32)
      reinterpret_cast<float*>(C)[mn] = v;
    else
      reinterpret_cast<__bf16*>(C)[mn] = (__bf16)v;
  }
}

template <int FMT, bool OUT_F32>
hipError_t launch_fmt(const GemmArgs& a) {
  // grid y: 16-row slices, at most 65535 per launch (taller A: several launches)
  const int64_t es = OUT_F32 ? 4 : 2;
  const int64_t chunk = (int64_t)65535 * 16;
  for (int64_t m = 0; m < a.M; m += chunk) {
    const int64_t rows = a.M - m < chunk ? a.M - m : chunk;
    Epilogue epi = a.epi;
    if (epi.res) epi.res = static_cast<const uint8_t*>(epi.res) + m * a.N * es;
    const dim3 grid((unsigned)((a.N + kRaggedCols - 1) / kRaggedCols), (unsigned)((rows + 15) / 16));
    const hipError_t e = launch_kernel(ragged_kernel<FMT, OUT_F32>, grid, dim3(256), 0, a.stream,
                                       a.A + m * a.K, a.packed, a.scales, a.zeros,
                                       static_cast<uint8_t*>(a.C) + m * a.N * es, (int)rows, (int)a.N,
                                       (int)a.K, epi);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_ragged(const GemmArgs& a) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  switch (a.fmt * 2 + (a.out_f32 ? 1 : 0)) {
    case 0: return launch_fmt<kInt4, false>(a);
    case 1: return launch_fmt<kInt4, true>(a);
    case 2: return launch_fmt<kNvfp4, false>(a);
    case 3: return launch_fmt<kNvfp4, true>(a);
    case 4: return launch_fmt<kMxfp4, false>(a);
    case 5: return launch_fmt<kMxfp4, true>(a);
    case 6: return launch_fmt<kInt4G32, false>(a);
    case 7: return launch_fmt<kInt4G32, true>(a);
    case 8: return launch_fmt<kInt4G64, false>(a);
    case 9: return launch_fmt<kInt4G64, true>(a);
    case 10: return launch_fmt<kInt4Sym, false>(a);
    default: return launch_fmt<kInt4Sym, true>(a);
  }
}

}  // namespace w4a16
