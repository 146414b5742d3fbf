// skinny.hip -- W4A16 GEMM for few activation rows (M <= 16 per slice), the
// decode regime that the "megakernel_int4_weight_decode.py" spec describes as
// pure weight bandwidth: its performance notes ask for 128-bit weight loads,
// unpacking in registers right before the multiply-accumulate, and the
// group's scale / zero kept in registers across the group.
//
// Layout of the work (MI355X-specific; none of the pages' kernels is used):
//   * one workgroup = one 16-column slice of C (16 weight rows) x one 16-row
//     slice of A; its W waves split K, each taking every W-th k-block of 128;
//   * lane l of a wave owns weight row n = n0 + l%16 and, inside a k-block,
//     the 32 consecutive codes of chunk l/16: one 16-byte load per k-block;
//     the four lanes of a row read 64 contiguous bytes;
//   * the 32 codes feed four bf16 MFMA 16x16x32 steps (8 codes per lane per
//     step); the matching A values (row m = m0 + l%16) come straight from
//     global memory / L2, in the same k order;
//   * partial sums of the W waves are added through LDS at the end (split-K
//     inside the workgroup: no workspace, no atomics, deterministic).
// Decode per format:
//   * int4: codes become the exact bf16 values 128 + code; a second MFMA per
//     step with the constant -(128 + zero) adds sum_k a_k (-(128 + zero)) to
//     the same accumulator, so the k-block's accumulator holds
//     sum_k a_k (code_k - zero) exactly as the MFMA sums it; the group scale
//     multiplies that once per k-block (k-block = int4 group);
//   * NVFP4: e2m1 -> fp32, times |e4m3 scale| (exact), -> bf16 (exact);
//   * MXFP4: hardware e2m1 conversion scaled by 2^(E-127) (exact).
#include "common.hpp"
#include "kernels.hpp"

namespace w4a16 {

namespace {

constexpr int kMaxWaves = 16;

template <int FMT, bool OUT_F32, int U>
__global__ __launch_bounds__(64 * kMaxWaves) void skinny_kernel(
    const uint16_t* __restrict__ A, const uint8_t* __restrict__ packed,
    const void* __restrict__ scales, const uint8_t* __restrict__ zeros, void* __restrict__ C,
    int M, int N, int K) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int waves = blockDim.x >> 6;
  const int nl = lane & 15;  // weight row within the slice / A row supplied
  const int g = lane >> 4;   // 32-code chunk within the k-block
  const int n0 = blockIdx.x * 16;
  const int m0 = blockIdx.y * 16;
  const int n = n0 + nl;
  const int nrow = n < N ? n : N - 1;  // clamped: rows past N are computed, never stored
  const int am = m0 + nl;
  const bool a_ok = am < M;
  const int chunks = K >> 5;           // 32-code chunks per row
  const int KB = (chunks + 3) >> 2;    // 128-code k-blocks (last may be partial)
  constexpr int G = FormatTraits<FMT>::kGroup;
  const int groups = K / G;

  const uint8_t* prow = packed + (int64_t)nrow * (K >> 1);
  const uint16_t* arow = A + (int64_t)(a_ok ? am : 0) * K;

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};

  for (int kb0 = wave; kb0 < KB; kb0 += waves * U) {
    u32x4_t q[U];
    u32x4_t a[U][4];
    uint32_t sraw[U];
    uint32_t zraw[U];
    // ---- issue every load of U k-blocks before any arithmetic -------------
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = kb0 + u * waves;
      const int c = kb * 4 + g;
      const bool ok = (kb < KB) && (c < chunks);
      q[u] = ok ? *reinterpret_cast<const u32x4_t*>(prow + (int64_t)c * 16) : u32x4_t{0, 0, 0, 0};
      if constexpr (FMT == kInt4) {
        const int gi = (int64_t)nrow * groups + kb;
        sraw[u] = ok ? reinterpret_cast<const uint16_t*>(scales)[gi] : 0u;
        zraw[u] = ok ? zeros[gi] : 0u;
      } else if constexpr (FMT == kNvfp4) {
        // the chunk's two e4m3 scales (blocks 2c and 2c+1), one 16-bit load
        sraw[u] = ok ? reinterpret_cast<const uint16_t*>(
                           reinterpret_cast<const uint8_t*>(scales) + (int64_t)nrow * groups)[c]
                     : 0u;
      } else {
        sraw[u] = ok ? reinterpret_cast<const uint8_t*>(scales)[(int64_t)nrow * groups + c] : 0u;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a[u][j] = (ok && a_ok)
                      ? *reinterpret_cast<const u32x4_t*>(arow + (int64_t)c * 32 + 8 * j)
                      : u32x4_t{0, 0, 0, 0};
      }
    }
    // ---- decode + MFMA ------------------------------------------------------
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (FMT == kInt4) {
        const u32x4_t nz = int4_neg_offset_zero(zraw[u]);
        f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          d = mfma16x16x32(a[u][j], int4x8_to_bf16_offset128(q[u][j]), d);
          d = mfma16x16x32(a[u][j], nz, d);
        }
        const float s = bf16_bits_to_f32(sraw[u]);
        acc[0] = __builtin_fmaf(s, d[0], acc[0]);
        acc[1] = __builtin_fmaf(s, d[1], acc[1]);
        acc[2] = __builtin_fmaf(s, d[2], acc[2]);
        acc[3] = __builtin_fmaf(s, d[3], acc[3]);
      } else if constexpr (FMT == kNvfp4) {
        const float s0 = e4m3_magnitude(sraw[u] & 0xFFu);
        const float s1 = e4m3_magnitude(sraw[u] >> 8);
        acc = mfma16x16x32(a[u][0], fp4x8_to_bf16_fscale(q[u][0], s0), acc);
        acc = mfma16x16x32(a[u][1], fp4x8_to_bf16_fscale(q[u][1], s0), acc);
        acc = mfma16x16x32(a[u][2], fp4x8_to_bf16_fscale(q[u][2], s1), acc);
        acc = mfma16x16x32(a[u][3], fp4x8_to_bf16_fscale(q[u][3], s1), acc);
      } else {
        const float es = e8m0_as_exponent_scale(sraw[u]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = mfma16x16x32(a[u][j], fp4x8_to_bf16_escale(q[u][j], es), acc);
      }
    }
  }

  // ---- split-K reduction across the waves, through LDS ----------------------
  __shared__ f32x4_t red[kMaxWaves][64];
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  f32x4_t sum = red[0][lane];
  for (int w = 1; w < waves; ++w) {
    const f32x4_t v = red[w][lane];
    sum[0] += v[0];
    sum[1] += v[1];
    sum[2] += v[2];
    sum[3] += v[3];
  }
  if (n >= N) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + 4 * g + i;
    if (m < M) {
      if constexpr (OUT_F32) {
        reinterpret_cast<float*>(C)[(int64_t)m * N + n] = sum[i];
      } else {
        reinterpret_cast<__bf16*>(C)[(int64_t)m * N + n] = (__bf16)sum[i];
      }
    }
  }
}

template <int FMT, bool OUT_F32>
hipError_t launch_fmt(const GemmArgs& a) {
  const int chunks = (int)(a.K >> 5);
  const int KB = (chunks + 3) >> 2;
  // k-blocks per wave: U loads of 16 B in flight per lane per pass
  constexpr int U = 4;
  int waves = (KB + U - 1) / U;
  if (waves > kMaxWaves) waves = kMaxWaves;
  if (waves < 1) waves = 1;
  dim3 grid((unsigned)((a.N + 15) / 16), (unsigned)((a.M + 15) / 16));
  hipLaunchKernelGGL((skinny_kernel<FMT, OUT_F32, U>), grid, dim3(64 * waves), 0, a.stream, a.A,
                     a.packed, a.scales, a.zeros, a.C, (int)a.M, (int)a.N, (int)a.K);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_skinny(const GemmArgs& a) {
  switch (a.fmt * 2 + (a.out_f32 ? 1 : 0)) {
    case 0: return launch_fmt<kInt4, false>(a);
    case 1: return launch_fmt<kInt4, true>(a);
    case 2: return launch_fmt<kNvfp4, false>(a);
    case 3: return launch_fmt<kNvfp4, true>(a);
    case 4: return launch_fmt<kMxfp4, false>(a);
    default: return launch_fmt<kMxfp4, true>(a);
  }
}

}  // namespace w4a16
