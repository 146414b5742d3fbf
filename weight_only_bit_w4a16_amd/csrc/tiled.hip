// tiled.hip -- W4A16 GEMM for many activation rows: C = A . dequant(B)^T with
// A and the PACKED weights staged through LDS and the weights decoded into
// bf16 MFMA B fragments in registers, fp32 accumulation.
//
// Prior art (page titles): the tiled dequant-GEMM of
// "example_dequant_gemm_bf16_fp4_hopper.py" (matmul / main: shared A and
// packed-B tiles, a dequant step, a GEMM with B transposed, a fragment
// accumulator) and the cooperative-decode kernel of "Matmul2dFp4"
// (run_smem_decode: coalesced loads of packed bytes, register-fed MMA).  This
// kernel differs from both: the LDS holds the weights still packed (4 bits,
// a quarter of a bf16 tile) and every wave decodes only the fragments it
// feeds to its own MFMAs, so no bf16 weight tile ever exists in memory.
//
// Workgroup tile 256 x 256 (M x N), k-tile 64, 8 waves as 2 x 4, each wave
// 128 x 64 = 8 x 4 MFMA 16x16x32 tiles.  Two LDS stages: while the waves
// multiply stage s, the next k-tile is in flight from global memory to
// registers, then written to stage s^1.  Inside a k-tile, lane group g (lanes
// 16g .. 16g+15) owns codes 16g .. 16g+15 of each row: one 8-byte LDS read
// per B fragment covers both 32-k MFMA steps, and the A fragment of step s is
// the 8 A values at k = 16g + 8s .. +7 (the same k order for A and B).
#include "common.hpp"
#include "kernels.hpp"

namespace w4a16 {

namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kThreads = 512;
constexpr int A_LD = BK + 8;        // bf16 elements per LDS row of A (144 B: 16-B slots rotate)
constexpr int B_LD = BK / 2 + 8;    // bytes per LDS row of packed B (40 B)
constexpr int S_LD = 4;             // decoded scale slots per B row per k-tile
constexpr int TM = 8, TN = 4;       // MFMA tiles per wave (M, N)

template <int FMT, bool OUT_F32>
__global__ __launch_bounds__(kThreads) void tiled_kernel(const uint16_t* __restrict__ A,
                                                         const uint8_t* __restrict__ packed,
                                                         const void* __restrict__ scales,
                                                         const uint8_t* __restrict__ zeros,
                                                         void* __restrict__ C, int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * A_LD];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BN * B_LD];
  __shared__ float Ss[2][BN * S_LD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 2;  // 0..1
  const int wn = wave & 3;   // 0..3
  const int l16 = lane & 15;
  const int g = lane >> 4;

  const int m_base = blockIdx.y * BM;
  const int n_base = blockIdx.x * BN;
  const int KT = (K + BK - 1) / BK;
  constexpr int G = FormatTraits<FMT>::kGroup;
  const int groups = K / G;

  // ---- global -> register staging of one k-tile --------------------------------
  // A: 256 rows x 8 chunks of 16 B: thread owns chunks tid + 512 i, i = 0..3
  // B: 256 rows x 2 chunks of 16 B: thread owns one
  // scales: thread t < 256 decodes row t's scales for the k-tile
  u32x4_t ra[4];
  u32x4_t rb;
  float rs[S_LD];

  auto load_tile = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + kThreads * i;
      const int row = id >> 3, cc = id & 7;
      const int m = m_base + row;
      const int k = k0 + cc * 8;
      ra[i] = (m < M && k < K) ? *reinterpret_cast<const u32x4_t*>(A + (int64_t)m * K + k)
                               : u32x4_t{0, 0, 0, 0};
    }
    {
      const int row = tid >> 1, half = tid & 1;
      const int n = n_base + row;
      const int k = k0 + half * 32;
      rb = (n < N && k < K)
               ? *reinterpret_cast<const u32x4_t*>(packed + (int64_t)n * (K >> 1) + (k >> 1))
               : u32x4_t{0, 0, 0, 0};
    }
    if (tid < BN) {
      const int n = n_base + tid;
      const int nr = n < N ? n : N - 1;
      if constexpr (FMT == kInt4) {
        const int64_t gi = (int64_t)nr * groups + k0 / 128;
        rs[0] = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(scales)[gi]);
        rs[1] = (float)zeros[gi];
        rs[2] = 0.f;
        rs[3] = 0.f;
      } else if constexpr (FMT == kNvfp4) {
        const uint8_t* sp = reinterpret_cast<const uint8_t*>(scales) + (int64_t)nr * groups + k0 / 16;
#pragma unroll
        for (int j = 0; j < 4; ++j) rs[j] = (k0 + 16 * j < K) ? e4m3_magnitude(sp[j]) : 0.f;
      } else {
        const uint8_t* sp = reinterpret_cast<const uint8_t*>(scales) + (int64_t)nr * groups + k0 / 32;
        rs[0] = e8m0_as_exponent_scale(sp[0]);
        rs[1] = (k0 + 32 < K) ? e8m0_as_exponent_scale(sp[1]) : 0.f;
        rs[2] = 0.f;
        rs[3] = 0.f;
      }
    }
  };

  auto store_tile = [&](int st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + kThreads * i;
      const int row = id >> 3, cc = id & 7;
      *reinterpret_cast<u32x4_t*>(&As[st][row * A_LD + cc * 8]) = ra[i];
    }
    {
      const int row = tid >> 1, half = tid & 1;
      // two 8-byte stores: the LDS row pitch (40 B) is only 8-byte aligned
      u32x2_t* dst = reinterpret_cast<u32x2_t*>(&Bs[st][row * B_LD + half * 16]);
      dst[0] = u32x2_t{rb[0], rb[1]};
      dst[1] = u32x2_t{rb[2], rb[3]};
    }
    if (tid < BN) {
#pragma unroll
      for (int j = 0; j < S_LD; ++j) Ss[st][tid * S_LD + j] = rs[j];
    }
  };

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int t = 0; t < TN; ++t) acc[i][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    const bool has_next = kt + 1 < KT;
    if (has_next) load_tile(kt + 1);

    // B fragments: 16 codes (8 bytes) per lane per tile, both MFMA steps
    u32x2_t bq[TN];
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const int row = wn * 64 + t * 16 + l16;
      bq[t] = *reinterpret_cast<const u32x2_t*>(&Bs[cur][row * B_LD + 8 * g]);
    }
    // a ragged last k-tile (K % 64 == 32) is zero-filled: A = 0 and code 0
    // with a finite scale past K, so both steps run unconditionally
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4_t bf[TN];
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const int row = wn * 64 + t * 16 + l16;
        const float* sc = &Ss[cur][row * S_LD];
        if constexpr (FMT == kInt4) {
          bf[t] = int4x8_to_bf16_weights(bq[t][s], sc[0], sc[1]);
        } else if constexpr (FMT == kNvfp4) {
          bf[t] = fp4x8_to_bf16_fscale(bq[t][s], sc[g]);      // codes 16g.. lie in block g
        } else {
          bf[t] = fp4x8_to_bf16_escale(bq[t][s], sc[g >> 1]); // codes 16g.. lie in block g/2
        }
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * 128 + i * 16 + l16;
        const u32x4_t af = *reinterpret_cast<const u32x4_t*>(&As[cur][row * A_LD + 16 * g + 8 * s]);
#pragma unroll
        for (int t = 0; t < TN; ++t) acc[i][t] = mfma16x16x32(af, bf[t], acc[i][t]);
      }
    }

    if (has_next) store_tile(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds rows 4g..4g+3 of each 16x16 tile, column l16 ----
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const int n = n_base + wn * 64 + t * 16 + l16;
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m_base + wm * 128 + i * 16 + 4 * g + r;
        if (m < M) {
          if constexpr (OUT_F32) {
            reinterpret_cast<float*>(C)[(int64_t)m * N + n] = acc[i][t][r];
          } else {
            reinterpret_cast<__bf16*>(C)[(int64_t)m * N + n] = (__bf16)acc[i][t][r];
          }
        }
      }
    }
  }
}

template <int FMT, bool OUT_F32>
hipError_t launch_fmt(const GemmArgs& a) {
  dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM));
  hipLaunchKernelGGL((tiled_kernel<FMT, OUT_F32>), grid, dim3(kThreads), 0, a.stream, a.A, a.packed,
                     a.scales, a.zeros, a.C, (int)a.M, (int)a.N, (int)a.K);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tiled(const GemmArgs& a) {
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
