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
constexpr int TM = 8, TN = 4;       // MFMA tiles per wave (M, N)

// Tile order: workgroups are dealt to the 8 XCDs round-robin by launch
// index, and each XCD has its own L2.  Index i goes to XCD i % 8; the tiles
// of one XCD are taken from a compact block of (tm, tn) so that the
// workgroups resident on an XCD at the same time share A and B tiles in its
// L2.  Within an XCD the order walks blocks of 4 x 8 tiles.
__device__ __forceinline__ void tile_of(int i, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  if (total % 8 != 0 || tiles_m % 4 != 0 || tiles_n % 8 != 0) {
    tm = i / tiles_n;
    tn = i % tiles_n;
    return;
  }
  const int xcd = i % 8, slot = i / 8;          // slot-th tile of this XCD
  const int per_xcd = total / 8;
  const int t = xcd * per_xcd + slot;           // contiguous range per XCD
  const int blk = t / 32, in = t % 32;          // 4 x 8 blocks
  const int bn = tiles_n / 8;
  tm = (blk / bn) * 4 + in / 8;
  tn = (blk % bn) * 8 + in % 8;
}

template <int FMT, bool OUT_F32>
__global__ __launch_bounds__(kThreads) void tiled_kernel(const uint16_t* __restrict__ A,
                                                         const uint8_t* __restrict__ packed,
                                                         const void* __restrict__ scales,
                                                         const uint8_t* __restrict__ zeros,
                                                         void* __restrict__ C, int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * A_LD];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BN * B_LD];
  __shared__ uint32_t Ss[2][BN];  // raw scale (and zero) bytes of each B row for the k-tile

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 2;  // 0..1
  const int wn = wave & 3;   // 0..3
  const int l16 = lane & 15;
  const int g = lane >> 4;

  int tm, tn;
  tile_of(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  const int m_base = tm * BM;
  const int n_base = tn * BN;
  const int KT = (K + BK - 1) / BK;
  constexpr int G = FormatTraits<FMT>::kGroup;
  const int groups = K / G;

  // Buffer descriptors over this workgroup's rows: rows past M / N read as 0.
  const uint32_t arow_b = (uint32_t)K * 2u, brow_b = (uint32_t)K >> 1;
  const rsrc_t ar = make_rsrc(A + (int64_t)m_base * K, (uint32_t)min(BM, M - m_base) * arow_b);
  const rsrc_t br = make_rsrc(packed + (int64_t)n_base * brow_b, (uint32_t)min(BN, N - n_base) * brow_b);
  const int brows = min(BN, N - n_base);
  constexpr int SB = FMT == kInt4 ? 2 : 1;
  const rsrc_t sr = make_rsrc(reinterpret_cast<const uint8_t*>(scales) + (int64_t)n_base * groups * SB,
                              (uint32_t)(brows * groups * SB));
  const rsrc_t zr = make_rsrc(FMT == kInt4 ? zeros + (int64_t)n_base * groups : nullptr,
                              FMT == kInt4 ? (uint32_t)(brows * groups) : 0u);

  // ---- global -> register staging of one k-tile (no use before store) -----------
  // A: 256 rows x 8 chunks of 16 B: thread owns chunks tid + 512 i, i = 0..3
  // B: 256 rows x 2 chunks of 16 B: thread owns one
  // scales: thread t < 256 fetches row t's raw scale bytes for the k-tile
  u32x4_t ra[4];
  u32x4_t rb;
  uint32_t rs0 = 0, rs1 = 0;

  auto load_tile = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + kThreads * i;
      const int row = id >> 3, k = k0 + (id & 7) * 8;
      ra[i] = buf_load_b128(ar, k < K ? (uint32_t)row * arow_b + (uint32_t)k * 2u : kBufferOOB);
    }
    {
      const int row = tid >> 1, k = k0 + (tid & 1) * 32;
      rb = buf_load_b128(br, k < K ? (uint32_t)row * brow_b + (uint32_t)(k >> 1) : kBufferOOB);
    }
    if (tid < BN) {
      const uint32_t rbase = (uint32_t)(tid * groups);
      if constexpr (FMT == kInt4) {
        const uint32_t gi = rbase + (uint32_t)(k0 / 128);
        rs0 = buf_load_b16(sr, gi * 2u);
        rs1 = buf_load_b8(zr, gi);
      } else if constexpr (FMT == kNvfp4) {
        // blocks k0/16 .. +3 (the two 16-bit halves; blocks past K read 0)
        const uint32_t b = rbase + (uint32_t)(k0 / 16);
        rs0 = buf_load_b16(sr, b);
        rs1 = buf_load_b16(sr, k0 + 32 < K ? b + 2u : kBufferOOB);
      } else {
        const uint32_t b = rbase + (uint32_t)(k0 / 32);
        rs0 = buf_load_b8(sr, b);
        rs1 = buf_load_b8(sr, k0 + 32 < K ? b + 1u : kBufferOOB);
      }
    }
  };

  auto store_tile = [&](int st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + kThreads * i;
      *reinterpret_cast<u32x4_t*>(&As[st][(id >> 3) * A_LD + (id & 7) * 8]) = ra[i];
    }
    {
      const int row = tid >> 1, half = tid & 1;
      // two 8-byte stores: the LDS row pitch (40 B) is only 8-byte aligned
      u32x2_t* dst = reinterpret_cast<u32x2_t*>(&Bs[st][row * B_LD + half * 16]);
      dst[0] = u32x2_t{rb[0], rb[1]};
      dst[1] = u32x2_t{rb[2], rb[3]};
    }
    if (tid < BN) {
      if constexpr (FMT == kInt4)
        Ss[st][tid] = rs0 | (rs1 << 16);   // bf16 scale | zero << 16
      else if constexpr (FMT == kNvfp4)
        Ss[st][tid] = rs0 | (rs1 << 16);   // e4m3 bytes of blocks 0..3
      else
        Ss[st][tid] = rs0 | (rs1 << 8);    // e8m0 bytes of blocks 0..1
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

    // B fragments: 16 codes (8 bytes) per lane per tile, both MFMA steps;
    // the lane's codes 16g .. 16g+15 of the k-tile lie in one scale block
    u32x2_t bq[TN];
    float bs[TN], bz[TN];
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const int row = wn * 64 + t * 16 + l16;
      bq[t] = *reinterpret_cast<const u32x2_t*>(&Bs[cur][row * B_LD + 8 * g]);
      const uint32_t sw = Ss[cur][row];
      if constexpr (FMT == kInt4) {
        bs[t] = bf16_bits_to_f32(sw & 0xFFFFu);
        bz[t] = (float)(sw >> 16);
      } else if constexpr (FMT == kNvfp4) {
        bs[t] = e4m3_magnitude((sw >> (8 * g)) & 0xFFu);
      } else {
        bs[t] = e8m0_as_exponent_scale((sw >> (8 * (g >> 1))) & 0xFFu);
      }
    }
    // a ragged last k-tile (K % 64 == 32) is zero-filled: A = 0 and code 0
    // with a finite scale past K, so both steps run unconditionally
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4_t bf[TN];
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        if constexpr (FMT == kInt4) {
          bf[t] = int4x8_to_bf16_weights(bq[t][s], bs[t], bz[t]);
        } else if constexpr (FMT == kNvfp4) {
          bf[t] = fp4x8_to_bf16_fscale(bq[t][s], bs[t]);
        } else {
          bf[t] = fp4x8_to_bf16_escale(bq[t][s], bs[t]);
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
  const int64_t tiles = ((a.N + BN - 1) / BN) * ((a.M + BM - 1) / BM);
  dim3 grid((unsigned)tiles);
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
