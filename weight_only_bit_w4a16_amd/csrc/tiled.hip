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
#include <stdlib.h>

#include "common.hpp"
#include "kernels.hpp"

namespace w4a16 {

namespace {

constexpr int BK = 64;
constexpr int A_LD = BK + 8;        // bf16 elements per LDS row of A (144 B: 16-B slots rotate)
constexpr int B_LD = BK / 2 + 8;    // bytes per LDS row of packed B (40 B)

// Workgroup tile BM x BN = (WGM * TM * 16) x (WGN * TN * 16): WGM x WGN waves,
// each computing TM x TN MFMA 16x16x32 tiles.
template <int WGM_, int WGN_, int TM_, int TN_>
struct TileCfg {
  static constexpr int WGM = WGM_, WGN = WGN_, TM = TM_, TN = TN_;
  static constexpr int BM = WGM * TM * 16, BN = WGN * TN * 16;
  static constexpr int kThreads = 64 * WGM * WGN;
  static constexpr int kAChunks = BM * (BK / 8) / kThreads;   // 16-byte A chunks per thread
  static constexpr int kBChunks = BN * (BK / 32) / kThreads;  // 16-byte B chunks per thread
  static_assert(kAChunks * kThreads == BM * (BK / 8), "A tile must split evenly");
  static_assert(kBChunks * kThreads == BN * (BK / 32), "B tile must split evenly");
  static_assert(BN <= kThreads, "one thread per B row fetches its scales");
};

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

template <int FMT, bool OUT_F32, class CFG>
__global__ __launch_bounds__(CFG::kThreads) void tiled_kernel(const uint16_t* __restrict__ A,
                                                              const uint8_t* __restrict__ packed,
                                                              const void* __restrict__ scales,
                                                              const uint8_t* __restrict__ zeros,
                                                              void* __restrict__ C, int M, int N,
                                                              int K) {
  constexpr int BM = CFG::BM, BN = CFG::BN, TM = CFG::TM, TN = CFG::TN;
  constexpr int kThreads = CFG::kThreads;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * A_LD];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BN * B_LD];
  __shared__ uint32_t Ss[2][BN];  // raw scale (and zero) bytes of each B row for the k-tile

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / CFG::WGN;
  const int wn = wave % CFG::WGN;
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
  // A: BM rows x 8 chunks of 16 B; B: BN rows x 2 chunks of 16 B; chunk ids
  // tid + kThreads * i.  Thread t < BN fetches row t's raw scale bytes.
  u32x4_t ra[CFG::kAChunks];
  u32x4_t rb[CFG::kBChunks];
  uint32_t rs0 = 0, rs1 = 0;

  auto load_tile = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < CFG::kAChunks; ++i) {
      const int id = tid + kThreads * i;
      const int row = id >> 3, k = k0 + (id & 7) * 8;
      ra[i] = buf_load_b128(ar, k < K ? (uint32_t)row * arow_b + (uint32_t)k * 2u : kBufferOOB);
    }
#pragma unroll
    for (int i = 0; i < CFG::kBChunks; ++i) {
      const int id = tid + kThreads * i;
      const int row = id >> 1, k = k0 + (id & 1) * 32;
      rb[i] = buf_load_b128(br, k < K ? (uint32_t)row * brow_b + (uint32_t)(k >> 1) : kBufferOOB);
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
    for (int i = 0; i < CFG::kAChunks; ++i) {
      const int id = tid + kThreads * i;
      *reinterpret_cast<u32x4_t*>(&As[st][(id >> 3) * A_LD + (id & 7) * 8]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < CFG::kBChunks; ++i) {
      const int id = tid + kThreads * i;
      // two 8-byte stores: the LDS row pitch (40 B) is only 8-byte aligned
      u32x2_t* dst = reinterpret_cast<u32x2_t*>(&Bs[st][(id >> 1) * B_LD + (id & 1) * 16]);
      dst[0] = u32x2_t{rb[i][0], rb[i][1]};
      dst[1] = u32x2_t{rb[i][2], rb[i][3]};
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

    // LDS reads first: this k-tile's B fragments (16 codes = 8 bytes per lane
    // per tile, both MFMA steps; codes 16g .. 16g+15 lie in one scale
    // block), their scale words and the A fragments of step 0; the decode
    // then overlaps the A reads, and the step-1 A reads overlap the step-0
    // MFMAs.  (A ragged last k-tile, K % 64 == 32, is zero-filled: A = 0 and
    // code 0 with a finite scale past K, so both steps run.)
    u32x2_t bq[TN];
    uint32_t sw[TN];
    u32x4_t af0[TM], af1[TM];
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const int row = wn * (TN * 16) + t * 16 + l16;
      bq[t] = *reinterpret_cast<const u32x2_t*>(&Bs[cur][row * B_LD + 8 * g]);
      sw[t] = Ss[cur][row];
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = wm * (TM * 16) + i * 16 + l16;
      af0[i] = *reinterpret_cast<const u32x4_t*>(&As[cur][row * A_LD + 16 * g]);
    }
    __builtin_amdgcn_sched_barrier(0);
    float bs[TN], bz[TN];
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      if constexpr (FMT == kInt4) {
        bs[t] = bf16_bits_to_f32(sw[t] & 0xFFFFu);
        bz[t] = (float)(sw[t] >> 16);
      } else if constexpr (FMT == kNvfp4) {
        bs[t] = e4m3_magnitude((sw[t] >> (8 * g)) & 0xFFu);
      } else {
        bs[t] = e8m0_as_exponent_scale((sw[t] >> (8 * (g >> 1))) & 0xFFu);
      }
    }
    auto decode = [&](int s, int t) -> u32x4_t {
      if constexpr (FMT == kInt4) {
        return int4x8_to_bf16_weights(bq[t][s], bs[t], bz[t]);
      } else if constexpr (FMT == kNvfp4) {
        return fp4x8_to_bf16_fscale(bq[t][s], bs[t]);
      } else {
        return fp4x8_to_bf16_escale(bq[t][s], bs[t]);
      }
    };
    // step 0: B column tile t is decoded right before its MFMAs (one decoded
    // fragment live at a time); the step-1 A reads are issued first
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = wm * (TM * 16) + i * 16 + l16;
      af1[i] = *reinterpret_cast<const u32x4_t*>(&As[cur][row * A_LD + 16 * g + 8]);
    }
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const u32x4_t bf = decode(0, t);
#pragma unroll
      for (int i = 0; i < TM; ++i) acc[i][t] = mfma16x16x32(af0[i], bf, acc[i][t]);
    }
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const u32x4_t bf = decode(1, t);
#pragma unroll
      for (int i = 0; i < TM; ++i) acc[i][t] = mfma16x16x32(af1[i], bf, acc[i][t]);
    }

    if (has_next) store_tile(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds rows 4g..4g+3 of each 16x16 tile, column l16 ----
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const int n = n_base + wn * (TN * 16) + t * 16 + l16;
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m_base + wm * (TM * 16) + i * 16 + 4 * g + r;
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

// the tile configuration in use: 256 x 256, waves 2 (M) x 4 (N), wave tile
// 128 x 64 (W4A16_TILED_CFG=1 selects waves 4 x 2 with 64 x 128 wave tiles,
// for tuning: it halves the A-fragment LDS reads but doubles the decode)
using CfgA = TileCfg<2, 4, 8, 4>;
using CfgB = TileCfg<4, 2, 4, 8>;

template <int FMT, bool OUT_F32, class CFG>
hipError_t launch_cfg(const GemmArgs& a) {
  const int64_t tiles = ((a.N + CFG::BN - 1) / CFG::BN) * ((a.M + CFG::BM - 1) / CFG::BM);
  hipLaunchKernelGGL((tiled_kernel<FMT, OUT_F32, CFG>), dim3((unsigned)tiles), dim3(CFG::kThreads),
                     0, a.stream, a.A, a.packed, a.scales, a.zeros, a.C, (int)a.M, (int)a.N,
                     (int)a.K);
  return hipGetLastError();
}

template <int FMT, bool OUT_F32>
hipError_t launch_fmt(const GemmArgs& a) {
  static const int cfg_env = [] {
    const char* e = getenv("W4A16_TILED_CFG");
    return e ? atoi(e) : 0;
  }();
  if (cfg_env == 1) return launch_cfg<FMT, OUT_F32, CfgB>(a);
  return launch_cfg<FMT, OUT_F32, CfgA>(a);
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
