// tiled.hip -- W4A16 GEMM for many activation rows: C = A . dequant(B)^T with
// A and the PACKED weights copied straight from global memory into LDS and
// the weights decoded into bf16 MFMA B fragments in registers, fp32
// accumulation.
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
// 128 x 64 = 8 x 4 MFMA 16x16x32 tiles, each computed transposed (weights as
// the MFMA's first operand) so that a lane ends up with 4 consecutive output
// columns of one row.  A and B k-tiles sit in two LDS stages filled by
// asynchronous global -> LDS copies (no staging registers, no LDS stores by
// the waves): while the waves multiply stage j, the copies of k-tile j+1 are
// in flight.  Scales arrive the same
// way, once per scale tile of several k-tiles, in two alternating buffers.
// Inside a k-tile, lane group g (lanes 16g .. 16g+15) owns codes 16g ..
// 16g+15 of each row: one 8-byte LDS read per B fragment covers both 32-k
// MFMA steps, and the A fragment of step s is the 8 A values at k = 16g + 8s
// .. +7 (the same k order for A and B).
//
// LDS layouts.  A copy writes 64 consecutive LDS slots, so each layout is a
// lane -> source permutation of whole copies; it keeps the lanes of a copy
// on few, contiguous global runs (global requests) and makes the MFMA-side
// reads free of bank conflicts:
//   A: row r of the tile is 128 B = 8 chunks of 8 k; chunk c sits in slot
//      c ^ f(r), f(r) = (r & 7) ^ ((r >> 3) & 1), so the 16 rows read by one
//      lane group at one chunk hit 16 distinct 16-B slots of each 256 B.
//   B: row r is 32 B = two 16-B halves (codes 32h .. 32h+31); half h sits in
//      slot h ^ ((r >> 2) & 1) (two lanes fetch one row's 32 contiguous bytes).
//   scales: per row, E consecutive scale elements (one dword slot each) of a
//      scale tile; element e sits in slot e ^ f_E(r) (see ScaleTile).
#include "common.hpp"
#include "kernels.hpp"

namespace w4a16 {

namespace {

constexpr int BK = 64;
constexpr int kStages = 2;

// Scale tile: each of the BN rows brings E consecutive elements of its scale
// row (E consecutive lanes, one global run per row), covering kKTiles k-tiles.
//   MXFP4: 1-byte e8m0 per 32 codes, E = 16 -> 8 k-tiles.
//   NVFP4: 2-byte element = the e4m3 bytes of two 16-code blocks, E = 8 -> 4 k-tiles.
//   int4:  2-byte bf16 scale (array 0) and 1-byte zero (array 1) per group:
//          groups of 128, E = 8 -> 16 k-tiles; of 64, E = 8 -> 8 k-tiles; of
//          32, E = 16 -> 8 k-tiles.
// Elements past K, and rows past N, are zero-filled by the copy.
template <int FMT>
struct ScaleTile;
template <>
struct ScaleTile<kMxfp4> {
  static constexpr int kElems = 16, kKTiles = 8, kArrays = 1;
};
template <>
struct ScaleTile<kNvfp4> {
  static constexpr int kElems = 8, kKTiles = 4, kArrays = 1;
};
template <>
struct ScaleTile<kInt4> {
  static constexpr int kElems = 8, kKTiles = 16, kArrays = 2;
};
template <>
struct ScaleTile<kInt4Sym> {  // scales only (the zero point is 8)
  static constexpr int kElems = 8, kKTiles = 16, kArrays = 1;
};
template <>
struct ScaleTile<kInt4G64> {
  static constexpr int kElems = 8, kKTiles = 8, kArrays = 2;
};
template <>
struct ScaleTile<kInt4G32> {
  static constexpr int kElems = 16, kKTiles = 8, kArrays = 2;
};
// slot swizzle of row r: 16 rows reading one element hit 16 distinct banks
template <int E>
__device__ __forceinline__ int scale_swz(int r) {
  return E == 16 ? (r >> 1) & 7 : (r >> 2) & 3;
}

// Workgroup tile BM x BN = (WGM * TM * 16) x (WGN * TN * 16): WGM x WGN waves,
// each computing TM x TN MFMA 16x16x32 tiles.
template <int WGM_, int WGN_, int TM_, int TN_>
struct TileCfg {
  static constexpr int WGM = WGM_, WGN = WGN_, TM = TM_, TN = TN_;
  static constexpr int BM = WGM * TM * 16, BN = WGN * TN * 16;
  static constexpr int kWaves = WGM * WGN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kABytes = BM * BK * 2;  // one stage of A (bf16)
  static constexpr int kBBytes = BN * BK / 2;  // one stage of packed B
  // 1-KB copy blocks per wave and k-tile (64 lanes x 16 B)
  static constexpr int kABlocks = kABytes / 1024 / kWaves;
  static constexpr int kBBlocks = kBBytes / 1024 / kWaves;
  static constexpr int kGroupOps = kABlocks + kBBlocks;  // copies per wave per k-tile
  static_assert(kABlocks * kWaves * 1024 == kABytes, "A stage must split into 1-KB blocks");
  static_assert(kBBlocks * kWaves * 1024 == kBBytes, "B stage must split into 1-KB blocks");
  static_assert(kGroupOps <= 15, "vmcnt immediate");
};

template <int FMT, class CFG>
struct Layout {
  using ST = ScaleTile<FMT>;
  static constexpr int kSArrayBytes = CFG::BN * ST::kElems * 4;
  static constexpr int kSBytes = ST::kArrays * kSArrayBytes;        // one scale buffer
  static constexpr int kSBlocks = kSBytes / 256 / CFG::kWaves;      // 64-dword copies per wave
  static constexpr int kBOff = kStages * CFG::kABytes;
  static constexpr int kSOff = kBOff + kStages * CFG::kBBytes;
  static constexpr int kBytes = kSOff + 2 * kSBytes;
  static_assert(kSBlocks * CFG::kWaves * 256 == kSBytes, "scale buffer must split into copies");
  static_assert((CFG::BN * ST::kElems) % 64 == 0, "a copy covers whole rows of one array");
  static_assert(kBytes <= 160 * 1024, "LDS");
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

// wait until at most N of this wave's copies are outstanding, then barrier
template <int N>
__device__ __forceinline__ void wait_copies_and_barrier() {
  static_assert(N >= 0 && N <= 15, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int FMT, bool OUT_F32, class CFG>
__global__ __launch_bounds__(CFG::kThreads) void tiled_kernel(const uint16_t* __restrict__ A,
                                                              const uint8_t* __restrict__ packed,
                                                              const void* __restrict__ scales,
                                                              const uint8_t* __restrict__ zeros,
                                                              void* __restrict__ C, int M, int N,
                                                              int K, int pre, Epilogue epi) {
  constexpr int BM = CFG::BM, BN = CFG::BN, TM = CFG::TM, TN = CFG::TN;
  constexpr int kABytes = CFG::kABytes, kBBytes = CFG::kBBytes;
  using L = Layout<FMT, CFG>;
  using ST = ScaleTile<FMT>;
  constexpr int E = ST::kElems;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[L::kBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int groups = (K + G - 1) / G;  // the last group may be shorter

  // Buffer descriptors over this workgroup's rows: rows past M / N read as 0.
  const uint32_t arow_b = (uint32_t)K * 2u, brow_b = (uint32_t)K >> 1;
  const int brows = min(BN, N - n_base);
  // (prepacked: whole 16-row tiles, zero bytes past N)
  const int brows_read = pre ? min(BN, ((N + 15) & ~15) - n_base) : brows;
  const rsrc_t ar = make_rsrc(A + (int64_t)m_base * K, (uint32_t)min(BM, M - m_base) * arow_b);
  const rsrc_t br = make_rsrc(packed + (int64_t)n_base * brow_b, (uint32_t)brows_read * brow_b);
  constexpr int SB = is_int4(FMT) ? 2 : 1;
  const rsrc_t sr = make_rsrc(reinterpret_cast<const uint8_t*>(scales) + (int64_t)n_base * groups * SB,
                              (uint32_t)(brows * groups * SB));
  const rsrc_t zr = make_rsrc(has_zeros(FMT) ? zeros + (int64_t)n_base * groups : nullptr,
                              has_zeros(FMT) ? (uint32_t)(brows * groups) : 0u);
  const uint32_t lds0 = lds_address(smem);
  // Resolve the output pointer's scalar load here: a scalar load still in
  // flight in the k-loop would turn every partial LDS wait there into a full one.
  asm volatile("" ::"s"(C));

  // ---- per-lane source offsets of this wave's A / B copy blocks (k0 = 0) ----
  // A block b = rows 8b .. 8b+7: lane -> row 8b + lane/8, LDS slot lane%8,
  // which holds logical chunk c = slot ^ f(row).
  uint32_t a_src[CFG::kABlocks];
  int a_k[CFG::kABlocks];
#pragma unroll
  for (int i = 0; i < CFG::kABlocks; ++i) {
    const int b = wave * CFG::kABlocks + i;
    const int row = 8 * b + (lane >> 3);
    const int c = (lane & 7) ^ (lane >> 3) ^ (b & 1);
    a_src[i] = (uint32_t)row * arow_b + (uint32_t)c * 16u;
    a_k[i] = 8 * c;
  }
  // B block: slot q = 64 bb + lane -> row q / 2, which holds half h = (q & 1) ^ ((row >> 2) & 1)
  // (k-tile j: chunk 2j + h of the row, at wchunk(row, 2j + h) = wchunk(row, h) + j * b_step)
  uint32_t b_src[CFG::kBBlocks];
  int b_k[CFG::kBBlocks];
#pragma unroll
  for (int i = 0; i < CFG::kBBlocks; ++i) {
    const int q = 64 * (wave * CFG::kBBlocks + i) + lane;
    const int row = q >> 1, h = (q & 1) ^ ((row >> 2) & 1);
    b_src[i] = wchunk((uint32_t)row, (uint32_t)h, brow_b, pre != 0);
    b_k[i] = 32 * h;
  }
  const uint32_t b_step = pre ? 512u : 32u;

  // issue the copies of k-tile kt into stage st (CFG::kGroupOps per wave)
  auto issue = [&](int kt, int st) {
    const int k0 = kt * BK;
    const uint32_t a_lds = lds0 + st * kABytes + wave * CFG::kABlocks * 1024;
#pragma unroll
    for (int i = 0; i < CFG::kABlocks; ++i)
      lds_dma_b128(ar, a_lds + i * 1024,
                   k0 + a_k[i] < K ? a_src[i] + (uint32_t)k0 * 2u : kBufferOOB);
    const uint32_t b_lds = lds0 + L::kBOff + st * kBBytes + wave * CFG::kBBlocks * 1024;
#pragma unroll
    for (int i = 0; i < CFG::kBBlocks; ++i)
      lds_dma_b128(br, b_lds + i * 1024, k0 + b_k[i] < K ? b_src[i] + (uint32_t)kt * b_step : kBufferOOB);
  };

  // issue the copies of scale tile u into buffer u & 1 (L::kSBlocks per wave):
  // copy block sb covers rows (sb % bpa) * 64/E .. + 64/E - 1 of array sb / bpa
  auto issue_scales = [&](int u) {
    constexpr int bpa = L::kSArrayBytes / 256;  // copy blocks per array
    const int m = lane / E, i = lane % E;
    const uint32_t s_lds = lds0 + L::kSOff + (u & 1) * L::kSBytes;
#pragma unroll
    for (int c = 0; c < L::kSBlocks; ++c) {
      const int sb = wave * L::kSBlocks + c;
      const int arr = sb / bpa;  // wave-uniform
      const int row = (sb % bpa) * (64 / E) + m;
      const int e = u * E + (i ^ scale_swz<E>(row));  // element index in the scale row
      const uint32_t dst = s_lds + sb * 256;
      if constexpr (FMT == kMxfp4) {
        lds_dma_b8(sr, dst, e < groups ? (uint32_t)(row * groups + e) : kBufferOOB);
      } else if constexpr (FMT == kNvfp4) {
        lds_dma_b16(sr, dst, 2 * e < groups ? (uint32_t)(row * groups + 2 * e) : kBufferOOB);
      } else {
        if (!has_zeros(FMT) || arr == 0)
          lds_dma_b16(sr, dst, e < groups ? (uint32_t)(row * groups + e) * 2u : kBufferOOB);
        else
          lds_dma_b8(zr, dst, e < groups ? (uint32_t)(row * groups + e) : kBufferOOB);
      }
    }
  };

  // ---- per-lane LDS read offsets -------------------------------------------
  const int fa = (l16 & 7) ^ ((l16 >> 3) & 1);
  const uint32_t a_rd0 = (uint32_t)(l16 * 128 + (((2 * g) ^ fa) * 16));
  const uint32_t a_rd1 = (uint32_t)(l16 * 128 + (((2 * g + 1) ^ fa) * 16));
  const uint32_t b_rd = (uint32_t)((l16 * 2 + ((g >> 1) ^ ((l16 >> 2) & 1))) * 16 + 8 * (g & 1));
  const int fs = scale_swz<E>(l16);  // rows of a lane differ by multiples of 16

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int t = 0; t < TN; ++t) acc[i][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // int4 whose group covers the k-tile (groups of 128 or 64): the MFMAs sum
  // the exact code - zero over the k-tile and the group scale of each output
  // row multiplies that partial sum in fp32 (exact weights, no bf16 rounding)
  constexpr bool kFold = is_int4(FMT) && FMT != kInt4G32;

  issue_scales(0);
  issue(0, 0);

  int cur = 0, nxt = 1;  // stage of k-tile j, stage of k-tile j + 1
  for (int j = 0; j < KT; ++j) {
    // this wave's copies of k-tile j (and of its scale tile) done, and every
    // wave's: then all waves are past k-tile j - 1, so its stage (= stage of
    // j + 1) and the scale buffer last read before it may be refilled
    wait_copies_and_barrier<0>();
    if (j + 1 < KT) {
      if ((j + 1) % ST::kKTiles == 0) issue_scales((j + 1) / ST::kKTiles);
      issue(j + 1, nxt);
    }

    const uint8_t* As = smem + cur * kABytes + (wm * TM * 16) * 128;
    const uint8_t* Bs = smem + L::kBOff + cur * kBBytes + (wn * TN * 16) * 32;
    // scale element of lane group g in this k-tile, and its slot
    const int jt = j % ST::kKTiles;
    // (lane group g holds codes 16g .. 16g+15 of the k-tile's 64)
    const int se = is_int4_g128(FMT) ? (jt >> 1) : FMT == kInt4G64 ? jt : 2 * jt + (g >> 1);
    const uint8_t* Ss = smem + L::kSOff + ((j / ST::kKTiles) & 1) * L::kSBytes +
                        ((wn * TN * 16 + l16) * E + (se ^ fs)) * 4;

    // LDS reads first: this k-tile's B fragments (16 codes = 8 bytes per lane
    // per tile, both MFMA steps; codes 16g .. 16g+15 lie in one scale
    // block), their scales and the A fragments of step 0; the decode then
    // overlaps the A reads, and the step-1 A reads overlap the step-0 MFMAs.
    // (A ragged last k-tile, K % 64 == 32, is zero-filled: A = 0 and code 0
    // with a zero scale past K, so both steps run.)
    u32x2_t bq[TN];
    uint32_t sw[TN], zw[TN];
    u32x4_t af0[TM], af1[TM];
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      bq[t] = *reinterpret_cast<const u32x2_t*>(Bs + b_rd + t * 16 * 32);
      sw[t] = *reinterpret_cast<const uint32_t*>(Ss + t * 16 * E * 4);
      if constexpr (has_zeros(FMT))
        zw[t] = *reinterpret_cast<const uint32_t*>(Ss + t * 16 * E * 4 + L::kSArrayBytes);
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
      af0[i] = *reinterpret_cast<const u32x4_t*>(As + i * 16 * 128 + a_rd0);
    __builtin_amdgcn_sched_barrier(0);
    float bs[TN], bz[TN];
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      if constexpr (is_int4(FMT)) {
        bs[t] = bf16_bits_to_f32(sw[t]);
        bz[t] = has_zeros(FMT) ? (float)zw[t] : (float)kSymZero;
      } else if constexpr (FMT == kNvfp4) {
        bs[t] = e4m3_magnitude((sw[t] >> (8 * (g & 1))) & 0xFFu);
      } else {
        bs[t] = e8m0_as_exponent_scale(sw[t]);
      }
    }
    // kFold: the group scales of the lane's output rows 4g .. 4g+3 of tile t
    // (the MFMA result rows; the lane supplies weight row l16)
    auto row_scales = [&](int t) {
      const uint8_t* Sb = smem + L::kSOff + ((j / ST::kKTiles) & 1) * L::kSBytes;
      f32x4_t so;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wn * TN * 16 + t * 16 + 4 * g + r;
        so[r] = bf16_bits_to_f32(
            *reinterpret_cast<const uint32_t*>(Sb + (row * E + (se ^ scale_swz<E>(row))) * 4));
      }
      return so;
    };
    auto decode = [&](int s, int t) -> u32x4_t {
      if constexpr (FMT == kNvfp4) {
        return fp4x8_to_bf16_fscale(bq[t][s], bs[t]);
      } else {
        return fp4x8_to_bf16_escale(bq[t][s], bs[t]);
      }
    };
    // the step-1 A reads are issued before the step-0 MFMAs
#pragma unroll
    for (int i = 0; i < TM; ++i)
      af1[i] = *reinterpret_cast<const u32x4_t*>(As + i * 16 * 128 + a_rd1);
    if constexpr (kFold) {
      // per (i, t): two MFMAs over the k-tile's exact code - zero from zero,
      // then the row scales fold the partial sum into the accumulator
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const f32x4_t so = row_scales(t);
        const u32x4_t b0 = int4x8_minus_zero(bq[t][0], bz[t]);
        const u32x4_t b1 = int4x8_minus_zero(bq[t][1], bz[t]);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          f32x4_t p = mfma16x16x32(b0, af0[i], f32x4_t{0.f, 0.f, 0.f, 0.f});
          p = mfma16x16x32(b1, af1[i], p);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][t][r] = __builtin_fmaf(so[r], p[r], acc[i][t][r]);
        }
      }
    } else if constexpr (is_int4(FMT)) {
      // groups of 32 (two per k-tile): the exact weights as hi + lo fragments
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int t = 0; t < TN; ++t) {
          u32x4_t hi, lo;
          int4x8_to_bf16_hilo(bq[t][st], bs[t], bz[t], hi, lo);
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            acc[i][t] = mfma16x16x32(hi, st ? af1[i] : af0[i], acc[i][t]);
            acc[i][t] = mfma16x16x32(lo, st ? af1[i] : af0[i], acc[i][t]);
          }
        }
    } else {
      // step 0: B column tile t is decoded right before its MFMAs (one
      // decoded fragment live at a time)
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const u32x4_t bf = decode(0, t);
#pragma unroll
        for (int i = 0; i < TM; ++i) acc[i][t] = mfma16x16x32(bf, af0[i], acc[i][t]);
      }
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const u32x4_t bf = decode(1, t);
#pragma unroll
        for (int i = 0; i < TM; ++i) acc[i][t] = mfma16x16x32(bf, af1[i], acc[i][t]);
      }
    }
    cur = cur == kStages - 1 ? 0 : cur + 1;
    nxt = nxt == kStages - 1 ? 0 : nxt + 1;
  }

// ---- epilogue: lane holds output row l16 of each 16x16 tile, columns
// 4g .. 4g+3 (one 8- or 16-byte store when the rows allow aligned vectors)
  const bool vec = (N % 4 == 0) && ((reinterpret_cast<uintptr_t>(C) & (OUT_F32 ? 15 : 7)) == 0);
  // Fused epilogue, in batches of kRB row blocks: the batch's residual is
  // loaded first (it may alias C, so the compiler could not hoist its loads
  // over the stores itself), alpha * c + bias and the activation run while
  // it is in flight, then the residual is added and the batch stored.  Loads
  // are unconditional at clamped indices (values past M / N come from a valid
  // element and are never stored), and each choice between code paths is
  // made once per batch, not per element, so the loads issue as one group.
  constexpr int kRW = OUT_F32 ? 4 : 2;                // residual words per (row block, column group)
  constexpr int kRB = OUT_F32 ? TM / 4 : TM / 2;      // 32 registers of residual per batch
  f32x4_t eb[TN];
  if (epi.on && epi.bias) {
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const int n0 = n_base + wn * (TN * 16) + t * 16 + 4 * g;
#pragma unroll
      for (int r = 0; r < 4; ++r) eb[t][r] = bf16_bits_to_f32(epi.bias[min(n0 + r, N - 1)]);
    }
  } else {
#pragma unroll
    for (int t = 0; t < TN; ++t) eb[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const bool res_vec = vec && epi.res &&
                       (reinterpret_cast<uintptr_t>(epi.res) & (OUT_F32 ? 15 : 7)) == 0;
#pragma unroll
  for (int i0 = 0; i0 < TM; i0 += kRB) {
    uint32_t rw[kRB][TN][kRW];
    if (epi.on && epi.res && res_vec) {
      // N % 4 == 0: the four columns of a group are all in range or all out
#pragma unroll
      for (int j = 0; j < kRB; ++j) {
        const int m = min(m_base + wm * (TM * 16) + (i0 + j) * 16 + l16, M - 1);
#pragma unroll
        for (int t = 0; t < TN; ++t) {
          const int n0 = n_base + wn * (TN * 16) + t * 16 + 4 * g;
          const int64_t mn = (int64_t)m * N + min(n0, N - 4);
          if constexpr (OUT_F32) {
            const u32x4_t q = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const float*>(epi.res) + mn);
#pragma unroll
            for (int w = 0; w < kRW; ++w) rw[j][t][w] = q[w];
          } else {
            const u32x2_t q = *reinterpret_cast<const u32x2_t*>(reinterpret_cast<const uint16_t*>(epi.res) + mn);
            rw[j][t][0] = q[0];
            rw[j][t][1] = q[1];
          }
        }
      }
    } else if (epi.on && epi.res) {
#pragma unroll
      for (int j = 0; j < kRB; ++j) {
        const int m = min(m_base + wm * (TM * 16) + (i0 + j) * 16 + l16, M - 1);
#pragma unroll
        for (int t = 0; t < TN; ++t) {
          const int n0 = n_base + wn * (TN * 16) + t * 16 + 4 * g;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int64_t mn = (int64_t)m * N + min(n0 + r, N - 1);
            if constexpr (OUT_F32) {
              rw[j][t][r] = reinterpret_cast<const uint32_t*>(epi.res)[mn];
            } else {
              const uint32_t h = reinterpret_cast<const uint16_t*>(epi.res)[mn];
              if (r & 1)
                rw[j][t][r >> 1] |= h << 16;
              else
                rw[j][t][r >> 1] = h;
            }
          }
        }
      }
    }
    if (epi.on) {
#pragma unroll
      for (int j = 0; j < kRB; ++j)
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i0 + j][t][r] = __builtin_fmaf(epi.alpha, acc[i0 + j][t][r], eb[t][r]);
      if (epi.act == 1) {
#pragma unroll
        for (int j = 0; j < kRB; ++j)
#pragma unroll
          for (int t = 0; t < TN; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i0 + j][t][r] = act_relu(acc[i0 + j][t][r]);
      } else if (epi.act == 2) {
#pragma unroll
        for (int j = 0; j < kRB; ++j)
#pragma unroll
          for (int t = 0; t < TN; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i0 + j][t][r] = act_silu(acc[i0 + j][t][r]);
      } else if (epi.act == 3) {
#pragma unroll
        for (int j = 0; j < kRB; ++j)
#pragma unroll
          for (int t = 0; t < TN; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i0 + j][t][r] = act_gelu_tanh(acc[i0 + j][t][r]);
      }
      if (epi.res) {
#pragma unroll
        for (int j = 0; j < kRB; ++j)
#pragma unroll
          for (int t = 0; t < TN; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float res = OUT_F32 ? __uint_as_float(rw[j][t][r])
                                        : bf16_bits_to_f32((rw[j][t][r >> 1] >> (16 * (r & 1))) & 0xFFFFu);
              acc[i0 + j][t][r] = __builtin_fmaf(epi.beta, res, acc[i0 + j][t][r]);
            }
      }
    }
#pragma unroll
    for (int j = 0; j < kRB; ++j) {
      const int i = i0 + j;
      const int m = m_base + wm * (TM * 16) + i * 16 + l16;
      if (m >= M) continue;
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const int n0 = n_base + wn * (TN * 16) + t * 16 + 4 * g;
        const f32x4_t v = acc[i][t];
        if (vec && n0 < N) {
          if constexpr (OUT_F32) {
            *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(C) + (int64_t)m * N + n0) = v;
          } else {
            *reinterpret_cast<u32x2_t*>(reinterpret_cast<__bf16*>(C) + (int64_t)m * N + n0) =
                u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (n0 + r < N) {
              if constexpr (OUT_F32)
                reinterpret_cast<float*>(C)[(int64_t)m * N + n0 + r] = v[r];
              else
                reinterpret_cast<__bf16*>(C)[(int64_t)m * N + n0 + r] = (__bf16)v[r];
            }
          }
        }
      }
    }
  }
}

// The tile configurations.  256 x 256, waves 2 (M) x 4 (N), wave tile 128 x 64
// (64 x 128 wave tiles halve the A-fragment reads but double the decode, and
// 128 x 128 wave tiles leave one wave per SIMD: both measured slower).  With
// fewer than 192 such tiles most CUs would idle: then 128 x 128 tiles of 4
// waves (64 x 64 wave tiles), whose time is set by the latency of each
// wave's k-loop rather than by the MFMA work (deeper copy pipelines measured
// slower; 128 x 64 and 64 x 128 tiles no faster).
using Cfg = TileCfg<2, 4, 8, 4>;
using CfgSmall = TileCfg<2, 2, 4, 4>;

template <int FMT, bool OUT_F32, class CFG>
hipError_t launch_cfg(const GemmArgs& a) {
  const int64_t tiles = ((a.N + CFG::BN - 1) / CFG::BN) * ((a.M + CFG::BM - 1) / CFG::BM);
  if (tiles > 0xFFFFFFFFll) return hipErrorInvalidConfiguration;  // (the grid counts tiles in 32 bits)
  return launch_kernel(tiled_kernel<FMT, OUT_F32, CFG>, dim3((unsigned)tiles), dim3(CFG::kThreads), 0,
                       a.stream, a.A, a.packed, a.scales, a.zeros, a.C, (int)a.M, (int)a.N, (int)a.K,
                       a.pre ? 1 : 0, a.epi);
}

template <int FMT, bool OUT_F32>
hipError_t launch_fmt(const GemmArgs& a) {
  const int64_t big_tiles = ((a.N + Cfg::BN - 1) / Cfg::BN) * ((a.M + Cfg::BM - 1) / Cfg::BM);
  if (big_tiles < 192) return launch_cfg<FMT, OUT_F32, CfgSmall>(a);
  return launch_cfg<FMT, OUT_F32, Cfg>(a);
}

}  // namespace

hipError_t launch_tiled(const GemmArgs& a) {
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
