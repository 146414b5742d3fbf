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
//   * int4: code - zero becomes an exact bf16 value (the code through the
//     scaled fp8 converter, the zero subtracted in fp32) -- in even / odd k
//     order when A sits in LDS (A is stored in that order), else in natural
//     k order; the group scale multiplies the sum once per k-block (k-block
//     = int4 group of 128);
//   * NVFP4: e2m1 -> fp32, times |e4m3 scale| (exact), -> bf16 (exact);
//   * MXFP4: hardware e2m1 conversion scaled by 2^(E-127) (exact).
#include <atomic>
#include <map>
#include <mutex>
#include <tuple>

#include "common.hpp"
#include "kernels.hpp"

namespace w4a16 {

namespace {

constexpr int kMaxWaves = 16;
int device_cus();
constexpr int kAStage = 2;  // 16-byte chunks of A per thread when A is staged in LDS
constexpr int kSStage = 3;  // scale dwords per thread when the scales are staged in LDS
constexpr int kZStage = 2;  // zero dwords per thread (int4)

// The GEMMs of one launch: a single one, or several of one K (member i: its
// A, packed / scales / zeros / C, N[i] columns).  Workgroup (x, y, z) runs
// columns x * rows .. of member z (none if past its N).  A single GEMM's
// launch carries one member (kernel arguments stay small), a grouped or
// batched one up to kMaxGroup.
struct SkinnyMember {
  const uint16_t* A;
  const uint8_t* packed;
  const void* scales;
  const uint8_t* zeros;
  void* C;
  int N;
};
template <int CAP>
struct SkinnyGroup {
  SkinnyMember m[CAP];  // one member's fields are contiguous
  int rows;  // weight rows (output columns) per workgroup, 1 .. 16 (16 when prepacked)
  int pre;   // the weights are in the prepacked layout
};
template <bool GROUPED>
using SkinnyGroupOf = SkinnyGroup<GROUPED ? kMaxGroup : 1>;

// One k-block of 128 codes into acc: a[j] is the lane's A fragment of MFMA
// step j (32 codes), q[j] its 8 codes of that step, sraw / zraw the raw scale
// (and zero) bytes of the lane's chunk.
//   int4 g128 (and symmetric): code - zero, exact in bf16, is formed for
//     each weight before the MFMA (a sum of a * code and a separate sum of
//     a * zero would lose small results to the rounding of the two large
//     sums), and the group scale multiplies the k-block's sum.  EVEN_ODD: A
//     sits in LDS in even / odd k order and the codes convert in that order;
//     otherwise in natural k order, like A.
//   int4 g32 / g64: groups shorter than a k-block; the lane's chunk has one
//     group, whose exact weights (code - zero) * scale are split into two
//     bf16 fragments hi + lo (both exact) that feed two MFMAs, so the
//     weights enter the sum unrounded.
//   NVFP4: chunk = two blocks of 16, one e4m3 scale each (low byte first).
//   MXFP4: chunk = one block of 32, one e8m0 scale.
template <int FMT, bool EVEN_ODD>
__device__ __forceinline__ f32x4_t kblock_mac(const u32x4_t (&a)[4], const u32x4_t& q, uint32_t sraw,
                                              uint32_t zraw, f32x4_t acc) {
  if constexpr (is_int4_g128(FMT)) {
    const float zf = (float)zraw;
    f32x4_t dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4_t b = EVEN_ODD ? int4x8_minus_zero_even_odd(q[j], zf) : int4x8_minus_zero(q[j], zf);
      dp = mfma16x16x32(a[j], b, dp);
    }
    const float s = bf16_bits_to_f32(sraw);
    acc[0] = __builtin_fmaf(s, dp[0], acc[0]);
    acc[1] = __builtin_fmaf(s, dp[1], acc[1]);
    acc[2] = __builtin_fmaf(s, dp[2], acc[2]);
    acc[3] = __builtin_fmaf(s, dp[3], acc[3]);
  } else if constexpr (is_int4(FMT)) {
    const float s = bf16_bits_to_f32(sraw);
    const float zf = (float)zraw;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4_t hi, lo;
      int4x8_to_bf16_hilo(q[j], s, zf, hi, lo);
      acc = mfma16x16x32(a[j], hi, acc);
      acc = mfma16x16x32(a[j], lo, acc);
    }
  } else if constexpr (FMT == kNvfp4) {
    const float s0 = e4m3_magnitude(sraw & 0xFFu);
    const float s1 = e4m3_magnitude(sraw >> 8);
    acc = mfma16x16x32(a[0], fp4x8_to_bf16_fscale(q[0], s0), acc);
    acc = mfma16x16x32(a[1], fp4x8_to_bf16_fscale(q[1], s0), acc);
    acc = mfma16x16x32(a[2], fp4x8_to_bf16_fscale(q[2], s1), acc);
    acc = mfma16x16x32(a[3], fp4x8_to_bf16_fscale(q[3], s1), acc);
  } else {
    const float es = e8m0_as_exponent_scale(sraw);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = mfma16x16x32(a[j], fp4x8_to_bf16_escale(q[j], es), acc);
  }
  return acc;
}

// kblock_mac for int4 with groups of 128 on fp16 operands: a[j] from an fp16
// A copy in the k order (0, 4, 1, 5, 2, 6, 3, 7) per 8, the codes to code -
// zero in fp16 in the same order (both exact: the same products as the bf16
// route, summed by the MFMA to the same bits), the group scale on the fp32
// sum.
__device__ __forceinline__ f32x4_t kblock_mac_f16(const u32x4_t (&a)[4], const u32x4_t& q, uint32_t sraw,
                                                  uint32_t zraw, f32x4_t acc, F16Consts fc) {
  const uint32_t zp = f16_zero_pair(zraw);
  f32x4_t dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) dp = mfma16x16x32_f16(a[j], int4x8_minus_zero_f16(q[j], fc, zp), dp);
  const float s = bf16_bits_to_f32(sraw);
  acc[0] = __builtin_fmaf(s, dp[0], acc[0]);
  acc[1] = __builtin_fmaf(s, dp[1], acc[1]);
  acc[2] = __builtin_fmaf(s, dp[2], acc[2]);
  acc[3] = __builtin_fmaf(s, dp[3], acc[3]);
  return acc;
}

// The split-K sum over the waves' partials red[w * 64 + lane] (w = 0 ..
// waves-1, in order) and the store of this workgroup's outputs, plain or
// through the fused epilogue; run by wave 0.  Lane (nl, g) holds rows
// m0 + 4g .. m0 + 4g + 3 of column n = n0 + nl; rows / arows bound the
// workgroup's columns / A rows.
template <bool OUT_F32>
__device__ __forceinline__ void skinny_store(const f32x4_t* red, int waves, int lane, int nl, int g,
                                             int rows, int arows, int m0, int n, int M, int N, void* C,
                                             const Epilogue& epi) {
  // the plain store and the fused epilogue are separate paths (one uniform
  // branch; the plain path carries no epilogue code)
  if (!epi.on) {
    f32x4_t sum = red[lane];
    for (int w = 1; w < waves; ++w) {
      const f32x4_t v = red[w * 64 + lane];
      sum[0] += v[0];
      sum[1] += v[1];
      sum[2] += v[2];
      sum[3] += v[3];
    }
    if (nl >= rows) return;
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
    return;
  }
  // epilogue operands first, all in one round trip (the residual may alias
  // C, so the compiler could not hoist them over the stores itself)
  float epi_b = 0.f, epi_r[4] = {0.f, 0.f, 0.f, 0.f};
  if (nl < rows) {
    if (epi.bias) epi_b = bf16_bits_to_f32(epi.bias[n]);
    if (epi.res) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * g + i < arows) epi_r[i] = residual_at<OUT_F32>(epi.res, (int64_t)(m0 + 4 * g + i) * N + n);
    }
  }
  f32x4_t sum = red[lane];
  for (int w = 1; w < waves; ++w) {
    const f32x4_t v = red[w * 64 + lane];
    sum[0] += v[0];
    sum[1] += v[1];
    sum[2] += v[2];
    sum[3] += v[3];
  }
  if (nl >= rows) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + 4 * g + i;
    if (m < M) {
      const int64_t mn = (int64_t)m * N + n;
      const float v = epilogue_value(epi, sum[i], epi_b, epi_r[i]);
      if constexpr (OUT_F32) {
        reinterpret_cast<float*>(C)[mn] = v;
      } else {
        reinterpret_cast<__bf16*>(C)[mn] = (__bf16)v;
      }
    }
  }
}

// FULL: K % 128 == 0, so every chunk of a k-block below KB exists and the
// validity of a k-block is the same for the whole wave.
// S_LDS: the workgroup's scale (and zero) bytes are copied to LDS once, in
// a few coalesced copies, instead of per-lane loads per k-block (those cost
// one memory request per row and k-block, as many as the weights).
// A_DMA (with !A_LDS): each wave copies the A rows of its own k-blocks
// straight into a private LDS region (asynchronous global -> LDS copies of
// contiguous 256-byte row pieces) instead of per-lane A loads.
// GROUPED: more than one member, blockIdx.z (a single GEMM reads member 0).
// PRIV (int4 groups of 128, few A rows; A_LDS, S_LDS and A_DMA off): each
// wave copies into an LDS region of its own exactly what it reads -- the A
// rows of its k-blocks (even / odd k order, plus a zero row) and the scales
// and zeros of its 16 rows and k-blocks -- so no workgroup barrier precedes
// the arithmetic (the wave's LDS writes and reads are ordered by themselves).
// The operands and their order are those of the A_LDS route: same bits.  With
// one virtual wave per wave (R = 1), a wave whose A pieces are all exact in
// fp16 stores them as fp16 and decodes on the fp16 route (kblock_mac_f16, 11
// instead of 19 VALU per 8 codes; the same bits), the others as bf16.  (With
// R = 2 the second route's registers cost a wave of occupancy, measured
// slower: decode chain +4 %.)
// R: virtual waves per wave.  The split of K is into virtual waves of U
// k-blocks each (virtual wave v sums k-blocks v U .. v U + U - 1, and the
// partial sums are added in v order); a wave computes R consecutive virtual
// waves into R accumulators.  The bits never depend on R, which launches of
// many workgroups set to 2 (half the waves per workgroup, so more of them
// fit a CU and more weight loads are in flight); R = 2 needs K covered in
// one pass.
// (PRIV, one virtual wave per wave, U = 2: at least 6 waves per SIMD, so that
// two workgroups of up to 12 waves share a CU -- one register more halves
// that, measured on the decode GEMV)
template <int FMT, bool OUT_F32, int U, int R, bool A_LDS, bool FULL, bool S_LDS, bool A_DMA, bool GROUPED,
          bool PRIV = false>
__global__ __launch_bounds__(64 * kMaxWaves)
__attribute__((amdgpu_waves_per_eu(PRIV && R == 1 && U == 2 ? 6 : 1)))
void skinny_kernel(SkinnyGroupOf<GROUPED> grp, int M, int K, Epilogue epi) {
  static_assert(!PRIV || ((is_int4_g128(FMT) || !is_int4(FMT)) && !A_LDS && !S_LDS && !A_DMA), "private staging");
  constexpr int UR = U * R;  // k-blocks per wave and pass
  // the group member whose columns this workgroup computes: its fields come
  // in one scalar load round trip at a workgroup-uniform offset
  const SkinnyMember& mem = grp.m[GROUPED ? (int)blockIdx.z : 0];
  const uint16_t* A = mem.A;
  const uint8_t* packed = mem.packed;
  const void* scales = mem.scales;
  const uint8_t* zeros = mem.zeros;
  void* C = mem.C;
  const int N = mem.N;
  const int n0 = (int)blockIdx.x * grp.rows;
  if (GROUPED && n0 >= N) return;  // past this member's columns (whole workgroup)
  // LDS copy of A: arows rows of K bf16, then one row of zeros that lanes
  // past M (and chunks past K) read instead of branching
  extern __shared__ __attribute__((aligned(16))) uint8_t a_lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int waves = blockDim.x >> 6;
  const int nl = lane & 15;  // weight row within the slice / A row supplied
  const int g = lane >> 4;   // 32-code chunk within the k-block
  const int m0 = blockIdx.y * 16;
  const int n = n0 + nl;
  const int chunks = K >> 5;           // 32-code chunks per row
  const int KB = (chunks + 3) >> 2;    // 128-code k-blocks (last may be partial)
  constexpr int G = FormatTraits<FMT>::kGroup;
  constexpr int SB = is_int4(FMT) ? 2 : 1;  // bytes per scale
  // int4: the group of 32-code chunk c is c >> GS (the k-block for G = 128)
  constexpr int GS = G == 128 ? 2 : (G == 64 ? 1 : 0);
  const int groups = (K + G - 1) / G;  // the last group may be shorter

  // Buffer descriptors over exactly this workgroup's 16 weight rows and 16 A
  // rows: rows past N or M, and k past K, read as 0 (hardware range check).
  const int rows = min(grp.rows, N - n0);  // lanes of rows past it read zeros
  const int arows = min(16, M - m0);

  const uint32_t rowb = (uint32_t)(K >> 1);
  // (prepacked: the whole 16-row tile, whose rows past N are zero bytes)
  const bool pre = grp.pre != 0;
  const rsrc_t wr = make_rsrc(packed + (int64_t)n0 * rowb, (uint32_t)(pre ? 16 : rows) * rowb);
  const rsrc_t ar = make_rsrc(A + (int64_t)m0 * K, (uint32_t)arows * (uint32_t)K * 2u);
  const rsrc_t sr = make_rsrc(reinterpret_cast<const uint8_t*>(scales) + (int64_t)n0 * groups * SB,
                              (uint32_t)(rows * groups * SB));
  const rsrc_t zr = make_rsrc(has_zeros(FMT) ? zeros + (int64_t)n0 * groups : nullptr,
                              has_zeros(FMT) ? (uint32_t)(rows * groups) : 0u);

  // Scale staging: rows n0 .. n0+rows-1 of the scales (and zeros) are one
  // contiguous block; it is read as dwords from the 4-byte aligned address at
  // or below its start (delta bytes before it) into registers, issued before
  // everything else, and written to LDS after the A region once they land.
  const int am = M < 16 ? M : 16;
  const uint32_t s_off = A_LDS ? (((uint32_t)(am + 1) * (uint32_t)K * 2u + 15u) & ~15u) : 0u;
  const uint32_t z_off = s_off + (((16u * (uint32_t)groups * SB + 6u) + 15u) & ~15u);
  const uint32_t z_cap = has_zeros(FMT) ? ((16u * (uint32_t)groups + 6u + 15u) & ~15u) : 0u;
  // per-wave A regions (A_DMA) after the scale and zero windows
  const uint32_t a_dma_off = S_LDS ? z_off + z_cap : s_off;
  const uint32_t a_wave = lds_address(a_lds) + a_dma_off +
                          (uint32_t)__builtin_amdgcn_readfirstlane(wave) * (uint32_t)(UR * 4096);
  // PRIV: this wave's region (priv_bytes, the launcher's skinny_priv_bytes):
  // A rows 0 .. am (row arows of the slice is zeros) x UR k-blocks x 256
  // bytes, then 16 x UR bf16 scales and 16 x UR zero bytes, entry r * UR + u
  // scale entries per row and k-block: the group (int4) or each chunk's scale (fp4)
  constexpr int kSC = is_int4(FMT) ? 1 : 4;
  constexpr int kNE = 16 * UR * kSC;  // entries of a wave: e = (r * UR + u) * kSC + chunk
  const uint32_t priv_a = (uint32_t)(am + 1) * (uint32_t)UR * 256u;
  const uint32_t priv_bytes = (priv_a + (uint32_t)kNE * 3u + 15u) & ~15u;
  uint8_t* const priv = a_lds + (uint32_t)__builtin_amdgcn_readfirstlane(wave) * priv_bytes;
  constexpr int kPS = 2;                   // 16-byte A pieces per lane
  constexpr int kPE = (kNE + 63) / 64;  // scale / zero entries per lane
  u32x4_t pst[kPS];
  uint32_t pss[kPE], pzs[kPE];
  uint32_t s_delta = 0, z_delta = 0, s_words = 0, z_words = 0;
  // staging loads are issued only by waves that hold some in-range slot
  // (a wave whose first slot is past the block skips the instruction)
  const uint32_t wave_slot0 = (uint32_t)__builtin_amdgcn_readfirstlane(wave) * 64u;
  uint32_t sst[kSStage], zst[kZStage];
  if constexpr (S_LDS) {
    auto window = [&](const uint8_t* start, uint32_t bytes, uint32_t& delta, uint32_t& words) {
      const uintptr_t al = reinterpret_cast<uintptr_t>(start) & ~(uintptr_t)3;
      delta = (uint32_t)(reinterpret_cast<uintptr_t>(start) - al);
      words = (delta + bytes + 3u) / 4u;  // may read <= 3 bytes past the block (same page)
      return make_rsrc(reinterpret_cast<const void*>(al), words * 4u);
    };
    const rsrc_t ss = window(reinterpret_cast<const uint8_t*>(scales) + (int64_t)n0 * groups * SB,
                             (uint32_t)(rows * groups * SB), s_delta, s_words);
#pragma unroll
    for (int i = 0; i < kSStage; ++i) {
      const uint32_t w = (uint32_t)(tid + i * (int)blockDim.x);
      sst[i] = wave_slot0 + i * blockDim.x < s_words ? buf_load_b32(ss, w < s_words ? w * 4u : kBufferOOB) : 0u;
    }
    if constexpr (has_zeros(FMT)) {
      const rsrc_t zs = window(zeros + (int64_t)n0 * groups, (uint32_t)(rows * groups), z_delta, z_words);
#pragma unroll
      for (int i = 0; i < kZStage; ++i) {
        const uint32_t w = (uint32_t)(tid + i * (int)blockDim.x);
        zst[i] = wave_slot0 + i * blockDim.x < z_words ? buf_load_b32(zs, w < z_words ? w * 4u : kBufferOOB) : 0u;
      }
    }
  }
  auto store_scales = [&]() {
    if constexpr (S_LDS) {
#pragma unroll
      for (int i = 0; i < kSStage; ++i) {
        const uint32_t w = (uint32_t)(tid + i * (int)blockDim.x);
        if (w < s_words) reinterpret_cast<uint32_t*>(a_lds + s_off)[w] = sst[i];
      }
      if constexpr (has_zeros(FMT)) {
#pragma unroll
        for (int i = 0; i < kZStage; ++i) {
          const uint32_t w = (uint32_t)(tid + i * (int)blockDim.x);
          if (w < z_words) reinterpret_cast<uint32_t*>(a_lds + z_off)[w] = zst[i];
        }
      }
    }
  };

  // A staging (few rows): the whole workgroup copies its A rows to LDS once.
  // These loads are issued first, so waiting for them (vmcnt retires in
  // issue order) does not wait for the weight stream issued after them.
  u32x4_t astage[kAStage];
  const int a16 = arows * K / 8;  // 16-byte chunks of this slice of A
  if constexpr (A_LDS) {
#pragma unroll
    for (int i = 0; i < kAStage; ++i) {
      const int ch = tid + i * (int)blockDim.x;
      astage[i] = (int)(wave_slot0 + i * blockDim.x) < a16
                      ? buf_load_b128(ar, ch < a16 ? (uint32_t)ch * 16u : kBufferOOB)
                      : u32x4_t{0, 0, 0, 0};
    }
  }

  f32x4_t acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  u32x4_t q[UR];
  u32x4_t a[UR][4];
  uint32_t sraw[UR];
  uint32_t zraw[UR];

  // Each wave owns UR consecutive k-blocks per pass (contiguous bytes of every
  // row it reads); pass p covers k-blocks [(p * waves + wave) * UR, +UR).
  auto valid = [&](int kb, int c) { return FULL ? (kb < KB) : (kb < KB && c < chunks); };
  auto issue = [&](int kbase) {
    if constexpr (PRIV) {
      // A piece i of lane l: qi = l + 64 i = (r * UR + u) * 16 + p -> row r,
      // k-block kbase + u, bytes 16 p .. of its 256 (launcher: arows * UR <= 8)
#pragma unroll
      for (int i = 0; i < kPS; ++i) {
        const int qi = lane + 64 * i;
        const int r = qi / (UR * 16), u = (qi / 16) % UR, p = qi % 16;
        const int kb = kbase + u;
        const bool ok = r < arows && kb < KB && (FULL || kb * 128 + p * 8 < K);
        pst[i] = buf_load_b128(ar, ok ? ((uint32_t)r * (uint32_t)K + (uint32_t)kb * 128u + (uint32_t)p * 8u) * 2u
                                      : kBufferOOB);
      }
      // scale (and zero) entry e = (r * UR + u) * kSC + h: row r, k-block
      // kbase + u, its group (int4) or chunk h's scale(s) (fp4: NVFP4 the
      // chunk's two e4m3 bytes, MXFP4 its e8m0 byte)
#pragma unroll
      for (int i = 0; i < kPE; ++i) {
        const int e = lane + 64 * i;
        const int r = e / (UR * kSC), kb = kbase + (e / kSC) % UR, c = kb * 4 + e % kSC;
        const bool ok = e < kNE && kb < KB && (is_int4(FMT) || FULL || c < chunks);
        if constexpr (is_int4(FMT)) {
          const uint32_t gi = (uint32_t)(r * groups + kb);
          pss[i] = buf_load_b16(sr, ok ? gi * 2u : kBufferOOB);
          pzs[i] = has_zeros(FMT) ? buf_load_b8(zr, ok ? gi : kBufferOOB) : kSymZero;
        } else if constexpr (FMT == kNvfp4) {
          pss[i] = buf_load_b16(sr, ok ? (uint32_t)(r * groups + 2 * c) : kBufferOOB);
          pzs[i] = 0u;
        } else {
          pss[i] = buf_load_b8(sr, ok ? (uint32_t)(r * groups + c) : kBufferOOB);
          pzs[i] = 0u;
        }
      }
    }
    // scales first: vmcnt retires in issue order, so the first k-block's
    // arithmetic then waits only for its own weights
#pragma unroll
    for (int u = 0; u < (S_LDS || PRIV ? 0 : UR); ++u) {
      const int kb = kbase + u;
      const int c = kb * 4 + g;
      const bool ok = valid(kb, c);
      if constexpr (is_int4(FMT)) {
        // groups of 128: every chunk of a k-block takes the k-block's group,
        // also chunks past K -- the MFMA sums the four chunks before the
        // lane applies the scale to its rows of the sum
        const uint32_t gi = (uint32_t)(nl * groups + (is_int4_g128(FMT) ? kb : c >> GS));
        const bool sok = is_int4_g128(FMT) ? kb < KB : ok;
        sraw[u] = buf_load_b16(sr, sok ? gi * 2u : kBufferOOB);
        zraw[u] = has_zeros(FMT) ? buf_load_b8(zr, sok ? gi : kBufferOOB) : kSymZero;
      } else if constexpr (FMT == kNvfp4) {
        // the chunk's two e4m3 scales (blocks 2c and 2c+1), one 16-bit load
        sraw[u] = buf_load_b16(sr, ok ? (uint32_t)(nl * groups + 2 * c) : kBufferOOB);
      } else {
        sraw[u] = buf_load_b8(sr, ok ? (uint32_t)(nl * groups + c) : kBufferOOB);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (A_DMA) {
      // k-block kb -> slot u: rows 4i .. 4i+3 per copy; lane -> row 4i + l/16,
      // LDS chunk l%16, which holds 16-byte chunk (l%16) ^ row of the row's
      // 256 bytes (the fragment reads of 16 rows then hit distinct banks)
#pragma unroll
      for (int u = 0; u < UR; ++u) {
        const int kb = kbase + u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * i + (lane >> 4);
          const int ch = (lane & 15) ^ r;
          const bool ok = kb < KB && (FULL || kb * 128 + 8 * ch < K);
          lds_dma_b128(ar, a_wave + (uint32_t)(u * 4096 + i * 1024),
                       ok ? ((uint32_t)r * (uint32_t)K + (uint32_t)kb * 128u + 8u * (uint32_t)ch) * 2u
                          : kBufferOOB);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < UR; ++u) {
      const int kb = kbase + u;
      const int c = kb * 4 + g;
      const bool ok = valid(kb, c);
      q[u] = buf_load_b128(wr, ok ? wchunk((uint32_t)nl, (uint32_t)c, rowb, pre) : kBufferOOB);
      if constexpr (!A_LDS && !A_DMA && !PRIV) {
        const uint32_t aoff = ((uint32_t)nl * (uint32_t)K + (uint32_t)c * 32u) * 2u;
#pragma unroll
        for (int j = 0; j < 4; ++j) a[u][j] = buf_load_b128(ar, ok ? aoff + 16u * j : kBufferOOB);
      }
    }
    // keep the whole batch of loads in flight: the scheduler may not sink
    // them next to their uses (that would serialise the memory latencies)
    __builtin_amdgcn_sched_barrier(0);
  };

  const int arow = nl < arows ? nl : arows;  // row arows of the LDS copy is zeros
  constexpr bool kF16 = PRIV && R == 1 && is_int4_g128(FMT);  // the fp16 route
  bool w16 = false;  // kF16: this wave's A copy is fp16 (set per pass, wave-uniform)
  const F16Consts fc = f16_consts();
  auto compute = [&](int kbase) {
    // the copies are invisible to the compiler's own waits: wait for all of
    // this pass's loads (whatever order they were issued in)
    if constexpr (A_DMA) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if constexpr (PRIV) {
      // this wave's region: its A pieces (even / odd k order), the zero row,
      // its scales and zeros; read back below by the same wave only
      // fp16 when every A value of this wave converts exactly (wave-uniform):
      // the fp16 pieces are written as they are converted, and rewritten in
      // bf16 when some value did not convert (the wave's LDS writes land in
      // order)
      if constexpr (kF16) {
        bool exact = true;
#pragma unroll
        for (int i = 0; i < kPS; ++i) {
          const int qi = lane + 64 * i;
          if (qi < arows * UR * 16) reinterpret_cast<u32x4_t*>(priv)[qi] = bf16x8_to_f16_k04(pst[i], exact);
        }
        w16 = __ballot(!exact) == 0;
      }
      if (!(kF16 && w16)) {
#pragma unroll
        for (int i = 0; i < kPS; ++i) {
          const int qi = lane + 64 * i;
          if (qi < arows * UR * 16)
            reinterpret_cast<u32x4_t*>(priv)[qi] = is_int4_g128(FMT) ? bf16x8_even_odd(pst[i]) : pst[i];
        }
      }
      for (int qi = lane; qi < UR * 16; qi += 64)
        reinterpret_cast<u32x4_t*>(priv + (uint32_t)arows * UR * 256u)[qi] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < kPE; ++i) {
        const int e = lane + 64 * i;
        if (e < kNE) {
          reinterpret_cast<uint16_t*>(priv + priv_a)[e] = (uint16_t)pss[i];
          (priv + priv_a + 2u * kNE)[e] = (uint8_t)pzs[i];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < UR; ++u) {
      const int kb = kbase + u;
      if (FULL && kb >= KB) break;  // wave-uniform: nothing was loaded
      if constexpr (PRIV) {
        // row arow of the region (arows: the zero row), chunk g of k-block u
        const u32x4_t* src = reinterpret_cast<const u32x4_t*>(priv + ((uint32_t)arow * UR + u) * 256u + g * 64u);
#pragma unroll
        for (int j = 0; j < 4; ++j) a[u][j] = src[j];
        const int e = (nl * UR + u) * kSC + (kSC == 4 ? g : 0);
        sraw[u] = reinterpret_cast<const uint16_t*>(priv + priv_a)[e];
        zraw[u] = (priv + priv_a + 2u * kNE)[e];
      }
      if constexpr (A_DMA) {
        const uint8_t* src = a_lds + a_dma_off + (size_t)wave * (UR * 4096) + u * 4096 + nl * 256;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          a[u][j] = *reinterpret_cast<const u32x4_t*>(src + (((4 * g + j) ^ nl) * 16));
      }
      if constexpr (A_LDS) {
        const int c = kb * 4 + g;
        const int col = (FULL || c < chunks) ? c * 32 : 0;
        const int row = (FULL || c < chunks) ? arow : arows;
        const u32x4_t* src =
            reinterpret_cast<const u32x4_t*>(a_lds + ((size_t)row * K + (size_t)col) * 2);
#pragma unroll
        for (int j = 0; j < 4; ++j) a[u][j] = src[j];
      }
      if constexpr (S_LDS) {
        // this lane's scale (and zero) bytes from the staged block; past K
        // the weights and A are zero, so any finite scale will do
        const int c = kb * 4 + g;
        const bool ok = FULL || c < chunks;
        const uint8_t* sb = a_lds + s_off + s_delta;
        if constexpr (is_int4(FMT)) {
          // groups of 128: the k-block's group for every chunk (see issue);
          // past the last k-block (nothing loaded) group 0 keeps the read
          // inside the window
          const int gi = nl * groups + (is_int4_g128(FMT) ? (kb < KB ? kb : 0) : (ok ? c >> GS : 0));
          sraw[u] = *reinterpret_cast<const uint16_t*>(sb + 2 * gi);
          zraw[u] = has_zeros(FMT) ? (uint32_t)(a_lds + z_off + z_delta)[gi] : kSymZero;
        } else if constexpr (FMT == kNvfp4) {
          sraw[u] = *reinterpret_cast<const uint16_t*>(sb + nl * groups + 2 * (ok ? c : 0));
        } else {
          sraw[u] = sb[nl * groups + (ok ? c : 0)];
        }
      }
      if (kF16 && w16)
        acc[u / U] = kblock_mac_f16(a[u], q[u], sraw[u], zraw[u], acc[u / U], fc);
      else
        acc[u / U] = kblock_mac<FMT, A_LDS || PRIV>(a[u], q[u], sraw[u], is_int4(FMT) ? zraw[u] : 0u, acc[u / U]);
    }
  };

  int kbase = wave * UR;
  issue(kbase);
  // LDS-only barriers: each wave's weights stay in flight, and its first
  // k-block's arithmetic waits for that k-block's load alone
  if constexpr (S_LDS && !A_LDS) {
    store_scales();
    lds_barrier();
  }
  if constexpr (A_LDS) {
    store_scales();
    // copy the staged rows, then zero row `arows` (a16 .. a16 + K/8 chunks)
#pragma unroll
    for (int i = 0; i < kAStage; ++i) {
      const int ch = tid + i * (int)blockDim.x;
      // int4 codes decode in the k order (0,2,4,6,1,3,5,7) per 8: A follows it
      const u32x4_t v = is_int4_g128(FMT) ? bf16x8_even_odd(astage[i]) : astage[i];
      if (ch < a16) reinterpret_cast<u32x4_t*>(a_lds)[ch] = v;
    }
    for (int ch = a16 + tid; ch < a16 + K / 8; ch += blockDim.x)
      reinterpret_cast<u32x4_t*>(a_lds)[ch] = u32x4_t{0, 0, 0, 0};
    lds_barrier();
  }
  compute(kbase);
  for (kbase += waves * UR; kbase < KB; kbase += waves * UR) {
    issue(kbase);
    compute(kbase);
  }

  // ---- split-K reduction across the waves, through LDS ----------------------
  // (virtual wave wave * R + r)
  __shared__ f32x4_t red[kMaxWaves][64];
#pragma unroll
  for (int r = 0; r < R; ++r) red[wave * R + r][lane] = acc[r];
  lds_barrier();
  if (wave != 0) return;
  skinny_store<OUT_F32>(&red[0][0], waves * R, lane, nl, g, rows, arows, m0, n, M, N, C, epi);
}

// ---- ring variant: every per-k-block operand through LDS copies ----------
//
// For A slices too large for the one-time LDS copy (e.g. 16 rows x 8192).
// K is split over kRingVirt = 8 virtual waves: virtual wave v sums k-blocks
// v, v + 8, v + 16, ... in that order, and the 8 partial sums are added in
// order v = 0 .. 7, whatever the number of real waves W = 8 / R: real wave w
// computes k-blocks w, w + W, w + 2W, ... and its j-th goes to accumulator
// j % R (virtual wave w + W (j % R)).  So every W gives the same bits, and a
// grouped launch (more workgroups, possibly another W) equals the single
// ones.  The A rows (16 x 256
// bytes) and the weight rows (16 x 64 bytes) of each k-block arrive by
// asynchronous global -> LDS copies in one of the wave's D ring slots, issued
// D k-blocks ahead, so the copies of the next D - 1 k-blocks are in flight
// while one is computed.  The scale (and zero) window arrives the same way,
// once.  No operand goes through a load the compiler can see, so every wait is
// an explicit count of the copies issued after the one needed (vmcnt retires
// in issue order) and never includes later copies.
// LDS: scale window, zero window (int4), W * D slots of kRingSlot bytes, then
// kRingVirt * 64 f32x4 partial sums.
constexpr uint32_t kRingSlot = 5120;  // A 16 x 256 bytes, then weights 16 x 64 bytes
constexpr int kRingVirt = 8;          // virtual waves of the K split

// wait until at most `later` k-blocks' copies (5 each) are still in flight
template <int D>
__device__ __forceinline__ void ring_wait(int later) {
  static_assert(D >= 2 && D <= 4, "ring depth");
  if (D > 3 && later >= 3) {
    asm volatile("s_waitcnt vmcnt(15)" ::: "memory");
  } else if (D > 2 && later >= 2) {
    asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
  } else if (later >= 1) {
    asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

// bytes of a copied window of `bytes` (plus <= 3 before and after it for
// dword alignment), whole 256-byte copy instructions
__host__ __device__ constexpr uint32_t ring_window_cap(uint32_t bytes) {
  return (bytes + 6u + 255u) / 256u * 256u;
}

template <int FMT, bool OUT_F32, int D, int R, bool FULL, bool GROUPED>
__global__ __launch_bounds__(64 * kRingVirt) void skinny_ring_kernel(SkinnyGroupOf<GROUPED> grp, int M, int K,
                                                                     Epilogue epi) {
  const SkinnyMember& mem = grp.m[GROUPED ? (int)blockIdx.z : 0];
  const uint16_t* A = mem.A;
  const uint8_t* packed = mem.packed;
  const uint8_t* scales = reinterpret_cast<const uint8_t*>(mem.scales);
  const uint8_t* zeros = mem.zeros;
  void* C = mem.C;
  const int N = mem.N;
  const int n0 = (int)blockIdx.x * grp.rows;
  if (GROUPED && n0 >= N) return;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int waves = kRingVirt / R;  // the launch has exactly these
  const int nl = lane & 15;
  const int g = lane >> 4;
  const int m0 = blockIdx.y * 16;
  const int n = n0 + nl;
  const int chunks = K >> 5;
  const int KB = (chunks + 3) >> 2;
  constexpr int G = FormatTraits<FMT>::kGroup;
  constexpr int SB = is_int4(FMT) ? 2 : 1;
  constexpr int GS = G == 128 ? 2 : (G == 64 ? 1 : 0);
  const int groups = (K + G - 1) / G;  // the last group may be shorter
  const int rows = min(grp.rows, N - n0);
  const int arows = min(16, M - m0);

  const uint32_t rowb = (uint32_t)(K >> 1);
  const bool pre = grp.pre != 0;
  const rsrc_t wr = make_rsrc(packed + (int64_t)n0 * rowb, (uint32_t)(pre ? 16 : rows) * rowb);
  const rsrc_t ar = make_rsrc(A + (int64_t)m0 * K, (uint32_t)arows * (uint32_t)K * 2u);

  const uint32_t s_cap = ring_window_cap(16u * (uint32_t)groups * SB);
  const uint32_t z_cap = has_zeros(FMT) ? ring_window_cap(16u * (uint32_t)groups) : 0u;
  const uint32_t base = lds_address(lds);
  const uint32_t my_ring = s_cap + z_cap + (uint32_t)wave * (uint32_t)(D * kRingSlot);
  f32x4_t* red = reinterpret_cast<f32x4_t*>(lds + s_cap + z_cap + (uint32_t)waves * (D * kRingSlot));

  // window copies: dwords from the 4-byte aligned address at or below the
  // block's start (delta bytes before it); instruction t of the window moves
  // dwords 64t .. 64t+63, and the waves take turns
  auto window = [&](const uint8_t* start, uint32_t bytes, uint32_t lds_off) {
    const uintptr_t al = reinterpret_cast<uintptr_t>(start) & ~(uintptr_t)3;
    const uint32_t delta = (uint32_t)(reinterpret_cast<uintptr_t>(start) - al);
    const uint32_t words = (delta + bytes + 3u) / 4u;  // may read <= 3 bytes past the block (same page)
    const rsrc_t r = make_rsrc(reinterpret_cast<const void*>(al), words * 4u);
    const int instrs = (int)((words + 63u) / 64u);
    for (int t = wave; t < instrs; t += waves)
      lds_dma_b32(r, base + lds_off + (uint32_t)t * 256u, ((uint32_t)t * 64u + (uint32_t)lane) * 4u);
    return delta;
  };
  const uint32_t s_delta = window(scales + (int64_t)n0 * groups * SB, (uint32_t)(rows * groups * SB), 0u);
  uint32_t z_delta = 0;
  if constexpr (has_zeros(FMT)) z_delta = window(zeros + (int64_t)n0 * groups, (uint32_t)(rows * groups), s_cap);

  // this wave's k-blocks: kb = i * waves + wave, i = 0 .. nk-1
  const int nk = wave < KB ? (KB - 1 - wave) / waves + 1 : 0;
  // k-block i -> slot i % D.  A: instruction r4 moves rows 4 r4 .. 4 r4 + 3,
  // lane -> row 4 r4 + l/16 and LDS chunk l%16, which holds 16-byte chunk
  // (l%16) ^ row of the row's 256 bytes (the fragment reads of 16 rows then
  // hit distinct banks).  Weights: lane -> row l/4, 16-byte chunk l%4.
  auto issue = [&](int i) {
    const int kb = i * waves + wave;
    const uint32_t slot = base + my_ring + (uint32_t)(i % D) * kRingSlot;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int r = 4 * r4 + (lane >> 4);
      const int ch = (lane & 15) ^ r;
      const bool ok = FULL || kb * 128 + 8 * ch < K;
      lds_dma_b128(ar, slot + (uint32_t)r4 * 1024u,
                   ok ? ((uint32_t)r * (uint32_t)K + (uint32_t)kb * 128u + 8u * (uint32_t)ch) * 2u : kBufferOOB);
    }
    // (prepacked: lane -> row l%16, chunk l/16: one contiguous kilobyte)
    const int wrow = pre ? (lane & 15) : (lane >> 2), wch = pre ? (lane >> 4) : (lane & 3);
    const bool okw = FULL || kb * 4 + wch < chunks;
    lds_dma_b128(wr, slot + 4096u,
                 okw ? wchunk((uint32_t)wrow, (uint32_t)(kb * 4 + wch), rowb, pre) : kBufferOOB);
  };
  const int first = nk < D ? nk : D;
  for (int i = 0; i < first; ++i) issue(i);
  // the window (issued first) and k-block 0 have landed in this wave's part;
  // after the barrier every wave's part has
  ring_wait<D>(first - 1);
  lds_barrier();

  f32x4_t acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint8_t* sb = lds + s_delta;
  const uint8_t* zb = lds + s_cap + z_delta;
  for (int i0 = 0; i0 < nk; i0 += R) {
#pragma unroll
   for (int r = 0; r < R; ++r) {
    const int i = i0 + r;
    if (i >= nk) break;  // wave-uniform
    if (i > 0) ring_wait<D>(min(D - 1, nk - 1 - i));
    const int kb = i * waves + wave;
    const uint8_t* slot = lds + my_ring + (uint32_t)(i % D) * kRingSlot;
    u32x4_t a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      a[j] = *reinterpret_cast<const u32x4_t*>(slot + nl * 256 + (((4 * g + j) ^ nl) * 16));
    const u32x4_t q = *reinterpret_cast<const u32x4_t*>(slot + 4096 + (pre ? nl + 16 * g : nl * 4 + g) * 16);
    // this lane's scale (and zero) bytes; past K the weights and A are zero,
    // so any finite scale will do
    const int c = kb * 4 + g;
    const bool ok = FULL || c < chunks;
    uint32_t sraw, zraw = 0u;
    if constexpr (is_int4(FMT)) {
      // groups of 128: the k-block's group for every chunk, also past K (the
      // MFMA sums the four chunks before the scale is applied)
      const int gi = nl * groups + (is_int4_g128(FMT) ? kb : (ok ? c >> GS : 0));
      sraw = *reinterpret_cast<const uint16_t*>(sb + 2 * gi);
      zraw = has_zeros(FMT) ? (uint32_t)zb[gi] : kSymZero;
    } else if constexpr (FMT == kNvfp4) {
      sraw = *reinterpret_cast<const uint16_t*>(sb + nl * groups + 2 * (ok ? c : 0));
    } else {
      sraw = sb[nl * groups + (ok ? c : 0)];
    }
    acc[r] = kblock_mac<FMT, false>(a, q, sraw, zraw, acc[r]);
    if (i + D < nk) {
      // the slot's reads have completed before its next copy is issued
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue(i + D);
    }
   }
  }

#pragma unroll
  for (int r = 0; r < R; ++r) red[(wave + waves * r) * 64 + lane] = acc[r];
  lds_barrier();
  if (wave != 0) return;
  skinny_store<OUT_F32>(red, kRingVirt, lane, nl, g, rows, arows, m0, n, M, N, C, epi);
}

// ---- streaming variant: one workgroup walks many column tiles -------------
//
// For launches of several rounds of 16-column tiles.  A workgroup stages A in
// LDS once and then computes tiles t = blockIdx.x, blockIdx.x + gridDim.x,
// ... with the same split of K over its waves as the one-tile kernel (so both
// give the same bits).  Loads run two tiles ahead: while tile s is computed,
// the weights of tiles s+1 and s+2 are in flight (three register sets) and
// the scales of tile s+1, loaded one step earlier, go to LDS.  Each step has
// one barrier, which orders LDS only and never waits for loads in flight.
// Every load is issued unconditionally (tiles past the last get empty
// descriptors), so the compiler's wait counts for one tile never include the
// loads of later tiles.
// Conditions, checked by the launcher: K % 128 == 0; each wave covers its U
// k-blocks of a tile in one pass (waves * U >= K / 128); the M <= 16 rows of
// A fit the staging registers; NS scale dwords per lane (and one zero dword,
// int4) cover a tile's scale window.
template <int FMT, bool OUT_F32, int U, int NS>
__global__ __launch_bounds__(64 * kMaxWaves) void skinny_stream_kernel(SkinnyGroup<1> grp, int M, int K,
                                                                       int tiles, Epilogue epi) {
  const uint16_t* A = grp.m[0].A;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int waves = blockDim.x >> 6;
  const int nl = lane & 15;  // weight row within the tile / A row supplied
  const int g = lane >> 4;   // 32-code chunk within the k-block
  const int KB = K >> 7;
  constexpr int G = FormatTraits<FMT>::kGroup;
  constexpr int SB = is_int4_g128(FMT) ? 2 : 1;
  const int groups = (K + G - 1) / G;  // the last group may be shorter
  const uint32_t rowb = (uint32_t)(K >> 1);
  const uint32_t wave_slot0 = (uint32_t)__builtin_amdgcn_readfirstlane(wave) * 64u;
  const int kw = __builtin_amdgcn_readfirstlane(wave) * U;  // this wave's first k-block

  // LDS: A (M rows, then a row of zeros), three scale/zero buffers, three
  // reduction buffers of [waves][64] f32x4
  const uint32_t s_cap = ((16u * (uint32_t)groups * SB + 6u) + 15u) & ~15u;
  const uint32_t z_cap = FMT == kInt4 ? ((16u * (uint32_t)groups + 6u + 15u) & ~15u) : 0u;
  const uint32_t buf0 = ((uint32_t)(M + 1) * (uint32_t)K * 2u + 15u) & ~15u;
  f32x4_t* red = reinterpret_cast<f32x4_t*>(lds + buf0 + 3u * (s_cap + z_cap));

  // A loads first (vmcnt retires in issue order)
  const rsrc_t ar = make_rsrc(A, (uint32_t)M * (uint32_t)K * 2u);
  const int a16 = M * K / 8;  // 16-byte chunks of A
  u32x4_t astage[kAStage];
#pragma unroll
  for (int i = 0; i < kAStage; ++i) {
    const int ch = tid + i * (int)blockDim.x;
    astage[i] = (int)(wave_slot0 + i * blockDim.x) < a16
                    ? buf_load_b128(ar, ch < a16 ? (uint32_t)ch * 16u : kBufferOOB)
                    : u32x4_t{0, 0, 0, 0};
  }

  // a tile: its place and its weights (in flight or landed)
  struct Tile {
    int t, n0, rows, N;
    void* C;
    const uint8_t* scales;
    const uint8_t* zeros;
    u32x4_t q[U];
  };
  // the scale (and zero) window of one tile, in flight in registers
  struct Scales {
    uint32_t delta, zdelta, words, zwords;
    uint32_t s[NS], z;
  };
  // t >= tiles: the same loads over empty ranges (they return zeros)
  auto issue = [&](Tile& T, Scales& S, int t) {
    const bool live = t < tiles;
    const uint8_t* packed = grp.m[0].packed;
    T.scales = reinterpret_cast<const uint8_t*>(grp.m[0].scales);
    T.zeros = grp.m[0].zeros;
    T.C = grp.m[0].C;
    T.N = grp.m[0].N;
    T.t = t;
    T.n0 = t * 16;
    T.rows = live ? min(16, T.N - T.n0) : 0;
    // the tile's scale (and zero) rows are one contiguous block, read as
    // dwords from the 4-byte aligned address at or below its start
    auto window = [&](const uint8_t* start, uint32_t bytes, uint32_t& delta, uint32_t& words) {
      const uintptr_t al = reinterpret_cast<uintptr_t>(start) & ~(uintptr_t)3;
      delta = (uint32_t)(reinterpret_cast<uintptr_t>(start) - al);
      words = bytes ? (delta + bytes + 3u) / 4u : 0u;  // may read <= 3 bytes past the block (same dword)
      return make_rsrc(reinterpret_cast<const void*>(al), words * 4u);
    };
    const rsrc_t ss = window(T.scales + (int64_t)T.n0 * groups * SB, (uint32_t)(T.rows * groups * SB),
                             S.delta, S.words);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const uint32_t w = (uint32_t)(tid + i * (int)blockDim.x);
      S.s[i] = buf_load_b32(ss, w < S.words ? w * 4u : kBufferOOB);
    }
    if constexpr (FMT == kInt4) {
      const rsrc_t zs = window(T.zeros + (int64_t)T.n0 * groups, (uint32_t)(T.rows * groups), S.zdelta, S.zwords);
      S.z = buf_load_b32(zs, (uint32_t)tid < S.zwords ? (uint32_t)tid * 4u : kBufferOOB);
    }
    // weights: rows past the tile's last read as zeros (descriptor range;
    // prepacked: the whole 16-row tile, zero bytes past N)
    const rsrc_t wr = make_rsrc(packed + (int64_t)T.n0 * rowb,
                                (uint32_t)(grp.pre && live ? 16 : T.rows) * rowb);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = kw + u;
      T.q[u] = buf_load_b128(wr, kb < KB ? wchunk((uint32_t)nl, (uint32_t)(kb * 4 + g), rowb, grp.pre != 0)
                                         : kBufferOOB);
    }
    // keep the batch in flight: no load may sink towards its use
    __builtin_amdgcn_sched_barrier(0);
  };
  // scale buffer b: the window's dwords, and where its first byte sits
  uint32_t sdelta[3], zdelta[3];
  auto store_scales = [&](const Scales& S, int b) {
    uint32_t* sbuf = reinterpret_cast<uint32_t*>(lds + buf0 + (uint32_t)b * (s_cap + z_cap));
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const uint32_t w = (uint32_t)(tid + i * (int)blockDim.x);
      if (w < S.words) sbuf[w] = S.s[i];
    }
    if constexpr (FMT == kInt4) {
      uint32_t* zbuf = reinterpret_cast<uint32_t*>(lds + buf0 + (uint32_t)b * (s_cap + z_cap) + s_cap);
      if ((uint32_t)tid < S.zwords) zbuf[tid] = S.z;
    }
    sdelta[b] = S.delta;
    zdelta[b] = S.zdelta;
  };
  const int arow = nl < M ? nl : M;  // row M of the LDS copy is zeros
  auto compute = [&](const Tile& T, int b) {
    const uint8_t* sb = lds + buf0 + (uint32_t)b * (s_cap + z_cap) + sdelta[b];
    const uint8_t* zb = lds + buf0 + (uint32_t)b * (s_cap + z_cap) + s_cap + zdelta[b];
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = kw + u;
      if (kb >= KB) break;  // wave-uniform
      const int c = kb * 4 + g;
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(lds + ((size_t)arow * K + (size_t)c * 32) * 2);
      u32x4_t a[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = src[j];
      if constexpr (is_int4_g128(FMT)) {
        // code - zero exact (in the even / odd k order A is stored in), the
        // group scale on the k-block's sum
        const int gi = nl * groups + kb;
        const float s = bf16_bits_to_f32(*reinterpret_cast<const uint16_t*>(sb + 2 * gi));
        const float zf = (float)(has_zeros(FMT) ? (uint32_t)zb[gi] : kSymZero);
        f32x4_t dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) dp = mfma16x16x32(a[j], int4x8_minus_zero_even_odd(T.q[u][j], zf), dp);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(s, dp[i], acc[i]);
      } else if constexpr (FMT == kNvfp4) {
        const uint32_t sraw = *reinterpret_cast<const uint16_t*>(sb + nl * groups + 2 * c);
        const float s0 = e4m3_magnitude(sraw & 0xFFu);
        const float s1 = e4m3_magnitude(sraw >> 8);
        acc = mfma16x16x32(a[0], fp4x8_to_bf16_fscale(T.q[u][0], s0), acc);
        acc = mfma16x16x32(a[1], fp4x8_to_bf16_fscale(T.q[u][1], s0), acc);
        acc = mfma16x16x32(a[2], fp4x8_to_bf16_fscale(T.q[u][2], s1), acc);
        acc = mfma16x16x32(a[3], fp4x8_to_bf16_fscale(T.q[u][3], s1), acc);
      } else {
        const float es = e8m0_as_exponent_scale(sb[nl * groups + c]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = mfma16x16x32(a[j], fp4x8_to_bf16_escale(T.q[u][j], es), acc);
      }
    }
    return acc;
  };
  // split-K sum over the waves (wave 0, in wave order) and the tile's stores
  auto reduce_store = [&](const Tile& T, int b) {
    // epilogue operands first (one round trip; the residual may alias C)
    float eb = 0.f, er[4] = {0.f, 0.f, 0.f, 0.f};
    if (epi.on && nl < T.rows) {
      const int n = T.n0 + nl;
      if (epi.bias) eb = bf16_bits_to_f32(epi.bias[n]);
      if (epi.res) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * g + i < M) er[i] = residual_at<OUT_F32>(epi.res, (int64_t)(4 * g + i) * T.N + n);
      }
    }
    const f32x4_t* r = red + b * waves * 64 + lane;
    f32x4_t sum = r[0];
    for (int w = 1; w < waves; ++w) {
      const f32x4_t v = r[w * 64];
      sum[0] += v[0];
      sum[1] += v[1];
      sum[2] += v[2];
      sum[3] += v[3];
    }
    if (nl >= T.rows) return;
    const int n = T.n0 + nl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * g + i;
      if (m < M) {
        const int64_t mn = (int64_t)m * T.N + n;
        const float v = epi.on ? epilogue_value(epi, sum[i], eb, er[i]) : sum[i];
        if constexpr (OUT_F32) {
          reinterpret_cast<float*>(T.C)[mn] = v;
        } else {
          reinterpret_cast<__bf16*>(T.C)[mn] = (__bf16)v;
        }
      }
    }
  };

  // prologue: tiles 0 and 1 of this workgroup in flight, A and tile 0's
  // scales in LDS
  Tile T0, T1, T2;
  Scales S;
  const int G0 = (int)gridDim.x;
  issue(T0, S, (int)blockIdx.x);
#pragma unroll
  for (int i = 0; i < kAStage; ++i) {
    const int ch = tid + i * (int)blockDim.x;
    // int4 codes decode in the k order (0,2,4,6,1,3,5,7) per 8: A follows it
    const u32x4_t v = is_int4_g128(FMT) ? bf16x8_even_odd(astage[i]) : astage[i];
    if (ch < a16) reinterpret_cast<u32x4_t*>(lds)[ch] = v;
  }
  for (int ch = a16 + tid; ch < a16 + K / 8; ch += blockDim.x)
    reinterpret_cast<u32x4_t*>(lds)[ch] = u32x4_t{0, 0, 0, 0};
  store_scales(S, 0);
  issue(T1, S, (int)blockIdx.x + G0);

  // step s (buffers s % 3): tile s+1's scales (loaded one step ago) to LDS,
  // tile s+2's loads issued, tile s computed, barrier, tile s reduced
  auto step = [&](Tile& cur, Tile& far, int b) {
    store_scales(S, (b + 1) % 3);
    issue(far, S, cur.t + 2 * G0);
    red[(b * waves + wave) * 64 + lane] = compute(cur, b);
    lds_barrier();
    if (wave == 0) reduce_store(cur, b);
  };
  lds_barrier();
  // a loop with its one exit at the bottom (an exit between steps would
  // reach the loop head, in the compiler's view, with loads pending in
  // registers it reuses, and cost a full wait)
  const int mine = (tiles - (int)blockIdx.x + G0 - 1) / G0;
  int i = 0;
  for (; i + 2 < mine; i += 3) {
    step(T0, T2, 0);
    step(T1, T0, 1);
    step(T2, T1, 2);
  }
  if (i < mine) step(T0, T2, 0);
  if (i + 1 < mine) step(T1, T0, 1);
}

// The launch's members (CAP slots: 1 for a single GEMM) and its grid: x =
// column tiles of `rows` (of the widest member), y = 16-row slices of A,
// z = members; a member with fewer tiles than the widest has workgroups that
// exit at once.
template <int CAP>
SkinnyGroup<CAP> skinny_group(const GroupedArgs& a, int rows) {
  SkinnyGroup<CAP> grp = {};
  for (int i = 0; i < a.count && i < CAP; ++i) {
    grp.m[i].A = a.A[i];
    grp.m[i].packed = a.packed[i];
    grp.m[i].scales = a.scales[i];
    grp.m[i].zeros = a.zeros[i];
    grp.m[i].C = a.C[i];
    grp.m[i].N = (int)a.N[i];
  }
  grp.rows = rows;
  grp.pre = a.pre ? 1 : 0;
  return grp;
}
dim3 skinny_grid(const GroupedArgs& a, int rows) {
  int64_t max_n = 0;
  for (int i = 0; i < a.count; ++i) max_n = a.N[i] > max_n ? a.N[i] : max_n;
  return dim3((unsigned)((max_n + rows - 1) / rows), (unsigned)((a.M + 15) / 16), (unsigned)a.count);
}

template <int FMT, bool OUT_F32, int U, int R, bool A_LDS, bool FULL, bool A_DMA, bool S_LDS>
hipError_t launch_k(const GroupedArgs& a, int rows, dim3 grid, dim3 block, unsigned lds) {
  if (a.count > 1)
    return launch_kernel(skinny_kernel<FMT, OUT_F32, U, R, A_LDS, FULL, S_LDS, A_DMA, true>, grid, block, lds,
                         a.stream, skinny_group<kMaxGroup>(a, rows), (int)a.M, (int)a.K, a.epi);
  return launch_kernel(skinny_kernel<FMT, OUT_F32, U, R, A_LDS, FULL, S_LDS, A_DMA, false>, grid, block, lds,
                       a.stream, skinny_group<1>(a, rows), (int)a.M, (int)a.K, a.epi);
}

// the private-staging route (PRIV): LDS = waves x this wave region
uint32_t skinny_priv_bytes(int64_t M, int UR, int sc) {
  const uint32_t am = (uint32_t)(M < 16 ? M : 16);
  return ((am + 1u) * (uint32_t)UR * 256u + 16u * (uint32_t)(UR * sc) * 3u + 15u) & ~15u;
}
template <int FMT, bool OUT_F32, int U, int R, bool FULL>
hipError_t launch_priv(const GroupedArgs& a, int rows, dim3 grid, dim3 block) {
  const unsigned lds = block.x / 64 * skinny_priv_bytes(a.M, U * R, is_int4(FMT) ? 1 : 4);
  if (a.count > 1)
    return launch_kernel(skinny_kernel<FMT, OUT_F32, U, R, false, FULL, false, false, true, true>, grid, block, lds,
                         a.stream, skinny_group<kMaxGroup>(a, rows), (int)a.M, (int)a.K, a.epi);
  return launch_kernel(skinny_kernel<FMT, OUT_F32, U, R, false, FULL, false, false, false, true>, grid, block, lds,
                       a.stream, skinny_group<1>(a, rows), (int)a.M, (int)a.K, a.epi);
}

template <int FMT, bool OUT_F32, int U, bool A_LDS, bool FULL, bool A_DMA, int R = 1>
hipError_t launch_s(const GroupedArgs& a, int rows, dim3 grid, dim3 block, bool s_lds,
                    unsigned lds_a, unsigned lds_s) {
  const unsigned lds_dma = A_DMA ? block.x / 64 * U * R * 4096u : 0u;
  if (s_lds)
    return launch_k<FMT, OUT_F32, U, R, A_LDS, FULL, A_DMA, true>(a, rows, grid, block, lds_a + lds_s + lds_dma);
  return launch_k<FMT, OUT_F32, U, R, A_LDS, FULL, A_DMA, false>(a, rows, grid, block, lds_a + lds_dma);
}

// Rows per workgroup: 16 unless fewer make the workgroup count fill whole
// rounds of 256 (one per CU) better -- e.g. N = 3072 gives 192 workgroups of
// 16 rows but 256 of 12.  Lanes of the missing rows read zeros.  A workgroup
// keeps >= 12 KB of weights (fewer rows would only add per-workgroup
// overhead).
int skinny_rows(const GroupedArgs& a) {
  int rows = 16;
  if (a.pre) return rows;  // the prepacked layout comes in tiles of 16 rows
  const int64_t r_min = (12288 + a.K / 2 - 1) / (a.K / 2);
  double best = -1.0;
  for (int r = 16; r >= (r_min > 4 ? (int)(r_min < 16 ? r_min : 16) : 4); --r) {
    int64_t wgs = 0;
    for (int i = 0; i < a.count; ++i) wgs += (a.N[i] + r - 1) / r;
    wgs *= (a.M + 15) / 16;
    const double fill = (double)wgs / (double)(256 * ((wgs + 255) / 256));
    if (fill > best + 0.02) {
      best = fill;
      rows = r;
    }
  }
  return rows;
}


template <int FMT, bool OUT_F32, int D, int R, bool FULL>
hipError_t launch_ring_k(const GroupedArgs& a, int rows, dim3 grid, unsigned lds) {
  const dim3 block(64 * (kRingVirt / R));
  if (a.count > 1)
    return launch_kernel(skinny_ring_kernel<FMT, OUT_F32, D, R, FULL, true>, grid, block, lds, a.stream,
                         skinny_group<kMaxGroup>(a, rows), (int)a.M, (int)a.K, a.epi);
  return launch_kernel(skinny_ring_kernel<FMT, OUT_F32, D, R, FULL, false>, grid, block, lds, a.stream,
                       skinny_group<1>(a, rows), (int)a.M, (int)a.K, a.epi);
}
template <int FMT, bool OUT_F32, int D, int R>
hipError_t launch_ring_f(const GroupedArgs& a, int rows, dim3 grid, unsigned lds) {
  return a.K % 128 == 0 ? launch_ring_k<FMT, OUT_F32, D, R, true>(a, rows, grid, lds)
                        : launch_ring_k<FMT, OUT_F32, D, R, false>(a, rows, grid, lds);
}

// The ring variant for A slices past the one-time LDS copy.  A grid of one
// round (<= 256 workgroups, one per CU): 8 waves with 3 slots each (120 KB of
// copies in flight per workgroup).  More rounds: 4 waves with 2 slots (40 KB
// plus the windows), so that several workgroups share a CU and the next
// round's copies overlap the current one's arithmetic (measured, e.g.
// 8 x 32000 x 4096 int4: 36.6 us with the per-pass kernel, 26.6 with 8 x 3
// slots, 23.7 with 4 x 2).  2 slots when the scale windows leave no room for
// 3; false when even that does not fit the 160 KB of LDS.
template <int FMT, bool OUT_F32>
bool try_ring(const GroupedArgs& a, hipError_t& err) {
  constexpr int SB = is_int4(FMT) ? 2 : 1;
  const int64_t groups = (a.K + FormatTraits<FMT>::kGroup - 1) / FormatTraits<FMT>::kGroup;
  const int64_t win = ring_window_cap((uint32_t)(16 * groups * SB)) +
                      (has_zeros(FMT) ? ring_window_cap((uint32_t)(16 * groups)) : 0);
  const int rows = skinny_rows(a);
  const dim3 grid = skinny_grid(a, rows);
  const bool one_round = (int64_t)grid.x * grid.y * grid.z <= 256;
  auto lds_of = [&](int w, int d) { return win + (int64_t)w * d * kRingSlot + (int64_t)kRingVirt * 1024; };
  constexpr int64_t kLds = 160 * 1024;
  if (!one_round && lds_of(4, 2) <= kLds) {
    err = launch_ring_f<FMT, OUT_F32, 2, 2>(a, rows, grid, (unsigned)lds_of(4, 2));
  } else if (lds_of(8, 3) <= kLds) {
    err = launch_ring_f<FMT, OUT_F32, 3, 1>(a, rows, grid, (unsigned)lds_of(8, 3));
  } else if (lds_of(8, 2) <= kLds) {
    err = launch_ring_f<FMT, OUT_F32, 2, 1>(a, rows, grid, (unsigned)lds_of(8, 2));
  } else {
    return false;
  }
  return true;
}

template <int FMT, bool OUT_F32, int U>
hipError_t launch_u(const GroupedArgs& a, int waves) {
  const int rows = skinny_rows(a);
  const dim3 grid = skinny_grid(a, rows);
  // int4 with groups of 128 and fp4, at most 8 A rows x k-blocks per wave:
  // private staging, no barrier before the arithmetic (same bits as the
  // A_LDS route); two virtual waves per wave as below when that still holds
  if constexpr (is_int4_g128(FMT) || !is_int4(FMT)) {
    const int64_t prow = a.M < 16 ? a.M : 16;
    if (prow * U <= 8) {
      const int KBp = (int)((a.K / 32 + 3) / 4);
      const int64_t wgs = (int64_t)grid.x * grid.y * grid.z;
      const bool full = a.K % 128 == 0;
      const bool halve = prow * U * 2 <= 8 && waves % 2 == 0 && waves * U >= KBp && wgs > 4 * (int64_t)device_cus();
      if (halve) {
        // int4 at M = 1 with 12 or 16 waves: four virtual waves per wave
        // (8 k-blocks of loads in flight per lane), measured on the decode
        // chain's K = 3072 launches
        if constexpr (U == 2 && is_int4_g128(FMT)) {
          if (prow * U * 4 <= 8 && waves % 4 == 0) {
            const dim3 quarter(64 * waves / 4);
            return full ? launch_priv<FMT, OUT_F32, U, 4, true>(a, rows, grid, quarter)
                        : launch_priv<FMT, OUT_F32, U, 4, false>(a, rows, grid, quarter);
          }
        }
        const dim3 half(64 * waves / 2);
        return full ? launch_priv<FMT, OUT_F32, U, 2, true>(a, rows, grid, half)
                    : launch_priv<FMT, OUT_F32, U, 2, false>(a, rows, grid, half);
      }
      const dim3 block(64 * waves);
      return full ? launch_priv<FMT, OUT_F32, U, 1, true>(a, rows, grid, block)
                  : launch_priv<FMT, OUT_F32, U, 1, false>(a, rows, grid, block);
    }
  }
  // stage A in LDS when the workgroup's A slice fits its staging registers
  const int64_t arows = a.M < 16 ? a.M : 16;
  const int64_t a_bytes = arows * a.K * 2;
  const bool a_lds = a_bytes <= (int64_t)kAStage * 16 * 64 * waves && a_bytes <= 64 * 1024;
  // LDS: A rows + a zero row (16-byte aligned), then the scale and zero windows
  const unsigned lds_a = a_lds ? (unsigned)(((arows + 1) * a.K * 2 + 15) & ~15) : 0u;
  constexpr int SB = is_int4(FMT) ? 2 : 1;
  const int64_t groups = (a.K + FormatTraits<FMT>::kGroup - 1) / FormatTraits<FMT>::kGroup;
  const int64_t s_cap = (16 * groups * SB + 6 + 15) & ~15;
  const int64_t z_cap = has_zeros(FMT) ? (16 * groups + 6 + 15) & ~15 : 0;
  const int64_t lds_s = s_cap + z_cap;
  // staged when every dword of the windows has a staging register (the zero
  // window exists for int4 only).  Exception, measured: a single fp4 row with
  // a window of 4 KB or more is one memory round trip per workgroup, and
  // per-lane scale loads that travel with the weights beat the staged copy
  // there (e.g. 3072 x 8192 NVFP4: 7.4 against 8.0 us).
  const int64_t threads = 64 * waves;
  const bool lane_scales = !is_int4(FMT) && a.M == 1 && 16 * groups * SB >= 4096;
  const bool s_lds = !lane_scales && (16 * groups * SB + 6) / 4 <= kSStage * threads &&
                     (!has_zeros(FMT) || (16 * groups + 6) / 4 <= kZStage * threads) && lds_s <= 32 * 1024;
  const bool full = a.K % 128 == 0;
  const dim3 block(64 * waves);
  const bool a_dma = !a_lds && waves * U * 4096 <= 128 * 1024;
  const unsigned ls = (unsigned)lds_s;
  // Two virtual waves per wave (same bits) when the launch has several
  // rounds of workgroups and K is covered in one pass: measured on the
  // decode chain's launches of thousands of workgroups, 404 -> 357 us per
  // pass; launches of one or two rounds keep the full wave count (the decode
  // GEMV's 512 workgroups: 5.7 us with it, 6.2 without).
  const int64_t wgs = (int64_t)grid.x * grid.y * grid.z;
  const int KB = (int)((a.K / 32 + 3) / 4);
  // (the staging loops cover kAStage / kSStage / kZStage items per thread:
  // A and the windows must still fit with half the threads)
  const int64_t half_threads = 32 * waves;
  const bool half_fits = a_bytes <= (int64_t)kAStage * 16 * half_threads &&
                         (!s_lds || ((16 * groups * SB + 6) / 4 <= kSStage * half_threads &&
                                     (!has_zeros(FMT) || (16 * groups + 6) / 4 <= kZStage * half_threads)));
  const bool halve = a_lds && half_fits && waves % 2 == 0 && waves * U >= KB &&
                     wgs > 4 * (int64_t)device_cus();
  if (halve) {
    const dim3 half(block.x / 2);
    if (full) return launch_s<FMT, OUT_F32, U, true, true, false, 2>(a, rows, grid, half, s_lds, lds_a, ls);
    return launch_s<FMT, OUT_F32, U, true, false, false, 2>(a, rows, grid, half, s_lds, lds_a, ls);
  }
  if (a_lds && full) return launch_s<FMT, OUT_F32, U, true, true, false>(a, rows, grid, block, s_lds, lds_a, ls);
  if (a_lds) return launch_s<FMT, OUT_F32, U, true, false, false>(a, rows, grid, block, s_lds, lds_a, ls);
  if (a_dma && full) return launch_s<FMT, OUT_F32, U, false, true, true>(a, rows, grid, block, s_lds, lds_a, ls);
  if (a_dma) return launch_s<FMT, OUT_F32, U, false, false, true>(a, rows, grid, block, s_lds, lds_a, ls);
  if (full) return launch_s<FMT, OUT_F32, U, false, true, false>(a, rows, grid, block, s_lds, lds_a, ls);
  return launch_s<FMT, OUT_F32, U, false, false, false>(a, rows, grid, block, s_lds, lds_a, ls);
}

// k-blocks of 128 per wave: 2 while K fits 16 waves that way, else 4.  The
// split sets the summation order, so every kernel for few rows uses it.
int skinny_split_u(int KB) { return (KB + 1) / 2 <= kMaxWaves ? 2 : 4; }

// compute units of the current device, cached per device (threads that race
// on a first call store the same value; the slots are atomic)
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// resident workgroups per compute unit of a kernel at a block size and
// dynamic LDS size (cached; occupancy does not depend on the device here)
int resident_per_cu(const void* kernel, int threads, unsigned lds) {
  static std::mutex mu;
  static std::map<std::tuple<const void*, int, unsigned>, int> cache;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_tuple(kernel, threads, lds);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, lds) != hipSuccess || n < 1) n = 1;
  cache.emplace(key, n);
  return n;
}

template <int FMT, bool OUT_F32, int U, int NS>
hipError_t launch_stream_k(const GroupedArgs& a, const SkinnyGroup<1>& grp, int tiles, int waves, unsigned lds) {
  const void* kern = reinterpret_cast<const void*>(&skinny_stream_kernel<FMT, OUT_F32, U, NS>);
  const int resident = resident_per_cu(kern, 64 * waves, lds) * device_cus();
  const dim3 grid((unsigned)(tiles < resident ? tiles : resident));
  const dim3 block(64 * waves);
  return launch_kernel(skinny_stream_kernel<FMT, OUT_F32, U, NS>, grid, block, lds, a.stream, grp,
                       (int)a.M, (int)a.K, tiles, a.epi);
}

// The streaming kernel when its conditions hold and the launch (one weight
// matrix) has at least `min_tiles` tiles of 16 columns; returns false
// (nothing launched) otherwise.
template <int FMT, bool OUT_F32>
bool try_stream(const GroupedArgs& a, int64_t min_tiles, hipError_t& err) {
  if constexpr (FMT == kInt4G32 || FMT == kInt4G64) {
    return false;  // the streaming variant decodes int4 with groups of 128 only
  } else {
  if (a.count != 1 || a.K % 128 != 0 || a.M > 16) return false;
  const int KB = (int)(a.K / 128);
  // the one-tile kernel's split of K (a column's bits never depend on N or
  // on the grouping)
  const int U = skinny_split_u(KB);
  const int waves = (KB + U - 1) / U;
  if (waves > kMaxWaves) return false;
  const int64_t threads = 64 * waves;
  const int64_t a16 = a.M * a.K / 8;
  if (a16 > kAStage * threads || a.M * a.K * 2 > 64 * 1024) return false;
  constexpr int SB = is_int4_g128(FMT) ? 2 : 1;
  const int64_t groups = (a.K + FormatTraits<FMT>::kGroup - 1) / FormatTraits<FMT>::kGroup;
  const int64_t s_words = (16 * groups * SB + 6) / 4, z_words = (16 * groups + 6) / 4;
  const int NS = s_words <= threads ? 1 : (s_words <= 2 * threads ? 2 : 0);
  if (NS == 0 || (FMT == kInt4 && z_words > threads)) return false;
  const int64_t tiles = (a.N[0] + 15) / 16;
  if (tiles < min_tiles || tiles < 1) return false;
  const SkinnyGroup<1> grp = skinny_group<1>(a, 16);
  const int64_t s_cap = (16 * groups * SB + 6 + 15) & ~15;
  const int64_t z_cap = FMT == kInt4 ? (16 * groups + 6 + 15) & ~15 : 0;
  const unsigned lds = (unsigned)((((a.M + 1) * a.K * 2 + 15) & ~15) + 3 * (s_cap + z_cap) + 3 * threads * 16);
  if (U == 4)
    err = NS == 1 ? launch_stream_k<FMT, OUT_F32, 4, 1>(a, grp, (int)tiles, waves, lds)
                  : launch_stream_k<FMT, OUT_F32, 4, 2>(a, grp, (int)tiles, waves, lds);
  else if (U == 2)
    err = NS == 1 ? launch_stream_k<FMT, OUT_F32, 2, 1>(a, grp, (int)tiles, waves, lds)
                  : launch_stream_k<FMT, OUT_F32, 2, 2>(a, grp, (int)tiles, waves, lds);
  else
    err = NS == 1 ? launch_stream_k<FMT, OUT_F32, 1, 1>(a, grp, (int)tiles, waves, lds)
                  : launch_stream_k<FMT, OUT_F32, 1, 2>(a, grp, (int)tiles, waves, lds);
  return true;
  }
}

// Work split: each wave takes U consecutive k-blocks per pass (U 16-byte
// weight loads in flight per lane), and the workgroup has enough waves
// (at most 16) to cover K in one pass when it can.  The streaming variant
// serves single matrices of 1024 tiles of 16 columns or more.
template <int FMT, bool OUT_F32>
hipError_t launch_fmt(const GroupedArgs& a) {
  {
    hipError_t err = hipSuccess;
    if (try_stream<FMT, OUT_F32>(a, 1024, err)) return err;
  }
  const int chunks = (int)(a.K >> 5);
  const int KB = (chunks + 3) >> 2;
  int U = skinny_split_u(KB);
  int waves = (KB + U - 1) / U;
  if (waves > kMaxWaves) waves = kMaxWaves;
  if (waves < 1) waves = 1;
  // A rows that do not fit the LDS copy go through per-wave LDS regions of
  // U k-blocks (4 KB each): keep those within 128 KB
  const int64_t arows = a.M < 16 ? a.M : 16;
  const bool a_big = arows * a.K * 2 > (int64_t)kAStage * 16 * 64 * waves || arows * a.K * 2 > 64 * 1024;
  if (a_big) {
    hipError_t err = hipSuccess;
    if (try_ring<FMT, OUT_F32>(a, err)) return err;
  }
  if (a_big && waves * U > 32) U = 32 / waves > 0 ? 32 / waves : 1;
  if (U == 1) return launch_u<FMT, OUT_F32, 1>(a, waves);
  if (U == 2) return launch_u<FMT, OUT_F32, 2>(a, waves);
  return launch_u<FMT, OUT_F32, 4>(a, waves);
}

}  // namespace

hipError_t launch_skinny_grouped(const GroupedArgs& a) {
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

hipError_t launch_skinny(const GemmArgs& a) {
  GroupedArgs g = {};
  g.fmt = a.fmt;
  g.out_f32 = a.out_f32;
  g.pre = a.pre;
  g.A[0] = a.A;
  g.count = 1;
  g.packed[0] = a.packed;
  g.scales[0] = a.scales;
  g.zeros[0] = a.zeros;
  g.C[0] = a.C;
  g.N[0] = a.N;
  g.M = a.M;
  g.K = a.K;
  g.stream = a.stream;
  g.epi = a.epi;
  return launch_skinny_grouped(g);
}

}  // namespace w4a16
