// mid.hip -- W4A16 GEMM for a middle number of activation rows (about 16 < M
// <= 192): tiles of 32 output columns x 16*MS rows (MS = 2, 3 or 4).
//
// At decode-batch sizes the tiled kernel's 256 x 256 tiles leave most CUs idle
// (N / 256 of them) and spend their MFMA work on padding rows, while the
// skinny kernel handles 16 rows at a time and so loads and decodes every
// weight once per 16-row slice.  Here a workgroup covers 32 weight rows (two
// 16-column slices) and MS 16-row slices of A: each weight is loaded and
// decoded once and feeds MS MFMA chains.  The waves split K (U 128-code
// k-blocks per wave and pass) and meet in LDS for a fixed-order sum.
//
//   * weights: lane l owns row 16h + l%16 of column slice h (h = 0, 1) and
//     chunk l/16 (32 codes) of each k-block: one 16-byte load per lane, slice
//     and k-block, the same operand layout as the skinny kernel;
//   * A: the lane supplies row 16s + l%16 of row slice s over the same 32 k,
//     loaded straight from memory (A is small and read once per workgroup, so
//     it is served from L2);
//   * int4 with groups of 128: code - zero, exact in bf16, is formed per
//     weight before the MFMA and the group scale multiplies once per k-block
//     (groups of 32 / 64: the exact weight as bf16 hi + lo fragments); fp4:
//     the scale is applied exactly in the decode;
//   * scales (and zeros) of the workgroup's 32 rows are one contiguous block:
//     copied once to LDS with coalesced dword loads when it fits the staging
//     registers (S_LDS), else each lane loads its own with its weights.
// That is the per-lane form.  The ring variant below (used whenever its LDS
// fits) keeps the tile and the operand layouts but moves every operand by
// global -> LDS copies.
#include "common.hpp"
#include "kernels.hpp"

namespace w4a16 {

namespace {

constexpr int kMidMaxWaves = 12;
constexpr int kMidCols = 32;   // output columns (weight rows) per workgroup
constexpr int kMidSStage = 4;  // staged scale / zero dwords per thread, at most

template <int FMT>
constexpr int mid_sb() { return is_int4(FMT) ? 2 : 1; }  // scale bytes

// scale (zero) window capacity in bytes: 32 rows plus the <= 3-byte lead of
// the dword-aligned start and the <= 3-byte tail of its last dword
__host__ __device__ constexpr uint32_t mid_cap(uint32_t bytes) { return (bytes + 6u + 15u) & ~15u; }

// The split-K sum and the stores of one workgroup: output block p = (row
// slice s, column slice h) is the sum of red[(w * P + p) * 64 + lane] over the
// waves w in order, stored (through the fused epilogue when on) by wave
// p % waves.  Lane (nl, g) holds rows 16s + 4g .. 16s + 4g + 3 of column
// 16h + nl; rows bounds the workgroup's columns.
template <bool OUT_F32, int MS>
__device__ __forceinline__ void mid_store(const f32x4_t* red, int wave, int waves, int lane, int nl, int g,
                                          int n0, int m0, int rows, int M, int N, void* C,
                                          const Epilogue& epi) {
  constexpr int P = MS * 2;
  for (int p = wave; p < P; p += waves) {
    const int s = p >> 1, h = p & 1;
    const int n = n0 + 16 * h + nl;
    const bool col_ok = 16 * h + nl < rows;
    // epilogue operands first, in one round trip (the residual may alias C)
    float eb = 0.f, er[4] = {0.f, 0.f, 0.f, 0.f};
    if (epi.on && col_ok) {
      if (epi.bias) eb = bf16_bits_to_f32(epi.bias[n]);
      if (epi.res) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + 16 * s + 4 * g + i;
          if (m < M) er[i] = residual_at<OUT_F32>(epi.res, (int64_t)m * N + n);
        }
      }
    }
    f32x4_t sum = red[p * 64 + lane];
    for (int w = 1; w < waves; ++w) {
      const f32x4_t v = red[(w * P + p) * 64 + lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) sum[i] += v[i];
    }
    if (!col_ok) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + 16 * s + 4 * g + i;
      if (m < M) {
        const int64_t mn = (int64_t)m * N + n;
        const float v = epi.on ? epilogue_value(epi, sum[i], eb, er[i]) : sum[i];
        if constexpr (OUT_F32) {
          reinterpret_cast<float*>(C)[mn] = v;
        } else {
          reinterpret_cast<__bf16*>(C)[mn] = (__bf16)v;
        }
      }
    }
  }
}

template <int FMT, bool OUT_F32, int U, int MS, bool S_LDS>
__global__ __launch_bounds__(64 * kMidMaxWaves) void mid_kernel(const uint16_t* __restrict__ A,
                                                               const uint8_t* __restrict__ packed,
                                                               const void* __restrict__ scales,
                                                               const uint8_t* __restrict__ zeros,
                                                               void* __restrict__ C, int M, int N, int K,
                                                               int pre, Epilogue epi) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int waves = blockDim.x >> 6;
  const int nl = lane & 15;
  const int g = lane >> 4;
  const int n0 = (int)blockIdx.x * kMidCols;
  const int m0 = (int)blockIdx.y * 16 * MS;
  const int KC = K >> 5;          // 32-code chunks (K % 32 == 0)
  const int KB = (KC + 3) >> 2;   // k-blocks, the last one possibly partial
  constexpr int G = FormatTraits<FMT>::kGroup;
  constexpr int SB = mid_sb<FMT>();
  // int4: the group of 32-code chunk c is c >> GS (the k-block for G = 128)
  constexpr int GS = G == 128 ? 2 : (G == 64 ? 1 : 0);
  const int groups = (K + G - 1) / G;  // the last group may be shorter
  const uint32_t rowb = (uint32_t)(K >> 1);
  const int rows = min(kMidCols, N - n0);
  const int arows = min(16 * MS, M - m0);
  const uint32_t wave_slot0 = (uint32_t)__builtin_amdgcn_readfirstlane(wave) * 64u;
  const int kw = __builtin_amdgcn_readfirstlane(wave) * U;

  const uint32_t s_cap = S_LDS ? mid_cap((uint32_t)(kMidCols * groups * SB)) : 0u;
  const uint32_t z_cap = S_LDS && has_zeros(FMT) ? mid_cap((uint32_t)(kMidCols * groups)) : 0u;
  f32x4_t* red = reinterpret_cast<f32x4_t*>(lds + s_cap + z_cap);  // [waves][MS * 2][64]

  const uint8_t* s_base = reinterpret_cast<const uint8_t*>(scales) + (int64_t)n0 * groups * SB;
  const uint8_t* z_base = has_zeros(FMT) ? zeros + (int64_t)n0 * groups : nullptr;
  // S_LDS: the windows' dwords, read from the 4-byte aligned address at or
  // below each block (at most 3 bytes past its end, in the same dword)
  uint32_t s_delta = 0, z_delta = 0, s_words = 0, z_words = 0;
  uint32_t sst[kMidSStage], zst[kMidSStage];
  // direct: per-lane scale / zero loads over the same blocks
  rsrc_t sr, zr;
  if constexpr (S_LDS) {
    auto window = [&](const uint8_t* start, uint32_t bytes, uint32_t& delta, uint32_t& words) {
      const uintptr_t al = reinterpret_cast<uintptr_t>(start) & ~(uintptr_t)3;
      delta = (uint32_t)(reinterpret_cast<uintptr_t>(start) - al);
      words = (delta + bytes + 3u) / 4u;
      return make_rsrc(reinterpret_cast<const void*>(al), words * 4u);
    };
    const rsrc_t ss = window(s_base, (uint32_t)(rows * groups * SB), s_delta, s_words);
#pragma unroll
    for (int i = 0; i < kMidSStage; ++i) {
      const uint32_t w = (uint32_t)(tid + i * (int)blockDim.x);
      sst[i] = wave_slot0 + i * blockDim.x < s_words ? buf_load_b32(ss, w < s_words ? w * 4u : kBufferOOB) : 0u;
    }
    if constexpr (has_zeros(FMT)) {
      const rsrc_t zs = window(z_base, (uint32_t)(rows * groups), z_delta, z_words);
#pragma unroll
      for (int i = 0; i < kMidSStage; ++i) {
        const uint32_t w = (uint32_t)(tid + i * (int)blockDim.x);
        zst[i] = wave_slot0 + i * blockDim.x < z_words ? buf_load_b32(zs, w < z_words ? w * 4u : kBufferOOB) : 0u;
      }
    }
  } else {
    sr = make_rsrc(s_base, (uint32_t)(rows * groups * SB));
    if constexpr (has_zeros(FMT)) zr = make_rsrc(z_base, (uint32_t)(rows * groups));
  }

  // weight rows past N, A rows past M and chunks past K read as 0 (the
  // prepacked layout's tiles of 16 rows end in zero bytes past N)
  const rsrc_t wr = make_rsrc(packed + (int64_t)n0 * rowb, (uint32_t)(pre ? (rows + 15) & ~15 : rows) * rowb);
  const rsrc_t ar = make_rsrc(A + (int64_t)m0 * K, (uint32_t)arows * (uint32_t)K * 2u);

  f32x4_t acc[MS][2];
#pragma unroll
  for (int s = 0; s < MS; ++s) acc[s][0] = acc[s][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  u32x4_t q[U][2];
  uint32_t sraw[U][2], zraw[U][2];

  // weights (and, direct, their scales) of one pass, issued together; every
  // load is issued (out of range past K), so no branch splits the waits
  auto issue = [&](int kbase) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = kbase + u;
      const int c = kb * 4 + g;
      const bool ok = c < KC;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t r = (uint32_t)(16 * h + nl);
        q[u][h] = buf_load_b128(wr, ok ? wchunk(r, (uint32_t)c, rowb, pre != 0) : kBufferOOB);
        if constexpr (!S_LDS) {
          if constexpr (is_int4(FMT)) {
            // groups of 128: the k-block's group for every chunk, also past
            // K (the MFMA sums the four chunks before the scale is applied)
            const uint32_t gi = r * (uint32_t)groups + (uint32_t)(is_int4_g128(FMT) ? kb : c >> GS);
            const bool sok = is_int4_g128(FMT) ? kb < KB : ok;
            sraw[u][h] = buf_load_b16(sr, sok ? gi * 2u : kBufferOOB);
            zraw[u][h] = has_zeros(FMT) ? buf_load_b8(zr, sok ? gi : kBufferOOB) : kSymZero;
          } else if constexpr (FMT == kNvfp4) {
            sraw[u][h] = buf_load_b16(sr, ok ? r * (uint32_t)groups + 2u * (uint32_t)c : kBufferOOB);
          } else {
            sraw[u][h] = buf_load_b8(sr, ok ? r * (uint32_t)groups + (uint32_t)c : kBufferOOB);
          }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  const uint8_t* sb = lds + s_delta;
  const uint8_t* zb = lds + s_cap + z_delta;
  auto compute = [&](int kbase) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = kbase + u;
      if (kb >= KB) break;  // wave-uniform
      const int c = kb * 4 + g;
      const bool ok = c < KC;
      const int cc = ok ? c : 0;  // LDS reads stay inside the window
      // both column slices decoded once, to bf16 MFMA operands (int4 with
      // groups of 32 / 64: the exact weights as hi + lo fragments)
      u32x4_t b[2][4], bl[2][4];
      float sc[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 16 * h + nl;
        if constexpr (is_int4_g128(FMT)) {
          const int gi = r * groups + kb;
          uint32_t sbits, z;
          if constexpr (S_LDS) {
            sbits = *reinterpret_cast<const uint16_t*>(sb + 2 * gi);
            z = has_zeros(FMT) ? (uint32_t)zb[gi] : kSymZero;
          } else {
            sbits = sraw[u][h];
            z = zraw[u][h];
          }
          sc[h] = bf16_bits_to_f32(sbits);
#pragma unroll
          for (int j = 0; j < 4; ++j) b[h][j] = int4x8_minus_zero(q[u][h][j], (float)z);
        } else if constexpr (is_int4(FMT)) {
          // groups shorter than a k-block: the chunk's group, applied in the
          // decode, the exact weight (code - zero) * scale as hi + lo
          const int gi = r * groups + (cc >> GS);
          uint32_t sbits, z;
          if constexpr (S_LDS) {
            sbits = *reinterpret_cast<const uint16_t*>(sb + 2 * gi);
            z = zb[gi];
          } else {
            sbits = sraw[u][h];
            z = zraw[u][h];
          }
          const float s = bf16_bits_to_f32(sbits), zf = (float)z;
#pragma unroll
          for (int j = 0; j < 4; ++j) int4x8_to_bf16_hilo(q[u][h][j], s, zf, b[h][j], bl[h][j]);
        } else if constexpr (FMT == kNvfp4) {
          const uint32_t s2 = S_LDS ? *reinterpret_cast<const uint16_t*>(sb + r * groups + 2 * cc) : sraw[u][h];
          const float s0 = e4m3_magnitude(s2 & 0xFFu), s1 = e4m3_magnitude(s2 >> 8);
          b[h][0] = fp4x8_to_bf16_fscale(q[u][h][0], s0);
          b[h][1] = fp4x8_to_bf16_fscale(q[u][h][1], s0);
          b[h][2] = fp4x8_to_bf16_fscale(q[u][h][2], s1);
          b[h][3] = fp4x8_to_bf16_fscale(q[u][h][3], s1);
        } else {
          const float es = e8m0_as_exponent_scale(S_LDS ? (uint32_t)sb[r * groups + cc] : sraw[u][h]);
#pragma unroll
          for (int j = 0; j < 4; ++j) b[h][j] = fp4x8_to_bf16_escale(q[u][h][j], es);
        }
      }
      // every row slice of A meets both decoded column slices
#pragma unroll
      for (int s = 0; s < MS; ++s) {
        const uint32_t off = ((uint32_t)(16 * s + nl) * (uint32_t)K + (uint32_t)c * 32u) * 2u;
        u32x4_t a[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) a[j] = buf_load_b128(ar, ok ? off + 16u * j : kBufferOOB);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if constexpr (is_int4_g128(FMT)) {
            f32x4_t dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) dp = mfma16x16x32(a[j], b[h][j], dp);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[s][h][i] = __builtin_fmaf(sc[h], dp[i], acc[s][h][i]);
          } else if constexpr (is_int4(FMT)) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              acc[s][h] = mfma16x16x32(a[j], b[h][j], acc[s][h]);
              acc[s][h] = mfma16x16x32(a[j], bl[h][j], acc[s][h]);
            }
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[s][h] = mfma16x16x32(a[j], b[h][j], acc[s][h]);
          }
        }
      }
    }
  };

  int kbase = kw;
  issue(kbase);
  if constexpr (S_LDS) {
    // scales to LDS; an LDS-only barrier leaves the weights in flight
#pragma unroll
    for (int i = 0; i < kMidSStage; ++i) {
      const uint32_t w = (uint32_t)(tid + i * (int)blockDim.x);
      if (w < s_words) reinterpret_cast<uint32_t*>(lds)[w] = sst[i];
      if constexpr (has_zeros(FMT)) {
        if (w < z_words) reinterpret_cast<uint32_t*>(lds + s_cap)[w] = zst[i];
      }
    }
    lds_barrier();
  }
  compute(kbase);
  for (kbase += waves * U; kbase < KB; kbase += waves * U) {
    issue(kbase);
    compute(kbase);
  }

  // ---- split-K sum over the waves through LDS ----
  constexpr int P = MS * 2;
#pragma unroll
  for (int s = 0; s < MS; ++s)
#pragma unroll
    for (int h = 0; h < 2; ++h) red[(wave * P + s * 2 + h) * 64 + lane] = acc[s][h];
  lds_barrier();
  mid_store<OUT_F32, MS>(red, wave, waves, lane, nl, g, n0, m0, rows, M, N, C, epi);
}

// ---- ring variant -----------------------------------------------------------
//
// The same tile (32 columns x 16 MS rows) and decode, with every operand
// moved by asynchronous global -> LDS copies: k-block kb's A rows (16 MS x
// 256 bytes, chunk c of row r in slot c ^ (r & 15) so that the fragment reads
// of 16 rows hit distinct banks) and weight rows (32 x 64 bytes) fill one of
// the wave's D ring slots, refilled D k-blocks ahead; the scale (and zero)
// window arrives the same way, once.  kMidRingWaves waves split K, wave w
// taking k-blocks w, w + W, ...; no operand goes through a load the compiler
// sees, so every wait is an explicit count of the copies issued after the
// one needed (vmcnt retires in issue order).  The per-lane A loads of the
// other form leave each CU reading A at about half the rate its memory
// pipeline sustains; here copies of D - 1 k-blocks stay in flight while one
// is computed.  The partial sums reuse the ring's LDS once every wave is done.
constexpr int kMidRingWaves = 4;

__host__ __device__ constexpr uint32_t mid_ring_slot(int ms) { return (uint32_t)ms * 4096u + 2048u; }
__host__ __device__ constexpr uint32_t mid_ring_window(uint32_t bytes) { return (bytes + 6u + 255u) / 256u * 256u; }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int FMT, bool OUT_F32, int MS, int D, bool FULL>
__global__ __launch_bounds__(64 * kMidRingWaves) void mid_ring_kernel(const uint16_t* __restrict__ A,
                                                                    const uint8_t* __restrict__ packed,
                                                                    const void* __restrict__ scales,
                                                                    const uint8_t* __restrict__ zeros,
                                                                    void* __restrict__ C, int M, int N, int K,
                                                                    int pre, Epilogue epi) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int W = kMidRingWaves;
  constexpr int CPK = 4 * MS + 2;  // copies per k-block
  static_assert((D - 1) * CPK <= 63, "vmcnt");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nl = lane & 15;
  const int g = lane >> 4;
  const int n0 = (int)blockIdx.x * kMidCols;
  const int m0 = (int)blockIdx.y * 16 * MS;
  const int KC = K >> 5;
  const int KB = (KC + 3) >> 2;
  constexpr int G = FormatTraits<FMT>::kGroup;
  constexpr int SB = mid_sb<FMT>();
  constexpr int GS = G == 128 ? 2 : (G == 64 ? 1 : 0);
  const int groups = (K + G - 1) / G;  // the last group may be shorter
  const uint32_t rowb = (uint32_t)(K >> 1);
  const int rows = min(kMidCols, N - n0);
  const int arows = min(16 * MS, M - m0);

  const rsrc_t wr = make_rsrc(packed + (int64_t)n0 * rowb, (uint32_t)(pre ? (rows + 15) & ~15 : rows) * rowb);
  const rsrc_t ar = make_rsrc(A + (int64_t)m0 * K, (uint32_t)arows * (uint32_t)K * 2u);
  const uint32_t s_cap = mid_ring_window((uint32_t)(kMidCols * groups * SB));
  const uint32_t z_cap = has_zeros(FMT) ? mid_ring_window((uint32_t)(kMidCols * groups)) : 0u;
  const uint32_t base = lds_address(lds);
  const uint32_t ring0 = s_cap + z_cap;
  const uint32_t my_ring = ring0 + (uint32_t)wave * (uint32_t)(D * mid_ring_slot(MS));

  // window copies: dwords from the 4-byte aligned address at or below the
  // block's start (delta bytes before it), 64 per copy, the waves in turn
  auto window = [&](const uint8_t* start, uint32_t bytes, uint32_t lds_off) {
    const uintptr_t al = reinterpret_cast<uintptr_t>(start) & ~(uintptr_t)3;
    const uint32_t delta = (uint32_t)(reinterpret_cast<uintptr_t>(start) - al);
    const uint32_t words = (delta + bytes + 3u) / 4u;  // may read <= 3 bytes past the block (same page)
    const rsrc_t r = make_rsrc(reinterpret_cast<const void*>(al), words * 4u);
    const int instrs = (int)((words + 63u) / 64u);
    for (int t = wave; t < instrs; t += W)
      lds_dma_b32(r, base + lds_off + (uint32_t)t * 256u, ((uint32_t)t * 64u + (uint32_t)lane) * 4u);
    return delta;
  };
  const uint32_t s_delta = window(reinterpret_cast<const uint8_t*>(scales) + (int64_t)n0 * groups * SB,
                                  (uint32_t)(rows * groups * SB), 0u);
  uint32_t z_delta = 0;
  if constexpr (has_zeros(FMT)) z_delta = window(zeros + (int64_t)n0 * groups, (uint32_t)(rows * groups), s_cap);

  const int nk = wave < KB ? (KB - 1 - wave) / W + 1 : 0;
  // k-block i -> slot i % D: A copy r4 moves rows 4 r4 .. 4 r4 + 3 (lane ->
  // row 4 r4 + l/16, LDS chunk l%16 holding chunk (l%16) ^ (row & 15));
  // weight copy t moves rows 16t .. 16t + 15 (lane -> row 16t + l/4, chunk l%4)
  auto issue = [&](int i) {
    const int kb = i * W + wave;
    const uint32_t slot = base + my_ring + (uint32_t)(i % D) * mid_ring_slot(MS);
#pragma unroll
    for (int r4 = 0; r4 < 4 * MS; ++r4) {
      const int r = 4 * r4 + (lane >> 4);
      const int ch = (lane & 15) ^ (r & 15);
      const bool ok = FULL || kb * 128 + 8 * ch < K;
      lds_dma_b128(ar, slot + (uint32_t)r4 * 1024u,
                   ok ? ((uint32_t)r * (uint32_t)K + (uint32_t)kb * 128u + 8u * (uint32_t)ch) * 2u : kBufferOOB);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      // (prepacked: lane -> row 16t + l%16, chunk l/16: one contiguous kilobyte)
      const int wrow = 16 * t + (pre ? (lane & 15) : (lane >> 2)), wch = pre ? (lane >> 4) : (lane & 3);
      const bool okw = FULL || kb * 4 + wch < KC;
      lds_dma_b128(wr, slot + (uint32_t)MS * 4096u + (uint32_t)t * 1024u,
                   okw ? wchunk((uint32_t)wrow, (uint32_t)(kb * 4 + wch), rowb, pre != 0) : kBufferOOB);
    }
  };
  auto ring_wait = [&](int later) {
    if (D > 2 && later >= 2) {
      wait_vmcnt<(D > 2 ? 2 * CPK : 0)>();
    } else if (later >= 1) {
      wait_vmcnt<CPK>();
    } else {
      wait_vmcnt<0>();
    }
  };
  const int first = nk < D ? nk : D;
  for (int i = 0; i < first; ++i) issue(i);
  // the windows (issued first) and k-block 0 have landed in this wave's part;
  // after the barrier every wave's part has
  ring_wait(first - 1);
  lds_barrier();

  f32x4_t acc[MS][2];
#pragma unroll
  for (int s = 0; s < MS; ++s) acc[s][0] = acc[s][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint8_t* sb = lds + s_delta;
  const uint8_t* zb = lds + s_cap + z_delta;
  for (int i = 0; i < nk; ++i) {
    if (i > 0) ring_wait(min(D - 1, nk - 1 - i));
    const int kb = i * W + wave;
    const int c = kb * 4 + g;
    const bool ok = FULL || c < KC;
    const int cc = ok ? c : 0;  // window reads stay inside it
    const uint8_t* slot = lds + my_ring + (uint32_t)(i % D) * mid_ring_slot(MS);
    // both column slices decoded once, to bf16 MFMA operands.  int4 with
    // groups of 128: code - zero, exact in bf16 (an integer in -255 .. 15),
    // one MFMA chain, the scale once per k-block (a k-block whose codes all
    // equal the zero point contributes exactly 0)
    // (int4 with groups of 32 / 64: the exact weights as hi + lo fragments)
    u32x4_t b[2][4], bl[2][4];
    float sc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 16 * h + nl;
      const u32x4_t q = *reinterpret_cast<const u32x4_t*>(
          slot + MS * 4096 + h * 1024 + (pre ? nl + 16 * g : nl * 4 + g) * 16);
      if constexpr (is_int4_g128(FMT)) {
        const int gi = r * groups + kb;
        sc[h] = bf16_bits_to_f32(*reinterpret_cast<const uint16_t*>(sb + 2 * gi));
        const float zf = (float)(has_zeros(FMT) ? (uint32_t)zb[gi] : kSymZero);
#pragma unroll
        for (int j = 0; j < 4; ++j) b[h][j] = int4x8_minus_zero(q[j], zf);
      } else if constexpr (is_int4(FMT)) {
        const int gi = r * groups + (cc >> GS);
        const float sv = bf16_bits_to_f32(*reinterpret_cast<const uint16_t*>(sb + 2 * gi));
        const float zf = (float)zb[gi];
#pragma unroll
        for (int j = 0; j < 4; ++j) int4x8_to_bf16_hilo(q[j], sv, zf, b[h][j], bl[h][j]);
      } else if constexpr (FMT == kNvfp4) {
        const uint32_t s2 = *reinterpret_cast<const uint16_t*>(sb + r * groups + 2 * cc);
        const float s0 = e4m3_magnitude(s2 & 0xFFu), s1 = e4m3_magnitude(s2 >> 8);
        b[h][0] = fp4x8_to_bf16_fscale(q[0], s0);
        b[h][1] = fp4x8_to_bf16_fscale(q[1], s0);
        b[h][2] = fp4x8_to_bf16_fscale(q[2], s1);
        b[h][3] = fp4x8_to_bf16_fscale(q[3], s1);
      } else {
        const float es = e8m0_as_exponent_scale((uint32_t)sb[r * groups + cc]);
#pragma unroll
        for (int j = 0; j < 4; ++j) b[h][j] = fp4x8_to_bf16_escale(q[j], es);
      }
    }
    // every row slice of A meets both decoded column slices
#pragma unroll
    for (int s = 0; s < MS; ++s) {
      u32x4_t a[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        a[j] = *reinterpret_cast<const u32x4_t*>(slot + (16 * s + nl) * 256 + (((4 * g + j) ^ nl) * 16));
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if constexpr (is_int4_g128(FMT)) {
          f32x4_t dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < 4; ++j) dp = mfma16x16x32(a[j], b[h][j], dp);
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[s][h][t] = __builtin_fmaf(sc[h], dp[t], acc[s][h][t]);
        } else if constexpr (is_int4(FMT)) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[s][h] = mfma16x16x32(a[j], b[h][j], acc[s][h]);
            acc[s][h] = mfma16x16x32(a[j], bl[h][j], acc[s][h]);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[s][h] = mfma16x16x32(a[j], b[h][j], acc[s][h]);
        }
      }
    }
    if (i + D < nk) {
      // the slot's reads have completed before its next copy is issued
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue(i + D);
    }
  }

  // ---- split-K sum: the partial sums take the ring's place once every wave
  // is past its last k-block (its copies all waited for) ----
  constexpr int P = MS * 2;
  f32x4_t* red = reinterpret_cast<f32x4_t*>(lds + ring0);
  lds_barrier();
#pragma unroll
  for (int s = 0; s < MS; ++s)
#pragma unroll
    for (int h = 0; h < 2; ++h) red[(wave * P + s * 2 + h) * 64 + lane] = acc[s][h];
  lds_barrier();
  mid_store<OUT_F32, MS>(red, wave, W, lane, nl, g, n0, m0, rows, M, N, C, epi);
}

// launch shape of one call: k-blocks per wave and pass, waves, row slices
struct MidPlan {
  int U, waves, MS;
  bool s_lds;
  unsigned lds;
};

MidPlan mid_plan(int fmt, int64_t M, int64_t K) {
  MidPlan p;
  const int KB = (int)((K / 32 + 3) / 4);
  // 2 k-blocks per wave while K fits the waves that way, else 4; passes over
  // K balanced so every wave gets the same number of k-blocks, within one
  p.U = (KB + 1) / 2 <= kMidMaxWaves ? 2 : 4;
  const int per_pass = kMidMaxWaves * p.U;
  const int passes = (KB + per_pass - 1) / per_pass;
  p.waves = (KB + p.U * passes - 1) / (p.U * passes);
  // rows: as few 64-row tiles as cover M, then as few 16-row slices per tile
  const int64_t slices = (M + 15) / 16;
  const int64_t row_tiles = (slices + 3) / 4;
  p.MS = (int)((slices + row_tiles - 1) / row_tiles);
  if (p.MS < 2) p.MS = 2;
  // scale windows in LDS when every dword has a staging register
  const bool int4 = is_int4(fmt);
  const int64_t G = is_int4_g128(fmt) ? 128 : fmt == kNvfp4 ? 16 : fmt == kInt4G64 ? 64 : 32;
  const int64_t groups = (K + G - 1) / G;
  const int64_t sb = int4 ? 2 : 1;
  const int64_t slots = (int64_t)kMidSStage * 64 * p.waves;
  const int64_t s_cap = mid_cap((uint32_t)(kMidCols * groups * sb));
  const int64_t z_cap = has_zeros(fmt) ? mid_cap((uint32_t)(kMidCols * groups)) : 0;
  const int64_t red = (int64_t)p.waves * p.MS * 2 * 1024;
  p.s_lds = s_cap / 4 <= slots && z_cap / 4 <= slots && s_cap + z_cap + red <= 160 * 1024;
  p.lds = (unsigned)((p.s_lds ? s_cap + z_cap : 0) + red);
  return p;
}

// row tiles go along grid y, at most 65535 per launch: taller A is split
// into launches over consecutive row ranges (offset A, C and the residual)
template <int FMT, bool OUT_F32, int U, int MS, bool S_LDS>
hipError_t launch_v(const GemmArgs& a, const MidPlan& p) {
  const int64_t chunk = (int64_t)65535 * 16 * MS;
  const int64_t es = OUT_F32 ? 4 : 2;
  for (int64_t m = 0; m < a.M; m += chunk) {
    const int64_t rows = a.M - m < chunk ? a.M - m : chunk;
    const dim3 grid((unsigned)((a.N + kMidCols - 1) / kMidCols), (unsigned)((rows + 16 * MS - 1) / (16 * MS)));
    Epilogue epi = a.epi;
    if (epi.res) epi.res = static_cast<const uint8_t*>(epi.res) + m * a.N * es;
    const hipError_t e =
        launch_kernel(mid_kernel<FMT, OUT_F32, U, MS, S_LDS>, grid, dim3(64 * p.waves), p.lds, a.stream,
                      a.A + m * a.K, a.packed, a.scales, a.zeros, static_cast<uint8_t*>(a.C) + m * a.N * es,
                      (int)rows, (int)a.N, (int)a.K, a.pre ? 1 : 0, epi);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int FMT, bool OUT_F32, int U, int MS>
hipError_t launch_s(const GemmArgs& a, const MidPlan& p) {
  return p.s_lds ? launch_v<FMT, OUT_F32, U, MS, true>(a, p) : launch_v<FMT, OUT_F32, U, MS, false>(a, p);
}

template <int FMT, bool OUT_F32, int U>
hipError_t launch_m(const GemmArgs& a, const MidPlan& p) {
  if (p.MS == 2) return launch_s<FMT, OUT_F32, U, 2>(a, p);
  if (p.MS == 3) return launch_s<FMT, OUT_F32, U, 3>(a, p);
  return launch_s<FMT, OUT_F32, U, 4>(a, p);
}

// the ring variant over row tiles of 16 MS rows, at most 65535 per launch
template <int FMT, bool OUT_F32, int MS, int D>
hipError_t launch_ring(const GemmArgs& a, unsigned lds) {
  const int64_t chunk = (int64_t)65535 * 16 * MS;
  const int64_t es = OUT_F32 ? 4 : 2;
  const bool full = a.K % 128 == 0;
  for (int64_t m = 0; m < a.M; m += chunk) {
    const int64_t rows = a.M - m < chunk ? a.M - m : chunk;
    const dim3 grid((unsigned)((a.N + kMidCols - 1) / kMidCols), (unsigned)((rows + 16 * MS - 1) / (16 * MS)));
    Epilogue epi = a.epi;
    if (epi.res) epi.res = static_cast<const uint8_t*>(epi.res) + m * a.N * es;
    const hipError_t e =
        full ? launch_kernel(mid_ring_kernel<FMT, OUT_F32, MS, D, true>, grid, dim3(64 * kMidRingWaves), lds,
                             a.stream, a.A + m * a.K, a.packed, a.scales, a.zeros,
                             static_cast<uint8_t*>(a.C) + m * a.N * es, (int)rows, (int)a.N, (int)a.K,
                             a.pre ? 1 : 0, epi)
             : launch_kernel(mid_ring_kernel<FMT, OUT_F32, MS, D, false>, grid, dim3(64 * kMidRingWaves), lds,
                             a.stream, a.A + m * a.K, a.packed, a.scales, a.zeros,
                             static_cast<uint8_t*>(a.C) + m * a.N * es, (int)rows, (int)a.N, (int)a.K,
                             a.pre ? 1 : 0, epi);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// The ring variant when its LDS fits beside the scale windows, 2 slots per
// wave (measured: 3 slots or 2 / 3 waves are no faster); tiles of 48 or 64
// rows that do not fit become 32-row tiles.
template <int FMT, bool OUT_F32>
bool try_mid_ring(const GemmArgs& a, int MS, hipError_t& err) {
  constexpr int SB = mid_sb<FMT>();
  const int64_t groups = (a.K + FormatTraits<FMT>::kGroup - 1) / FormatTraits<FMT>::kGroup;
  const int64_t win = mid_ring_window((uint32_t)(kMidCols * groups * SB)) +
                      (has_zeros(FMT) ? mid_ring_window((uint32_t)(kMidCols * groups)) : 0);
  constexpr int64_t kLds = 160 * 1024;
  if (MS > 2 && win + (int64_t)kMidRingWaves * 2 * mid_ring_slot(MS) > kLds) MS = 2;
  auto lds_of = [&](int d) { return win + (int64_t)kMidRingWaves * d * mid_ring_slot(MS); };
  if (lds_of(2) > kLds) return false;
  const unsigned lds = (unsigned)lds_of(2);
  err = MS == 2 ? launch_ring<FMT, OUT_F32, 2, 2>(a, lds)
      : MS == 3 ? launch_ring<FMT, OUT_F32, 3, 2>(a, lds)
                : launch_ring<FMT, OUT_F32, 4, 2>(a, lds);
  return true;
}

template <int FMT, bool OUT_F32>
hipError_t launch_fmt(const GemmArgs& a) {
  const MidPlan p = mid_plan(FMT, a.M, a.K);
  hipError_t err = hipSuccess;
  if (try_mid_ring<FMT, OUT_F32>(a, p.MS, err)) return err;
  return p.U == 2 ? launch_m<FMT, OUT_F32, 2>(a, p) : launch_m<FMT, OUT_F32, 4>(a, p);
}

}  // namespace

hipError_t launch_mid(const GemmArgs& a) {
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
