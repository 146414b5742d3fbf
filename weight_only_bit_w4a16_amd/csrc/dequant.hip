// dequant.hip -- standalone dequantisation W = dequant(packed, scales, zeros)
// to bf16 (N, K), the checking path for bit-exactness of the decoders the
// GEMM kernels share.  One thread turns one 16-byte packed chunk (32 codes of
// one row, inside one group for every format) into 64 bytes of bf16; when K
// is an odd multiple of 16 (rows of K/2 bytes only 8-byte aligned), one
// 8-byte chunk of 16 codes into 32 bytes.
//
// Element rules (page titles): int4 -- "megakernel_int4_weight_decode.py",
// "The weight format": (code - zero) * scale, the subtraction first, per
// group of 128 (its configuration's `group`; 32 and 64 also served); NVFP4 --
// "Matmul2dFp4", run: e2m1 times |e4m3 scale| per 16; MXFP4 -- e2m1 times
// 2^(E-127) per 32.  Each weight is exact in fp32 and rounded once to bf16.
#include "common.hpp"
#include "kernels.hpp"

namespace w4a16 {

namespace {

// 16 codes (8 bytes, one group for every format) of row n at chunk c
template <int FMT>
__device__ __forceinline__ void dequant16(const uint8_t* __restrict__ packed, const void* __restrict__ scales,
                                          const uint8_t* __restrict__ zeros, uint16_t* __restrict__ W,
                                          int64_t K, int64_t groups, int64_t n, int64_t c) {
  constexpr int G = FormatTraits<FMT>::kGroup;
  const u32x2_t q = *reinterpret_cast<const u32x2_t*>(packed + n * (K / 2) + c * 8);
  u32x4_t out[2];
  if constexpr (is_int4(FMT)) {
    const int64_t g = (c * 16) / G;
    const float s = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(scales)[n * groups + g]);
    const float zf = has_zeros(FMT) ? (float)zeros[n * groups + g] : (float)kSymZero;
    out[0] = int4x8_to_bf16_weights(q[0], s, zf);
    out[1] = int4x8_to_bf16_weights(q[1], s, zf);
  } else if constexpr (FMT == kNvfp4) {
    const float s = e4m3_magnitude(reinterpret_cast<const uint8_t*>(scales)[n * groups + c]);
    out[0] = fp4x8_to_bf16_fscale(q[0], s);
    out[1] = fp4x8_to_bf16_fscale(q[1], s);
  } else {
    const uint32_t E = reinterpret_cast<const uint8_t*>(scales)[n * groups + (c * 16) / 32];
    const float es = e8m0_as_exponent_scale(E);  // exponent field 255: NaN from the converter
    out[0] = fp4x8_to_bf16_escale(q[0], es);
    out[1] = fp4x8_to_bf16_escale(q[1], es);
  }
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(W + n * K + c * 16);
  dst[0] = out[0];
  dst[1] = out[1];
}

template <int FMT>
__global__ __launch_bounds__(256) void dequant16_kernel(const uint8_t* __restrict__ packed,
                                                        const void* __restrict__ scales,
                                                        const uint8_t* __restrict__ zeros,
                                                        uint16_t* __restrict__ W, int64_t N, int64_t K) {
  const int64_t chunks_per_row = K / 16;
  const int64_t total = N * chunks_per_row;
  constexpr int G = FormatTraits<FMT>::kGroup;
  const int64_t groups = (K + G - 1) / G;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = i / chunks_per_row;
    dequant16<FMT>(packed, scales, zeros, W, K, groups, n, i - n * chunks_per_row);
  }
}

template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ packed,
                                                      const void* __restrict__ scales,
                                                      const uint8_t* __restrict__ zeros,
                                                      uint16_t* __restrict__ W, int64_t N,
                                                      int64_t K, int pre) {
  const int64_t chunks_per_row = K / 32;
  const int64_t total = N * chunks_per_row;
  constexpr int G = FormatTraits<FMT>::kGroup;
  const int64_t groups = (K + G - 1) / G;  // the last group may be shorter
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = i / chunks_per_row;
    const int64_t c = i - n * chunks_per_row;
    // (prepacked: chunk c of row n at slot n % 16 + 16 (c % 4) of the tile's
    // 1-KB block c / 4)
    const int64_t src = pre ? (n >> 4) * 16 * (K / 2) + (c >> 2) * 1024 + ((n & 15) + 16 * (c & 3)) * 16
                            : n * (K / 2) + c * 16;
    const u32x4_t q = *reinterpret_cast<const u32x4_t*>(packed + src);
    u32x4_t out[4];
    if constexpr (is_int4(FMT)) {
      const int64_t g = (c * 32) / G;
      const float s = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(scales)[n * groups + g]);
      const float zf = has_zeros(FMT) ? (float)zeros[n * groups + g] : (float)kSymZero;
#pragma unroll
      for (int d = 0; d < 4; ++d) out[d] = int4x8_to_bf16_weights(q[d], s, zf);
    } else if constexpr (FMT == kNvfp4) {
      const uint8_t* sp = reinterpret_cast<const uint8_t*>(scales) + n * groups + c * 2;
      const float s0 = e4m3_magnitude(sp[0]);
      const float s1 = e4m3_magnitude(sp[1]);
      out[0] = fp4x8_to_bf16_fscale(q[0], s0);
      out[1] = fp4x8_to_bf16_fscale(q[1], s0);
      out[2] = fp4x8_to_bf16_fscale(q[2], s1);
      out[3] = fp4x8_to_bf16_fscale(q[3], s1);
    } else {
      const uint32_t E = reinterpret_cast<const uint8_t*>(scales)[n * groups + c];
      if (E != 255u) {
        const float es = e8m0_as_exponent_scale(E);
#pragma unroll
        for (int d = 0; d < 4; ++d) out[d] = fp4x8_to_bf16_escale(q[d], es);
      } else {
        // NaN scale: every weight of the block is NaN
#pragma unroll
        for (int d = 0; d < 4; ++d) out[d] = u32x4_t{0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
      }
    }
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(W + n * K + c * 32);
#pragma unroll
    for (int d = 0; d < 4; ++d) dst[d] = out[d];
  }
}

template <int FMT>
hipError_t launch_dequant16(const uint8_t* packed, const void* scales, const uint8_t* zeros, uint16_t* W,
                            int64_t N, int64_t K, hipStream_t stream) {
  const int64_t total = N * (K / 16);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;  // grid-stride loop covers the rest
  return launch_kernel(dequant16_kernel<FMT>, dim3((unsigned)blocks), dim3(256), 0, stream, packed, scales,
                       zeros, W, N, K);
}

}  // namespace

hipError_t launch_dequant(int fmt, const uint8_t* packed, const void* scales, const uint8_t* zeros,
                          uint16_t* W, int64_t N, int64_t K, bool pre, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  if (K % 32 != 0) {
    switch (fmt) {
      case kInt4: return launch_dequant16<kInt4>(packed, scales, zeros, W, N, K, stream);
      case kNvfp4: return launch_dequant16<kNvfp4>(packed, scales, zeros, W, N, K, stream);
      case kInt4G32: return launch_dequant16<kInt4G32>(packed, scales, zeros, W, N, K, stream);
      case kInt4G64: return launch_dequant16<kInt4G64>(packed, scales, zeros, W, N, K, stream);
      case kInt4Sym: return launch_dequant16<kInt4Sym>(packed, scales, zeros, W, N, K, stream);
      default: return launch_dequant16<kMxfp4>(packed, scales, zeros, W, N, K, stream);
    }
  }
  const int64_t total = N * (K / 32);
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;  // grid-stride loop covers the rest
  switch (fmt) {
    case kInt4:
      return launch_kernel(dequant_kernel<kInt4>, dim3((unsigned)blocks), dim3(threads), 0, stream,
                           packed, scales, zeros, W, N, K, pre ? 1 : 0);
    case kNvfp4:
      return launch_kernel(dequant_kernel<kNvfp4>, dim3((unsigned)blocks), dim3(threads), 0, stream,
                           packed, scales, zeros, W, N, K, pre ? 1 : 0);
    case kInt4G32:
      return launch_kernel(dequant_kernel<kInt4G32>, dim3((unsigned)blocks), dim3(threads), 0, stream,
                           packed, scales, zeros, W, N, K, pre ? 1 : 0);
    case kInt4G64:
      return launch_kernel(dequant_kernel<kInt4G64>, dim3((unsigned)blocks), dim3(threads), 0, stream,
                           packed, scales, zeros, W, N, K, pre ? 1 : 0);
    case kInt4Sym:
      return launch_kernel(dequant_kernel<kInt4Sym>, dim3((unsigned)blocks), dim3(threads), 0, stream,
                           packed, scales, zeros, W, N, K, pre ? 1 : 0);
    default:
      return launch_kernel(dequant_kernel<kMxfp4>, dim3((unsigned)blocks), dim3(threads), 0, stream,
                           packed, scales, zeros, W, N, K, pre ? 1 : 0);
  }
}

// ---- prepacking ------------------------------------------------------------------
// One thread per 16-byte chunk of the output, in output order (contiguous
// stores; each 1-KB block gathers 64 bytes from each of 16 rows).  Rows past
// N (the last tile's padding) become zero bytes.
namespace {
__global__ __launch_bounds__(256) void prepack_kernel(const uint8_t* __restrict__ packed,
                                                      uint8_t* __restrict__ out, int64_t N, int64_t K) {
  const int64_t rowb = K / 2, kblocks = K / 128;
  const int64_t total = ((N + 15) / 16) * kblocks * 64;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t l = i & 63, blk = i >> 6;
    const int64_t t = blk / kblocks, b = blk - t * kblocks;
    const int64_t n = 16 * t + (l & 15), c = 4 * b + (l >> 4);
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (n < N) v = *reinterpret_cast<const u32x4_t*>(packed + n * rowb + c * 16);
    *reinterpret_cast<u32x4_t*>(out + i * 16) = v;
  }
}
}  // namespace

hipError_t launch_prepack(const uint8_t* packed, uint8_t* out, int64_t N, int64_t K, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const int64_t total = ((N + 15) / 16) * (K / 128) * 64;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;  // grid-stride loop covers the rest
  return launch_kernel(prepack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, packed, out, N, K);
}

}  // namespace w4a16
