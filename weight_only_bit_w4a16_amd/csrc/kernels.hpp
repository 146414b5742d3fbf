// kernels.hpp -- launchers of the gfx950 kernels, called by the C ABI in
// api.cpp after it has validated every argument.  Each returns the HIP error
// of its launch (hipSuccess when nothing needed launching).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <type_traits>
#include <utility>

namespace w4a16 {

// Enqueue `kernel` on `stream` and return the status of this launch itself
// (hipLaunchKernel's own result: an earlier, unrelated error of the calling
// thread is neither reported nor cleared).  The arguments are converted to
// the kernel's parameter types and passed by address.  A grid whose
// work-items along one dimension exceed 2^32 - 1 (the dispatch packet's
// 32-bit sizes) is refused here, before any launch.
template <typename... Params, typename... Args>
inline hipError_t launch_kernel(void (*kernel)(Params...), dim3 grid, dim3 block, unsigned lds,
                                hipStream_t stream, Args&&... args) {
  static_assert(sizeof...(Params) == sizeof...(Args), "kernel argument count");
  constexpr uint64_t kMaxItems = 0xFFFFFFFFull;
  if ((uint64_t)grid.x * block.x > kMaxItems || (uint64_t)grid.y * block.y > kMaxItems ||
      (uint64_t)grid.z * block.z > kMaxItems)
    return hipErrorInvalidConfiguration;
  std::tuple<std::decay_t<Params>...> vals(std::forward<Args>(args)...);
  void* ptrs[sizeof...(Params) > 0 ? sizeof...(Params) : 1];
  std::apply([&ptrs](auto&... v) {
    int i = 0;
    ((ptrs[i++] = static_cast<void*>(&v)), ...);
  }, vals);
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, lds, stream);
}

// Fused epilogue on the fp32 accumulator c: C = act(alpha * c + bias[n]) +
// beta * R[m, n] (bias bf16 (N) or null; R (M, N) in C's dtype, read only
// when non-null and beta != 0).  `on` false: C = c.
struct Epilogue {
  const uint16_t* bias;
  const void* res;
  float alpha, beta;
  int act;  // 0 none, 1 ReLU, 2 SiLU, 3 GELU (tanh form)
  int on;
};

struct GemmArgs {
  int fmt;        // 0 int4 g128, 1 NVFP4, 2 MXFP4
  bool out_f32;   // C is fp32 (else bf16)
  bool pre;       // packed is in the prepacked layout (K % 128 == 0)
  const uint16_t* A;
  const uint8_t* packed;
  const void* scales;
  const uint8_t* zeros;
  void* C;
  int64_t M, N, K;
  hipStream_t stream;
  Epilogue epi;
};

// Several weight matrices of one K in one launch: member i has its own
// activations A[i] (the same pointer for every member of a w4a16_gemm_grouped
// call), packed / scales / zeros / C and N[i] output columns.
constexpr int kMaxGroup = 32;
struct GroupedArgs {
  int fmt;
  bool out_f32;
  bool pre;   // every member's weights in the prepacked layout
  int count;  // 1 .. kMaxGroup, every member with N[i] > 0
  const uint16_t* A[kMaxGroup];
  const uint8_t* packed[kMaxGroup];
  const void* scales[kMaxGroup];
  const uint8_t* zeros[kMaxGroup];
  void* C[kMaxGroup];
  int64_t N[kMaxGroup];
  int64_t M, K;
  hipStream_t stream;
  Epilogue epi;  // single-matrix launches only (count == 1)
};

hipError_t launch_dequant(int fmt, const uint8_t* packed, const void* scales, const uint8_t* zeros,
                          uint16_t* W, int64_t N, int64_t K, bool pre, hipStream_t stream);

// the prepacked layout of row-major packed weights (N, K/2), K % 128 == 0
hipError_t launch_prepack(const uint8_t* packed, uint8_t* out, int64_t N, int64_t K, hipStream_t stream);

// M <= 16 per 16-row slice: split-K over the waves of a workgroup, weights
// decoded in registers.
hipError_t launch_skinny(const GemmArgs& a);
// the same kernel over all members of a group in one launch
hipError_t launch_skinny_grouped(const GroupedArgs& a);

// 16 < M <= ~192: 32-column x 32..64-row tiles, split-K over the waves of a
// workgroup, each weight decoded once for all of the tile's rows.
hipError_t launch_mid(const GemmArgs& a);

// large M: LDS-staged tiles, decode into MFMA B fragments.
hipError_t launch_tiled(const GemmArgs& a);

// K an odd multiple of 16 (rows of K/2 bytes only 8-byte aligned), any M:
// 4-byte weight loads, one MFMA per 32-code step.
hipError_t launch_ragged(const GemmArgs& a);

}  // namespace w4a16
