// probe.hip -- measurement kernels (libw4a16_probe.so), not part of the GEMM
// library: the bounds that the GEMM kernels are compared with.
//   * an empty launch (the per-launch floor of a replayed HIP graph);
//   * a plain read of a buffer, 16-byte loads, several launch shapes (the
//     floor of a launch that must move a given number of bytes);
//   * a loop of independent v_mfma_f32_16x16x32_bf16 on every CU (the matrix
//     rate the chip sustains, clock included);
//   * a split-K hand-off: each of `slices` workgroups per group writes a
//     3-KB partial sum and the last to arrive adds them (device-scope fence
//     and counter), or the partials alone, or a second reduction kernel.
// Every loop is bounded; no kernel waits on another workgroup.
#include <hip/hip_runtime.h>

#include "kernels.hpp"
#include "w4a16_probe.h"

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4p_t;

__global__ void empty_kernel(unsigned* sink) {
  if (threadIdx.x == 0 && sink != nullptr && blockIdx.x == 0x7FFFFFFF) sink[0] = 1u;
}

// every thread reads L 16-byte chunks (grid-stride), XORs them, and writes
// only if the XOR hits a magic value
template <int L>
__global__ __launch_bounds__(1024) void read_kernel(const uint4* __restrict__ p, long long n16,
                                                    unsigned* __restrict__ sink) {
  const long long base = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long stride = (long long)gridDim.x * blockDim.x;
  uint4 v[L];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const long long idx = base + i * stride;
    v[i] = idx < n16 ? p[idx] : make_uint4(0u, 0u, 0u, 0u);
  }
  unsigned acc = 0u;
#pragma unroll
  for (int i = 0; i < L; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

__global__ __launch_bounds__(1024) void mfma_kernel(int iters, float* __restrict__ sink) {
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1e-3f * (float)(threadIdx.x + i));
    b[i] = (__bf16)(1e-3f * (float)(i + 1));
  }
  f32x4p_t acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f32x4p_t{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  if (s == 12345.f) sink[0] = s;
}

// workgroup g * slices + s writes partial (g, s) of 768 floats; mode 1: the
// last workgroup of group g (device-scope fence + counter, one fence per
// workgroup) adds the slices in order; mode 2: the same with a fence in
// every thread; mode 0: partials only.  The last workgroup resets the counter.
__global__ __launch_bounds__(256) void handoff_kernel(float* __restrict__ scratch, unsigned* __restrict__ counters,
                                                      float* __restrict__ out, int slices, int mode) {
  const int g = blockIdx.x / slices, s = blockIdx.x % slices;
  const int t = threadIdx.x;
  float* mine = scratch + ((size_t)g * slices + s) * 768;
#pragma unroll
  for (int i = 0; i < 3; ++i) mine[t + 256 * i] = (float)(g + s + t + i);
  if (mode == 0) return;
  __shared__ int last;
  if (mode == 2) __threadfence();
  __syncthreads();
  if (t == 0) {
    if (mode == 1) __threadfence();
    last = atomicAdd(&counters[g], 1u) == (unsigned)(slices - 1);
    if (last) __threadfence();
  }
  __syncthreads();
  if (!last) return;
  float sum[3] = {0.f, 0.f, 0.f};
  for (int j = 0; j < slices; ++j)
#pragma unroll
    for (int i = 0; i < 3; ++i) sum[i] += __builtin_nontemporal_load(&scratch[((size_t)g * slices + j) * 768 + t + 256 * i]);
#pragma unroll
  for (int i = 0; i < 3; ++i) out[(size_t)g * 768 + t + 256 * i] = sum[i];
  if (t == 0) counters[g] = 0u;
}

__global__ __launch_bounds__(256) void reduce_kernel(const float* __restrict__ scratch, float* __restrict__ out,
                                                     int slices) {
  const int g = blockIdx.x, t = threadIdx.x;
  float sum[3] = {0.f, 0.f, 0.f};
  for (int j = 0; j < slices; ++j)
#pragma unroll
    for (int i = 0; i < 3; ++i) sum[i] += scratch[((size_t)g * slices + j) * 768 + t + 256 * i];
#pragma unroll
  for (int i = 0; i < 3; ++i) out[(size_t)g * 768 + t + 256 * i] = sum[i];
}

int status(hipError_t e) { return e == hipSuccess ? W4A16_PROBE_OK : W4A16_PROBE_ERR_HIP; }
using w4a16::launch_kernel;

}  // namespace

extern "C" {

int w4a16_probe_empty(void* sink, void* stream) {
  return status(launch_kernel(empty_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                              static_cast<unsigned*>(sink)));
}

int w4a16_probe_read(const void* p, int64_t bytes, int threads, int per_thread, void* sink, void* stream) {
  if (!p || !sink) return W4A16_PROBE_ERR_ARG;
  if (bytes <= 0 || bytes % 16 != 0 || ((uintptr_t)p & 15u) != 0) return W4A16_PROBE_ERR_ARG;
  if (threads < 64 || threads > 1024 || threads % 64 != 0) return W4A16_PROBE_ERR_ARG;
  if (per_thread != 1 && per_thread != 2 && per_thread != 4 && per_thread != 8) return W4A16_PROBE_ERR_ARG;
  const long long n16 = bytes / 16;
  const long long total = (n16 + per_thread - 1) / per_thread;
  const long long blocks = (total + threads - 1) / threads;
  if (blocks > 0x7FFFFFFF) return W4A16_PROBE_ERR_ARG;
  const auto st = static_cast<hipStream_t>(stream);
  const auto src = static_cast<const uint4*>(p);
  auto* out = static_cast<unsigned*>(sink);
  const dim3 grid((unsigned)blocks), block(threads);
  switch (per_thread) {
    case 1: return status(launch_kernel(read_kernel<1>, grid, block, 0, st, src, n16, out));
    case 2: return status(launch_kernel(read_kernel<2>, grid, block, 0, st, src, n16, out));
    case 4: return status(launch_kernel(read_kernel<4>, grid, block, 0, st, src, n16, out));
    default: return status(launch_kernel(read_kernel<8>, grid, block, 0, st, src, n16, out));
  }
}

int w4a16_probe_mfma(int workgroups, int threads, int iters, void* sink, void* stream) {
  if (!sink || workgroups < 1 || iters < 1 || threads < 64 || threads > 1024 || threads % 64 != 0)
    return W4A16_PROBE_ERR_ARG;
  return status(launch_kernel(mfma_kernel, dim3(workgroups), dim3(threads), 0, static_cast<hipStream_t>(stream),
                              iters, static_cast<float*>(sink)));
}

int w4a16_probe_handoff(void* scratch, void* counters, void* out, int groups, int slices, int mode,
                        void* stream) {
  if (!scratch || !counters || !out || groups < 1 || slices < 1 || mode < 0 || mode > 3 ||
      (int64_t)groups * slices > 0x7FFFFFFF)
    return W4A16_PROBE_ERR_ARG;
  const auto st = static_cast<hipStream_t>(stream);
  auto* sc = static_cast<float*>(scratch);
  auto* cnt = static_cast<unsigned*>(counters);
  auto* o = static_cast<float*>(out);
  if (mode == 3) {  // partials, then a second kernel sums them
    const hipError_t e = launch_kernel(handoff_kernel, dim3(groups * slices), dim3(256), 0, st, sc, cnt, o, slices, 0);
    if (e != hipSuccess) return status(e);
    return status(launch_kernel(reduce_kernel, dim3(groups), dim3(256), 0, st, static_cast<const float*>(sc), o,
                                slices));
  }
  return status(launch_kernel(handoff_kernel, dim3(groups * slices), dim3(256), 0, st, sc, cnt, o, slices, mode));
}

}  // extern "C"
