/*
 * w4a16_probe.h -- measurement kernels of libw4a16_probe.so (not part of the
 * W4A16 GEMM library): the bounds the GEMM kernels are compared with in
 * bench.py --bounds.  Every pointer is a caller-owned DEVICE pointer; calls
 * only enqueue one or two kernels on `stream` (a hipStream_t, NULL = default)
 * and return W4A16_PROBE_OK, W4A16_PROBE_ERR_ARG (argument rejected on the
 * host, nothing enqueued) or W4A16_PROBE_ERR_HIP (the launch's own status).
 */
#ifndef W4A16_PROBE_H
#define W4A16_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A16_PROBE_OK 0
#define W4A16_PROBE_ERR_ARG (-2)
#define W4A16_PROBE_ERR_HIP (-5)

/* One workgroup of one wave that does nothing (writes `sink`, a uint32, only
 * on an impossible block index): the per-launch floor. */
int w4a16_probe_empty(void* sink, void* stream);

/* Reads `bytes` (> 0, multiple of 16) at `p` (16-byte aligned) once with
 * 16-byte loads: `threads` per workgroup (64 .. 1024, multiple of 64),
 * `per_thread` loads per thread (1, 2, 4, 8; grid-stride), as many
 * workgroups as that takes.  `sink`: a uint32, written only if the XOR of
 * everything read equals a magic value. */
int w4a16_probe_read(const void* p, int64_t bytes, int threads, int per_thread, void* sink, void* stream);

/* `workgroups` x `threads` (64 .. 1024) threads each issue `iters` x 8
 * independent v_mfma_f32_16x16x32_bf16 on registers (16384 flops each per
 * wave).  `sink`: one float, written only on a magic sum. */
int w4a16_probe_mfma(int workgroups, int threads, int iters, void* sink, void* stream);

/* A split-K hand-off between workgroups.  `groups` x `slices` workgroups of
 * 256 threads; workgroup (g, s) writes 768 floats to scratch[(g*slices+s)*768 ..]
 * (scratch: groups*slices*768 floats).  mode 0: nothing more; mode 1: after a
 * device-scope fence in one thread, an atomic add on counters[g] (groups
 * uint32, zero before the first call; every call leaves them zero) picks the
 * last workgroup of the group, which adds the slices in order into
 * out[g*768 ..] (groups*768 floats); mode 2: the same with a fence in every
 * thread; mode 3: mode 0, then a second kernel of `groups` workgroups adds the
 * slices into `out`. */
int w4a16_probe_handoff(void* scratch, void* counters, void* out, int groups, int slices, int mode,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_PROBE_H */
