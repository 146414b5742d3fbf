// api.cpp -- the C ABI declared in include/w4a16.h: host-side validation and
// kernel dispatch.  Every check runs before any HIP call, so a rejected call
// enqueues nothing (and never touches the HIP runtime).
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "w4a16.h"
#include "kernels.hpp"

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;  // kernels index rows with 32-bit ints
constexpr int64_t kMaxK = (int64_t)1 << 22;    // a 256-row tile of A fits a 32-bit byte offset

// formats whose weights come with a zero array (required non-NULL; NULL
// required for every other format)
bool has_zeros(int fmt) {
  return fmt == W4A16_INT4_G128 || fmt == W4A16_INT4_G32 || fmt == W4A16_INT4_G64;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// format, flags and shape checks shared by w4a16_gemm and w4a16_gemm_path
// (W4A16_PREPACKED is accepted everywhere; allow_flags adds the output type
// and the kernel choice)
int check_format_shape(int format, int64_t M, int64_t N, int64_t K, bool allow_flags) {
  const int fmt = format & W4A16_FORMAT_MASK;
  const int flags = format & ~W4A16_FORMAT_MASK;
  if (fmt > W4A16_INT4_SYM) return W4A16_ERR_FORMAT;
  const int allowed = W4A16_PREPACKED | (allow_flags ? (W4A16_OUT_F32 | W4A16_PATH_MASK) : 0);
  if (flags & ~allowed) return W4A16_ERR_FORMAT;
  if (M < 0 || N < 0 || K <= 0) return W4A16_ERR_SHAPE;
  if (K % 16 != 0) return W4A16_ERR_SHAPE;  // the last group may be shorter than G
  if ((format & W4A16_PREPACKED) && K % 128 != 0) return W4A16_ERR_SHAPE;  // whole 1-KB blocks
  if (M >= kMaxDim || N >= kMaxDim || K > kMaxK) return W4A16_ERR_SHAPE;
  return W4A16_OK;
}

// The skinny kernel reads and decodes the weights once per 16-row slice of
// A; the mid kernel once per tile of up to 64 rows, but each of its
// workgroups (32 columns) reads all of A through its CU, which sets a
// workgroup's time (~15 us at 64 rows, K = 3072) however many run; the tiled
// kernel (256 x 256 tiles, or 128 x 128 when the large ones would leave CUs
// idle) runs the whole of K inside each tile, and with few tiles its time is
// one tile's k-loop (~33 us MXFP4, ~53 us int4 at K = 3072).  So, measured
// (us at N = 8192, K = 3072: M = 64 skinny 29 / mid 17 / tiled 30 (MXFP4);
// M = 192 int4 83 / 46 / 53, MXFP4 70 / 46 / 33; M = 384 int4 162 / 88 / 56):
// the mid kernel while it runs in at most 2 rounds of 256 workgroups (3 for
// int4, whose tiled decode is dearer) and has >= 160 of them; the skinny
// kernel when it would have fewer (narrow matrices: N = 1024, M = 64: 4.8 /
// 15 / 51); with 256 or more large tiles the tiled kernel, except at M <= 48
// (LM head 128256 x 3072, M = 32: 242 / 144 / 219).  N: the widest matrix.
int choose_path(int format, int64_t M, int64_t N, int64_t K) {
  if (K % 32 != 0) return W4A16_PATH_RAGGED;  // the only kernel for rows 8-byte aligned
  const int forced = format & W4A16_PATH_MASK;
  if (forced) return forced;
  if (M <= 16) return W4A16_PATH_SKINNY;
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (tiles >= 256) return M <= 64 ? W4A16_PATH_MID : W4A16_PATH_TILED;
  const int64_t mid_wgs = ((N + 31) / 32) * ((M + 63) / 64);
  if (mid_wgs < 160) return M <= 384 ? W4A16_PATH_SKINNY : W4A16_PATH_TILED;
  // up to 3.5 rounds of 256 workgroups (measured crossover against the
  // tiled kernel, every format)
  return mid_wgs <= 896 ? W4A16_PATH_MID : W4A16_PATH_TILED;
}

hipError_t launch_path(int path, const w4a16::GemmArgs& a) {
  if (path == W4A16_PATH_RAGGED) return w4a16::launch_ragged(a);
  if (path == W4A16_PATH_SKINNY) return w4a16::launch_skinny(a);
  if (path == W4A16_PATH_MID) return w4a16::launch_mid(a);
  return w4a16::launch_tiled(a);
}

}  // namespace

extern "C" {

int w4a16_version(void) { return 106; }

const char* w4a16_strerror(int status) {
  switch (status) {
    case W4A16_OK: return "success";
    case W4A16_ERR_FORMAT: return "unknown weight format or flag bits";
    case W4A16_ERR_SHAPE:
      return "bad shape: need 0 <= M, N < 2^31, 0 < K <= 2^22 and K % 16 == 0 (K % 128 == 0 for "
             "prepacked weights; 1 <= count <= W4A16_MAX_GROUP for a group)";
    case W4A16_ERR_NULL: return "a required pointer is NULL, or zeros is non-NULL for a format without zeros";
    case W4A16_ERR_ALIGN: return "a pointer violates its alignment requirement";
    case W4A16_ERR_HIP:
      return "the HIP runtime rejected a kernel launch, or its grid would exceed 2^32 - 1 work-items "
             "along a dimension";
    case W4A16_ERR_OVERLAP: return "the output of w4a16_prepack overlaps its input";
    case W4A16_ERR_EPILOGUE:
      return "bad epilogue: unknown activation, nonzero reserved field, or a residual that "
             "overlaps C without being C";
    default: return "unknown status";
  }
}

int w4a16_gemm_path(int format, int64_t M, int64_t N, int64_t K) {
  const int rc = check_format_shape(format, M, N, K, true);
  if (rc != W4A16_OK) return rc;
  return choose_path(format, M, N, K);
}

int w4a16_gemm(int format, const void* A, const void* packed, const void* scales,
               const void* zeros, void* C, int64_t M, int64_t N, int64_t K, void* stream) {
  return w4a16_gemm_ex(format, A, packed, scales, zeros, C, M, N, K, nullptr, stream);
}

int w4a16_gemm_ex(int format, const void* A, const void* packed, const void* scales,
                  const void* zeros, void* C, int64_t M, int64_t N, int64_t K,
                  const w4a16_epilogue* ep, void* stream) {
  const int rc = check_format_shape(format, M, N, K, true);
  if (rc != W4A16_OK) return rc;
  if (ep && (ep->activation < W4A16_ACT_NONE || ep->activation > W4A16_ACT_GELU_TANH ||
             ep->reserved != 0))
    return W4A16_ERR_EPILOGUE;
  const int fmt = format & W4A16_FORMAT_MASK;
  const bool out_f32 = (format & W4A16_OUT_F32) != 0;
  if (M == 0 || N == 0) return W4A16_OK;  // nothing is read or written
  if (!A || !packed || !scales || !C) return W4A16_ERR_NULL;
  if (has_zeros(fmt) ? !zeros : zeros != nullptr) return W4A16_ERR_NULL;
  if (!aligned(A, 16) || !aligned(packed, 16)) return W4A16_ERR_ALIGN;
  if (fmt != W4A16_MXFP4 && !aligned(scales, 2)) return W4A16_ERR_ALIGN;
  const uintptr_t es = out_f32 ? 4 : 2;
  if (!aligned(C, es)) return W4A16_ERR_ALIGN;
  w4a16::Epilogue epi = {};
  if (ep) {
    const bool res = ep->residual && ep->beta != 0.0f;
    if (ep->bias && !aligned(ep->bias, 2)) return W4A16_ERR_ALIGN;
    if (res && !aligned(ep->residual, es)) return W4A16_ERR_ALIGN;
    if (res && ep->residual != C) {
      const uintptr_t r0 = (uintptr_t)ep->residual, c0 = (uintptr_t)C;
      const uintptr_t bytes = (uintptr_t)M * (uintptr_t)N * es;
      if (r0 < c0 + bytes && c0 < r0 + bytes) return W4A16_ERR_EPILOGUE;
    }
    epi.bias = static_cast<const uint16_t*>(ep->bias);
    epi.res = res ? ep->residual : nullptr;
    epi.alpha = ep->alpha;
    epi.beta = ep->beta;
    epi.act = ep->activation;
    epi.on = 1;
  }

  w4a16::GemmArgs a;
  a.epi = epi;
  a.fmt = fmt;
  a.out_f32 = out_f32;
  a.pre = (format & W4A16_PREPACKED) != 0;
  a.A = static_cast<const uint16_t*>(A);
  a.packed = static_cast<const uint8_t*>(packed);
  a.scales = scales;
  a.zeros = static_cast<const uint8_t*>(zeros);
  a.C = C;
  a.M = M;
  a.N = N;
  a.K = K;
  a.stream = static_cast<hipStream_t>(stream);
  return launch_path(choose_path(format, M, N, K), a) == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

int w4a16_gemm_grouped(int format, const void* A, int count, const void* const* packed,
                       const void* const* scales, const void* const* zeros, void* const* C,
                       const int64_t* N, int64_t M, int64_t K, void* stream) {
  int rc = check_format_shape(format, M, 0, K, true);
  if (rc != W4A16_OK) return rc;
  if (count < 1 || count > W4A16_MAX_GROUP) return W4A16_ERR_SHAPE;
  if (!N) return W4A16_ERR_NULL;
  for (int i = 0; i < count; ++i)
    if ((rc = check_format_shape(format, M, N[i], K, true)) != W4A16_OK) return rc;
  const int fmt = format & W4A16_FORMAT_MASK;
  const bool out_f32 = (format & W4A16_OUT_F32) != 0;
  int active = 0;
  for (int i = 0; i < count; ++i) active += N[i] > 0;
  if (M == 0 || active == 0) return W4A16_OK;  // nothing is read or written
  if (!A || !packed || !scales || !C) return W4A16_ERR_NULL;
  if (has_zeros(fmt) ? !zeros : zeros != nullptr) return W4A16_ERR_NULL;
  if (!aligned(A, 16)) return W4A16_ERR_ALIGN;
  for (int i = 0; i < count; ++i) {
    if (N[i] == 0) continue;
    if (!packed[i] || !scales[i] || !C[i] || (has_zeros(fmt) && !zeros[i]))
      return W4A16_ERR_NULL;
    if (!aligned(packed[i], 16)) return W4A16_ERR_ALIGN;
    if (fmt != W4A16_MXFP4 && !aligned(scales[i], 2)) return W4A16_ERR_ALIGN;
    if (!aligned(C[i], out_f32 ? 4 : 2)) return W4A16_ERR_ALIGN;
  }

  int64_t max_n = 0;
  for (int i = 0; i < count; ++i) max_n = N[i] > max_n ? N[i] : max_n;
  const int path = choose_path(format, M, max_n, K);
  if (path == W4A16_PATH_SKINNY) {
    w4a16::GroupedArgs g = {};
    g.fmt = fmt;
    g.out_f32 = out_f32;
    g.pre = (format & W4A16_PREPACKED) != 0;
    for (int i = 0; i < count; ++i) {
      if (N[i] == 0) continue;
      g.A[g.count] = static_cast<const uint16_t*>(A);
      g.packed[g.count] = static_cast<const uint8_t*>(packed[i]);
      g.scales[g.count] = scales[i];
      g.zeros[g.count] = has_zeros(fmt) ? static_cast<const uint8_t*>(zeros[i]) : nullptr;
      g.C[g.count] = C[i];
      g.N[g.count] = N[i];
      ++g.count;
    }
    g.M = M;
    g.K = K;
    g.stream = static_cast<hipStream_t>(stream);
    return w4a16::launch_skinny_grouped(g) == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
  }
  // larger M: one mid or tiled launch per member
  for (int i = 0; i < count; ++i) {
    if (N[i] == 0) continue;
    w4a16::GemmArgs a;
    a.epi = w4a16::Epilogue{};
    a.fmt = fmt;
    a.out_f32 = out_f32;
    a.pre = (format & W4A16_PREPACKED) != 0;
    a.A = static_cast<const uint16_t*>(A);
    a.packed = static_cast<const uint8_t*>(packed[i]);
    a.scales = scales[i];
    a.zeros = has_zeros(fmt) ? static_cast<const uint8_t*>(zeros[i]) : nullptr;
    a.C = C[i];
    a.M = M;
    a.N = N[i];
    a.K = K;
    a.stream = static_cast<hipStream_t>(stream);
    if (launch_path(path, a) != hipSuccess) return W4A16_ERR_HIP;
  }
  return W4A16_OK;
}

int w4a16_gemm_batched(int format, int64_t M, int count, const w4a16_batch_item* items, void* stream) {
  // format and flags (output dtype only: the kernel is chosen per launch)
  const int fmt = format & W4A16_FORMAT_MASK;
  if (fmt > W4A16_INT4_SYM || (format & ~(W4A16_FORMAT_MASK | W4A16_OUT_F32 | W4A16_PREPACKED)))
    return W4A16_ERR_FORMAT;
  if (count < 0 || M < 0) return W4A16_ERR_SHAPE;
  if (count > 0 && !items) return W4A16_ERR_NULL;
  const bool out_f32 = (format & W4A16_OUT_F32) != 0;
  const bool pre = (format & W4A16_PREPACKED) != 0;
  // every item is checked before anything is enqueued
  int rc = W4A16_OK;
  for (int i = 0; i < count; ++i)
    if ((rc = check_format_shape(fmt | (format & W4A16_PREPACKED), M, items[i].N, items[i].K, false)) !=
        W4A16_OK)
      return rc;
  if (M == 0) return W4A16_OK;
  for (int i = 0; i < count; ++i) {
    const w4a16_batch_item& it = items[i];
    if (it.N == 0) continue;  // nothing is read or written
    if (!it.A || !it.packed || !it.scales || !it.C) return W4A16_ERR_NULL;
    if (has_zeros(fmt) ? !it.zeros : it.zeros != nullptr) return W4A16_ERR_NULL;
    if (!aligned(it.A, 16) || !aligned(it.packed, 16)) return W4A16_ERR_ALIGN;
    if (fmt != W4A16_MXFP4 && !aligned(it.scales, 2)) return W4A16_ERR_ALIGN;
    if (!aligned(it.C, out_f32 ? 4 : 2)) return W4A16_ERR_ALIGN;
  }
  auto single = [&](const w4a16_batch_item& it) {
    w4a16::GemmArgs a;
    a.epi = w4a16::Epilogue{};
    a.fmt = fmt;
    a.out_f32 = out_f32;
    a.pre = pre;
    a.A = static_cast<const uint16_t*>(it.A);
    a.packed = static_cast<const uint8_t*>(it.packed);
    a.scales = it.scales;
    a.zeros = static_cast<const uint8_t*>(it.zeros);
    a.C = it.C;
    a.M = M;
    a.N = it.N;
    a.K = it.K;
    a.stream = static_cast<hipStream_t>(stream);
    return launch_path(choose_path(fmt, M, it.N, it.K), a);
  };
  if (choose_path(fmt, M, 1, 32) != W4A16_PATH_SKINNY) {
    // larger M: every item is its own mid or tiled launch
    for (int i = 0; i < count; ++i)
      if (items[i].N > 0 && single(items[i]) != hipSuccess) return W4A16_ERR_HIP;
    return W4A16_OK;
  }
  // M <= 16: the items of one (K, N) share a skinny launch, up to kMaxGroup
  // members each (workgroup z = member); an item alone on its shape takes
  // the single-GEMM launch (which may be the streaming variant).  The skinny
  // kernel's split of K depends on the format, M and K only, so every item's
  // output equals w4a16_gemm's for it, bit for bit.
  std::vector<int> order;
  order.reserve((size_t)count);
  for (int i = 0; i < count; ++i) {
    if (items[i].N == 0) continue;
    if (items[i].K % 32 != 0) {  // the ragged-K kernel, one launch per item
      if (single(items[i]) != hipSuccess) return W4A16_ERR_HIP;
      continue;
    }
    order.push_back(i);
  }
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) {
    return items[x].K != items[y].K ? items[x].K < items[y].K : items[x].N < items[y].N;
  });
  for (size_t b = 0; b < order.size();) {
    size_t e = b + 1;
    while (e < order.size() && items[order[e]].K == items[order[b]].K && items[order[e]].N == items[order[b]].N)
      ++e;
    for (size_t c = b; c < e; c += w4a16::kMaxGroup) {
      const size_t n = std::min(e - c, (size_t)w4a16::kMaxGroup);
      if (n == 1) {
        if (single(items[order[c]]) != hipSuccess) return W4A16_ERR_HIP;
        continue;
      }
      w4a16::GroupedArgs g = {};
      g.fmt = fmt;
      g.out_f32 = out_f32;
      g.pre = pre;
      for (size_t j = 0; j < n; ++j) {
        const w4a16_batch_item& it = items[order[c + j]];
        g.A[g.count] = static_cast<const uint16_t*>(it.A);
        g.packed[g.count] = static_cast<const uint8_t*>(it.packed);
        g.scales[g.count] = it.scales;
        g.zeros[g.count] = has_zeros(fmt) ? static_cast<const uint8_t*>(it.zeros) : nullptr;
        g.C[g.count] = it.C;
        g.N[g.count] = it.N;
        ++g.count;
      }
      g.M = M;
      g.K = items[order[c]].K;
      g.stream = static_cast<hipStream_t>(stream);
      if (w4a16::launch_skinny_grouped(g) != hipSuccess) return W4A16_ERR_HIP;
    }
    b = e;
  }
  return W4A16_OK;
}

int w4a16_dequant(int format, const void* packed, const void* scales, const void* zeros, void* W,
                  int64_t N, int64_t K, void* stream) {
  const int rc = check_format_shape(format, 0, N, K, false);
  if (rc != W4A16_OK) return rc;
  const int fmt = format & W4A16_FORMAT_MASK;
  if (N == 0) return W4A16_OK;  // nothing is read or written
  if (!packed || !scales || !W) return W4A16_ERR_NULL;
  if (has_zeros(fmt) ? !zeros : zeros != nullptr) return W4A16_ERR_NULL;
  if (!aligned(packed, 16) || !aligned(W, 16)) return W4A16_ERR_ALIGN;
  if (fmt != W4A16_MXFP4 && !aligned(scales, 2)) return W4A16_ERR_ALIGN;
  const hipError_t e = w4a16::launch_dequant(fmt, static_cast<const uint8_t*>(packed), scales,
                                             static_cast<const uint8_t*>(zeros),
                                             static_cast<uint16_t*>(W), N, K,
                                             (format & W4A16_PREPACKED) != 0,
                                             static_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

int64_t w4a16_prepacked_bytes(int64_t N, int64_t K) {
  const int rc = check_format_shape(W4A16_INT4_G128 | W4A16_PREPACKED, 0, N, K, false);
  if (rc != W4A16_OK) return rc;
  return ((N + 15) / 16) * 16 * (K / 2);
}

int w4a16_prepack(const void* packed, void* out, int64_t N, int64_t K, void* stream) {
  const int rc = check_format_shape(W4A16_INT4_G128 | W4A16_PREPACKED, 0, N, K, false);
  if (rc != W4A16_OK) return rc;
  if (N == 0) return W4A16_OK;  // nothing is read or written
  if (!packed || !out) return W4A16_ERR_NULL;
  if (!aligned(packed, 16) || !aligned(out, 16)) return W4A16_ERR_ALIGN;
  // the output must not overlap the input (the copy gathers across rows)
  const uintptr_t p0 = (uintptr_t)packed, o0 = (uintptr_t)out;
  const uintptr_t in_bytes = (uintptr_t)(N * (K / 2)), out_bytes = (uintptr_t)(((N + 15) / 16) * 16 * (K / 2));
  if (p0 < o0 + out_bytes && o0 < p0 + in_bytes) return W4A16_ERR_OVERLAP;
  const hipError_t e = w4a16::launch_prepack(static_cast<const uint8_t*>(packed), static_cast<uint8_t*>(out),
                                             N, K, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

}  // extern "C"
