// C ABI of libbitmm (declared in include/bitmm.h): argument validation, the device
// check, and dispatch to the kernels. Validation is pure host logic: it never
// dereferences a pointer and makes no HIP call, so every error except
// BITMM_ERR_DEVICE and BITMM_ERR_LAUNCH can be produced on a machine without a GPU.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <string>

#include "bitmm.h"
#include "kernels.hpp"

namespace bitmm {

namespace {
thread_local std::string t_launches;  // this thread's kernel-choice record
}

void launch_log_begin() { t_launches.clear(); }

int device_compute_units() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return 256;
  }
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    cus = 256;
  }
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

void launch_log(dim3 grid, dim3 block, size_t lds_bytes, const char* fmt, ...) {
  char name[256];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(name, sizeof name, fmt, ap);
  va_end(ap);
  char line[384];
  snprintf(line, sizeof line, "%s grid=%ux%u block=%u lds=%zu\n", name, grid.x, grid.y, block.x, lds_bytes);
  t_launches += line;
}

}  // namespace bitmm

namespace {

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other architecture.
std::atomic<int> g_arch[kMaxDevices];

// The engine's arch checks refuse a mismatched build with a named error instead of
// an opaque load failure (issue #1538, "Baseline recorded" comment); this library is
// built for gfx950 alone and says so the same way.
bitmm_status device_check(hipStream_t) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return BITMM_ERR_DEVICE;
  }
  if (dev >= kMaxDevices) return BITMM_ERR_DEVICE;
  int known = g_arch[dev].load(std::memory_order_relaxed);
  if (known == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return BITMM_ERR_DEVICE;
    }
    known = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch[dev].store(known, std::memory_order_relaxed);
  }
  return known == 1 ? BITMM_OK : BITMM_ERR_DEVICE;
}

// Largest K of the dense calls (see validate_dense): 320 * K * 2 < 2^31.
constexpr int64_t kMaxDenseK = (int64_t)INT32_MAX / 640;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Quantization groups along K the kernels take (each 16-byte chunk of codes lies in one).
bool group_ok(int g) { return g == 32 || g == 64 || g == 128; }

// Code widths: 4 and 8 bits with any group; 2 bits (64 codes per 16-byte chunk) with
// groups of 64 and 128.
bool bits_ok(int bits, int group) { return bits == 4 || bits == 8 || (bits == 2 && group != 32); }

// Shared by qmv / qmm. Sets *empty when there is nothing to compute.
bitmm_status validate_dense(const void* x, const uint32_t* w, const void* s, const void* b,
                            const void* y, int64_t M, int64_t N, int64_t K, int bits, int group,
                            bitmm_out out, bool* empty) {
  if (!group_ok(group) || !bits_ok(bits, group)) return BITMM_ERR_UNSUPPORTED;
  if (out != BITMM_OUT_BF16 && out != BITMM_OUT_F32) return BITMM_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || K < 1 || K % group != 0 || K % 64 != 0) return BITMM_ERR_SHAPE;
  // Index arithmetic inside the kernels is 32-bit per dimension.
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return BITMM_ERR_SHAPE;
  // Byte offsets into a tile of activation rows (up to 320 rows of K bf16 values) and the
  // buffer descriptors over them are 32-bit: K * 2 * 320 must stay below 2^31.
  if (K > kMaxDenseK) return BITMM_ERR_UNSUPPORTED;
  *empty = (M == 0 || N == 0);
  if (*empty) return BITMM_OK;
  if (!x || !w || !s || !b || !y) return BITMM_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(s, 2) || !aligned(b, 2) ||
      !aligned(y, out == BITMM_OUT_F32 ? 4 : 2))
    return BITMM_ERR_ALIGN;
  return BITMM_OK;
}

}  // namespace

extern "C" {

int bitmm_abi_version(void) { return BITMM_ABI_VERSION; }

size_t bitmm_last_launches(char* buf, size_t len) {
  const std::string& s = bitmm::t_launches;
  if (buf && len > 0) {
    const size_t n = s.size() < len - 1 ? s.size() : len - 1;
    memcpy(buf, s.data(), n);
    buf[n] = '\0';
  }
  return s.size();
}

const char* bitmm_status_string(bitmm_status s) {
  switch (s) {
    case BITMM_OK: return "ok";
    case BITMM_ERR_NULL: return "a required pointer is NULL";
    case BITMM_ERR_SHAPE: return "invalid shape";
    case BITMM_ERR_UNSUPPORTED: return "unsupported bits, group size, type, layout or size";
    case BITMM_ERR_ALIGN: return "misaligned pointer";
    case BITMM_ERR_WORKSPACE: return "workspace missing or too small";
    case BITMM_ERR_DEVICE: return "no HIP device, or the current device is not gfx950";
    case BITMM_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

bitmm_status bitmm_qmv(const void* x, const uint32_t* w, const void* scales, const void* biases,
                       void* y, int64_t M, int64_t N, int64_t K, int bits, int group_size,
                       bitmm_out out, void* stream) {
  try {
    bitmm::launch_log_begin();
    bool empty = false;
    bitmm_status st = validate_dense(x, w, scales, biases, y, M, N, K, bits, group_size, out, &empty);
    if (st != BITMM_OK || empty) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if ((st = device_check(hs)) != BITMM_OK) return st;
    hipError_t e = bitmm::launch_qmv(static_cast<const uint16_t*>(x), w,
                                     static_cast<const uint16_t*>(scales),
                                     static_cast<const uint16_t*>(biases), y, M, N, K, bits,
                                     group_size, out == BITMM_OUT_F32, hs);
    return e == hipSuccess ? BITMM_OK : BITMM_ERR_LAUNCH;
  } catch (...) {
    return BITMM_ERR_LAUNCH;
  }
}

bitmm_status bitmm_qmm(const void* x, const uint32_t* w, const void* scales, const void* biases,
                       void* y, int64_t M, int64_t N, int64_t K, int bits, int group_size,
                       bitmm_out out, void* stream) {
  try {
    bitmm::launch_log_begin();
    bool empty = false;
    bitmm_status st = validate_dense(x, w, scales, biases, y, M, N, K, bits, group_size, out, &empty);
    if (st != BITMM_OK || empty) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if ((st = device_check(hs)) != BITMM_OK) return st;
    const uint16_t* xs = static_cast<const uint16_t*>(x);
    const uint16_t* ss = static_cast<const uint16_t*>(scales);
    const uint16_t* bs = static_cast<const uint16_t*>(biases);
    // M*B >= 8 selects the GEMM (the engine's routing rule); below it the GEMV kernel
    // streams W once for all rows. At M = 8 the GEMV's matrix-core form is still the
    // faster one where it takes the shape (K = 5120, N = 13824: 17.6 against 33.9 us at
    // 4 bits, 26.5 against 36.1 at 8), so it keeps those rows too.
    const bool gemv = M < 8 || (M == 8 && bitmm::qmv_mfma_takes(K, bits, M));
    hipError_t e = gemv ? bitmm::launch_qmv(xs, w, ss, bs, y, M, N, K, bits, group_size,
                                            out == BITMM_OUT_F32, hs)
                        : bitmm::launch_qmm_mfma(xs, w, ss, bs, y, M, N, K, bits, group_size,
                                                 out == BITMM_OUT_F32, hs);
    return e == hipSuccess ? BITMM_OK : BITMM_ERR_LAUNCH;
  } catch (...) {
    return BITMM_ERR_LAUNCH;
  }
}

size_t bitmm_gather_qmm_workspace_bytes(int64_t B, int64_t N, int64_t E) {
  if (B < 0 || N < 0 || E < 1 || E > INT32_MAX - 2) return 0;
  return bitmm::gather_workspace_bytes(E);
}

bitmm_status bitmm_gather_qmm(const void* x, const uint32_t* w, const void* scales,
                              const void* biases, const int32_t* expert_idx, void* y, int64_t B,
                              int64_t N, int64_t K, int64_t E, int bits, int group_size,
                              bitmm_out out, void* workspace, size_t workspace_bytes,
                              void* stream) {
  try {
    bitmm::launch_log_begin();
    if (!group_ok(group_size) || !bits_ok(bits, group_size)) return BITMM_ERR_UNSUPPORTED;
    if (out != BITMM_OUT_BF16 && out != BITMM_OUT_F32) return BITMM_ERR_UNSUPPORTED;
    if (B < 0 || N < 0 || K < 1 || E < 1 || K % group_size != 0 || K % 64 != 0) return BITMM_ERR_SHAPE;
    if (B > INT32_MAX || N > INT32_MAX || K > INT32_MAX || E > INT32_MAX - 2)
      return BITMM_ERR_SHAPE;
    if (B == 0 || N == 0) return BITMM_OK;
    if (!x || !w || !scales || !biases || !expert_idx || !y) return BITMM_ERR_NULL;
    if (!workspace || workspace_bytes < bitmm_gather_qmm_workspace_bytes(B, N, E))
      return BITMM_ERR_WORKSPACE;
    if (!aligned(x, 16) || !aligned(w, 16) || !aligned(scales, 2) || !aligned(biases, 2) ||
        !aligned(expert_idx, 4) || !aligned(workspace, 16) ||
        !aligned(y, out == BITMM_OUT_F32 ? 4 : 2))
      return BITMM_ERR_ALIGN;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    bitmm_status st = device_check(hs);
    if (st != BITMM_OK) return st;
    hipError_t e = bitmm::launch_gather_qmm(
        static_cast<const uint16_t*>(x), w, static_cast<const uint16_t*>(scales),
        static_cast<const uint16_t*>(biases), expert_idx, y, B, N, K, E, bits, group_size,
        out == BITMM_OUT_F32, workspace, hs);
    return e == hipSuccess ? BITMM_OK : BITMM_ERR_LAUNCH;
  } catch (...) {
    return BITMM_ERR_LAUNCH;
  }
}

bitmm_status bitmm_gather_qmm_noalloc(const void* x, const uint32_t* w, const void* scales,
                                      const void* biases, const int32_t* expert_idx, void* y,
                                      int64_t B, int64_t N, int64_t K, int64_t E, int bits,
                                      int group_size, bitmm_out out, uint32_t* status,
                                      void* stream) {
  try {
    bitmm::launch_log_begin();
    if (!group_ok(group_size) || !bits_ok(bits, group_size)) return BITMM_ERR_UNSUPPORTED;
    if (out != BITMM_OUT_BF16 && out != BITMM_OUT_F32) return BITMM_ERR_UNSUPPORTED;
    if (B < 0 || N < 0 || K < 1 || E < 1 || K % group_size != 0 || K % 64 != 0) return BITMM_ERR_SHAPE;
    if (B > INT32_MAX || N > INT32_MAX || K > INT32_MAX || E > INT32_MAX - 2)
      return BITMM_ERR_SHAPE;
    // The static workspace holds the status word and E + 1 offsets.
    if (E > bitmm::gather_noalloc_max_experts()) return BITMM_ERR_UNSUPPORTED;
    if (B == 0 || N == 0) return BITMM_OK;
    if (!x || !w || !scales || !biases || !expert_idx || !y) return BITMM_ERR_NULL;
    if (!aligned(x, 16) || !aligned(w, 16) || !aligned(scales, 2) || !aligned(biases, 2) ||
        !aligned(expert_idx, 4) || !aligned(status, 4) || !aligned(y, out == BITMM_OUT_F32 ? 4 : 2))
      return BITMM_ERR_ALIGN;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    bitmm_status st = device_check(hs);
    if (st != BITMM_OK) return st;
    hipError_t e = bitmm::launch_gather_qmm_noalloc(
        static_cast<const uint16_t*>(x), w, static_cast<const uint16_t*>(scales),
        static_cast<const uint16_t*>(biases), expert_idx, y, B, N, K, E, bits, group_size,
        out == BITMM_OUT_F32, status, hs);
    return e == hipSuccess ? BITMM_OK : BITMM_ERR_LAUNCH;
  } catch (...) {
    return BITMM_ERR_LAUNCH;
  }
}

size_t bitmm_gather_qmm_indexed_workspace_bytes(int64_t B, int64_t N, int64_t E) {
  if (B < 0 || N < 0 || E < 1 || E > INT32_MAX - 2 || B > INT32_MAX) return 0;
  return bitmm::gather_indexed_workspace_bytes(B, E);
}

bitmm_status bitmm_gather_qmm_indexed(const void* x, const uint32_t* w, const void* scales,
                                      const void* biases, const int32_t* token_idx,
                                      const int32_t* expert_idx, void* y, int64_t B, int64_t N,
                                      int64_t K, int64_t E, int64_t T, int bits, int group_size,
                                      bitmm_out out, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  try {
    bitmm::launch_log_begin();
    if (!group_ok(group_size) || !bits_ok(bits, group_size)) return BITMM_ERR_UNSUPPORTED;
    if (out != BITMM_OUT_BF16 && out != BITMM_OUT_F32) return BITMM_ERR_UNSUPPORTED;
    if (B < 0 || N < 0 || T < 0 || K < 1 || E < 1 || K % group_size != 0 || K % 64 != 0) return BITMM_ERR_SHAPE;
    if (B > INT32_MAX || N > INT32_MAX || K > INT32_MAX || T > INT32_MAX || E > INT32_MAX - 2)
      return BITMM_ERR_SHAPE;
    // Per-expert counters live in LDS; activation offsets are 32-bit.
    if (E > bitmm::gather_indexed_max_experts() || T * K * 2 > (int64_t)INT32_MAX)
      return BITMM_ERR_UNSUPPORTED;
    if (B == 0 || N == 0) return BITMM_OK;
    if ((T > 0 && !x) || !w || !scales || !biases || !expert_idx || !y) return BITMM_ERR_NULL;
    if (!workspace || workspace_bytes < bitmm_gather_qmm_indexed_workspace_bytes(B, N, E))
      return BITMM_ERR_WORKSPACE;
    if (!aligned(x, 16) || !aligned(w, 16) || !aligned(scales, 2) || !aligned(biases, 2) ||
        !aligned(expert_idx, 4) || !aligned(token_idx, 4) || !aligned(workspace, 16) ||
        !aligned(y, out == BITMM_OUT_F32 ? 4 : 2))
      return BITMM_ERR_ALIGN;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    bitmm_status st = device_check(hs);
    if (st != BITMM_OK) return st;
    hipError_t e = bitmm::launch_gather_qmm_indexed(
        static_cast<const uint16_t*>(x), w, static_cast<const uint16_t*>(scales),
        static_cast<const uint16_t*>(biases), token_idx, expert_idx, y, B, N, K, E, T, bits,
        group_size, out == BITMM_OUT_F32, workspace, hs);
    return e == hipSuccess ? BITMM_OK : BITMM_ERR_LAUNCH;
  } catch (...) {
    return BITMM_ERR_LAUNCH;
  }
}

bitmm_status bitmm_gather_qmv(const void* x, const uint32_t* w, const void* scales,
                              const void* biases, const int32_t* token_idx,
                              const int32_t* expert_idx, void* y, int64_t B, int64_t N, int64_t K,
                              int64_t E, int64_t T, int bits, int group_size, bitmm_out out,
                              void* stream) {
  try {
    bitmm::launch_log_begin();
    if (!group_ok(group_size) || !bits_ok(bits, group_size)) return BITMM_ERR_UNSUPPORTED;
    if (out != BITMM_OUT_BF16 && out != BITMM_OUT_F32) return BITMM_ERR_UNSUPPORTED;
    if (B < 0 || N < 0 || T < 0 || K < 1 || E < 1 || K % group_size != 0 || K % 64 != 0) return BITMM_ERR_SHAPE;
    if (B > INT32_MAX || N > INT32_MAX || K > INT32_MAX || E > INT32_MAX || T > INT32_MAX)
      return BITMM_ERR_SHAPE;
    if (B == 0 || N == 0) return BITMM_OK;
    if ((T > 0 && !x) || !w || !scales || !biases || !expert_idx || !y) return BITMM_ERR_NULL;
    if (!aligned(x, 16) || !aligned(w, 16) || !aligned(scales, 2) || !aligned(biases, 2) ||
        !aligned(expert_idx, 4) || !aligned(token_idx, 4) ||
        !aligned(y, out == BITMM_OUT_F32 ? 4 : 2))
      return BITMM_ERR_ALIGN;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    bitmm_status st = device_check(hs);
    if (st != BITMM_OK) return st;
    hipError_t e = bitmm::launch_gather_qmv(
        static_cast<const uint16_t*>(x), w, static_cast<const uint16_t*>(scales),
        static_cast<const uint16_t*>(biases), token_idx, expert_idx, y, B, N, K, E, T, bits,
        group_size, out == BITMM_OUT_F32, hs);
    return e == hipSuccess ? BITMM_OK : BITMM_ERR_LAUNCH;
  } catch (...) {
    return BITMM_ERR_LAUNCH;
  }
}

size_t bitmm_gather_mm_workspace_bytes(int64_t B, int64_t N, int64_t E) {
  if (B < 0 || N < 0 || E < 1 || E > INT32_MAX - 2 || B > INT32_MAX) return 0;
  return bitmm::gather_indexed_workspace_bytes(B, E);
}

bitmm_status bitmm_gather_mm(const void* x, const void* w, const int32_t* token_idx,
                             const int32_t* expert_idx, void* y, int64_t B, int64_t N, int64_t K,
                             int64_t E, int64_t T, bitmm_dtype dtype, bitmm_layout layout,
                             bitmm_out out, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    bitmm::launch_log_begin();
    if (dtype != BITMM_DTYPE_BF16 && dtype != BITMM_DTYPE_F16) return BITMM_ERR_UNSUPPORTED;
    if (layout != BITMM_LAYOUT_NK && layout != BITMM_LAYOUT_KN) return BITMM_ERR_UNSUPPORTED;
    if (out != BITMM_OUT_BF16 && out != BITMM_OUT_F32 && out != BITMM_OUT_F16)
      return BITMM_ERR_UNSUPPORTED;
    if (B < 0 || N < 0 || T < 0 || K < 1 || E < 1) return BITMM_ERR_SHAPE;
    if (B > INT32_MAX || N > INT32_MAX || K > INT32_MAX || T > INT32_MAX || E > INT32_MAX - 2)
      return BITMM_ERR_SHAPE;
    // The tile's k-steps are 16 wide; [K, N] rows are copied in 16-byte chunks; the
    // per-expert counters live in LDS; offsets into x and into one expert's W are 32-bit.
    if (K % 16 != 0 || (layout == BITMM_LAYOUT_KN && N % 8 != 0) ||
        E > bitmm::gather_indexed_max_experts() || T * K * 2 > (int64_t)INT32_MAX ||
        N * K * 2 > (int64_t)INT32_MAX)
      return BITMM_ERR_UNSUPPORTED;
    if (B == 0 || N == 0) return BITMM_OK;
    if ((T > 0 && !x) || !w || !expert_idx || !y) return BITMM_ERR_NULL;
    if (!workspace || workspace_bytes < bitmm_gather_mm_workspace_bytes(B, N, E))
      return BITMM_ERR_WORKSPACE;
    if (!aligned(x, 16) || !aligned(w, 16) || !aligned(expert_idx, 4) || !aligned(token_idx, 4) ||
        !aligned(workspace, 16) || !aligned(y, out == BITMM_OUT_F32 ? 4 : 2))
      return BITMM_ERR_ALIGN;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    bitmm_status st = device_check(hs);
    if (st != BITMM_OK) return st;
    const int otype = out == BITMM_OUT_F32 ? bitmm::kOutF32 : (out == BITMM_OUT_F16 ? bitmm::kOutF16 : bitmm::kOutBf16);
    hipError_t e = bitmm::launch_gather_mm(static_cast<const uint16_t*>(x),
                                           static_cast<const uint16_t*>(w), token_idx, expert_idx,
                                           y, B, N, K, E, T, (int)dtype, (int)layout, otype,
                                           workspace, hs);
    return e == hipSuccess ? BITMM_OK : BITMM_ERR_LAUNCH;
  } catch (...) {
    return BITMM_ERR_LAUNCH;
  }
}

}  // extern "C"
