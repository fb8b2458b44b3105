// Measurement kernels for the benchmark's "measured ceiling" legs; not part of libbitmm.
//
//   bitmm_probe_stream_read: reads `bytes` of device memory once, in the access shape the
//     decode GEMV uses (each wave instruction reads 1 KB contiguous, every lane 16 bytes),
//     each wave issuing all U of its loads before it uses any. The achievable HBM read
//     rate for a buffer of that size is bytes / kernel time.
//   bitmm_probe_mfma: a loop of independent v_mfma_f32_32x32x16_bf16 on register
//     operands (no memory traffic), the achievable dense bf16 matrix-core rate.
//
// Each wave writes one word to `sink` so that the compiler keeps the work.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const char* __restrict__ src, int64_t bytes,
                                                          uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t base = wave * U * 1024;
  // Descriptor over the wave's span only (at most U KB): offsets past `bytes` read zeros.
  const int64_t left = bytes - base;
  const int span = (int)(left < (int64_t)U * 1024 ? (left > 0 ? left : 0) : (int64_t)U * 1024);
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src) + base, (short)0, span, 0x00020000);
  u32x4_t v[U];
#pragma unroll
  for (int u = 0; u < U; ++u)
    v[u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)(u * 1024 + lane * 16), 0, 2));
  uint32_t x = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  x ^= __shfl_xor(x, 32, 64);
  x ^= __shfl_xor(x, 16, 64);
  x ^= __shfl_xor(x, 8, 64);
  x ^= __shfl_xor(x, 4, 64);
  x ^= __shfl_xor(x, 2, 64);
  x ^= __shfl_xor(x, 1, 64);
  if (lane == 0) sink[wave] = x;
}

__global__ __launch_bounds__(256) void mfma_loop_kernel(float* __restrict__ sink, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)((lane + i) & 7));
    b[i] = (__bf16)(0.001f * (float)((lane * 3 + i) & 7));
  }
  f32x16_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
#pragma unroll 1
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float t = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) t += acc[j][lane & 15];
  if (lane == 0) sink[(int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)] = t;
}

template <int U>
hipError_t launch_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t s) {
  const int64_t waves = (bytes + U * 1024 - 1) / (U * 1024);
  const int64_t blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((stream_read_kernel<U>), dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<const char*>(src), bytes, sink);
  return hipGetLastError();
}

}  // namespace

extern "C" {

// Words `sink` must hold for a read of `bytes` with `unroll` loads per wave.
int64_t bitmm_probe_stream_read_sink_words(int64_t bytes, int unroll) {
  if (bytes < 1 || unroll < 1) return 0;
  const int64_t waves = (bytes + (int64_t)unroll * 1024 - 1) / ((int64_t)unroll * 1024);
  return (waves + 3) / 4 * 4;
}

// Returns 0 on success, 1 for an unsupported argument, 2 for a launch error.
int bitmm_probe_stream_read(const void* src, int64_t bytes, int unroll, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes < 1 || bytes > ((int64_t)1 << 40)) return 1;
  if (bytes / ((int64_t)unroll * 1024) > ((int64_t)1 << 31) - 1) return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (unroll) {
    case 2: e = launch_read<2>(src, bytes, sink, s); break;
    case 4: e = launch_read<4>(src, bytes, sink, s); break;
    case 8: e = launch_read<8>(src, bytes, sink, s); break;
    case 16: e = launch_read<16>(src, bytes, sink, s); break;
    default: return 1;
  }
  return e == hipSuccess ? 0 : 2;
}

// `waves` waves (a multiple of 4) each run `iters` x 8 MFMAs of 32x32x16 bf16 (32768 flops
// each); `sink` holds one float per wave.
int bitmm_probe_mfma(float* sink, int waves, int iters, void* stream) {
  if (!sink || waves < 4 || waves % 4 != 0 || iters < 1) return 1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(waves / 4), dim3(256), 0, static_cast<hipStream_t>(stream), sink,
                     iters);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
