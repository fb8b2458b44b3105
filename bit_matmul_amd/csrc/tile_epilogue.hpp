// Epilogue shared by the matrix-core tiles: f32 accumulators of 32x32 MFMA blocks to
// y[rows, col0 .. col0+32) of one wave, as bf16, binary16 (both rounded to nearest even)
// or f32.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace bitmm {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ __forceinline__ uint16_t f32_to_half_bits(float f, int otype) {
  return otype == kOutF16 ? f32_to_f16_bits(f) : f32_to_bf16(f);
}

// acc[mb] holds rows 32 mb .. 32 mb + 31 of the wave's 32 columns: lane (c, h) has rows
// 8 (j/4) + 4 h + j%4 of column c in element j. Tile row r goes to row perm[r] of y (RMAP)
// or row r; rows from `rows` on are not stored. `tile` is this wave's LDS scratch of
// 32 MB x 64 bytes, free for the epilogue (the caller has passed a barrier after its last
// LDS read).
template <int MB, bool RMAP>
__device__ __forceinline__ void store_tile(const f32x16_t (&acc)[MB], int rows, int col0, int N,
                                           void* __restrict__ y_rows, int otype, char* tile,
                                           const int32_t* __restrict__ perm) {
  // Offsets from an opaque lane index, so that a caller's loop does not hoist them.
  int etid = threadIdx.x;
  asm volatile("" : "+v"(etid));
  const int elane = etid & 63, elc = elane & 31, elh = elane >> 5;
  const int col = col0 + elc;
  const bool packed = otype != kOutF32 && (N % 8) == 0 &&
                      (reinterpret_cast<uintptr_t>(y_rows) & 15) == 0 && col0 + 32 <= N;  // wave-uniform
  if (packed) {
    // 16-bit values through LDS (32 MB rows x 64 bytes), then 16-byte stores of 8
    // columns each: 20 stores per 320 rows instead of 160 two-byte ones. Row r sits at
    // row slot r ^ ((r >> 2) & 1), so the two 32-lane halves of a write (rows r and r+4)
    // and the four rows of a 16-lane read hit distinct banks.
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = mb * 32 + 8 * (j >> 2) + 4 * elh + (j & 3);
        *reinterpret_cast<uint16_t*>(tile + (r ^ ((r >> 2) & 1)) * 64 + elc * 2) =
            f32_to_half_bits(acc[mb][j], otype);
      }
    }
#pragma unroll
    for (int t = 0; t < 2 * MB; ++t) {
      const int r = 16 * t + (elane >> 2);
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(tile + (r ^ ((r >> 2) & 1)) * 64 + (elane & 3) * 16);
      if (r < rows)
        *reinterpret_cast<u32x4_t*>(static_cast<char*>(y_rows) +
                                    ((int64_t)(RMAP ? perm[r] : r) * N + col0 + (elane & 3) * 8) * 2) = v;
    }
  } else if (col < N) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = mb * 32 + 8 * (j >> 2) + 4 * elh + (j & 3);
        if (r < rows) {
          const int64_t o = (int64_t)(RMAP ? perm[r] : r) * N + col;
          if (otype == kOutF32)
            static_cast<float*>(y_rows)[o] = acc[mb][j];
          else
            static_cast<uint16_t*>(y_rows)[o] = f32_to_half_bits(acc[mb][j], otype);
        }
      }
    }
  }
}

}  // namespace bitmm
