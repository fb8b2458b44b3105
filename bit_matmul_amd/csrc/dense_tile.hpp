// Matrix-core tile of the dense grouped product (gather_mm): y[perm[r], n0 .. n0+128) =
// x[row of r, :] * W^T for the r < rows gathered rows of one expert, with x and W both
// bf16 or both binary16 and no dequantization (PR #1562: the grouped GEMM that
// non-quantized MoE checkpoints reach through SwitchLinear::Regular::forward).
//
// Without a dequantization step the product is a weight stream: at the MoE prefill
// shapes each expert's W feeds only its few dozen rows, about 36 flop per byte of W,
// far below the matrix cores' ridge. So the tile is built around the copy shape:
//   * Both operands go HBM -> LDS by direct buffer loads (no registers), K in stages of
//     KS = 64 or 128: per stage a W tile of 128 columns and a BM-row activation tile,
//     NS stages in LDS, copies NS-1 stages ahead. Every copy instruction moves 1 KB
//     (4 rows x 256 bytes, or 8 x 128 for row-contiguous tiles at KS = 64).
//   * W stored [N, K] (layout 0) and the activations are row-contiguous tiles: 16-byte
//     chunk c of tile row r sits at position c ^ swz(r), so the 16 rows one MFMA
//     operand quarter reads hit distinct banks. The MFMA operands are 16-byte LDS
//     reads: lane (c, h) of k-step u reads chunk 2u + h of its row.
//   * W stored [K, N] (layout 1) arrives as KS k-rows x 128 columns; chunk c of k-row r
//     sits at position c ^ 4(r & 3). The B operand comes from transposing LDS reads
//     (ds_read_b64_tr_b16): within each 16-lane group, lane m points at k-row m/4,
//     columns 4(m%4) .. +3, and lane i receives column i at the four k-rows, which is
//     the MFMA's layout (lane (c, h): column c, k = 16u + 8h .. +7).
// Four waves, one per SIMD, each owning 32 columns and all BM = 32 MB rows; f32
// accumulation in 32x32x16 MFMAs (bf16 or f16 inputs, exact products).
// K a multiple of 16: the last stage runs (K mod KS)/16 k-steps; the bytes its copies
// bring from past K (the next row, or zeros past the tensor) are never multiplied.
#pragma once

#include <stdio.h>

#include <string>

#include "common.hpp"
#include "tile_epilogue.hpp"

namespace bitmm {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

template <int DT, int LAYOUT, int MB, int KS = 128, int NS = 3>
struct MmTileD {
  static constexpr int WAVES = 4;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BM = 32 * MB;
  static constexpr int BN = 32 * WAVES;
  static constexpr int ROWB = KS * 2;           // bytes of a row-contiguous tile row
  static constexpr int CPR = ROWB / 16;         // 16-byte chunks per such row
  static constexpr int WB = BN * KS * 2;        // W tile (either layout)
  static constexpr int XB = BM * ROWB;          // activation tile
  static constexpr int SB = WB + XB;
  static constexpr int LDS_BYTES = NS * SB;
  static constexpr int CW = WB / 1024 / WAVES;  // 1 KB copies per wave and stage
  static constexpr int CX = XB / 1024 / WAVES;
  static constexpr int C = CW + CX;
  static_assert(DT == 0 || DT == 1, "operand type");
  static_assert(KS == 64 || KS == 128, "stage depth");
  static_assert(NS >= 2, "stages");
  static_assert(LAYOUT == 0 || LAYOUT == 1, "weight layout");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(WAVES * BM * 64 <= LDS_BYTES, "epilogue scratch");
  static_assert((NS - 2) * C <= 63, "vmcnt range");

  // The template arguments as text (host side, for the kernel-choice record).
  static const char* name() {
    static const std::string s = [] {
      char b[96];
      snprintf(b, sizeof b, "MmTileD<%d, %d, %d, %d, %d>", DT, LAYOUT, MB, KS, NS);
      return std::string(b);
    }();
    return s.c_str();
  }

  __device__ static __forceinline__ f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
    if constexpr (DT == 0)
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                     __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                    __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }

  // Position of chunk c of row r of a row-contiguous tile: c ^ swz(r). 256-byte rows
  // start on the same bank, so 16 consecutive rows take 16 distinct positions; 128-byte
  // rows alternate between two bank halves, so pairs of rows share a position.
  __device__ static __forceinline__ int swz(int r) { return ROWB == 256 ? (r & 15) : ((r >> 1) & 7); }

  // x: [T, K]; tile row r (< rows) is output row perm[r] and reads activation row
  // tok[perm[r]] (perm[r] when tok is null). we: the expert's W, [N, K] or [K, N].
  __device__ static void run(const uint16_t* __restrict__ x_in, int T, const int32_t* __restrict__ perm,
                             const int32_t* __restrict__ tok, int rows_in,
                             const uint16_t* __restrict__ we_in, int n0_in, int N, int K,
                             void* __restrict__ y, int otype, char* lds) {
    const uint16_t* x = uniform_ptr(x_in);
    const uint16_t* we = uniform_ptr(we_in);
    const int rows = __builtin_amdgcn_readfirstlane(rows_in);
    const int n0 = __builtin_amdgcn_readfirstlane(n0_in);
    // Opaque lane index: keeps the per-lane offsets below inside a caller's loop.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lc = lane & 31;
    const int lh = lane >> 5;

    // Descriptors: x over [T, K]; W from column block n0 to the end of the expert's
    // slab. Layout 0: rows past N read as zeros. Layout 1: k-rows past K read as zeros;
    // columns past N read the next k-row and feed only output columns never stored.
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (int64_t)T * K * 2);
    const __amdgpu_buffer_rsrc_t rw =
        LAYOUT == 0 ? make_rsrc(we + (int64_t)n0 * K, (int64_t)(N - n0) * K * 2)
                    : make_rsrc(we + n0, ((int64_t)K * N - n0) * 2);
    // Per-lane byte offsets of the copies of stage 0; stage s adds s * (w_step, x_step).
    // A copy moves 1 KB: rows of a row-contiguous tile (ROWB bytes each), or 4 k-rows of
    // 256 bytes of a [K, N] tile; lane L carries chunk (L mod chunks per row) of its row
    // into that position, i.e. the chunk the swizzle puts there.
    uint32_t wo[CW], xo[CX];
#pragma unroll
    for (int jj = 0; jj < CW; ++jj) {
      const int j = wave + jj * WAVES;
      if constexpr (LAYOUT == 0) {
        const int r = (1024 / ROWB) * j + lane / CPR, p = lane % CPR;
        wo[jj] = (uint32_t)(r * K * 2 + ((p ^ swz(r)) << 4));
      } else {
        const int r = 4 * j + (lane >> 4), p = lane & 15;
        wo[jj] = (uint32_t)(r * N * 2 + ((p ^ (4 * (r & 3))) << 4));
      }
    }
#pragma unroll
    for (int kk = 0; kk < CX; ++kk) {
      const int r = (1024 / ROWB) * (wave + kk * WAVES) + lane / CPR, p = lane % CPR;
      int src = 0;
      if (r < rows) {
        src = perm[r];
        if (tok) src = tok[src];
      }
      xo[kk] = r < rows ? (uint32_t)(src * K * 2 + ((p ^ swz(r)) << 4)) : 0x80000000u;
    }
    const uint32_t w_step = LAYOUT == 0 ? KS * 2 : (uint32_t)KS * N * 2;
    constexpr uint32_t x_step = KS * 2;
    auto copy_stage = [&](int s, int b) {
      char* base = lds + b * SB;
      const uint32_t dw = (uint32_t)s * w_step, dx = (uint32_t)s * x_step;
#pragma unroll
      for (int jj = 0; jj < CW; ++jj) dma<16>(rw, wo[jj] + dw, base + (wave + jj * WAVES) * 1024);
#pragma unroll
      for (int kk = 0; kk < CX; ++kk) dma<16>(rx, xo[kk] + dx, base + WB + (wave + kk * WAVES) * 1024);
    };

    // Operand read offsets within a stage. Row-contiguous tiles: lane (c, h) at k-step u
    // reads chunk 2u + h of row c (plus 32 mb rows, or the wave's 32 W rows) at position
    // (2u + h) ^ swz(c) = 2u ^ q, q = h ^ swz(c) (swz(c) equals swz of those rows).
    const int q = lh ^ swz(lc);
    const int arow = lc * ROWB;
    const int brow = (32 * wave + lc) * ROWB;
    // Transposing reads (layout 1): lane m of 16-lane group g of half h points at
    // k-row 16u + 8h + 4 t2 + m/4, columns 32 wave + 16 g + 4 (m%4) .. +3.
    const int tm = lane & 15, tg = (lane >> 4) & 1;
    const int tchunk = 4 * wave + 2 * tg + ((tm & 3) >> 1);
    const int toff = (8 * lh + (tm >> 2)) * 256 + ((tchunk ^ (4 * (tm >> 2))) << 4) + 8 * (tm & 1);

    f32x16_t acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[mb][j] = 0.f;

    auto kstep = [&](const char* wsb, const char* xsb, int u) {
      const int po = (((2 * u) ^ q) << 4);
      u32x4_t bv;
      if constexpr (LAYOUT == 0) {
        bv = *reinterpret_cast<const u32x4_t*>(wsb + brow + po);
      } else {
        typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
        const char* tb = wsb + toff + u * 4096;
        const u32x2_t lo = __builtin_bit_cast(
            u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tb)));
        const u32x2_t hi = __builtin_bit_cast(
            u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tb + 1024)));
        bv = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const u32x4_t av = *reinterpret_cast<const u32x4_t*>(xsb + mb * 32 * ROWB + arow + po);
        acc[mb] = mfma(av, bv, acc[mb]);
      }
    };

    const int S = (K + KS - 1) / KS;
#pragma unroll
    for (int i = 0; i < NS - 1; ++i)
      if (i < S) copy_stage(i, i);
#pragma unroll 1
    for (int s = 0; s < S; ++s) {
      // This wave's copies of stage s have landed (those of the min(NS-2, S-1-s) stages
      // after it may still fly); after the barrier every wave's have, and every wave is
      // done with stage s-1, whose buffer the copies issued next overwrite.
      const int ahead = min(NS - 2, S - 1 - s);
      static_for<0, NS - 1>([&](auto Jc) {
        constexpr int J = decltype(Jc)::value;
        if (ahead == J) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(J * C) : "memory");
      });
      barrier_no_fence();
      if (s + NS - 1 < S) copy_stage(s + NS - 1, (s + NS - 1) % NS);
      const int b = __builtin_amdgcn_readfirstlane((s % NS) * SB);
      const char* wsb = lds + b;
      const char* xsb = lds + b + WB;
      const int nks = min(KS / 16, (K - s * KS) / 16);
      if (nks == KS / 16) {
#pragma unroll
        for (int u = 0; u < KS / 16; ++u) kstep(wsb, xsb, u);
      } else {
#pragma unroll 1
        for (int u = 0; u < nks; ++u) kstep(wsb, xsb, u);
      }
    }
    // Every LDS read has been consumed; no copy is in flight (vmcnt(0) above).
    barrier_no_fence();
    store_tile<MB, true>(acc, rows, n0 + 32 * wave, N, y, otype, lds + wave * (BM * 64), perm);
  }
};

}  // namespace bitmm
