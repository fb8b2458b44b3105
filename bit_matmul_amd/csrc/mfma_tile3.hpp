// Matrix-core tile: y[rows, n0 .. n0+BN) = x[rows, :] * dequant(w)^T, one 64-wide
// quantization group per iteration.
//
// Workgroup of WM x WN waves. Wave (wm, wn) owns activation rows wm*16*MB .. +16*MB
// and weight rows (columns of y) n0 + wn*16*NBW .. +16*NBW.
//
// Operand staging, all row-contiguous from HBM (16 bytes per lane, whole 128-byte
// row segments), then through LDS:
//   x  double buffer of one group (BM rows x 128 bytes). Group s+1 is fetched
//      while group s is multiplied.
//   W  three buffers of one weight step: 128 bytes of every weight row, i.e. GPS =
//      4 groups at 4 bits or 2 at 8 bits, plus that step's scales and biases. The
//      step two ahead of the current one is fetched in GPS parts of BN/GPS rows,
//      one part per group, so every iteration does the same work and the loop body
//      has no branch; when a step is first needed it has been complete for a
//      whole iteration.
// The B operands (dequantized weights) of group s+1 are formed while the MFMAs of
// group s run; one barrier per group.
//
// LDS layout of a 128-byte-row tile: rows in blocks of 16 (2 KB); row r of a block
// at (r & 7) * 256 + (r >> 3) * 128, its 16-byte chunk c at (c ^ (r & 7)) * 16.
// With it the reads of one MFMA operand (16 rows, one chunk each) and the writes of
// row-contiguous loads (8 rows x 8 chunks) are free of LDS bank conflicts on gfx950.
//
// K order within a group (a contraction, so any order that pairs x and w alike is
// exact): at sub-step t, MFMA lane group j takes 32-bit code word 2j + t of the group
// (4-bit) or words 4j + 2t, 4j + 2t + 1 (8-bit), and the matching 8 activations,
// 16-byte chunk 2j + t of the group's activation row. w = fma(s, q, b) in f32,
// rounded to bf16 for the MFMA.
#pragma once

#include "common.hpp"

namespace bitmm {

template <int BITS, int MB, int NBW, int WM, int WN>
struct MmTile3 {
  static constexpr int WAVES = WM * WN;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BM = 16 * MB * WM;
  static constexpr int BN = 16 * NBW * WN;
  static constexpr int GPS = 16 / BITS;                 // groups per 128-byte row segment
  static constexpr int PROWS = BN / GPS;                // weight rows fetched per group
  static constexpr int XB = BM * 128;                   // bytes of one x buffer
  static constexpr int WB = BN * 128;                   // bytes of one weight step
  static constexpr int SB = BN * GPS;                   // scales (or biases) per step
  static constexpr int XI = BM / 8;                     // 1 KB copies per x group
  static constexpr int WI = PROWS / 8;                  // 1 KB copies per weight part
  static constexpr int SI = 2 * PROWS * GPS / 64;       // 64-element scale/bias copies per part
  // Copies every wave issues for one weight part (codes, then scales and biases);
  // a wave may issue one more of each when WAVES does not divide the count.
  static constexpr int kPartCopies = WI / WAVES + SI / WAVES;
  static constexpr int LDS_BYTES = 2 * XB + 3 * WB + 3 * 2 * SB * 4;
  static_assert(BITS == 4 || BITS == 8, "bits");
  static_assert(PROWS % 16 == 0 && (PROWS * GPS) % 64 == 0, "weight part shape");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

  // Byte offset of 16-byte chunk c of row r in a 128-byte-row tile.
  __device__ static __forceinline__ int loff(int r, int c) {
    return (r >> 4) * 2048 + (r & 7) * 256 + ((r >> 3) & 1) * 128 + ((c ^ (r & 7)) << 4);
  }
  // Inverse for a copy: lane L of the copy into bytes [1024 I, 1024 I + 1024) carries
  // chunk dma_chunk(I, L) of row dma_row(I, L).
  __device__ static __forceinline__ int dma_row(int I, int L) {
    return (I >> 1) * 16 + ((L >> 3) & 1) * 8 + (I & 1) * 4 + (L >> 4);
  }
  __device__ static __forceinline__ int dma_chunk(int I, int L) {
    return (L & 7) ^ ((I & 1) * 4 + (L >> 4));
  }

  __device__ static void run(const uint16_t* __restrict__ x_rows_in, int rows_in,
                             const uint32_t* __restrict__ w_in, const uint16_t* __restrict__ sc_in,
                             const uint16_t* __restrict__ bi_in, int n0_in, int N, int K,
                             void* __restrict__ y_rows, bool out_f32, char* lds) {
    // The tile's coordinates are workgroup-uniform; say so, so that the buffer
    // descriptors built from them live in scalar registers.
    const uint16_t* x_rows = uniform_ptr(x_rows_in);
    const uint32_t* w = uniform_ptr(w_in);
    const uint16_t* sc = uniform_ptr(sc_in);
    const uint16_t* bi = uniform_ptr(bi_in);
    const int rows = __builtin_amdgcn_readfirstlane(rows_in);
    const int n0 = __builtin_amdgcn_readfirstlane(n0_in);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN;
    const int wn = wave % WN;
    const int ln = lane & 15;
    const int lj = lane >> 4;
    const int G = K / kGroup;
    const int rowbytes = K * BITS / 8;
    const int nws = (G + GPS - 1) / GPS;

    char* xb = lds;                                     // [2][XB]
    char* wb = lds + 2 * XB;                            // [3][WB]
    char* sb = wb + 3 * WB;                             // [3][2][SB] 4-byte slots

    // ---- HBM -> LDS copies (wave-uniform destinations) ----
    // Per-lane byte offsets are fixed for the whole K loop; the group or weight step
    // moves the (uniform) descriptor base. Rows past the tile's last valid row fall
    // outside the descriptor and read as zeros.
    constexpr int XC = (XI + WAVES - 1) / WAVES;
    constexpr int WC = (WI + WAVES - 1) / WAVES;
    constexpr int SC = (SI + WAVES - 1) / WAVES;
    uint32_t xoff[XC], woff[WC], soff[SC];
#pragma unroll
    for (int k = 0; k < XC; ++k) {
      const int I = wave + k * WAVES;
      xoff[k] = (uint32_t)(dma_row(I, lane) * K * 2 + dma_chunk(I, lane) * 16);
    }
#pragma unroll
    for (int k = 0; k < WC; ++k) {
      const int j = wave + k * WAVES;
      woff[k] = (uint32_t)(dma_row(j, lane) * rowbytes + dma_chunk(j, lane) * 16);
    }
#pragma unroll
    for (int k = 0; k < SC; ++k) {
      const int e = ((wave + k * WAVES) % (SI / 2)) * 64 + lane;  // row e / GPS, group e % GPS
      soff[k] = (uint32_t)(((e / GPS) * G + e % GPS) * 2);
    }
    auto copy_x = [&](int g, int buf) {
      const __amdgpu_buffer_rsrc_t r = make_rsrc(x_rows + (int64_t)g * kGroup, (int64_t)rows * K * 2 - g * 128);
#pragma unroll
      for (int k = 0; k < XC; ++k) {
        const int I = wave + k * WAVES;
        if (XI % WAVES == 0 || I < XI) dma<16>(r, xoff[k], xb + buf * XB + I * 1024);
      }
    };
    // Part p of weight step S: rows p*PROWS .. of the tile, bytes S*128 .. +128 of
    // each, and the step's GPS scales and biases of those rows.
    auto copy_part = [&](int S, int p, int buf) {
      const int64_t row0 = (int64_t)n0 + p * PROWS;
      const __amdgpu_buffer_rsrc_t rw = make_rsrc(reinterpret_cast<const char*>(w) + row0 * rowbytes + S * 128,
                                                  (N - row0) * rowbytes - S * 128);
#pragma unroll
      for (int k = 0; k < WC; ++k) {
        const int j = wave + k * WAVES;
        if (WI % WAVES == 0 || j < WI) dma<16>(rw, woff[k], wb + buf * WB + (p * WI + j) * 1024);
      }
#pragma unroll
      for (int k = 0; k < SC; ++k) {
        const int j = wave + k * WAVES;
        if (SI % WAVES == 0 || j < SI) {
          const int which = j / (SI / 2);  // 0 scales, 1 biases (uniform per wave)
          const __amdgpu_buffer_rsrc_t rs = make_rsrc((which ? bi : sc) + row0 * G + S * GPS,
                                                      ((N - row0) * G - S * GPS) * 2);
          dma<2>(rs, soff[k], sb + ((buf * 2 + which) * SB + p * PROWS * GPS + (j % (SI / 2)) * 64) * 4);
        }
      }
    };

    // ---- dequantization of one B operand half, in pieces ----
    // Raw inputs of half t of group g for column block nb: the code word(s), scale
    // and bias, read from the weight buffer of the group's step.
    struct Raw {
      uint32_t wd[BITS / 4];  // 4-bit: word 2j + t; 8-bit: words 4j + 2t, 4j + 2t + 1
      float scale, bias;
    };
    auto read_raw = [&](int g, int t, int nb, Raw& raw) {
      const int buf = (g / GPS) % 3;
      const int gs = g % GPS;
      const char* wbuf = wb + buf * WB;
      const uint32_t* sbuf = reinterpret_cast<const uint32_t*>(sb) + buf * 2 * SB;
      const int r = (wn * NBW + nb) * 16 + ln;
      raw.scale = __uint_as_float(sbuf[r * GPS + gs] << 16);
      raw.bias = __uint_as_float(sbuf[SB + r * GPS + gs] << 16);
      if constexpr (BITS == 4) {
        // word 2j + t of the group: byte 32 gs + 8 j + 4 t of the row segment
        raw.wd[0] = *reinterpret_cast<const uint32_t*>(wbuf + loff(r, 2 * gs + (lj >> 1)) + (lj & 1) * 8 + t * 4);
      } else {
        // words 4j + 2t, 4j + 2t + 1: chunk 4 gs + j, bytes 8 t .. 8 t + 7
        const uint2 v = *reinterpret_cast<const uint2*>(wbuf + loff(r, 4 * gs + lj) + t * 8);
        raw.wd[0] = v.x;
        raw.wd[1] = v.y;
      }
    };
    // Packed bf16 pair e (k-slots 2e, 2e+1 of the lane's 8) of a B operand.
    auto pair = [&](const Raw& raw, int e) -> uint32_t {
      uint32_t c0, c1;
      if constexpr (BITS == 4) {
        // slot 2e holds code e of the word's low nibbles, slot 2e+1 the high nibble
        c0 = (raw.wd[0] >> (8 * e)) & 0xFu;
        c1 = (raw.wd[0] >> (8 * e + 4)) & 0xFu;
      } else {
        c0 = (raw.wd[e >> 1] >> (16 * (e & 1))) & 0xFFu;
        c1 = (raw.wd[e >> 1] >> (16 * (e & 1) + 8)) & 0xFFu;
      }
      return pack_bf16x2(fmaf(raw.scale, (float)c0, raw.bias), fmaf(raw.scale, (float)c1, raw.bias));
    };

    f32x4_t acc[MB][NBW];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int xrow0 = wm * MB * 16;
    // One half (k sub-step t) of the group in xbuf: MB x NBW MFMAs with the B operand
    // bcur, while half td of group gd is dequantized into bnew. Instruction order is
    // fixed by the source: one MFMA per fenced piece, the dequantization spread over
    // the pieces, activation reads several row blocks ahead.
    auto half = [&](const char* xbuf, int t, const bf16x8_t (&bcur)[NBW], int gd, int td,
                    bf16x8_t (&bnew)[NBW]) {
      constexpr int NM = MB * NBW;   // MFMAs in the half
      constexpr int NP = NBW * 4;    // bf16 pairs to dequantize
      // activation reads run PF row blocks (at least 16 MFMAs) ahead of their use
      constexpr int PF = NBW >= 4 ? 4 : 8;
      u32x4_t av[MB];
#pragma unroll
      for (int mb = 0; mb < (PF < MB ? PF : MB); ++mb)
        av[mb] = *reinterpret_cast<const u32x4_t*>(xbuf + loff(xrow0 + mb * 16 + ln, 2 * lj + t));
      Raw raw[NBW];
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) read_raw(gd, td, nb, raw[nb]);
      uint32_t d[NBW][4];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        const int mb = i / NBW;
        const int nb = i % NBW;
        if (nb == 0 && mb + PF < MB)
          av[mb + PF] = *reinterpret_cast<const u32x4_t*>(xbuf + loff(xrow0 + (mb + PF) * 16 + ln, 2 * lj + t));
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[mb]), bcur[nb],
                                                              acc[mb][nb], 0, 0, 0);
        // pairs p with first MFMA slot >= 2 (the raw reads have landed by then)
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const int slot = NM > 2 ? 2 + p * (NM - 2) / NP : NM - 1;
          if (slot == i) {
            // The empty asm statements keep the pair's arithmetic inside this piece.
            Raw r = raw[p / 4];
            asm volatile("" : "+v"(r.wd[(p % 4) * BITS / 16]));
            d[p / 4][p % 4] = pair(r, p % 4);
            asm volatile("" : "+v"(d[p / 4][p % 4]));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
        bnew[nb] = __builtin_bit_cast(bf16x8_t, u32x4_t{d[nb][0], d[nb][1], d[nb][2], d[nb][3]});
    };

    // ---- prologue: weight steps 0 and 1, x group 0 ----
#pragma unroll 1
    for (int q = 0; q < 2 * GPS; ++q) copy_part(min(q / GPS, nws - 1), q % GPS, q / GPS);
    copy_x(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    bf16x8_t b0[NBW], b1[NBW];  // B operand halves t = 0, 1
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      Raw raw;
      read_raw(0, 0, nb, raw);
      b0[nb] = __builtin_bit_cast(bf16x8_t, u32x4_t{pair(raw, 0), pair(raw, 1), pair(raw, 2), pair(raw, 3)});
    }

#pragma unroll 1
    for (int s = 0; s < G; ++s) {
      const int S = s / GPS;
      const int gn = min(s + 1, G - 1);
      // Copies for later iterations: x of group s+1 into the other x buffer, part
      // s % GPS of weight step S+2 into the third weight buffer. Neither buffer is
      // read in this iteration.
      copy_x(gn, (s + 1) & 1);
      copy_part(min(S + 2, nws - 1), s % GPS, (S + 2) % 3);
      static_assert(kPartCopies <= 63, "vmcnt range");
      const char* xbuf = xb + (s & 1) * XB;
      // Half 0 of group s while half 1 of group s is dequantized; then half 1 of
      // group s while half 0 of group s+1 is (its weight step, S or S+1, is complete).
      half(xbuf, 0, b0, s, 1, b1);
      half(xbuf, 1, b1, gn, 0, b0);
      // Wait for this iteration's x copies and everything issued before them; the
      // weight-part copies just issued may stay in flight for one more iteration
      // (they are first read two groups or more later). Loads retire in order.
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kPartCopies) : "memory");
      __syncthreads();
    }

    // Epilogue: lane holds rows 4*lj + i of column ln in each 16x16 block.
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      const int col = n0 + (wn * NBW + nb) * 16 + ln;
      if (col >= N) continue;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = xrow0 + mb * 16 + lj * 4 + i;
          if (r < rows) {
            const int64_t o = (int64_t)r * N + col;
            if (out_f32)
              static_cast<float*>(y_rows)[o] = acc[mb][nb][i];
            else
              static_cast<uint16_t*>(y_rows)[o] = f32_to_bf16(acc[mb][nb][i]);
          }
        }
      }
    }
  }
};

}  // namespace bitmm
