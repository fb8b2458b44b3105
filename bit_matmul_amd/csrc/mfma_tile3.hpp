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
// 16-byte chunk 2j + t of the group's activation row. w = s q + b in f32 (one
// fused multiply-add on an exact f16 form of the code, see read_raw), rounded to
// bf16 for the MFMA.
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
    // Codes as exact f16 values: a code field masked into 0x6400 (1024.0) reads as
    // 1024 + q when it sits in bits 0..3 (or 0..7 at 8 bits) of a 16-bit half and as
    // 1024 + 16q in bits 4..7, so w = s q + b is one v_fma_mix_f32 per code:
    //   s * (1024 + q) + (b - 1024 s)   or   (s / 16) * (1024 + 16 q) + (b - 64 s).
    // Raw inputs of half t of group g for column block nb: four registers of packed
    // f16 code values and the affine constants, from the weight buffer of the
    // group's step.
    struct Raw {
      uint32_t m[4];       // 4-bit: (q0,q4) (q1,q5) (q2,q6) (q3,q7); 8-bit: (q0,q2) (q1,q3) (q4,q6) (q5,q7)
      float s, b0, s16, b1;
    };
    auto read_raw = [&](int g, int t, int nb, Raw& raw) {
      const int buf = (g / GPS) % 3;
      const int gs = g % GPS;
      const char* wbuf = wb + buf * WB;
      const uint32_t* sbuf = reinterpret_cast<const uint32_t*>(sb) + buf * 2 * SB;
      const int r = (wn * NBW + nb) * 16 + ln;
      const float scale = __uint_as_float(sbuf[r * GPS + gs] << 16);
      const float bias = __uint_as_float(sbuf[SB + r * GPS + gs] << 16);
      raw.s = scale;
      raw.b0 = fmaf(-1024.f, scale, bias);
      const uint32_t magic = 0x64006400u;  // f16 pair (1024, 1024)
      if constexpr (BITS == 4) {
        // word 2j + t of the group: byte 32 gs + 8 j + 4 t of the row segment
        const uint32_t wd = *reinterpret_cast<const uint32_t*>(wbuf + loff(r, 2 * gs + (lj >> 1)) + (lj & 1) * 8 + t * 4);
        const uint32_t w8 = wd >> 8;
        raw.m[0] = and_or_b32(wd, 0x000F000Fu, magic);
        raw.m[1] = and_or_b32(wd, 0x00F000F0u, magic);
        raw.m[2] = and_or_b32(w8, 0x000F000Fu, magic);
        raw.m[3] = and_or_b32(w8, 0x00F000F0u, magic);
        raw.s16 = scale * 0.0625f;
        raw.b1 = fmaf(-64.f, scale, bias);
      } else {
        // words 4j + 2t, 4j + 2t + 1: chunk 4 gs + j, bytes 8 t .. 8 t + 7
        const uint2 v = *reinterpret_cast<const uint2*>(wbuf + loff(r, 4 * gs + lj) + t * 8);
        raw.m[0] = and_or_b32(v.x, 0x00FF00FFu, magic);
        raw.m[1] = and_or_b32(v.x >> 8, 0x00FF00FFu, magic);
        raw.m[2] = and_or_b32(v.y, 0x00FF00FFu, magic);
        raw.m[3] = and_or_b32(v.y >> 8, 0x00FF00FFu, magic);
        raw.s16 = scale;
        raw.b1 = raw.b0;
      }
    };
    // Packed bf16 pair e (k-slots 2e, 2e+1 of the lane's 8, codes 2e and 2e+1 of the
    // lane's 8 in K order) of a B operand; `m0`, `m1` are the two packed-code
    // registers it draws on.
    auto pair = [&](const Raw& raw, int e, uint32_t m0, uint32_t m1) -> uint32_t {
      float lo, hi;
      if constexpr (BITS == 4) {
        // codes 2e', 2e'+1 for e' = e & 1 come from m[2e'] (plain) and m[2e'+1] (x16),
        // in their low halves for e < 2 and their high halves (codes + 4) otherwise
        if (e < 2) {
          lo = fma_mix_f16<0>(raw.s, m0, raw.b0);
          hi = fma_mix_f16<0>(raw.s16, m1, raw.b1);
        } else {
          lo = fma_mix_f16<1>(raw.s, m0, raw.b0);
          hi = fma_mix_f16<1>(raw.s16, m1, raw.b1);
        }
      } else {
        // codes 2e, 2e+1: low (e even) or high (e odd) halves of m[2(e>>1)], m[2(e>>1)+1]
        if ((e & 1) == 0) {
          lo = fma_mix_f16<0>(raw.s, m0, raw.b0);
          hi = fma_mix_f16<0>(raw.s, m1, raw.b0);
        } else {
          lo = fma_mix_f16<1>(raw.s, m0, raw.b0);
          hi = fma_mix_f16<1>(raw.s, m1, raw.b0);
        }
      }
      return pack_bf16x2(lo, hi);
    };
    // Which packed-code registers pair e uses.
    auto pair_regs = [](int e) -> int {  // index of the first register; the second is +1
      if constexpr (BITS == 4) return 2 * (e & 1);
      else return 2 * (e >> 1);
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
                    bf16x8_t (&bnew)[NBW], auto&& extra) {
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
        extra(i);  // other work placed in this piece (copies for later iterations)
        // pairs p with first MFMA slot >= 2 (the raw reads have landed by then)
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const int slot = NM > 2 ? 2 + p * (NM - 2) / NP : NM - 1;
          if (slot == i) {
            // The empty asm statements keep the pair's arithmetic inside this piece.
            const Raw& r = raw[p / 4];
            uint32_t m0 = r.m[pair_regs(p % 4)], m1 = r.m[pair_regs(p % 4) + 1];
            asm volatile("" : "+v"(m0), "+v"(m1));
            d[p / 4][p % 4] = pair(r, p % 4, m0, m1);
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
      uint32_t d4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) d4[e] = pair(raw, e, raw.m[pair_regs(e)], raw.m[pair_regs(e) + 1]);
      b0[nb] = __builtin_bit_cast(bf16x8_t, u32x4_t{d4[0], d4[1], d4[2], d4[3]});
    }

#pragma unroll 1
    for (int s = 0; s < G; ++s) {
      const int S = s / GPS;
      const int gn = min(s + 1, G - 1);
      // Copies for later iterations: x of group s+1 into the other x buffer, part
      // s % GPS of weight step S+2 into the third weight buffer. Neither buffer is
      // read in this iteration.
      // Their descriptors are formed here; the copy instructions themselves are
      // spread over the MFMA pieces of half 0, x first (the in-order wait below
      // relies on the weight-part copies being the last ones issued).
      static_assert(kPartCopies <= 63, "vmcnt range");
      const __amdgpu_buffer_rsrc_t rx = make_rsrc(x_rows + (int64_t)gn * kGroup, (int64_t)rows * K * 2 - gn * 128);
      char* xdst = xb + ((s + 1) & 1) * XB;
      const int Sp = min(S + 2, nws - 1);
      const int pp = s % GPS;
      char* wdst = wb + ((S + 2) % 3) * WB;
      char* sdst = sb + ((S + 2) % 3) * 2 * SB * 4;
      const int64_t row0 = (int64_t)n0 + pp * PROWS;
      const __amdgpu_buffer_rsrc_t rw = make_rsrc(reinterpret_cast<const char*>(w) + row0 * rowbytes + Sp * 128,
                                                  (N - row0) * rowbytes - Sp * 128);
      constexpr int NCOPY = XC + WC + SC;
      constexpr int NM0 = MB * NBW;  // pieces of half 0
      auto copies = [&](int i) {
#pragma unroll
        for (int c = 0; c < NCOPY; ++c) {
          if (c * NM0 / NCOPY != i) continue;
          if (c < XC) {
            const int I = wave + c * WAVES;
            if (XI % WAVES == 0 || I < XI) dma<16>(rx, xoff[c], xdst + I * 1024);
          } else if (c < XC + WC) {
            const int j = wave + (c - XC) * WAVES;
            if (WI % WAVES == 0 || j < WI) dma<16>(rw, woff[c - XC], wdst + (pp * WI + j) * 1024);
          } else {
            const int k = c - XC - WC;
            const int j = wave + k * WAVES;
            if (SI % WAVES == 0 || j < SI) {
              const int which = j / (SI / 2);  // 0 scales, 1 biases (uniform per wave)
              const __amdgpu_buffer_rsrc_t rs = make_rsrc((which ? bi : sc) + row0 * G + Sp * GPS,
                                                          ((N - row0) * G - Sp * GPS) * 2);
              dma<2>(rs, soff[k], sdst + (which * SB + pp * PROWS * GPS + (j % (SI / 2)) * 64) * 4);
            }
          }
        }
      };
      const char* xbuf = xb + (s & 1) * XB;
      // Half 0 of group s while half 1 of group s is dequantized; then half 1 of
      // group s while half 0 of group s+1 is (its weight step, S or S+1, is complete).
      half(xbuf, 0, b0, s, 1, b1, copies);
      half(xbuf, 1, b1, gn, 0, b0, [](int) {});
      // Wait for this iteration's x copies and everything issued before them; the
      // weight-part copies just issued may stay in flight for one more iteration
      // (they are first read two groups or more later). Loads retire in order.
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kPartCopies) : "memory");
      barrier_no_fence();
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
