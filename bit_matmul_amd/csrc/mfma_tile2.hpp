// Matrix-core tile, LDS-staged form: y[rows, n0 .. n0+BN) = x[rows, :] * dequant(w)^T.
//
// Why the staging: the MFMA operand layout wants 16 weight rows per instruction,
// but a load instruction that reads 64 bytes from each of 16 rows streams from HBM
// at a fraction of the rate of one reading whole 128-byte lines. So every operand
// is fetched row-contiguously (16 bytes per lane, 8 rows x 128 bytes or 4 rows x
// 256 bytes per wave instruction) and written to LDS in a swizzled layout, where
// the MFMA lanes read it.
//
// Workgroup: WAVES waves; wave w owns RW = 16*NBW weight rows (columns of y) and
// all BM = 16*MB activation rows of the tile.
//   x:  LDS double buffer of one group step (64 k = 128 bytes per row), filled by
//       all waves together; one barrier per group step.
//   W:  per-wave LDS double buffer of one weight step of 4 groups (128 bytes per
//       row at 4 bits, 256 at 8), with its scales and biases. Step S+1 is requested
//       at the first group of step S and written to LDS after its third.
//   Software pipeline: the B operands (dequantized weights) of group s+1 are
//       formed while the MFMAs of group s run.
// Chunk c (16 bytes) of LDS row r is stored at chunk c ^ ((r >> 1) & 7) (8 chunks
// per row) or c ^ (r & 15) (16 chunks per row), so the 16 rows one MFMA operand
// read touches fall on 16 distinct 16-byte bank groups.
//
// K order (a contraction, so free): in group g, lane group j of an MFMA takes the
// codes of word 2j + t of the group (4-bit) or words 4j + 2t, 4j + 2t + 1 (8-bit)
// at sub-step t, and the A operand the matching 8 activations, which is chunk
// 2j + t of the activation group in both cases. w = fma(s, q, b) in f32 is rounded
// to bf16 for the MFMA.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace bitmm {

template <int BITS, int MB, int NBW, int WAVES>
struct MmTile2 {
  static constexpr int BM = 16 * MB;
  static constexpr int RW = 16 * NBW;              // weight rows per wave
  static constexpr int BN = RW * WAVES;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int GPS = 4;                    // groups per weight step
  static constexpr int ROWB = GPS * 8 * BITS;      // weight bytes per row per step
  static constexpr int CPR = ROWB / 16;            // 16-byte chunks per row per step
  static constexpr int RPI = 64 / CPR;             // rows per load instruction
  static constexpr int XBUF = BM * 128;            // bytes per x buffer
  static constexpr int WBUF = RW * ROWB;           // bytes per weight buffer (one wave)
  static constexpr int SEL = RW * GPS;             // scale elements per step
  static constexpr int XINS = BM / 8;              // 1 KB load instructions per x step
  static constexpr int XPER = (XINS + WAVES - 1) / WAVES;
  static constexpr int WINS = RW / RPI;            // 1 KB load instructions per weight step
  static constexpr int SPL = (SEL + 63) / 64;      // scale loads per lane per step
  static constexpr int PER_WAVE = 2 * WBUF + 4 * SEL * 2;
  static constexpr int LDS_BYTES = 2 * XBUF + WAVES * PER_WAVE;
  static_assert(BM % 8 == 0 && RW % RPI == 0, "tile rows");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

  __device__ static __forceinline__ int swx(int r, int c) { return c ^ ((r >> 1) & 7); }
  __device__ static __forceinline__ int sww(int r, int c) {
    if constexpr (CPR == 8) return c ^ ((r >> 1) & 7);
    else return c ^ (r & 15);
  }

  __device__ static void run(const uint16_t* __restrict__ x_rows, int rows,
                             const uint32_t* __restrict__ w, const uint16_t* __restrict__ sc,
                             const uint16_t* __restrict__ bi, int n0, int N, int K,
                             void* __restrict__ y_rows, bool out_f32, char* lds) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ln = lane & 15;
    const int lj = lane >> 4;
    const int G = K / kGroup;
    const int rowbytes = K * BITS / 8;
    const int nws = (G + GPS - 1) / GPS;  // weight steps

    char* xb = lds;                                   // [2][XBUF]
    char* wv = lds + 2 * XBUF + wave * PER_WAVE;      // this wave's region
    char* wb = wv;                                    // [2][WBUF]
    uint16_t* sb = reinterpret_cast<uint16_t*>(wv + 2 * WBUF);  // [2][SEL]
    uint16_t* bb = sb + 2 * SEL;                                // [2][SEL]

    // ---- loaders (global -> registers; the LDS writes come later) ----
    u32x4_t xr[XPER];
    auto load_x = [&](int s) {
#pragma unroll
      for (int k = 0; k < XPER; ++k) {
        const int i = min(wave + k * WAVES, XINS - 1);  // surplus slots re-read (not stored)
        const int r = i * 8 + (lane >> 3);
        const int c = swx(r, lane & 7);
        const int rr = min(r, rows - 1);
        xr[k] = load_u128(x_rows + (int64_t)rr * K + s * kGroup + c * 8);
      }
    };
    auto store_x = [&](int buf) {
#pragma unroll
      for (int k = 0; k < XPER; ++k) {
        const int i = wave + k * WAVES;
        if (i < XINS)
          *reinterpret_cast<u32x4_t*>(xb + buf * XBUF + i * 1024 + lane * 16) = xr[k];
      }
    };
    const int wrow0 = n0 + wave * RW;
    u32x4_t wr[WINS];
    uint16_t sr[SPL], br[SPL];
    auto load_w = [&](int S) {
#pragma unroll
      for (int i = 0; i < WINS; ++i) {
        const int r = i * RPI + lane / CPR;
        const int c = sww(r, lane % CPR);
        const int n = min(wrow0 + r, N - 1);
        const int off = min(S * ROWB + c * 16, rowbytes - 16);  // last step may be partial
        wr[i] = load_stream(reinterpret_cast<const uint32_t*>(
            reinterpret_cast<const char*>(w) + (int64_t)n * rowbytes + off));
      }
#pragma unroll
      for (int h = 0; h < SPL; ++h) {
        const int e = h * 64 + lane;  // element r * GPS + gi of the step
        const int r = min(e / GPS, RW - 1);
        const int g = min(S * GPS + e % GPS, G - 1);
        const int n = min(wrow0 + r, N - 1);
        sr[h] = sc[(int64_t)n * G + g];
        br[h] = bi[(int64_t)n * G + g];
      }
    };
    auto store_w = [&](int buf) {
#pragma unroll
      for (int i = 0; i < WINS; ++i)
        *reinterpret_cast<u32x4_t*>(wb + buf * WBUF + i * 1024 + lane * 16) = wr[i];
#pragma unroll
      for (int h = 0; h < SPL; ++h) {
        const int e = h * 64 + lane;
        if (e < SEL) {
          sb[buf * SEL + e] = sr[h];
          bb[buf * SEL + e] = br[h];
        }
      }
    };

    // ---- B operands of group s from the weight buffer of its step ----
    auto dequant = [&](int s, bf16x8_t (&bop)[NBW][2]) {
      const int wbuf = (s / GPS) & 1;
      const int gs = s % GPS;
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        const int r = nb * 16 + ln;
        const float scale = bf16_to_f32(sb[wbuf * SEL + r * GPS + gs]);
        const float bias = bf16_to_f32(bb[wbuf * SEL + r * GPS + gs]);
        const char* row = wb + wbuf * WBUF + r * ROWB;
        if constexpr (BITS == 4) {
          // words 2j, 2j+1 of the group: 8 bytes at byte 32 gs + 8 j of the row
          const int c = 2 * gs + (lj >> 1);
          const uint2 v = *reinterpret_cast<const uint2*>(row + sww(r, c) * 16 + (lj & 1) * 8);
          const uint32_t wd[2] = {v.x, v.y};
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const uint32_t lo = wd[t] & 0x0F0F0F0Fu;         // codes 0,2,4,6
            const uint32_t hi = (wd[t] >> 4) & 0x0F0F0F0Fu;  // codes 1,3,5,7
            uint32_t d[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              d[e] = pack_bf16x2(fmaf(scale, (float)((lo >> (8 * e)) & 0xFFu), bias),
                                 fmaf(scale, (float)((hi >> (8 * e)) & 0xFFu), bias));
            bop[nb][t] = __builtin_bit_cast(bf16x8_t, u32x4_t{d[0], d[1], d[2], d[3]});
          }
        } else {
          // words 4j .. 4j+3 of the group: chunk 4 gs + j of the row
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(row + sww(r, 4 * gs + lj) * 16);
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            uint32_t d[4];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const uint32_t wd = v[2 * t + h];
              d[2 * h] = pack_bf16x2(fmaf(scale, (float)(wd & 0xFFu), bias),
                                     fmaf(scale, (float)((wd >> 8) & 0xFFu), bias));
              d[2 * h + 1] = pack_bf16x2(fmaf(scale, (float)((wd >> 16) & 0xFFu), bias),
                                         fmaf(scale, (float)(wd >> 24), bias));
            }
            bop[nb][t] = __builtin_bit_cast(bf16x8_t, u32x4_t{d[0], d[1], d[2], d[3]});
          }
        }
      }
    };

    f32x4_t acc[MB][NBW];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // ---- prologue: x group 0 and weight step 0 in LDS, weight step 1 in registers ----
    load_w(0);
    load_x(0);
    store_w(0);
    store_x(0);
    if (nws > 1) load_w(1);
    __syncthreads();
    bf16x8_t bop[NBW][2];
    dequant(0, bop);

    for (int s = 0; s < G; ++s) {
      const int S = s / GPS;
      const int gs = s % GPS;
      const bool more = s + 1 < G;
      if (more) load_x(s + 1);
      if (gs == 0 && s > 0 && S + 1 < nws) load_w(S + 1);
      // Weight step S+1 goes to LDS after the third group of step S, one group
      // before its first group is dequantized (this wave alone reads it).
      if (gs == GPS - 2 && S + 1 < nws) store_w((S + 1) & 1);

      // MFMAs of group s; the dequantization of group s+1 is independent of them.
      const char* xrow = xb + (s & 1) * XBUF;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int r = mb * 16 + ln;
          const bf16x8_t a = __builtin_bit_cast(
              bf16x8_t, *reinterpret_cast<const u32x4_t*>(xrow + r * 128 + swx(r, 2 * lj + t) * 16));
#pragma unroll
          for (int nb = 0; nb < NBW; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bop[nb][t], acc[mb][nb], 0, 0, 0);
        }
      }
      bf16x8_t bnext[NBW][2];
      if (more) dequant(s + 1, bnext);

      if (more) store_x((s & 1) ^ 1);
      __syncthreads();
      if (more) {
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
          bop[nb][0] = bnext[nb][0];
          bop[nb][1] = bnext[nb][1];
        }
      }
    }

    // Epilogue: lane holds rows 4*lj + i of column ln in each 16x16 block.
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      const int col = wrow0 + nb * 16 + ln;
      if (col >= N) continue;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = mb * 16 + lj * 4 + i;
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
