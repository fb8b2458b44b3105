// Matrix-core tile, LDS-staged form: y[rows, n0 .. n0+BN) = x[rows, :] * dequant(w)^T.
//
// Why the staging: the MFMA operand layout wants 16 weight rows per instruction,
// but a load instruction that reads 64 bytes from each of 16 rows streams from HBM
// at a fraction of the rate of one reading whole 128-byte lines. So every operand
// is fetched row-contiguously (8 rows x 128 bytes per wave instruction, 16 bytes
// per lane) and written to LDS in a swizzled layout, where the MFMA lanes read it.
//
// Workgroup: WAVES waves; wave w owns RW = 16*NBW weight rows (columns of y) and
// all BM = 16*MB activation rows of the tile.
//   x:  LDS double buffer of one group step (64 k = 128 bytes per row), filled by
//       all waves together; one barrier per group step.
//   W:  per-wave LDS double buffer of one weight step (128 bytes per row = 256
//       codes at 4 bits, 128 at 8), requested one weight step ahead; scales and
//       biases of that step ride along.
// LDS rows are 128 bytes = 8 chunks of 16; chunk c of row r is stored at chunk
// c ^ ((r >> 1) & 7), so the 16 rows an MFMA operand read touches fall on 16
// distinct 16-byte bank groups.
//
// K order (a contraction, so free): in group g, lane group j of an MFMA takes the
// codes of words 2j + t of the group (4-bit) or 8j + 4t .. of its 16-byte slice
// (8-bit) at sub-step t, and the A operand the matching 8 activations, which is
// chunk 2j + t of the activation group in both cases. w = fma(s, q, b) in f32 is
// rounded to bf16 for the MFMA.
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
  static constexpr int GPS = BITS == 4 ? 4 : 2;    // groups per weight step (128 B / row)
  static constexpr int XBUF = BM * 128;            // bytes per x buffer
  static constexpr int WBUF = RW * 128;            // bytes per weight buffer (one wave)
  static constexpr int SBUF = RW * GPS * 2;        // bytes per scale (or bias) buffer
  static constexpr int XINS = BM / 8;              // 1 KB load instructions per x step
  static constexpr int XPER = (XINS + WAVES - 1) / WAVES;  // per wave (upper bound)
  static constexpr int WINS = RW / 8;              // 1 KB load instructions per weight step
  static constexpr int SPL = (RW * GPS + 63) / 64; // scale loads per lane per step
  static constexpr int PER_WAVE = 2 * WBUF + 4 * SBUF;
  static constexpr int LDS_BYTES = 2 * XBUF + WAVES * PER_WAVE;
  static_assert(BM % 8 == 0 && RW % 8 == 0, "tile rows");

  __device__ static __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

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
    uint16_t* sb = reinterpret_cast<uint16_t*>(wv + 2 * WBUF);  // [2][RW*GPS]
    uint16_t* bb = sb + 2 * RW * GPS;                           // [2][RW*GPS]

    // ---- loaders (into registers; the LDS writes come later) ----
    // x step s (group s): instruction i covers tile rows 8i..8i+7, lane l the 16-byte
    // chunk at physical slot l % 8 of row 8i + l / 8.
    u32x4_t xr[XPER];
    auto load_x = [&](int s) {
#pragma unroll
      for (int k = 0; k < XPER; ++k) {
        const int i = min(wave + k * WAVES, XINS - 1);  // surplus slots re-read (not stored)
        const int r = i * 8 + (lane >> 3);
        const int c = swz(r, lane & 7);
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
    // Weight step S: this wave's rows, 128 bytes each; scales and biases of its GPS
    // groups.
    const int wrow0 = n0 + wave * RW;
    u32x4_t wr[WINS];
    uint16_t sr[SPL], br[SPL];
    auto load_w = [&](int S) {
#pragma unroll
      for (int i = 0; i < WINS; ++i) {
        const int r = i * 8 + (lane >> 3);
        const int c = swz(r, lane & 7);
        const int n = min(wrow0 + r, N - 1);
        const int off = min(S * 128 + c * 16, rowbytes - 16);  // last step may be partial
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
        if (e < RW * GPS) {
          sb[buf * RW * GPS + e] = sr[h];
          bb[buf * RW * GPS + e] = br[h];
        }
      }
    };

    f32x4_t acc[MB][NBW];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // ---- prologue: x step 0, weight steps 0 (stored) and 1 (in registers) ----
    load_w(0);
    load_x(0);
    store_w(0);
    store_x(0);
    if (nws > 1) load_w(1);
    __syncthreads();

    for (int s = 0; s < G; ++s) {
      const int S = s / GPS;
      const int gs = s % GPS;
      const int xbuf = s & 1;
      const int wbuf = S & 1;
      if (s + 1 < G) load_x(s + 1);

      // B operands: this lane's codes of group s for each of its column blocks.
      bf16x8_t bop[NBW][2];
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        const int r = nb * 16 + ln;
        const float scale = bf16_to_f32(sb[wbuf * RW * GPS + r * GPS + gs]);
        const float bias = bf16_to_f32(bb[wbuf * RW * GPS + r * GPS + gs]);
        const char* row = wb + wbuf * WBUF + r * 128;
        if constexpr (BITS == 4) {
          // words 2j, 2j+1 of the group: 8 bytes at byte 32 gs + 8 j of the row
          const int c = 2 * gs + (lj >> 1);
          const uint2 v = *reinterpret_cast<const uint2*>(row + swz(r, c) * 16 + (lj & 1) * 8);
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
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(row + swz(r, 4 * gs + lj) * 16);
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
      // At the first group of a weight step, request the next weight step.
      if (gs == 0 && S + 1 < nws && s > 0) load_w(S + 1);

      // A operands and MFMAs.
      const char* xrow = xb + xbuf * XBUF;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int r = mb * 16 + ln;
          const bf16x8_t a = __builtin_bit_cast(
              bf16x8_t, *reinterpret_cast<const u32x4_t*>(xrow + r * 128 + swz(r, 2 * lj + t) * 16));
#pragma unroll
          for (int nb = 0; nb < NBW; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bop[nb][t], acc[mb][nb], 0, 0, 0);
        }
      }

      // End of a weight step: the next one goes to the other weight buffer (this
      // wave alone reads it, in order, so no barrier is needed for it).
      if (gs == GPS - 1 || s + 1 == G) {
        if (S + 1 < nws) store_w((S + 1) & 1);
      }
      if (s + 1 < G) store_x(xbuf ^ 1);
      __syncthreads();
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
