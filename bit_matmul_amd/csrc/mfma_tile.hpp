// Matrix-core tile shared by the dense GEMM (qmm, M >= 8) and the expert-gathered
// GEMM: y[rows, n0 .. n0+BN) = x[rows, :] * dequant(w)^T for one block of output.
//
// Layout of one workgroup (WAVES waves, each owning NBW blocks of 16 columns and all
// BM = 16*MB rows of the tile):
//   - Activations: the x tile [BM x KSTEP] bf16 is staged through LDS, double
//     buffered, with rows padded by 16 bytes so the 16 lanes of an MFMA operand read
//     hit distinct banks.
//   - Weights never touch LDS: each lane streams 16 bytes of codes (one chunk) of one
//     weight row per K step, dequantizes them in registers, w = fma(s, q, b) in f32
//     rounded to bf16, and feeds them straight into v_mfma_f32_16x16x32_bf16 as the
//     B operand. A wave dequantizes only its own columns, so no weight is
//     dequantized twice within a workgroup.
//   - K order inside a step is free (it is a contraction): lane group j (lanes
//     16j..16j+15) takes the j-th chunk of the step's KSTEP = 4 chunks, MFMA sub-step
//     t takes codes 8t..8t+7 of each lane's chunk, and the A operand is read from the
//     LDS tile at the same k positions.
// The pages' prefill kernel ran scalar FMA tiles (epic #1536, diagnosis item 1) and
// their grouped GEMM SIMT tiles (PR #1562, "Nothing was computing wrong"); the
// matrix-core path is the MI355X replacement for both.
#pragma once

#include "common.hpp"

namespace bitmm {

template <int BITS, int MB, int NBW, int WAVES>
struct MmTile {
  static constexpr int CC = 128 / BITS;        // codes per 16-byte chunk
  static constexpr int KSTEP = 4 * CC;         // k per main-loop step
  static constexpr int SUB = CC / 8;           // MFMA sub-steps per chunk
  static constexpr int BM = 16 * MB;
  static constexpr int BN = 16 * NBW * WAVES;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int PITCH = KSTEP * 2 + 16; // bytes per LDS row
  static constexpr int BUF = BM * PITCH;       // bytes per LDS buffer
  static constexpr int LDS_BYTES = 2 * BUF;
  static constexpr int XPIECES = BM * KSTEP / 8;              // 16-byte pieces per x tile
  static constexpr int XPER = (XPIECES + THREADS - 1) / THREADS;
  static constexpr int PIECES_PER_ROW = KSTEP / 8;
  static_assert(KSTEP % kGroup == 0 || kGroup % KSTEP == 0, "step vs group");

  // Dequantize one 16-byte chunk into SUB bf16x8 B operands.
  __device__ static __forceinline__ void dequant(const u32x4_t q, float s, float b,
                                                 bf16x8_t (&out)[SUB]) {
    if constexpr (BITS == 4) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t wd = q[t];
        const uint32_t lo = wd & 0x0F0F0F0Fu;          // codes 0,2,4,6
        const uint32_t hi = (wd >> 4) & 0x0F0F0F0Fu;   // codes 1,3,5,7
        uint32_t d[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float a = fmaf(s, (float)((lo >> (8 * j)) & 0xFFu), b);
          const float c = fmaf(s, (float)((hi >> (8 * j)) & 0xFFu), b);
          d[j] = pack_bf16x2(a, c);
        }
        u32x4_t v = {d[0], d[1], d[2], d[3]};
        out[t] = __builtin_bit_cast(bf16x8_t, v);
      }
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        uint32_t d[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t wd = q[2 * t + h];
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const float a = fmaf(s, (float)((wd >> (16 * j)) & 0xFFu), b);
            const float c = fmaf(s, (float)((wd >> (16 * j + 8)) & 0xFFu), b);
            d[2 * h + j] = pack_bf16x2(a, c);
          }
        }
        u32x4_t v = {d[0], d[1], d[2], d[3]};
        out[t] = __builtin_bit_cast(bf16x8_t, v);
      }
    }
  }

  // One output tile. x_rows: first activation row of the tile (row stride K);
  // rows: valid rows (<= BM); w, s, b: the weight slab ([N, K*BITS/32], [N, K/64]);
  // y_rows: first output row (row stride N).
  __device__ static void run(const uint16_t* __restrict__ x_rows, int rows,
                             const uint32_t* __restrict__ w, const uint16_t* __restrict__ sc,
                             const uint16_t* __restrict__ bi, int n0, int N, int K,
                             void* __restrict__ y_rows, bool out_f32, char* lds) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ln = lane & 15;   // column (B, C) or row (A) inside a 16-block
    const int lj = lane >> 4;   // chunk slot inside the K step
    const int G = K / kGroup;
    const int64_t wrow = (int64_t)K * BITS / 32;
    const int nsteps = (K + KSTEP - 1) / KSTEP;  // 4-bit K may end on half a step

    // Weight rows of this lane (clamped into range; clamped columns are not stored).
    const uint32_t* wp[NBW];
    const uint16_t* sp[NBW];
    const uint16_t* bp[NBW];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      const int col = min(n0 + wave * 16 * NBW + nb * 16 + ln, N - 1);
      wp[nb] = w + (int64_t)col * wrow + lj * 4;
      sp[nb] = sc + (int64_t)col * G;
      bp[nb] = bi + (int64_t)col * G;
    }

    f32x4_t acc[MB][NBW];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // x tile pieces owned by this thread.
    u32x4_t xs[XPER];
    auto load_x = [&](int step) {
#pragma unroll
      for (int i = 0; i < XPER; ++i) {
        const int id = i * THREADS + tid;
        const int r = id / PIECES_PER_ROW;
        const int c = id % PIECES_PER_ROW;
        u32x4_t v = {0u, 0u, 0u, 0u};
        const int k = step * KSTEP + c * 8;
        if (id < XPIECES && r < rows && k < K) v = load_u128(x_rows + (int64_t)r * K + k);
        xs[i] = v;
      }
    };
    auto store_x = [&](int buf) {
#pragma unroll
      for (int i = 0; i < XPER; ++i) {
        const int id = i * THREADS + tid;
        if (id < XPIECES) {
          const int r = id / PIECES_PER_ROW;
          const int c = id % PIECES_PER_ROW;
          *reinterpret_cast<u32x4_t*>(lds + buf * BUF + r * PITCH + c * 16) = xs[i];
        }
      }
    };

    u32x4_t qc[NBW];
    float sv[NBW], bv[NBW];
    auto load_w = [&](int step) {
      const int k = step * KSTEP + lj * CC;
      const bool kok = k < K;  // chunks past K (half step) dequantize to zero
      const int g = kok ? k / kGroup : 0;
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        qc[nb] = kok ? load_stream(wp[nb] + (int64_t)step * (KSTEP * BITS / 32))
                     : u32x4_t{0u, 0u, 0u, 0u};
        sv[nb] = kok ? bf16_to_f32(sp[nb][g]) : 0.f;
        bv[nb] = kok ? bf16_to_f32(bp[nb][g]) : 0.f;
      }
    };

    load_x(0);
    load_w(0);
    store_x(0);
    __syncthreads();

    for (int step = 0; step < nsteps; ++step) {
      const int buf = step & 1;
      // Dequantize this step's weights, then prefetch the next step.
      bf16x8_t bop[NBW][SUB];
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) dequant(qc[nb], sv[nb], bv[nb], bop[nb]);
      const bool more = step + 1 < nsteps;
      if (more) {
        load_x(step + 1);
        load_w(step + 1);
      }
      const char* ab = lds + buf * BUF + ln * PITCH + lj * CC * 2;
#pragma unroll
      for (int t = 0; t < SUB; ++t) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const bf16x8_t a =
              __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(ab + mb * 16 * PITCH + t * 16));
#pragma unroll
          for (int nb = 0; nb < NBW; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bop[nb][t], acc[mb][nb], 0, 0, 0);
        }
      }
      if (more) store_x(buf ^ 1);
      __syncthreads();
    }

    // Epilogue: lane holds rows 4*lj + i of column ln in each 16x16 block.
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      const int col = n0 + wave * 16 * NBW + nb * 16 + ln;
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
