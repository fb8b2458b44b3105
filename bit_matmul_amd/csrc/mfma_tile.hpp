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

#include <type_traits>

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
  //
  // Pipeline: weight chunks are requested two K steps ahead (their HBM latency is
  // longer than one step of MFMAs); the x tile one step ahead, into the other LDS
  // buffer. Loads are branch-free (out-of-range rows and k re-read valid memory and
  // are zeroed by a select) and scales/biases stay raw bf16 until use, so nothing
  // forces a wait on the loads before the step's MFMAs are issued.
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

    // x tile pieces owned by this thread (row r, 16-byte column c of the step).
    u32x4_t xs[XPER];
    auto load_x = [&](int step) {
#pragma unroll
      for (int i = 0; i < XPER; ++i) {
        const int id = min(i * THREADS + tid, XPIECES - 1);
        const int r = min(id / PIECES_PER_ROW, rows - 1);
        const int k = min(step * KSTEP + (id % PIECES_PER_ROW) * 8, K - 8);
        xs[i] = load_u128(x_rows + (int64_t)r * K + k);
      }
    };
    auto store_x = [&](int buf, int step) {
#pragma unroll
      for (int i = 0; i < XPER; ++i) {
        const int id = i * THREADS + tid;
        if (id < XPIECES) {
          const int r = id / PIECES_PER_ROW;
          const int c = id % PIECES_PER_ROW;
          const bool ok = r < rows && step * KSTEP + c * 8 < K;
          *reinterpret_cast<u32x4_t*>(lds + buf * BUF + r * PITCH + c * 16) =
              ok ? xs[i] : u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    };

    // Weight prefetch ring, two steps deep (slot = step & 1).
    u32x4_t qc[2][NBW];
    uint16_t sr[2][NBW], br[2][NBW];
    auto load_w = [&](int step, u32x4_t (&q)[NBW], uint16_t (&s)[NBW], uint16_t (&b)[NBW]) {
      const int k = min(step * KSTEP + lj * CC, K - CC);  // past K: re-read, zeroed below
      const int g = k / kGroup;
      const int64_t off = (int64_t)k * BITS / 32 - lj * 4;
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        q[nb] = load_stream(wp[nb] + off);
        s[nb] = sp[nb][g];
        b[nb] = bp[nb][g];
      }
    };

    auto body = [&](int step, auto slot_c) {
      constexpr int slot = decltype(slot_c)::value;
      const int buf = step & 1;
      const bool kok = step * KSTEP + lj * CC < K;  // chunks past K dequantize to zero
      bf16x8_t bop[NBW][SUB];
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
        dequant(qc[slot][nb], kok ? bf16_to_f32(sr[slot][nb]) : 0.f,
                kok ? bf16_to_f32(br[slot][nb]) : 0.f, bop[nb]);
      if (step + 2 < nsteps) load_w(step + 2, qc[slot], sr[slot], br[slot]);
      const bool more = step + 1 < nsteps;
      if (more) load_x(step + 1);
      const char* ab = lds + buf * BUF + ln * PITCH + lj * CC * 2;
#pragma unroll
      for (int t = 0; t < SUB; ++t) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const bf16x8_t a = __builtin_bit_cast(
              bf16x8_t, *reinterpret_cast<const u32x4_t*>(ab + mb * 16 * PITCH + t * 16));
#pragma unroll
          for (int nb = 0; nb < NBW; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bop[nb][t], acc[mb][nb], 0, 0, 0);
        }
      }
      if (more) store_x(buf ^ 1, step + 1);
      __syncthreads();
    };

    load_w(0, qc[0], sr[0], br[0]);
    if (nsteps > 1) load_w(1, qc[1], sr[1], br[1]);
    load_x(0);
    store_x(0, 0);
    __syncthreads();

    for (int step = 0; step < nsteps; step += 2) {
      body(step, std::integral_constant<int, 0>{});
      if (step + 1 < nsteps) body(step + 1, std::integral_constant<int, 1>{});
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
