// GEMV / small-M kernel: y[m][n] = sum_k x[m][k] * (s[n][g] q[n][k] + b[n][g]).
//
// Bandwidth-bound (about 3.6 flop per byte of weights at 4 bits), so the design
// is about the HBM stream: each wave owns RPW consecutive rows n of W; lane l
// owns the 16-byte code chunks l, l+64, ... of every one of those rows, so a
// wave's loads of one row cover 1 KB of contiguous memory. All CPL chunks of all
// RPW rows are requested before any arithmetic, keeping many 128-bit loads in
// flight per lane. The activation chunk a lane needs is the same for all RPW rows
// and is loaded and rearranged once.
//
// Arithmetic: the affine split of one chunk (all of its codes share a group):
//     sum_k x_k (s q_k + b) = s * sum_k x_k q_k + b * sum_k x_k.
// 4-bit: a masked nibble pair OR 0x4300 is the bf16 pair (128+q_i, 128+q_{i+4}),
// exact, so v_dot2_f32_bf16 against the matching activation pair gives
// P = sum x (128 + q) with exact products; then s*P + (b - 128 s)*sum x. 2-bit: each
// 16-bit half of a code word is spread to a nibble word first, then as 4-bit.
// 8-bit: codes convert to f32 one byte at a time and multiply f32 activations.
// Every product is exact in f32; accumulation is f32 (the pages' decode fix,
// epic #1536 diagnosis item 3: accumulate the 4-bit GEMV in float, not bf16).
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace bitmm {
namespace qmv_detail {

struct QmvParams {
  const uint16_t* x;
  const uint32_t* w;
  const uint16_t* s;
  const uint16_t* b;
  void* y;
  int N, K;
  int gshift;    // log2 of the quantization group along K (5, 6 or 7: groups of 32, 64, 128)
  int out_f32;
  GemvBatch bt;  // gathered rows (blockIdx.y, one activation row each), or none
};

constexpr int kQmvThreads = 256;
constexpr int kQmvWaves = kQmvThreads / kWave;

template <int BITS, int MR, int RPW, int CPL>
__global__ __launch_bounds__(kQmvThreads) void qmv_kernel(QmvParams p) {
  constexpr int CC = 128 / BITS;  // codes per 16-byte chunk
  constexpr int XU = CC / 8;      // 16-byte activation loads per chunk and row
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = blockIdx.x * kQmvWaves + (threadIdx.x >> 6);
  const int n0 = wave * RPW;
  const uint16_t* xg = p.x;
  const uint32_t* wg = p.w;
  const uint16_t* sg = p.s;
  const uint16_t* bg = p.b;
  void* yg = p.y;
  if (!gemv_row(p.bt, p.K, p.N, p.out_f32 != 0, xg, wg, sg, bg, yg)) {
    const int w0 = blockIdx.x * kQmvWaves * RPW;
    zero_outputs(yg, min(w0, p.N), min(w0 + kQmvWaves * RPW, p.N), p.out_f32 != 0);
    return;
  }
  if (n0 >= p.N) return;  // uniform per wave
  const int nch = p.K / CC;
  const int G = p.K >> p.gshift;  // scales (and biases) per weight row
  const int64_t wrow = (int64_t)p.K * BITS / 32;

  // Rows past N repeat the last row (loads stay in bounds); they are not stored.
  const uint32_t* wr[RPW];
  const uint16_t* sr[RPW];
  const uint16_t* br[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int n = min(n0 + r, p.N - 1);
    wr[r] = wg + (int64_t)n * wrow;
    sr[r] = sg + (int64_t)n * G;
    br[r] = bg + (int64_t)n * G;
  }

  float acc[RPW][MR];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[r][m] = 0.f;

  for (int kb = 0; kb < nch; kb += kWave * CPL) {
    // 1. Every load of this pass, with no arithmetic between them: codes of all
    //    RPW rows, their scales and biases (kept as raw bits), then activations.
    //    Chunks past the end of the row re-read the last chunk (in bounds) and are
    //    zeroed through their activations below.
    u32x4_t q[CPL][RPW];
    uint16_t sraw[CPL][RPW], braw[CPL][RPW];
    u32x4_t xr[CPL][MR][XU];
    bool ok[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = kb + i * kWave + lane;
      ok[i] = c < nch;
      const int cc = ok[i] ? c : nch - 1;
      const int g = (cc * CC) >> p.gshift;
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        q[i][r] = load_stream(wr[r] + 4 * (int64_t)cc);
        sraw[i][r] = sr[r][g];
        braw[i][r] = br[r][g];
      }
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        const uint16_t* xp = xg + (int64_t)m * p.K + (int64_t)cc * CC;
#pragma unroll
        for (int u = 0; u < XU; ++u) xr[i][m][u] = load_u128(xp + 8 * u);
      }
    }
    // Keep the compiler from pulling arithmetic (and the waits it implies) in
    // between the loads above.
    __builtin_amdgcn_sched_barrier(0);

    // 2. Arithmetic.
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
#pragma unroll
      for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int u = 0; u < XU; ++u)
          if (!ok[i]) xr[i][m][u] = u32x4_t{0u, 0u, 0u, 0u};
      if constexpr (BITS == 4 || BITS == 2) {
        // Nibble words of 8 codes each (2-bit codes are spread to nibbles first, so
        // both widths share the arithmetic). Activation pairs matching the nibble
        // pairs (j, j+4) of each word.
        constexpr int NWD = 16 / BITS;
        uint32_t xp[MR][NWD][4];
        float sx[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          float t = 0.f;
#pragma unroll
          for (int wd = 0; wd < NWD; ++wd) {
            const u32x4_t d = xr[i][m][wd];
            xp[m][wd][0] = perm_b32(d[2], d[0], 0x05040100u);  // (x0, x4)
            xp[m][wd][1] = perm_b32(d[2], d[0], 0x07060302u);  // (x1, x5)
            xp[m][wd][2] = perm_b32(d[3], d[1], 0x05040100u);  // (x2, x6)
            xp[m][wd][3] = perm_b32(d[3], d[1], 0x07060302u);  // (x3, x7)
#pragma unroll
            for (int e = 0; e < 4; ++e) t = dot2_bf16(d[e], 0x3F803F80u, t);
          }
          sx[m] = t;
        }
        const uint32_t magic = 0x43004300u;  // bf16 pair (128, 128)
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          float P[MR];
#pragma unroll
          for (int m = 0; m < MR; ++m) P[m] = 0.f;
#pragma unroll
          for (int wd = 0; wd < NWD; ++wd) {
            const uint32_t w0 = BITS == 4 ? q[i][r][wd] : spread_2bit(q[i][r][wd >> 1], wd & 1);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              // bf16 pair (128 + q_j, 128 + q_{j+4}), exact.
              const uint32_t qp = and_or_b32(w0 >> (4 * j), 0x000F000Fu, magic);
#pragma unroll
              for (int m = 0; m < MR; ++m) P[m] = dot2_bf16(qp, xp[m][wd][j], P[m]);
            }
          }
          const float s = bf16_to_f32(sraw[i][r]);
          const float cb = fmaf(-128.f, s, bf16_to_f32(braw[i][r]));
#pragma unroll
          for (int m = 0; m < MR; ++m) acc[r][m] = fmaf(s, P[m], fmaf(cb, sx[m], acc[r][m]));
        }
      } else {
        float xf[MR][16];
        float sx[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          float t = 0.f;
#pragma unroll
          for (int u = 0; u < 2; ++u) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t d = xr[i][m][u][e];
              xf[m][8 * u + 2 * e] = bf16_lo(d);
              xf[m][8 * u + 2 * e + 1] = bf16_hi(d);
              t = dot2_bf16(d, 0x3F803F80u, t);
            }
          }
          sx[m] = t;
        }
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          float P[MR];
#pragma unroll
          for (int m = 0; m < MR; ++m) P[m] = 0.f;
#pragma unroll
          for (int wd = 0; wd < 4; ++wd) {
            const uint32_t w0 = q[i][r][wd];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float qf = (float)((w0 >> (8 * j)) & 0xFFu);  // v_cvt_f32_ubyte<j>
#pragma unroll
              for (int m = 0; m < MR; ++m) P[m] = fmaf(xf[m][4 * wd + j], qf, P[m]);
            }
          }
          const float s = bf16_to_f32(sraw[i][r]);
          const float b = bf16_to_f32(braw[i][r]);
#pragma unroll
          for (int m = 0; m < MR; ++m) acc[r][m] = fmaf(s, P[m], fmaf(b, sx[m], acc[r][m]));
        }
      }
    }
  }

  // 3. Wave reductions; lane 63 holds each sum and stores it.
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const float v = wave_sum_lane63(acc[r][m]);
      const int n = n0 + r;
      if (lane == kWave - 1 && n < p.N) {
        const int64_t o = (int64_t)m * p.N + n;
        if (p.out_f32)
          static_cast<float*>(yg)[o] = v;
        else
          static_cast<uint16_t*>(yg)[o] = f32_to_bf16(v);
      }
    }
  }
}

template <int BITS, int MR, int RPW, int CPL>
hipError_t launch_one(const QmvParams& p, hipStream_t stream) {
  const int waves = (p.N + RPW - 1) / RPW;
  const int blocks = (waves + kQmvWaves - 1) / kQmvWaves;
  hipLaunchKernelGGL((qmv_kernel<BITS, MR, RPW, CPL>), dim3(blocks, gemv_grid_rows(p.bt)),
                     dim3(kQmvThreads), 0, stream, p);
  launch_log(dim3(blocks, gemv_grid_rows(p.bt)), dim3(kQmvThreads), 0, "qmv_kernel<%d, %d, %d, %d>", BITS,
             MR, RPW, CPL);
  return hipGetLastError();
}

// Rows of W per wave: more rows share one activation load; fewer rows give more
// waves (and more loads in flight) when N is small.
template <int BITS, int MR, int CPL>
hipError_t pick_rpw(const QmvParams& p, hipStream_t stream) {
  constexpr int RPW = MR <= 2 ? 4 : 2;
  return launch_one<BITS, MR, RPW, CPL>(p, stream);
}

// At most 4 chunks per lane; at 2 bits (64 activations per chunk and row) 2 for one
// row and 1 beyond (the host chooses cpl within that).
template <int BITS, int MR>
hipError_t pick_cpl(const QmvParams& p, int cpl, hipStream_t stream) {
  constexpr int CMAX = BITS == 2 ? (MR == 1 ? 2 : 1) : 4;
  if (cpl <= 1 || CMAX == 1) return pick_rpw<BITS, MR, 1>(p, stream);
  if constexpr (CMAX >= 2)
    if (cpl == 2 || CMAX == 2) return pick_rpw<BITS, MR, 2>(p, stream);
  if constexpr (CMAX >= 3)
    if (cpl == 3 || CMAX == 3) return pick_rpw<BITS, MR, 3>(p, stream);
  if constexpr (CMAX >= 4) return pick_rpw<BITS, MR, 4>(p, stream);
  return hipErrorInvalidValue;
}

template <int BITS>
hipError_t launch_bits(const QmvParams& p, int mr, int cpl, hipStream_t stream) {
  if constexpr (BITS == 2) {  // four rows per launch at 2 bits
    switch (mr) {
      case 1: return pick_cpl<BITS, 1>(p, cpl, stream);
      case 2: return pick_cpl<BITS, 2>(p, cpl, stream);
      case 3: return pick_cpl<BITS, 3>(p, cpl, stream);
      default: return pick_cpl<BITS, 4>(p, cpl, stream);
    }
  } else {
  switch (mr) {
    case 1: return pick_cpl<BITS, 1>(p, cpl, stream);
    case 2: return pick_cpl<BITS, 2>(p, cpl, stream);
    case 3: return pick_cpl<BITS, 3>(p, cpl, stream);
    case 4: return pick_cpl<BITS, 4>(p, cpl, stream);
    case 5: return pick_cpl<BITS, 5>(p, cpl, stream);
    case 6: return pick_cpl<BITS, 6>(p, cpl, stream);
    case 7: return pick_cpl<BITS, 7>(p, cpl, stream);
    default: return pick_cpl<BITS, 8>(p, cpl, stream);
  }
  }
}

}  // namespace qmv_detail

// One explicit instantiation per bit width, each in its own translation unit.
extern template hipError_t qmv_detail::launch_bits<2>(const qmv_detail::QmvParams&, int, int, hipStream_t);
extern template hipError_t qmv_detail::launch_bits<4>(const qmv_detail::QmvParams&, int, int, hipStream_t);
extern template hipError_t qmv_detail::launch_bits<8>(const qmv_detail::QmvParams&, int, int, hipStream_t);

}  // namespace bitmm
