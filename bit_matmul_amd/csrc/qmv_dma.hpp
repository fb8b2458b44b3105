// Decode GEMV, y[n] = sum_k x[k] (s[n][g] q[n][k] + b[n][g]) for one activation row,
// built around the HBM stream.
//
// A step is R = 64 / L consecutive weight rows; lane l works on row l / L of the
// step and, within it, on the 16-byte code chunks (l % L) + L*m, m < C. A lane's
// chunks are the same in every step, and the R rows of a step are one contiguous
// span of W, fetched by C loads of 1 KB per wave (the fastest HBM access shape).
//
// Each wave owns consecutive steps and keeps up to five in registers: with one or two
// steps per wave all of its loads go out first; with more, the loads of step i+4 are
// issued before step i is computed, so four steps (about 20 KB at K = 5120) are in
// flight per wave. The activations (the same for every
// row) are prepared once per workgroup in LDS and then held in registers. Loads go through buffer descriptors
// over the rows that exist: rows past N, and chunks past the end of a row, read as
// zeros (their scale and bias too, so they add nothing).
//
// Arithmetic per chunk, the affine split (all codes of a chunk share a group):
//   sum_k x_k (s q_k + b) = s * sum_k x_k q_k + b * sum_k x_k.
// 4-bit: a nibble pair masked into 0x4300 is the exact bf16 pair (128+q_j, 128+q_{j+4});
// v_dot2_f32_bf16 against the matching activation pair gives P = sum x (128 + q),
// then s*P + (b - 128 s) * sum x. 8-bit: codes convert to f32 byte by byte. 2-bit: the
// code pair (j, j+8) of a word, masked at bit 0, 2 or 4 into the bf16 pair of 128, 32 or
// 8, is that offset plus (q_j, q_{j+8}) exactly (the activation pairs come from LDS at
// each step: a 64-code chunk has 32 of them).
// Products are exact in f32 and accumulation is f32 (the decode fix of epic #1536,
// diagnosis item 3: accumulate the 4-bit GEMV in float).
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace bitmm {
namespace qmv_dma_detail {

struct Params {
  const uint16_t* x;
  const uint32_t* w;
  const uint16_t* s;
  const uint16_t* b;
  void* y;
  int N, K;
  int gshift;    // log2 of the quantization group along K (5, 6 or 7: groups of 32, 64, 128)
  int out_f32;
  int steps_per_wave;  // consecutive steps each wave owns
  int total_steps;     // ceil(N / R)
  GemvBatch bt;        // gathered rows (blockIdx.y), or none
};

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
// Launch target in waves per CU. At 16, shapes from 8192 steps on give each wave two
// steps (all of its loads issued up front: one 5 KB burst per wave at K = 5120, 4 bits)
// and smaller ones one step. Measured on one box, same session: 4-bit N = 13824
// 11.05 -> 10.30 us against a target of 32 (one step per wave), N = 5120, 8-bit, 2-bit
// and the MoE decode shapes unchanged within the box's noise. A target of 8 (four steps
// per wave at N = 13824) is slower: 10.8 us 4-bit, and earlier 17.2 against 13.6 us
// 8-bit (more arithmetic left for each wave once its codes arrive).
constexpr int kWavesPerCu = 16;

template <int BITS, int L, int C, int SPW>
struct Cfg {
  static constexpr int R = 64 / L;       // rows per step
  static constexpr int CC = 128 / BITS;  // codes per 16-byte chunk
  static constexpr int LOADS = 3 * C;    // load instructions per step (codes, scales, biases)
  // Steps in flight at once: up to 2 steps per wave every load goes out before the
  // activations are prepared (the memory pipe fills from the first cycle); beyond, at
  // most 4 steps ahead (register budget).
  static constexpr int D = SPW <= 2 ? SPW + 1 : (SPW < 5 ? SPW : 5);
  static constexpr int XCH = 64 * C;     // activation chunks held in LDS (covers L * C)
  // Activations per chunk in LDS: 4-bit 16 bf16 pairs matched to nibble pairs (64 B);
  // 8-bit 16 f32 (64 B); 2-bit 32 pairs (128 B, a chunk holds 64 codes). Stored as NPL
  // planes of 16 bytes, plane u of chunk c at (u * XCH + c) * 16, so the 64 lanes' reads
  // of one plane are contiguous.
  static constexpr int NPL = BITS == 2 ? 8 : 4;
  static constexpr int X_BYTES = NPL * XCH * 16;
  // + per-chunk activation sums (2-bit: also the offset term of the chunk, see below)
  static constexpr int NSUM = BITS == 2 ? 2 : 1;
  static constexpr int LDS_BYTES = X_BYTES + NSUM * XCH * 4;
};

// Byte offset outside every descriptor: such a load reads zeros.
constexpr uint32_t kNoChunk = 0x80000000u;

template <int BITS, int L, int C, int SPW>
__global__ __launch_bounds__(kThreads) void qmv_dma_kernel(Params p) {
  using T = Cfg<BITS, L, C, SPW>;
  __shared__ __attribute__((aligned(16))) char lds[T::LDS_BYTES];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int step0 = (blockIdx.x * kWaves + wave) * SPW;
  const bool active = step0 < p.total_steps;  // uniform per wave
  const int slast = active ? min(step0 + SPW, p.total_steps) - 1 : p.total_steps - 1;
  const int N = p.N, K = p.K;
  const int nch = K / T::CC;          // chunks per row
  const int G = K >> p.gshift;           // scales (and biases) per weight row
  const int64_t rowbytes = (int64_t)K * BITS / 8;
  const int r = lane / L;             // row of the step
  const int li = lane % L;
  const uint16_t* xq = p.x;
  const uint32_t* wq = p.w;
  const uint16_t* sq = p.s;
  const uint16_t* bq = p.b;
  void* yq = p.y;
  if (!gemv_row(p.bt, K, N, p.out_f32 != 0, xq, wq, sq, bq, yq)) {
    const int s0 = blockIdx.x * kWaves * SPW;
    zero_outputs(yq, min(s0 * T::R, N), min((s0 + kWaves * SPW) * T::R, N), p.out_f32 != 0);
    return;
  }
  wq = uniform_ptr(wq);
  sq = uniform_ptr(sq);
  bq = uniform_ptr(bq);

  // Per-lane byte offsets of the lane's chunks, relative to the step's first row.
  uint32_t coff[C], soff[C];
#pragma unroll
  for (int m = 0; m < C; ++m) {
    const int c = li + L * m;
    const bool ok = c < nch;
    coff[m] = ok ? (uint32_t)(r * rowbytes + c * 16) : kNoChunk;
    soff[m] = ok ? (uint32_t)((r * G + ((c * T::CC) >> p.gshift)) * 2) : kNoChunk;
  }
  struct Step {
    u32x4_t q[C];
    uint32_t s[C], b[C];
  };
  auto load_step = [&](int step, Step& S) {
    const int64_t row0 = (int64_t)step * T::R;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(reinterpret_cast<const char*>(wq) + row0 * rowbytes,
                                                (N - row0) * rowbytes);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(sq + row0 * G, (N - row0) * G * 2);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(bq + row0 * G, (N - row0) * G * 2);
#pragma unroll
    for (int m = 0; m < C; ++m)
      S.q[m] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, coff[m], 0, kNonTemporal));
#pragma unroll
    for (int m = 0; m < C; ++m) S.s[m] = __builtin_amdgcn_raw_buffer_load_b16(rs, soff[m], 0, 0);
#pragma unroll
    for (int m = 0; m < C; ++m) S.b[m] = __builtin_amdgcn_raw_buffer_load_b16(rb, soff[m], 0, 0);
  };

  // Activations, once per workgroup: thread t prepares chunks t, t + 256, ... into
  // LDS; each lane then copies its own C chunks into registers for the whole kernel.
  // The loads go through a descriptor over the row, so chunks past its end read as
  // zeros with no per-word select (N = 13824, K = 5120: 11.1 -> 10.1 us). They are
  // issued first, so waiting for them never waits for weight loads (loads retire in
  // order).
  constexpr int XPT = (T::XCH + kThreads - 1) / kThreads;  // chunks per thread
  constexpr int XU = T::CC / 8;                             // 16-byte activation loads per chunk
  u32x4_t xin[XPT][XU];
  {
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(uniform_ptr(xq), (int64_t)K * 2);
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const uint32_t c = threadIdx.x + j * kThreads;
#pragma unroll
      for (int u = 0; u < XU; ++u)
        xin[j][u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rx, c * (T::CC * 2) + 16 * u, 0, 0));
    }
  }

  __builtin_amdgcn_sched_barrier(0);  // activation loads first: they retire first
  // The wave's SPW steps are straight-line code: the loads of step i+D-1 go out
  // before step i is computed (past the wave's last step they repeat that step, an
  // L2 hit), so the number of loads in flight at every wait is known exactly. A
  // wave without steps loads a valid step too, to keep the prologue branch-free.
  Step ring[SPW];
#pragma unroll
  for (int i = 0; i < T::D - 1; ++i) load_step(min(step0 + i, slast), ring[i]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < XPT; ++j) {
    const int c = threadIdx.x + j * kThreads;
    if (c >= T::XCH) break;
    uint32_t raw[4 * XU];
#pragma unroll
    for (int u = 0; u < XU; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) raw[4 * u + e] = xin[j][u][e];
    uint32_t out[4 * T::NPL];
    if constexpr (BITS == 2) {
      // code word d holds codes 16 d .. 16 d + 15; the 2-bit pair (j, j+8) meets the
      // activation pair (x_{16d+j}, x_{16d+j+8}), stored as out[8 d + j]. The pairs of
      // codes j = 0, 3, 6 are read at offset 128, j = 1, 4, 7 at 32 and j = 2, 5 at 8
      // (see the arithmetic below): besides the chunk's sum, keep the offset term
      // 128 sA + 32 sB + 8 sC over those three classes of pairs.
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          out[8 * d + j] = perm_b32(raw[8 * d + 4 + j / 2], raw[8 * d + j / 2], (j & 1) ? 0x07060302u : 0x05040100u);
      float tc[3] = {0.f, 0.f, 0.f};
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int j = 0; j < 8; ++j) tc[j % 3] = dot2_bf16(out[8 * d + j], 0x3F803F80u, tc[j % 3]);
      reinterpret_cast<float*>(lds + T::X_BYTES)[c] = (tc[0] + tc[1]) + tc[2];
      reinterpret_cast<float*>(lds + T::X_BYTES + T::XCH * 4)[c] = fmaf(128.f, tc[0], fmaf(32.f, tc[1], 8.f * tc[2]));
    } else {
      float t = 0.f;
#pragma unroll
      for (int d = 0; d < 4 * XU; ++d) t = dot2_bf16(raw[d], 0x3F803F80u, t);
      reinterpret_cast<float*>(lds + T::X_BYTES)[c] = t;
    }
    if constexpr (BITS == 4) {
      // code word wd holds codes 8 wd .. 8 wd + 7; nibble pair (j, j+4) meets the
      // activation pair (x_{8wd+j}, x_{8wd+j+4}).
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const uint32_t d0 = raw[4 * wd], d1 = raw[4 * wd + 1], d2 = raw[4 * wd + 2], d3 = raw[4 * wd + 3];
        out[4 * wd + 0] = perm_b32(d2, d0, 0x05040100u);
        out[4 * wd + 1] = perm_b32(d2, d0, 0x07060302u);
        out[4 * wd + 2] = perm_b32(d3, d1, 0x05040100u);
        out[4 * wd + 3] = perm_b32(d3, d1, 0x07060302u);
      }
    } else if constexpr (BITS == 8) {
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        out[2 * d] = raw[d] << 16;             // f32 bits of the low bf16
        out[2 * d + 1] = raw[d] & 0xFFFF0000u;  // f32 bits of the high bf16
      }
    }
#pragma unroll
    for (int u = 0; u < T::NPL; ++u)
      *reinterpret_cast<u32x4_t*>(lds + (u * T::XCH + c) * 16) =
          u32x4_t{out[4 * u], out[4 * u + 1], out[4 * u + 2], out[4 * u + 3]};
  }
  __syncthreads();
  if (!active) return;
  // The lane's activation pairs stay in registers (2-bit: 32 per chunk, read from LDS
  // at each step instead).
  constexpr int XRP = BITS == 2 ? 1 : 4;
  u32x4_t xr[C][XRP];
  float sx[C], ox[C];
#pragma unroll
  for (int m = 0; m < C; ++m) {
    const int c = li + L * m;
    if constexpr (BITS != 2) {
#pragma unroll
      for (int u = 0; u < 4; ++u) xr[m][u] = *reinterpret_cast<const u32x4_t*>(lds + (u * T::XCH + c) * 16);
    }
    sx[m] = reinterpret_cast<const float*>(lds + T::X_BYTES)[c];
    ox[m] = BITS == 2 ? reinterpret_cast<const float*>(lds + T::X_BYTES + (T::NSUM - 1) * T::XCH * 4)[c] : 0.f;
  }

  const uint32_t magic = 0x43004300u;  // bf16 pair (128, 128)
  auto compute = [&](int step, const Step& S) {
    float acc = 0.f;
#pragma unroll
    for (int m = 0; m < C; ++m) {
      const float s = __uint_as_float(S.s[m] << 16);
      const float b = __uint_as_float(S.b[m] << 16);
      // One accumulator per chunk: the chains of the C chunks and of the other waves
      // hide the latency, and no partial sums are left to add (N = 5120: 5.72 -> 5.62 us).
      float P = 0.f;
      if constexpr (BITS == 2) {
        // 2-bit pair (j, j+8) of code word d, against activation pair 8 d + j (planes
        // 2d, 2d+1). A 2-bit field at bit 0, 2 or 4 of a half, ORed into 0x4300, 0x4200
        // or 0x4100 (bf16 128, 32, 8: mantissa steps 1, 1/4, 1/16), reads as the exact
        // bf16 128 + q, 32 + q or 8 + q. So the word, shifted by 0, 6 and 12, gives all
        // eight pairs with one mask each: codes j = 0, 3, 6 at offset 128, 1, 4, 7 at 32,
        // 2, 5 at 8, and P = sum x q + (the chunk's offset term ox).
        const int c = li + L * m;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const u32x4_t x0 = *reinterpret_cast<const u32x4_t*>(lds + ((2 * d) * T::XCH + c) * 16);
          const u32x4_t x1 = *reinterpret_cast<const u32x4_t*>(lds + ((2 * d + 1) * T::XCH + c) * 16);
          const uint32_t wd = S.q[m][d];
          const uint32_t w6 = wd >> 6, w12 = wd >> 12;
          constexpr uint32_t M0 = 0x00030003u, M2 = 0x000C000Cu, M4 = 0x00300030u;
          constexpr uint32_t O128 = 0x43004300u, O32 = 0x42004200u, O8 = 0x41004100u;
          P = dot2_bf16(and_or_b32(wd, M0, O128), x0[0], P);
          P = dot2_bf16(and_or_b32(wd, M2, O32), x0[1], P);
          P = dot2_bf16(and_or_b32(wd, M4, O8), x0[2], P);
          P = dot2_bf16(and_or_b32(w6, M0, O128), x0[3], P);
          P = dot2_bf16(and_or_b32(w6, M2, O32), x1[0], P);
          P = dot2_bf16(and_or_b32(w6, M4, O8), x1[1], P);
          P = dot2_bf16(and_or_b32(w12, M0, O128), x1[2], P);
          P = dot2_bf16(and_or_b32(w12, M2, O32), x1[3], P);
        }
        // s (P - ox) + b sum x
        acc = fmaf(s, P, fmaf(b, sx[m], fmaf(-s, ox[m], acc)));
      } else if constexpr (BITS == 4) {
#pragma unroll
        for (int wd = 0; wd < 4; ++wd)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            P = dot2_bf16(and_or_b32(S.q[m][wd] >> (4 * j), 0x000F000Fu, magic), xr[m][wd][j], P);
        acc = fmaf(s, P, fmaf(fmaf(-128.f, s, b), sx[m], acc));
      } else {
#pragma unroll
        for (int wd = 0; wd < 4; ++wd)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            P = fmaf(__uint_as_float(xr[m][wd][j]), (float)((S.q[m][wd] >> (8 * j)) & 0xFFu), P);
        acc = fmaf(s, P, fmaf(b, sx[m], acc));
      }
    }
    const float v = lane_group_sum<L>(acc);
    const int n = step * T::R + r;
    if (li == L - 1 && n < N) {
      if (p.out_f32)
        static_cast<float*>(yq)[n] = v;
      else
        static_cast<uint16_t*>(yq)[n] = f32_to_bf16(v);
    }
  };

#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    if (i + T::D - 1 < SPW) load_step(min(step0 + i + T::D - 1, slast), ring[i + T::D - 1]);
    if (step0 + i > slast) break;  // uniform: the wave's last step is done
    compute(step0 + i, ring[i]);
  }
}

// Chunk layout for K (0 if this kernel does not take it): lanes per row L and chunks per
// lane C. The fewest lanes per row that need at most 3 chunks each (less work per wave:
// N = 5120, K = 5120 at 4 bits 5.9 -> 5.5 us with 64 lanes x 3 chunks instead of
// 32 x 5; MoE down decode 11.3 -> 10.4 us); else C <= 5 with the fewest idle chunk
// slots, ties to more lanes per row.
inline int pick_lanes(int64_t nch) {
  for (int L : {16, 32, 64}) {
    const int64_t c = (nch + L - 1) / L;
    if (c >= 1 && c <= 3) return L;
  }
  int best = 0;
  int64_t waste = 1 << 30;
  for (int L : {64, 32, 16}) {
    const int64_t c = (nch + L - 1) / L;
    if (c < 1 || c > 5) continue;
    const int64_t w = c * L - nch;
    if (w < waste) {
      waste = w;
      best = L;
    }
  }
  return best;
}

template <int BITS, int L, int C, int SPW>
hipError_t launch(Params p, hipStream_t stream) {
  using T = Cfg<BITS, L, C, SPW>;
  p.total_steps = (p.N + T::R - 1) / T::R;
  p.steps_per_wave = SPW;
  const int waves = (p.total_steps + SPW - 1) / SPW;
  const int blocks = (waves + kWaves - 1) / kWaves;
  hipLaunchKernelGGL((qmv_dma_kernel<BITS, L, C, SPW>), dim3(blocks, gemv_grid_rows(p.bt)), dim3(kThreads), 0,
                     stream, p);
  launch_log(dim3(blocks, gemv_grid_rows(p.bt)), dim3(kThreads), T::LDS_BYTES, "qmv_dma_kernel<%d, %d, %d, %d>",
             BITS, L, C, SPW);
  return hipGetLastError();
}

// Steps per wave: the largest of 8, 4, 2, 1 that still gives every SIMD of the chip
// at least `waves_per_cu` / 4 waves (counting the steps of every gathered row).
template <int BITS, int L, int C>
hipError_t launch_spw(const Params& p, int cus, int waves_per_cu, hipStream_t stream) {
  const int64_t steps = (int64_t)((p.N + (64 / L) - 1) / (64 / L)) * gemv_grid_rows(p.bt);
  const int64_t want = (int64_t)cus * waves_per_cu;
  if (steps >= want * 8) return launch<BITS, L, C, 8>(p, stream);
  if (steps >= want * 4) return launch<BITS, L, C, 4>(p, stream);
  if (steps >= want * 2) return launch<BITS, L, C, 2>(p, stream);
  return launch<BITS, L, C, 1>(p, stream);
}

template <int BITS, int L>
hipError_t launch_c(const Params& p, int c, int cus, int wpc, hipStream_t stream) {
  switch (c) {
    case 1: return launch_spw<BITS, L, 1>(p, cus, wpc, stream);
    case 2: return launch_spw<BITS, L, 2>(p, cus, wpc, stream);
    case 3: return launch_spw<BITS, L, 3>(p, cus, wpc, stream);
    case 4: return launch_spw<BITS, L, 4>(p, cus, wpc, stream);
    default: return launch_spw<BITS, L, 5>(p, cus, wpc, stream);
  }
}

// Returns hipErrorNotSupported when K has more than 5 chunks per lane.
template <int BITS>
hipError_t launch_bits(const Params& p, int cus, int wpc, hipStream_t stream) {
  const int64_t nch = (int64_t)p.K * BITS / 128;
  const int L = pick_lanes(nch);
  if (L == 0) return hipErrorNotSupported;
  const int c = (int)((nch + L - 1) / L);
  if (wpc <= 0) wpc = kWavesPerCu;
  if (L == 64) return launch_c<BITS, 64>(p, c, cus, wpc, stream);
  if (L == 32) return launch_c<BITS, 32>(p, c, cus, wpc, stream);
  return launch_c<BITS, 16>(p, c, cus, wpc, stream);
}

}  // namespace qmv_dma_detail

extern template hipError_t qmv_dma_detail::launch_bits<2>(const qmv_dma_detail::Params&, int, int, hipStream_t);
extern template hipError_t qmv_dma_detail::launch_bits<4>(const qmv_dma_detail::Params&, int, int, hipStream_t);
extern template hipError_t qmv_dma_detail::launch_bits<8>(const qmv_dma_detail::Params&, int, int, hipStream_t);

}  // namespace bitmm
