// Small-M GEMV on the matrix cores: y[m][n] = sum_k x[m][k] (s[n][g] q[n][k] + b[n][g])
// for M <= 8 activation rows, with the weights streamed from HBM once.
//
// What limits a small-M GEMV is that every weight must meet every activation row. On
// the vector ALU that is one dot product per row and code pair, and the activations of
// all rows must sit beside each lane's codes. Here the v_mfma_f32_4x4x4_16b_bf16
// instruction does that reuse: its 16 independent 4x4x4 blocks give lane (b, i) (block
// b = lane / 4, i = lane % 4) the A element row i and the B element column i of block
// b, and it returns D[0..3][i] of its block (lane layout checked on the device). So lane
// (b, i) holds the codes of weight row i and the activations of activation row i, both
// over the same four k, and receives the four rows' partial products for its weight
// row: each lane keeps the activations of one row only, and one MFMA forms 4 x 4 x 4
// products in each of the 16 blocks. Five to eight rows take two row groups (MG = 2):
// lane (b, i) also holds activation row 4 + i, and each B operand feeds two MFMAs.
//
// Layout of the work. The 16-byte code chunks along K are split across the W waves of a
// workgroup: wave w owns chunks 16 C w .. 16 C (w + 1) - 1 and lane (b, i) the chunks
// 16 C w + b + 16 j, j < C (so one load instruction of a wave reads four weight rows x
// 256 contiguous bytes). The activations of those chunks stay in registers for the
// whole kernel. A workgroup computes SPW steps of four consecutive weight rows, and each
// wave keeps the loads of D steps in flight: those of step i + D go out as soon as step
// i has been computed and its registers are free (straight-line code, so the compiler's
// wait counts are exact). The scales and biases of the workgroup's rows, one
// contiguous span of each array, are copied into LDS at the start by a few coalesced
// direct-to-LDS loads (the lanes of one MFMA block read four different rows, so loading
// them per lane cost a third of the kernel's time). Per step the 16 blocks' partial sums of each row
// are added within each row of 16 lanes (row rotations); the four row sums of the W
// waves meet in LDS once at the end and are added in a fixed order (results do not
// depend on timing).
//
// Arithmetic, exact products and f32 accumulation (the decode fix of epic #1536,
// diagnosis item 3). A chunk lies inside one quantization group, so
//   sum_k x_k (s q_k + b) = s P + (b - o s) X,   P = sum_k x_k (o + q_k),  X = sum_k x_k.
// 4-bit: a nibble pair masked into 0x4300 is the exact bf16 pair (128 + q_j, 128 + q_{j+4})
// (o = 128); the MFMA k order within each word is (0, 4, 1, 5) and (2, 6, 3, 7), and the
// activations are permuted to match. 2-bit: each half word is spread to a nibble word
// first. 8-bit: bytes convert to f32 and pack exactly to bf16 (o = 0). Products of bf16
// values are exact in f32.
#pragma once

#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace bitmm {
namespace qmv_mfma_detail {

struct Params {
  const uint16_t* x;
  const uint32_t* w;
  const uint16_t* s;
  const uint16_t* b;
  void* y;
  int M, N, K;   // M: activation rows of this launch, 1..8
  int gshift;    // log2 of the quantization group along K (5, 6 or 7)
  int out_f32;
  // The nibble mask 0x000F000F and the bf16 pair (128, 128), 0x43004300. They come in as
  // arguments so that the compiler forms v_and_or_b32 itself (one instruction, mask in a
  // scalar register): the masked codes feed the MFMA directly, and the compiler's hazard
  // checks, which see through its own instructions but not through inline assembly,
  // must place the wait states a vector write needs before an MFMA reads it.
  uint32_t mask, magic;
};

typedef short s16x4_t __attribute__((ext_vector_type(4)));

constexpr uint32_t kNone = 0x80000000u;  // outside every descriptor: reads zeros
constexpr int kMaxWaves = 8;

template <int BITS>
struct Fmt {
  static constexpr int CC = 128 / BITS;  // codes per 16-byte chunk
  static constexpr int MF = CC / 4;      // MFMAs per chunk (four codes each)
  static constexpr int XU = CC / 8;      // 16-byte activation loads per chunk
};

// DPP row rotation by N lanes (within each row of 16).
template <int N>
__device__ __forceinline__ float rot_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x120 + N, 0xF, 0xF, false));
}

// Sum over the four lanes of each residue class mod 4 within each row of 16 lanes
// (lanes i, i + 4, i + 8, i + 12 of the row); every lane receives its class's row sum.
__device__ __forceinline__ float row_class_sum(float v) {
  v = rot_add<4>(v);
  return rot_add<8>(v);
}

// Value of lane 4 (lane / 4) + R (quad broadcast).
template <int R>
__device__ __forceinline__ float quad_get(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), R | (R << 2) | (R << 4) | (R << 6),
                                                            0xF, 0xF, false));
}

__device__ __forceinline__ f32x4_t mfma4(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f32x4_t c) {
  const u32x2_t a = {a0, a1}, b = {b0, b1};
  return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b), c,
                                                0, 0, 0);
}

// LDS bytes of the partial sums: [wave][lane row][weight row][activation row].
template <int SPW, int MG>
constexpr int part_bytes() { return kMaxWaves * 4 * 4 * SPW * 4 * MG * 4; }

// SBM: how the scales and biases reach the lanes. 1: staged in LDS by 4-byte copies (two
// values per lane; G even and both arrays 4-byte aligned); 2: staged by 2-byte copies
// (each value in the low half of a 4-byte slot); 0: 2-byte loads per lane and chunk
// (when the staged span would not fit).
template <int BITS, int C, int SPW, int D, int SBM, int MG>
__global__ __launch_bounds__(64 * kMaxWaves) void qmv_mfma_kernel(Params p) {
  static_assert(D >= 1 && D <= SPW, "steps in flight");
  static_assert(MG == 1 || MG == 2, "row groups");
  constexpr int MR = 4 * MG;  // activation rows the MFMAs cover
  using F = Fmt<BITS>;
  constexpr int CC = F::CC, MF = F::MF, XU = F::XU;
  constexpr int RW = 4 * SPW;  // weight rows of the workgroup
  constexpr int EL = SBM == 1 ? 2 : 4;  // LDS bytes per staged value
  extern __shared__ __attribute__((aligned(16))) char dsm[];
  float (*part)[4][RW][MR] = reinterpret_cast<float (*)[4][RW][MR]>(dsm);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = __builtin_amdgcn_readfirstlane(blockDim.x >> 6);
  const int blk = lane >> 2;
  const int ri = lane & 3;
  const int N = p.N, K = p.K, M = p.M;
  const int nch = K / CC;
  const int G = K >> p.gshift;
  const int64_t rowbytes = (int64_t)K * BITS / 8;
  const int n0 = blockIdx.x * 4 * SPW;
  const char* wq = reinterpret_cast<const char*>(uniform_ptr(p.w));
  const uint16_t* sq = uniform_ptr(p.s);
  const uint16_t* bq = uniform_ptr(p.b);

  // Per-lane offsets of the lane's chunks (weight row ri of each step; activation row ri).
  uint32_t coff[C], soff[C], xoff[MG][C];
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int c = wave * 16 * C + blk + 16 * j;
    const bool ok = c < nch;
    coff[j] = ok ? (uint32_t)(ri * rowbytes + c * 16) : kNone;
    soff[j] = ok ? (uint32_t)((ri * G + ((c * CC) >> p.gshift)) * 2) : kNone;
#pragma unroll
    for (int g = 0; g < MG; ++g) {
      const int r = 4 * g + ri;
      xoff[g][j] = ok && r < M ? (uint32_t)(((int64_t)r * K + (int64_t)c * CC) * 2) : kNone;
    }
  }

  // 1. Activation loads first (they retire first), then the scale and bias copies, then
  //    every code load of every step.
  u32x4_t xin[MG][C][XU];
  {
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(uniform_ptr(p.x), (int64_t)M * K * 2);
#pragma unroll
    for (int g = 0; g < MG; ++g)
#pragma unroll
      for (int j = 0; j < C; ++j)
#pragma unroll
        for (int u = 0; u < XU; ++u)
          xin[g][j][u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rx, xoff[g][j], 16 * u, 0));
  }
  // The codes (and, unstaged, the scales and biases) of D steps at a time: step t lives in
  // ring slot t % D, and the loads of step t + D go out as soon as step t is computed.
  struct Step {
    u32x4_t q[C];
    uint32_t s[C], b[C];
  };
  Step st[D];
  auto load_step = [&](int t, Step& S) {
    const int64_t row0 = n0 + 4 * t;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(wq + row0 * rowbytes, (N - row0) * rowbytes);
#pragma unroll
    for (int j = 0; j < C; ++j)
      S.q[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, coff[j], 0, kNonTemporal));
    if constexpr (SBM == 0) {
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(sq + row0 * G, (N - row0) * G * 2);
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(bq + row0 * G, (N - row0) * G * 2);
#pragma unroll
      for (int j = 0; j < C; ++j) {
        S.s[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, soff[j], 0, 0);
        S.b[j] = __builtin_amdgcn_raw_buffer_load_b16(rb, soff[j], 0, 0);
      }
    }
  };
  // Staged scales and biases: the RW * G values of each array from row n0 on (rows past N
  // read as zeros), value v of the scales at sbs + EL v, of the biases at sbb + EL v.
  const int nsb = SBM == 0 ? 0 : (RW * G * EL + 255) / 256;  // copies (256 LDS bytes) per array
  char* const sbs = dsm + part_bytes<SPW, MG>();
  char* const sbb = sbs + nsb * 256;
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (SBM != 0) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(sq + (int64_t)n0 * G, (int64_t)(N - n0) * G * 2);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(bq + (int64_t)n0 * G, (int64_t)(N - n0) * G * 2);
    for (int k = wave; k < nsb; k += nw) {
      const uint32_t vo = (uint32_t)((k * 64 + lane) * (SBM == 1 ? 4 : 2));
      if constexpr (SBM == 1) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t*)(sbs + k * 256), 4, vo, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t*)(sbb + k * 256), 4, vo, 0, 0, 0);
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t*)(sbs + k * 256), 2, vo, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t*)(sbb + k * 256), 2, vo, 0, 0, 0);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < D; ++t) load_step(t, st[t]);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (SBM != 0) {
    // The copies of every wave have landed (only the code loads, issued after them, may
    // still be in flight) and are visible to the whole workgroup after the barrier.
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(D * C) : "memory");
    barrier_no_fence();
  }
  // Scale and bias of step t, chunk slot j (a chunk past the row's end takes zeros; soff
  // is (row ri, group of the chunk) in values * 2 from the step's first row).
  auto scale_bias = [&](int t, const Step& S, int j, uint32_t& sv, uint32_t& bv) {
    if constexpr (SBM == 0) {
      sv = S.s[j];
      bv = S.b[j];
    } else {
      const bool ok = soff[j] != kNone;
      const int o = ok ? (int)(soff[j] >> 1) + 4 * t * G : 0;
      const uint32_t a = *reinterpret_cast<const uint16_t*>(sbs + o * EL);
      const uint32_t c = *reinterpret_cast<const uint16_t*>(sbb + o * EL);
      sv = ok ? a : 0u;
      bv = ok ? c : 0u;
    }
  };

  // 2. The lane's A operands (activation row ri over its chunks, in the MFMA k order of
  //    the codes) and the chunk sums X of all four activation rows.
  uint32_t av[MG][C][2 * MF];
  float xs[C][MR];
#pragma unroll
  for (int g = 0; g < MG; ++g)
#pragma unroll
    for (int j = 0; j < C; ++j) {
      uint32_t raw[4 * XU];
#pragma unroll
      for (int u = 0; u < XU; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) raw[4 * u + e] = xin[g][j][u][e];
      float t = 0.f;
#pragma unroll
      for (int d = 0; d < 4 * XU; ++d) t = dot2_bf16(raw[d], 0x3F803F80u, t);
      xs[j][4 * g + 0] = quad_get<0>(t);
      xs[j][4 * g + 1] = quad_get<1>(t);
      xs[j][4 * g + 2] = quad_get<2>(t);
      xs[j][4 * g + 3] = quad_get<3>(t);
      if constexpr (BITS == 8) {
        // word d of the codes holds k = 4 d .. 4 d + 3 in byte order: activations as loaded
#pragma unroll
        for (int d = 0; d < 4 * XU; ++d) av[g][j][d] = raw[d];
      } else {
        // nibble word wd (8 codes, k = 8 wd ..): MFMA 2 wd takes k (0, 4, 1, 5), 2 wd + 1 (2, 6, 3, 7)
#pragma unroll
        for (int wd = 0; wd < 2 * XU / 2; ++wd) {
          const uint32_t d0 = raw[4 * wd], d1 = raw[4 * wd + 1], d2 = raw[4 * wd + 2], d3 = raw[4 * wd + 3];
          av[g][j][4 * wd + 0] = perm_b32(d2, d0, 0x05040100u);
          av[g][j][4 * wd + 1] = perm_b32(d2, d0, 0x07060302u);
          av[g][j][4 * wd + 2] = perm_b32(d3, d1, 0x05040100u);
          av[g][j][4 * wd + 3] = perm_b32(d3, d1, 0x07060302u);
        }
      }
    }

  // 3. The steps, in order: products of the lane's chunks for weight row n0 + 4 t + ri
  //    and the four activation rows, the affine terms, the sum over the 16 blocks.
  // magic in a vector register (moved there once) and the mask in a scalar one: the
  // compiler then forms each mask-and-or as one v_and_or_b32.
  uint32_t magic;
  asm volatile("v_mov_b32 %0, %1" : "=v"(magic) : "s"(p.magic));
  const uint32_t kMask = p.mask;
#pragma unroll
  for (int t = 0; t < SPW; ++t) {
    Step& S = st[t % D];
    float acc[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) acc[r] = 0.f;
#pragma unroll
    for (int j = 0; j < C; ++j) {
      uint32_t sraw, braw;
      scale_bias(t, S, j, sraw, braw);
      f32x4_t d[MG];
#pragma unroll
      for (int g = 0; g < MG; ++g) d[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if constexpr (BITS == 8) {
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
          const uint32_t q = S.q[j][wd];
          const uint32_t b0 = pack_bf16x2((float)(q & 0xFFu), (float)((q >> 8) & 0xFFu));
          const uint32_t b1 = pack_bf16x2((float)((q >> 16) & 0xFFu), (float)(q >> 24));
#pragma unroll
          for (int g = 0; g < MG; ++g) d[g] = mfma4(av[g][j][2 * wd], av[g][j][2 * wd + 1], b0, b1, d[g]);
        }
      } else {
        constexpr int NWD = 16 / BITS;  // nibble words per chunk: 4 (4-bit), 8 (2-bit, spread)
#pragma unroll
        for (int wd = 0; wd < NWD; ++wd) {
          const uint32_t q = BITS == 4 ? S.q[j][wd] : spread_2bit(S.q[j][wd >> 1], wd & 1);
          const uint32_t h0 = (q & kMask) | magic;          // (q0, q4)
          const uint32_t h1 = ((q >> 4) & kMask) | magic;   // (q1, q5)
          const uint32_t h2 = ((q >> 8) & kMask) | magic;   // (q2, q6)
          const uint32_t h3 = ((q >> 12) & kMask) | magic;  // (q3, q7)
#pragma unroll
          for (int g = 0; g < MG; ++g) {
            d[g] = mfma4(av[g][j][4 * wd], av[g][j][4 * wd + 1], h0, h1, d[g]);
            d[g] = mfma4(av[g][j][4 * wd + 2], av[g][j][4 * wd + 3], h2, h3, d[g]);
          }
        }
      }
      const float sc = bf16_lo(sraw);
      const float bc = bf16_lo(braw);
      const float cb = BITS == 8 ? bc : fmaf(-128.f, sc, bc);
#pragma unroll
      for (int r = 0; r < MR; ++r) acc[r] = fmaf(sc, d[r >> 2][r & 3], fmaf(cb, xs[j][r], acc[r]));
    }
    // slot t % D is spent: the loads of step t + D go out now
    if (t + D < SPW) load_step(t + D, S);
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      const float v = row_class_sum(acc[r]);
      if ((lane & 15) < 4 && r < M) part[wave][lane >> 4][4 * t + ri][r] = v;
    }
  }

  // 4. The partial sums of the waves and lane rows, added in a fixed order, and the stores.
  __syncthreads();
  for (int e = threadIdx.x; e < 4 * SPW * M; e += blockDim.x) {
    const int row = e / M, r = e - row * M;
    float v = 0.f;
    for (int w = 0; w < nw; ++w)
#pragma unroll
      for (int q = 0; q < 4; ++q) v += part[w][q][row][r];
    const int n = n0 + row;
    if (n < N) {
      const int64_t o = (int64_t)r * N + n;
      if (p.out_f32)
        static_cast<float*>(p.y)[o] = v;
      else
        static_cast<uint16_t*>(p.y)[o] = f32_to_bf16(v);
    }
  }
}

// Chunks per lane (C) for K: the fewest that cover a row with at most kMaxWaves waves
// (0 if none does).
inline int pick_c(int64_t K, int bits) {
  const int64_t nch = K * bits / 128;
  for (int c : {1, 2, 4})
    if ((nch + 16 * c - 1) / (16 * c) <= kMaxWaves) return c;
  return 0;
}

inline bool fits(int64_t K, int bits, int64_t M) { return M >= 1 && M <= 8 && pick_c(K, bits) != 0; }

// LDS for the staged scales and biases beyond which they are loaded per lane instead.
constexpr int kMaxStageBytes = 24 * 1024;

template <int BITS, int C, int SPW, int D, int MG>
hipError_t launch(const Params& p, hipStream_t stream) {
  const int64_t nch = (int64_t)p.K * BITS / 128;
  const int nw = (int)((nch + 16 * C - 1) / (16 * C));
  const int grid = (p.N + 4 * SPW - 1) / (4 * SPW);
  const int G = p.K >> p.gshift;
  const bool wide = G % 2 == 0 && (reinterpret_cast<uintptr_t>(p.s) & 3) == 0 &&
                    (reinterpret_cast<uintptr_t>(p.b) & 3) == 0;
  const int el = wide ? 2 : 4;
  const int stage = 2 * ((4 * SPW * G * el + 255) / 256) * 256;
  const size_t lds = (size_t)part_bytes<SPW, MG>() + (stage <= kMaxStageBytes ? stage : 0);
  if (stage > kMaxStageBytes)
    hipLaunchKernelGGL((qmv_mfma_kernel<BITS, C, SPW, D, 0, MG>), dim3(grid), dim3(64 * nw), lds, stream, p);
  else if (wide)
    hipLaunchKernelGGL((qmv_mfma_kernel<BITS, C, SPW, D, 1, MG>), dim3(grid), dim3(64 * nw), lds, stream, p);
  else
    hipLaunchKernelGGL((qmv_mfma_kernel<BITS, C, SPW, D, 2, MG>), dim3(grid), dim3(64 * nw), lds, stream, p);
  launch_log(dim3(grid), dim3(64 * nw), lds, "qmv_mfma_kernel<%d, %d, %d, %d, %d, %d>", BITS, C, SPW, D,
             stage > kMaxStageBytes ? 0 : (wide ? 1 : 2), MG);
  return hipGetLastError();
}

// Steps of four weight rows per workgroup (SPW) and steps in flight per wave (D), from
// measurements at K = 5120, three activation rows (us at N = 13824 / 5120):
//   4-bit: SPW 8, D 2: 11.8 / 8.3; SPW 5, D 2: 11.9 / 6.9; SPW 4, D 4: 13.6 / 8.3;
//          SPW 16, D 2: 13.1 / 12.4; SPW 8, D 1: 12.9 / 9.8;
//   8-bit: SPW 8, D 1: 16.3 / 11.1; SPW 8, D 2: 19.9 / 10.7; SPW 5, D 2: 21.7 / 8.9.
// Two steps in flight hide the stream behind the arithmetic at 4 bits; at 8 bits one
// step (fewer registers, more waves per CU) does better once every CU has several
// workgroups. Below about ten steps per CU, workgroups of 5 steps; very small N, fewer.
template <int BITS, int C, int MG>
hipError_t launch_c(const Params& p, int cus, hipStream_t stream) {
  const int64_t steps = (p.N + 3) / 4;
  if (steps > 10LL * cus) return BITS == 8 ? launch<BITS, C, 8, 1, MG>(p, stream) : launch<BITS, C, 8, 2, MG>(p, stream);
  if (steps > 4LL * cus) return launch<BITS, C, 5, 2, MG>(p, stream);
  if (steps > 2LL * cus) return launch<BITS, C, 2, 2, MG>(p, stream);
  return launch<BITS, C, 1, 1, MG>(p, stream);
}

template <int BITS, int MG>
hipError_t launch_mg(const Params& p, int cus, hipStream_t stream) {
  switch (pick_c(p.K, BITS)) {
    case 1: return launch_c<BITS, 1, MG>(p, cus, stream);
    case 2: return launch_c<BITS, 2, MG>(p, cus, stream);
    default: return launch_c<BITS, 4, MG>(p, cus, stream);
  }
}

// Caller guarantees fits(p.K, BITS, p.M).
template <int BITS>
hipError_t launch_bits(const Params& p, int cus, hipStream_t stream) {
  return p.M > 4 ? launch_mg<BITS, 2>(p, cus, stream) : launch_mg<BITS, 1>(p, cus, stream);
}

}  // namespace qmv_mfma_detail

extern template hipError_t qmv_mfma_detail::launch_bits<2>(const qmv_mfma_detail::Params&, int, hipStream_t);
extern template hipError_t qmv_mfma_detail::launch_bits<4>(const qmv_mfma_detail::Params&, int, hipStream_t);
extern template hipError_t qmv_mfma_detail::launch_bits<8>(const qmv_mfma_detail::Params&, int, hipStream_t);

}  // namespace bitmm
