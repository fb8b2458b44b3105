// Small-M GEMV with K split across the waves of a workgroup:
//   y[m][n] = sum_k x[m][k] (s[n][g] q[n][k] + b[n][g]),  m < MR <= 8.
//
// The weights are read once, so the kernel is built around their HBM stream, and the
// activations of every row must meet every code. Each of the W waves of a workgroup
// owns a slice of 32 consecutive 16-byte code chunks of K; lane l of a wave works on
// row l / 32 of a two-row step and on chunk l % 32 of the wave's slice. So:
//   * a step is two rows x 512 contiguous bytes per wave load instruction;
//   * a lane needs the activations of one chunk only (all MR rows of it), prepared
//     once into registers: 16 bf16 pairs per row at 4 bits, 16 f32 at 8 bits;
//   * every load of the workgroup's S steps is issued before any arithmetic.
// Per step each lane forms its chunk's dot products for all MR rows, the 32 lanes of
// a row sum them with DPP moves, and lane 31 of the half-wave writes the partial sum
// to LDS. After the last step the partial sums of the W waves are added in wave order
// (a fixed order: results do not depend on timing) and stored.
//
// Arithmetic (all codes of a chunk share a group, so the affine split applies):
//   sum_k x_k (s q_k + b) = s * sum_k x_k q_k + b * sum_k x_k.
// 4-bit: a nibble pair masked into 0x4300 is the exact bf16 pair (128 + q_j, 128 + q_{j+4});
// v_dot2_f32_bf16 against the activation pair (x_j, x_{j+4}) forms P = sum x (128 + q)
// with exact products, then s P + (b - 128 s) sum x. 8-bit: codes convert to f32 byte by
// byte. 2-bit (up to 3 rows): the code pair (j, j+8) of a word, masked at bit 0, 2 or 4
// into the bf16 pair of 128, 32 or 8, is that offset plus (q_j, q_{j+8}) exactly; P then
// carries the offset term o = 128 sA + 32 sB + 8 sC of the three classes of activation
// pairs, and the chunk adds s (P - o) + b sum x. Accumulation is f32 throughout (the
// decode fix of epic #1536, diagnosis item 3).
#pragma once

#include <algorithm>
#include <atomic>

#include "common.hpp"
#include "kernels.hpp"

namespace bitmm {
namespace qmv_split_detail {

struct Params {
  const uint16_t* x;
  const uint32_t* w;
  const uint16_t* s;
  const uint16_t* b;
  void* y;
  int N, K;
  int gshift;    // log2 of the quantization group along K (5, 6 or 7: groups of 32, 64, 128)
  int out_f32;
  GemvBatch bt;  // gathered rows (blockIdx.y), or none
};

constexpr uint32_t kNoChunk = 0x80000000u;   // outside every descriptor: reads zeros

// Launch shape per row count: up to 3 rows, up to 16 waves (1024 threads, at most 128
// registers per lane); from 4 rows the activations need more registers, so up to 8
// waves (256 registers). Blocks of 2 two-row steps, 3 for three rows at 8 bits
// (measured at K = 5120, N = 13824: 8-bit M = 3 27.1 -> 24.2 us with 3; 8-bit M = 2 20.3 ->
// 23.2 and 4-bit M = 3 18.0 -> 18.1 with 3, and 4-bit M = 3 or 4 rows slower with 4).
constexpr int max_waves(int mr) { return mr <= 3 ? 16 : 8; }
// 2-bit: 32 activation pairs per row and lane, so up to 3 rows and 8 waves.
constexpr int max_waves(int mr, int bits) { return bits == 2 ? 8 : max_waves(mr); }
template <int BITS>
constexpr int steps(int mr) { return BITS == 8 && mr == 3 ? 3 : 2; }

// 16-byte code chunks per weight row, and whether this kernel takes the shape.
inline int64_t chunks(int64_t K, int bits) { return K * bits / 128; }
inline bool fits(int64_t K, int bits, int64_t mr) {
  return mr >= 1 && mr <= (bits == 2 ? 3 : 8) && chunks(K, bits) <= 32 * max_waves((int)mr, bits);
}

template <int BITS, int MR, int S, int MAXW>
__global__ __launch_bounds__(64 * MAXW) void qmv_split_kernel(Params p) {
  constexpr int CC = 128 / BITS;         // codes per chunk
  constexpr int XU = CC / 8;             // 16-byte activation loads per chunk and row
  constexpr int XV = BITS == 2 ? 32 : 16;  // activation registers per row
  constexpr int RW = 2 * S;              // weight rows per block
  constexpr int NL = 3 * S;              // load instructions per block
  __shared__ float part[2][MAXW * RW * MR];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = __builtin_amdgcn_readfirstlane(blockDim.x >> 6);
  const int r = lane >> 5;
  const int li = lane & 31;
  const int K = p.K, N = p.N;
  const int nch = K / CC;
  const int G = K >> p.gshift;  // scales (and biases) per weight row
  const int c = wave * 32 + li;
  const bool ok = c < nch;
  const int64_t rowbytes = (int64_t)K * BITS / 8;
  const int nblk = (N + RW - 1) / RW;
  const int stride = gridDim.x;
  const uint16_t* xq = p.x;
  const uint32_t* wq0 = p.w;
  const uint16_t* sq = p.s;
  const uint16_t* bq = p.b;
  void* yq = p.y;
  if (!gemv_row(p.bt, K, N, p.out_f32 != 0, xq, wq0, sq, bq, yq)) {
    for (int bk = blockIdx.x; bk < nblk; bk += stride)
      zero_outputs(yq, bk * RW, min(bk * RW + RW, N), p.out_f32 != 0);
    return;
  }
  const char* wq = reinterpret_cast<const char*>(uniform_ptr(wq0));
  sq = uniform_ptr(sq);
  bq = uniform_ptr(bq);
  const uint32_t voff = ok ? (uint32_t)(r * rowbytes + c * 16) : kNoChunk;
  const uint32_t soff = ok ? (uint32_t)((r * G + ((c * CC) >> p.gshift)) * 2) : kNoChunk;

  // Codes, scales and biases of one block of RW rows. Rows past N, and chunks past the
  // row end, read as zeros through the descriptors (a block past the last one reads
  // nothing at all).
  struct Buf {
    u32x4_t q[S];
    uint32_t s[S], b[S];
  };
  auto load = [&](int blk, Buf& B) {
    const int64_t base = (int64_t)blk * RW;
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const int64_t row0 = base + 2 * i;
      const __amdgpu_buffer_rsrc_t rw = make_rsrc(wq + row0 * rowbytes, (N - row0) * rowbytes);
      B.q[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, voff, 0, kNonTemporal));
    }
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const int64_t row0 = base + 2 * i;
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(sq + row0 * G, (N - row0) * G * 2);
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(bq + row0 * G, (N - row0) * G * 2);
      B.s[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, soff, 0, 0);
      B.b[i] = __builtin_amdgcn_raw_buffer_load_b16(rb, soff, 0, 0);
    }
  };

  // 1. Loads of the lane's activations, then of this workgroup's first two blocks: at
  //    the loop head below the loads of two blocks are in flight, in that order, on
  //    entry as on every iteration, so the compiler's wait counts stay exact.
  Buf A, Bn;
  int blk = blockIdx.x;
  u32x4_t xin[MR][XU];
  {
    const int cc = ok ? c : 0;  // in bounds; zeroed below when the chunk does not exist
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int u = 0; u < XU; ++u) xin[m][u] = load_u128(xq + (int64_t)m * K + (int64_t)cc * CC + 8 * u);
  }
  __builtin_amdgcn_sched_barrier(0);
  load(blk, A);
  load(blk + stride, Bn);
  __builtin_amdgcn_sched_barrier(0);

  // 2. Activations of this lane's chunk, per row: the pairs (4-bit) or f32 values
  //    (8-bit) that meet the codes, and their sum.
  uint32_t xv[MR][XV];
  float sx[MR], ox[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    uint32_t raw[4 * XU];
#pragma unroll
    for (int u = 0; u < XU; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) raw[4 * u + e] = ok ? xin[m][u][e] : 0u;
    ox[m] = 0.f;
    if constexpr (BITS == 2) {
      // code word d holds codes 16 d .. 16 d + 15; the pair (j, j+8) meets the activation
      // pair (x_{16d+j}, x_{16d+j+8}); classes j = 0, 3, 6 / 1, 4, 7 / 2, 5 (offsets 128,
      // 32, 8) have their own sums.
      float tc[3] = {0.f, 0.f, 0.f};
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          xv[m][8 * d + j] = perm_b32(raw[8 * d + 4 + j / 2], raw[8 * d + j / 2], (j & 1) ? 0x07060302u : 0x05040100u);
          tc[j % 3] = dot2_bf16(xv[m][8 * d + j], 0x3F803F80u, tc[j % 3]);
        }
      sx[m] = (tc[0] + tc[1]) + tc[2];
      ox[m] = fmaf(128.f, tc[0], fmaf(32.f, tc[1], 8.f * tc[2]));
      continue;
    }
    float t = 0.f;
#pragma unroll
    for (int d = 0; d < 4 * XU; ++d) t = dot2_bf16(raw[d], 0x3F803F80u, t);
    sx[m] = t;
    if constexpr (BITS == 4) {
      // word wd of the codes holds k = 8 wd .. 8 wd + 7; nibble pair (j, j+4) meets the
      // activation pair (x_{8wd+j}, x_{8wd+j+4}).
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const uint32_t d0 = raw[4 * wd], d1 = raw[4 * wd + 1], d2 = raw[4 * wd + 2], d3 = raw[4 * wd + 3];
        xv[m][4 * wd + 0] = perm_b32(d2, d0, 0x05040100u);
        xv[m][4 * wd + 1] = perm_b32(d2, d0, 0x07060302u);
        xv[m][4 * wd + 2] = perm_b32(d3, d1, 0x05040100u);
        xv[m][4 * wd + 3] = perm_b32(d3, d1, 0x07060302u);
      }
    } else {
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        xv[m][2 * d] = raw[d] << 16;              // f32 bits of the low bf16
        xv[m][2 * d + 1] = raw[d] & 0xFFFF0000u;  // f32 bits of the high bf16
      }
    }
  }

  // 3. One block: dot products of the chunk for every row, 32-lane sums, partial sums
  //    to LDS (buffer `par`), a barrier, then the sum over the waves in wave order (a
  //    fixed order: results do not depend on timing) and the store. The two LDS
  //    buffers alternate, so the barrier of the next block separates this block's
  //    reads from the next writes to the same buffer.
  const uint32_t magic = 0x43004300u;  // bf16 pair (128, 128)
  auto block = [&](int bk, const Buf& B, int par) {
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const float s = __uint_as_float(B.s[i] << 16);
      const float b = __uint_as_float(B.b[i] << 16);
      float P[MR];
#pragma unroll
      for (int m = 0; m < MR; ++m) P[m] = 0.f;
      if constexpr (BITS == 2) {
        constexpr uint32_t MK[3] = {0x00030003u, 0x000C000Cu, 0x00300030u};
        constexpr uint32_t OF[3] = {0x43004300u, 0x42004200u, 0x41004100u};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t wsh[3] = {B.q[i][d], B.q[i][d] >> 6, B.q[i][d] >> 12};
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t qp = and_or_b32(wsh[j / 3], MK[j % 3], OF[j % 3]);
#pragma unroll
            for (int m = 0; m < MR; ++m) P[m] = dot2_bf16(qp, xv[m][8 * d + j], P[m]);
          }
        }
      } else if constexpr (BITS == 4) {
#pragma unroll
        for (int wd = 0; wd < 4; ++wd)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t qp = and_or_b32(B.q[i][wd] >> (4 * j), 0x000F000Fu, magic);
#pragma unroll
            for (int m = 0; m < MR; ++m) P[m] = dot2_bf16(qp, xv[m][4 * wd + j], P[m]);
          }
      } else {
#pragma unroll
        for (int wd = 0; wd < 4; ++wd)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float qf = (float)((B.q[i][wd] >> (8 * j)) & 0xFFu);  // v_cvt_f32_ubyte<j>
#pragma unroll
            for (int m = 0; m < MR; ++m) P[m] = fmaf(__uint_as_float(xv[m][4 * wd + j]), qf, P[m]);
          }
      }
      const float cb = BITS == 4 ? fmaf(-128.f, s, b) : b;
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        const float Pm = BITS == 2 ? P[m] - ox[m] : P[m];
        const float v = lane_group_sum<32>(fmaf(s, Pm, cb * sx[m]));
        if (li == 31) part[par][(wave * RW + 2 * i + r) * MR + m] = v;
      }
    }
    // The partial sums are written (LDS writes complete in order for the whole wave);
    // a bare barrier keeps the next block's loads in flight across it.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    barrier_no_fence();
    const int n0 = bk * RW;
    for (int t = threadIdx.x; t < RW * MR; t += blockDim.x) {
      const int row = t / MR, m = t - row * MR;
      float v = 0.f;
      for (int w = 0; w < nw; ++w) v += part[par][(w * RW + row) * MR + m];
      const int n = n0 + row;
      if (n < N) {
        const int64_t o = (int64_t)m * N + n;
        if (p.out_f32)
          static_cast<float*>(yq)[o] = v;
        else
          static_cast<uint16_t*>(yq)[o] = f32_to_bf16(v);
      }
    }
  };

  // 4. Blocks blockIdx.x, + gridDim.x, ...: the loads of the next block are in flight
  //    while one is computed (the two register sets alternate).
#pragma unroll 1
  for (;;) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NL) : "memory");  // A has landed
    block(blk, A, 0);
    blk += stride;
    if (blk >= nblk) break;
    load(blk + stride, A);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NL) : "memory");  // Bn has landed
    block(blk, Bn, 1);
    blk += stride;
    if (blk >= nblk) break;
    load(blk + stride, Bn);
  }
}

// Workgroups that fit on the device at once for this kernel and block size (cached).
template <int BITS, int MR, int S>
int resident_blocks(int nw) {
  static std::atomic<int> cache[17];
  int v = cache[nw].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int per_cu = 0, dev = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, qmv_split_kernel<BITS, MR, S, max_waves(MR, BITS)>,
                                                   64 * nw, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  (void)hipGetLastError();
  v = per_cu * cus;
  cache[nw].store(v, std::memory_order_relaxed);
  return v;
}

template <int BITS, int MR, int S>
hipError_t launch_s(const Params& p, hipStream_t stream) {
  const int nw = (int)((chunks(p.K, BITS) + 31) / 32);
  const int nblk = (p.N + 2 * S - 1) / (2 * S);
  const unsigned rows = gemv_grid_rows(p.bt);
  const int grid = std::max(1, std::min(nblk, resident_blocks<BITS, MR, S>(nw) / (int)rows));
  hipLaunchKernelGGL((qmv_split_kernel<BITS, MR, S, max_waves(MR, BITS)>), dim3(grid, rows), dim3(64 * nw), 0,
                     stream, p);
  launch_log(dim3(grid, rows), dim3(64 * nw), 0, "qmv_split_kernel<%d, %d, %d, %d>", BITS, MR, S,
             max_waves(MR, BITS));
  return hipGetLastError();
}

template <int BITS, int MR>
hipError_t launch_mr(const Params& p, hipStream_t stream) {
  return launch_s<BITS, MR, steps<BITS>(MR)>(p, stream);
}

// Caller guarantees fits(K, BITS, mr).
template <int BITS>
hipError_t launch_bits(const Params& p, int mr, hipStream_t stream) {
  if constexpr (BITS == 2) {
    return mr == 1 ? launch_mr<2, 1>(p, stream) : mr == 2 ? launch_mr<2, 2>(p, stream) : launch_mr<2, 3>(p, stream);
  } else {
    switch (mr) {
      case 1: return launch_mr<BITS, 1>(p, stream);
      case 2: return launch_mr<BITS, 2>(p, stream);
      case 3: return launch_mr<BITS, 3>(p, stream);
      case 4: return launch_mr<BITS, 4>(p, stream);
      case 5: return launch_mr<BITS, 5>(p, stream);
      case 6: return launch_mr<BITS, 6>(p, stream);
      case 7: return launch_mr<BITS, 7>(p, stream);
      default: return launch_mr<BITS, 8>(p, stream);
    }
  }
}

}  // namespace qmv_split_detail

extern template hipError_t qmv_split_detail::launch_bits<2>(const qmv_split_detail::Params&, int, hipStream_t);
extern template hipError_t qmv_split_detail::launch_bits<4>(const qmv_split_detail::Params&, int, hipStream_t);
extern template hipError_t qmv_split_detail::launch_bits<8>(const qmv_split_detail::Params&, int, hipStream_t);

}  // namespace bitmm
