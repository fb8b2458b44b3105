// GEMV / small-M kernel on the matrix cores: y[m][n] for up to 8 activation rows.
//
// The affine split of one quantization group g (64 consecutive k of weight row n),
//     sum_{k in g} x_k (s q_k + b) = s * sum x_k q~_k + c * sum x_k,
// needs one exact dot product per (row n, group g): q~ is the code as an exact
// bf16 value (4-bit: 128 + q, from a mask-and-OR of a nibble pair; 8-bit: q,
// converted), and c = b - 128 s (4-bit) or b (8-bit). v_mfma_f32_16x16x32_bf16
// forms 16 columns x 16 activation rows of those dot products in two instructions
// per group: lane (n, j) supplies 8 codes of weight row n and lane (m, j) the
// matching 8 activations of row m (activation rows past M are don't-care). The
// products are exact and the MFMA reduces over k itself, so no lane reduction is
// needed. Per group and column the lane then applies s and c in f32.
//
// Work: one workgroup per 16 weight rows (NB = 1) split over SK waves along K; the
// activations live in LDS for the whole workgroup (rearranged to match the code
// pairs), with their group sums. Each wave streams its share of groups with loads
// issued one batch of UG groups ahead; partial sums are added across waves
// through LDS in a fixed order (deterministic).
#pragma once

#include "common.hpp"

namespace bitmm {
namespace qmv_detail {

struct QmvMfmaParams {
  const uint16_t* x;  // [MR, K]
  const uint32_t* w;  // [N, K*BITS/32]
  const uint16_t* s;  // [N, K/64]
  const uint16_t* b;
  void* y;            // [MR, N]
  int N, K;
  int out_f32;
};

template <int BITS, int MR, int SK>
struct QmvMfma {
  static constexpr int THREADS = 64 * SK;
  static constexpr int UB = 6;  // units per load batch (two batches are requested up front)
  // A unit is what one 16-byte load per lane covers for 16 weight rows:
  // 4-bit: two groups (lane group j holds words 4j..4j+3 of the 16-word pair);
  // 8-bit: one group (lane group j holds words 4j..4j+3 of the 16-word group).
  static constexpr int GPU_ = BITS == 4 ? 2 : 1;  // groups per unit
  static constexpr int STEPS = BITS == 4 ? 4 : 2;  // MFMA steps per unit (8 codes per lane each)

  __device__ static void run(const QmvMfmaParams& p, char* lds) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ln = lane & 15;
    const int lj = lane >> 4;
    const int K = p.K;
    const int G = K / kGroup;
    const int U = (G + GPU_ - 1) / GPU_;  // units per row
    const int XP = K + 8;                 // LDS row pitch (elements)
    uint16_t* xl = reinterpret_cast<uint16_t*>(lds);
    float* gsum = reinterpret_cast<float*>(lds + (((size_t)MR * XP * 2 + 15) / 16) * 16);
    float* red = gsum + ((G * MR + 3) / 4) * 4;

    // 1. This wave's units and this lane's weight row. The first batch of codes is
    //    requested before the activations are staged, so its latency overlaps it.
    const int u0 = (int)((int64_t)U * wave / SK);
    const int u1 = (int)((int64_t)U * (wave + 1) / SK);
    const int n = min((int)blockIdx.x * 16 + ln, p.N - 1);
    const int64_t wrow = (int64_t)K * BITS / 32;
    const uint32_t* wr = p.w + (int64_t)n * wrow;
    const uint16_t* sr = p.s + (int64_t)n * G;
    const uint16_t* br = p.b + (int64_t)n * G;
    // The group this lane's chunk belongs to, inside a unit.
    const int lg = BITS == 4 ? (lj >> 1) : 0;

    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    struct Batch {
      u32x4_t q[UB];
      uint32_t s[UB], b[UB];  // raw bf16 bits, widened (keeps each load in its own register)
    };
    auto load_batch = [&](int ub, Batch& B) {
#pragma unroll
      for (int v = 0; v < UB; ++v) {
        const int u = min(ub + v, u1 - 1);         // past the wave's range: re-read (unused)
        const int g = min(u * GPU_ + lg, G - 1);    // odd G: the missing group is masked later
        const int64_t word = (int64_t)g * (2 * BITS) + (BITS == 4 ? (lj & 1) * 4 : lj * 4);
        B.q[v] = load_u128(wr + word);  // cached: the next unit reads the other half-line
        B.s[v] = sr[g];
        B.b[v] = br[g];
      }
    };
    // Both batches are requested before anything else: with at most 2 UB units per
    // wave (the host picks SK so), every code load of the wave is in flight at once.
    Batch bA, bB;
    load_batch(u0, bA);
    load_batch(u0 + UB, bB);

    // 2. Stage activations: 16-byte pieces (8 k). 4-bit pieces are stored as the
    //    pairs (x_j, x_{j+4}) that meet the nibble pairs of a code word; 8-bit pieces
    //    keep k order. Lanes 8t..8t+7 hold one group of one row and sum it with DPP.
    const int pieces = MR * (K / 8);
    for (int base = 0; base < pieces; base += THREADS) {
      const int id = base + tid;
      const bool ok = id < pieces;
      const int idc = ok ? id : pieces - 1;
      const int m = idc / (K / 8);
      const int k = (idc % (K / 8)) * 8;
      u32x4_t v = load_u128(p.x + (int64_t)m * K + k);
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) t = dot2_bf16(v[e], 0x3F803F80u, t);
      if constexpr (BITS == 4) {
        const u32x4_t d = v;
        v[0] = perm_b32(d[2], d[0], 0x05040100u);  // (x0, x4)
        v[1] = perm_b32(d[2], d[0], 0x07060302u);  // (x1, x5)
        v[2] = perm_b32(d[3], d[1], 0x05040100u);  // (x2, x6)
        v[3] = perm_b32(d[3], d[1], 0x07060302u);  // (x3, x7)
      }
      if (ok) *reinterpret_cast<u32x4_t*>(xl + (size_t)m * XP + k) = v;
      t = dpp_add<0xB1, 0xF, true>(t);   // quad_perm [1,0,3,2]
      t = dpp_add<0x4E, 0xF, true>(t);   // quad_perm [2,3,0,1]
      t = dpp_add<0x141, 0xF, true>(t);  // row_half_mirror: all 8 lanes hold the sum
      if (ok && (lane & 7) == 0) gsum[(k / kGroup) * MR + m] = t;
    }
    __syncthreads();

    // A operand. 4-bit: MFMA rows 0-7 carry activation rows for the unit's first
    // group and rows 8-15 for its second; a lane whose chunk belongs to the other
    // group supplies zeros, so C row r = (m = r % 8, group = r / 8) is one group's
    // dot product. 8-bit: rows are activation rows, the unit is one group.
    const int arow = BITS == 4 ? (ln & 7) : ln;
    const bool azero = BITS == 4 ? ((ln >> 3) != lg) : false;
    const uint16_t* xa = xl + (size_t)min(arow, MR - 1) * XP;
    const int koff = BITS == 4 ? lj * 32 : lj * 16;  // k of this lane's chunk inside a unit
    // C rows held by this lane: r = 4 lj + i.
    const uint32_t magic = 0x43004300u;  // bf16 pair (128, 128)
    auto compute_batch = [&](int ub, const Batch& B) {
#pragma unroll
      for (int v = 0; v < UB; ++v) {
        const int u = ub + v;
        if (u >= u1) break;  // uniform
        f32x4_t c = {0.f, 0.f, 0.f, 0.f};
        // A 4-bit row with an odd number of groups ends on half a unit: the missing
        // group's activations are zero (and its address is clamped into the row).
        const bool aoff = azero || (u * GPU_ + lg >= G);
        const int kbase = min(u * GPU_ * kGroup + koff, K - 8 * STEPS);
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
          uint32_t bw[4];
          if constexpr (BITS == 4) {
            const uint32_t wd = B.q[v][t];
#pragma unroll
            for (int j = 0; j < 4; ++j) bw[j] = and_or_b32(wd >> (4 * j), 0x000F000Fu, magic);
          } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const uint32_t wd = B.q[v][2 * t + h];
              bw[2 * h] = pack_bf16x2((float)(wd & 0xFFu), (float)((wd >> 8) & 0xFFu));
              bw[2 * h + 1] = pack_bf16x2((float)((wd >> 16) & 0xFFu), (float)(wd >> 24));
            }
          }
          u32x4_t av = *reinterpret_cast<const u32x4_t*>(xa + kbase + 8 * t);
          if (aoff) av = u32x4_t{0u, 0u, 0u, 0u};
          const u32x4_t bv = {bw[0], bw[1], bw[2], bw[3]};
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                      __builtin_bit_cast(bf16x8_t, bv), c, 0, 0, 0);
        }
        // Scale this lane's C rows with the group they belong to.
        const int rg = BITS == 4 ? u * 2 + (lj >> 1) : u;  // group of rows 4 lj + i
        const bool gok = rg < G;
        const int rgc = gok ? rg : G - 1;
        // s, b of group rg: lanes of lane group lj loaded group u*GPU_ + lg; for 4-bit
        // lg = lj >> 1 = the row group, so the lane's own s, b are the right ones.
        const float s = gok ? __uint_as_float(B.s[v] << 16) : 0.f;
        const float b = gok ? __uint_as_float(B.b[v] << 16) : 0.f;
        const float cb = BITS == 4 ? fmaf(-128.f, s, b) : b;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = BITS == 4 ? 4 * (lj & 1) + i : 4 * lj + i;
          if (BITS == 8 ? (i < MR) : (i < MR || MR > 4)) {
            acc[i] = fmaf(s, c[i], fmaf(cb, gsum[rgc * MR + min(m, MR - 1)], acc[i]));
          }
        }
      }
    };

    compute_batch(u0, bA);
    compute_batch(u0 + UB, bB);
    // Longer rows than 2 UB units per wave (large K): the rest batch by batch.
    for (int ub = u0 + 2 * UB; ub < u1; ub += UB) {
      load_batch(ub, bA);
      compute_batch(ub, bA);
    }

    // 3. Add the partial sums: over the SK waves in wave order, and for 4-bit over the
    //    two row halves (lane l holds the first group's rows, lane l + 32 the second's).
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wave * 4 + i) * 64 + lane] = acc[i];
    __syncthreads();
    if (wave != 0) return;
    constexpr int HALVES = BITS == 4 ? 2 : 1;
    if (BITS == 4 && lane >= 32) return;
    const int col = blockIdx.x * 16 + ln;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < SK; ++w)
#pragma unroll
        for (int h = 0; h < HALVES; ++h) v += red[(w * 4 + i) * 64 + lane + 32 * h];
      const int m = 4 * lj + i;
      if (col < p.N && m < MR) {
        const int64_t o = (int64_t)m * p.N + col;
        if (p.out_f32)
          static_cast<float*>(p.y)[o] = v;
        else
          static_cast<uint16_t*>(p.y)[o] = f32_to_bf16(v);
      }
    }
  }
};

template <int BITS, int MR, int SK>
__global__ __launch_bounds__(64 * SK) void qmv_mfma_kernel(QmvMfmaParams p) {
  extern __shared__ __attribute__((aligned(16))) char qmv_lds[];
  QmvMfma<BITS, MR, SK>::run(p, qmv_lds);
}

// LDS bytes of one workgroup (same layout as QmvMfma::run).
inline size_t qmv_mfma_lds_bytes(int MR, int SK, int64_t K) {
  const size_t xb = (size_t)MR * (K + 8) * 2;
  const size_t gs = (size_t)(K / kGroup) * MR * 4;
  const size_t red = (size_t)SK * 4 * 64 * 4;
  return ((xb + 15) / 16) * 16 + ((gs + 15) / 16) * 16 + red;
}

template <int BITS, int MR, int SK>
hipError_t launch_mfma_one(const QmvMfmaParams& p, hipStream_t stream) {
  const size_t lds = qmv_mfma_lds_bytes(MR, SK, p.K);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)qmv_mfma_kernel<BITS, MR, SK>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int blocks = (p.N + 15) / 16;
  hipLaunchKernelGGL((qmv_mfma_kernel<BITS, MR, SK>), dim3(blocks), dim3(64 * SK), lds, stream, p);
  return hipGetLastError();
}

template <int BITS, int MR>
hipError_t launch_mfma_sk(const QmvMfmaParams& p, int sk, hipStream_t stream) {
  switch (sk) {
    case 1: return launch_mfma_one<BITS, MR, 1>(p, stream);
    case 2: return launch_mfma_one<BITS, MR, 2>(p, stream);
    case 4: return launch_mfma_one<BITS, MR, 4>(p, stream);
    default: return launch_mfma_one<BITS, MR, 8>(p, stream);
  }
}

// mr in [1, 8]; sk in {1, 2, 4, 8}.
template <int BITS>
hipError_t launch_mfma_bits(const QmvMfmaParams& p, int mr, int sk, hipStream_t stream) {
  switch (mr) {
    case 1: return launch_mfma_sk<BITS, 1>(p, sk, stream);
    case 2: return launch_mfma_sk<BITS, 2>(p, sk, stream);
    case 3: return launch_mfma_sk<BITS, 3>(p, sk, stream);
    case 4: return launch_mfma_sk<BITS, 4>(p, sk, stream);
    case 5: return launch_mfma_sk<BITS, 5>(p, sk, stream);
    case 6: return launch_mfma_sk<BITS, 6>(p, sk, stream);
    case 7: return launch_mfma_sk<BITS, 7>(p, sk, stream);
    default: return launch_mfma_sk<BITS, 8>(p, sk, stream);
  }
}

}  // namespace qmv_detail

extern template hipError_t qmv_detail::launch_mfma_bits<4>(const qmv_detail::QmvMfmaParams&, int, int,
                                                           hipStream_t);
extern template hipError_t qmv_detail::launch_mfma_bits<8>(const qmv_detail::QmvMfmaParams&, int, int,
                                                           hipStream_t);
}  // namespace bitmm
