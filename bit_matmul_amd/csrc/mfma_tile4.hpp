// Matrix-core tile with 32x32x16 MFMAs: y[rows, n0 .. n0+BN) = x[rows, :] * dequant(w)^T,
// one 64-wide quantization group per loop body.
//
// Workgroup of WN waves, one per SIMD. Every wave owns all BM = 32*MB activation rows of
// the tile and 32 weight rows (columns of y), so each weight is dequantized exactly once
// per tile, and each wave's B operand never leaves its registers.
//
// The instruction stream is what limits a one-wave-per-SIMD matrix-core loop on gfx950:
// an MFMA holds the wave's issue port for part of its run, and each other instruction
// (vector, scalar, LDS or memory) takes a slot of its own. A 32x32x16 MFMA carries twice
// the work of a 16x16x32 one for the same issue cost, so the per-MFMA budget for the
// dequantization, the LDS reads and the copies doubles. The design keeps that stream
// short:
//   * Weights go straight from HBM to registers: lane (c, h) of wave wn holds, for group
//     g, the 16 bytes (4-bit) or 32 bytes (8-bit) of weight row n0 + 32 wn + c that hold
//     codes 32h .. 32h+31 of the group, plus the group's scale and bias. Loads for group
//     g+PD are issued while group g is multiplied. No LDS traffic, no barrier. With WS
//     the loads read 16 rows x 64 contiguous bytes per instruction and one lane swap
//     per register puts the bytes in that layout.
//   * Activations are the only operand staged in LDS (three buffers of one group, BM rows
//     x 128 bytes, copied HBM -> LDS without passing through registers, two groups ahead).
//     One barrier per group.
//   * Buffer descriptors are formed once; only scalar offsets move with the group (the
//     group's LDS buffer too). The loop body is unrolled PD times so every slot of the
//     weight ring is a constant register index.
//
// K order within a group (a contraction, so any order that pairs x and w alike is exact):
// MFMA k-step u (0..3) gives k-slot 8h + i of lane (c, h) code 32h + 8u + i of the group,
// and the A operand of lane (r, h) the activation with the same index: 16-byte chunk
// 4h + u of the row's 128-byte group segment.
//
// Dequantization, per code: w = s q + b as one v_fma_mix_f32 on an exact f16 form of the
// code (a code field ORed into 0x6400 = 1024.0 reads as 1024 + q in bits 0..7 of a half,
// or 1024 + 16 q in bits 4..7), so w = s (1024 + q) + (b - 1024 s) or (s/16)(1024 + 16q)
// + (b - 64 s); rounded to bf16 for the MFMA; f32 accumulation.
#pragma once

#include <stdio.h>

#include <string>

#include "common.hpp"
#include "tile_epilogue.hpp"

namespace bitmm {

// SBM chooses where a wave finds the scales and biases of its 32 weight rows:
//   0: two 2-byte loads per group and lane, into registers, PD groups ahead;
//   1: staged once into LDS by 4-byte copies of the wave's contiguous block (the 32 rows
//      times GS = K/group values of each array are one contiguous span), needs 4-byte
//      aligned blocks;
//   2: the same with 2-byte copies (each value in a 4-byte LDS slot), any alignment.
// A per-group load touches one cache line per weight row; the staged copies touch one
// or two per 64 values. GMAX is the largest GS the staging area holds (SBM != 0).
// RMAP: tile rows are gathered. Tile row i is output row perm[i] of y[., N], and it
// reads activation row tok[perm[i]] of x[T, K] (row perm[i] when tok is null); without
// RMAP, tile row i is row i of both x_rows and y_rows.
// WS: weight loads of 16 rows x 64 contiguous bytes (rows 0-15 and 16-31 of the wave's
// block in two instructions) instead of 32 rows x 32 bytes, redistributed to the
// MFMA layout with v_permlane16_swap (see load_w); 4-bit needs an even PD (each pair
// of instructions carries two groups) and XD = 2.
template <int BITS, int MB, int WN, int PD = 3, int XD = 2, int SBM = 0, int GMAX = 0, bool RMAP = false,
          bool WS = false>
struct MmTile4 {
  // The same tile with M2 row blocks: a caller whose row count varies at run time (the
  // grouped GEMMs, per expert) runs the smallest one that holds the rows.
  template <int M2>
  using WithMB = MmTile4<BITS, M2, WN, PD, XD, SBM, GMAX, RMAP, WS>;
  static constexpr int WAVES = WN;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BM = 32 * MB;
  static constexpr int BN = 32 * WN;
  static constexpr int XB = BM * 128;            // one activation buffer (one group)
  static constexpr int NB = XD + 1;              // activation buffers (copies XD groups ahead)
  static constexpr int SB_EL = SBM == 1 ? 2 : 4;  // LDS bytes per staged value
  static constexpr int SB_NDMA = SBM == 0 ? 0 : (32 * GMAX * SB_EL + 255) / 256;  // copies per array
  static constexpr int SB_ARR = SB_NDMA * 256;    // LDS bytes per array and wave
  static constexpr int SB_BYTES = WN * 2 * SB_ARR;
  static constexpr int LDS_BYTES = NB * XB + SB_BYTES;
  static constexpr int XI = BM / 8;              // 1 KB copies per group
  static constexpr int XC = XI / WAVES;          // copies per wave per group
  static constexpr int WV = BITS == 8 ? 2 : 1;   // code loads per lane per group (16 B; 8 B at 2 bits)
  static constexpr int GB = 8 * BITS;            // bytes of one group of codes (32 WV)
  static constexpr int WL = WV + (SBM == 0 ? 2 : 0);  // weight-side loads per group
  static constexpr int NP = 4 * MB;              // MFMAs per group
  static constexpr int PF = 4;                   // activation reads in flight
  static_assert(BITS == 2 || BITS == 4 || BITS == 8, "bits");
  static_assert(!WS || BITS != 2, "2-bit codes load 8 bytes per lane");
  static_assert(SBM >= 0 && SBM <= 2 && (SBM == 0) == (GMAX == 0), "scale/bias staging");
  static_assert(XI % WAVES == 0, "every wave issues the same number of copies");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  // Only the measured and tested depths: weights four groups ahead, activation copies two
  // groups ahead. Paired 4-bit loads six or eight groups ahead, and copies one group ahead
  // (with 160-row tiles), once gave wrong results on the device, most likely from the
  // miscount that vm_after_copy_tail removes (the last bodies' weight loads, unused, were
  // dropped by the compiler while the waits still counted them); they stay disabled.
  static_assert(PD == 4 && XD == 2, "prefetch depths: only the tested PD = 4, XD = 2");
  static_assert(!WS || BITS == 8 || PD % 2 == 0, "paired weight loads");
  // Weight-side loads issued by body h: WL each, or with paired 4-bit loads 2 WL from odd
  // bodies and none from even ones (only h's parity matters; h may be negative).
  static constexpr int loads_of(int h) { return (WS && BITS == 4) ? ((h & 1) ? 2 * WL : 0) : WL; }
  // Body g (slot I, same parity) waits for the copies of group g+1, issued at steps 0-2 of
  // body g+1-XD: after them come that body's weight loads, then the copies and weight
  // loads of the XD-1 bodies up to g.
  static constexpr int vm_after_copy(int I) {
    int t = (XD - 1) * XC;
    for (int d = 0; d < XD; ++d) t += loads_of(I - d);
    return t;
  }
  // The same for the last G % PD bodies, which issue no weight loads (their groups would
  // lie past the end): after the copies of group g+1 come only the loads of the body
  // before, when that is the last body of the unrolled loop, and this body's copies.
  // Counts of loads that were never issued would let the wait pass early, so the tail
  // issues none rather than relying on loads the compiler may drop as unused or merge
  // (two clamped to the same last group read the same address).
  static constexpr int vm_after_copy_tail(int I) { return (XD - 1) * XC + (I == 0 ? loads_of(PD - 1) : 0); }
  static_assert(PD * WL + XD * XC <= 63, "vmcnt range");
  static_assert(WAVES * BM * 64 <= NB * XB, "epilogue staging fits in the activation buffers");

  // The template arguments as text (host side, for the kernel-choice record).
  static const char* name() {
    static const std::string s = [] {
      char b[128];
      snprintf(b, sizeof b, "MmTile4<%d, %d, %d, %d, %d, %d, %d, %s, %s>", BITS, MB, WN, PD, XD, SBM, GMAX,
               RMAP ? "true" : "false", WS ? "true" : "false");
      return std::string(b);
    }();
    return s.c_str();
  }

  // Byte offset of 16-byte chunk c of row r in a 128-byte-row tile: rows in blocks of
  // 16 (2 KB), row r of a block at (r & 7) * 256 + (r >> 3) * 128, chunk c at
  // (c ^ (r & 7)) * 16. The reads of one MFMA operand (each 16-lane quarter: 16 rows,
  // one chunk each) and the writes of row-contiguous copies are free of bank conflicts.
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

  // Raw weight-side registers of one group: codes, scale and bias (bf16 in the low half).
  struct Wraw {
    u32x4_t q[WV];
    uint32_t s, b;
  };
  // Affine constants of one group, see the dequantization note above.
  struct Aff {
    float s, b0, s16, b1;
  };

  // Always inlined: a kernel that runs tiles of two sizes would otherwise call them as
  // functions, whose calling convention costs it about 45 registers.
  __device__ __forceinline__ static void run(const uint16_t* __restrict__ x_rows_in, int rows_in,
                             const uint32_t* __restrict__ w_in, const uint16_t* __restrict__ sc_in,
                             const uint16_t* __restrict__ bi_in, int n0_in, int N, int K,
                             int group, void* __restrict__ y_rows, bool out_f32, char* lds,
                             const int32_t* __restrict__ perm = nullptr,
                             const int32_t* __restrict__ tok = nullptr, int T = 0) {
    const uint16_t* x_rows = uniform_ptr(x_rows_in);
    const uint32_t* w = uniform_ptr(w_in);
    const uint16_t* sc = uniform_ptr(sc_in);
    const uint16_t* bi = uniform_ptr(bi_in);
    const int rows = __builtin_amdgcn_readfirstlane(rows_in);
    const int n0 = __builtin_amdgcn_readfirstlane(n0_in);
    // The lane index passes through an empty asm statement so that the per-lane offsets
    // derived from it are computed here: a caller that runs the tile in a loop would
    // otherwise get them hoisted out of its loop, each holding a register for good.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lc = lane & 31;
    const int lh = lane >> 5;
    const int G = K / 64;       // 64-code blocks along K: one loop body each
    const int GS = K / group;   // scale (and bias) values per weight row
    // Group of the lane's 32 codes in block g: lane half lh covers codes 32 lh .. 32 lh + 31.
    const int gshift = group == 32 ? 1 : (group == 64 ? 0 : -1);
    auto gidx_uniform = [&](int g) { return gshift > 0 ? 2 * g : (gshift == 0 ? g : g >> 1); };
    const int glane = gshift > 0 ? lh : 0;
    const int rowbytes = K * BITS / 8;
    const int col0 = n0 + wave * 32;  // first weight row of this wave

    // Descriptors for the whole K loop. Out-of-range rows (activation rows past `rows`,
    // weight rows past N) sit in the checked per-lane offset and read as zeros; the
    // group offset, always inside a row, travels in the scalar offset.
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x_rows, (int64_t)(RMAP ? T : rows) * K * 2);
    const __amdgpu_buffer_rsrc_t rw =
        make_rsrc(reinterpret_cast<const char*>(w) + (int64_t)col0 * rowbytes, (int64_t)(N - col0) * rowbytes);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(sc + (int64_t)col0 * GS, (int64_t)(N - col0) * GS * 2);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(bi + (int64_t)col0 * GS, (int64_t)(N - col0) * GS * 2);
    uint32_t xoff[XC];
#pragma unroll
    for (int k = 0; k < XC; ++k) {
      const int I = wave + k * WAVES;
      const int tr = dma_row(I, lane);
      if constexpr (RMAP) {
        // Gathered row: its activation row; tile rows past `rows` read nothing.
        int src = 0;
        if (tr < rows) {
          src = perm[tr];
          if (tok) src = tok[src];
        }
        xoff[k] = tr < rows ? (uint32_t)(src * K * 2 + dma_chunk(I, lane) * 16) : 0x80000000u;
      } else {
        xoff[k] = (uint32_t)(tr * K * 2 + dma_chunk(I, lane) * 16);
      }
    }
    const uint32_t woff = (uint32_t)(lc * rowbytes + lh * 4 * BITS);  // codes 32h .. 32h+31
    // WS: lane (m, q) = (lane % 16, lane / 16) loads chunk c(q) of a 64-byte span of row m
    // (first instruction) and of row 16 + m (second); c(q) = q at 8 bits (the span is one
    // group) and 0, 2, 1, 3 at 4 bits (two groups: the swap must leave chunk h of each
    // group in lane half h).
    const int wq = lane >> 4;
    const int wchunk = BITS == 8 ? wq : (((wq & 1) << 1) | (wq >> 1));
    const uint32_t wsx = (uint32_t)((lane & 15) * rowbytes + wchunk * 16);
    const uint32_t wsy = wsx + (uint32_t)(16 * rowbytes);
    const uint32_t soff = (uint32_t)((lc * GS + glane) * 2);
    // Activation read offsets within a buffer for k-step u (row lc of row block 0).
    int aoff[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) aoff[u] = loff(lc, 4 * lh + u);

    // Default cache policy: the other row tiles of the same columns read these codes
    // again shortly after, from L2.
    auto load_w = [&](int g, Wraw& r) {
      const int gc = min(g, G - 1);  // past the end: a valid group, never used
      if constexpr (WS && BITS == 8) {
        r.q[0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, wsx, gc * GB, 0));
        r.q[1] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, wsy, gc * GB, 0));
      } else if constexpr (BITS == 2) {
        const u32x2_t v = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rw, woff, gc * GB, 0));
        r.q[0] = u32x4_t{v[0], v[1], 0u, 0u};
      } else {
#pragma unroll
        for (int v = 0; v < WV; ++v)
          r.q[v] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                   rw, woff + v * 16, gc * GB, 0));
      }
      if constexpr (SBM == 0) {
        // Scalar offset forced into an SGPR: built in a VGPR, each load would sit in a
        // waterfall loop.
        const int so = __builtin_amdgcn_readfirstlane(gidx_uniform(gc) * 2);
        r.s = __builtin_amdgcn_raw_buffer_load_b16(rs, soff, so, 0);
        r.b = __builtin_amdgcn_raw_buffer_load_b16(rb, soff, so, 0);
      }
    };
    // WS, 4 bits: groups ge, ge+1 (ge even) of rows 0-15 and 16-31 (one 64-byte span per
    // row). Rows past N read zeros through the checked per-lane offset.
    auto load_pair = [&](int ge, Wraw& r0, Wraw& r1) {
      const int gp = min(ge, (G - 1) & ~1);
      const uint32_t go = (uint32_t)(gp * GB);
      // With G odd the last pair has one group: the lanes of the missing second group
      // read nothing (an offset past every descriptor) instead of the next row's first
      // bytes, which would cost a second fetch of that line.
      const uint32_t past = (gp + 1 < G || wchunk < 2) ? 0u : 0x80000000u;
      r0.q[0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, (wsx + go) | past, 0, 0));
      r1.q[0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, (wsy + go) | past, 0, 0));
      if constexpr (SBM == 0) {
        const int so0 = __builtin_amdgcn_readfirstlane(gidx_uniform(min(ge, G - 1)) * 2);
        const int so1 = __builtin_amdgcn_readfirstlane(gidx_uniform(min(ge + 1, G - 1)) * 2);
        r0.s = __builtin_amdgcn_raw_buffer_load_b16(rs, soff, so0, 0);
        r0.b = __builtin_amdgcn_raw_buffer_load_b16(rb, soff, so0, 0);
        r1.s = __builtin_amdgcn_raw_buffer_load_b16(rs, soff, so1, 0);
        r1.b = __builtin_amdgcn_raw_buffer_load_b16(rb, soff, so1, 0);
      }
    };
    // Redistribution after the WS loads. v_permlane16_swap exchanges lanes 16-31 of its
    // first operand with lanes 0-15 of its second, and 48-63 with 32-47 (lane layout
    // checked on the device). For instructions X (rows 0-15) and Y (rows 16-31) as
    // loaded, lane (c, h) afterwards holds, of row c, chunk h of group ge in X and chunk
    // h of group ge+1 in Y (4 bits), or chunks 2h and 2h+1 of the group (8 bits): exactly
    // the non-WS layout.
    auto wswap = [&](u32x4_t& a, u32x4_t& b) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const auto r = __builtin_amdgcn_permlane16_swap(a[e], b[e], false, false);
        a[e] = r[0];
        b[e] = r[1];
      }
    };
    // Staged scales and biases: this wave's region, value of row lc and group g.
    char* const sbw = lds + NB * XB + wave * 2 * SB_ARR;
    auto sb_read = [&](int g, uint32_t& sv, uint32_t& bv) {
      const int o = (lc * GS + gidx_uniform(min(g, G - 1)) + glane) * SB_EL;
      sv = *reinterpret_cast<const uint16_t*>(sbw + o);
      bv = *reinterpret_cast<const uint16_t*>(sbw + SB_ARR + o);
    };
    auto copy_x = [&](int g, char* dst, int k) {
      const int gc = min(g, G - 1);
      dma<16>(rx, xoff[k], dst + (wave + k * WAVES) * 1024, gc * 128);
    };
    auto affine = [&](const Wraw& r) -> Aff {
      Aff a;
      a.s = __uint_as_float(r.s << 16);
      const float b = __uint_as_float(r.b << 16);
      a.b0 = fmaf(-1024.f, a.s, b);
      if constexpr (BITS <= 4) {
        a.s16 = a.s * 0.0625f;
        a.b1 = fmaf(-64.f, a.s, b);
      } else {
        a.s16 = a.s;
        a.b1 = a.b0;
      }
      return a;
    };
    // Packed f16 code registers for k-step u: 4-bit (q0,q4) (16q1,16q5) (q2,q6)
    // (16q3,16q7); 8-bit (q0,q2) (q1,q3) (q4,q6) (q5,q7). 2-bit codes 8u .. 8u+7 of the
    // lane are spread to a nibble word first and then taken as 4-bit.
    auto masks = [&](const Wraw& r, int u, uint32_t (&m)[4]) {
      const uint32_t magic = 0x64006400u;  // f16 pair (1024, 1024)
      if constexpr (BITS <= 4) {
        const uint32_t wd = BITS == 4 ? r.q[0][u] : spread_2bit(r.q[0][u >> 1], u & 1);
        const uint32_t w8 = wd >> 8;
        m[0] = and_or_b32(wd, 0x000F000Fu, magic);
        m[1] = and_or_b32(wd, 0x00F000F0u, magic);
        m[2] = and_or_b32(w8, 0x000F000Fu, magic);
        m[3] = and_or_b32(w8, 0x00F000F0u, magic);
      } else {
        const uint32_t lo = r.q[u >> 1][2 * (u & 1)];
        const uint32_t hi = r.q[u >> 1][2 * (u & 1) + 1];
        m[0] = and_or_b32(lo, 0x00FF00FFu, magic);
        m[1] = and_or_b32(lo >> 8, 0x00FF00FFu, magic);
        m[2] = and_or_b32(hi, 0x00FF00FFu, magic);
        m[3] = and_or_b32(hi >> 8, 0x00FF00FFu, magic);
      }
    };
    // bf16 pair e (k-slots 2e, 2e+1 of the lane's 8) of a B operand.
    auto pair = [&](const Aff& a, const uint32_t (&m)[4], int e) -> uint32_t {
      float lo, hi;
      if constexpr (BITS <= 4) {
        // (w0,w1) low halves of m0,m1; (w2,w3) low of m2,m3; (w4,w5), (w6,w7) high halves
        const uint32_t p0 = m[2 * (e & 1)], p1 = m[2 * (e & 1) + 1];
        if (e < 2) {
          lo = fma_mix_f16<0>(a.s, p0, a.b0);
          hi = fma_mix_f16<0>(a.s16, p1, a.b1);
        } else {
          lo = fma_mix_f16<1>(a.s, p0, a.b0);
          hi = fma_mix_f16<1>(a.s16, p1, a.b1);
        }
      } else {
        // (w0,w1) low of m0,m1; (w2,w3) high of m0,m1; (w4,w5), (w6,w7) from m2,m3
        const uint32_t p0 = m[2 * (e >> 1)], p1 = m[2 * (e >> 1) + 1];
        if ((e & 1) == 0) {
          lo = fma_mix_f16<0>(a.s, p0, a.b0);
          hi = fma_mix_f16<0>(a.s, p1, a.b0);
        } else {
          lo = fma_mix_f16<1>(a.s, p0, a.b0);
          hi = fma_mix_f16<1>(a.s, p1, a.b0);
        }
      }
      return pack_bf16x2(lo, hi);
    };

    f32x16_t acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[mb][j] = 0.f;

    char* const xb = lds;

    // ---- prologue: activations of groups 0 .. XD-1, weights of groups 0 .. PD-1 ----
    Wraw wr[PD];
#pragma unroll
    for (int i = 0; i < XD; ++i)
#pragma unroll
      for (int k = 0; k < XC; ++k) copy_x(i, xb + i * XB, k);
    if constexpr (WS && BITS == 4) {
#pragma unroll
      for (int i = 0; i < PD; i += 2) load_pair(i, wr[i], wr[i + 1]);
    } else {
#pragma unroll
      for (int i = 0; i < PD; ++i) load_w(i, wr[i]);
    }
    if constexpr (SBM != 0) {
      // Lane L of copy j carries values 64 j + L (2-byte form) or 128 j + 2 L, +1 (4-byte
      // form) of the wave's block; rows past N read as zeros.
      const int ncopy = (32 * GS * SB_EL + 255) / 256;
      for (int j = 0; j < ncopy; ++j) {
        const uint32_t vo = (uint32_t)((j * 64 + lane) * (SBM == 1 ? 4 : 2));
        if constexpr (SBM == 1) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t*)(sbw + j * 256), 4, vo, 0, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t*)(sbw + SB_ARR + j * 256), 4, vo, 0, 0, 0);
        } else {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t*)(sbw + j * 256), 2, vo, 0, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t*)(sbw + SB_ARR + j * 256), 2, vo, 0, 0, 0);
        }
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if constexpr (SBM != 0) {
      uint32_t s0, b0;
      sb_read(0, s0, b0);
      wr[0].s = s0;
      wr[0].b = b0;
    }
    if constexpr (WS && BITS == 4) wswap(wr[0].q[0], wr[1].q[0]);
    if constexpr (WS && BITS == 8) wswap(wr[0].q[0], wr[0].q[1]);
    Aff acur = affine(wr[0]);
    u32x4_t bcur;
    {
      uint32_t m[4];
      masks(wr[0], 0, m);
#pragma unroll
      for (int e = 0; e < 4; ++e) bcur[e] = pair(acur, m, e);
    }

    // One group: MFMAs of group g from LDS buffer g % NB with B operands dequantized one
    // k-step ahead from ring slot I (group g) and slot I+1 (group g+1, for the next body's
    // step 0). Issues the activation copies of group g+XD and the weight loads of group
    // g+PD (into slot I, spent by then). Ends with the wait for the copies of group g+1
    // and the barrier.
    auto body = [&](auto Ic, int g, auto Tc) {
      constexpr int I = decltype(Ic)::value;
      constexpr bool TAIL = decltype(Tc)::value;  // one of the last G % PD bodies
      const Wraw& wc = wr[I];
      Wraw& wn = wr[(I + 1) % PD];
      uint32_t sn = 0, bn = 0;  // staged scale and bias of group g+1
      if constexpr (SBM != 0) sb_read(g + 1, sn, bn);
      // Buffer of group g and of group g + XD: scalar byte offsets.
      const int xsel = __builtin_amdgcn_readfirstlane((g % NB) * XB);
      const int xdsel = __builtin_amdgcn_readfirstlane(((g + XD) % NB) * XB);
      char* xdst = xb + xdsel;
      int ab[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        ab[u] = aoff[u] + xsel;
        asm volatile("" : "+v"(ab[u]));
      }
      auto aread = [&](int p) -> u32x4_t {
        const int u = p / MB, mb = p % MB;
        return *reinterpret_cast<const u32x4_t*>(xb + ab[u] + mb * 4096);
      };
      u32x4_t av[PF];
#pragma unroll
      for (int p = 0; p < PF; ++p) av[p] = aread(p);
      Aff anext = acur;
      u32x4_t bnext = bcur;
      uint32_t m[4];
      uint32_t d[4];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int u = p / MB, mb = p % MB;
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av[p % PF]),
                                                          __builtin_bit_cast(bf16x8_t, bcur), acc[mb], 0, 0, 0);
        if (p + PF < NP) av[p % PF] = aread(p + PF);
        // Activation copies of group g+XD, spread over steps 0..2.
#pragma unroll
        for (int k = 0; k < XC; ++k)
          if (k * (3 * MB) / XC == p) copy_x(g + XD, xdst, k);
        // Weight loads of group g+PD once the codes of group g are spent (step 3); paired
        // 4-bit loads go out from odd bodies, for groups g+PD-1 and g+PD.
        if (!TAIL && p == 3 * MB) {
          if constexpr (WS && BITS == 4) {
            if constexpr (I % 2 == 1) load_pair(g + PD - 1, wr[(I + PD - 1) % PD], wr[I]);
          } else {
            load_w(g + PD, wr[I]);
          }
        }
        // Dequantization of the next B operand (step u+1 of group g, or step 0 of group
        // g+1), spread over the step's MFMAs: masks, then four pairs.
        {
          const Wraw& src = u < 3 ? wc : wn;
          const int un = (u + 1) & 3;
          // slot of each part within the step (mb index)
          constexpr int S_AFF = 0, S_MASK = 1;
          if (u == 3 && mb == S_AFF) {
            uint32_t s = SBM == 0 ? src.s : sn, b = SBM == 0 ? src.b : bn;
            asm volatile("" : "+v"(s), "+v"(b));
            Wraw t;
            t.s = s;
            t.b = b;
            anext = affine(t);
          }
          if (mb == (MB > 1 ? S_MASK : 0)) {
            // First use of group g+1's codes: redistribute them (a pair starts at an
            // even group).
            if (u == 3) {
              if constexpr (WS && BITS == 4 && I % 2 == 1) wswap(wn.q[0], wr[(I + 2) % PD].q[0]);
              if constexpr (WS && BITS == 8) wswap(wn.q[0], wn.q[1]);
            }
            masks(src, un, m);
#pragma unroll
            for (int e = 0; e < 4; ++e) asm volatile("" : "+v"(m[e]));
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int slot = MB > 2 ? 2 + e * (MB - 2) / 4 : MB - 1;
            if (mb == slot) {
              d[e] = pair(u == 3 ? anext : acur, m, e);
              asm volatile("" : "+v"(d[e]));
            }
          }
          if (mb == MB - 1) bnext = u32x4_t{d[0], d[1], d[2], d[3]};
        }
        __builtin_amdgcn_sched_barrier(0);
        if (mb == MB - 1) bcur = bnext;
      }
      acur = anext;
      // The copies of group g+1 (issued XD-1 bodies earlier) and everything before them
      // have landed; later copies and weight loads may still fly.
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(TAIL ? vm_after_copy_tail(I) : vm_after_copy(I)) : "memory");
      barrier_no_fence();
    };

    // The ring slot of group g is g % PD: the loop body covers PD groups so that every
    // slot index is a constant; the last G % PD groups run one body each.
    int g = 0;
#pragma unroll 1
    for (; g + PD <= G; g += PD)
      static_for<0, PD>([&](auto Ic) { body(Ic, g + decltype(Ic)::value, std::false_type{}); });
    static_for<0, PD - 1>([&](auto Ic) {
      if (g + decltype(Ic)::value < G) body(Ic, g + decltype(Ic)::value, std::true_type{});
    });
    // No copy may still be writing LDS when the workgroup moves on or ends, and no wave
    // reads the activation buffers any more once all have passed this barrier.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    barrier_no_fence();
    // Epilogue through this wave's region of the (now idle) activation buffers.
    store_tile<MB, RMAP>(acc, rows, col0, N, y_rows, out_f32 ? kOutF32 : kOutBf16, lds + wave * (BM * 64),
                         perm);
  }
};

}  // namespace bitmm
