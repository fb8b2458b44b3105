// Device helpers shared by the bitmm kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace bitmm {

constexpr int kWave = 64;    // CDNA wavefront width

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// 128-bit streaming load (non-temporal hint: the weights are read once).
__device__ __forceinline__ u32x4_t load_stream(const uint32_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ u32x4_t load_u128(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// bf16 bit pattern -> f32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Two f32 -> packed bf16 pair (lo, hi), round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// v_dot2_f32_bf16: c + a.lo*b.lo + a.hi*b.hi (bf16 products are exact in f32).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// v_perm_b32: byte i of the result is byte sel[i] of the 8-byte value {hi:lo}.
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// 2-bit codes k = 0..7 in bits [2k, 2k+2) of half h of a word, spread to nibbles: code k
// in bits [4k, 4k+2) of the result (a 4-bit code word holding the same values).
// One byte permute (bytes 0 and 1 of the half to bytes 0 and 2, zeros between), then
// two shift-or-mask steps.
__device__ __forceinline__ uint32_t spread_2bit(uint32_t w, int h) {
  uint32_t x = __builtin_amdgcn_perm(0u, w, h ? 0x0c030c02u : 0x0c010c00u);
  x = (x | (x << 4)) & 0x0F0F0F0Fu;
  x = (x | (x << 2)) & 0x33333333u;
  return x;
}

// v_and_or_b32 (a & m) | c. Written out because gfx9 VOP3 encodings take no
// literal operands: given two constants the compiler splits it into v_and + v_or.
// The mask lives in an SGPR, the OR constant in a VGPR.
__device__ __forceinline__ uint32_t and_or_b32(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(m), "v"(c));
  return d;
}

// Wave-wide sum with DPP lane moves (VALU only, no LDS round trips). Rows of 16
// lanes are summed with quad permutes and mirrors; row_bcast then carries row
// sums upward. The full sum ends in lane 63 (other lanes hold partial sums).
template <int CTRL, int ROW_MASK, bool BOUND_CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                                ROW_MASK, 0xF, BOUND_CTRL));
}
__device__ __forceinline__ float wave_sum_lane63(float v) {
  v = dpp_add<0xB1, 0xF, true>(v);    // quad_perm [1,0,3,2]
  v = dpp_add<0x4E, 0xF, true>(v);    // quad_perm [2,3,0,1]
  v = dpp_add<0x141, 0xF, true>(v);   // row_half_mirror
  v = dpp_add<0x140, 0xF, true>(v);   // row_mirror: every lane holds its row's sum
  v = dpp_add<0x142, 0xA, false>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xC, false>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// v_fma_mix_f32: a * h + c in f32 with one rounding, h the low (HI = 0) or high
// (HI = 1) f16 half of `packed`, converted exactly.
template <int HI>
__device__ __forceinline__ float fma_mix_f16(float a, uint32_t packed, float c) {
  float d;
  if constexpr (HI)
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "=v"(d) : "v"(a), "v"(packed), "v"(c));
  else
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,0,0] op_sel_hi:[0,1,0]" : "=v"(d) : "v"(a), "v"(packed), "v"(c));
  return d;
}

// Sum over each aligned group of L lanes (L = 16, 32 or 64), with the same DPP
// steps: the group's sum ends in its last lane (lane L-1 of the group).
template <int L>
__device__ __forceinline__ float lane_group_sum(float v) {
  static_assert(L == 16 || L == 32 || L == 64, "group width");
  v = dpp_add<0xB1, 0xF, true>(v);
  v = dpp_add<0x4E, 0xF, true>(v);
  v = dpp_add<0x141, 0xF, true>(v);
  v = dpp_add<0x140, 0xF, true>(v);
  if constexpr (L >= 32) v = dpp_add<0x142, 0xA, false>(v);
  if constexpr (L == 64) v = dpp_add<0x143, 0xC, false>(v);
  return v;
}

typedef __attribute__((address_space(3))) void lds_ptr_t;

// A pointer every lane of the wave holds, moved to scalar registers.
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const T*>(((uint64_t)hi << 32) | lo);
}

// Buffer descriptor over [base, base + bytes): loads at byte offsets outside it
// return zeros (checked per dword), so ragged rows need no clamping. The fourth
// descriptor word is the raw-buffer format of the gfx9 family.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = (int)min(max(bytes, (int64_t)0), (int64_t)0x7FFFFFFF);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// Direct HBM -> LDS copy through a descriptor: lane L's SIZE bytes at byte offset
// voff land at dst + 16 L (SIZE 16) or in the low half of the 4-byte slot dst + 4 L
// (SIZE 2), without passing through registers.
// `soff` (a wave-uniform scalar offset) is added to the address but takes no part in
// the range check, so it may only carry offsets that stay inside the checked row.
template <int SIZE>
__device__ __forceinline__ void dma(__amdgpu_buffer_rsrc_t r, uint32_t voff, char* dst, int soff = 0) {
  static_assert(SIZE == 16 || SIZE == 2, "copy size");
  if constexpr (SIZE == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t*)dst, 16, voff, soff, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t*)dst, 2, voff, soff, 0, 0);
}

// Workgroup barrier without the memory fence of __syncthreads(). The fence makes the
// compiler wait for every outstanding load, including HBM -> LDS copies meant to stay
// in flight across the barrier; callers wait for the copies they need themselves
// (s_waitcnt vmcnt) and consume every LDS read they issue before arriving here. The
// "memory" clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

// f(integral_constant<int, I>) for I = B .. E-1, in order, each a separate instantiation.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Workgroups are dealt round-robin to the 8 XCDs, each with its own L2. Remaps the
// hardware id so that every XCD gets a contiguous run of logical ids: neighbouring
// logical tiles (which share operands) then run on one XCD and meet in its L2.
__device__ __forceinline__ int xcd_remap(int b, int total) {
  if (total % 8 != 0) return b;
  return (b % 8) * (total / 8) + b / 8;
}

// Cache-policy operand of a buffer load: non-temporal (data read once).
constexpr int kNonTemporal = 2;

// Row indirection of the gathered GEMV: output row r = row0 + blockIdx.y reads
// activation row tok[r] (row r when tok is null) and the weights, scales and biases of
// expert exp[r]. Dense calls pass exp == nullptr and one row of blocks.
struct GemvBatch {
  const int32_t* tok;
  const int32_t* exp;
  int T, E;            // activation rows, experts
  int rows, row0;      // output rows of this launch (gridDim.y) and the first of them
  int64_t w_stride;    // uint32 words per expert
  int64_t sb_stride;   // scale (and bias) values per expert
};

// Moves the operand pointers to the workgroup's output row. Returns false when the
// row's token or expert id is out of range: the caller then writes zeros to its outputs.
__device__ __forceinline__ bool gemv_row(const GemvBatch& bt, int K, int N, bool out_f32,
                                         const uint16_t*& x, const uint32_t*& w, const uint16_t*& s,
                                         const uint16_t*& b, void*& y) {
  if (bt.exp == nullptr) return true;
  const int r = bt.row0 + (int)blockIdx.y;
  const int e = bt.exp[r];
  const int t = bt.tok ? bt.tok[r] : r;
  y = static_cast<char*>(y) + (size_t)r * N * (out_f32 ? 4 : 2);
  if (e < 0 || e >= bt.E || t < 0 || t >= bt.T) return false;
  x += (int64_t)t * K;
  w += (int64_t)e * bt.w_stride;
  s += (int64_t)e * bt.sb_stride;
  b += (int64_t)e * bt.sb_stride;
  return true;
}

// log2 of a quantization group size (32, 64 or 128): the GEMV kernels index scales with
// shifts, since an integer division ahead of their first loads delays every wave.
inline int group_shift(int group) { return group == 32 ? 5 : (group == 64 ? 6 : 7); }

// Grid rows of a launch: one per gathered output row, or one.
inline unsigned gemv_grid_rows(const GemvBatch& bt) { return bt.exp ? (unsigned)bt.rows : 1u; }

// Zeros outputs [n0, n1) of one output row, all threads of the workgroup.
__device__ __forceinline__ void zero_outputs(void* y, int n0, int n1, bool out_f32) {
  for (int n = n0 + (int)threadIdx.x; n < n1; n += (int)blockDim.x) {
    if (out_f32)
      static_cast<float*>(y)[n] = 0.f;
    else
      static_cast<uint16_t*>(y)[n] = 0;
  }
}

}  // namespace bitmm
