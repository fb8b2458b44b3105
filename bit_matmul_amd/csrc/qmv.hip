// Host side of the GEMV / small-M path (kernel in qmv_impl.hpp).
#include <stdlib.h>

#include <atomic>

#include "kernels.hpp"
#include "qmv_dma.hpp"
#include "qmv_impl.hpp"
#include "qmv_mfma.hpp"

namespace bitmm {

namespace {

// Rows per wave for the streaming GEMV: enough waves to fill the chip (about
// 4096 resident waves at four per SIMD), with a multiple of three rows each so
// the three-deep row ring runs without padding rows. BITMM_QMV_ROWS_PER_WAVE overrides it (tuning knob).
int stream_rows_per_wave(int64_t N) {
  const char* e = getenv("BITMM_QMV_ROWS_PER_WAVE");
  const int forced = e ? atoi(e) : 0;
  if (forced > 0) return forced;
  // The row ring is three deep: blocks of 3 or 6 rows keep it free of padding.
  return N > 4096 * 3 ? 6 : 3;
}

// Waves per workgroup along K for the matrix-core GEMV: enough workgroups x waves
// to occupy every SIMD about twice over, each wave keeping at least one group.
// At least enough waves that each holds at most 12 units (two load batches), so all
// of a wave's code loads are issued at once.
int mfma_split_k(int64_t N, int64_t K, int bits) {
  const int64_t blocks = (N + 15) / 16;
  const int64_t groups = K / kGroup;
  const int64_t units = bits == 4 ? (groups + 1) / 2 : groups;
  int sk = 1;
  while (sk < 8 && (blocks * sk < 2048 || units > 12 * sk) && 2 * sk <= units) sk *= 2;
  return sk;
}

constexpr size_t kMaxLds = 160 * 1024;  // gfx950 LDS per workgroup

// Kernel choice: 0 = automatic (streaming VALU form for M = 1, batched VALU form
// for 2..8 rows), 1 = streaming, 2 = batched, 3 = matrix-core form (when its LDS
// fits). BITMM_QMV_PATH = auto | stream | valu | mfma (comparison knob).
int forced_path() {
  const char* e = getenv("BITMM_QMV_PATH");
  if (!e) return 0;
  if (e[0] == 's') return 1;
  if (e[0] == 'v') return 2;
  if (e[0] == 'm') return 3;
  if (e[0] == 'd') return 4;
  return 0;
}

// Integer tuning knob from the environment (0 when unset).
int env_int(const char* name) {
  const char* e = getenv(name);
  return e ? atoi(e) : 0;
}

// Compute units of the current device (cached per device id).
int compute_units() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace

hipError_t launch_qmv(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
                      const uint16_t* biases, void* y, int64_t M, int64_t N, int64_t K, int bits,
                      bool out_f32, hipStream_t stream) {
  const int64_t cc = 128 / bits;
  const int64_t nch = K / cc;
  const size_t ysz = out_f32 ? 4 : 2;
  for (int64_t m0 = 0; m0 < M; m0 += 8) {
    const int mr = (int)(M - m0 < 8 ? M - m0 : 8);
    // Chunks per lane per pass over K: as few passes as possible, with at most
    // 4 chunks, and at most 12 chunk-rows of activations held per lane.
    const int64_t cap = mr <= 3 ? 4 : (12 / mr > 0 ? 12 / mr : 1);
    const int64_t passes = (nch + cap * kWave - 1) / (cap * kWave);
    const int cpl = (int)((nch + passes * kWave - 1) / (passes * kWave));
    qmv_detail::QmvParams p;
    p.x = x + m0 * K;
    p.w = w;
    p.s = scales;
    p.b = biases;
    p.y = static_cast<char*>(y) + (size_t)(m0 * N) * ysz;
    p.N = (int)N;
    p.K = (int)K;
    p.out_f32 = out_f32 ? 1 : 0;
    const int64_t cpl_all = (nch + kWave - 1) / kWave;  // chunks per lane for a whole row
    const int sk = mfma_split_k(N, K, bits);
    hipError_t e;
    const int path = forced_path();
    if (path == 3 && qmv_detail::qmv_mfma_lds_bytes(mr, sk, K) <= kMaxLds) {
      qmv_detail::QmvMfmaParams mp;
      mp.x = p.x;
      mp.w = w;
      mp.s = scales;
      mp.b = biases;
      mp.y = p.y;
      mp.N = (int)N;
      mp.K = (int)K;
      mp.out_f32 = p.out_f32;
      e = bits == 4 ? qmv_detail::launch_mfma_bits<4>(mp, mr, sk, stream)
                    : qmv_detail::launch_mfma_bits<8>(mp, mr, sk, stream);
    } else if ((path == 0 || path == 4) && mr == 1 &&
               qmv_dma_detail::pick_lanes(nch) != 0) {
      qmv_dma_detail::Params dp;
      dp.x = p.x;
      dp.w = w;
      dp.s = scales;
      dp.b = biases;
      dp.y = p.y;
      dp.N = (int)N;
      dp.K = (int)K;
      dp.out_f32 = p.out_f32;
      dp.steps_per_wave = dp.total_steps = 0;
      const int cus = compute_units();
      const int wpc = env_int("BITMM_QMV_WAVES_PER_CU");
      e = bits == 4 ? qmv_dma_detail::launch_bits<4>(dp, cus, wpc, stream)
                    : qmv_dma_detail::launch_bits<8>(dp, cus, wpc, stream);
    } else if ((path == 0 || path == 1) && mr == 1 && cpl_all <= 5) {
      const int rpw = stream_rows_per_wave(N);
      e = bits == 4 ? qmv_detail::launch_stream_bits<4>(p, (int)cpl_all, rpw, stream)
                    : qmv_detail::launch_stream_bits<8>(p, (int)cpl_all, rpw, stream);
    } else {
      e = bits == 4 ? qmv_detail::launch_bits<4>(p, mr, cpl, stream)
                    : qmv_detail::launch_bits<8>(p, mr, cpl, stream);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace bitmm
