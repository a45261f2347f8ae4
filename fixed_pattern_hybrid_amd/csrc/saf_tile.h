// Cooperative global -> register -> LDS staging of bf16 row tiles.
#pragma once

#include "saf_device.h"

namespace saf {

// A [ROWS][D] bf16 tile of a strided tensor, staged by NTHR threads in 16-byte
// chunks.  Rows at or beyond `T` are filled with zeros, so no out-of-range
// address is ever formed.
template <int D, int ROWS, int NTHR>
struct TileStage {
  static constexpr int CPR = D / 8;  // 16-byte chunks per row
  static constexpr int CHUNKS = ROWS * CPR;
  static constexpr int PER = (CHUNKS + NTHR - 1) / NTHR;
  static_assert(CHUNKS % NTHR == 0, "tile must split evenly over the threads");
  u32x4 buf[PER];

  __device__ __forceinline__ void load(const __bf16* base, int64_t st, int row0, int T) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int idx = threadIdx.x + p * NTHR;
      const int row = idx / CPR, ch = idx % CPR;
      const int t = row0 + row;
      if (t < T) {
        buf[p] = gload16(base + (int64_t)t * st + ch * 8);
      } else {
        buf[p] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  // store into a tile with the LdsLayout<D> arrangement
  __device__ __forceinline__ void store(lds_bf16* lds) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int idx = threadIdx.x + p * NTHR;
      const int row = idx / CPR, ch = idx % CPR;
      lds_store16(lds + LdsLayout<D>::off(row, ch * 8), buf[p]);
    }
  }
};

}  // namespace saf
