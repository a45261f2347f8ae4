// Cooperative global -> register -> LDS staging of bf16 row tiles.
#pragma once

#include "saf_device.h"

namespace saf {

// A [ROWS][D] bf16 tile of a strided tensor, staged by NTHR threads in 16-byte
// chunks: loaded into registers at the start of a tile, stored to LDS at its
// end.  Rows at or beyond `T` read row T-1 (always in range, T >= 1) and are
// replaced by zeros when stored.  The loads carry no branches and nothing
// consumes them before the store, so the compiler neither waits for them
// early nor serialises the compute that overlaps them.
template <int D, int ROWS, int NTHR>
struct TileStage {
  static constexpr int CPR = D / 8;  // 16-byte chunks per row
  static constexpr int CHUNKS = ROWS * CPR;
  static constexpr int PER = (CHUNKS + NTHR - 1) / NTHR;
  static_assert(CHUNKS % NTHR == 0, "tile must split evenly over the threads");
  u32x4 buf[PER];
  bool in[PER];

  __device__ __forceinline__ void load(const __bf16* base, int64_t st, int row0, int T) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int idx = threadIdx.x + p * NTHR;
      const int row = idx / CPR, ch = idx % CPR;
      const int t = row0 + row;
      in[p] = t < T;
      buf[p] = gload16(base + (int64_t)(t < T ? t : T - 1) * st + ch * 8);
    }
  }

  // store into a tile with the LdsLayout<D> arrangement
  __device__ __forceinline__ void store(lds_bf16* lds) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int idx = threadIdx.x + p * NTHR;
      const int row = idx / CPR, ch = idx % CPR;
      const u32x4 v = buf[p];
      lds_store16(lds + LdsLayout<D>::off(row, ch * 8),
                  u32x4{in[p] ? v[0] : 0u, in[p] ? v[1] : 0u, in[p] ? v[2] : 0u, in[p] ? v[3] : 0u});
    }
  }
};

// One float per thread from src[i0 + threadIdx.x], prefetched into a register
// at the start of a tile and written to LDS at its end.  Out-of-range rows
// read row T-1 (in range) and report valid = false.
struct ScalarStage {
  float v;
  bool valid;
  __device__ __forceinline__ void load(const float* src, int i0, int T) {
    const int i = i0 + (int)threadIdx.x;
    valid = i < T;
    v = src[valid ? i : T - 1];
  }
};

// The relative-position band of a frozen tile, band[x] = log2(e) * r[dmin + x]
// for x in [0, BAND) (-inf where dmin + x falls outside [0, T)), stored in LDS
// as four copies: copy c holds band[y + c] at y (-inf past the band's end), so
// that aligned 16-byte reads fetch four consecutive offsets in any phase.
// Thread x loads band[x] once and writes it into every copy that holds it.
template <int BAND, int NTHR>
struct BandStage {
  static_assert(BAND + 3 <= NTHR, "one band entry per thread");
  float v;
  bool valid;
  __device__ __forceinline__ void load(const float* rrow, int dmin, int T) {
    const int x = threadIdx.x;
    const int d = dmin + x;
    valid = x < BAND && d >= 0 && d < T;
    const int dc = d < 0 ? 0 : (d < T ? d : T - 1);
    v = rrow[dc];
  }
  __device__ __forceinline__ void store(lds_f32* rs) const {
    const int x = threadIdx.x;
    if (x < BAND + 3) {
      const float val = valid ? v * kLog2e : kNegInf;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int y = x - c;
        if (y >= 0 && y < BAND) rs[c * BAND + y] = val;
      }
    }
  }
};

}  // namespace saf
