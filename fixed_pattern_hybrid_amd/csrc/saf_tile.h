// Staging from global memory into LDS: bf16 row tiles copied straight into
// LDS by the block's waves, and per-row values and relative-position bands
// that pass through registers.
#pragma once

#include "saf_device.h"

namespace saf {

// Word 3 of a raw (unformatted, unswizzled) buffer resource on gfx9-family
// parts: 32-bit data format, so dword loads return the stored bits.
constexpr int kBufferFlags = 0x00020000;

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

// Distance in floats between the copies of a band: the smallest value
// >= BAND that is 16 (mod 64).  A wave reads the copies with 16-byte (or
// 8-byte) loads whose copy index follows the lane's position; with copies 4
// granules apart in bank order (64 banks of 4 bytes), 16 consecutive lanes
// touch each bank at most twice (copies a multiple of 64 floats apart share
// banks: 4-way conflicts).
constexpr int band_stride(int band) { return (band + 47) / 64 * 64 + 16; }

// The relative-position band of a frozen tile, band[x] = log2(e) * r[dmin + x]
// for x in [0, BAND) (-inf where dmin + x falls outside [0, T)), stored in LDS
// as NCOPY copies STRIDE floats apart: copy c holds band[y + c] at y (-inf
// past the band's end), so that aligned reads of NCOPY floats fetch NCOPY
// consecutive offsets in any phase (four copies: one 16-byte read for four
// offsets; two copies: two 8-byte reads).  Thread x loads band[x] once and
// writes it into every copy that holds it.
template <int BAND, int NTHR, int NCOPY = 4>
struct BandStage {
  static constexpr int STRIDE = band_stride(BAND);
  static_assert(BAND + NCOPY - 1 <= NTHR, "one band entry per thread");
  static_assert(STRIDE >= BAND && STRIDE % 4 == 0, "copies keep 16-byte alignment");
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
    if (x < BAND + NCOPY - 1) {
      const float val = valid ? v * kLog2e : kNegInf;
#pragma unroll
      for (int c = 0; c < NCOPY; ++c) {
        const int y = x - c;
        if (y >= 0 && y < BAND) rs[c * STRIDE + y] = val;
      }
    }
  }
  // The same copies holding 2^(log2(e) r - shift) (0 outside [0, T)).
  __device__ __forceinline__ void store_exp(lds_f32* rs, float shift) const {
    const int x = threadIdx.x;
    if (x < BAND + NCOPY - 1) {
      const float val = valid ? fast_exp2(v * kLog2e - shift) : 0.f;
#pragma unroll
      for (int c = 0; c < NCOPY; ++c) {
        const int y = x - c;
        if (y >= 0 && y < BAND) rs[c * STRIDE + y] = val;
      }
    }
  }
};

// Maximum of x over the block (every thread gets it); scratch: 4 floats of
// LDS, free until the barrier this makes.
__device__ __forceinline__ float block_max(float x, lds_f32* scratch) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = x;
  __syncthreads();
  x = fmaxf(fmaxf(scratch[0], scratch[1]), fmaxf(scratch[2], scratch[3]));
  __syncthreads();
  return x;
}

// A [ROWS][D] bf16 tile copied from global memory straight into LDS (buffer
// loads with the LDS modifier; no registers, no LDS store instructions), in
// the arrangement of layout L (padded LdsLayout<D> by default).  One
// wave-wide load writes 64 consecutive 16-byte granules of LDS (lane l at
// granule l); a row is L::NG granules, so lane l of load m fills granule
// g = 64 m + l, i.e. row g / NG, position g % NG, with the global chunk the
// layout keeps there; a pad granule and rows >= T take an offset outside the
// buffer range and are written as zeros.  The four waves of the block share
// the loads (wave w issues loads w, w+4, ...).
// The data is visible to the block after s_waitcnt vmcnt(0) in every wave
// and a barrier.
template <int D, int ROWS, bool KEEP = true, class L = LdsLayout<D>>
struct TileDma {
  static constexpr int NG = L::NG;           // granules per row
  static constexpr int NI = ROWS * NG / 64;  // wave-wide loads per tile
  static constexpr int PER = (NI + 3) / 4;   // loads per wave (4 waves)
  static constexpr int kOob = 0x7ffffff0;    // beyond any buffer range used here
  static_assert(ROWS * NG % 64 == 0, "tile must be whole wave-wide loads");
  // Per-lane byte offsets of this wave's loads: kept in registers (KEEP) or
  // recomputed at each issue where registers are scarcer.
  static constexpr bool kKeep = KEEP;
  int off[kKeep ? PER : 1];
  int ste;

  __device__ __forceinline__ int offset(int k) const {
    const int m = __builtin_amdgcn_readfirstlane(wave_id()) + 4 * k;
    int lane;
    if constexpr (kKeep) {
      lane = lane_id();
    } else {
      // recomputed at each use (volatile), so that no per-load constant
      // stays live between the tiles
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
    }
    const int g = 64 * m + lane;
    const int row = g / NG, pos = g - row * NG;
    return (m >= NI || pos >= D / 8) ? kOob : row * ste * 2 + L::chunk(row, pos) * 16;
  }

  // st: row stride of the tensor (elements, at most SAF_MAX_T_STRIDE)
  __device__ __forceinline__ void init(int64_t st) {
    ste = (int)(st > D ? st : D);  // a one-row tensor may have any stride
    if constexpr (kKeep) {
#pragma unroll
      for (int k = 0; k < PER; ++k) off[k] = offset(k);
    }
  }

  // Copy rows row0 .. row0+ROWS-1 of `base` into `tile` (zeros from row T).
  // The loads are issued from inline assembly, which the compiler's wait
  // insertion does not see: otherwise it would wait for them before the
  // first LDS read of the tile being computed (it cannot tell the two
  // buffers apart).  Completion is awaited explicitly (wait_vm_loads); waits
  // the compiler places for its own loads stay correct, as they only become
  // stricter.  The buffer must not be read before that wait and a barrier.
  __device__ __forceinline__ void issue(const __bf16* base, int64_t st, int row0, int T,
                                        lds_bf16* tile) const {
    const int rows = T - row0 < ROWS ? T - row0 : ROWS;
    const int nrec = rows >= 1 ? (int)((int64_t)(rows - 1) * ste * 2 + D * 2) : 0;
    const uint64_t addr = (uint64_t)(base + (int64_t)row0 * st);
    // raw buffer resource: 48-bit base, stride 0, byte range, data format.
    // Every input is the same across the block; readfirstlane makes that
    // explicit so that the descriptor is formed in scalar registers.
    const u32x4 rsrc = {(unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)addr),
                        (unsigned)__builtin_amdgcn_readfirstlane((int)((unsigned)(addr >> 32) & 0xffffu)),
                        (unsigned)__builtin_amdgcn_readfirstlane(nrec), (unsigned)kBufferFlags};
    const int w = __builtin_amdgcn_readfirstlane(wave_id());
    const unsigned lds0 = (unsigned)(uintptr_t)tile;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int m = w + 4 * k;
      if (m < NI) {
        // M0 holds the LDS destination; its previous value is restored so
        // that the statement has no effect on registers the compiler owns.
        unsigned saved;
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %2\n\t"
            "s_nop 0\n\t"
            "buffer_load_dwordx4 %1, %3, 0 offen lds\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "v"(kKeep ? off[kKeep ? k : 0] : offset(k)), "s"(lds0 + 1024u * m), "s"(rsrc)
            : "memory");
      }
    }
  }
};

// Wait until this wave's outstanding vector-memory loads (including loads
// into LDS) have completed.
__device__ __forceinline__ void wait_vm_loads() { __builtin_amdgcn_s_waitcnt(0x0f70); }

}  // namespace saf
