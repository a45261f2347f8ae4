// Device helpers for gfx950 (CDNA4, wave64): bf16 MFMA fragments, LDS
// fragment reads and small conversions.
//
// MFMA v_mfma_f32_32x32x16_bf16, C[32x32] += A[32x16] * B[16x32]:
//   A: lane l holds row (l % 32), k = 8*(l/32) + e for e = 0..7
//   B: lane l holds col (l % 32), k = 8*(l/32) + e
//   C: lane l, register r holds col (l % 32), row 8*(r/4) + 4*(l/32) + r%4
// (verified on the device).  The contraction index k may be relabelled freely
// as long as A and B use the same labelling; the kernels use that to feed
// softmax / pattern weights straight from C registers into the next product.
//
// ds_read_b64_tr_b16 (LDS transpose read), per group of 16 lanes: if source
// lane 4e + c of the group addresses 4 consecutive 16-bit values starting at
// X[R + e][C + 4c], then output lane t of the group receives
// X[R + 0..3][C + t].  Two such reads give an MFMA operand whose k index runs
// along the rows of a row-major LDS tile.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace saf {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;
// LDS pointers carry their address space so that every access compiles to a
// ds_* instruction (a generic pointer would become a flat access).
typedef __attribute__((address_space(3))) __bf16 lds_bf16;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;

// Base of the dynamic LDS allocation as an LDS pointer.
#define SAF_DYN_LDS(name)                                   \
  extern __shared__ __align__(16) char name##_raw[];         \
  lds_bf16* name = (lds_bf16*)(name##_raw)

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// Round 8 fp32 values to bf16 (nearest-even) and pack them as an operand.
__device__ __forceinline__ bf16x8 pack_bf16x8(float x0, float x1, float x2, float x3, float x4,
                                              float x5, float x6, float x7) {
  bf16x8 v;
  v[0] = (__bf16)x0; v[1] = (__bf16)x1; v[2] = (__bf16)x2; v[3] = (__bf16)x3;
  v[4] = (__bf16)x4; v[5] = (__bf16)x5; v[6] = (__bf16)x6; v[7] = (__bf16)x7;
  return v;
}

// Operand registers r0..r0+7 of an accumulator as a bf16 fragment.
__device__ __forceinline__ bf16x8 pack_acc8(const f32x16& c, int r0) {
  return pack_bf16x8(c[r0], c[r0 + 1], c[r0 + 2], c[r0 + 3], c[r0 + 4], c[r0 + 5], c[r0 + 6],
                     c[r0 + 7]);
}

// 16-byte LDS read: 8 consecutive bf16 at element offset `off` of `base`.
__device__ __forceinline__ bf16x8 lds_read8(const lds_bf16* base, int off) {
  return *(const lds_bf16x8*)(base + off);
}

// Transposed 4-element read (see header comment); `off` is the element
// offset this lane addresses.
__device__ __forceinline__ bf16x4 lds_read_tr4(const lds_bf16* base, int off) {
  i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + off));
  return __builtin_bit_cast(bf16x4, t);
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 lo, bf16x4 hi) {
  bf16x8 v;
  v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
  v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
  return v;
}

// Row-major [rows][D] bf16 tile in LDS with rows padded by 16 bytes
// (pitch D + 8 elements).  Measured on gfx950, this keeps 16-byte fragment
// reads of 32 consecutive rows near the LDS read rate (about 170 B/clk/CU)
// and serves the transposing reads at about 110 B/clk/CU (two-way bank
// conflicts).  NG: 16-byte chunks per row (the last one is padding).
template <int D>
struct LdsLayout {
  static constexpr int PITCH = D + 8;  // elements per row
  static constexpr int NG = PITCH / 8;
  // element offset of (row, col)
  __device__ static __forceinline__ int off(int row, int col) { return row * PITCH + col; }
  // global chunk held at chunk position pos of a row (pos = D/8 is padding)
  __device__ static __forceinline__ int chunk(int row, int pos) { return pos; }
};

// Row-major [rows][D] bf16 tile without padding for D = 64 and 128: chunk c
// of row r sits at chunk position c ^ swz(r).  With 64 banks of 4 bytes, both
// fragment reads touch every bank once per pass: 16 lanes reading one chunk
// of 16 consecutive rows, and 32 lanes reading 4 consecutive chunks of 4
// consecutive rows (the transposing read), which the padded layout serves
// with two-way conflicts.  The lane offsets cost registers (a chunk position
// per fragment), so it is used where those are available.  Other D: padded.
template <int D>
struct SwzLayout {
  static constexpr bool SWZ = D == 64 || D == 128;
  static constexpr int PITCH = SWZ ? D : D + 8;
  static constexpr int NG = PITCH / 8;
  __device__ static __forceinline__ int swz(int row) {
    if constexpr (D == 64) return ((row >> 1) & 3) | ((((row >> 1) ^ (row >> 3)) & 1) << 2);
    else if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
    else return 0;
  }
  __device__ static __forceinline__ int off(int row, int col) {
    return row * PITCH + ((((col >> 3) ^ swz(row))) << 3) + (col & 7);
  }
  __device__ static __forceinline__ int chunk(int row, int pos) { return pos ^ swz(row); }
};

// MFMA operand whose k index runs along rows of a row-major LDS tile X.
// Lane l receives
//   X[row0 + 4*(l/32) + e][col0 + l%32]       for e = 0..3 (slots 0..3)
//   X[row0 + 8 + 4*(l/32) + e][col0 + l%32]   for e = 0..3 (slots 4..7)
// i.e. slot e of half h maps to row row0 + 8*(e/4) + 4*h + e%4 -- exactly the
// row labelling of the C registers 8*(s%2)..8*(s%2)+7 of a 32x32 accumulator
// block, so a C block converted with pack_acc8 pairs with this operand.
template <int D, class L = LdsLayout<D>>
__device__ __forceinline__ bf16x8 lds_frag_tr(const lds_bf16* X, int row0, int col0) {
  const int l = lane_id();
  const int g = l >> 4;        // 16-lane group
  const int s16 = l & 15;
  const int e = s16 >> 2, c = s16 & 3;
  const int row = row0 + 4 * (g >> 1) + e;
  const int col = col0 + 16 * (g & 1) + 4 * c;
  bf16x4 lo = lds_read_tr4(X, L::off(row, col));
  bf16x4 hi = lds_read_tr4(X, L::off(row + 8, col));
  return cat8(lo, hi);
}

// MFMA operand whose k index runs along columns of a row-major LDS tile:
// lane l receives X[row0 + l%32][col0 + 8*(l/32) + e], e = 0..7.
template <int D, class L = LdsLayout<D>>
__device__ __forceinline__ bf16x8 lds_frag_nat(const lds_bf16* X, int row0, int col0) {
  const int l = lane_id();
  return lds_read8(X, L::off(row0 + (l & 31), col0 + 8 * (l >> 5)));
}

// Exchange with the lane 32 positions away (the other half of a C column).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// Vector loads/stores of 16 bytes from global memory.
__device__ __forceinline__ u32x4 gload16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void sstore16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ f32x4 lds_read_f4(const lds_f32* p) { return *(const lds_f32x4*)p; }

}  // namespace saf
