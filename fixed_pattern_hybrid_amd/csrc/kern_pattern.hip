// Row normalisers and the dense eager pattern of frozen heads
// ("When Can Attention Heads Be Statically Defined?", Section 3.2,
// Equation 3: N(i) = sum_{k<=i} exp(a[k] + r[i-k])).
//
// Normalisers are computed over chunks of 256 keys.  One block handles 64
// rows; each of its four waves takes every fourth key of a row, and the four
// partial sums are merged at the end.  Within a (row block, key chunk) the
// terms factor as
//   exp2(a2[k] + r2[i-k]) = 2^(ma + mr) * exp2(a2[k] - ma) * exp2(r2[i-k] - mr)
// with ma, mr the chunk maxima of a2 and of the chunk's r2 band (log2 units),
// so each term costs one FMA on two staged exponentials.  Both factors are
// <= 1; a term lost to underflow is below 2^-126 of 2^(ma+mr), so when a
// lane's chunk sum is >= 2^-20 the relative loss is below 2^-98.  Smaller
// sums are recomputed exactly with a max-shifted sum.  Partial results are
// (max, sum) pairs in log2 units merged as a log-sum-exp.
//
//   lognorm_kernel          one block per (head, row block), all chunks in
//                           turn; writes log N (natural log).  Used by
//                           saf_pattern_lognorm and the fp32 forward; the
//                           bf16 forward takes key-group partials from the
//                           band-sum program of kern_fit.hip.
#include "saf_internal.h"
#include "saf_device.h"
#include "saf_tile.h"

namespace saf {
namespace {

constexpr int kRows = 64;   // rows per block (one per lane of each wave)
constexpr int kLanes = 4;   // key lanes: wave w takes the chunk's key groups 4w..4w+3, 4w+16.., ...
constexpr int kTK = kLognormChunk;  // keys per chunk
constexpr int kBand = kRows + kTK;
constexpr int kNT = kRows * kLanes;
constexpr int kBS = band_stride(kBand);  // distance between the copies of exp2(r2 - mr)
static_assert(kTK % 16 == 0 && kBand + 3 <= 2 * kNT, "chunk layout");

struct ChunkSmem {
  float a2s[kTK];    // a (log2 units) of the chunk
  float r2s[kBand];  // r (log2 units) of the chunk's band
  __attribute__((aligned(16))) float eas[kTK];  // exp2(a2 - ma)
  // exp2(r2 - mr) in four copies: copy c holds band entry y + c at y (0
  // past the end), so four consecutive entries starting anywhere are one
  // aligned 16-byte read
  __attribute__((aligned(16))) float ers[4 * kBS];
  float red[8];
  float cm[kLanes][kRows];
  float cs[kLanes][kRows];
};

// Maxima of two values over the block (4 waves).
__device__ __forceinline__ void block_max2(float& u, float& v, float* red) {
  for (int o = 32; o >= 1; o >>= 1) {
    u = fmaxf(u, __shfl_xor(u, o, 64));
    v = fmaxf(v, __shfl_xor(v, o, 64));
  }
  __syncthreads();
  if (lane_id() == 0) {
    red[wave_id()] = u;
    red[4 + wave_id()] = v;
  }
  __syncthreads();
  u = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  v = fmaxf(fmaxf(red[4], red[5]), fmaxf(red[6], red[7]));
}

__device__ __forceinline__ void lse_merge(float& M, float& S, float cm, float cs) {
  if (cs > 0.f) {
    const float Mn = fmaxf(M, cm);
    S = S * fast_exp2(M - Mn) + cs * fast_exp2(cm - Mn);
    M = Mn;
  }
}

// (max, sum) in log2 units of row (i0 + lane)'s terms with keys in
// [k0, k0 + kTK), merged over the four key lanes; valid in wave 0.  Every
// thread of the block must call this (it synchronises).
__device__ void chunk_partial(const float* arow, const float* rrow, int T, int i0, int k0,
                              ChunkSmem& sm, float& Mout, float& Sout) {
  const int row = lane_id(), kl = wave_id();
  const int i = i0 + row;
  // stage a2 over the chunk keys and r2 over offsets [i0-k0-kTK+1, i0+kRows-1-k0]
  const int dmin = i0 - k0 - (kTK - 1);
  float lmax_a = kNegInf, lmax_r = kNegInf;
  for (int x = threadIdx.x; x < kTK; x += kNT) {
    const int k = k0 + x;
    const float v = (k < T) ? arow[k] * kLog2e : kNegInf;
    sm.a2s[x] = v;
    lmax_a = fmaxf(lmax_a, v);
  }
  for (int x = threadIdx.x; x < kBand; x += kNT) {
    const int d = dmin + x;
    const float v = (d >= 0 && d < T) ? rrow[d] * kLog2e : kNegInf;
    sm.r2s[x] = v;
    lmax_r = fmaxf(lmax_r, v);
  }
  // shifts; an all -inf chunk (possible only for -inf inputs) shifts by 0
  float ma = lmax_a, mr = lmax_r;
  block_max2(ma, mr, sm.red);
  if (ma == kNegInf) ma = 0.f;
  if (mr == kNegInf) mr = 0.f;
  for (int x = threadIdx.x; x < kTK; x += kNT) sm.eas[x] = fast_exp2(sm.a2s[x] - ma);
  for (int x = threadIdx.x; x < kBand + 3; x += kNT) {
    const float e = x < kBand ? fast_exp2(sm.r2s[x] - mr) : 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int y = x - c;
      if (y >= 0 && y < kBand) sm.ers[c * kBS + y] = e;
    }
  }
  __syncthreads();

  // This wave's keys: groups of four, x = 4 * (kl + 4u), up to the last key
  // any row of the block reaches (later keys of a row have band offset < 0,
  // whose exp2(r2 - mr) is 0, and keys >= T have exp2(a2 - ma) = 0, so every
  // lane may run the same loop).  Interleaving the groups over the waves
  // balances the diagonal chunk, where rows reach only its first keys.
  const int xq = 4 * __builtin_amdgcn_readfirstlane(kl);
  const int xlast = min(min(i0 + kRows, T) - 1 - k0, kTK - 1);
  float M = kNegInf, S = 0.f;
  if (xq <= xlast) {
    const int xb = i - k0 - dmin;  // band index of offset i - k0 (key 0 of the chunk)
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
    // keys x..x+3 need band entries xb-x-3 .. xb-x (reversed); y0 mod 4 is
    // the same for every x (a multiple of 4), which picks the copy
    const int cpy = (xb + 1) & 3;  // = (xb - x - 3) mod 4
    const lds_f32* rc = (const lds_f32*)sm.ers + cpy * kBS - cpy;
    const lds_f32* ea = (const lds_f32*)sm.eas;
#pragma unroll 4
    for (int x = xq; x <= xlast; x += 4 * kLanes) {
      const f32x4 e4 = lds_read_f4(ea + x);
      const f32x4 r4 = lds_read_f4(rc + (xb - x - 3));
      s0 = fmaf(e4[0], r4[3], s0);
      s1 = fmaf(e4[1], r4[2], s1);
      s2 = fmaf(e4[2], r4[1], s2);
      s3 = fmaf(e4[3], r4[0], s3);
    }
    const float s = (s0 + s1) + (s2 + s3);
    if (i < T) {
      if (s >= 0x1p-20f) {
        M = ma + mr;
        S = s;
      } else {
        // exact fallback: max-shifted sum of this lane's terms in the chunk
        // (this wave's groups of four keys)
        const int kend = min(xlast, i - k0);
        float cm = kNegInf;
        for (int g = xq; g <= kend; g += 4 * kLanes)
          for (int y = g; y < g + 4 && y <= kend; ++y) cm = fmaxf(cm, sm.a2s[y] + sm.r2s[xb - y]);
        float cs = 0.f;
        if (cm != kNegInf)
          for (int g = xq; g <= kend; g += 4 * kLanes)
            for (int y = g; y < g + 4 && y <= kend; ++y) cs += fast_exp2(sm.a2s[y] + sm.r2s[xb - y] - cm);
        if (cs > 0.f) {
          M = cm;
          S = cs;
        }
      }
    }
  }
  sm.cm[kl][row] = M;
  sm.cs[kl][row] = S;
  __syncthreads();
  float Mt = kNegInf, St = 0.f;
  if (kl == 0)
    for (int x = 0; x < kLanes; ++x) lse_merge(Mt, St, sm.cm[x][row], sm.cs[x][row]);
  Mout = Mt;
  Sout = St;
  __syncthreads();  // the shared buffers are reused by the caller's next chunk
}

__global__ __launch_bounds__(kNT) void lognorm_kernel(LognormArgs A, int identity_heads) {
  __shared__ ChunkSmem sm;
  const int h = identity_heads ? (int)blockIdx.y : (int)A.heads[blockIdx.y];
  const int T = A.T;
  const int i0 = blockIdx.x * kRows;
  const int i = i0 + lane_id();
  const float* arow = A.a + (int64_t)h * A.prior_len;
  const float* rrow = A.r + (int64_t)h * A.prior_len;
  const int last_row = min(i0 + kRows, T) - 1;
  float M = kNegInf, S = 0.f;
  for (int k0 = 0; k0 <= last_row; k0 += kTK) {
    float cm, cs;
    chunk_partial(arow, rrow, T, i0, k0, sm, cm, cs);
    lse_merge(M, S, cm, cs);
  }
  if (wave_id() == 0 && i < T) {
    const float lz = (M + fast_log2(S)) * kLn2;  // natural log
    for (int b = 0; b < A.B; ++b)
      A.out[(int64_t)b * A.out_b_stride + (int64_t)h * A.out_h_stride + i] = lz;
  }
}

// Dense eager pattern of one head: row i per block, exact max-shifted sum.
__device__ __forceinline__ float block_max(float v, float* red) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  __syncthreads();
  if (lane_id() == 0) red[wave_id()] = v;
  __syncthreads();
  float m = red[0];
  for (int x = 1; x < (int)(blockDim.x >> 6); ++x) m = fmaxf(m, red[x]);
  return m;
}

__global__ __launch_bounds__(256) void pattern_dense_kernel(int T, const float* a, const float* r,
                                                            float* w) {
  __shared__ float red[8];
  const int i = blockIdx.x;
  float lm = kNegInf;
  for (int k = threadIdx.x; k <= i; k += blockDim.x) lm = fmaxf(lm, (a[k] + r[i - k]) * kLog2e);
  float m = block_max(lm, red);
  if (m == kNegInf) m = 0.f;  // only for -inf inputs
  float ls = 0.f;
  for (int k = threadIdx.x; k <= i; k += blockDim.x) ls += fast_exp2((a[k] + r[i - k]) * kLog2e - m);
  // block sum
  for (int o = 32; o >= 1; o >>= 1) ls += __shfl_xor(ls, o, 64);
  __syncthreads();
  if (lane_id() == 0) red[4 + wave_id()] = ls;
  __syncthreads();
  float s = 0.f;
  for (int x = 0; x < (int)(blockDim.x >> 6); ++x) s += red[4 + x];
  const float z2 = m + fast_log2(s);
  float* row = w + (int64_t)i * T;
  for (int j = threadIdx.x; j < T; j += blockDim.x)
    row[j] = (j <= i) ? fast_exp2((a[j] + r[i - j]) * kLog2e - z2) : 0.f;
}

}  // namespace

hipError_t launch_lognorm(const LognormArgs& args, hipStream_t stream) {
  if (args.n_heads <= 0 || args.T <= 0) return hipSuccess;
  dim3 grid((args.T + kRows - 1) / kRows, args.n_heads);
  hipLaunchKernelGGL(lognorm_kernel, grid, dim3(kNT), 0, stream, args, 0);
  return hipGetLastError();
}

hipError_t launch_lognorm_identity(const LognormArgs& args, hipStream_t stream) {
  if (args.n_heads <= 0 || args.T <= 0) return hipSuccess;
  dim3 grid((args.T + kRows - 1) / kRows, args.n_heads);
  hipLaunchKernelGGL(lognorm_kernel, grid, dim3(kNT), 0, stream, args, 1);
  return hipGetLastError();
}

hipError_t launch_pattern_dense(int T, int prior_len, const float* a, const float* r, float* w,
                                hipStream_t stream) {
  (void)prior_len;
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(pattern_dense_kernel, dim3(T), dim3(256), 0, stream, T, a, r, w);
  return hipGetLastError();
}

}  // namespace saf
