// Row normalisers and the dense eager pattern of frozen heads
// ("When Can Attention Heads Be Statically Defined?", Section 3.2,
// Equation 3: N(i) = sum_{k<=i} exp(a[k] + r[i-k])).
//
// Normaliser kernel.  One block per (head, 64-row block); each of its four
// waves takes every fourth key of a row, so a row's sum is split over four
// lanes and merged at the end.  Keys come in tiles of 256.  Within a
// (row block, key tile) the terms factor as
//   exp2(a2[k] + r2[i-k]) = 2^(ma + mr) * exp2(a2[k] - ma) * exp2(r2[i-k] - mr)
// with ma, mr the tile maxima of a2 and of the tile's r2 band (log2 units),
// so each term costs one FMA on two staged exponentials.  Both factors are
// <= 1; a term lost to underflow is below 2^-126 of 2^(ma+mr), so when a
// lane's tile sum is >= 2^-20 the relative loss is below 2^-98.  Smaller
// sums are recomputed exactly with a max-shifted sum.  Partial results are
// merged with a running (max, sum) log-sum-exp.
#include "saf_internal.h"
#include "saf_device.h"

namespace saf {
namespace {

constexpr int kRows = 64;   // rows per block (one per lane of each wave)
constexpr int kLanes = 4;   // key lanes: wave w takes keys w, w+4, w+8, ...
constexpr int kTK = 1024;   // keys per tile
constexpr int kBand = kRows + kTK;

// Maxima of two values over the block (4 waves); red holds 8 floats.
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

__device__ __forceinline__ float block_max(float v, float* red) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  __syncthreads();
  if (lane_id() == 0) red[wave_id()] = v;
  __syncthreads();
  float m = red[0];
  for (int x = 1; x < (int)(blockDim.x >> 6); ++x) m = fmaxf(m, red[x]);
  return m;
}

__global__ __launch_bounds__(kRows * kLanes) void lognorm_kernel(LognormArgs A, int identity_heads) {
  __shared__ float a2s[kTK];    // a (log2 units) of the tile
  __shared__ float r2s[kBand];  // r (log2 units) of the tile's band
  __shared__ float eas[kTK];    // exp2(a2 - ma)
  __shared__ float ers[kBand];  // exp2(r2 - mr)
  __shared__ float red[8];
  __shared__ float cm_s[kLanes][kRows];
  __shared__ float cs_s[kLanes][kRows];

  const int hidx = blockIdx.y;
  const int h = identity_heads ? hidx : (int)A.heads[hidx];
  const int T = A.T;
  const int i0 = blockIdx.x * kRows;
  const int row = lane_id(), kl = wave_id();
  const int i = i0 + row;
  const float* arow = A.a + (int64_t)h * A.prior_len;
  const float* rrow = A.r + (int64_t)h * A.prior_len;
  const int last_row = min(i0 + kRows, T) - 1;
  constexpr int NT = kRows * kLanes;

  float M = kNegInf, S = 0.f;  // running log2-sum-exp of this lane's share of the row
  for (int k0 = 0; k0 <= last_row; k0 += kTK) {
    // stage a2 over the tile keys and r2 over offsets [i0-k0-kTK+1, i0+kRows-1-k0]
    const int dmin = i0 - k0 - (kTK - 1);
    float lmax_a = kNegInf, lmax_r = kNegInf;
    for (int x = threadIdx.x; x < kTK; x += NT) {
      const int k = k0 + x;
      const float v = (k < T) ? arow[k] * kLog2e : kNegInf;
      a2s[x] = v;
      lmax_a = fmaxf(lmax_a, v);
    }
    for (int x = threadIdx.x; x < kBand; x += NT) {
      const int d = dmin + x;
      const float v = (d >= 0 && d < T) ? rrow[d] * kLog2e : kNegInf;
      r2s[x] = v;
      lmax_r = fmaxf(lmax_r, v);
    }
    // shifts; an all -inf tile (possible only for -inf inputs) shifts by 0
    float ma = lmax_a, mr = lmax_r;
    block_max2(ma, mr, red);
    if (ma == kNegInf) ma = 0.f;
    if (mr == kNegInf) mr = 0.f;
    for (int x = threadIdx.x; x < kTK; x += NT) eas[x] = fast_exp2(a2s[x] - ma);
    for (int x = threadIdx.x; x < kBand; x += NT) ers[x] = fast_exp2(r2s[x] - mr);
    __syncthreads();

    if (i < T && k0 + kl <= i) {
      const int kend = min(kTK - 1, i - k0);  // last tile-local key of this row
      const int xb = i - k0 - dmin;           // band index of offset i - k0
      float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
      int x = kl;
      for (; x + 3 * kLanes <= kend; x += 4 * kLanes) {
        s0 = fmaf(eas[x], ers[xb - x], s0);
        s1 = fmaf(eas[x + kLanes], ers[xb - x - kLanes], s1);
        s2 = fmaf(eas[x + 2 * kLanes], ers[xb - x - 2 * kLanes], s2);
        s3 = fmaf(eas[x + 3 * kLanes], ers[xb - x - 3 * kLanes], s3);
      }
      for (; x <= kend; x += kLanes) s0 = fmaf(eas[x], ers[xb - x], s0);
      const float s = (s0 + s1) + (s2 + s3);
      float cm, cs;
      if (s >= 0x1p-20f) {
        cm = ma + mr;
        cs = s;
      } else {
        // exact fallback: max-shifted sum of this lane's terms in the tile
        cm = kNegInf;
        for (int x = kl; x <= kend; x += kLanes) cm = fmaxf(cm, a2s[x] + r2s[xb - x]);
        cs = 0.f;
        if (cm != kNegInf)
          for (int x = kl; x <= kend; x += kLanes) cs += fast_exp2(a2s[x] + r2s[xb - x] - cm);
      }
      if (cs > 0.f) {
        const float Mn = fmaxf(M, cm);
        S = S * fast_exp2(M - Mn) + cs * fast_exp2(cm - Mn);
        M = Mn;
      }
    }
    __syncthreads();
  }
  cm_s[kl][row] = M;
  cs_s[kl][row] = S;
  __syncthreads();
  if (kl == 0 && i < T) {
    float Mt = kNegInf;
    for (int x = 0; x < kLanes; ++x)
      if (cs_s[x][row] > 0.f) Mt = fmaxf(Mt, cm_s[x][row]);
    float St = 0.f;
    for (int x = 0; x < kLanes; ++x)
      if (cs_s[x][row] > 0.f) St += cs_s[x][row] * fast_exp2(cm_s[x][row] - Mt);
    const float lz = (Mt + fast_log2(St)) * kLn2;  // natural log
    for (int b = 0; b < A.B; ++b)
      A.out[(int64_t)b * A.out_b_stride + (int64_t)h * A.out_h_stride + i] = lz;
  }
}

// Dense eager pattern of one head: row i per block, exact max-shifted sum.
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
  hipLaunchKernelGGL(lognorm_kernel, grid, dim3(kRows * kLanes), 0, stream, args, 0);
  return hipGetLastError();
}

hipError_t launch_lognorm_identity(const LognormArgs& args, hipStream_t stream) {
  if (args.n_heads <= 0 || args.T <= 0) return hipSuccess;
  dim3 grid((args.T + kRows - 1) / kRows, args.n_heads);
  hipLaunchKernelGGL(lognorm_kernel, grid, dim3(kRows * kLanes), 0, stream, args, 1);
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
