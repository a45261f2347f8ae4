// fp32 path of the SAF hybrid attention layer: plain FMA kernels, one thread
// per row, for small fp32 workloads and fp32 parity checks.  Same
// mathematics as the bf16 path ("When Can Attention Heads Be Statically
// Defined?", Section 3.2 Equation 3, Section 3.3, Appendix A.1 Equations 5-7,
// Appendix D.2), everything in fp32.
//   forward : ordinary rows use a two-pass softmax (row maximum, then
//             normalised weighted sum); frozen rows apply
//             W[i][j] = exp(a[j] + r[i-j] - log N(i)) with log N from lse.
//   backward: delta per row; dK, dV per key row (loop over queries i >= j);
//             dQ per query row (loop over keys j <= i).
#include "saf_internal.h"
#include "saf_device.h"

namespace saf {
namespace {

constexpr int kRowsPerBlock = 64;

template <int D>
__device__ __forceinline__ void load_row(float (&x)[D], const float* p) {
#pragma unroll
  for (int d = 0; d < D; ++d) x[d] = p[d];
}

template <int D>
__device__ __forceinline__ float dot_row(const float (&x)[D], const float* p) {
  float s = 0.f;
#pragma unroll
  for (int d = 0; d < D; ++d) s = fmaf(x[d], p[d], s);
  return s;
}

__device__ __forceinline__ const float* rowp(const TensorRef& t, int b, int h, int i) {
  return (const float*)t.ptr + (int64_t)b * t.sb + (int64_t)h * t.sh + (int64_t)i * t.st;
}
__device__ __forceinline__ float* rowp_w(const TensorRef& t, int b, int h, int i) {
  return (float*)t.ptr + (int64_t)b * t.sb + (int64_t)h * t.sh + (int64_t)i * t.st;
}

// The head kind is looked up from the head lists in the argument block.
__device__ __forceinline__ bool head_is_frozen(const uint8_t* frz, int n_frz, int h) {
  for (int x = 0; x < n_frz; ++x)
    if (frz[x] == h) return true;
  return false;
}

// Grid: (ceil(T/64), B*H), one thread per query row.
template <int D>
__global__ __launch_bounds__(kRowsPerBlock) void fwd_f32(FwdArgs A) {
  const int bh = blockIdx.y;
  const int b = bh / A.H, h = bh - b * A.H;
  const int hk = h / A.kv_group;  // key/value head of this query head
  const int hq = A.qk_slot[h];    // its Q slot
  const int kk = A.kv_group == 1 ? hq : hk;  // its K slot
  const int i = blockIdx.x * kRowsPerBlock + threadIdx.x;
  const int T = A.T;
  if (i >= T) return;
  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  float* orow = rowp_w(A.o, b, h, i);
  if (head_is_frozen(A.frz_heads, A.n_frz, h)) {
    const float* arow = A.a + (int64_t)h * A.prior_len;
    const float* rrow = A.r + (int64_t)h * A.prior_len;
    float* lrow = A.lse + ((int64_t)b * A.H + h) * T;
    if (A.logz) lrow[i] = A.logz[(int64_t)h * T + i];  // the caller's precomputed log N
    const float z2 = lrow[i] * kLog2e;
    for (int j = 0; j <= i; ++j) {
      const float wv = fast_exp2((arow[j] + rrow[i - j]) * kLog2e - z2);
      const float* vr = rowp(A.v, b, hk, j);
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(wv, vr[d], acc[d]);
    }
#pragma unroll
    for (int d = 0; d < D; ++d) orow[d] = acc[d];
    return;
  }
  float q[D];
  load_row<D>(q, rowp(A.q, b, hq, i));
  float m = kNegInf;
  for (int j = 0; j <= i; ++j) m = fmaxf(m, dot_row<D>(q, rowp(A.k, b, kk, j)) * A.scale_log2);
  float lsum = 0.f;
  for (int j = 0; j <= i; ++j) {
    const float p = fast_exp2(dot_row<D>(q, rowp(A.k, b, kk, j)) * A.scale_log2 - m);
    lsum += p;
    const float* vr = rowp(A.v, b, hk, j);
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vr[d], acc[d]);
  }
  const float inv = 1.f / lsum;
#pragma unroll
  for (int d = 0; d < D; ++d) orow[d] = acc[d] * inv;
  A.lse[((int64_t)b * A.H + h) * T + i] = (m + fast_log2(lsum)) * kLn2;
}

template <int D>
__global__ __launch_bounds__(kRowsPerBlock) void bwd_pre_f32(BwdArgs A) {
  const int bh = blockIdx.y;
  const int b = bh / A.H, h = bh - b * A.H;
  const int i = blockIdx.x * kRowsPerBlock + threadIdx.x;
  if (i >= A.T) return;
  if (A.is_frozen[h]) {
    if (A.qk_packed) return;  // no dQ/dK rows for frozen heads
    float* dq = rowp_w(A.dq, b, h, i);
    float* dk = rowp_w(A.dk, b, h, i);
#pragma unroll
    for (int d = 0; d < D; ++d) {
      dq[d] = 0.f;
      dk[d] = 0.f;
    }
    return;
  }
  const float* o = rowp(A.o, b, h, i);
  const float* g = rowp(A.dout, b, h, i);
  float s = 0.f;
#pragma unroll
  for (int d = 0; d < D; ++d) s = fmaf(o[d], g[d], s);
  A.delta[((int64_t)b * A.H + h) * A.T + i] = s;
}

template <int D>
__global__ __launch_bounds__(kRowsPerBlock) void bwd_kv_f32(BwdArgs A) {
  const int bh = blockIdx.y;
  const int b = bh / A.H, h = bh - b * A.H;
  const int j = blockIdx.x * kRowsPerBlock + threadIdx.x;
  const int T = A.T;
  if (j >= T) return;
  const float* lse = A.lse + ((int64_t)b * A.H + h) * T;
  float dv[D];
#pragma unroll
  for (int d = 0; d < D; ++d) dv[d] = 0.f;
  float* dvrow = rowp_w(A.dv, b, h, j);
  if (A.is_frozen[h]) {
    const float* arow = A.a + (int64_t)h * A.prior_len;
    const float* rrow = A.r + (int64_t)h * A.prior_len;
    for (int i = j; i < T; ++i) {
      const float wv = fast_exp2((arow[j] + rrow[i - j]) * kLog2e - lse[i] * kLog2e);
      const float* g = rowp(A.dout, b, h, i);
#pragma unroll
      for (int d = 0; d < D; ++d) dv[d] = fmaf(wv, g[d], dv[d]);
    }
#pragma unroll
    for (int d = 0; d < D; ++d) dvrow[d] = dv[d];
    return;
  }
  const float* dl = A.delta + ((int64_t)b * A.H + h) * T;
  float k[D], v[D], dk[D];
  const int hs = A.qk_slot[h];  // Q/K/dQ/dK slot of this head
  load_row<D>(k, rowp(A.k, b, hs, j));
  load_row<D>(v, rowp(A.v, b, h, j));
#pragma unroll
  for (int d = 0; d < D; ++d) dk[d] = 0.f;
  for (int i = j; i < T; ++i) {
    const float* qr = rowp(A.q, b, hs, i);
    const float* g = rowp(A.dout, b, h, i);
    const float p = fast_exp2(dot_row<D>(k, qr) * A.scale_log2 - lse[i] * kLog2e);
    const float dp = dot_row<D>(v, g);
    const float ds = p * (dp - dl[i]);
#pragma unroll
    for (int d = 0; d < D; ++d) {
      dv[d] = fmaf(p, g[d], dv[d]);
      dk[d] = fmaf(ds, qr[d], dk[d]);
    }
  }
  float* dkrow = rowp_w(A.dk, b, hs, j);
#pragma unroll
  for (int d = 0; d < D; ++d) {
    dvrow[d] = dv[d];
    dkrow[d] = dk[d] * A.scale;
  }
}

template <int D>
__global__ __launch_bounds__(kRowsPerBlock) void bwd_q_f32(BwdArgs A) {
  const int bh = blockIdx.y;
  const int b = bh / A.H, h = bh - b * A.H;
  const int i = blockIdx.x * kRowsPerBlock + threadIdx.x;
  const int T = A.T;
  if (i >= T || A.is_frozen[h]) return;
  const int64_t rv = ((int64_t)b * A.H + h) * T + i;
  const float l2 = A.lse[rv] * kLog2e;
  const float dl = A.delta[rv];
  float q[D], g[D], dq[D];
  const int hs = A.qk_slot[h];  // Q/K/dQ/dK slot of this head
  load_row<D>(q, rowp(A.q, b, hs, i));
  load_row<D>(g, rowp(A.dout, b, h, i));
#pragma unroll
  for (int d = 0; d < D; ++d) dq[d] = 0.f;
  for (int j = 0; j <= i; ++j) {
    const float* kr = rowp(A.k, b, hs, j);
    const float p = fast_exp2(dot_row<D>(q, kr) * A.scale_log2 - l2);
    const float ds = p * (dot_row<D>(g, rowp(A.v, b, h, j)) - dl);
#pragma unroll
    for (int d = 0; d < D; ++d) dq[d] = fmaf(ds, kr[d], dq[d]);
  }
  float* out = rowp_w(A.dq, b, hs, i);
#pragma unroll
  for (int d = 0; d < D; ++d) out[d] = dq[d] * A.scale;
}

#define SAF_F32_DISPATCH(NAME, ARGT)                                                   \
  hipError_t NAME##_launch(const ARGT& args, int D, hipStream_t stream) {               \
    dim3 grid((args.T + kRowsPerBlock - 1) / kRowsPerBlock, args.B * args.H);           \
    switch (D) {                                                                        \
      case 16: hipLaunchKernelGGL(NAME<16>, grid, dim3(kRowsPerBlock), 0, stream, args); break; \
      case 32: hipLaunchKernelGGL(NAME<32>, grid, dim3(kRowsPerBlock), 0, stream, args); break; \
      case 64: hipLaunchKernelGGL(NAME<64>, grid, dim3(kRowsPerBlock), 0, stream, args); break; \
      case 96: hipLaunchKernelGGL(NAME<96>, grid, dim3(kRowsPerBlock), 0, stream, args); break; \
      case 128: hipLaunchKernelGGL(NAME<128>, grid, dim3(kRowsPerBlock), 0, stream, args); break; \
      default: return hipErrorInvalidValue;                                             \
    }                                                                                   \
    return hipGetLastError();                                                           \
  }

SAF_F32_DISPATCH(fwd_f32, FwdArgs)
SAF_F32_DISPATCH(bwd_pre_f32, BwdArgs)
SAF_F32_DISPATCH(bwd_kv_f32, BwdArgs)
SAF_F32_DISPATCH(bwd_q_f32, BwdArgs)

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& args, int D, hipStream_t stream) {
  return fwd_f32_launch(args, D, stream);
}
hipError_t launch_bwd_pre_f32(const BwdArgs& args, int D, hipStream_t stream) {
  return bwd_pre_f32_launch(args, D, stream);
}
hipError_t launch_bwd_kv_f32(const BwdArgs& args, int D, hipStream_t stream) {
  return bwd_kv_f32_launch(args, D, stream);
}
hipError_t launch_bwd_q_f32(const BwdArgs& args, int D, hipStream_t stream) {
  return bwd_q_f32_launch(args, D, stream);
}

}  // namespace saf
