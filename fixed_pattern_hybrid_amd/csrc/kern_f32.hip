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
// A row is one thread for d <= 64 and a pair of neighbouring threads for
// d = 96, 128 (each holds half of the row's d values and the pair adds its
// halves of every dot product), so that no kernel keeps more than 4 x 64
// fp32 values per thread live.
#include "saf_internal.h"
#include "saf_device.h"

namespace saf {
namespace {

constexpr int kRowsPerBlock = 64;  // threads per block

// threads per row (S), d values per thread (DD), rows per block (RPB)
template <int D>
struct RowSplit {
  static constexpr int S = D > 64 ? 2 : 1;
  static constexpr int DD = D / S;
  static constexpr int RPB = kRowsPerBlock / S;
};

// A row's dot product from this thread's part: both threads of a pair get
// the same sum (the two additions are the same two operands).
template <int S>
__device__ __forceinline__ float pair_sum(float x) {
  if constexpr (S == 2) return x + __shfl_xor(x, 1, 64);
  else return x;
}

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

// Grid: (ceil(T/RPB), B*H); a query row per thread (or thread pair).
template <int D>
__global__ __launch_bounds__(kRowsPerBlock) void fwd_f32(FwdArgs A) {
  using RS = RowSplit<D>;
  constexpr int DD = RS::DD;
  const int bh = blockIdx.y;
  const int b = bh / A.H, h = bh - b * A.H;
  const int hk = h / A.kv_group;  // key/value head of this query head
  const int hq = A.qk_slot[h];    // its Q slot
  const int kk = A.kv_group == 1 ? hq : hk;  // its K slot
  const int i = blockIdx.x * RS::RPB + (int)threadIdx.x / RS::S;
  const int part = (int)threadIdx.x % RS::S, o = part * DD;  // this thread's d values: o .. o+DD-1
  const int T = A.T;
  if (i >= T) return;  // both threads of a pair
  float acc[DD];
#pragma unroll
  for (int d = 0; d < DD; ++d) acc[d] = 0.f;
  float* orow = rowp_w(A.o, b, h, i) + o;
  if (head_is_frozen(A.frz_heads, A.n_frz, h)) {
    const float* arow = A.a + (int64_t)h * A.prior_len;
    const float* rrow = A.r + (int64_t)h * A.prior_len;
    float* lrow = A.lse + ((int64_t)b * A.H + h) * T;
    const float lz = A.logz ? A.logz[(int64_t)h * T + i] : lrow[i];  // the caller's precomputed log N
    if (A.logz && part == 0) lrow[i] = lz;
    const float z2 = lz * kLog2e;
    for (int j = 0; j <= i; ++j) {
      const float wv = fast_exp2((arow[j] + rrow[i - j]) * kLog2e - z2);
      const float* vr = rowp(A.v, b, hk, j) + o;
#pragma unroll
      for (int d = 0; d < DD; ++d) acc[d] = fmaf(wv, vr[d], acc[d]);
    }
#pragma unroll
    for (int d = 0; d < DD; ++d) orow[d] = acc[d];
    return;
  }
  float q[DD];
  load_row<DD>(q, rowp(A.q, b, hq, i) + o);
  float m = kNegInf;
  for (int j = 0; j <= i; ++j)
    m = fmaxf(m, pair_sum<RS::S>(dot_row<DD>(q, rowp(A.k, b, kk, j) + o)) * A.scale_log2);
  float lsum = 0.f;
  for (int j = 0; j <= i; ++j) {
    const float p = fast_exp2(pair_sum<RS::S>(dot_row<DD>(q, rowp(A.k, b, kk, j) + o)) * A.scale_log2 - m);
    lsum += p;
    const float* vr = rowp(A.v, b, hk, j) + o;
#pragma unroll
    for (int d = 0; d < DD; ++d) acc[d] = fmaf(p, vr[d], acc[d]);
  }
  const float inv = 1.f / lsum;
#pragma unroll
  for (int d = 0; d < DD; ++d) orow[d] = acc[d] * inv;
  if (part == 0) A.lse[((int64_t)b * A.H + h) * T + i] = (m + fast_log2(lsum)) * kLn2;
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
  using RS = RowSplit<D>;
  constexpr int DD = RS::DD;
  const int bh = blockIdx.y;
  const int b = bh / A.H, h = bh - b * A.H;
  const int j = blockIdx.x * RS::RPB + (int)threadIdx.x / RS::S;
  const int o = ((int)threadIdx.x % RS::S) * DD;  // this thread's d values
  const int T = A.T;
  if (j >= T) return;  // both threads of a pair
  const float* lse = A.lse + ((int64_t)b * A.H + h) * T;
  float dv[DD];
#pragma unroll
  for (int d = 0; d < DD; ++d) dv[d] = 0.f;
  float* dvrow = rowp_w(A.dv, b, h, j) + o;
  if (A.is_frozen[h]) {
    const float* arow = A.a + (int64_t)h * A.prior_len;
    const float* rrow = A.r + (int64_t)h * A.prior_len;
    for (int i = j; i < T; ++i) {
      const float wv = fast_exp2((arow[j] + rrow[i - j]) * kLog2e - lse[i] * kLog2e);
      const float* g = rowp(A.dout, b, h, i) + o;
#pragma unroll
      for (int d = 0; d < DD; ++d) dv[d] = fmaf(wv, g[d], dv[d]);
    }
#pragma unroll
    for (int d = 0; d < DD; ++d) dvrow[d] = dv[d];
    return;
  }
  const float* dl = A.delta + ((int64_t)b * A.H + h) * T;
  float k[DD], v[DD], dk[DD];
  const int hs = A.qk_slot[h];  // Q/K/dQ/dK slot of this head
  load_row<DD>(k, rowp(A.k, b, hs, j) + o);
  load_row<DD>(v, rowp(A.v, b, h, j) + o);
#pragma unroll
  for (int d = 0; d < DD; ++d) dk[d] = 0.f;
  for (int i = j; i < T; ++i) {
    const float* qr = rowp(A.q, b, hs, i) + o;
    const float* g = rowp(A.dout, b, h, i) + o;
    const float p = fast_exp2(pair_sum<RS::S>(dot_row<DD>(k, qr)) * A.scale_log2 - lse[i] * kLog2e);
    const float dp = pair_sum<RS::S>(dot_row<DD>(v, g));
    const float ds = p * (dp - dl[i]);
#pragma unroll
    for (int d = 0; d < DD; ++d) {
      dv[d] = fmaf(p, g[d], dv[d]);
      dk[d] = fmaf(ds, qr[d], dk[d]);
    }
  }
  float* dkrow = rowp_w(A.dk, b, hs, j) + o;
#pragma unroll
  for (int d = 0; d < DD; ++d) {
    dvrow[d] = dv[d];
    dkrow[d] = dk[d] * A.scale;
  }
}

template <int D>
__global__ __launch_bounds__(kRowsPerBlock) void bwd_q_f32(BwdArgs A) {
  using RS = RowSplit<D>;
  constexpr int DD = RS::DD;
  const int bh = blockIdx.y;
  const int b = bh / A.H, h = bh - b * A.H;
  const int i = blockIdx.x * RS::RPB + (int)threadIdx.x / RS::S;
  const int o = ((int)threadIdx.x % RS::S) * DD;  // this thread's d values
  const int T = A.T;
  if (i >= T || A.is_frozen[h]) return;  // both threads of a pair
  const int64_t rv = ((int64_t)b * A.H + h) * T + i;
  const float l2 = A.lse[rv] * kLog2e;
  const float dl = A.delta[rv];
  float q[DD], g[DD], dq[DD];
  const int hs = A.qk_slot[h];  // Q/K/dQ/dK slot of this head
  load_row<DD>(q, rowp(A.q, b, hs, i) + o);
  load_row<DD>(g, rowp(A.dout, b, h, i) + o);
#pragma unroll
  for (int d = 0; d < DD; ++d) dq[d] = 0.f;
  for (int j = 0; j <= i; ++j) {
    const float* kr = rowp(A.k, b, hs, j) + o;
    const float p = fast_exp2(pair_sum<RS::S>(dot_row<DD>(q, kr)) * A.scale_log2 - l2);
    const float ds = p * (pair_sum<RS::S>(dot_row<DD>(g, rowp(A.v, b, h, j) + o)) - dl);
#pragma unroll
    for (int d = 0; d < DD; ++d) dq[d] = fmaf(ds, kr[d], dq[d]);
  }
  float* out = rowp_w(A.dq, b, hs, i) + o;
#pragma unroll
  for (int d = 0; d < DD; ++d) out[d] = dq[d] * A.scale;
}

// RPB(D): rows per block of kernel NAME at head dimension D
#define SAF_F32_DISPATCH(NAME, ARGT, RPB)                                              \
  hipError_t NAME##_launch(const ARGT& args, int D, hipStream_t stream) {               \
    switch (D) {                                                                        \
      case 16: return NAME##_go<16, RPB(16)>(args, stream);                            \
      case 32: return NAME##_go<32, RPB(32)>(args, stream);                            \
      case 64: return NAME##_go<64, RPB(64)>(args, stream);                            \
      case 96: return NAME##_go<96, RPB(96)>(args, stream);                            \
      case 128: return NAME##_go<128, RPB(128)>(args, stream);                         \
      default: return hipErrorInvalidValue;                                             \
    }                                                                                   \
  }

#define SAF_F32_GO(NAME, ARGT)                                                          \
  template <int D, int RPB>                                                             \
  hipError_t NAME##_go(const ARGT& args, hipStream_t stream) {                          \
    dim3 grid((args.T + RPB - 1) / RPB, args.B * args.H);                               \
    hipLaunchKernelGGL(NAME<D>, grid, dim3(kRowsPerBlock), 0, stream, args);             \
    return hipGetLastError();                                                           \
  }

#define SAF_F32_SPLIT_RPB(D) RowSplit<D>::RPB
#define SAF_F32_ROW_RPB(D) kRowsPerBlock

SAF_F32_GO(fwd_f32, FwdArgs)
SAF_F32_GO(bwd_pre_f32, BwdArgs)
SAF_F32_GO(bwd_kv_f32, BwdArgs)
SAF_F32_GO(bwd_q_f32, BwdArgs)

SAF_F32_DISPATCH(fwd_f32, FwdArgs, SAF_F32_SPLIT_RPB)
SAF_F32_DISPATCH(bwd_pre_f32, BwdArgs, SAF_F32_ROW_RPB)
SAF_F32_DISPATCH(bwd_kv_f32, BwdArgs, SAF_F32_SPLIT_RPB)
SAF_F32_DISPATCH(bwd_q_f32, BwdArgs, SAF_F32_SPLIT_RPB)

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
