// Calibration statistics of ordinary attention heads ("When Can Attention
// Heads Be Statically Defined?", Section 3.1, Equations 1 and 2; the
// attention of Appendix A.1, Equations 5-6), bf16 inputs, gfx950.
//
// Over N calibration sequences of one head, with A^(n) the causal row softmax
// of scale * Q^(n) K^(n)T:
//   A-hat = N^-1 sum_n A^(n)                                  (mean)
//   s_var = sum_n ||A^(n) - A-hat||_F^2 / ((N - 1) T^2)         (Equation 1)
//   s_KL  = (N T)^-1 sum_n sum_i KL(A^(n)[i] || A-hat[i])      (Equation 2)
// in one pass over the sequences and without storing any A^(n):
//   calib_lse_kernel    program (query block, head, sequence): the row
//                       log-sum-exp of the scores (log2 units), with K tiles
//                       streamed through LDS as in the forward.
//   calib_stats_kernel  program (query block, key tile, head): for each
//                       sequence in turn the 128 x 64 score tile is
//                       recomputed on MFMA, A = exp2(s - lse), and every
//                       entry's sums of deviations from its first
//                       sequence's value, s1 = sum (A - A0) and s2 =
//                       sum (A - A0)^2, are accumulated in registers (the
//                       shifted-data algorithm of Chan, Golub and LeVeque:
//                       mean = A0 + s1/N, sum of squared deviations =
//                       s2 - s1^2/N, stable because A0 is one of the
//                       samples), so the variance needs no second pass;
//                       sum A log A is accumulated on the way.  Since log A-hat does not
//                       depend on n, sum_n KL(A^(n) || A-hat) =
//                       sum_n sum A log A - N sum A-hat log A-hat, which the
//                       program completes from its final mean.  The tile's
//                       mean is stored once; per-program sums (fp64) go to
//                       the workspace.
//   calib_reduce_kernel one block per head: fixed-order sums of the
//                       programs' partials, then both scores.
// Products are transposed (S^T = K Q^T) so that a lane owns one query: lane
// l of wave w holds query q0 + 32 w + l % 32 and keys
// j0 + 32 c + 8 (r / 4) + 4 (l / 32) + r % 4 of its two accumulators.
#include <type_traits>

#include "saf_internal.h"
#include "saf_tile.h"

namespace saf {
namespace {

constexpr int kBM = kCalibBM;  // queries per program (4 waves x 32)
constexpr int kBN = kCalibBN;  // keys per tile

template <int D>
struct CalCfg {
  using L = LdsLayout<D>;
  static constexpr int NKS = D / 16;
  static constexpr int TILE = kBN * L::PITCH;
};

template <int D>
__device__ __forceinline__ void load_q(const CalibArgs& A, int n, int h, int i, bf16x8* qf) {
  const int hl = lane_id() >> 5;
  const __bf16* qg = (const __bf16*)A.q.ptr + (int64_t)n * A.q.sb + (int64_t)h * A.q.sh;
  const int ic = i < A.T ? i : A.T - 1;  // rows past T read row T-1 (unused)
#pragma unroll
  for (int ks = 0; ks < CalCfg<D>::NKS; ++ks)
    qf[ks] = __builtin_bit_cast(bf16x8, gload16(qg + (int64_t)ic * A.q.st + 16 * ks + 8 * hl));
}

template <int D>
__device__ __forceinline__ void score_tile(const lds_bf16* K, const bf16x8* qf, f32x16* s) {
  using C = CalCfg<D>;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    s[c] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) s[c] = mfma32(lds_frag_nat<D>(K, 32 * c, 16 * ks), qf[ks], s[c]);
  }
}

// ---------------------------------------------------------------------------
// Pass 1: row log-sum-exp (log2 units) of every sequence's scores.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void calib_lse_kernel(CalibArgs A) {
  using C = CalCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 smem_raw[2 * C::TILE];
  lds_bf16* smem = (lds_bf16*)smem_raw;
  const int qb = blockIdx.x, h = blockIdx.y, n = blockIdx.z;
  const int l = lane_id(), w = wave_id(), hl = l >> 5;
  const int T = A.T;
  const int q0 = qb * kBM;
  const int i = q0 + 32 * w + (l & 31);
  const float sl2 = A.scale_log2;
  bf16x8 qf[C::NKS];
  load_q<D>(A, n, h, i, qf);
  const __bf16* kg = (const __bf16*)A.k.ptr + (int64_t)n * A.k.sb + (int64_t)h * A.k.sh;
  const int ntiles = (min(q0 + kBM, T) - 1) / kBN + 1;
  TileDma<D, kBN> kdma;
  kdma.init(A.k.st);
  kdma.issue(kg, A.k.st, 0, T, smem);
  wait_vm_loads();
  __syncthreads();
  // Online log-sum-exp with a lazy reference maximum (as in the forward):
  // exponentials are taken against m (log2 units) and the tile maximum is
  // only formed when a lane's sum exceeds 2^8 (the first tile, a grown
  // maximum, or a rare false alarm); the result is exact for any reference.
  float m = kNegInf, sum = 0.f;
  auto tile = [&](int t, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int j0 = t * kBN;
    const bool more = t + 1 < ntiles;
    if (more) kdma.issue(kg, A.k.st, j0 + kBN, T, smem + ((t + 1) & 1) * C::TILE);
    f32x16 s[2];
    score_tile<D>(smem + (t & 1) * C::TILE, qf, s);
    if constexpr (MASK) {
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + 32 * c + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (j > i) s[c][r] = kNegInf;
        }
    }
    auto exps = [&](float ref) {
      float ps = 0.f;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) ps += fast_exp2(fmaf(s[c][r], sl2, -ref));
      return ps;
    };
    float ps = exps(m);
    if (__any(!(ps <= 256.f))) {
      asm volatile("");
      float mx = kNegInf;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[c][r]);
      const float mn = fmaxf(m, mx * sl2);
      if (mn > kNegInf) {
        sum *= fast_exp2(m - mn);
        m = mn;
        ps = exps(m);
      } else {
        ps = 0.f;  // no key of this tile reaches the lane's query yet
      }
    }
    sum += ps;
    if (more) wait_vm_loads();
    __syncthreads();
  };
  // tiles wholly below the block's first query need no mask
  const int t_diag = min(q0 / kBN, ntiles);
  int t = 0;
  for (; t < t_diag; ++t) tile(t, std::false_type{});
  for (; t < ntiles; ++t) tile(t, std::true_type{});
  // merge the two halves of the lane pair that share a query
  const float mo = xor32(m), so = xor32(sum);
  const float mt = fmaxf(m, mo);
  const float st = (sum > 0.f ? sum * fast_exp2(m - mt) : 0.f) + (so > 0.f ? so * fast_exp2(mo - mt) : 0.f);
  if (hl == 0 && i < T) A.lse2[((int64_t)n * A.H + h) * T + i] = mt + fast_log2(st);
}

// ---------------------------------------------------------------------------
// Pass 2: running mean and squared deviations of every entry over the
// sequences.
// ---------------------------------------------------------------------------

// Fixed-order sum of three doubles over the block (4 waves); thread 0 gets it.
__device__ __forceinline__ void block_sum3(double& a, double& b, double& c, double* red) {
  for (int o = 32; o >= 1; o >>= 1) {
    a += __shfl_xor(a, o, 64);
    b += __shfl_xor(b, o, 64);
    c += __shfl_xor(c, o, 64);
  }
  if (lane_id() == 0) {
    red[3 * wave_id() + 0] = a;
    red[3 * wave_id() + 1] = b;
    red[3 * wave_id() + 2] = c;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    a = (red[0] + red[3]) + (red[6] + red[9]);
    b = (red[1] + red[4]) + (red[7] + red[10]);
    c = (red[2] + red[5]) + (red[8] + red[11]);
  }
}

template <int D>
__global__ __launch_bounds__(256) void calib_stats_kernel(CalibArgs A) {
  using C = CalCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 smem_raw[2 * C::TILE];
  __shared__ double red[12];
  lds_bf16* smem = (lds_bf16*)smem_raw;
  const int T = A.T;
  const int h = blockIdx.y;
  // program x -> (query block qb, key tile kt), kt < 2 (qb + 1): the causal
  // tiles of query block qb number 2 (qb + 1), so qb's first program is
  // qb (qb + 1)
  const int x = blockIdx.x;
  int qb = (int)((sqrtf(4.f * (float)x + 1.f) - 1.f) * 0.5f);
  while ((qb + 1) * (qb + 2) <= x) ++qb;
  while (qb * (qb + 1) > x) --qb;
  const int kt = x - qb * (qb + 1);
  const int q0 = qb * kBM, j0 = kt * kBN;
  if (j0 >= T) {  // whole block: a tile past the last key contributes nothing
    if (threadIdx.x == 0) {
      double* p = A.part + ((int64_t)h * A.nprog + x) * 3;
      p[0] = p[1] = p[2] = 0.0;
    }
    return;
  }
  const int l = lane_id(), w = wave_id(), hl = l >> 5;
  const int i = q0 + 32 * w + (l & 31);
  const float sl2 = A.scale_log2;

  // shifted sums (shift = the first sequence's value): s1 = sum (a - a0),
  // s2 = sum (a - a0)^2
  f32x16 a0[2], s1[2], s2[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    a0[c] = f32x16{};
    s1[c] = f32x16{};
    s2[c] = f32x16{};
  }
  double alogA = 0.0;  // sum over sequences of this lane's A log2 A
  // causal entries of this lane: key j <= i (and i < T)
  auto valid = [&](int c, int r) {
    const int j = j0 + 32 * c + 8 * (r >> 2) + 4 * hl + (r & 3);
    return j <= i && i < T;
  };

  TileDma<D, kBN> kdma;
  kdma.init(A.k.st);
  auto kbase = [&](int n) { return (const __bf16*)A.k.ptr + (int64_t)n * A.k.sb + (int64_t)h * A.k.sh; };
  const float* lse_h = A.lse2 + (int64_t)h * T;
  const int ic = i < T ? i : T - 1;
  bf16x8 qf[C::NKS], qn[C::NKS];
  load_q<D>(A, 0, h, i, qf);
  float lse = lse_h[ic];
  kdma.issue(kbase(0), A.k.st, j0, T, smem);
  wait_vm_loads();
  __syncthreads();
  // tiles wholly below the diagonal, in query blocks inside [0, T), need no mask
  const bool nomask = j0 + kBN - 1 <= q0 && q0 + kBM <= T;
  auto step = [&](auto mask_tag, auto first_tag, int n) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr bool FIRST = decltype(first_tag)::value;
    const bool more = n + 1 < A.N;
    float lse_n = 0.f;
    if (more) {
      kdma.issue(kbase(n + 1), A.k.st, j0, T, smem + ((n + 1) & 1) * C::TILE);
      load_q<D>(A, n + 1, h, i, qn);
      lse_n = lse_h[(int64_t)(n + 1) * A.H * T + ic];
    }
    f32x16 s[2];
    score_tile<D>(smem + (n & 1) * C::TILE, qf, s);
    float alog = 0.f;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool ok = !MASK || valid(c, r);
        const float xl = fmaf(s[c][r], sl2, -lse);  // log2 A
        const float a = ok ? fast_exp2(xl) : 0.f;
        alog = ok ? fmaf(a, xl, alog) : alog;
        if constexpr (FIRST) {
          a0[c][r] = a;
        } else {
          const float d = a - a0[c][r];
          s1[c][r] += d;
          s2[c][r] = fmaf(d, d, s2[c][r]);
        }
      }
    alogA += (double)alog;
    if (more) {
#pragma unroll
      for (int ks = 0; ks < C::NKS; ++ks) qf[ks] = qn[ks];
      lse = lse_n;
      wait_vm_loads();
    }
    __syncthreads();
  };
  if (nomask) {
    step(std::false_type{}, std::true_type{}, 0);
    for (int n = 1; n < A.N; ++n) step(std::false_type{}, std::false_type{}, n);
  } else {
    step(std::true_type{}, std::true_type{}, 0);
    for (int n = 1; n < A.N; ++n) step(std::true_type{}, std::false_type{}, n);
  }
  const float invN = 1.f / (float)A.N;
  f32x16 mean[2], m2[2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      mean[c][r] = fmaf(s1[c][r], invN, a0[c][r]);
      m2[c][r] = fmaf(-s1[c][r], s1[c][r] * invN, s2[c][r]);
    }

  // store the mean of the causal entries; sums for the scores
  double sm2 = 0.0, shat = 0.0;
  float* arow = A.ahat + (int64_t)h * A.head_a + (int64_t)ic * A.ld_a;
  // every key of the tile precedes every query, and rows start 16-byte aligned
  const bool below = j0 + kBN - 1 <= q0 && A.ahat_vec;
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int jb = j0 + 32 * c + 8 * q4 + 4 * hl;
      if (below && i < T) {
        const f32x4 v = {mean[c][4 * q4], mean[c][4 * q4 + 1], mean[c][4 * q4 + 2], mean[c][4 * q4 + 3]};
        *reinterpret_cast<f32x4*>(arow + jb) = v;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (jb + e <= i && i < T) arow[jb + e] = mean[c][4 * q4 + e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * q4 + e;
        if (valid(c, r)) {
          sm2 += (double)fmaxf(m2[c][r], 0.f);
          const float mu = mean[c][r];
          if (mu > 0.f) shat += (double)(mu * fast_log2(mu));
        }
      }
    }
  block_sum3(sm2, alogA, shat, red);
  if (threadIdx.x == 0) {
    double* p = A.part + ((int64_t)h * A.nprog + x) * 3;
    p[0] = sm2;
    p[1] = alogA;
    p[2] = shat;
  }
}

__global__ __launch_bounds__(256) void calib_reduce_kernel(CalibArgs A) {
  __shared__ double red[12];
  const int h = blockIdx.x;
  const double* p = A.part + (int64_t)h * A.nprog * 3;
  double a = 0.0, b = 0.0, c = 0.0;
  for (int x = threadIdx.x; x < A.nprog; x += blockDim.x) {
    a += p[3 * x];
    b += p[3 * x + 1];
    c += p[3 * x + 2];
  }
  block_sum3(a, b, c, red);
  if (threadIdx.x == 0) {
    const double N = (double)A.N, T = (double)A.T;
    A.s_var[h] = A.N > 1 ? a / ((N - 1.0) * T * T) : 0.0;
    // sum_n KL = sum_n sum A ln A - N sum A-hat ln A-hat (log2 sums times ln 2)
    A.s_kl[h] = (b - N * c) * 0.6931471805599453 / (N * T);
  }
}

template <int D>
hipError_t launch_calib_d(const CalibArgs& A, hipStream_t stream) {
  hipLaunchKernelGGL(calib_lse_kernel<D>, dim3(A.nqb, A.H, A.N), dim3(256), 0, stream, A);
  hipLaunchKernelGGL(calib_stats_kernel<D>, dim3(A.nprog, A.H), dim3(256), 0, stream, A);
  hipLaunchKernelGGL(calib_reduce_kernel, dim3(A.H), dim3(256), 0, stream, A);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_calib(const CalibArgs& args, int D, hipStream_t stream) {
  switch (D) {
    case 64: return launch_calib_d<64>(args, stream);
    case 96: return launch_calib_d<96>(args, stream);
    case 128: return launch_calib_d<128>(args, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace saf
