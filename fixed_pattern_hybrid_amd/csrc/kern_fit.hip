// Fitting a compact pattern to a calibration mean ("When Can Attention Heads
// Be Statically Defined?": Algorithm 1's target preparation, fit and
// acceptance statistic; Section 3.2 "Fitting", Equation 4; Appendix A.2 for
// the initialisation and the Adam settings; Appendix D.1, Equation 20).
//
// Target statistics (HBM-bound; the calibration mean is read three times):
//   fit_rows_kernel   one wave per pair of rows (i, T-1-i), so every wave
//                     reads T+1 causal entries: the row sum s_i of the
//                     entries floored at `floor`, and the row's
//                     sum_j p log p for p = floored / s_i.
//   fit_tmarg_kernel  one thread per column (kind 0) or per diagonal
//                     (kind 1), looping over a segment of kSeg rows: the
//                     diagonal d's entry in row i is column i - d, so both
//                     kinds read a contiguous run of each row.  Per-segment
//                     partial sums go to the workspace.
//   fit_tred_kernel   fixed-order sums of the segment partials (eta_abs,
//                     eta_rel); fit_negent_kernel sums the row entropies.
//
// The fit (two launches per Adam step):
//   the normaliser kernel of the forward writes log N of the current (a, r);
//   fit_step_kernel computes the fitted marginals
//     mu_abs(k) = exp(a_k) * sum_{i >= k} exp(r_{i-k} - z_i)
//     mu_rel(d) = exp(r_d) * sum_{k < T-d} exp(a_k - z_{k+d})
//   for 64 parameters per block (one per lane; kind 0 = a, kind 1 = r), the
//   gradient (mu - eta) / T (Equation 20) and the Adam update, written to
//   the other of two parameter buffers so that every block of a step reads
//   the same point.
//
// The marginal sums factor like the normaliser's: over a chunk of kTK
// summation indices, exp2(X[x] + Y[y]) = 2^(mx + my) exp2(X[x] - mx)
// exp2(Y[y] - my), where X is indexed by the summation index (kind 0: -log2
// N of row i; kind 1: log2 e * a_k) and Y by a band index that moves with
// both the summation index and the lane (kind 0: log2 e * r at offset i - k;
// kind 1: -log2 N of row k + d).  Each term is one FMA on two staged
// exponentials (both <= 1); a lane whose chunk sum falls below 2^-20 is
// recomputed exactly with a max-shifted sum, as in the normaliser.
#include "saf_internal.h"
#include "saf_device.h"
#include "saf_tile.h"

namespace saf {
namespace {

// ---------------------------------------------------------------------------
// Target statistics.
// ---------------------------------------------------------------------------

constexpr int kRowWaves = 4;
constexpr int kTChunk = 256;  // outputs (columns or diagonals) per marginal block
constexpr int kSeg = kFitSegRows;

__device__ __forceinline__ float wave_sum(float v) {
  // butterfly in a fixed order: every lane ends with the same value
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__global__ __launch_bounds__(64 * kRowWaves) void fit_rows_kernel(FitTargetArgs A) {
  const int h = blockIdx.y;
  const int T = A.T;
  const int p = blockIdx.x * kRowWaves + wave_id();
  const int npairs = (T + 1) / 2;
  if (p >= npairs) return;  // no block-level synchronisation below
  const int lane = lane_id();
  const float fl = A.floor;
  for (int pass = 0; pass < 2; ++pass) {
    const int i = pass == 0 ? p : T - 1 - p;
    if (pass == 1 && i == p) break;
    const float* row = A.ahat + (int64_t)h * A.head_stride + (int64_t)i * A.row_stride;
    float s = 0.f, t = 0.f;
    auto take = [&](float v) {
      const float x = fmaxf(v, fl);
      s += x;
      t = fmaf(x, fast_log2(x), t);
    };
    if ((reinterpret_cast<uintptr_t>(row) & 15) == 0) {
      // 16-byte reads; the last partial group of four is read by element
      for (int j = 4 * lane; j <= i; j += 256) {
        if (j + 3 <= i) {
          const f32x4 q = *reinterpret_cast<const f32x4*>(row + j);
          take(q[0]);
          take(q[1]);
          take(q[2]);
          take(q[3]);
        } else {
          for (int e = 0; j + e <= i; ++e) take(row[j + e]);
        }
      }
    } else {
      for (int j = lane; j <= i; j += 64) take(row[j]);
    }
    s = wave_sum(s);
    t = wave_sum(t);
    if (lane == 0) {
      const float inv = 1.f / s;
      A.inv_s[(int64_t)h * T + i] = inv;
      // sum_j (x_j / s) ln(x_j / s) = (sum_j x_j ln x_j) / s - ln s
      A.row_ent[(int64_t)h * T + i] = (t * inv - fast_log2(s)) * kLn2;
    }
  }
}

__global__ __launch_bounds__(kTChunk) void fit_tmarg_kernel(FitTargetArgs A) {
  const int T = A.T;
  const int kind = blockIdx.z & 1;
  const int h = blockIdx.z >> 1;
  const int c0 = blockIdx.x * kTChunk;
  const int seg = blockIdx.y;
  const int ib = max(c0, seg * kSeg);
  const int ie = min((seg + 1) * kSeg, T);
  if (ib >= ie) return;  // whole block
  const int o = c0 + (int)threadIdx.x;  // column k (kind 0) or diagonal d (kind 1)
  const float fl = A.floor;
  const float* base = A.ahat + (int64_t)h * A.head_stride;
  const float* inv_s = A.inv_s + (int64_t)h * T;
  float acc = 0.f;
  // every thread walks the same rows (row i's reads are one contiguous run);
  // a column or diagonal o reaches row i only for i >= o
#pragma unroll 8
  for (int i = ib; i < ie; ++i) {
    const float inv = inv_s[i];
    if (i >= o) {
      const int col = kind == 0 ? o : i - o;
      acc = fmaf(fmaxf(base[(int64_t)i * A.row_stride + col], fl), inv, acc);
    }
  }
  if (o < T) A.part[(((int64_t)h * 2 + kind) * A.nseg + seg) * T + o] = acc;
}

__global__ __launch_bounds__(kTChunk) void fit_tred_kernel(FitTargetArgs A) {
  const int T = A.T;
  const int h = blockIdx.y;
  const int c0 = blockIdx.x * kTChunk;
  const int o = c0 + (int)threadIdx.x;
  if (o >= T) return;
  const int s0 = c0 / kSeg;  // first segment holding rows >= c0
#pragma unroll
  for (int kind = 0; kind < 2; ++kind) {
    const float* pp = A.part + ((int64_t)h * 2 + kind) * A.nseg * T + o;
    float acc = 0.f;
    for (int s = s0; s < A.nseg; ++s) acc += pp[(int64_t)s * T];
    (kind == 0 ? A.eta_abs : A.eta_rel)[(int64_t)h * T + o] = acc;
  }
}

// Fixed-order double sum of x[0..n) over one block of 256 threads.
__device__ double block_sum_f64(double v, double* red) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  if (lane_id() == 0) red[wave_id()] = v;
  __syncthreads();
  double s = 0.0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) s += red[w];
  __syncthreads();
  return s;
}

__global__ __launch_bounds__(256) void fit_negent_kernel(FitTargetArgs A) {
  __shared__ double red[4];
  const int h = blockIdx.x;
  const float* e = A.row_ent + (int64_t)h * A.T;
  double acc = 0.0;
  for (int i = threadIdx.x; i < A.T; i += blockDim.x) acc += (double)e[i];
  const double s = block_sum_f64(acc, red);
  if (threadIdx.x == 0) A.negent[h] = (float)s;
}

// ---------------------------------------------------------------------------
// The fit.
// ---------------------------------------------------------------------------

constexpr int kOut = 64;  // parameters per step block (one per lane)
constexpr int kWaves = 4;
constexpr int kNT = kOut * kWaves;
constexpr int kTK = 256;  // summation indices per chunk
constexpr int kBand = kOut + kTK - 1;
constexpr int kBS = band_stride(kBand);
static_assert(kBand + 3 <= 2 * kNT && kBS % 4 == 0 && kBS >= kBand + 3, "band layout");

struct StepSmem {
  float x2[kTK];    // X of the chunk (log2 units)
  float y2[kBand];  // Y of the chunk's band (log2 units)
  __attribute__((aligned(16))) float xe[kTK];  // exp2(X - mx)
  // exp2(Y - my) in four copies: copy c holds band entry y + c at y (0 past
  // the end), so four consecutive entries starting anywhere are one aligned
  // 16-byte read
  __attribute__((aligned(16))) float ye[4 * kBS];
  float red[8];
  float cm[kWaves][kOut];
  float cs[kWaves][kOut];
};

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

// One block: parameters o0 .. o0+63 of kind KIND for head h.
//   KIND 0 (a): output k = o0 + lane; chunk rows i = c0 + x;
//               X[x] = -z2[i], band y = x - lane + (kOut - 1) at offset
//               i - k = c0 - o0 - (kOut - 1) + y, Y[y] = r2[offset].
//   KIND 1 (r): output d = o0 + lane; chunk keys k = c0 + x;
//               X[x] = a2[k], band y = x + lane at row i = c0 + o0 + y,
//               Y[y] = -z2[i].
// Entries outside [0, T) are -inf (their exponentials 0).
template <int KIND>
__device__ void fit_step_block(const FitStepArgs& A, StepSmem& sm) {
  const int T = A.T;
  const int h = blockIdx.z;
  const int o0 = blockIdx.x * kOut;
  const int lane = lane_id(), w = wave_id();
  const float* ah = A.a_cur + (int64_t)h * T;
  const float* rh = A.r_cur + (int64_t)h * T;
  const float* zh = A.logz + (int64_t)h * T;
  const int o = o0 + lane;
  const int sgn = KIND == 0 ? -1 : 1;
  const int yoff = KIND == 0 ? kOut - 1 : 0;
  // summation range: kind 0 rows [o0, T); kind 1 keys [0, T - o0)
  const int cbeg = KIND == 0 ? o0 : 0;
  const int cend = KIND == 0 ? T : T - o0;
  float M = kNegInf, S = 0.f;
  for (int c0 = cbeg; c0 < cend; c0 += kTK) {
    float lmx = kNegInf, lmy = kNegInf;
    for (int x = threadIdx.x; x < kTK; x += kNT) {
      const int n = c0 + x;
      float v = kNegInf;
      if (n < T) v = KIND == 0 ? -zh[n] * kLog2e : ah[n] * kLog2e;
      sm.x2[x] = v;
      lmx = fmaxf(lmx, v);
    }
    for (int y = threadIdx.x; y < kBand; y += kNT) {
      float v = kNegInf;
      if (KIND == 0) {
        const int d = c0 - o0 - (kOut - 1) + y;
        if (d >= 0 && d < T) v = rh[d] * kLog2e;
      } else {
        const int i = c0 + o0 + y;
        if (i < T) v = -zh[i] * kLog2e;
      }
      sm.y2[y] = v;
      lmy = fmaxf(lmy, v);
    }
    float mx = lmx, my = lmy;
    block_max2(mx, my, sm.red);
    if (mx == kNegInf) mx = 0.f;
    if (my == kNegInf) my = 0.f;
    for (int x = threadIdx.x; x < kTK; x += kNT) sm.xe[x] = fast_exp2(sm.x2[x] - mx);
    for (int y = threadIdx.x; y < kBand + 3; y += kNT) {
      const float e = y < kBand ? fast_exp2(sm.y2[y] - my) : 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int yy = y - c;
        if (yy >= 0 && yy < kBS) sm.ye[c * kBS + yy] = e;
      }
    }
    __syncthreads();

    // wave w takes the groups of four x = 4 (w + 4u); x past the summation
    // range has a zero factor on one side, so all lanes run the same loop
    const int xlast = min(kTK, cend - c0) - 1;
    const int xq = 4 * __builtin_amdgcn_readfirstlane(w);
    if (xq <= xlast && o < T) {
      const int yb = sgn * lane + yoff;  // band index of x = 0
      const int cpy = yb & 3;            // x is a multiple of 4
      const lds_f32* yc = (const lds_f32*)sm.ye + cpy * kBS - cpy;
      const lds_f32* xe = (const lds_f32*)sm.xe;
      float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll 4
      for (int x = xq; x <= xlast; x += 4 * kWaves) {
        const f32x4 e4 = lds_read_f4(xe + x);
        const f32x4 y4 = lds_read_f4(yc + (x + yb));
        s0 = fmaf(e4[0], y4[0], s0);
        s1 = fmaf(e4[1], y4[1], s1);
        s2 = fmaf(e4[2], y4[2], s2);
        s3 = fmaf(e4[3], y4[3], s3);
      }
      const float s = (s0 + s1) + (s2 + s3);
      if (s >= 0x1p-20f) {
        lse_merge(M, S, mx + my, s);
      } else {
        // exact max-shifted sum of this lane's terms in this wave's groups
        float cm = kNegInf;
        for (int g = xq; g <= xlast; g += 4 * kWaves)
          for (int x = g; x < g + 4 && x <= xlast; ++x) cm = fmaxf(cm, sm.x2[x] + sm.y2[x + yb]);
        float cs = 0.f;
        if (cm != kNegInf)
          for (int g = xq; g <= xlast; g += 4 * kWaves)
            for (int x = g; x < g + 4 && x <= xlast; ++x) cs += fast_exp2(sm.x2[x] + sm.y2[x + yb] - cm);
        lse_merge(M, S, cm, cs);
      }
    }
    __syncthreads();  // the chunk buffers are restaged next
  }
  sm.cm[w][lane] = M;
  sm.cs[w][lane] = S;
  __syncthreads();
  if (w != 0 || o >= T) return;
  float Mt = kNegInf, St = 0.f;
  for (int x = 0; x < kWaves; ++x) lse_merge(Mt, St, sm.cm[x][lane], sm.cs[x][lane]);
  const float theta = KIND == 0 ? ah[o] : rh[o];
  const float mu = St > 0.f ? St * fast_exp2(theta * kLog2e + Mt) : 0.f;
  const float eta = (KIND == 0 ? A.eta_abs : A.eta_rel)[(int64_t)h * T + o];
  const float g = (mu - eta) / (float)T;  // Equation 20
  const int64_t idx = (int64_t)h * T + o;
  float* mom1 = KIND == 0 ? A.m_a : A.m_r;
  float* mom2 = KIND == 0 ? A.v_a : A.v_r;
  const float m = A.beta1 * mom1[idx] + (1.f - A.beta1) * g;
  const float v = A.beta2 * mom2[idx] + (1.f - A.beta2) * g * g;
  mom1[idx] = m;
  mom2[idx] = v;
  // theta - lr m_hat / (sqrt(v_hat) + eps) with the bias corrections of step t
  const float denom = sqrtf(v) * A.inv_sqrt_bc2 + A.eps;
  (KIND == 0 ? A.a_next : A.r_next)[idx] = theta - A.lr_bc1 * m / denom;
}

__global__ __launch_bounds__(kNT) void fit_step_kernel(FitStepArgs A) {
  __shared__ StepSmem sm;
  if (blockIdx.y == 0)
    fit_step_block<0>(A, sm);
  else
    fit_step_block<1>(A, sm);
}

// a = 0, r(d) = log max(eta_rel(d) / (T - d), floor), zero Adam moments.
__global__ __launch_bounds__(256) void fit_init_kernel(FitStepArgs A) {
  const int h = blockIdx.y;
  const int d = blockIdx.x * blockDim.x + threadIdx.x;
  const int T = A.T;
  if (d >= T) return;
  const int64_t idx = (int64_t)h * T + d;
  A.a_next[idx] = 0.f;
  A.r_next[idx] = logf(fmaxf(A.eta_rel[idx] / (float)(T - d), kFitInitFloor));
  A.m_a[idx] = 0.f;
  A.v_a[idx] = 0.f;
  A.m_r[idx] = 0.f;
  A.v_r[idx] = 0.f;
}

// Equation 4 at the final parameters, and kappa = negent / T + loss.
__global__ __launch_bounds__(256) void fit_loss_kernel(FitStepArgs A, const float* negent, float* loss,
                                                       float* kappa) {
  __shared__ double red[4];
  const int h = blockIdx.x;
  const int T = A.T;
  const int64_t base = (int64_t)h * T;
  double acc = 0.0;
  for (int i = threadIdx.x; i < T; i += blockDim.x)
    acc += (double)A.logz[base + i] - (double)A.eta_abs[base + i] * (double)A.a_cur[base + i] -
           (double)A.eta_rel[base + i] * (double)A.r_cur[base + i];
  const double L = block_sum_f64(acc, red) / (double)T;
  if (threadIdx.x == 0) {
    if (loss) loss[h] = (float)L;
    if (kappa) kappa[h] = (float)((double)negent[h] / (double)T + L);
  }
}

}  // namespace

hipError_t launch_fit_targets(const FitTargetArgs& args, hipStream_t stream) {
  if (args.n_heads <= 0 || args.T <= 0) return hipSuccess;
  const int T = args.T;
  const int npairs = (T + 1) / 2;
  hipLaunchKernelGGL(fit_rows_kernel, dim3((npairs + kRowWaves - 1) / kRowWaves, args.n_heads),
                     dim3(64 * kRowWaves), 0, stream, args);
  const int nchunk = (T + kTChunk - 1) / kTChunk;
  hipLaunchKernelGGL(fit_tmarg_kernel, dim3(nchunk, args.nseg, 2 * args.n_heads), dim3(kTChunk), 0,
                     stream, args);
  hipLaunchKernelGGL(fit_tred_kernel, dim3(nchunk, args.n_heads), dim3(kTChunk), 0, stream, args);
  hipLaunchKernelGGL(fit_negent_kernel, dim3(args.n_heads), dim3(256), 0, stream, args);
  return hipGetLastError();
}

hipError_t launch_fit_init(const FitStepArgs& args, hipStream_t stream) {
  hipLaunchKernelGGL(fit_init_kernel, dim3((args.T + 255) / 256, args.n_heads), dim3(256), 0, stream,
                     args);
  return hipGetLastError();
}

hipError_t launch_fit_step(const FitStepArgs& args, hipStream_t stream) {
  hipLaunchKernelGGL(fit_step_kernel, dim3((args.T + kOut - 1) / kOut, 2, args.n_heads), dim3(kNT), 0,
                     stream, args);
  return hipGetLastError();
}

hipError_t launch_fit_loss(const FitStepArgs& args, const float* negent, float* loss, float* kappa,
                           hipStream_t stream) {
  hipLaunchKernelGGL(fit_loss_kernel, dim3(args.n_heads), dim3(256), 0, stream, args, negent, loss, kappa);
  return hipGetLastError();
}

}  // namespace saf
