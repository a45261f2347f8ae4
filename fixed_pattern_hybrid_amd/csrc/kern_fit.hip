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
//   fit_cmarg4_kernel / fit_dmarg4_kernel  (rows 16-byte aligned) column
//                     and diagonal sums with 16-byte reads over segments of
//                     kSeg rows: a thread owns four columns, or reads the
//                     aligned run (i, 4(m - k) .. +3) of rows i = 4m + u,
//                     whose entries lie on four fixed diagonals.
//   fit_tmarg_kernel  (other layouts) one thread per column (kind 0) or per
//                     diagonal (kind 1), reading 4 bytes per row.
//   Per-segment partial sums go to the workspace, [h][seg][5][T]: slot 0
//   the column sums, slots 1..4 the diagonal sums (one slot per run
//   position e in the aligned kernel, slot 1 alone otherwise).
//   fit_tred_kernel   fixed-order sums of the segment partials (eta_abs,
//                     eta_rel); fit_negent_kernel sums the row entropies.
//
// The fit (four launches per Adam step).  Two run one band-sum program with
// 256 outputs per block (four per lane), over groups of at most
// kFitGroupChunks chunks, writing (max, sum) partials; two merge them:
//   fit_norm_part_kernel + fit_norm_merge_kernel  log N(i) of the current
//     (a, r) (Equation 3) and the segment maxima of -log N;
//   fit_marg_part_kernel + fit_update_kernel  the fitted marginals
//     mu_abs(k) = exp(a_k) * sum_{i >= k} exp(r_{i-k} - z_i)
//     mu_rel(d) = exp(r_d) * sum_{k < T-d} exp(a_k - z_{k+d})
//   (kind 0 = a, kind 1 = r), the gradient (mu - eta) / T (Equation 20) and
//   the Adam update, written to the other of two parameter buffers so that
//   every block of a step reads the same point.
// The forward's normaliser of frozen heads (norm_segmax_kernel, then the
// same fit_norm_part_kernel) reuses the normaliser kind.
//
// The sums factor like the forward's normaliser: over a chunk of kTK
// summation indices, exp2(X[x] + Y[y]) = 2^(mx + my) exp2(X[x] - mx)
// exp2(Y[y] - my), where X is indexed by the summation index and Y by a band
// index that moves with both the summation index and the output.  Each term
// is one FMA on two staged exponentials (both <= 1); an output whose chunk
// sum falls below 2^-96 (where underflowed terms could matter) is recomputed
// exactly with a max-shifted sum.  The
// next chunk's staging values are loaded while the current chunk is summed.
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
constexpr int kPartSlots = 5;  // partial-sum slots per segment: columns, four diagonal slots

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
  if (o < T) A.part[(((int64_t)h * A.nseg + seg) * kPartSlots + kind) * T + o] = acc;
}

// Column sums with 16-byte reads: thread t owns columns o .. o+3, o = 1024
// blockIdx.x + 4t, and sums rows [max(seg start, o), seg end).  Every
// thread writes its slot-0 partials, zero where it has no rows.
__global__ __launch_bounds__(kTChunk) void fit_cmarg4_kernel(FitTargetArgs A) {
  const int T = A.T;
  const int h = blockIdx.z, seg = blockIdx.y;
  const int c0 = blockIdx.x * 4 * kTChunk;
  const int o = c0 + 4 * (int)threadIdx.x;
  const int rb = max(c0, seg * kSeg), re = min((seg + 1) * kSeg, T);
  const float fl = A.floor;
  const float* base = A.ahat + (int64_t)h * A.head_stride;
  const float* inv_s = A.inv_s + (int64_t)h * T;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  // rows i >= o + 3, where the whole run is causal and inside [0, T): every
  // lane runs the same loop, lanes without such a row reading column 0
  // (a valid address) and discarding it
#pragma unroll 4
  for (int i = rb; i < re; ++i) {
    const bool ok = i >= o + 3;
    const float inv = inv_s[i];
    const f32x4 x = *reinterpret_cast<const f32x4*>(base + (int64_t)i * A.row_stride + (ok ? o : 0));
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = ok ? fmaf(fmaxf(x[e], fl), inv, acc[e]) : acc[e];
  }
  // rows o .. o+2 cross the diagonal
  for (int i = max(o, rb); i < min(o + 3, re); ++i) {
    const float inv = inv_s[i];
    const float* row = base + (int64_t)i * A.row_stride;
    for (int e = 0; e <= i - o; ++e) acc[e] = fmaf(fmaxf(row[o + e], fl), inv, acc[e]);
  }
  float* out = A.part + ((int64_t)h * A.nseg + seg) * kPartSlots * T;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (o + e < T) out[o + e] = acc[e];
}

// Diagonal sums with 16-byte reads.  Wave u reads rows i = 4m + u; lane L
// owns k = 64 blockIdx.x + L and reads the aligned run (i, 4(m-k) .. +3)
// for m >= k.  Entry e of the run lies on diagonal d = 4k + u - e, and its
// sum over the segment goes to slot 1 + e of d.  A (slot, diagonal) pair
// has one owner, k = floor((d + e) / 4), u = (d + e) mod 4, whose rows are
// all >= d.  Every owner writes its partials, zero where it has no rows.
__global__ __launch_bounds__(kTChunk) void fit_dmarg4_kernel(FitTargetArgs A) {
  const int T = A.T;
  const int h = blockIdx.z, seg = blockIdx.y;
  const int u = __builtin_amdgcn_readfirstlane(wave_id());
  const int k = 64 * blockIdx.x + lane_id();
  const int ilo = seg * kSeg, ihi = min((seg + 1) * kSeg, T);
  // m with ilo <= 4m + u < ihi
  const int mb = ilo - u <= 0 ? 0 : (ilo - u + 3) / 4;
  const int me = ihi - u <= 0 ? 0 : (ihi - u + 3) / 4;
  const float fl = A.floor;
  const float* base = A.ahat + (int64_t)h * A.head_stride;
  const float* inv_s = A.inv_s + (int64_t)h * T;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const int m0 = max(mb, 64 * (int)blockIdx.x);  // no lane has rows before this
  // k >= 1: columns 4(m-k) .. 4(m-k)+3 < 4m <= i are causal and inside the
  // row.  Every lane runs the same loop; a lane with m < k (or k = 0) reads
  // column 0 (a valid address) and discards it.
#pragma unroll 4
  for (int m = m0; m < me; ++m) {
    const bool ok = m >= k && k > 0;
    const int i = 4 * m + u;
    const float inv = inv_s[i];
    const f32x4 x =
        *reinterpret_cast<const f32x4*>(base + (int64_t)i * A.row_stride + (ok ? 4 * (m - k) : 0));
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = ok ? fmaf(fmaxf(x[e], fl), inv, acc[e]) : acc[e];
  }
  // k = 0: the run (i, 4m .. 4m+3) crosses the diagonal; entries e <= u
  if (k == 0) {
    for (int m = mb; m < me; ++m) {
      const int i = 4 * m + u;
      const float inv = inv_s[i];
      const float* run = base + (int64_t)i * A.row_stride + 4 * m;
      for (int e = 0; e <= u; ++e) acc[e] = fmaf(fmaxf(run[e], fl), inv, acc[e]);
    }
  }
  float* out = A.part + ((int64_t)h * A.nseg + seg) * kPartSlots * T;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int d = 4 * k + u - e;
    if (d >= 0 && d < T) out[(int64_t)(1 + e) * T + d] = acc[e];
  }
}

// rel_slots: diagonal slots the marginal kernels wrote (4 aligned, else 1).
__global__ __launch_bounds__(kTChunk) void fit_tred_kernel(FitTargetArgs A, int rel_slots) {
  const int T = A.T;
  const int h = blockIdx.y;
  const int c0 = blockIdx.x * kTChunk;
  const int o = c0 + (int)threadIdx.x;
  if (o >= T) return;
  const int s0 = c0 / kSeg;  // first segment holding rows >= c0
  const float* pp = A.part + (int64_t)h * A.nseg * kPartSlots * T + o;
  float ca = 0.f, cr = 0.f;
  for (int s = s0; s < A.nseg; ++s) {
    const float* ps = pp + (int64_t)s * kPartSlots * T;
    ca += ps[0];
    for (int e = 0; e < rel_slots; ++e) cr += ps[(int64_t)(1 + e) * T];
  }
  A.eta_abs[(int64_t)h * T + o] = ca;
  A.eta_rel[(int64_t)h * T + o] = cr;
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

constexpr int kQ = 4;                 // parameters per lane
#ifndef SAF_FIT_WAVES
#define SAF_FIT_WAVES 4
#endif
constexpr int kWaves = SAF_FIT_WAVES;  // waves per block, splitting each chunk
constexpr int kNT = 64 * kWaves;
constexpr int kOut = 64 * kQ;         // parameters per step block
constexpr int kTK = 256;              // summation indices per chunk
constexpr int kWaveSpan = kTK / kWaves;  // summation indices per wave and chunk
static_assert(kWaveSpan % 4 == 0, "waves sum whole groups of four");
constexpr int kBand = kOut + kTK - 1; // band entries a chunk touches
constexpr int kBandPad = kBand + 1;   // one zero entry past the end
static_assert(kBandPad % 4 == 0, "band rows are read 16 bytes at a time");

struct StageBuf {
  float x2[kTK];        // X of the chunk (log2 units)
  float y2[kBandPad];   // Y of the chunk's band (log2 units)
  __attribute__((aligned(16))) float xe[kTK];      // exp2(X - mx)
  __attribute__((aligned(16))) float ye[kBandPad]; // exp2(Y - my), 0 past the band
};

struct StepSmem {
  StageBuf buf[2];  // chunk c uses buf[c & 1]
  float red[kWaves];
  float cm[kWaves][kOut];
  float cs[kWaves][kOut];
};

static_assert(kSegMax == kOut && kSegMax == kTK, "segment maxima cover one block's outputs / one chunk");

// Maximum over the block of v; every thread gets it.
__device__ __forceinline__ float block_max1(float v, float* red) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  __syncthreads();
  if (lane_id() == 0) red[wave_id()] = v;
  __syncthreads();
  float m = red[0];
  for (int x = 1; x < (int)(blockDim.x >> 6); ++x) m = fmaxf(m, red[x]);
  return m;
}

__device__ __forceinline__ void lse_merge(float& M, float& S, float cm, float cs) {
  if (cs > 0.f) {
    const float Mn = fmaxf(M, cm);
    S = S * fast_exp2(M - Mn) + cs * fast_exp2(cm - Mn);
    M = Mn;
  }
}

// Band-sum programs.  A block owns 256 outputs o0 .. o0+255 of head h; lane
// L of every wave owns o0 + 4L + q (q = 0..3), and the four waves split
// each chunk's summation indices in groups of four (x = 4 (w + 4u)).  Per
// kind, with chunk index n = c0 + x:
//   KIND 0 (gradient of a, output k): rows i = n, X[x] = -z2[i]; the band
//     entry of (x, k) is y = x - (k - o0) + (kOut - 1), at offset
//     i - k = c0 - o0 - (kOut - 1) + y, Y[y] = r2[offset].
//   KIND 1 (gradient of r, output d): keys k = n, X[x] = a2[k]; band
//     y = x + (d - o0) at row i = c0 + o0 + y, Y[y] = -z2[i].
//   KIND 2 (normaliser, output row i): keys k = n, X[x] = a2[k]; band
//     y = (i - o0) - x + (kTK - 1) at offset i - k = o0 - c0 - (kTK - 1) + y,
//     Y[y] = r2[offset].
// So y = SX x + SO (4L + q) + OFF, and the seven entries a lane needs for a
// group x..x+3 start at yb = SX x + SO 4L + OFFB, a multiple of four: two
// aligned 16-byte reads.  A wave sums a contiguous range of a chunk, so the
// next group's window shares one of those reads: one new 16-byte read per
// sixteen products.  Entries outside [0, T) are -inf (their exponentials 0).
template <int KIND>
struct BandKind {
  static constexpr int SX = KIND == 2 ? -1 : 1;
  static constexpr int SO = KIND == 0 ? -1 : 1;
  static constexpr int OFF = KIND == 0 ? kOut - 1 : (KIND == 1 ? 0 : kTK - 1);
  static constexpr int OFFB = KIND == 0 ? kOut - 4 : (KIND == 1 ? 0 : kTK - 4);
  // position of entry (q, e) among the seven starting at yb
  __device__ static constexpr int idx(int q, int e) {
    return KIND == 0 ? 3 + e - q : (KIND == 1 ? q + e : 3 + q - e);
  }
};

// Staging values are loaded raw from a clamped (always valid) index, one
// chunk ahead and without branches, so the loads stay in flight while the
// current chunk is summed; band_val turns a raw value into log2 units (-inf
// where the index falls outside the band or [0, T)).
template <int KIND>
__device__ __forceinline__ int band_x_idx(int n, int T, bool& ok) {
  ok = n < T;
  return min(n, T - 1);
}

template <int KIND>
__device__ __forceinline__ int band_y_idx(int c0, int o0, int y, int T, bool& ok) {
  const int n = KIND == 1 ? c0 + o0 + y : (KIND == 0 ? c0 - o0 - (kOut - 1) + y : o0 - c0 - (kTK - 1) + y);
  ok = y < kBand && n >= 0 && n < T;
  return min(max(n, 0), T - 1);
}

__device__ __forceinline__ float band_val(float raw, bool ok, bool negate) {
  return ok ? (negate ? -raw : raw) * kLog2e : kNegInf;
}

// Exact max-shifted sum of one output's terms over a wave's range of a
// chunk (x = xq .. xend; band index SX x + yq), as a (max, sum) pair in log2
// units.  Rarely taken, so kept out of line: the summing loop keeps its
// registers.
__device__ __attribute__((noinline)) float2 exact_chunk_sum(const float* x2, const float* y2, int sx, int yq,
                                                            int xq, int xend) {
  float cm = kNegInf;
  for (int x = xq; x <= xend; ++x) cm = fmaxf(cm, x2[x] + y2[sx * x + yq]);
  float cs = 0.f;
  if (cm != kNegInf)
    for (int x = xq; x <= xend; ++x) cs += fast_exp2(x2[x] + y2[sx * x + yq] - cm);
  return make_float2(cm, cs);
}

// Whether any of a wave's summation indices (xq <= x <= xend) falls in
// output o's causal range for the chunk at c0:
//   kind 0 (output k): rows i = c0 + x with k <= i < T;
//   kind 1 (output d): keys k = c0 + x with 0 <= k < T - d;
//   kind 2 (output i): keys k = c0 + x with 0 <= k <= i.
// Terms in that range are finite (a, r and log N are), so a zero sum with
// no such index is exact and needs no recomputation.
template <int KIND>
__device__ __forceinline__ bool wave_has_terms(int o, int c0, int xq, int xend, int T) {
  const int lo = KIND == 0 ? o - c0 : -c0;
  const int hi = KIND == 0 ? T - 1 - c0 : (KIND == 1 ? T - 1 - o - c0 : o - c0);
  return max(lo, xq) <= min(hi, xend);
}

// Sixteen products of one group of four summation indices; ya and yc hold
// band entries yb..yb+3 and yb+4..yb+7.
template <int KIND>
__device__ __forceinline__ void group_fma(const f32x4& e4, const f32x4& ya, const f32x4& yc, float* s) {
  using K = BandKind<KIND>;
  const float yv[8] = {ya[0], ya[1], ya[2], ya[3], yc[0], yc[1], yc[2], yc[3]};
#pragma unroll
  for (int q = 0; q < kQ; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e) s[q] = fmaf(e4[e], yv[K::idx(q, e)], s[q]);
}

// Products of the groups starting at x, x + 4, ... (ng of them): each step
// moves the band window by SX * 4 entries, so one half of it is carried
// over and the other read.
template <int KIND, bool UNROLL>
__device__ __forceinline__ void range_fma(const lds_f32* xe, const lds_f32* ye, int x, int ng, int yb, float* s) {
  using K = BandKind<KIND>;
  f32x4 ya = lds_read_f4(ye + yb);
  f32x4 yc = lds_read_f4(ye + (yb + 4));
  auto step = [&](int u) {
    if (u > 0) {
      if (K::SX > 0) {
        ya = yc;
        yc = lds_read_f4(ye + (yb + 4 * u + 4));
      } else {
        yc = ya;
        ya = lds_read_f4(ye + (yb - 4 * u));
      }
    }
    group_fma<KIND>(lds_read_f4(xe + (x + 4 * u)), ya, yc, s);
  };
  if constexpr (UNROLL) {
#pragma unroll
    for (int u = 0; u < kWaveSpan / 4; ++u) step(u);
  } else {
#pragma unroll 2
    for (int u = 0; u < ng; ++u) step(u);
  }
}

// Summation range of an output block (chunks of kTK from cbeg to cend):
// kind 0 rows [o0, T); kind 1 keys [0, T - o0); kind 2 keys [0, min(o0 +
// kOut, T)).  A block sums one group of at most A.grp_chunks chunks.
template <int KIND>
__device__ __forceinline__ void sum_range(int o0, int T, int& cbeg, int& cend) {
  cbeg = KIND == 0 ? o0 : 0;
  cend = KIND == 0 ? T : (KIND == 1 ? T - o0 : min(o0 + kOut, T));
}

template <int KIND>
__device__ __forceinline__ int n_groups(int o0, int T, int gchunks) {
  int cbeg, cend;
  sum_range<KIND>(o0, T, cbeg, cend);
  const int chunks = (cend - cbeg + kTK - 1) / kTK;
  return (chunks + gchunks - 1) / gchunks;
}

// Sums of the block's outputs over chunk group grp, as (max, sum) pairs in
// log2 units, merged over the waves into sm.cm[0][t], sm.cs[0][t] for output
// o0 + t.
template <int KIND>
__device__ void band_sums(const FitStepArgs& A, StepSmem& sm, int h, int o0, int grp) {
  using K = BandKind<KIND>;
  const int T = A.T;
  const int lane = lane_id(), w = wave_id();
  const int tid = threadIdx.x;
  const int hp = A.use_heads ? (int)A.heads[h] : h;  // row of a and r
  const float* ah = A.a_cur + (int64_t)hp * A.prm_stride;
  const float* rh = A.r_cur + (int64_t)hp * A.prm_stride;
  const float* zh = A.logz + (int64_t)h * T;
  const int ol = o0 + kQ * lane;  // this lane's first output
  int cbeg, cend;
  sum_range<KIND>(o0, T, cbeg, cend);
  cbeg += grp * A.grp_chunks * kTK;
  cend = min(cend, cbeg + A.grp_chunks * kTK);
  float M[kQ], S[kQ];
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    M[q] = kNegInf;
    S[q] = 0.f;
  }
  // thread tid stages X entry tid (tid < kTK) and Y entries tid + j kNT
  constexpr int kYPer = (kBandPad + kNT - 1) / kNT;
  static_assert(kTK <= kNT, "one X entry per thread at most");
  // X reads z (kind 0) or a; Y reads z (kind 1) or r.  Their shifts are
  // upper bounds from the maxima of 256-entry segments (of a, r and -z):
  // a chunk's X is one segment, its band of kBand entries two.
  const float* xsrc = KIND == 0 ? zh : ah;
  const float* ysrc = KIND == 1 ? zh : rh;
  const int nseg = A.nseg;
  const float* xmax = (KIND == 0 ? A.smax_z : A.smax_a_cur) + (int64_t)h * nseg;
  const float* ymax = (KIND == 1 ? A.smax_z : A.smax_r_cur) + (int64_t)h * nseg;
  constexpr bool XNEG = KIND == 0, YNEG = KIND == 1;
  // band start (source index of y = 0) of the chunk at c0
  auto band_lo = [&](int c0) {
    return KIND == 1 ? c0 + o0 : (KIND == 0 ? c0 - o0 - (kOut - 1) : o0 - c0 - (kTK - 1));
  };
  // raw staging values and segment maxima for the chunk at c, loaded a chunk
  // ahead from clamped (always valid) indices
  bool okx, oky[kYPer], okm0, okm1;
  float px, py[kYPer], pmx, pmy0, pmy1;
  auto prefetch = [&](int c) {
    px = xsrc[band_x_idx<KIND>(c + tid, T, okx)];
#pragma unroll
    for (int j = 0; j < kYPer; ++j) py[j] = ysrc[band_y_idx<KIND>(c, o0, tid + j * kNT, T, oky[j])];
    // the maxima are the same for every thread; their indices are moved to
    // vector registers so that the loads are vector loads, which the chunk's
    // barrier does not wait for (it waits for scalar loads)
    int ix = min(c / kSegMax, nseg - 1);
    const int lo = band_lo(c);
    const int s0 = (lo < 0 ? lo - (kSegMax - 1) : lo) / kSegMax;  // floor
    okm0 = s0 >= 0 && s0 < nseg;
    okm1 = s0 + 1 >= 0 && s0 + 1 < nseg;
    int iy0 = min(max(s0, 0), nseg - 1), iy1 = min(max(s0 + 1, 0), nseg - 1);
    asm volatile("" : "+v"(ix), "+v"(iy0), "+v"(iy1));
    pmx = xmax[ix];
    pmy0 = ymax[iy0];
    pmy1 = ymax[iy1];
  };
  prefetch(cbeg);
  int par = 0;
  for (int c0 = cbeg; c0 < cend; c0 += kTK, par ^= 1) {
    StageBuf& sb = sm.buf[par];
    const float vx = band_val(px, okx, XNEG);
    float vy[kYPer];
#pragma unroll
    for (int j = 0; j < kYPer; ++j) vy[j] = band_val(py[j], oky[j], YNEG);
    float mx = pmx * kLog2e;
    float my = fmaxf(okm0 ? pmy0 * kLog2e : kNegInf, okm1 ? pmy1 * kLog2e : kNegInf);
    if (!(mx > kNegInf)) mx = 0.f;
    if (!(my > kNegInf)) my = 0.f;
    prefetch(c0 + kTK);  // past the range on the last chunk: clamped, unused
    if (tid < kTK) {
      sb.x2[tid] = vx;
      sb.xe[tid] = fast_exp2(vx - mx);
    }
#pragma unroll
    for (int j = 0; j < kYPer; ++j) {
      const int y = tid + j * kNT;
      if (y < kBandPad) {
        sb.y2[y] = vy[j];
        sb.ye[y] = fast_exp2(vy[j] - my);
      }
    }
    // one barrier per chunk: it publishes this buffer, and every wave has
    // finished the chunk before the last, which used the other buffer
    __syncthreads();

    // wave w sums x in [xq, xend], a contiguous quarter of the chunk; x past
    // the summation range has a zero factor on one side, so every lane runs
    // the same loop
    const int xlast = min(kTK, cend - c0) - 1;
    const int xq = kWaveSpan * __builtin_amdgcn_readfirstlane(w);
    const int xend = min(xq + kWaveSpan - 1, xlast);
    const int ybl = K::SO * kQ * lane + K::OFFB;  // yb - SX x
    if (xq <= xlast && ol < T) {
      const lds_f32* xe = (const lds_f32*)sb.xe;
      const lds_f32* ye = (const lds_f32*)sb.ye;
      float s[kQ] = {0.f, 0.f, 0.f, 0.f};
      if (xend == xq + kWaveSpan - 1) {
        // the whole range: straight-line code, so reads can be issued ahead
        range_fma<KIND, true>(xe, ye, xq, kWaveSpan / 4, K::SX * xq + ybl, s);
      } else {
        range_fma<KIND, false>(xe, ye, xq, (xend - xq) / 4 + 1, K::SX * xq + ybl, s);
      }
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        if (ol + q >= T) continue;
        // a lane sums at most 64 terms of a chunk, each factor <= 1; a term
        // lost to underflow is below 2^-126 (of 2^(mx + my)), so all lost
        // terms stay below 2^-120, which is 2^-24 of any sum >= 2^-96
        if (s[q] >= 0x1p-96f) {
          lse_merge(M[q], S[q], mx + my, s[q]);
        } else if (wave_has_terms<KIND>(ol + q, c0, xq, xend, T)) {
          const float2 ex = exact_chunk_sum(sb.x2, sb.y2, K::SX, K::SO * (kQ * lane + q) + K::OFF, xq, xend);
          lse_merge(M[q], S[q], ex.x, ex.y);
        }
      }
    }
  }
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    sm.cm[w][kQ * lane + q] = M[q];
    sm.cs[w][kQ * lane + q] = S[q];
  }
  __syncthreads();
  float Mt = kNegInf, St = 0.f;
  if (tid < kOut)
    for (int x = 0; x < kWaves; ++x) lse_merge(Mt, St, sm.cm[x][tid], sm.cs[x][tid]);
  __syncthreads();
  if (tid < kOut) {
    sm.cm[0][tid] = Mt;
    sm.cs[0][tid] = St;
  }
}

// Partial sums of one chunk group of an output block: (max, sum) per output
// into part[(slot * maxg + grp) * T + o].
template <int KIND>
__device__ void band_part(const FitStepArgs& A, StepSmem& sm, int h, int o0, int grp, float2* part,
                          int64_t slot) {
  if (grp >= n_groups<KIND>(o0, A.T, A.grp_chunks)) return;  // whole block
  band_sums<KIND>(A, sm, h, o0, grp);
  const int t = threadIdx.x;
  if (t < kOut && o0 + t < A.T)
    part[(slot * A.maxg + grp) * A.T + o0 + t] = make_float2(sm.cm[0][t], sm.cs[0][t]);
}

// (max, sum) of output o over its groups, merged in group order.
__device__ __forceinline__ float2 merge_groups(const float2* part, int64_t slot, int maxg, int T, int o, int ng) {
  float M = kNegInf, S = 0.f;
  for (int g = 0; g < ng; ++g) {
    const float2 p = part[(slot * maxg + g) * T + o];
    lse_merge(M, S, p.x, p.y);
  }
  return make_float2(M, S);
}

// Grid (output blocks, chunk groups, heads): partial normaliser sums.
__global__ __launch_bounds__(kNT) void fit_norm_part_kernel(FitStepArgs A) {
  __shared__ StepSmem sm;
  band_part<2>(A, sm, blockIdx.z, blockIdx.x * kOut, blockIdx.y, A.part_z, blockIdx.z);
}

// Grid (output blocks, chunk groups, 2 x heads): partial marginal sums.
__global__ __launch_bounds__(kNT) void fit_marg_part_kernel(FitStepArgs A) {
  __shared__ StepSmem sm;
  const int h = blockIdx.z >> 1;
  if (blockIdx.z & 1)
    band_part<1>(A, sm, h, blockIdx.x * kOut, blockIdx.y, A.part_m, blockIdx.z);
  else
    band_part<0>(A, sm, h, blockIdx.x * kOut, blockIdx.y, A.part_m, blockIdx.z);
}

// Grid (output blocks, heads): log N(i) (natural log) of the current
// parameters into logz from the groups' partials, and the maximum of -log N
// over each 256-row segment into A.smax_z.
__global__ __launch_bounds__(kSegMax) void fit_norm_merge_kernel(FitStepArgs A, float* logz) {
  __shared__ float red[kSegMax / 64];
  const int h = blockIdx.y, o0 = blockIdx.x * kOut;
  const int o = o0 + (int)threadIdx.x;
  float nz = kNegInf;
  if (o < A.T) {
    const float2 p = merge_groups(A.part_z, h, A.maxg, A.T, o, n_groups<2>(o0, A.T, A.grp_chunks));
    const float z = (p.x + fast_log2(p.y)) * kLn2;
    logz[(int64_t)h * A.T + o] = z;
    nz = -z;
  }
  const float mx = block_max1(nz, red);
  if (threadIdx.x == 0) A.smax_z[(int64_t)h * A.nseg + o0 / kSegMax] = mx;
}

// Gradient and Adam update of parameters o0 .. o0+255 of kind KIND (0: a,
// 1: r) from the groups' marginal partials.
template <int KIND>
__device__ void fit_update(const FitStepArgs& A, float* red, int h, int o0) {
  const int T = A.T;
  const int t = threadIdx.x;
  const int o = o0 + t;
  float next = kNegInf;
  if (o < T) {
    const int64_t idx = (int64_t)h * T + o;
    const float2 p = merge_groups(A.part_m, 2 * h + KIND, A.maxg, T, o, n_groups<KIND>(o0, T, A.grp_chunks));
    const float theta = (KIND == 0 ? A.a_cur : A.r_cur)[idx];
    const float mu = p.y > 0.f ? p.y * fast_exp2(theta * kLog2e + p.x) : 0.f;
    const float eta = (KIND == 0 ? A.eta_abs : A.eta_rel)[idx];
    const float g = (mu - eta) / (float)T;  // Equation 20
    float* mom1 = KIND == 0 ? A.m_a : A.m_r;
    float* mom2 = KIND == 0 ? A.v_a : A.v_r;
    const float m = A.beta1 * mom1[idx] + (1.f - A.beta1) * g;
    const float v = A.beta2 * mom2[idx] + (1.f - A.beta2) * g * g;
    mom1[idx] = m;
    mom2[idx] = v;
    // theta - lr m_hat / (sqrt(v_hat) + eps) with the bias corrections of step t
    const float denom = sqrtf(v) * A.inv_sqrt_bc2 + A.eps;
    next = theta - A.lr_bc1 * m / denom;
    (KIND == 0 ? A.a_next : A.r_next)[idx] = next;
  }
  // the new parameters' maximum over this 256-entry segment
  const float mx = block_max1(next, red);
  if (t == 0) (KIND == 0 ? A.smax_a_next : A.smax_r_next)[(int64_t)h * A.nseg + o0 / kSegMax] = mx;
}

// Grid (output blocks, 2, heads).
__global__ __launch_bounds__(kSegMax) void fit_update_kernel(FitStepArgs A) {
  __shared__ float red[kSegMax / 64];
  const int h = blockIdx.z, o0 = blockIdx.x * kOut;
  if (blockIdx.y == 0)
    fit_update<0>(A, red, h, o0);
  else
    fit_update<1>(A, red, h, o0);
}

// Grid (segments, listed heads): maxima of a and r over each 256-entry
// segment [0, T) of the listed heads' rows.
__global__ __launch_bounds__(kSegMax) void norm_segmax_kernel(FitStepArgs A, float* smax_a, float* smax_r) {
  __shared__ float red[kSegMax / 64];
  const int h = blockIdx.y;
  const int hp = A.use_heads ? (int)A.heads[h] : h;
  const int x = blockIdx.x * kSegMax + threadIdx.x;
  const bool ok = x < A.T;
  const float va = ok ? A.a_cur[(int64_t)hp * A.prm_stride + x] : kNegInf;
  const float vr = ok ? A.r_cur[(int64_t)hp * A.prm_stride + x] : kNegInf;
  const float ma = block_max1(va, red);
  __syncthreads();  // red is reused
  const float mr = block_max1(vr, red);
  if (threadIdx.x == 0) {
    smax_a[(int64_t)h * A.nseg + blockIdx.x] = ma;
    smax_r[(int64_t)h * A.nseg + blockIdx.x] = mr;
  }
}

// a = 0, r(d) = log max(eta_rel(d) / (T - d), floor), zero Adam moments.
__global__ __launch_bounds__(kSegMax) void fit_init_kernel(FitStepArgs A) {
  __shared__ float red[8];
  const int h = blockIdx.y;
  const int d = blockIdx.x * kSegMax + threadIdx.x;
  const int T = A.T;
  float rv = kNegInf;
  if (d < T) {
    const int64_t idx = (int64_t)h * T + d;
    rv = logf(fmaxf(A.eta_rel[idx] / (float)(T - d), kFitInitFloor));
    A.a_next[idx] = 0.f;
    A.r_next[idx] = rv;
    A.m_a[idx] = 0.f;
    A.v_a[idx] = 0.f;
    A.m_r[idx] = 0.f;
    A.v_r[idx] = 0.f;
  }
  const float mx = block_max1(rv, red);
  if (threadIdx.x == 0) {
    A.smax_a_next[(int64_t)h * A.nseg + blockIdx.x] = 0.f;
    A.smax_r_next[(int64_t)h * A.nseg + blockIdx.x] = mx;
  }
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
  // every row starts 16-byte aligned (and has the four columns that lanes
  // without work read): the 16-byte-read kernels
  const bool vec = (reinterpret_cast<uintptr_t>(args.ahat) & 15) == 0 && args.row_stride % 4 == 0 &&
                   args.head_stride % 4 == 0 && T >= 4;
  if (vec) {
    const int nk = (T + 2) / 4 + 1;  // k of every (slot, diagonal) owner
    hipLaunchKernelGGL(fit_cmarg4_kernel, dim3((T + 4 * kTChunk - 1) / (4 * kTChunk), args.nseg, args.n_heads),
                       dim3(kTChunk), 0, stream, args);
    hipLaunchKernelGGL(fit_dmarg4_kernel, dim3((nk + 63) / 64, args.nseg, args.n_heads), dim3(kTChunk), 0,
                       stream, args);
  } else {
    hipLaunchKernelGGL(fit_tmarg_kernel, dim3(nchunk, args.nseg, 2 * args.n_heads), dim3(kTChunk), 0,
                       stream, args);
  }
  hipLaunchKernelGGL(fit_tred_kernel, dim3(nchunk, args.n_heads), dim3(kTChunk), 0, stream, args, vec ? 4 : 1);
  hipLaunchKernelGGL(fit_negent_kernel, dim3(args.n_heads), dim3(256), 0, stream, args);
  return hipGetLastError();
}

hipError_t launch_fit_init(const FitStepArgs& args, hipStream_t stream) {
  hipLaunchKernelGGL(fit_init_kernel, dim3(args.nseg, args.n_heads), dim3(kSegMax), 0, stream,
                     args);
  return hipGetLastError();
}

hipError_t launch_fit_step(const FitStepArgs& args, hipStream_t stream) {
  const int nb = (args.T + kOut - 1) / kOut;
  hipLaunchKernelGGL(fit_marg_part_kernel, dim3(nb, args.maxg, 2 * args.n_heads), dim3(kNT), 0, stream, args);
  hipLaunchKernelGGL(fit_update_kernel, dim3(nb, 2, args.n_heads), dim3(kSegMax), 0, stream, args);
  return hipGetLastError();
}

hipError_t launch_fit_norm(const FitStepArgs& args, float* logz, hipStream_t stream) {
  const int nb = (args.T + kOut - 1) / kOut;
  hipLaunchKernelGGL(fit_norm_part_kernel, dim3(nb, args.maxg, args.n_heads), dim3(kNT), 0, stream, args);
  hipLaunchKernelGGL(fit_norm_merge_kernel, dim3(nb, args.n_heads), dim3(kSegMax), 0, stream, args, logz);
  return hipGetLastError();
}

hipError_t launch_lognorm_band(const FitStepArgs& args, float* smax_a, float* smax_r, hipStream_t stream) {
  if (args.n_heads <= 0 || args.T <= 0) return hipSuccess;
  hipLaunchKernelGGL(norm_segmax_kernel, dim3(args.nseg, args.n_heads), dim3(kSegMax), 0, stream, args, smax_a,
                     smax_r);
  const int nb = (args.T + kOut - 1) / kOut;
  hipLaunchKernelGGL(fit_norm_part_kernel, dim3(nb, args.maxg, args.n_heads), dim3(kNT), 0, stream, args);
  return hipGetLastError();
}

hipError_t launch_fit_loss(const FitStepArgs& args, const float* negent, float* loss, float* kappa,
                           hipStream_t stream) {
  hipLaunchKernelGGL(fit_loss_kernel, dim3(args.n_heads), dim3(256), 0, stream, args, negent, loss, kappa);
  return hipGetLastError();
}

}  // namespace saf
