// Internal declarations shared by the C-ABI layer and the kernel sources.
// Kernel argument blocks are plain structs passed by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace saf {

// A kernel that uses more than 64 KB of dynamic LDS needs its attribute
// raised once per device.  The result is remembered per (kernel, device)
// only when it succeeds, so a failed attempt is retried by the next call.
template <auto Kernel>
hipError_t ensure_dynamic_lds(size_t bytes) {
  static std::atomic<uint64_t> done{0};  // one bit per device index < 64
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t(1) << dev) : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(Kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

constexpr int kMaxHeads = 256;
constexpr int kLognormChunk = 256;     // keys per step of a normaliser block
constexpr int kLognormMaxGroups = 32;  // at most this many partials per row

// Keys per normaliser partial: a multiple of kLognormChunk chosen so that a
// row has at most kLognormMaxGroups partials (bounding the workspace).
inline int lognorm_group_keys(int T) {
  const int per = (T + kLognormMaxGroups - 1) / kLognormMaxGroups;
  const int rounded = (per + kLognormChunk - 1) / kLognormChunk * kLognormChunk;
  return rounded > kLognormChunk ? rounded : kLognormChunk;
}
inline int lognorm_groups(int T) {
  const int g = lognorm_group_keys(T);
  return (T + g - 1) / g;
}

// One strided [B][H][T][D] tensor: base pointer and element strides of
// (b, h, t); the d stride is 1.
struct TensorRef {
  void* ptr;
  int64_t sb, sh, st;
};

// Forward arguments (both dtypes).
struct FwdArgs {
  TensorRef q, k, v, o;
  const float* a;    // [H][prior_len]
  const float* r;    // [H][prior_len]
  float* lse;        // [B][H][T]; frozen heads' rows already hold log N
  int B, H, T, prior_len;
  float scale_log2;  // softmax_scale * log2(e)
  int n_ord, n_frz;  // number of ordinary / frozen heads
  int kv_group;      // query heads per key/value head (1: multi-head)
  int frz_group;     // batch elements per frozen program
  int n_groups;      // ceil(B / frz_group)
  int nqb;           // number of query blocks
  // bf16 path: normaliser partials (max, sum) in log2 units over groups of
  // lz_group keys, [n_frz][lz_ngroups][T]; the frozen programs merge them
  // and write lse.
  const float2* lz_part;
  int lz_group, lz_ngroups;
  // precomputed log N [H][T] (natural log) of the caller, or null
  const float* logz;
  uint8_t ord_heads[kMaxHeads];
  uint8_t frz_heads[kMaxHeads];
  // head slot of head h in Q (and K with multi-head K/V): h, or h's rank
  // among the ordinary heads when the caller packs Q/K without frozen slots
  uint8_t qk_slot[kMaxHeads];
};

// Backward arguments (both dtypes).
struct BwdArgs {
  TensorRef q, k, v, o, dout, dq, dk, dv;
  const float* a;
  const float* r;
  const float* lse;  // [B][H][T]
  float* delta;      // workspace [B][H][T]: rowsum(dO * O) of ordinary heads
  float* dqacc;      // fused-dQ workspace [B][n_ord][T][D] fp32 (else null)
  int B, H, T, prior_len;
  float scale;       // softmax_scale
  float scale_log2;  // softmax_scale * log2(e)
  int n_ord, n_frz;
  int frz_group, n_groups;
  int nqb, nkb;      // query / key blocks of the respective passes
  uint8_t ord_heads[kMaxHeads];
  uint8_t frz_heads[kMaxHeads];
  uint8_t is_frozen[kMaxHeads];
  // head slot of head h in Q, K, dQ and dK (as in FwdArgs); qk_packed: the
  // frozen heads have no slot there (their zero dQ/dK rows are not written)
  uint8_t qk_slot[kMaxHeads];
  int qk_packed;
};

// Pattern-parameter gradients of frozen heads (both dtypes).
struct PgradArgs {
  TensorRef v, o, dout;
  const float* a;    // [H][prior_len]
  const float* r;    // [H][prior_len]
  const float* lse;  // [B][H][T]; frozen rows hold log N
  float* da;         // [H][prior_len] output
  float* dr;         // [H][prior_len] output
  float* delta;      // workspace [n_frz][B][T]: rowsum(dO * O)
  // bf16 workspace, one row per program (frozen head, batch group, key
  // block, query chunk): column sums [kPgradBN] and diagonal sums [kPgradDiag]
  float* da_part;
  float* dr_part;
  int B, H, T, prior_len;
  int n_frz, frz_group, n_groups, nkb, nch;
  uint8_t frz_heads[kMaxHeads];
};

// Normaliser arguments: for each listed head h, logZ over rows [0, T) is
// written to out[(b * H + h) * T + i] for every b in [0, B).
struct LognormArgs {
  const float* a;
  const float* r;
  float* out;
  int64_t out_b_stride;  // elements between batch copies (0 for one copy)
  int64_t out_h_stride;  // elements between head rows of out
  int n_heads;           // entries of heads[]
  int B;                 // number of batch copies to write
  int T, prior_len;
  uint8_t heads[kMaxHeads];
};

// Launchers (return hipSuccess or the launch error).
hipError_t launch_lognorm(const LognormArgs& args, hipStream_t stream);
hipError_t launch_pattern_dense(int T, int prior_len, const float* a, const float* r, float* w,
                                hipStream_t stream);

hipError_t launch_lognorm_identity(const LognormArgs& args, hipStream_t stream);

// bf16 path: one mixed-head launch for the forward and for the key-block pass.
hipError_t launch_fwd_bf16(const FwdArgs& args, int D, hipStream_t stream);
hipError_t launch_bwd_kv_bf16(const BwdArgs& args, int D, hipStream_t stream);
hipError_t launch_bwd_q_bf16(const BwdArgs& args, int D, hipStream_t stream);
// Fused-dQ backward (bf16, d = 64): delta and dqacc := 0, one key-block launch
// that also accumulates dQ (atomic adds), dQ conversion.  Records ev[*next_ev]
// after each kernel while *next_ev < nev (and advances *next_ev).
hipError_t launch_bwd_fused_bf16(const BwdArgs& args, int D, hipStream_t stream, hipEvent_t* ev, int nev,
                                 int* next_ev);

// fp32 path: one kernel per pass covers both head kinds.
hipError_t launch_fwd_f32(const FwdArgs& args, int D, hipStream_t stream);
hipError_t launch_bwd_pre_f32(const BwdArgs& args, int D, hipStream_t stream);
hipError_t launch_bwd_kv_f32(const BwdArgs& args, int D, hipStream_t stream);
hipError_t launch_bwd_q_f32(const BwdArgs& args, int D, hipStream_t stream);

// Pattern-parameter gradients: rowsum(dO * O) of frozen rows, then the
// column/diagonal sums (bf16: key-block programs and a fixed-order reduction;
// fp32: one thread per output entry).
hipError_t launch_pgrad_delta(const PgradArgs& args, int dtype_bf16, int D, hipStream_t stream);
hipError_t launch_pgrad_bf16(const PgradArgs& args, int D, hipStream_t stream);
hipError_t launch_pgrad_reduce(const PgradArgs& args, hipStream_t stream);
hipError_t launch_pgrad_f32(const PgradArgs& args, int D, hipStream_t stream);
constexpr int kPgradGroup = 2;   // batch elements per bf16 program
constexpr int kPgradBN = 128;    // keys per bf16 program
constexpr int kPgradQC = 512;    // queries per bf16 program
constexpr int kPgradDiag = 640;  // offsets per program: kPgradQC + kPgradBN - 1, padded

// Compact-pattern fitting: target statistics of calibration means.
struct FitTargetArgs {
  const float* ahat;    // [n][T] rows of row_stride floats, heads head_stride apart
  int64_t head_stride, row_stride;
  float floor;          // causal entries are floored at this value
  int n_heads, T, nseg;
  float* inv_s;         // workspace [n][T]: 1 / row sum of the floored entries
  float* row_ent;       // workspace [n][T]: sum_j p log p of each row
  float* part;          // workspace [n][nseg][5][T]: segment partial marginals
  float* eta_abs;       // [n][T] output
  float* eta_rel;       // [n][T] output
  float* negent;        // [n] output
};

// One Adam step of the fit (also the initialisation and the final loss).
struct FitStepArgs {
  const float* eta_abs;  // [n][T]
  const float* eta_rel;  // [n][T]
  const float* a_cur;    // [n][T] parameters at the current point
  const float* r_cur;
  const float* logz;     // [n][T] log N at the current point (natural log)
  float* a_next;         // [n][T] updated parameters
  float* r_next;
  float* m_a;            // [n][T] Adam moments
  float* v_a;
  float* m_r;
  float* v_r;
  // maxima over 256-entry segments ([n][nseg]) of a_cur, r_cur, of the
  // updated a_next, r_next, and of -logz
  const float* smax_a_cur;
  const float* smax_r_cur;
  float* smax_a_next;
  float* smax_r_next;
  float* smax_z;
  // (max, sum) partials of chunk groups: normalisers [n][maxg][T],
  // marginals [n][2][maxg][T]
  float2* part_z;
  float2* part_m;
  int n_heads, T, nseg, maxg;
  int grp_chunks;       // chunks of 256 summation indices per block group
  int64_t prm_stride;   // elements between the a (and r) rows of two heads
  int use_heads;        // a, r row of listed head x is heads[x] (else x)
  float beta1, beta2, eps;
  float lr_bc1;          // lr / (1 - beta1^t)
  float inv_sqrt_bc2;    // 1 / sqrt(1 - beta2^t)
  uint8_t heads[kMaxHeads];
};

constexpr int kFitSegRows = 512;       // rows per partial of the target marginals
constexpr int kSegMax = 256;           // entries per segment maximum of the fit
constexpr int kFitGroupChunks = 4;     // chunks of 256 summation indices per fit block
constexpr float kFitInitFloor = 1e-9f;  // floor inside the initial r

hipError_t launch_fit_targets(const FitTargetArgs& args, hipStream_t stream);
hipError_t launch_fit_init(const FitStepArgs& args, hipStream_t stream);
hipError_t launch_fit_step(const FitStepArgs& args, hipStream_t stream);
// log N of (a_cur, r_cur) into logz (natural log)
hipError_t launch_fit_norm(const FitStepArgs& args, float* logz, hipStream_t stream);
// Normaliser partials of the listed heads for the forward: segment maxima of
// their a and r rows into smax_a / smax_r ([n][nseg]), then (max, sum)
// partials over key groups of grp_chunks * 256 keys into part_z
// ([n][maxg][T], log2 units).
hipError_t launch_lognorm_band(const FitStepArgs& args, float* smax_a, float* smax_r, hipStream_t stream);
hipError_t launch_fit_loss(const FitStepArgs& args, const float* negent, float* loss, float* kappa,
                           hipStream_t stream);

// Calibration statistics over N sequences of ordinary heads.
struct CalibArgs {
  TensorRef q, k;     // bf16 [N][H][T][D]: sb is the sequence stride
  float* ahat;        // [H] heads head_a apart, rows ld_a floats apart
  int64_t ld_a, head_a;
  float* lse2;        // workspace [N][H][T]: row log-sum-exp (log2 units)
  double* part;       // workspace [H][nprog][3]: per-program sums
  double* s_var;      // [H]
  double* s_kl;       // [H]
  int N, H, T;
  int nqb, nprog;     // query blocks; programs per head nqb (nqb + 1)
  int ahat_vec;       // every row of ahat starts 16-byte aligned
  float scale_log2;   // softmax_scale * log2(e)
};

constexpr int kCalibBM = 128;  // queries per calibration program
constexpr int kCalibBN = 64;   // keys per calibration tile

hipError_t launch_calib(const CalibArgs& args, int D, hipStream_t stream);

// Tile geometry of the bf16 kernels (used by the host for grid sizes).
constexpr int kFwdBM = 128;     // queries per forward program
constexpr int kBwdKvBN = 128;   // keys per key-block program
constexpr int kBwdQBM = 128;    // queries per query-block program

}  // namespace saf
