// C ABI of the SAF hybrid attention library: argument validation, head
// lists, workspace accounting and kernel sequencing.  Every check runs on the
// host before anything is enqueued.
#include "saf_hybrid.h"
#include "saf_internal.h"

#include <cmath>
#include <climits>
#include <cstring>
#include <mutex>

namespace {

using saf::BwdArgs;
using saf::FwdArgs;
using saf::LognormArgs;
using saf::TensorRef;

constexpr int32_t kVersion = (1 << 16) | 0;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elem_bytes(int dtype) { return dtype == SAF_BF16 ? 2 : 4; }

bool supported_d(int dtype, int D) {
  if (dtype == SAF_BF16) return D == 64 || D == 96 || D == 128;
  if (dtype == SAF_F32) return D == 16 || D == 32 || D == 64 || D == 96 || D == 128;
  return false;
}

// Common shape checks; counts heads of each kind.
int check_params(const saf_attn_params* p, int* n_ord, int* n_frz) {
  if (!p) return SAF_EINVAL;
  if (p->struct_bytes != sizeof(saf_attn_params)) return SAF_EINVAL;
  if (p->kv_heads < 0 || p->kv_heads > p->H || (p->kv_heads > 0 && p->H % p->kv_heads != 0))
    return SAF_EINVAL;
  if (p->B < 1 || p->H < 1 || p->T < 1 || p->D < 1) return SAF_EINVAL;
  if (p->T > SAF_MAX_T) return SAF_EUNSUPPORTED;
  if (p->H > SAF_MAX_HEADS) return SAF_EUNSUPPORTED;
  if (p->B > 65535) return SAF_EUNSUPPORTED;
  if (p->prior_len < p->T) return SAF_EINVAL;
  if (p->dtype != SAF_F32 && p->dtype != SAF_BF16) return SAF_EUNSUPPORTED;
  if (!supported_d(p->dtype, p->D)) return SAF_EUNSUPPORTED;
  if (std::isnan(p->softmax_scale) || std::isinf(p->softmax_scale)) return SAF_EINVAL;
  if (!p->frozen) return SAF_EINVAL;
  if (p->qk_packed != 0 && p->qk_packed != 1) return SAF_EINVAL;
  if (p->fused_dq != 0 && p->fused_dq != 1) return SAF_EINVAL;
  if (p->n_stage_events < 0 || (p->n_stage_events > 0 && !p->stage_events)) return SAF_EINVAL;
  int o = 0, f = 0;
  for (int h = 0; h < p->H; ++h) {
    if (p->frozen[h] == 1) ++f;
    else if (p->frozen[h] == 0) ++o;
    else return SAF_EINVAL;
  }
  *n_ord = o;
  *n_frz = f;
  // every (b, h, t) offset and B*H*T must fit comfortably in int64 / grids
  if ((int64_t)p->B * p->H * p->T > (int64_t)1 << 40) return SAF_EUNSUPPORTED;
  if (p->dtype == SAF_BF16) {
    // one-dimensional grids of at most B * H * ceil(T / 128) programs
    if ((int64_t)p->B * p->H * ((p->T + 127) / 128) > INT32_MAX) return SAF_EUNSUPPORTED;
  } else if ((int64_t)p->B * p->H > 65535) {
    return SAF_EUNSUPPORTED;  // fp32 kernels put (b, h) in the grid's second dimension
  }
  return SAF_OK;
}

int check_tensor(const void* ptr, const int64_t* s, const saf_attn_params* p) {
  if (!ptr) return SAF_EINVAL;
  if (!aligned(ptr, 16)) return SAF_EINVAL;
  const size_t eb = elem_bytes(p->dtype);
  const int64_t vec = (int64_t)(16 / eb);  // elements per 16 bytes
  for (int x = 0; x < 3; ++x) {
    if (s[x] < 0) return SAF_EINVAL;
    if (s[x] % vec != 0) return SAF_EINVAL;
  }
  if (p->T > 1 && s[2] < p->D) return SAF_EINVAL;  // rows of one head may not overlap
  if (s[2] > SAF_MAX_T_STRIDE) return SAF_EUNSUPPORTED;  // 32-bit tile offsets
  return SAF_OK;
}

TensorRef ref(const void* ptr, const int64_t* s) {
  TensorRef t;
  t.ptr = const_cast<void*>(ptr);
  t.sb = s[0];
  t.sh = s[1];
  t.st = s[2];
  return t;
}

float resolve_scale(const saf_attn_params* p) {
  return p->softmax_scale > 0.f ? p->softmax_scale : 1.0f / std::sqrt((float)p->D);
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// delta [B][H][T]; with the fused-dQ schedule also the fp32 dQ accumulator
// [B][n_ord][T][D].
size_t bwd_ws_bytes(const saf_attn_params* p, int n_ord) {
  const size_t delta = round_up((size_t)p->B * p->H * p->T * sizeof(float), 256);
  if (!p->fused_dq) return delta;
  return delta + round_up((size_t)p->B * n_ord * p->T * p->D * sizeof(float), 256);
}

// bf16 forward with frozen heads: normaliser partials, one float2 per
// (frozen head, key group, row), at most 32 groups, then the maxima of the
// frozen heads' a and r over 256-entry segments.  The fp32 forward needs
// none.
size_t lz_part_bytes(const saf_attn_params* p, int n_frz) {
  return round_up((size_t)n_frz * saf::lognorm_groups(p->T) * p->T * 2 * sizeof(float), 256);
}

size_t fwd_ws_bytes(const saf_attn_params* p, int n_frz) {
  if (p->dtype != SAF_BF16 || n_frz == 0 || p->logz) return 0;
  const size_t nseg = ((size_t)p->T + saf::kSegMax - 1) / saf::kSegMax;
  return lz_part_bytes(p, n_frz) + round_up(2 * (size_t)n_frz * nseg * sizeof(float), 256);
}

// Pattern gradients: D_b of frozen rows; for bf16 also, per program (frozen
// head, batch group, key block, query chunk), the partial column sums and
// diagonal sums.
size_t pgrad_programs(const saf_attn_params* p, int n_frz) {
  const size_t groups = (size_t)(p->B + saf::kPgradGroup - 1) / saf::kPgradGroup;
  const size_t nkb = (size_t)(p->T + saf::kPgradBN - 1) / saf::kPgradBN;
  const size_t nch = (size_t)(p->T + saf::kPgradQC - 1) / saf::kPgradQC;
  return (size_t)n_frz * groups * nkb * nch;
}

struct PgradWs {
  size_t delta, da_part, dr_part, total;
};
PgradWs pgrad_ws(const saf_attn_params* p, int n_frz) {
  PgradWs w{0, 0, 0, 0};
  if (n_frz == 0) return w;
  w.delta = round_up((size_t)n_frz * p->B * p->T * sizeof(float), 256);
  if (p->dtype == SAF_BF16) {
    const size_t progs = pgrad_programs(p, n_frz);
    w.da_part = round_up(progs * saf::kPgradBN * sizeof(float), 256);
    w.dr_part = round_up(progs * saf::kPgradDiag * sizeof(float), 256);
  }
  w.total = w.delta + w.da_part + w.dr_part;
  return w;
}

// Records stage event k when the caller asked for it.
struct Stages {
  const saf_attn_params* p;
  hipStream_t s;
  int next = 0;
  hipError_t mark() {
    if (p->stage_events && next < p->n_stage_events) {
      hipError_t e = hipEventRecord(p->stage_events[next], s);
      ++next;
      return e;
    }
    ++next;
    return hipSuccess;
  }
};

void fill_heads(const saf_attn_params* p, uint8_t* ord, uint8_t* frz, uint8_t* isf) {
  int o = 0, f = 0;
  for (int h = 0; h < p->H; ++h) {
    if (isf) isf[h] = p->frozen[h];
    if (p->frozen[h]) frz[f++] = (uint8_t)h;
    else ord[o++] = (uint8_t)h;
  }
}

// Q/K head slots: h, or the rank among the ordinary heads (packed layout;
// frozen heads get slot 0, which no kernel uses for them).
void fill_slots(const saf_attn_params* p, uint8_t* slot) {
  int o = 0;
  for (int h = 0; h < p->H; ++h) {
    slot[h] = (uint8_t)(p->qk_packed ? (p->frozen[h] ? 0 : o) : h);
    if (!p->frozen[h]) ++o;
  }
}

// Argument checks of the forward (everything but the workspace); counts
// the heads of each kind.
int fwd_check(const saf_attn_params* p, const void* q, const void* k, const void* v, const float* a,
              const float* r, const void* o, const float* lse, int* n_ord_out, int* n_frz_out) {
  int n_ord = 0, n_frz = 0;
  int st = check_params(p, &n_ord, &n_frz);
  if (st != SAF_OK) return st;
  if (n_ord > 0) {
    if ((st = check_tensor(q, p->q_stride, p)) != SAF_OK) return st;
    if ((st = check_tensor(k, p->k_stride, p)) != SAF_OK) return st;
  }
  if ((st = check_tensor(v, p->v_stride, p)) != SAF_OK) return st;
  if ((st = check_tensor(o, p->o_stride, p)) != SAF_OK) return st;
  if (!lse || !aligned(lse, 4)) return SAF_EINVAL;
  if (n_frz > 0 && (!a || !r || !aligned(a, 4) || !aligned(r, 4))) return SAF_EINVAL;
  if (p->logz && !aligned(p->logz, 4)) return SAF_EINVAL;
  *n_ord_out = n_ord;
  *n_frz_out = n_frz;
  return SAF_OK;
}

// The forward's kernels on `stream`, after fwd_check; ws holds at least
// fwd_ws_bytes(p, n_frz) bytes, 256-byte aligned.
int fwd_run(const saf_attn_params* p, int n_ord, int n_frz, const void* q, const void* k, const void* v,
            const float* a, const float* r, void* o, float* lse, void* ws, hipStream_t stream) {
  FwdArgs args;
  std::memset(&args, 0, sizeof(args));
  args.q = ref(q, p->q_stride);
  args.k = ref(k, p->k_stride);
  args.v = ref(v, p->v_stride);
  args.o = ref(o, p->o_stride);
  args.a = a;
  args.r = r;
  args.lse = lse;
  args.B = p->B;
  args.H = p->H;
  args.T = p->T;
  args.prior_len = p->prior_len;
  args.scale_log2 = resolve_scale(p) * 1.4426950408889634f;
  args.n_ord = n_ord;
  args.n_frz = n_frz;
  args.kv_group = p->kv_heads > 0 ? p->H / p->kv_heads : 1;
  fill_heads(p, args.ord_heads, args.frz_heads, nullptr);
  fill_slots(p, args.qk_slot);

  args.logz = p->logz;

  Stages stg{p, stream};
  if (stg.mark() != hipSuccess) return SAF_EHIP;
  if (n_frz > 0 && !p->logz) {
    LognormArgs la;
    std::memset(&la, 0, sizeof(la));
    la.a = a;
    la.r = r;
    la.out = lse;
    la.out_b_stride = (int64_t)p->H * p->T;
    la.out_h_stride = p->T;
    la.n_heads = n_frz;
    la.B = p->B;
    la.T = p->T;
    la.prior_len = p->prior_len;
    std::memcpy(la.heads, args.frz_heads, sizeof(la.heads));
    if (p->dtype == SAF_BF16) {
      // partials only; the forward's frozen programs merge them and write lse
      args.lz_part = static_cast<const float2*>(ws);
      args.lz_group = saf::lognorm_group_keys(p->T);
      args.lz_ngroups = saf::lognorm_groups(p->T);
      // the band-sum program of the fit, over the frozen heads' rows of a, r
      saf::FitStepArgs na;
      std::memset(&na, 0, sizeof(na));
      na.a_cur = a;
      na.r_cur = r;
      na.prm_stride = p->prior_len;
      na.use_heads = 1;
      std::memcpy(na.heads, args.frz_heads, sizeof(na.heads));
      na.n_heads = n_frz;
      na.T = p->T;
      na.nseg = (p->T + saf::kSegMax - 1) / saf::kSegMax;
      na.grp_chunks = args.lz_group / saf::kSegMax;
      na.maxg = args.lz_ngroups;
      na.part_z = static_cast<float2*>(ws);
      float* smax = reinterpret_cast<float*>(static_cast<char*>(ws) + lz_part_bytes(p, n_frz));
      na.smax_a_cur = smax;
      na.smax_r_cur = smax + (size_t)n_frz * na.nseg;
      if (saf::launch_lognorm_band(na, smax, smax + (size_t)n_frz * na.nseg, stream) != hipSuccess)
        return SAF_EHIP;
    } else {
      if (saf::launch_lognorm(la, stream) != hipSuccess) return SAF_EHIP;
    }
    if (stg.mark() != hipSuccess) return SAF_EHIP;
  }
  if (p->dtype == SAF_BF16) {
    if (saf::launch_fwd_bf16(args, p->D, stream) != hipSuccess) return SAF_EHIP;
    if (stg.mark() != hipSuccess) return SAF_EHIP;
  } else {
    if (saf::launch_fwd_f32(args, p->D, stream) != hipSuccess) return SAF_EHIP;
    if (stg.mark() != hipSuccess) return SAF_EHIP;
  }
  return SAF_OK;
}

// Scratch of saf_hybrid_attn_fwd_noalloc: one array per device, for callers
// that cannot allocate.  Host code never uses the array's name as an
// address: the device address comes from hipGetSymbolAddress, taken once per
// device with that device current, and is kept per device.
static __device__ __align__(256) unsigned char scratch[SAF_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, or null on a HIP error.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* saf_status_string(int status) {
  switch (status) {
    case SAF_OK: return "ok";
    case SAF_EINVAL: return "invalid argument (pointer, size, stride or alignment)";
    case SAF_EUNSUPPORTED: return "unsupported configuration (head dim, dtype or size)";
    case SAF_EWORKSPACE: return "workspace missing, misaligned or too small";
    case SAF_EHIP: return "HIP runtime or launch failure";
    case SAF_ESCRATCH: return "shape needs more scratch than the no-allocation entry point holds";
    default: return "unknown status";
  }
}

int32_t saf_version(void) { return kVersion; }

size_t saf_hybrid_attn_workspace_bytes(const saf_attn_params* p, int for_bwd) {
  int o, f;
  if (check_params(p, &o, &f) != SAF_OK) return 0;
  return for_bwd ? bwd_ws_bytes(p, o) : fwd_ws_bytes(p, f);
}

int saf_hybrid_attn_fwd(const saf_attn_params* p, const void* q, const void* k, const void* v,
                        const float* a, const float* r, void* o, float* lse, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  int n_ord = 0, n_frz = 0;
  int st = fwd_check(p, q, k, v, a, r, o, lse, &n_ord, &n_frz);
  if (st != SAF_OK) return st;
  const size_t need = fwd_ws_bytes(p, n_frz);
  if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 256))) return SAF_EWORKSPACE;
  return fwd_run(p, n_ord, n_frz, q, k, v, a, r, o, lse, ws, stream);
}

int saf_hybrid_attn_fwd_noalloc(const saf_attn_params* p, const void* q, const void* k, const void* v,
                                const float* a, const float* r, void* o, float* lse,
                                hipStream_t stream) {
  int n_ord = 0, n_frz = 0;
  int st = fwd_check(p, q, k, v, a, r, o, lse, &n_ord, &n_frz);
  if (st != SAF_OK) return st;
  if (fwd_ws_bytes(p, n_frz) > SAF_NOALLOC_SCRATCH_BYTES) return SAF_ESCRATCH;
  void* ws = nullptr;
  if (fwd_ws_bytes(p, n_frz) > 0 && !(ws = scratch_ptr())) return SAF_EHIP;
  return fwd_run(p, n_ord, n_frz, q, k, v, a, r, o, lse, ws, stream);
}

int saf_hybrid_attn_bwd(const saf_attn_params* p, const void* q, const void* k, const void* v,
                        const void* o, const void* dout, const float* lse, const float* a,
                        const float* r, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  int n_ord = 0, n_frz = 0;
  int st = check_params(p, &n_ord, &n_frz);
  if (st != SAF_OK) return st;
  if (p->kv_heads != 0 && p->kv_heads != p->H) return SAF_EUNSUPPORTED;  // grouped-query: forward only
  if (n_ord > 0) {
    if ((st = check_tensor(q, p->q_stride, p)) != SAF_OK) return st;
    if ((st = check_tensor(k, p->k_stride, p)) != SAF_OK) return st;
    if ((st = check_tensor(v, p->v_stride, p)) != SAF_OK) return st;
    if ((st = check_tensor(o, p->o_stride, p)) != SAF_OK) return st;
  }
  if ((st = check_tensor(dout, p->do_stride, p)) != SAF_OK) return st;
  if (n_ord > 0 || !p->qk_packed) {  // packed with no ordinary head: no dQ/dK rows at all
    if ((st = check_tensor(dq, p->dq_stride, p)) != SAF_OK) return st;
    if ((st = check_tensor(dk, p->dk_stride, p)) != SAF_OK) return st;
  }
  if ((st = check_tensor(dv, p->dv_stride, p)) != SAF_OK) return st;
  if (!lse || !aligned(lse, 4)) return SAF_EINVAL;
  if (n_frz > 0 && (!a || !r || !aligned(a, 4) || !aligned(r, 4))) return SAF_EINVAL;
  if (p->fused_dq && (p->dtype != SAF_BF16 || p->D != 64)) return SAF_EUNSUPPORTED;
  const size_t need = bwd_ws_bytes(p, n_ord);
  if (!ws || ws_bytes < need || !aligned(ws, 256)) return SAF_EWORKSPACE;

  BwdArgs args;
  std::memset(&args, 0, sizeof(args));
  args.q = ref(q, p->q_stride);
  args.k = ref(k, p->k_stride);
  args.v = ref(v, p->v_stride);
  args.o = ref(o, p->o_stride);
  args.dout = ref(dout, p->do_stride);
  args.dq = ref(dq, p->dq_stride);
  args.dk = ref(dk, p->dk_stride);
  args.dv = ref(dv, p->dv_stride);
  args.a = a;
  args.r = r;
  args.lse = lse;
  args.delta = static_cast<float*>(ws);
  if (p->fused_dq)
    args.dqacc = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                          round_up((size_t)p->B * p->H * p->T * sizeof(float), 256));
  args.B = p->B;
  args.H = p->H;
  args.T = p->T;
  args.prior_len = p->prior_len;
  args.scale = resolve_scale(p);
  args.scale_log2 = args.scale * 1.4426950408889634f;
  args.n_ord = n_ord;
  args.n_frz = n_frz;
  fill_heads(p, args.ord_heads, args.frz_heads, args.is_frozen);
  fill_slots(p, args.qk_slot);
  args.qk_packed = p->qk_packed;

  Stages stg{p, stream};
  if (stg.mark() != hipSuccess) return SAF_EHIP;
  hipError_t e;
  if (p->dtype == SAF_BF16 && p->fused_dq) {
    e = saf::launch_bwd_fused_bf16(args, p->D, stream, p->stage_events, p->n_stage_events, &stg.next);
    if (e != hipSuccess) return SAF_EHIP;
  } else if (p->dtype == SAF_BF16) {
    // query-block pass (also stores delta), then the mixed key-block pass
    // (which reads delta and writes the frozen heads' zero dQ/dK rows)
    if (n_ord > 0) {
      e = saf::launch_bwd_q_bf16(args, p->D, stream);
      if (e != hipSuccess || stg.mark() != hipSuccess) return SAF_EHIP;
    }
    e = saf::launch_bwd_kv_bf16(args, p->D, stream);
    if (e != hipSuccess || stg.mark() != hipSuccess) return SAF_EHIP;
  } else {
    e = saf::launch_bwd_pre_f32(args, p->D, stream);
    if (e != hipSuccess || stg.mark() != hipSuccess) return SAF_EHIP;
    e = saf::launch_bwd_kv_f32(args, p->D, stream);
    if (e != hipSuccess || stg.mark() != hipSuccess) return SAF_EHIP;
    if (n_ord > 0) {
      e = saf::launch_bwd_q_f32(args, p->D, stream);
      if (e != hipSuccess || stg.mark() != hipSuccess) return SAF_EHIP;
    }
  }
  return SAF_OK;
}

size_t saf_pattern_grad_workspace_bytes(const saf_attn_params* p) {
  int o, f;
  if (check_params(p, &o, &f) != SAF_OK) return 0;
  return pgrad_ws(p, f).total;
}

int saf_pattern_grad(const saf_attn_params* p, const void* v, const void* o, const void* dout,
                     const float* lse, const float* a, const float* r, float* da, float* dr,
                     void* ws, size_t ws_bytes, hipStream_t stream) {
  int n_ord = 0, n_frz = 0;
  int st = check_params(p, &n_ord, &n_frz);
  if (st != SAF_OK) return st;
  if (p->kv_heads != 0 && p->kv_heads != p->H) return SAF_EUNSUPPORTED;  // grouped-query: forward only
  if ((st = check_tensor(v, p->v_stride, p)) != SAF_OK) return st;
  if ((st = check_tensor(o, p->o_stride, p)) != SAF_OK) return st;
  if ((st = check_tensor(dout, p->do_stride, p)) != SAF_OK) return st;
  if (!lse || !a || !r || !da || !dr) return SAF_EINVAL;
  if (!aligned(lse, 4) || !aligned(a, 4) || !aligned(r, 4) || !aligned(da, 4) || !aligned(dr, 4))
    return SAF_EINVAL;
  // bf16: one program per (frozen head, batch group, key block, query chunk)
  if (p->dtype == SAF_BF16 && pgrad_programs(p, n_frz) > (size_t)INT32_MAX) return SAF_EUNSUPPORTED;
  const PgradWs w = pgrad_ws(p, n_frz);
  if (w.total > 0 && (!ws || ws_bytes < w.total || !aligned(ws, 256))) return SAF_EWORKSPACE;
  if (n_frz == 0) return SAF_OK;

  saf::PgradArgs args;
  std::memset(&args, 0, sizeof(args));
  args.v = ref(v, p->v_stride);
  args.o = ref(o, p->o_stride);
  args.dout = ref(dout, p->do_stride);
  args.a = a;
  args.r = r;
  args.lse = lse;
  args.da = da;
  args.dr = dr;
  char* base = static_cast<char*>(ws);
  args.delta = reinterpret_cast<float*>(base);
  args.da_part = w.da_part ? reinterpret_cast<float*>(base + w.delta) : nullptr;
  args.dr_part = w.dr_part ? reinterpret_cast<float*>(base + w.delta + w.da_part) : nullptr;
  args.B = p->B;
  args.H = p->H;
  args.T = p->T;
  args.prior_len = p->prior_len;
  args.n_frz = n_frz;
  args.frz_group = saf::kPgradGroup;
  args.n_groups = (p->B + saf::kPgradGroup - 1) / saf::kPgradGroup;
  args.nkb = (p->T + saf::kPgradBN - 1) / saf::kPgradBN;
  args.nch = (p->T + saf::kPgradQC - 1) / saf::kPgradQC;
  uint8_t ord[saf::kMaxHeads];
  fill_heads(p, ord, args.frz_heads, nullptr);

  Stages stg{p, stream};
  if (stg.mark() != hipSuccess) return SAF_EHIP;
  const int bf16 = p->dtype == SAF_BF16;
  hipError_t e = saf::launch_pgrad_delta(args, bf16, p->D, stream);
  if (e != hipSuccess || stg.mark() != hipSuccess) return SAF_EHIP;
  if (bf16) {
    e = saf::launch_pgrad_bf16(args, p->D, stream);
    if (e != hipSuccess || stg.mark() != hipSuccess) return SAF_EHIP;
    e = saf::launch_pgrad_reduce(args, stream);
    if (e != hipSuccess || stg.mark() != hipSuccess) return SAF_EHIP;
  } else {
    e = saf::launch_pgrad_f32(args, p->D, stream);
    if (e != hipSuccess || stg.mark() != hipSuccess) return SAF_EHIP;
  }
  return SAF_OK;
}

int saf_pattern_dense(int32_t T, int32_t prior_len, const float* a, const float* r, float* w,
                      hipStream_t stream) {
  if (T < 1 || T > 32768 || prior_len < T) return SAF_EINVAL;
  if (!a || !r || !w || !aligned(a, 4) || !aligned(r, 4) || !aligned(w, 4)) return SAF_EINVAL;
  return saf::launch_pattern_dense(T, prior_len, a, r, w, stream) == hipSuccess ? SAF_OK : SAF_EHIP;
}

int saf_pattern_lognorm(int32_t n_heads, int32_t T, int32_t prior_len, const float* a,
                        const float* r, float* logz, hipStream_t stream) {
  if (n_heads < 1 || n_heads > 65535 || T < 1 || T > SAF_MAX_T || prior_len < T) return SAF_EINVAL;
  if (!a || !r || !logz || !aligned(a, 4) || !aligned(r, 4) || !aligned(logz, 4)) return SAF_EINVAL;
  LognormArgs la;
  std::memset(&la, 0, sizeof(la));
  la.a = a;
  la.r = r;
  la.out = logz;
  la.out_b_stride = 0;
  la.out_h_stride = T;
  la.n_heads = n_heads;
  la.B = 1;
  la.T = T;
  la.prior_len = prior_len;
  return saf::launch_lognorm_identity(la, stream) == hipSuccess ? SAF_OK : SAF_EHIP;
}

namespace {

bool fit_sizes_ok(int32_t n_heads, int32_t T) {
  return n_heads >= 1 && n_heads <= SAF_MAX_FIT_HEADS && T >= 1 && T <= SAF_MAX_T;
}

size_t fit_targets_ws(int32_t n_heads, int32_t T) {
  const size_t nT = (size_t)n_heads * (size_t)T;
  const size_t nseg = ((size_t)T + saf::kFitSegRows - 1) / saf::kFitSegRows;
  return 2 * round_up(nT * sizeof(float), 256) + round_up(nT * 5 * nseg * sizeof(float), 256);
}

size_t fit_maxg(int32_t T) {
  const size_t nseg = ((size_t)T + saf::kSegMax - 1) / saf::kSegMax;
  return (nseg + saf::kFitGroupChunks - 1) / saf::kFitGroupChunks;
}

size_t fit_pattern_ws(int32_t n_heads, int32_t T) {
  const size_t nseg = ((size_t)T + saf::kSegMax - 1) / saf::kSegMax;
  const size_t part = (size_t)n_heads * fit_maxg(T) * (size_t)T * 2 * sizeof(float);
  return 6 * round_up((size_t)n_heads * (size_t)T * sizeof(float), 256) +
         5 * round_up((size_t)n_heads * nseg * sizeof(float), 256) + round_up(part, 256) + round_up(2 * part, 256);
}

}  // namespace

size_t saf_fit_targets_workspace_bytes(int32_t n_heads, int32_t T) {
  return fit_sizes_ok(n_heads, T) ? fit_targets_ws(n_heads, T) : 0;
}

int saf_fit_targets(int32_t n_heads, int32_t T, const float* ahat, int64_t head_stride,
                    int64_t row_stride, float floor, float* eta_abs, float* eta_rel, float* negent,
                    void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!fit_sizes_ok(n_heads, T)) return SAF_EINVAL;
  if (!(floor > 0.f) || !std::isfinite(floor)) return SAF_EINVAL;
  if (!ahat || !aligned(ahat, 4) || row_stride < T || head_stride < 0) return SAF_EINVAL;
  if (!eta_abs || !eta_rel || !negent || !aligned(eta_abs, 4) || !aligned(eta_rel, 4) ||
      !aligned(negent, 4))
    return SAF_EINVAL;
  const size_t need = fit_targets_ws(n_heads, T);
  if (!ws || !aligned(ws, 256) || ws_bytes < need) return SAF_EWORKSPACE;
  const size_t nT = (size_t)n_heads * (size_t)T;
  char* w = static_cast<char*>(ws);
  saf::FitTargetArgs ta;
  std::memset(&ta, 0, sizeof(ta));
  ta.ahat = ahat;
  ta.head_stride = head_stride;
  ta.row_stride = row_stride;
  ta.floor = floor;
  ta.n_heads = n_heads;
  ta.T = T;
  ta.nseg = (T + saf::kFitSegRows - 1) / saf::kFitSegRows;
  ta.inv_s = reinterpret_cast<float*>(w);
  ta.row_ent = reinterpret_cast<float*>(w + round_up(nT * sizeof(float), 256));
  ta.part = reinterpret_cast<float*>(w + 2 * round_up(nT * sizeof(float), 256));
  ta.eta_abs = eta_abs;
  ta.eta_rel = eta_rel;
  ta.negent = negent;
  return saf::launch_fit_targets(ta, stream) == hipSuccess ? SAF_OK : SAF_EHIP;
}

size_t saf_fit_pattern_workspace_bytes(int32_t n_heads, int32_t T) {
  return fit_sizes_ok(n_heads, T) ? fit_pattern_ws(n_heads, T) : 0;
}

int saf_fit_pattern(int32_t n_heads, int32_t T, const float* eta_abs, const float* eta_rel,
                    const float* negent, int32_t steps, float lr, float beta1, float beta2, float eps,
                    float* a, float* r, float* logz, float* loss, float* kappa, void* ws,
                    size_t ws_bytes, hipStream_t stream) {
  if (!fit_sizes_ok(n_heads, T) || steps < 0) return SAF_EINVAL;
  if (!(lr > 0.f) || !std::isfinite(lr) || !(beta1 >= 0.f && beta1 < 1.f) ||
      !(beta2 >= 0.f && beta2 < 1.f) || !(eps > 0.f) || !std::isfinite(eps))
    return SAF_EINVAL;
  const float* in[] = {eta_abs, eta_rel, a, r, logz};
  for (const float* x : in)
    if (!x || !aligned(x, 4)) return SAF_EINVAL;
  if ((negent && !aligned(negent, 4)) || (loss && !aligned(loss, 4)) || (kappa && !aligned(kappa, 4)))
    return SAF_EINVAL;
  if (kappa && !negent) return SAF_EINVAL;
  const size_t need = fit_pattern_ws(n_heads, T);
  if (!ws || !aligned(ws, 256) || ws_bytes < need) return SAF_EWORKSPACE;
  const size_t vec = round_up((size_t)n_heads * (size_t)T * sizeof(float), 256);
  char* w = static_cast<char*>(ws);
  float* pa[2] = {a, reinterpret_cast<float*>(w)};
  float* pr[2] = {r, reinterpret_cast<float*>(w + vec)};

  saf::FitStepArgs fa;
  std::memset(&fa, 0, sizeof(fa));
  fa.eta_abs = eta_abs;
  fa.eta_rel = eta_rel;
  fa.logz = logz;
  fa.m_a = reinterpret_cast<float*>(w + 2 * vec);
  fa.v_a = reinterpret_cast<float*>(w + 3 * vec);
  fa.m_r = reinterpret_cast<float*>(w + 4 * vec);
  fa.v_r = reinterpret_cast<float*>(w + 5 * vec);
  const size_t segv = round_up((size_t)n_heads * (((size_t)T + saf::kSegMax - 1) / saf::kSegMax) * sizeof(float), 256);
  float* sa[2] = {reinterpret_cast<float*>(w + 6 * vec), reinterpret_cast<float*>(w + 6 * vec + segv)};
  float* sr[2] = {reinterpret_cast<float*>(w + 6 * vec + 2 * segv), reinterpret_cast<float*>(w + 6 * vec + 3 * segv)};
  fa.smax_z = reinterpret_cast<float*>(w + 6 * vec + 4 * segv);
  const size_t part = (size_t)n_heads * fit_maxg(T) * (size_t)T * 2 * sizeof(float);
  fa.part_z = reinterpret_cast<float2*>(w + 6 * vec + 5 * segv);
  fa.part_m = reinterpret_cast<float2*>(w + 6 * vec + 5 * segv + round_up(part, 256));
  fa.maxg = (int)fit_maxg(T);
  fa.grp_chunks = saf::kFitGroupChunks;
  fa.prm_stride = T;
  fa.use_heads = 0;
  fa.n_heads = n_heads;
  fa.T = T;
  fa.nseg = (T + saf::kSegMax - 1) / saf::kSegMax;
  fa.beta1 = beta1;
  fa.beta2 = beta2;
  fa.eps = eps;

  // step t reads buffer (t - 1 + s0) & 1 and writes (t + s0) & 1, so the
  // last step lands in the caller's a and r
  const int s0 = steps & 1;
  fa.a_next = pa[s0];
  fa.r_next = pr[s0];
  fa.smax_a_next = sa[s0];
  fa.smax_r_next = sr[s0];
  if (saf::launch_fit_init(fa, stream) != hipSuccess) return SAF_EHIP;
  for (int t = 1; t <= steps; ++t) {
    const int cur = (t - 1 + s0) & 1, nxt = (t + s0) & 1;
    fa.a_cur = pa[cur];
    fa.r_cur = pr[cur];
    fa.smax_a_cur = sa[cur];
    fa.smax_r_cur = sr[cur];
    if (saf::launch_fit_norm(fa, logz, stream) != hipSuccess) return SAF_EHIP;
    fa.a_next = pa[nxt];
    fa.r_next = pr[nxt];
    fa.smax_a_next = sa[nxt];
    fa.smax_r_next = sr[nxt];
    const double bc1 = 1.0 - std::pow((double)beta1, (double)t);
    const double bc2 = 1.0 - std::pow((double)beta2, (double)t);
    fa.lr_bc1 = (float)((double)lr / bc1);
    fa.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(bc2));
    if (saf::launch_fit_step(fa, stream) != hipSuccess) return SAF_EHIP;
  }
  fa.a_cur = a;
  fa.r_cur = r;
  fa.smax_a_cur = sa[0];
  fa.smax_r_cur = sr[0];
  if (saf::launch_fit_norm(fa, logz, stream) != hipSuccess) return SAF_EHIP;
  if (loss || kappa) {
    if (saf::launch_fit_loss(fa, negent, loss, kappa, stream) != hipSuccess) return SAF_EHIP;
  }
  return SAF_OK;
}

namespace {

bool calib_sizes_ok(int32_t N, int32_t H, int32_t T) {
  return N >= 1 && N <= 65535 && H >= 1 && H <= 65535 && T >= 1 && T <= SAF_MAX_T;
}

size_t calib_ws(int32_t N, int32_t H, int32_t T) {
  const size_t nqb = ((size_t)T + saf::kCalibBM - 1) / saf::kCalibBM;
  const size_t nprog = nqb * (nqb + 1);
  return round_up((size_t)N * H * T * sizeof(float), 256) + round_up((size_t)H * nprog * 3 * sizeof(double), 256);
}

bool calib_tensor_ok(const void* p, const int64_t* st, int32_t D) {
  if (!p || !st || !aligned(p, 16)) return false;
  for (int x = 0; x < 3; ++x)
    if (st[x] < 0 || st[x] % 8 != 0) return false;
  return st[2] >= D && st[2] <= SAF_MAX_T_STRIDE;
}

}  // namespace

size_t saf_calib_stats_workspace_bytes(int32_t N, int32_t H, int32_t T) {
  return calib_sizes_ok(N, H, T) ? calib_ws(N, H, T) : 0;
}

int saf_calib_stats(int32_t N, int32_t H, int32_t T, int32_t D, float softmax_scale, const void* q,
                    const int64_t q_stride[3], const void* k, const int64_t k_stride[3], float* ahat,
                    int64_t ahat_head_stride, int64_t ahat_row_stride, double* s_var, double* s_kl,
                    void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!calib_sizes_ok(N, H, T)) return SAF_EINVAL;
  if (D != 64 && D != 96 && D != 128) return SAF_EUNSUPPORTED;
  if (!std::isfinite(softmax_scale)) return SAF_EINVAL;
  if (!calib_tensor_ok(q, q_stride, D) || !calib_tensor_ok(k, k_stride, D)) return SAF_EINVAL;
  if (!ahat || !aligned(ahat, 4) || ahat_row_stride < T || ahat_head_stride < 0) return SAF_EINVAL;
  if (!s_var || !s_kl || !aligned(s_var, 8) || !aligned(s_kl, 8)) return SAF_EINVAL;
  const size_t need = calib_ws(N, H, T);
  if (!ws || !aligned(ws, 256) || ws_bytes < need) return SAF_EWORKSPACE;
  const int nqb = (T + saf::kCalibBM - 1) / saf::kCalibBM;
  const int64_t nprog = (int64_t)nqb * (nqb + 1);
  if (nprog > INT32_MAX) return SAF_EUNSUPPORTED;
  saf::CalibArgs ca;
  std::memset(&ca, 0, sizeof(ca));
  ca.q = TensorRef{const_cast<void*>(q), q_stride[0], q_stride[1], q_stride[2]};
  ca.k = TensorRef{const_cast<void*>(k), k_stride[0], k_stride[1], k_stride[2]};
  ca.ahat = ahat;
  ca.ld_a = ahat_row_stride;
  ca.head_a = ahat_head_stride;
  char* w = static_cast<char*>(ws);
  ca.lse2 = reinterpret_cast<float*>(w);
  ca.part = reinterpret_cast<double*>(w + round_up((size_t)N * H * T * sizeof(float), 256));
  ca.s_var = s_var;
  ca.s_kl = s_kl;
  ca.N = N;
  ca.H = H;
  ca.T = T;
  ca.nqb = nqb;
  ca.nprog = (int)nprog;
  ca.ahat_vec = aligned(ahat, 16) && ahat_row_stride % 4 == 0 && ahat_head_stride % 4 == 0;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.f / std::sqrt((float)D);
  ca.scale_log2 = scale * 1.4426950408889634f;
  return saf::launch_calib(ca, D, stream) == hipSuccess ? SAF_OK : SAF_EHIP;
}

}  // extern "C"
