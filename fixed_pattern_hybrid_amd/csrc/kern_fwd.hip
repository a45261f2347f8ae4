// Forward of the SAF hybrid attention layer, bf16, gfx950.
//
// Head kinds ("When Can Attention Heads Be Statically Defined?", Section 3.3
// "Fused computation" and Appendix D.2):
//   * ordinary head, one program per (b, h, query block): online-softmax
//     tiling of causal attention (Appendix A.1, Equations 5-7);
//   * frozen head, one program per (h, query block, group of batch
//     elements): each causal tile of the compact pattern (Section 3.2,
//     Equation 3) is rebuilt in registers once from a, r and the precomputed
//     row normalisers, then multiplied with the value tiles of every batch
//     element of the group.  The weights do not depend on the batch index,
//     so one rebuild serves the whole group.
// Outputs are written in the original head order.  Both kinds run in one
// launch; with accumulators in VGPRs and batch groups of two, the two program
// bodies need about the same registers and LDS, so sharing a launch costs no
// occupancy and lets the few frozen programs fill gaps in the schedule.
//
// Work layout: 4 waves, 32 queries per wave, key tiles of 64.  Products are
// computed transposed (S^T = K Q^T, O^T = V^T P^T) so that every lane owns
// one query: row max, row sum and rescaling stay in the lane, and the C
// registers of S^T convert directly into the B operand of the second product
// (V^T comes from LDS through transposing reads).
#include <type_traits>

#include "saf_internal.h"
#include "saf_tile.h"

namespace saf {
namespace {

constexpr int kBM = kFwdBM;  // queries per program
constexpr int kBN = 64;      // keys per tile
constexpr int kThreads = 256;

template <int D>
struct FwdCfg {
  // K and V tiles in LDS: swizzled at d = 128, where the transposing reads
  // of V bound the frozen programs (5-6% faster forward); padded at d = 64,
  // where the swizzle's lane offsets cost more registers than it saves (2%)
  using L = std::conditional_t<D == 128, SwzLayout<D>, LdsLayout<D>>;
  static constexpr int PITCH = L::PITCH;     // LDS row pitch (elements)
  static constexpr int NDB = D / 32;   // 32-wide blocks of the head dimension
  static constexpr int NKS = D / 16;   // 16-deep k steps over the head dimension
  static constexpr int G = 2;                  // batch elements per frozen program
  static constexpr int TILE = kBN * PITCH;     // elements of one staged tile
  static constexpr int BAND = kBM + kBN;       // r band length (BM + BN - 1, padded)
  // per buffer: a2[kBN], then 2 copies of the band, copy c shifted by c
  // (two, not four: 40.7 KB per frozen program keeps four blocks per CU)
  static constexpr int BSTRIDE = band_stride(BAND);  // distance between band copies
  static constexpr int FSTRIDE = kBN + 2 * BSTRIDE;
  static constexpr size_t ord_lds = size_t(2) * 2 * TILE * 2;
  static constexpr size_t frz_lds = size_t(2) * G * TILE * 2 + size_t(2) * FSTRIDE * 4;
};

template <int D>
__device__ __forceinline__ void store_out_rows(const TensorRef& o, int b, int h, int i, int T,
                                               const f32x16* acc, float mul) {
  if (i >= T) return;
  const int hl = lane_id() >> 5;
  __bf16* row = (__bf16*)o.ptr + (int64_t)b * o.sb + (int64_t)h * o.sh + (int64_t)i * o.st;
#pragma unroll
  for (int db = 0; db < FwdCfg<D>::NDB; ++db) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = 32 * db + 8 * q4 + 4 * hl;
      bf16x4 v;
      v[0] = (__bf16)(acc[db][4 * q4 + 0] * mul);
      v[1] = (__bf16)(acc[db][4 * q4 + 1] * mul);
      v[2] = (__bf16)(acc[db][4 * q4 + 2] * mul);
      v[3] = (__bf16)(acc[db][4 * q4 + 3] * mul);
      *reinterpret_cast<bf16x4*>(row + d) = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Ordinary head program (b, h, query block): causal softmax attention with an
// online row maximum.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void fwd_ordinary(const FwdArgs& A, int b, int h, int qb, lds_bf16* smem) {
  using C = FwdCfg<D>;

  const int l = lane_id(), w = wave_id(), hl = l >> 5;
  const int T = A.T;
  const int q0 = qb * kBM;
  const int i = q0 + 32 * w + (l & 31);  // this lane's query
  const int wq_lo = q0 + 32 * w, wq_hi = wq_lo + 31;

  const int hk = h / A.kv_group;  // key/value head of this query head
  const int kslot = A.kv_group == 1 ? A.qk_slot[h] : hk;  // its K slot
  const __bf16* qg = (const __bf16*)A.q.ptr + (int64_t)b * A.q.sb + (int64_t)A.qk_slot[h] * A.q.sh;
  const __bf16* kg = (const __bf16*)A.k.ptr + (int64_t)b * A.k.sb + (int64_t)kslot * A.k.sh;
  const __bf16* vg = (const __bf16*)A.v.ptr + (int64_t)b * A.v.sb + (int64_t)hk * A.v.sh;

  // Q as the B operand of S^T = K Q^T: lane holds Q[i][16ks + 8*hl + 0..7].
  bf16x8 qf[C::NKS];
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks) {
    if (i < T) {
      qf[ks] = __builtin_bit_cast(bf16x8, gload16(qg + (int64_t)i * A.q.st + 16 * ks + 8 * hl));
    } else {
      qf[ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
  }

  // LDS: K[buf], V[buf] at (2*kind + buf) * TILE
  const int last_key = min(q0 + kBM, T) - 1;
  const int ntiles = last_key / kBN + 1;

  // K and V tiles are copied straight into the idle LDS buffer at the start
  // of the previous tile.
  TileDma<D, kBN, true, typename C::L> kdma, vdma;
  kdma.init(A.k.st);
  vdma.init(A.v.st);
  kdma.issue(kg, A.k.st, 0, T, smem);
  vdma.issue(vg, A.v.st, 0, T, smem + 2 * C::TILE);
  wait_vm_loads();
  __syncthreads();

  f32x16 oacc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) oacc[db] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;
  const float sl2 = A.scale_log2;

  // One key tile: S^T = K Q^T, online softmax, O^T += V^T P^T.  MASK is set
  // only for the tiles that reach the diagonal (the last two of the block),
  // so the unmasked tiles carry no masking instructions.
  auto tile = [&](int t, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int j0 = t * kBN;
    const bool more = (t + 1) < ntiles;
    if (more) {
      kdma.issue(kg, A.k.st, j0 + kBN, T, smem + ((t + 1) & 1) * C::TILE);
      vdma.issue(vg, A.v.st, j0 + kBN, T, smem + (2 + ((t + 1) & 1)) * C::TILE);
    }
    const lds_bf16* K = smem + (t & 1) * C::TILE;
    const lds_bf16* V = smem + (2 + (t & 1)) * C::TILE;
    if (!MASK || j0 <= wq_hi) {
      f32x16 s[2];
      auto scores = [&]() {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          s[c] = f32x16{};
#pragma unroll
          for (int ks = 0; ks < C::NKS; ++ks)
            s[c] = mfma32(lds_frag_nat<D, typename C::L>(K, 32 * c, 16 * ks), qf[ks], s[c]);
        }
        if constexpr (MASK) {
#pragma unroll
          for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int j = j0 + 32 * c + 8 * (r >> 2) + 4 * hl + (r & 3);
              if (j > i) s[c][r] = kNegInf;
            }
        }
      };
      // p = exp2(s * scale_log2 - m) in place; returns this lane's sum
      auto exps = [&](float m) {
        float psum = 0.f;
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = fast_exp2(fmaf(s[c][r], sl2, -m));
            s[c][r] = p;
            psum += p;
          }
        return psum;
      };
      scores();
      // Lazy rescaling: the reference maximum m_run only moves when a score
      // exceeds it by more than 8 (log2 units), so every p <= 2^8.  The
      // exponentials are first taken against m_run; a lane sum <= 2^8 proves
      // every p <= 2^8 (and finite), and then the tile maximum is never
      // needed.  Otherwise (the first tile, a grown maximum, or a rare false
      // alarm) the scores are recomputed and the maximum is taken as usual.
      // The final O = acc / l and lse = m + log2(l) are exact for any
      // reference value.
      float psum = exps(m_run);
      if (__any(!(psum <= 256.f))) {
        // keep this a real branch (it is taken on few tiles)
        asm volatile("");
        scores();
        float mx = kNegInf;
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[c][r]);
        mx = fmaxf(mx, xor32(mx));
        const float mt = mx * sl2;
        const bool grow = mt > m_run + 8.f;
        const float m_new = grow ? mt : m_run;
        const float alpha = fast_exp2(m_run - m_new);
        psum = exps(m_new);
        l_run *= alpha;
        m_run = m_new;
        if (__any(grow)) {
#pragma unroll
          for (int db = 0; db < C::NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        }
      }
      l_run += psum;
      // O^T += V^T P^T
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const bf16x8 pf = pack_acc8(s[st >> 1], 8 * (st & 1));
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
          oacc[db] = mfma32(lds_frag_tr<D, typename C::L>(V, 16 * st, 32 * db), pf, oacc[db]);
      }
    }
    if (more) {
      wait_vm_loads();
    }
    __syncthreads();
  };

  // tiles with every key below the block's first query need no mask
  const int t_diag = min(q0 / kBN, ntiles);
  int t = 0;
  for (; t < t_diag; ++t) tile(t, std::false_type{});
  for (; t < ntiles; ++t) tile(t, std::true_type{});

  const float l_tot = l_run + xor32(l_run);
  store_out_rows<D>(A.o, b, h, i, T, oacc, 1.f / l_tot);
  if (hl == 0 && i < T) A.lse[((int64_t)b * A.H + h) * T + i] = (m_run + fast_log2(l_tot)) * kLn2;
}

// ---------------------------------------------------------------------------
// Frozen head program (h, query block, batch group):
// W[i][j] = exp(a[j] + r[i-j] - log N(i)), rebuilt per tile.
// ---------------------------------------------------------------------------
// NG: batch elements this program covers (the group size, or 1 for a
// final group of one, which would otherwise repeat its element).
template <int D, int NG>
__device__ __forceinline__ void fwd_frozen(const FwdArgs& A, int hidx, int grp, int qb, lds_bf16* smem) {
  using C = FwdCfg<D>;
  constexpr int G = NG;      // batch elements computed
  constexpr int GL = C::G;   // batch slots of the LDS layout

  const int l = lane_id(), w = wave_id(), hl = l >> 5;
  const int T = A.T;
  const int q0 = qb * kBM;
  const int i = q0 + 32 * w + (l & 31);
  const int wq_hi = q0 + 32 * w + 31;
  const int b0 = grp * GL;  // groups are GL batch elements apart
  const int nb = min(G, A.B - b0);

  // LDS: V tiles [buf][gb], then per buffer a2[kBN] and 2 shifted copies of
  // the r band (copy c holds band[y + c] at y), so that each lane reads the
  // four offsets of four consecutive keys with two aligned 8-byte reads.
  lds_f32* fbase = (lds_f32*)(smem + 2 * GL * C::TILE);
  constexpr int FSTRIDE = C::FSTRIDE;

  const int h = A.frz_heads[hidx];
  const float* arow = A.a + (int64_t)h * A.prior_len;
  const float* rrow = A.r + (int64_t)h * A.prior_len;
  // log N(i) in log2 units: merge the key-group partials of this row, and
  // record it as the row's lse for every batch element of the group.
  float z2 = 0.f;
  if (i < T && A.logz) {
    z2 = A.logz[(int64_t)h * T + i] * kLog2e;  // the caller's precomputed log N
    if (hl == 0)
      for (int gb = 0; gb < nb; ++gb) A.lse[((int64_t)(b0 + gb) * A.H + h) * T + i] = A.logz[(int64_t)h * T + i];
  } else if (i < T) {
    float M = kNegInf, S = 0.f;
    const float2* part = A.lz_part + (int64_t)hidx * A.lz_ngroups * T + i;
    const int cmax = i / A.lz_group;  // groups 0..cmax hold this row's terms
    for (int c0 = 0; c0 <= cmax; c0 += 8) {
      float2 p[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) p[u] = part[(int64_t)min(c0 + u, cmax) * T];  // eight loads in flight
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (c0 + u <= cmax && p[u].y > 0.f) {
          const float Mn = fmaxf(M, p[u].x);
          S = S * fast_exp2(M - Mn) + p[u].y * fast_exp2(p[u].x - Mn);
          M = Mn;
        }
      }
    }
    z2 = M + fast_log2(S);
    if (hl == 0)
      for (int gb = 0; gb < nb; ++gb) A.lse[((int64_t)(b0 + gb) * A.H + h) * T + i] = z2 * kLn2;
  }

  const int last_key = min(q0 + kBM, T) - 1;
  const int ntiles = last_key / kBN + 1;

  // Factored weights: W[i][j] = ea[j] er[i-j] f_i with ea = 2^(a2[j] - ca),
  // er = 2^(r2[d] - cr) (both <= 1; ca, cr the maxima over the block's keys
  // and offsets) and f_i = 2^(ca + cr - z2_i), which scales the output row:
  // one multiply per weight instead of an exponential.  Every row of the
  // block must have f_i <= 2^90 (terms that underflow are then below 2^-36
  // of their row); otherwise (a and r whose ranges are far apart) the block
  // takes the exponential per weight.
  // (offsets 0 .. last_key are the block's; eight strides of loads are
  // issued before any is awaited, at addresses clamped to last_key, which
  // leaves the maxima unchanged)
  float ca = kNegInf, cr = kNegInf;
  for (int x0 = threadIdx.x; x0 <= last_key; x0 += 8 * kThreads) {
    float av[8], rv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int x = min(x0 + u * kThreads, last_key);
      av[u] = arow[x];
      rv[u] = rrow[x];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      ca = fmaxf(ca, av[u]);
      cr = fmaxf(cr, rv[u]);
    }
  }
  ca = block_max(ca, fbase) * kLog2e;
  cr = block_max(cr, fbase) * kLog2e;
  const bool exact = __syncthreads_or(i < T && !(ca + cr - z2 <= 90.f));

  // Next-tile operands, loaded into registers at the start of a tile and
  // written to LDS at its end: the V tiles of the group, a (log2 units) of
  // the tile keys (-inf for keys >= T) and the r band over the offsets of the
  // tile, band[x] = r2[q0 - j0 - (BN-1) + x] (factored: ea and er).
  TileDma<D, kBN, true, typename C::L> vdma;
  vdma.init(A.v.st);
  ScalarStage av;
  BandStage<C::BAND, kThreads, 2> band;
  auto load_next = [&](int j0, int buf) {
#pragma unroll
    for (int gb = 0; gb < G; ++gb) {
      const int b = b0 + (gb < nb ? gb : 0);
      const __bf16* vg = (const __bf16*)A.v.ptr + (int64_t)b * A.v.sb + (int64_t)(h / A.kv_group) * A.v.sh;
      vdma.issue(vg, A.v.st, j0, T, smem + (buf * GL + gb) * C::TILE);
    }
    av.load(arow, j0, T);
    band.load(rrow, q0 - j0 - (kBN - 1), T);
  };
  auto store_next = [&](int buf) {
    lds_f32* as = fbase + buf * FSTRIDE;
    if (exact) {
      if (threadIdx.x < kBN) as[threadIdx.x] = av.valid ? av.v * kLog2e : kNegInf;
      band.store(as + kBN);
    } else {
      if (threadIdx.x < kBN) as[threadIdx.x] = av.valid ? fast_exp2(av.v * kLog2e - ca) : 0.f;
      band.store_exp(as + kBN, cr);
    }
    wait_vm_loads();
  };

  load_next(0, 0);
  store_next(0);
  __syncthreads();

  f32x16 oacc[G][C::NDB];
#pragma unroll
  for (int gb = 0; gb < G; ++gb)
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) oacc[gb][db] = f32x16{};

  auto tiles = [&](auto exact_tag) {
  constexpr bool EXACT = decltype(exact_tag)::value;
  for (int t = 0; t < ntiles; ++t) {
    const int j0 = t * kBN;
    const bool more = (t + 1) < ntiles;
    if (more) load_next(j0 + kBN, (t & 1) ^ 1);
    const int buf = t & 1;
    const lds_f32* as = fbase + buf * FSTRIDE;
    const lds_f32* rs = as + kBN;
    if (j0 <= wq_hi) {
      // band index of (i, j): (i - q0) - (j - j0) + BN - 1.  For four keys
      // base..base+3 (base a multiple of 4) the offsets are y0+3..y0 with
      // y0 = xi - base - 3, and y0 mod 2 = (xi + 1) mod 2 is fixed per lane.
      const int xi = (i - q0) + kBN - 1;
      const int cpy = (xi + 1) & 1;
      const lds_f32* rc = rs + cpy * C::BSTRIDE - cpy;  // rc[y] = band[y] for even-aligned reads
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        float wv[8];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int base = 16 * st + 8 * hh + 4 * hl;
          const f32x4 a4 = lds_read_f4(as + base);
          const lds_f32* rp = rc + (xi - base - 3);  // band[y0 .. y0+3]
          typedef __attribute__((ext_vector_type(2))) float f32x2;
          const f32x2 rlo = *(const __attribute__((address_space(3))) f32x2*)rp;
          const f32x2 rhi = *(const __attribute__((address_space(3))) f32x2*)(rp + 2);
          const f32x4 r4 = {rlo[0], rlo[1], rhi[0], rhi[1]};
#pragma unroll
          for (int k = 0; k < 4; ++k)
            wv[4 * hh + k] = EXACT ? fast_exp2(a4[k] + r4[3 - k] - z2) : a4[k] * r4[3 - k];
        }
        const bf16x8 wf = pack_bf16x8(wv[0], wv[1], wv[2], wv[3], wv[4], wv[5], wv[6], wv[7]);
#pragma unroll
        for (int gb = 0; gb < G; ++gb)
#pragma unroll
          for (int db = 0; db < C::NDB; ++db)
            oacc[gb][db] = mfma32(lds_frag_tr<D, typename C::L>(smem + (buf * GL + gb) * C::TILE, 16 * st, 32 * db),
                                  wf, oacc[gb][db]);
      }
    }
    if (more) store_next(buf ^ 1);
    __syncthreads();
  }
  };
  if (exact) tiles(std::true_type{});
  else tiles(std::false_type{});

  const float f_i = exact ? 1.f : fast_exp2(ca + cr - z2);
#pragma unroll
  for (int gb = 0; gb < G; ++gb)
    if (gb < nb) store_out_rows<D>(A.o, b0 + gb, h, i, T, oacc[gb], f_i);
}

// One launch for every head: program p -> (query block rank, slot); each
// query block rank holds B * n_ord ordinary and n_frz * n_groups frozen
// programs, and ranks run longest query blocks first.  The head-state flag
// (which list the slot falls in) selects the program body.
template <int D>
__global__ __launch_bounds__(kThreads, (D == 64 ? 4 : 1)) void fwd_kernel(FwdArgs A) {
  SAF_DYN_LDS(smem);
  const int n_ord_prog = A.B * A.n_ord;
  const int per_q = n_ord_prog + A.n_frz * A.n_groups;
  const int qrank = blockIdx.x / per_q;
  const int rem = blockIdx.x - qrank * per_q;
  const int qb = A.nqb - 1 - qrank;
  if (rem < n_ord_prog) {
    const int b = rem / A.n_ord;
    fwd_ordinary<D>(A, b, A.ord_heads[rem - b * A.n_ord], qb, smem);
  } else {
    const int f = rem - n_ord_prog;
    const int hidx = f / A.n_groups, grp = f % A.n_groups;
    if (A.B - grp * FwdCfg<D>::G >= FwdCfg<D>::G) fwd_frozen<D, FwdCfg<D>::G>(A, hidx, grp, qb, smem);
    else fwd_frozen<D, 1>(A, hidx, grp, qb, smem);
  }
}

template <int D>
hipError_t launch_fwd_d(FwdArgs args, hipStream_t stream) {
  using C = FwdCfg<D>;
  constexpr size_t lds = C::ord_lds > C::frz_lds ? C::ord_lds : C::frz_lds;
  static_assert(lds <= 160 * 1024, "LDS budget");
  const hipError_t attr = ensure_dynamic_lds<fwd_kernel<D>>(lds);
  if (attr != hipSuccess) return attr;
  args.frz_group = C::G;
  args.n_groups = (args.B + C::G - 1) / C::G;
  args.nqb = (args.T + kBM - 1) / kBM;
  const int64_t grid = (int64_t)(args.B * args.n_ord + args.n_frz * args.n_groups) * args.nqb;
  if (grid <= 0) return hipSuccess;
  // only the program kinds present need room (less LDS, more blocks per CU)
  const size_t need = args.n_frz > 0 ? (args.n_ord > 0 ? lds : C::frz_lds) : C::ord_lds;
  hipLaunchKernelGGL(fwd_kernel<D>, dim3((unsigned)grid), dim3(kThreads), need, stream, args);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& args, int D, hipStream_t stream) {
  switch (D) {
    case 64: return launch_fwd_d<64>(args, stream);
    case 96: return launch_fwd_d<96>(args, stream);
    case 128: return launch_fwd_d<128>(args, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace saf
