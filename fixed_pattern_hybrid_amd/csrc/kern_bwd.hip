// Backward of the SAF hybrid attention layer, bf16, gfx950
// ("When Can Attention Heads Be Statically Defined?", Section 3.3 and
// Appendix D.2).  Two launches: the first walks the key tiles of each
// ordinary query block and writes dQ (plus delta); the second walks the query
// tiles of each 128-key block and writes dV of every head and dK of the
// ordinary heads.  A frozen head contributes only dV = W^T dO.
//
// Ordinary heads follow the chain rule of causal softmax attention
// (Appendix A.1, Equations 5-7) with P recomputed from the saved row
// log-sum-exp:  P = exp(s*QK^T - L), dP = dO V^T,
// dS = P o (dP - delta), delta_i = sum_d dO[i][d] * O[i][d],
// dV = P^T dO, dK = s dS^T Q, dQ = s dS K.
//
// Kernels (in launch order):
//   bwd_q   : one program per (b, h, 128-query block) of ordinary heads; keys
//             in tiles of 64; accumulator dQ^T.  It also computes
//             delta = rowsum(dO * O) for its rows (each lane already holds
//             half of its row of dO) and stores it for the next pass.
//   bwd_kv  : one launch; one program per (b, h, 128-key block) for ordinary
//             heads and per (h, 128-key block, batch group) for frozen heads;
//             queries in tiles of 64.  Accumulators are dV^T and dK^T so that
//             each lane owns one key and the C registers of S feed the
//             products.  Frozen programs also write the +0.0 rows of dQ and
//             dK for their keys.
#include <type_traits>

#include "saf_internal.h"
#include "saf_tile.h"

namespace saf {
namespace {

constexpr int kThreads = 256;
constexpr int kKvBN = kBwdKvBN;  // keys per key-block program
constexpr int kKvBM = 64;        // queries per tile in the key-block pass
constexpr int kQBM = kBwdQBM;    // queries per query-block program
constexpr int kQBN = 64;         // keys per tile in the query-block pass

template <int D>
struct BwdCfg {
  static constexpr int PITCH = LdsLayout<D>::PITCH;
  static constexpr int NDB = D / 32;
  static constexpr int NKS = D / 16;
  static constexpr int G = 2;
  static constexpr int CG = D == 64 ? 2 : 1;  // key-block pass: 32-query halves computed together
  static constexpr int TILE = 64 * PITCH;
  static constexpr int BAND = kKvBM + kKvBN;  // r band of a (query tile, key block)
  // per buffer: z2[kKvBM], then 4 copies of the band, copy c shifted by c
  static constexpr int BSTRIDE = band_stride(BAND);  // distance between band copies
  static constexpr int FSTRIDE = kKvBM + 4 * BSTRIDE;
  // key-block pass, ordinary: Q and dO tiles (double-buffered) + lse2 and delta
  static constexpr size_t kv_ord_lds = size_t(2) * 2 * TILE * 2 + size_t(2) * 2 * kKvBM * 4;
  // key-block pass, frozen: G dO tiles (double-buffered) + z2 and the r band
  static constexpr size_t kv_frz_lds = size_t(2) * G * TILE * 2 + size_t(2) * FSTRIDE * 4;
  static constexpr size_t kv_lds = kv_ord_lds > kv_frz_lds ? kv_ord_lds : kv_frz_lds;
  static constexpr size_t q_lds = size_t(2) * 2 * TILE * 2;
};

template <int D>
__device__ __forceinline__ void store_rows_t(const TensorRef& o, int b, int h, int row, int T,
                                             const f32x16* acc, float mul) {
  if (row >= T) return;
  const int hl = lane_id() >> 5;
  __bf16* p = (__bf16*)o.ptr + (int64_t)b * o.sb + (int64_t)h * o.sh + (int64_t)row * o.st;
#pragma unroll
  for (int db = 0; db < BwdCfg<D>::NDB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = 32 * db + 8 * q4 + 4 * hl;
      bf16x4 v;
      v[0] = (__bf16)(acc[db][4 * q4 + 0] * mul);
      v[1] = (__bf16)(acc[db][4 * q4 + 1] * mul);
      v[2] = (__bf16)(acc[db][4 * q4 + 2] * mul);
      v[3] = (__bf16)(acc[db][4 * q4 + 3] * mul);
      *reinterpret_cast<bf16x4*>(p + d) = v;
    }
}

__device__ __forceinline__ float bf16lo(unsigned u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16hi(unsigned u) { return __builtin_bit_cast(float, u & 0xffff0000u); }

// ---------------------------------------------------------------------------
// Key-block pass, ordinary head (b, h, kb).
// ---------------------------------------------------------------------------
// FUSED (d = 64 only): the program also accumulates dQ = s dS K of its 128
// keys into the fp32 workspace A.dqacc with atomic adds (see bwd_kvq_kernel).
// oi: rank of head h among the ordinary heads (the dqacc slot).
template <int D, bool FUSED = false>
__device__ __forceinline__ void kv_ordinary(const BwdArgs& A, int b, int h, int oi, int kb, lds_bf16* smem) {
  using C = BwdCfg<D>;
  static_assert(!FUSED || D == 64, "the fused dQ programs are built for d = 64");
  const int l = lane_id(), w = wave_id(), hl = l >> 5;
  const int T = A.T;
  const int k0 = kb * kKvBN;
  const int j = k0 + 32 * w + (l & 31);  // this lane's key
  const int wk_lo = k0 + 32 * w;

  const int hs = A.qk_slot[h];  // Q/K/dQ/dK slot of this head
  const int64_t qoff = (int64_t)b * A.q.sb + (int64_t)hs * A.q.sh;
  const int64_t ooff = (int64_t)b * A.dout.sb + (int64_t)h * A.dout.sh;
  const __bf16* qg = (const __bf16*)A.q.ptr + qoff;
  const __bf16* dog = (const __bf16*)A.dout.ptr + ooff;
  const __bf16* kg = (const __bf16*)A.k.ptr + (int64_t)b * A.k.sb + (int64_t)hs * A.k.sh;
  const __bf16* vg = (const __bf16*)A.v.ptr + (int64_t)b * A.v.sb + (int64_t)h * A.v.sh;
  const float* lse = A.lse + ((int64_t)b * A.H + h) * T;
  const float* dl = A.delta + ((int64_t)b * A.H + h) * T;

  // K and V rows of this lane's key as B operands (col = key, k = d).
  bf16x8 kf[C::NKS], vf[C::NKS];
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks) {
    if (j < T) {
      kf[ks] = __builtin_bit_cast(bf16x8, gload16(kg + (int64_t)j * A.k.st + 16 * ks + 8 * hl));
      vf[ks] = __builtin_bit_cast(bf16x8, gload16(vg + (int64_t)j * A.v.st + 16 * ks + 8 * hl));
    } else {
      kf[ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      vf[ks] = kf[ks];
    }
  }

  // LDS: Q[buf] at buf*TILE, dO[buf] at (2+buf)*TILE, then lse2[buf] and
  // -delta[buf] (the negated delta seeds the dP accumulator).
  lds_f32* fb = (lds_f32*)(smem + 4 * C::TILE);

  const int qt0 = k0 / kKvBM;  // < nqt since k0 < T
  const int nqt = (T + kKvBM - 1) / kKvBM;

  // Next-tile operands are requested at the start of a tile (Q and dO copied
  // straight into the idle LDS buffer, lse and delta into registers) and
  // completed at its end.
  TileDma<D, kKvBM, (D == 64)> qdma, odma;
  qdma.init(A.q.st);
  odma.init(A.dout.st);
  ScalarStage lsv, dlv;
  auto load_next = [&](int i0, int buf) {
    qdma.issue(qg, A.q.st, i0, T, smem + buf * C::TILE);
    odma.issue(dog, A.dout.st, i0, T, smem + (2 + buf) * C::TILE);
    lsv.load(lse, i0, T);
    dlv.load(dl, i0, T);
  };
  auto store_next = [&](int buf) {
    if (threadIdx.x < kKvBM) {
      fb[buf * kKvBM + threadIdx.x] = lsv.valid ? lsv.v * kLog2e : __builtin_inff();  // padding: P = 0
      fb[(2 + buf) * kKvBM + threadIdx.x] = dlv.valid ? -dlv.v : 0.f;
    }
    wait_vm_loads();
  };
  // Fused dQ: per query tile, each wave writes its 32 keys' bf16 dS rows
  // (key-major, [128 keys][64 queries], padded) into dS buffer bi; after the
  // tile's barrier, wave w computes the 32x32 block (queries 32*(w&1).., d
  // 32*(w>>1)..) of dS K over the block's 128 keys -- during the next tile,
  // reading buffer bi while that tile writes the other one -- and adds it to
  // dqacc.  The B operands K[128 keys][32 d] of that product stay in
  // registers (kt); they are read once from a staged copy of the key block.
  lds_bf16* dsb = smem + 4 * C::TILE + 2 * (2 * kKvBM) * 2;  // after the float rows
  constexpr int DSB = kKvBN * C::PITCH;                     // elements per dS buffer
  bf16x8 kt[FUSED ? 8 : 1];
  const int qh = w & 1, dbw = w >> 1;
  if constexpr (FUSED) {
    // the key block, staged in dS buffer 1 (first written by the second tile,
    // after a barrier that every wave reaches only once it has read kt)
    TileDma<D, kKvBN, true> kst;
    kst.init(A.k.st);
    kst.issue(kg, A.k.st, k0, T, dsb + DSB);
  }

  load_next(qt0 * kKvBM, 0);
  store_next(0);
  __syncthreads();
  if constexpr (FUSED) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kt[ks] = lds_frag_tr<D>(dsb + DSB, 16 * ks, 32 * dbw);
  }
  // dQ of the query tile at i0p from dS buffer `buf` (fused programs)
  auto dq_tile = [&](int buf, int i0p) {
    f32x16 acc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) acc = mfma32(lds_frag_tr<D>(dsb + buf * DSB, 16 * ks, 32 * qh), kt[ks], acc);
    float* dst = A.dqacc + ((int64_t)(b * A.n_ord + oi) * T) * D + 32 * dbw + (l & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int q = i0p + 32 * qh + 8 * (r >> 2) + 4 * hl + (r & 3);
      if (q < T)
        __hip_atomic_fetch_add(dst + (int64_t)q * D, acc[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };

  f32x16 dva[C::NDB], dka[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    dva[db] = f32x16{};
    dka[db] = f32x16{};
  }
  const float sl2 = A.scale_log2;

  // One query tile.  MASK only for the two tiles that overlap the key
  // block's diagonal (queries k0 .. k0+127); later tiles need no mask.
  auto tile = [&](int qt, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int i0 = qt * kKvBM;
    const int bi = (qt - qt0) & 1;
    const bool more = (qt + 1) < nqt;
    if (more) load_next(i0 + kKvBM, bi ^ 1);
    const lds_bf16* Q = smem + bi * C::TILE;
    const lds_bf16* O = smem + (2 + bi) * C::TILE;
    const lds_f32* ls = fb + bi * kKvBM;
    const lds_f32* nd = fb + (2 + bi) * kKvBM;
    if constexpr (FUSED) {
      if (qt > qt0) dq_tile(bi ^ 1, i0 - kKvBM);
    }
    // this lane's dS row in buffer bi (fused programs)
    lds_bf16* dsrow = dsb + bi * DSB + (32 * w + (l & 31)) * C::PITCH + 4 * hl;
    if (!MASK || i0 + kKvBM - 1 >= wk_lo) {
      // The tile's two 32-query halves are processed together (d = 64) or
      // one after the other (larger d, which halves the live S and dP
      // registers so that two waves fit per SIMD).
      constexpr int CG = C::CG;
#pragma unroll
      for (int c0 = 0; c0 < 2; c0 += CG) {
        // S = Q K^T and dP - delta = dO V^T - delta (accumulator seeded with -delta)
        f32x16 s[CG], dp[CG];
#pragma unroll
        for (int cc = 0; cc < CG; ++cc) {
          const int c = c0 + cc;
          s[cc] = f32x16{};
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 d4 = lds_read_f4(nd + 32 * c + 8 * q4 + 4 * hl);
#pragma unroll
            for (int e = 0; e < 4; ++e) dp[cc][4 * q4 + e] = d4[e];
          }
#pragma unroll
          for (int ks = 0; ks < C::NKS; ++ks) {
            s[cc] = mfma32(lds_frag_nat<D>(Q, 32 * c, 16 * ks), kf[ks], s[cc]);
            dp[cc] = mfma32(lds_frag_nat<D>(O, 32 * c, 16 * ks), vf[ks], dp[cc]);
          }
        }
#pragma unroll
        for (int cc = 0; cc < CG; ++cc)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int ib = 32 * (c0 + cc) + 8 * q4 + 4 * hl;  // first of 4 consecutive tile rows
            const f32x4 l4 = lds_read_f4(ls + ib);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * q4 + e;
              float p = fast_exp2(fmaf(s[cc][r], sl2, -l4[e]));
              if constexpr (MASK) {
                if ((i0 + ib + e) < j) p = 0.f;
              }
              s[cc][r] = p;
              dp[cc][r] = p * dp[cc][r];
            }
          }
        // dV^T += dO^T P ; dK^T += Q^T dS
#pragma unroll
        for (int st = 2 * c0; st < 2 * (c0 + CG); ++st) {
          const bf16x8 pf = pack_acc8(s[(st >> 1) - c0], 8 * (st & 1));
          const bf16x8 sf = pack_acc8(dp[(st >> 1) - c0], 8 * (st & 1));
          if constexpr (FUSED) {
            // queries 16 st + 4 hl + 0..3 and 16 st + 8 + 4 hl + 0..3
            *(lds_u32x2*)(dsrow + 16 * st) = __builtin_bit_cast(u32x4, sf).xy;
            *(lds_u32x2*)(dsrow + 16 * st + 8) = __builtin_bit_cast(u32x4, sf).zw;
          }
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) {
            dva[db] = mfma32(lds_frag_tr<D>(O, 16 * st, 32 * db), pf, dva[db]);
            dka[db] = mfma32(lds_frag_tr<D>(Q, 16 * st, 32 * db), sf, dka[db]);
          }
        }
      }
    }
    if constexpr (FUSED) {
      if (MASK && !(i0 + kKvBM - 1 >= wk_lo)) {
        // no query of this tile sees the wave's keys: their dS rows are 0
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          *(lds_u32x2*)(dsrow + 16 * st) = u32x2{0u, 0u};
          *(lds_u32x2*)(dsrow + 16 * st + 8) = u32x2{0u, 0u};
        }
      }
    }
    if (more) store_next(bi ^ 1);
    __syncthreads();
  };
  const int qt_full = min(qt0 + 2, nqt);
  int qt = qt0;
  for (; qt < qt_full; ++qt) tile(qt, std::true_type{});
  for (; qt < nqt; ++qt) tile(qt, std::false_type{});
  if constexpr (FUSED) dq_tile((nqt - 1 - qt0) & 1, (nqt - 1) * kKvBM);
  store_rows_t<D>(A.dv, b, h, j, T, dva, 1.f);
  store_rows_t<D>(A.dk, b, hs, j, T, dka, A.scale);
}

// ---------------------------------------------------------------------------
// Key-block pass, frozen head (h, kb, batch group): dV = W^T dO.
// ---------------------------------------------------------------------------
// NG: batch elements this program covers (the group size, or 1 for a
// final group of one, which would otherwise repeat its element).
template <int D, int NG>
__device__ __forceinline__ void kv_frozen(const BwdArgs& A, int h, int grp, int kb, lds_bf16* smem) {
  using C = BwdCfg<D>;
  constexpr int G = NG;      // batch elements computed
  constexpr int GL = C::G;   // batch slots of the LDS layout
  const int l = lane_id(), w = wave_id(), hl = l >> 5;
  const int T = A.T;
  const int k0 = kb * kKvBN;
  const int j = k0 + 32 * w + (l & 31);
  const int wk_lo = k0 + 32 * w;
  const int b0 = grp * GL;  // groups are GL batch elements apart
  const int nb = min(G, A.B - b0);

  const float* arow = A.a + (int64_t)h * A.prior_len;
  const float* rrow = A.r + (int64_t)h * A.prior_len;
  const float a2 = (j < T) ? arow[j] * kLog2e : kNegInf;

  // frozen heads have no query/key path: dQ and dK rows are exactly +0.0
  // (a packed layout has no rows for them)
  if (j < T && hl == 0 && !A.qk_packed) {
#pragma unroll
    for (int gb = 0; gb < G; ++gb) {
      if (gb < nb) {
        const int b = b0 + gb;
        __bf16* dq = (__bf16*)A.dq.ptr + (int64_t)b * A.dq.sb + (int64_t)h * A.dq.sh + (int64_t)j * A.dq.st;
        __bf16* dk = (__bf16*)A.dk.ptr + (int64_t)b * A.dk.sb + (int64_t)h * A.dk.sh + (int64_t)j * A.dk.st;
#pragma unroll
        for (int c = 0; c < D / 8; ++c) {
          sstore16(dq + 8 * c, u32x4{0u, 0u, 0u, 0u});
          sstore16(dk + 8 * c, u32x4{0u, 0u, 0u, 0u});
        }
      }
    }
  }
  const float* lse = A.lse + ((int64_t)b0 * A.H + h) * T;  // log N, same for every b

  // LDS: dO tiles [buf][gb], then per buffer z2[kKvBM] (or f[kKvBM]) and 4
  // shifted copies of the r band (copy c holds band[y + c] at y)
  lds_f32* fb = (lds_f32*)(smem + 2 * GL * C::TILE);
  constexpr int FSTRIDE = C::FSTRIDE;

  const int qt0 = k0 / kKvBM;
  const int nqt = (T + kKvBM - 1) / kKvBM;

  // Factored weights, as in the forward: W[i][j] = ea[j] er[i-j] f_i with
  // ea = 2^(a2[j] - ca), er = 2^(r2[d] - cr), f_i = 2^(ca + cr - z2_i), ca
  // and cr the maxima over the block's keys and over the offsets 0 .. T-1-k0
  // it meets.  A tile stages er and f, a weight is er * f (one multiply
  // instead of an exponential) and ea scales the key's dV row at the end.
  // Taken when every row i >= k0 has f_i <= 2^90 and both maxima are finite
  // (terms that then underflow are below 2^-36 of their row); otherwise the
  // program takes the exponential per weight.  Eight strides of loads are
  // issued before any is awaited, at addresses clamped into range (which
  // leaves the maxima and the test unchanged).
  // (d = 96 and 128 keep the exponential: there the factored tiles' extra
  // registers would spill)
  const int last_d = T - 1 - k0;  // offsets 0 .. last_d; rows k0 .. T-1
  bool exact = true;
  float ea = 1.f, cr = 0.f, cacr = 0.f;
  if constexpr (D == 64) {
    float ca = (j < T) ? a2 : kNegInf;
    cr = kNegInf;
    for (int x0 = threadIdx.x; x0 <= last_d; x0 += 8 * kThreads) {
      float rv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) rv[u] = rrow[min(x0 + u * kThreads, last_d)];
#pragma unroll
      for (int u = 0; u < 8; ++u) cr = fmaxf(cr, rv[u]);
    }
    ca = block_max(ca, fb);
    cr = block_max(cr, fb) * kLog2e;
    const float zlo = ca + cr - 90.f;  // every z2_i must be >= zlo
    bool bad = !(ca > kNegInf && cr > kNegInf);
    for (int x0 = threadIdx.x; x0 <= last_d && !bad; x0 += 8 * kThreads) {
      float zv8[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) zv8[u] = lse[k0 + min(x0 + u * kThreads, last_d)];
#pragma unroll
      for (int u = 0; u < 8; ++u) bad |= !(zv8[u] * kLog2e >= zlo);
    }
    exact = __syncthreads_or(bad);
    if (!exact) ea = fast_exp2(a2 - ca);  // 0 for keys >= T (a2 = -inf)
    cacr = ca + cr;
  }

  TileDma<D, kKvBM, (D == 64)> odma;
  odma.init(A.dout.st);
  auto load_do = [&](int i0, int buf) {
#pragma unroll
    for (int gb = 0; gb < G; ++gb) {
      const int b = b0 + (gb < nb ? gb : 0);
      const __bf16* g = (const __bf16*)A.dout.ptr + (int64_t)b * A.dout.sb + (int64_t)h * A.dout.sh;
      odma.issue(g, A.dout.st, i0, T, smem + (buf * GL + gb) * C::TILE);
    }
  };
  // Next-tile operands: dO tiles, z2 = log N (log2 units) of the tile rows,
  // and the r band over offsets [i0 - k0 - (BN-1), i0 + BM - 1 - k0]; loaded
  // into registers at the start of a tile, written to LDS at its end.  Band
  // offsets beyond T-1-k0 (met only by the padding rows of the last tile)
  // count as outside the pattern, so that er stays <= 1 there.
  ScalarStage zv;
  BandStage<C::BAND, kThreads> band;
  auto load_next = [&](int i0, int buf) {
    load_do(i0, buf);
    zv.load(lse, i0, T);
    band.load(rrow, i0 - k0 - (kKvBN - 1), T - k0);
  };
  auto store_next = [&](int buf) {
    lds_f32* zs = fb + buf * FSTRIDE;
    if (D != 64 || exact) {
      if (threadIdx.x < kKvBM) zs[threadIdx.x] = zv.valid ? zv.v * kLog2e : __builtin_inff();
      band.store(zs + kKvBM);
    } else {
      if (threadIdx.x < kKvBM) zs[threadIdx.x] = zv.valid ? fast_exp2(cacr - zv.v * kLog2e) : 0.f;
      band.store_exp(zs + kKvBM, cr);
    }
    wait_vm_loads();
  };

  load_next(qt0 * kKvBM, 0);  // qt0 < nqt since k0 < T
  store_next(0);
  __syncthreads();

  f32x16 dva[G][C::NDB];
#pragma unroll
  for (int gb = 0; gb < G; ++gb)
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) dva[gb][db] = f32x16{};

  auto tiles = [&](auto exact_tag) {
  constexpr bool EXACT = decltype(exact_tag)::value;
  for (int qt = qt0; qt < nqt; ++qt) {
    const int i0 = qt * kKvBM;
    const int bi = (qt - qt0) & 1;
    const bool more = (qt + 1) < nqt;
    if (more) load_next(i0 + kKvBM, bi ^ 1);
    const lds_f32* zs = fb + bi * FSTRIDE;
    const lds_f32* rs = zs + kKvBM;
    if (i0 + kKvBM - 1 >= wk_lo) {
      // band index of (i, j): (i - i0) - (j - k0) + BN - 1.  Four consecutive
      // rows base..base+3 (base a multiple of 4) read band[base + xj + 0..3],
      // and (base + xj) mod 4 = xj mod 4 is fixed per lane.
      const int xj = (kKvBN - 1) - (j - k0);
      const int cpy = xj & 3;
      const lds_f32* rc = rs + cpy * C::BSTRIDE - cpy;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        float wv[8];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int base = 16 * st + 8 * hh + 4 * hl;  // first of four tile rows
          const f32x4 z4 = lds_read_f4(zs + base);
          const f32x4 r4 = lds_read_f4(rc + base + xj);
#pragma unroll
          for (int k = 0; k < 4; ++k) wv[4 * hh + k] = EXACT ? fast_exp2(a2 + r4[k] - z4[k]) : r4[k] * z4[k];
        }
        const bf16x8 wf = pack_bf16x8(wv[0], wv[1], wv[2], wv[3], wv[4], wv[5], wv[6], wv[7]);
#pragma unroll
        for (int gb = 0; gb < G; ++gb)
#pragma unroll
          for (int db = 0; db < C::NDB; ++db)
            dva[gb][db] = mfma32(lds_frag_tr<D>(smem + (bi * GL + gb) * C::TILE, 16 * st, 32 * db),
                                 wf, dva[gb][db]);
      }
    }
    if (more) store_next(bi ^ 1);
    __syncthreads();
  }
  };
  if (exact) tiles(std::true_type{});
  else if constexpr (D == 64) tiles(std::false_type{});
#pragma unroll
  for (int gb = 0; gb < G; ++gb)
    if (gb < nb) store_rows_t<D>(A.dv, b0 + gb, h, j, T, dva[gb], ea);
}

// Key-block pass for every head in one launch: program p -> (key block, slot),
// key block 0 (the most queries) first; the slot's list selects the body.
template <int D>
__global__ __launch_bounds__(kThreads, (D == 64 ? 3 : 2)) void bwd_kv_kernel(BwdArgs A) {
  SAF_DYN_LDS(smem);
  const int n_ord_prog = A.B * A.n_ord;
  const int per_k = n_ord_prog + A.n_frz * A.n_groups;
  const int kb = blockIdx.x / per_k;
  const int rem = blockIdx.x - kb * per_k;
  if (rem < n_ord_prog) {
    const int b = rem / A.n_ord;
    kv_ordinary<D>(A, b, A.ord_heads[rem - b * A.n_ord], rem - b * A.n_ord, kb, smem);
  } else {
    const int f = rem - n_ord_prog;
    const int h = A.frz_heads[f / A.n_groups], grp = f % A.n_groups;
    if (A.B - grp * BwdCfg<D>::G >= BwdCfg<D>::G) kv_frozen<D, BwdCfg<D>::G>(A, h, grp, kb, smem);
    else kv_frozen<D, 1>(A, h, grp, kb, smem);
  }
}

// ---------------------------------------------------------------------------
// Fused-dQ backward (d = 64): one key-block launch computes dV, dK and, with
// fp32 atomic adds into the workspace, dQ; no query-block pass.  Launch
// order: bwd_pre_kernel (delta of the ordinary rows, dqacc := 0), this
// kernel, dq_convert_kernel (dQ = scale * dqacc in bf16).  The atomic adds
// make dQ's rounding depend on their order: results are not bitwise
// reproducible (dK, dV are).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_kvq_kernel(BwdArgs A) {
  SAF_DYN_LDS(smem);
  const int n_ord_prog = A.B * A.n_ord;
  const int per_k = n_ord_prog + A.n_frz * A.n_groups;
  const int kb = blockIdx.x / per_k;
  const int rem = blockIdx.x - kb * per_k;
  if (rem < n_ord_prog) {
    const int b = rem / A.n_ord;
    kv_ordinary<D, true>(A, b, A.ord_heads[rem - b * A.n_ord], rem - b * A.n_ord, kb, smem);
  } else {
    const int f = rem - n_ord_prog;
    const int h = A.frz_heads[f / A.n_groups], grp = f % A.n_groups;
    if (A.B - grp * BwdCfg<D>::G >= BwdCfg<D>::G) kv_frozen<D, BwdCfg<D>::G>(A, h, grp, kb, smem);
    else kv_frozen<D, 1>(A, h, grp, kb, smem);
  }
}

// delta_i = sum_d dO[i][d] O[i][d] of the ordinary rows (four threads per
// row), and the row's dqacc entries set to 0.  Grid: (row blocks of 64,
// B * n_ord).
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(BwdArgs A) {
  const int bo = blockIdx.y;
  const int b = bo / A.n_ord, oi = bo - b * A.n_ord;
  const int h = A.ord_heads[oi];
  const int i = blockIdx.x * 64 + (threadIdx.x >> 2);
  const int t4 = threadIdx.x & 3;
  float dl = 0.f;
  if (i < A.T) {
    const __bf16* og = (const __bf16*)A.o.ptr + (int64_t)b * A.o.sb + (int64_t)h * A.o.sh + (int64_t)i * A.o.st;
    const __bf16* dg = (const __bf16*)A.dout.ptr + (int64_t)b * A.dout.sb + (int64_t)h * A.dout.sh +
                       (int64_t)i * A.dout.st;
#pragma unroll
    for (int c = t4; c < D / 8; c += 4) {
      const bf16x8 ov = __builtin_bit_cast(bf16x8, gload16(og + 8 * c));
      const bf16x8 dv = __builtin_bit_cast(bf16x8, gload16(dg + 8 * c));
#pragma unroll
      for (int e = 0; e < 8; ++e) dl = fmaf((float)dv[e], (float)ov[e], dl);
    }
  }
  dl += __shfl_xor(dl, 1, 64);
  dl += __shfl_xor(dl, 2, 64);
  if (i < A.T) {
    if (t4 == 0) A.delta[((int64_t)b * A.H + h) * A.T + i] = dl;
    float* z = A.dqacc + ((int64_t)bo * A.T + i) * D;
#pragma unroll
    for (int c = t4; c < D / 4; c += 4) sstore16(z + 4 * c, u32x4{0u, 0u, 0u, 0u});
  }
}

// dQ[b][slot][i] = bf16(scale * dqacc[b][oi][i]): eight entries per thread.
// Grid: (row blocks of 256 / (D / 8) rows, B * n_ord).
template <int D>
__global__ __launch_bounds__(kThreads) void dq_convert_kernel(BwdArgs A) {
  constexpr int PER_ROW = D / 8;
  constexpr int ROWS = kThreads / PER_ROW;
  const int bo = blockIdx.y;
  const int b = bo / A.n_ord, oi = bo - b * A.n_ord;
  const int hs = A.qk_slot[A.ord_heads[oi]];
  const int i = blockIdx.x * ROWS + threadIdx.x / PER_ROW;
  const int c = threadIdx.x % PER_ROW;
  if (i >= A.T) return;
  const float* src = A.dqacc + ((int64_t)bo * A.T + i) * D + 8 * c;
  const f32x4 x0 = *(const f32x4*)src, x1 = *(const f32x4*)(src + 4);
  const float sc = A.scale;
  const bf16x8 y = pack_bf16x8(x0[0] * sc, x0[1] * sc, x0[2] * sc, x0[3] * sc, x1[0] * sc, x1[1] * sc,
                               x1[2] * sc, x1[3] * sc);
  __bf16* dst = (__bf16*)A.dq.ptr + (int64_t)b * A.dq.sb + (int64_t)hs * A.dq.sh + (int64_t)i * A.dq.st + 8 * c;
  sstore16(dst, __builtin_bit_cast(u32x4, y));
}

// ---------------------------------------------------------------------------
// Query-block pass, ordinary head (b, h, qb): dQ = s dS K.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads, (D == 64 ? 3 : 1)) void bwd_q_kernel(BwdArgs A) {
  using C = BwdCfg<D>;
  SAF_DYN_LDS(smem);
  const int per_q = A.B * A.n_ord;
  const int qrank = blockIdx.x / per_q;
  const int rem = blockIdx.x - qrank * per_q;
  const int qb = A.nqb - 1 - qrank;
  const int b = rem / A.n_ord;
  const int h = A.ord_heads[rem - b * A.n_ord];

  const int l = lane_id(), w = wave_id(), hl = l >> 5;
  const int T = A.T;
  const int q0 = qb * kQBM;
  const int i = q0 + 32 * w + (l & 31);
  const int wq_lo = q0 + 32 * w, wq_hi = wq_lo + 31;

  const int hs = A.qk_slot[h];  // Q/K/dQ/dK slot of this head
  const __bf16* qg = (const __bf16*)A.q.ptr + (int64_t)b * A.q.sb + (int64_t)hs * A.q.sh;
  const __bf16* dog = (const __bf16*)A.dout.ptr + (int64_t)b * A.dout.sb + (int64_t)h * A.dout.sh;
  const __bf16* kg = (const __bf16*)A.k.ptr + (int64_t)b * A.k.sb + (int64_t)hs * A.k.sh;
  const __bf16* vg = (const __bf16*)A.v.ptr + (int64_t)b * A.v.sb + (int64_t)h * A.v.sh;

  bf16x8 qf[C::NKS], of[C::NKS];
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks) {
    if (i < T) {
      qf[ks] = __builtin_bit_cast(bf16x8, gload16(qg + (int64_t)i * A.q.st + 16 * ks + 8 * hl));
      of[ks] = __builtin_bit_cast(bf16x8, gload16(dog + (int64_t)i * A.dout.st + 16 * ks + 8 * hl));
    } else {
      qf[ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      of[ks] = qf[ks];
    }
  }
  // delta_i = sum_d dO[i][d] O[i][d]: this lane holds half of the row (the
  // other half is in lane l ^ 32); stored for the key-block pass.
  const int64_t rowv = ((int64_t)b * A.H + h) * T + i;
  const float l2 = (i < T) ? A.lse[rowv] * kLog2e : __builtin_inff();
  float dl = 0.f;
  if (i < T) {
    const __bf16* og = (const __bf16*)A.o.ptr + (int64_t)b * A.o.sb + (int64_t)h * A.o.sh + (int64_t)i * A.o.st;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      const bf16x8 ov = __builtin_bit_cast(bf16x8, gload16(og + 16 * ks + 8 * hl));
#pragma unroll
      for (int e = 0; e < 8; ++e) dl = fmaf((float)of[ks][e], (float)ov[e], dl);
    }
  }
  dl += xor32(dl);
  if (hl == 0 && i < T) A.delta[rowv] = dl;

  const int last_key = min(q0 + kQBM, T) - 1;
  const int ntiles = last_key / kQBN + 1;

  // K and V tiles are copied straight into the idle LDS buffer at the start
  // of the previous tile.
  TileDma<D, kQBN> kdma, vdma;
  kdma.init(A.k.st);
  vdma.init(A.v.st);
  kdma.issue(kg, A.k.st, 0, T, smem);
  vdma.issue(vg, A.v.st, 0, T, smem + 2 * C::TILE);
  wait_vm_loads();
  __syncthreads();

  f32x16 dqa[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) dqa[db] = f32x16{};
  const float sl2 = A.scale_log2;
  // d = 64: the tile's two 32-key halves are computed in sequence, which
  // leaves room for -delta in 16 registers, the C operand of each half's
  // first dP product, so that the accumulator arrives as dP - delta (one
  // subtraction fewer per score).  Larger d computes both halves at once
  // and subtracts delta in the softmax step (a seed would spill there).
  constexpr bool SEQ = D == 64;
  f32x16 ndl;
#pragma unroll
  for (int r = 0; r < 16; ++r) ndl[r] = -dl;

  // One key tile.  MASK only for the tiles that reach the diagonal.
  auto tile = [&](int t, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int j0 = t * kQBN;
    const bool more = (t + 1) < ntiles;
    if (more) {
      kdma.issue(kg, A.k.st, j0 + kQBN, T, smem + ((t + 1) & 1) * C::TILE);
      vdma.issue(vg, A.v.st, j0 + kQBN, T, smem + (2 + ((t + 1) & 1)) * C::TILE);
    }
    const lds_bf16* K = smem + (t & 1) * C::TILE;
    const lds_bf16* V = smem + (2 + (t & 1)) * C::TILE;
    const bool live = !MASK || j0 <= wq_hi;
    if constexpr (SEQ) {
      if (live) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          f32x16 s = f32x16{}, dp = ndl;
#pragma unroll
          for (int ks = 0; ks < C::NKS; ++ks) {
            s = mfma32(lds_frag_nat<D>(K, 32 * c, 16 * ks), qf[ks], s);
            dp = mfma32(lds_frag_nat<D>(V, 32 * c, 16 * ks), of[ks], dp);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float p = fast_exp2(fmaf(s[r], sl2, -l2));
            if constexpr (MASK) {
              const int jj = j0 + 32 * c + 8 * (r >> 2) + 4 * hl + (r & 3);
              if (jj > i) p = 0.f;
            }
            dp[r] = p * dp[r];
          }
          // dQ^T += K^T dS^T over this half's 32 keys
#pragma unroll
          for (int st = 2 * c; st < 2 * c + 2; ++st) {
            const bf16x8 sf = pack_acc8(dp, 8 * (st & 1));
#pragma unroll
            for (int db = 0; db < C::NDB; ++db)
              dqa[db] = mfma32(lds_frag_tr<D>(K, 16 * st, 32 * db), sf, dqa[db]);
          }
        }
      }
    } else if (live) {
      f32x16 s[2], dp[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        s[c] = f32x16{};
        dp[c] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) {
          s[c] = mfma32(lds_frag_nat<D>(K, 32 * c, 16 * ks), qf[ks], s[c]);
          dp[c] = mfma32(lds_frag_nat<D>(V, 32 * c, 16 * ks), of[ks], dp[c]);
        }
      }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(fmaf(s[c][r], sl2, -l2));
          if constexpr (MASK) {
            const int jj = j0 + 32 * c + 8 * (r >> 2) + 4 * hl + (r & 3);
            if (jj > i) p = 0.f;
          }
          dp[c][r] = p * (dp[c][r] - dl);
        }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const bf16x8 sf = pack_acc8(dp[st >> 1], 8 * (st & 1));
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
          dqa[db] = mfma32(lds_frag_tr<D>(K, 16 * st, 32 * db), sf, dqa[db]);
      }
    }
    if (more) {
      wait_vm_loads();
    }
    __syncthreads();
  };
  const int t_diag = min(q0 / kQBN, ntiles);
  int t = 0;
  for (; t < t_diag; ++t) tile(t, std::false_type{});
  for (; t < ntiles; ++t) tile(t, std::true_type{});
  store_rows_t<D>(A.dq, b, hs, i, T, dqa, A.scale);
}


template <int D>
hipError_t launch_kv_d(BwdArgs args, hipStream_t stream) {
  using C = BwdCfg<D>;
  static_assert(C::kv_lds <= 160 * 1024, "LDS budget");
  const hipError_t attr = ensure_dynamic_lds<bwd_kv_kernel<D>>(C::kv_lds);
  if (attr != hipSuccess) return attr;
  args.frz_group = C::G;
  args.n_groups = (args.B + C::G - 1) / C::G;
  args.nkb = (args.T + kKvBN - 1) / kKvBN;
  const int64_t grid = (int64_t)(args.B * args.n_ord + args.n_frz * args.n_groups) * args.nkb;
  if (grid <= 0) return hipSuccess;
  // only the program kinds present need room (less LDS, more blocks per CU)
  const size_t need = args.n_frz > 0 ? (args.n_ord > 0 ? C::kv_lds : C::kv_frz_lds) : C::kv_ord_lds;
  hipLaunchKernelGGL(bwd_kv_kernel<D>, dim3((unsigned)grid), dim3(kThreads), need, stream, args);
  return hipGetLastError();
}

template <int D>
hipError_t launch_q_d(BwdArgs args, hipStream_t stream) {
  using C = BwdCfg<D>;
  args.nqb = (args.T + kQBM - 1) / kQBM;
  const int64_t grid = (int64_t)args.B * args.n_ord * args.nqb;
  if (grid <= 0) return hipSuccess;
  const hipError_t attr = ensure_dynamic_lds<bwd_q_kernel<D>>(C::q_lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(bwd_q_kernel<D>, dim3((unsigned)grid), dim3(kThreads), C::q_lds, stream,
                     args);
  return hipGetLastError();
}

// Fused-dQ sequence (d = 64): pre, key-block programs with dQ, convert.
hipError_t launch_bwd_fused_d64(BwdArgs args, hipStream_t stream, hipEvent_t* ev, int nev, int* next_ev) {
  using C = BwdCfg<64>;
  constexpr size_t lds = C::kv_lds + size_t(2) * kKvBN * C::PITCH * 2;  // + two dS buffers
  static_assert(lds <= 80 * 1024, "two blocks per CU");
  const hipError_t attr = ensure_dynamic_lds<bwd_kvq_kernel<64>>(lds);
  if (attr != hipSuccess) return attr;
  auto mark = [&]() -> hipError_t {
    hipError_t e = hipSuccess;
    if (ev && *next_ev < nev) e = hipEventRecord(ev[*next_ev], stream);
    ++*next_ev;
    return e;
  };
  args.frz_group = C::G;
  args.n_groups = (args.B + C::G - 1) / C::G;
  args.nkb = (args.T + kKvBN - 1) / kKvBN;
  if (args.n_ord > 0) {
    hipLaunchKernelGGL(bwd_pre_kernel<64>, dim3((unsigned)((args.T + 63) / 64), (unsigned)(args.B * args.n_ord)),
                       dim3(kThreads), 0, stream, args);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || (e = mark()) != hipSuccess) return e;
  }
  const int64_t grid = (int64_t)(args.B * args.n_ord + args.n_frz * args.n_groups) * args.nkb;
  hipLaunchKernelGGL(bwd_kvq_kernel<64>, dim3((unsigned)grid), dim3(kThreads), lds, stream, args);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || (e = mark()) != hipSuccess) return e;
  if (args.n_ord > 0) {
    constexpr int rows = kThreads / (64 / 8);
    hipLaunchKernelGGL(dq_convert_kernel<64>, dim3((unsigned)((args.T + rows - 1) / rows), (unsigned)(args.B * args.n_ord)),
                       dim3(kThreads), 0, stream, args);
    e = hipGetLastError();
    if (e != hipSuccess || (e = mark()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_bwd_fused_bf16(const BwdArgs& args, int D, hipStream_t stream, hipEvent_t* ev, int nev,
                                 int* next_ev) {
  if (D != 64) return hipErrorInvalidValue;
  return launch_bwd_fused_d64(args, stream, ev, nev, next_ev);
}

hipError_t launch_bwd_kv_bf16(const BwdArgs& args, int D, hipStream_t stream) {
  switch (D) {
    case 64: return launch_kv_d<64>(args, stream);
    case 96: return launch_kv_d<96>(args, stream);
    case 128: return launch_kv_d<128>(args, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_q_bf16(const BwdArgs& args, int D, hipStream_t stream) {
  switch (D) {
    case 64: return launch_q_d<64>(args, stream);
    case 96: return launch_q_d<96>(args, stream);
    case 128: return launch_q_d<128>(args, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace saf
