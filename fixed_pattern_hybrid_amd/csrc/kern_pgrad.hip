// Gradients of the frozen heads' pattern parameters a and r, for the variant
// that keeps training them ("When Can Attention Heads Be Statically
// Defined?", Appendix C.3.2 "Pattern content and trainability"; pattern of
// Section 3.2, Equation 3).
//
// With W the compact pattern, dW_b = dO_b V_b^T, D_b[i] = rowsum(dO_b * O_b)
// and dG_b = W o (dW_b - D_b) (chain rule through the row softmax, its
// normaliser included), a[j] receives the column sums of sum_b dG_b and r[d]
// its diagonal sums (i - j = d).
//
// Kernels (in launch order):
//   pg_delta  : D_b[i] for frozen rows, one thread per row.
//   pg_kv     (bf16) one program per (frozen head, batch group of two, key
//             block of 128, chunk of 512 queries), four waves of 32 keys;
//             query tiles of 64 stream through LDS as in the key-block pass of
//             the backward.  Each lane owns a key: the accumulator of
//             C[query][key] products is seeded with -(D_b0 + D_b1) and
//             collects dO_b V_b^T of both batch elements, so that W (shared by
//             the group) multiplies it once.  Column sums stay in the lane.
//             Diagonal sums: within a 32 x 32 block a cross-lane permute
//             rotates register r of lane t to lane t - m_r, m_r being the
//             block row of register r, after which lane t holds terms of two
//             diagonals only (i - j = -t or 32 - t relative to the block);
//             those sums go into a per-wave LDS array over the chunk's
//             offsets (plain adds, no atomics), summed over the waves in a
//             fixed order at the end.
//   pg_reduce (bf16) sums the partials of the chunks, key blocks and batch
//             groups in a fixed order and writes da, dr (zeros from T to
//             prior_len).
//   pg_f32    (fp32) one thread per output entry, looping over rows.
#include "saf_internal.h"
#include "saf_tile.h"

namespace saf {
namespace {

constexpr int kThreads = 256;
constexpr int kBM = 64;         // queries per tile
constexpr int kBN = kPgradBN;   // keys per program
constexpr int kQC = kPgradQC;   // queries per program (a chunk of the key block's rows)
constexpr int kDiag = kPgradDiag;  // offsets i - j a program can meet: kQC + kBN - 1, padded

template <int D>
struct PgCfg {
  static constexpr int PITCH = LdsLayout<D>::PITCH;
  static constexpr int NKS = D / 16;
  static constexpr int G = kPgradGroup;
  static constexpr int TILE = kBM * PITCH;
  static constexpr int BAND = kBM + kBN;
  static constexpr int BSTRIDE = band_stride(BAND);
  // per buffer: z2[BM], -sum_b D_b [BM], then 4 shifted copies of the r band
  static constexpr int FSTRIDE = 2 * kBM + 4 * BSTRIDE;
  static constexpr size_t lds = size_t(2) * G * TILE * 2 + size_t(2) * FSTRIDE * 4 + size_t(4) * kDiag * 4;
};

// D_b[i] = sum_d dO[b][h][i][d] * O[b][h][i][d] of frozen heads; E is the
// element type.  Grid: n_frz * B * ceil(T / 256) blocks.
template <typename E, int D>
__global__ __launch_bounds__(kThreads) void pg_delta_kernel(PgradArgs A) {
  const int nrb = (A.T + kThreads - 1) / kThreads;
  const int hb = blockIdx.x / nrb;  // hidx * B + b
  const int i = (blockIdx.x - hb * nrb) * kThreads + threadIdx.x;
  if (i >= A.T) return;
  const int hidx = hb / A.B, b = hb - hidx * A.B;
  const int h = A.frz_heads[hidx];
  const E* o = (const E*)A.o.ptr + (int64_t)b * A.o.sb + (int64_t)h * A.o.sh + (int64_t)i * A.o.st;
  const E* g = (const E*)A.dout.ptr + (int64_t)b * A.dout.sb + (int64_t)h * A.dout.sh + (int64_t)i * A.dout.st;
  constexpr int PER = 16 / sizeof(E);  // elements per 16-byte load
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < D / PER; ++c) {
    const u32x4 ov = gload16(o + PER * c), gv = gload16(g + PER * c);
    if constexpr (sizeof(E) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s = fmaf(__builtin_bit_cast(float, gv[e] << 16), __builtin_bit_cast(float, ov[e] << 16), s);
        s = fmaf(__builtin_bit_cast(float, gv[e] & 0xffff0000u), __builtin_bit_cast(float, ov[e] & 0xffff0000u), s);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // copies: the bit cast of a vector element lvalue reads element 0
        const unsigned gu = gv[e], ou = ov[e];
        s = fmaf(__builtin_bit_cast(float, gu), __builtin_bit_cast(float, ou), s);
      }
    }
  }
  A.delta[(int64_t)hb * A.T + i] = s;
}

// Program (frozen head hidx, batch group grp, key block kb, query chunk ch).
// NG: batch elements it covers (the group size, or 1 for a final group of
// one).
template <int D, int NG>
__device__ __forceinline__ void pg_program(const PgradArgs& A, int hidx, int grp, int kb, int ch, lds_bf16* smem) {
  using C = PgCfg<D>;
  constexpr int G = NG;     // batch elements computed
  constexpr int GL = C::G;  // batch slots of the LDS layout
  const int l = lane_id(), w = wave_id(), hl = l >> 5, t = l & 31;
  const int T = A.T;
  const int k0 = kb * kBN;
  const int j = k0 + 32 * w + t;  // this lane's key
  const int wk_lo = k0 + 32 * w;
  const int b0 = grp * GL;
  const int h = A.frz_heads[hidx];
  const float* arow = A.a + (int64_t)h * A.prior_len;
  const float* rrow = A.r + (int64_t)h * A.prior_len;
  const float a2 = (j < T) ? arow[j] * kLog2e : kNegInf;
  const int64_t prog = (((int64_t)hidx * A.n_groups + grp) * A.nkb + kb) * A.nch + ch;

  // V rows of this lane's key, one per batch element, as B operands
  // (col = key, k = d).
  bf16x8 vf[G][C::NKS];
#pragma unroll
  for (int gb = 0; gb < G; ++gb) {
    const __bf16* vg = (const __bf16*)A.v.ptr + (int64_t)(b0 + gb) * A.v.sb + (int64_t)h * A.v.sh;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks)
      vf[gb][ks] = (j < T) ? __builtin_bit_cast(bf16x8, gload16(vg + (int64_t)j * A.v.st + 16 * ks + 8 * hl))
                           : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  }

  // Register r of a 32 x 32 C block holds block row m_r = 8(r/4) + 4hl + r%4.
  // Lane t takes register r from lane (t + m_r) mod 32 of its half-wave: the
  // term of key t + m_r (row m_r), on diagonal m_r - (t + m_r) = -t, or 32 - t
  // when t + m_r wraps past 31.
  int src[16];
  bool nowrap[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = 8 * (r >> 2) + 4 * hl + (r & 3);
    src[r] = (((t + m) & 31) + 32 * hl) * 4;
    nowrap[r] = t + m < 32;
  }

  // LDS: dO tiles [buf][gb]; per buffer z2, -sum D and the band; then one
  // array per wave over the chunk's offsets: entry x is offset
  // ch * QC - (BN - 1) + x.
  lds_f32* fb = (lds_f32*)(smem + 2 * GL * C::TILE);
  lds_f32* diag = fb + 2 * C::FSTRIDE;
  for (int x = threadIdx.x; x < 4 * kDiag; x += kThreads) diag[x] = 0.f;
  lds_f32* mydiag = diag + w * kDiag;

  const int q_start = k0 + ch * kQC;  // < T (the grid skips empty chunks)
  const int q_end = min(q_start + kQC, T);
  const int qt0 = q_start / kBM;
  const int nqt = (q_end + kBM - 1) / kBM;
  const float* lse = A.lse + ((int64_t)b0 * A.H + h) * T;  // log N, the same for every b
  const float* dl = A.delta + ((int64_t)hidx * A.B + b0) * T;

  TileDma<D, kBM, (D == 64)> odma;
  odma.init(A.dout.st);
  ScalarStage zv;
  ScalarStage dlv[G];
  BandStage<C::BAND, kThreads> band;
  auto load_next = [&](int i0, int buf) {
#pragma unroll
    for (int gb = 0; gb < G; ++gb) {
      const __bf16* g = (const __bf16*)A.dout.ptr + (int64_t)(b0 + gb) * A.dout.sb + (int64_t)h * A.dout.sh;
      odma.issue(g, A.dout.st, i0, T, smem + (buf * GL + gb) * C::TILE);
    }
    zv.load(lse, i0, T);
#pragma unroll
    for (int gb = 0; gb < G; ++gb) dlv[gb].load(dl + (int64_t)gb * T, i0, T);
    band.load(rrow, i0 - k0 - (kBN - 1), T);
  };
  auto store_next = [&](int buf) {
    lds_f32* zs = fb + buf * C::FSTRIDE;
    if (threadIdx.x < kBM) {
      float s = 0.f;
#pragma unroll
      for (int gb = 0; gb < G; ++gb) s += dlv[gb].v;
      zs[threadIdx.x] = zv.valid ? zv.v * kLog2e : __builtin_inff();  // rows >= T: W = 0
      zs[kBM + threadIdx.x] = zv.valid ? -s : 0.f;
    }
    band.store(zs + 2 * kBM);
    wait_vm_loads();
  };

  load_next(qt0 * kBM, 0);
  store_next(0);
  __syncthreads();

  float colsum = 0.f;
  for (int qt = qt0; qt < nqt; ++qt) {
    const int i0 = qt * kBM;
    const int bi = (qt - qt0) & 1;
    const bool more = (qt + 1) < nqt;
    if (more) load_next(i0 + kBM, bi ^ 1);
    const lds_f32* zs = fb + bi * C::FSTRIDE;
    const lds_f32* nd = zs + kBM;
    const lds_f32* rs = zs + 2 * kBM;
    if (i0 + kBM - 1 >= wk_lo) {
      // band index of (i, j): (i - i0) - (j - k0) + BN - 1; four consecutive
      // rows base..base+3 read band[base + xj + 0..3] from copy xj mod 4.
      const int xj = (kBN - 1) - (j - k0);
      const int cpy = xj & 3;
      const lds_f32* rc = rs + cpy * C::BSTRIDE - cpy;
      float tot[2], nw[2];  // per block: all rotated terms, the unwrapped ones
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        // acc[query][key] = sum_b (dO_b V_b^T - D_b): C register r holds row
        // 32c + 8(r/4) + 4hl + r%4 of the tile, column = this lane's key.
        f32x16 acc;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 d4 = lds_read_f4(nd + 32 * c + 8 * q4 + 4 * hl);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[4 * q4 + e] = d4[e];
        }
#pragma unroll
        for (int gb = 0; gb < G; ++gb)
#pragma unroll
          for (int ks = 0; ks < C::NKS; ++ks)
            acc = mfma32(lds_frag_nat<D>(smem + (bi * GL + gb) * C::TILE, 32 * c, 16 * ks), vf[gb][ks], acc);
        tot[c] = 0.f;
        nw[c] = 0.f;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int base = 32 * c + 8 * q4 + 4 * hl;  // first of four tile rows
          const f32x4 z4 = lds_read_f4(zs + base);
          const f32x4 r4 = lds_read_f4(rc + base + xj);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * q4 + e;
            const float g = fast_exp2(a2 + r4[e] - z4[e]) * acc[r];  // sum_b dG_b[i][j]
            colsum += g;
            const float x = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src[r], __builtin_bit_cast(int, g)));
            tot[c] += x;
            nw[c] += nowrap[r] ? x : 0.f;
          }
        }
      }
      // Offsets relative to (i0 - jw): -t (block 0 unwrapped), 32 - t (block
      // 0 wrapped, block 1 unwrapped), 64 - t (block 1 wrapped); the two
      // half-waves hold the same offsets for their rows.
      float s0 = nw[0], s1 = (tot[0] - nw[0]) + nw[1], s2 = tot[1] - nw[1];
      s0 += xor32(s0);
      s1 += xor32(s1);
      s2 += xor32(s2);
      if (hl == 0) {
        const int x0 = (i0 - q_start) - 32 * w + (kBN - 1) - t;  // entry of offset i0 - jw - t
        mydiag[x0] += s0;
        mydiag[x0 + 32] += s1;
        mydiag[x0 + 64] += s2;
      }
    }
    if (more) store_next(bi ^ 1);
    __syncthreads();
  }
  // diagonal partials: the four waves summed in a fixed order
  float* drp = A.dr_part + prog * kDiag;
  for (int x = threadIdx.x; x < kDiag; x += kThreads)
    drp[x] = ((diag[x] + diag[kDiag + x]) + diag[2 * kDiag + x]) + diag[3 * kDiag + x];
  // this lane's key column over the chunk: the two half-waves hold different rows
  const float ctot = colsum + xor32(colsum);
  if (hl == 0) A.da_part[prog * kBN + (j - k0)] = ctot;
}

// One launch: program p -> (chunk, key block, frozen head, batch group), the
// chunk index slowest; chunks past a key block's last row exit at once.
template <int D>
__global__ __launch_bounds__(kThreads, 2) void pg_kv_kernel(PgradArgs A) {
  SAF_DYN_LDS(smem);
  const int per_c = A.nkb * A.n_frz * A.n_groups;
  const int ch = blockIdx.x / per_c;
  int f = blockIdx.x - ch * per_c;
  const int kb = f / (A.n_frz * A.n_groups);
  f -= kb * (A.n_frz * A.n_groups);
  const int hidx = f / A.n_groups, grp = f - hidx * A.n_groups;
  if (kb * kBN + ch * kQC >= A.T) return;
  if (A.B - grp * PgCfg<D>::G >= PgCfg<D>::G) pg_program<D, PgCfg<D>::G>(A, hidx, grp, kb, ch, smem);
  else pg_program<D, 1>(A, hidx, grp, kb, ch, smem);
}

// da[h][x], dr[h][x] for x < prior_len: fixed-order sums of the partials of
// the programs that met key x (key block x / BN, every chunk) or offset x
// (chunks whose window [ch QC - (BN - 1), ch QC + QC - 1] holds x, in key
// blocks that reach it: kb <= (T - 1 - x) / BN).  A block covers 32 entries
// of one head with eight threads per entry: thread part p takes the chunks
// ch = p mod 8 (da) and the key blocks kb = p mod 8 (dr, four independent
// running sums so that loads overlap), and the parts are added in order.
constexpr int kRedX = 32;
constexpr int kRedP = kThreads / kRedX;
__global__ __launch_bounds__(kThreads) void pg_reduce_kernel(PgradArgs A) {
  __shared__ float part[2][kRedP][kRedX];
  const int nxb = (A.prior_len + kRedX - 1) / kRedX;
  const int hidx = blockIdx.x / nxb;
  const int xi = threadIdx.x % kRedX, wp = threadIdx.x / kRedX;
  const int x = (blockIdx.x - hidx * nxb) * kRedX + xi;
  const int T = A.T;
  float da = 0.f, dr = 0.f;
  if (x < T) {
    const int kbx = x / kBN;
    const int nch_x = (T - kbx * kBN + kQC - 1) / kQC;
    const int kbmax = (T - 1 - x) / kBN;
    const int ch_lo = x + (kBN - 1) - (kDiag - 1) > 0 ? (x + (kBN - 1) - (kDiag - 1) + kQC - 1) / kQC : 0;
    const int ch_hi = (x + (kBN - 1)) / kQC;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int g = 0; g < A.n_groups; ++g) {
      const int64_t gk = ((int64_t)hidx * A.n_groups + g) * A.nkb;
      for (int ch = wp; ch < nch_x; ch += kRedP) da += A.da_part[((gk + kbx) * A.nch + ch) * kBN + (x - kbx * kBN)];
      int u = 0;
      for (int kb = wp; kb <= kbmax; kb += kRedP, u = (u + 1) & 3) {
        for (int ch = ch_lo; ch <= ch_hi; ++ch)
          if (ch * kQC + kb * kBN < T)  // the chunk exists in this key block
            acc[u] += A.dr_part[((gk + kb) * A.nch + ch) * kDiag + (x - ch * kQC + (kBN - 1))];
      }
    }
    dr = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  }
  part[0][wp][xi] = da;
  part[1][wp][xi] = dr;
  __syncthreads();
  if (wp == 0 && x < A.prior_len) {
    const int h = A.frz_heads[hidx];
    float sa = 0.f, sr = 0.f;
#pragma unroll
    for (int q = 0; q < kRedP; ++q) {
      sa += part[0][q][xi];
      sr += part[1][q][xi];
    }
    A.da[(int64_t)h * A.prior_len + x] = sa;
    A.dr[(int64_t)h * A.prior_len + x] = sr;
  }
}

// fp32: one thread per output entry x of one frozen head; blocks
// [hidx][kind][x-block] with kind 0 = da (column x), 1 = dr (offset x).
template <int D>
__global__ __launch_bounds__(64) void pg_f32_kernel(PgradArgs A) {
  const int nxb = (A.prior_len + 63) / 64;
  const int hk = blockIdx.x / nxb;
  const int x = (blockIdx.x - hk * nxb) * 64 + threadIdx.x;
  const int hidx = hk >> 1, kind = hk & 1;
  if (x >= A.prior_len) return;
  const int h = A.frz_heads[hidx];
  const int T = A.T;
  const float* arow = A.a + (int64_t)h * A.prior_len;
  const float* rrow = A.r + (int64_t)h * A.prior_len;
  float acc = 0.f;
  if (x < T) {
    for (int b = 0; b < A.B; ++b) {
      const float* vb = (const float*)A.v.ptr + (int64_t)b * A.v.sb + (int64_t)h * A.v.sh;
      const float* gb = (const float*)A.dout.ptr + (int64_t)b * A.dout.sb + (int64_t)h * A.dout.sh;
      const float* lse = A.lse + ((int64_t)b * A.H + h) * T;
      const float* dl = A.delta + ((int64_t)hidx * A.B + b) * T;
      for (int i = x; i < T; ++i) {
        const int j = kind == 0 ? x : i - x;
        const float wv = fast_exp2((arow[j] + rrow[i - j] - lse[i]) * kLog2e);
        const float* vr = vb + (int64_t)j * A.v.st;
        const float* gr = gb + (int64_t)i * A.dout.st;
        float dw = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) dw = fmaf(gr[d], vr[d], dw);
        acc = fmaf(wv, dw - dl[i], acc);
      }
    }
  }
  (kind == 0 ? A.da : A.dr)[(int64_t)h * A.prior_len + x] = acc;
}

template <int D>
hipError_t launch_pgrad_bf16_d(PgradArgs args, hipStream_t stream) {
  using C = PgCfg<D>;
  static_assert(C::lds <= 160 * 1024, "LDS budget");
  const hipError_t attr = ensure_dynamic_lds<pg_kv_kernel<D>>(C::lds);
  if (attr != hipSuccess) return attr;
  const int64_t grid = (int64_t)args.nch * args.nkb * args.n_frz * args.n_groups;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(pg_kv_kernel<D>, dim3((unsigned)grid), dim3(kThreads), C::lds, stream, args);
  return hipGetLastError();
}

template <int D>
hipError_t launch_pgrad_f32_d(const PgradArgs& args, hipStream_t stream) {
  const int64_t grid = (int64_t)args.n_frz * 2 * ((args.prior_len + 63) / 64);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(pg_f32_kernel<D>, dim3((unsigned)grid), dim3(64), 0, stream, args);
  return hipGetLastError();
}

template <typename E, int D>
hipError_t launch_delta_d(const PgradArgs& args, hipStream_t stream) {
  const int64_t grid = (int64_t)args.n_frz * args.B * ((args.T + kThreads - 1) / kThreads);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((pg_delta_kernel<E, D>), dim3((unsigned)grid), dim3(kThreads), 0, stream, args);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pgrad_delta(const PgradArgs& args, int dtype_bf16, int D, hipStream_t stream) {
  if (dtype_bf16) {
    switch (D) {
      case 64: return launch_delta_d<__bf16, 64>(args, stream);
      case 96: return launch_delta_d<__bf16, 96>(args, stream);
      case 128: return launch_delta_d<__bf16, 128>(args, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (D) {
    case 16: return launch_delta_d<float, 16>(args, stream);
    case 32: return launch_delta_d<float, 32>(args, stream);
    case 64: return launch_delta_d<float, 64>(args, stream);
    case 96: return launch_delta_d<float, 96>(args, stream);
    case 128: return launch_delta_d<float, 128>(args, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_pgrad_bf16(const PgradArgs& args, int D, hipStream_t stream) {
  switch (D) {
    case 64: return launch_pgrad_bf16_d<64>(args, stream);
    case 96: return launch_pgrad_bf16_d<96>(args, stream);
    case 128: return launch_pgrad_bf16_d<128>(args, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_pgrad_reduce(const PgradArgs& args, hipStream_t stream) {
  const int64_t grid = (int64_t)args.n_frz * ((args.prior_len + kRedX - 1) / kRedX);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(pg_reduce_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, args);
  return hipGetLastError();
}

hipError_t launch_pgrad_f32(const PgradArgs& args, int D, hipStream_t stream) {
  switch (D) {
    case 16: return launch_pgrad_f32_d<16>(args, stream);
    case 32: return launch_pgrad_f32_d<32>(args, stream);
    case 64: return launch_pgrad_f32_d<64>(args, stream);
    case 96: return launch_pgrad_f32_d<96>(args, stream);
    case 128: return launch_pgrad_f32_d<128>(args, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace saf
