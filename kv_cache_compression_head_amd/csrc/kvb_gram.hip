// Gram-based Soft-Riesz kernels: key norms, fused pairwise-interaction row
// sums (disturbance and density fix-ups) and the ordered crossing scan.
//
// DensityKV paper-summary page, Method ("Soft-Riesz Density", "Online
// Density-Constrained Bank Update") and appendix B.1: the interaction of two
// post-RoPE keys is a softened inverse power of their squared distance; the
// exact update touches bank x candidate pairs, admitted x evicted pairs and
// admitted x admitted pairs.  Squared distances come from bf16 MFMA dot
// products: |a - b|^2 = |a|^2 + |b|^2 - 2 a.b with fp32 accumulation.
#include "kvb_common.hpp"
#include "kvb_launch.hpp"

namespace kvb {

// ---------------------------------------------------------------------------
// squared norms: one group of CPR lanes per row, 16-byte chunks
// ---------------------------------------------------------------------------
template <typename E, int CPR>
__global__ __launch_bounds__(256) void norms_kernel(const E* __restrict__ keys, int64_t nrows, int d,
                                                    float scale, float* __restrict__ out) {
  constexpr int EPC = 16 / sizeof(E);
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / CPR;
  const int c = (int)(gid % CPR);
  float s = 0.0f;
  if (row < nrows) {
    const E* p = keys + row * d + c * EPC;
    const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(p);
    const E* e = reinterpret_cast<const E*>(&raw);
#pragma unroll
    for (int j = 0; j < EPC; ++j) {
      float x = Ops<E>::to_f32(e[j]);
      s = __builtin_fmaf(x, x, s);
    }
  }
#pragma unroll
  for (int o = CPR / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  if (row < nrows && c == 0) out[row] = s * scale;
}

hipError_t launch_norms(const void* keys, int et, int H, int rows, int d, float scale, float* out,
                        hipStream_t st) {
  const int64_t nrows = (int64_t)H * rows;
  if (nrows == 0) return hipSuccess;
  const int esz = et == ET_BF16 ? 2 : 4;
  const int cpr = d * esz / 16;
  const int64_t threads = nrows * cpr;
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (et == ET_BF16) {
    if (cpr == 8) hipLaunchKernelGGL((norms_kernel<uint16_t, 8>), grid, dim3(256), 0, st, (const uint16_t*)keys, nrows, d, scale, out);
    else hipLaunchKernelGGL((norms_kernel<uint16_t, 16>), grid, dim3(256), 0, st, (const uint16_t*)keys, nrows, d, scale, out);
  } else {
    if (cpr == 16) hipLaunchKernelGGL((norms_kernel<float, 16>), grid, dim3(256), 0, st, (const float*)keys, nrows, d, scale, out);
    else hipLaunchKernelGGL((norms_kernel<float, 32>), grid, dim3(256), 0, st, (const float*)keys, nrows, d, scale, out);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// tile staging: TR key rows of D elements gathered by virtual index into LDS
// (row stride LDR elements), 16-byte chunks, 256 threads.
// ---------------------------------------------------------------------------
template <typename E, int D, int TR>
struct TileLoader {
  static constexpr int EPC = 16 / sizeof(E);     // elements per chunk
  static constexpr int CPR = D / EPC;            // chunks per row
  static constexpr int RPP = 256 / CPR;          // rows per pass
  static constexpr int PASSES = TR / RPP;
  static_assert(TR % RPP == 0, "tile rows");
  u32x4_t reg[PASSES];

  // v_of(r) returns the virtual row index of tile row r or -1 (zero fill)
  template <typename KS, typename F>
  KVB_DEV void load(const KS& ks, int h, F v_of) {
    const int t = threadIdx.x;
    const int c = t % CPR;
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
      const int r = t / CPR + i * RPP;
      const int v = v_of(r);
      if (v >= 0) reg[i] = *reinterpret_cast<const u32x4_t*>(ks.row(h, v) + c * EPC);
      else reg[i] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  template <int LDR>
  KVB_DEV void store(E* lds) const {
    const int t = threadIdx.x;
    const int c = t % CPR;
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
      const int r = t / CPR + i * RPP;
      *reinterpret_cast<u32x4_t*>(lds + r * LDR + c * EPC) = reg[i];
    }
  }
};

// ---------------------------------------------------------------------------
// gram row sums.  Work-group: 4 waves x 16 rows; column tiles of 64 staged
// through LDS (double buffered).  A operand = column keys (LDS), B operand =
// the wave's 16 row keys (registers).  Lane accumulates phi for its row
// (lane & 15) over columns 4*(lane>>4)+i of each 16-column subtile.
// ---------------------------------------------------------------------------
template <typename E, int D, int MODE, bool SELF>
__global__ __launch_bounds__(256) void gram_kernel(KeySpace<E> ks, VList rows, VList cols, float* __restrict__ out,
                                                   int64_t out_hstride, int64_t split_stride, PhiConst pc,
                                                   uint64_t active) {
  using O = Ops<E>;
  constexpr int LDR = D + O::PAD;
  constexpr int TC = 64;
  constexpr int NK = D / O::K16;
  __shared__ __attribute__((aligned(16))) E sY[2][TC * LDR];
  __shared__ float sYn[2][TC];
  __shared__ int sYv[2][TC];

  const int h = blockIdx.y;
  if (!head_on(active, h)) return;
  const int nrows = vlist_count(rows, h);
  const int r0 = blockIdx.x * 64;
  if (r0 >= nrows) return;
  const int ncols = vlist_count(cols, h);
  const int ntiles = (ncols + TC - 1) / TC;
  const int per = (ntiles + (int)gridDim.z - 1) / (int)gridDim.z;
  const int t0 = blockIdx.z * per;
  const int t1 = min(ntiles, t0 + per);

  const int lane = lane_id(), w = wave_id();
  const int myrow = r0 + w * 16 + (lane & 15);
  const int rv0 = myrow < nrows ? vlist_at(rows, h, myrow) : -1;
  const bool rvalid = ks.ok(rv0);
  const int rv = rvalid ? rv0 : -1;

  typename O::frag xf[NK];
  {
    const E* xp = rvalid ? ks.row(h, rv) : nullptr;
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      if (rvalid) xf[k] = O::load(xp + O::off16(k, lane));
      else xf[k] = typename O::frag{};
    }
  }
  const float xs = rvalid ? ks.nrm(h, rv) + pc.eps : pc.eps;
  float acc = 0.0f;

  TileLoader<E, D, TC> ld;
  auto vof = [&](int tile) {
    return [&, tile](int r) -> int {
      const int c = tile * TC + r;
      const int v = c < ncols ? vlist_at(cols, h, c) : -1;
      return ks.ok(v) ? v : -1;
    };
  };
  if (t0 < t1) {
    ld.load(ks, h, vof(t0));
    ld.template store<LDR>(sY[0]);
    if (threadIdx.x < TC) {
      const int c = t0 * TC + threadIdx.x;
      int v = c < ncols ? vlist_at(cols, h, c) : -1;
      v = ks.ok(v) ? v : -1;
      sYn[0][threadIdx.x] = v >= 0 ? ks.nrm(h, v) : 0.0f;
      sYv[0][threadIdx.x] = v;
    }
  }
  __syncthreads();
  for (int tile = t0; tile < t1; ++tile) {
    const int cur = (tile - t0) & 1;
    const bool more = tile + 1 < t1;
    float nn = 0.0f;
    int nv = -1;
    if (more) {
      ld.load(ks, h, vof(tile + 1));
      if (threadIdx.x < TC) {
        const int c = (tile + 1) * TC + threadIdx.x;
        nv = c < ncols ? vlist_at(cols, h, c) : -1;
        nv = ks.ok(nv) ? nv : -1;
        nn = nv >= 0 ? ks.nrm(h, nv) : 0.0f;
      }
    }
    const bool full = (tile + 1) * TC <= ncols;
    const E* Y = sY[cur];
#pragma unroll
    for (int s = 0; s < TC / 16; ++s) {
      f32x4_t c = {0.f, 0.f, 0.f, 0.f};
      const E* yp = Y + (16 * s + (lane & 15)) * LDR;
#pragma unroll
      for (int k = 0; k < NK; ++k) c = O::mma16(O::load(yp + O::off16(k, lane)), xf[k], c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int yi = 16 * s + 4 * (lane >> 4) + i;
        float f = phi_pair<MODE>(c[i], xs + sYn[cur][yi], pc);
        if (SELF || !full) {
          const int yv = sYv[cur][yi];
          const bool ok = yv >= 0 && (!SELF || yv != rv);
          f = ok ? f : 0.0f;
        }
        acc += f;
      }
    }
    if (more) {
      ld.template store<LDR>(sY[cur ^ 1]);
      if (threadIdx.x < TC) {
        sYn[cur ^ 1][threadIdx.x] = nn;
        sYv[cur ^ 1][threadIdx.x] = nv;
      }
    }
    __syncthreads();
  }
  acc += __shfl_xor(acc, 16);
  acc += __shfl_xor(acc, 32);
  if (rvalid && (lane >> 4) == 0) out[(int64_t)h * out_hstride + (int64_t)blockIdx.z * split_stride + myrow] = acc;
}

template <typename E, int D, int MODE>
static void gram_dispatch_self(const GramLaunch& g, dim3 grid, hipStream_t st) {
  KeySpace<E> ks{(const E*)g.k.bankK, (const E*)g.k.candK, g.k.bankN, g.k.candN, g.k.M, g.k.N, g.k.d};
  if (g.self_excl)
    hipLaunchKernelGGL((gram_kernel<E, D, MODE, true>), grid, dim3(256), 0, st, ks, g.rows, g.cols, g.out,
                       g.out_hstride, g.split_stride, g.pc, g.active);
  else
    hipLaunchKernelGGL((gram_kernel<E, D, MODE, false>), grid, dim3(256), 0, st, ks, g.rows, g.cols, g.out,
                       g.out_hstride, g.split_stride, g.pc, g.active);
}

template <typename E, int D>
static void gram_dispatch_mode(const GramLaunch& g, dim3 grid, hipStream_t st) {
  switch (g.phi_mode) {
    case PHI_P2: gram_dispatch_self<E, D, PHI_P2>(g, grid, st); break;
    case PHI_P0: gram_dispatch_self<E, D, PHI_P0>(g, grid, st); break;
    case PHI_P1: gram_dispatch_self<E, D, PHI_P1>(g, grid, st); break;
    case PHI_P4: gram_dispatch_self<E, D, PHI_P4>(g, grid, st); break;
    default: gram_dispatch_self<E, D, PHI_GEN>(g, grid, st); break;
  }
}

hipError_t launch_gram(const GramLaunch& g, hipStream_t st) {
  if (g.rows.n <= 0) return hipSuccess;
  const dim3 grid((unsigned)((g.rows.n + 63) / 64), (unsigned)g.k.H, (unsigned)(g.splits > 0 ? g.splits : 1));
  if (g.k.et == ET_BF16) {
    if (g.k.d == 128) gram_dispatch_mode<uint16_t, 128>(g, grid, st);
    else gram_dispatch_mode<uint16_t, 64>(g, grid, st);
  } else {
    if (g.k.d == 128) gram_dispatch_mode<float, 128>(g, grid, st);
    else gram_dispatch_mode<float, 64>(g, grid, st);
  }
  return hipGetLastError();
}

__global__ void sum_splits_kernel(const float* __restrict__ src, int64_t src_hstride, int64_t split_stride,
                                  int splits, float* __restrict__ dst, int64_t dst_hstride, int n) {
  const int h = blockIdx.y;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float s = 0.0f;
  for (int k = 0; k < splits; ++k) s += src[(int64_t)h * src_hstride + k * split_stride + i];
  dst[(int64_t)h * dst_hstride + i] = s;
}

hipError_t launch_sum_splits(const float* src, int64_t src_hstride, int64_t split_stride, int splits, float* dst,
                             int64_t dst_hstride, int H, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(sum_splits_kernel, dim3((n + 255) / 256, H), dim3(256), 0, st, src, src_hstride,
                     split_stride, splits, dst, dst_hstride, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// ordered crossing scan.
//
// For bank state b and prefix length k the projected density is
//   S_b(k) = rho_b + sum_{j<k} phi(b, c_{order[j]}).
// The candidate axis is cut into 32-candidate subtiles; a 32x32 MFMA tile
// (A = candidates, B = bank rows) gives lane l the 16 values of bank row
// (l & 31) for candidates 8q + 4h + r (q = 0..3, h = l >> 5, r = 0..3), i.e.
// eight groups of four in candidate order, alternating between the lane and
// its partner l ^ 32.  The canonical running sum inside a subtile is
//   carry + (E_G + P_G(r)),  E_0 = 0, E_{G+1} = E_G + T_G,
// with T_G and P_G the sequential sums of group G; the carry advances by E_8.
// This value is monotone in k, identical in the scan and the sum pass, and
// its subtile totals are what the checkpoints store.
//
// scan pass: t_b = smallest k with S_b(k) > tau * rho0_b (kmax+1 if none).
// sum pass:  rhoP_b = S_b(k*) starting from the nearest checkpoint.
// ---------------------------------------------------------------------------
template <typename E, int D, int MODE, bool SUM>
__global__ __launch_bounds__(256) void scan_kernel(KeySpace<E> ks, const float* __restrict__ rho,
                                                   const float* __restrict__ rho0, const int32_t* __restrict__ count,
                                                   const int32_t* __restrict__ order, uint64_t active,
                                                   int kmax, float tau, int cps, int ncp, float* __restrict__ cp,
                                                   int32_t* __restrict__ t_out, const int32_t* __restrict__ kstar_p,
                                                   float* __restrict__ rhoP, PhiConst pc) {
  using O = Ops<E>;
  constexpr int LDR = D + O::PAD;
  constexpr int TC = 64;               // candidates per LDS stage (two subtiles)
  constexpr int NK = D / O::K32;
  __shared__ __attribute__((aligned(16))) E sC[2][TC * LDR];
  __shared__ float sCn[2][TC];

  const int h = blockIdx.y;
  if (!head_on(active, h)) return;
  const int M = ks.M;
  const int n = count[h];
  const int b0 = blockIdx.x * 128;
  if (b0 >= n) return;
  const int lane = lane_id(), w = wave_id();
  const int hh = lane >> 5;
  const int b = b0 + w * 32 + (lane & 31);
  const bool valid = b < n;
  const int64_t hb = (int64_t)h * M + b;
  const float r_b = valid ? rho[hb] : 0.0f;
  const bool finite = __builtin_isfinite(tau);
  const float thr = (valid && finite) ? tau * rho0[hb] : __builtin_inff();

  int kst = 0;
  int sub_begin = 0, sub_end = 0;   // subtiles [begin, end)
  float carry = r_b;
  bool done = !valid;
  bool need = false;
  int t_b = kmax + 1;
  if constexpr (SUM) {
    kst = *kstar_p;
    // mandatory rows (t_b <= k*) are evicted; their projected density is unused
    need = valid && kst > 0 && t_out[hb] > kst;
    if (!__syncthreads_or(need)) {
      if (valid) rhoP[hb] = r_b;
      return;
    }
    const int tstar = (kst > 0) ? (kst - 1) / 32 : 0;
    const int c = tstar / cps;
    sub_begin = c * cps;
    sub_end = kst > 0 ? tstar + 1 : 0;
    if (c > 0 && valid) carry = cp[((int64_t)h * ncp + c) * M + b];
    done = !need;
  } else {
    sub_begin = 0;
    sub_end = (kmax + 31) / 32;
    if (valid && finite && r_b > thr) { t_b = 0; done = true; }
  }

  typename O::frag bf[NK];
  {
    const E* bp = ks.bankK + hb * D;
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      if (valid) bf[k] = O::load(bp + O::off32(k, lane));
      else bf[k] = typename O::frag{};
    }
  }
  const float xs = valid ? ks.bankN[hb] + pc.eps : pc.eps;

  // LDS stages hold 64 candidates = subtiles 2*stage, 2*stage + 1
  const int st_begin = sub_begin / 2, st_end = (sub_end + 1) / 2;
  TileLoader<E, D, TC> ld;
  auto vof = [&](int stage) {
    return [&, stage](int r) -> int {
      const int j = stage * TC + r;
      const unsigned c = j < kmax ? (unsigned)order[(int64_t)h * ks.N + j] : 0xFFFFFFFFu;
      return c < (unsigned)ks.N ? M + (int)c : -1;
    };
  };
  if (st_begin < st_end) {
    ld.load(ks, h, vof(st_begin));
    ld.template store<LDR>(sC[0]);
    if (threadIdx.x < TC) {
      const int j = st_begin * TC + threadIdx.x;
      const unsigned c = j < kmax ? (unsigned)order[(int64_t)h * ks.N + j] : 0xFFFFFFFFu;
      sCn[0][threadIdx.x] = c < (unsigned)ks.N ? ks.candN[(int64_t)h * ks.N + c] : 0.0f;
    }
  }
  __syncthreads();
  for (int stg = st_begin; stg < st_end; ++stg) {
    const int cur = (stg - st_begin) & 1;
    const bool more = stg + 1 < st_end;
    float nn = 0.0f;
    if (more) {
      ld.load(ks, h, vof(stg + 1));
      if (threadIdx.x < TC) {
        const int j = (stg + 1) * TC + threadIdx.x;
        const unsigned c = j < kmax ? (unsigned)order[(int64_t)h * ks.N + j] : 0xFFFFFFFFu;
        nn = c < (unsigned)ks.N ? ks.candN[(int64_t)h * ks.N + c] : 0.0f;
      }
    }
    const bool wave_busy = __any(!done);
    if (wave_busy) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int sub = 2 * stg + half;
        if (sub < sub_begin || sub >= sub_end) continue;
        if constexpr (!SUM) {
          if (sub % cps == 0 && sub > 0 && valid) cp[((int64_t)h * ncp + sub / cps) * M + b] = carry;
        }
        f32x16_t acc;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
        const E* cpp = sC[cur] + (32 * half + (lane & 31)) * LDR;
#pragma unroll
        for (int k = 0; k < NK; ++k) acc = O::mma32(O::load(cpp + O::off32(k, lane)), bf[k], acc);
        float v[16];
        const int pos0 = 32 * sub;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int m = 8 * (i >> 2) + 4 * hh + (i & 3);
          const float f = phi_pair<MODE>(acc[i], xs + sCn[cur][32 * half + m], pc);
          v[i] = (pos0 + m < kmax) ? f : 0.0f;
        }
        float T[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) T[q] = ((v[4 * q] + v[4 * q + 1]) + v[4 * q + 2]) + v[4 * q + 3];
        float Tp[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) Tp[q] = __shfl_xor(T[q], 32);
        float Eg[9];
        Eg[0] = 0.0f;
#pragma unroll
        for (int G = 0; G < 8; ++G) {
          const float tg = ((G & 1) == hh) ? T[G >> 1] : Tp[G >> 1];
          Eg[G + 1] = Eg[G] + tg;
        }
        if constexpr (!SUM) {
          if (!done) {
            const float s_end = carry + Eg[8];
            if (s_end > thr) {
              int first = 1 << 30;
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                float P = 0.0f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                  P = (r == 0) ? v[4 * q] : P + v[4 * q + r];
                  const float S = carry + (Eg[2 * q + hh] + P);
                  const int m = 8 * q + 4 * hh + r;
                  if (S > thr && m < first) first = m;
                }
              }
              const int other = __shfl_xor(first, 32);
              first = min(first, other);
              t_b = pos0 + first + 1;
              done = true;
            }
            carry = s_end;
          }
        } else {
          if (sub < sub_end - 1) {
            carry = carry + Eg[8];
          } else {
            const int j = (kst - 1) - pos0;         // element index inside the subtile
            const int q = j >> 3, jh = (j >> 2) & 1, r = j & 3;
            float P = 0.0f;
            float S = 0.0f;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
              float PP = 0.0f;
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) {
                PP = (rr == 0) ? v[4 * qq] : PP + v[4 * qq + rr];
                if (qq == q && rr == r) P = PP;
              }
            }
            S = carry + (Eg[2 * q + jh] + P);
            const float So = __shfl_xor(S, 32);
            carry = (hh == jh) ? S : So;
          }
        }
      }
    }
    if (more) {
      ld.template store<LDR>(sC[cur ^ 1]);
      if (threadIdx.x < TC) sCn[cur ^ 1][threadIdx.x] = nn;
    }
    if constexpr (!SUM) {
      if (!__syncthreads_or(!done)) {
        // every row of the work-group has crossed: later checkpoints are
        // never read (the sum pass skips rows with t_b <= k*)
        break;
      }
    } else {
      __syncthreads();
    }
  }
  if (valid && hh == 0) {
    if constexpr (SUM) rhoP[hb] = need ? carry : r_b;
    else t_out[hb] = t_b;
  }
}

template <typename E, int D, int MODE>
static void scan_dispatch(const ScanLaunch& a, bool sum, dim3 grid, hipStream_t st) {
  KeySpace<E> ks{(const E*)a.k.bankK, (const E*)a.k.candK, a.k.bankN, a.k.candN, a.k.M, a.k.N, a.k.d};
  if (sum)
    hipLaunchKernelGGL((scan_kernel<E, D, MODE, true>), grid, dim3(256), 0, st, ks, a.rho, a.rho0, a.count,
                       a.order, a.active, a.kmax, a.tau, a.cps, a.ncp, a.cp, a.t_out, a.kstar, a.rhoP, a.pc);
  else
    hipLaunchKernelGGL((scan_kernel<E, D, MODE, false>), grid, dim3(256), 0, st, ks, a.rho, a.rho0, a.count,
                       a.order, a.active, a.kmax, a.tau, a.cps, a.ncp, a.cp, a.t_out, a.kstar, a.rhoP, a.pc);
}

template <typename E, int D>
static void scan_dispatch_mode(const ScanLaunch& a, bool sum, dim3 grid, hipStream_t st) {
  switch (a.phi_mode) {
    case PHI_P2: scan_dispatch<E, D, PHI_P2>(a, sum, grid, st); break;
    case PHI_P0: scan_dispatch<E, D, PHI_P0>(a, sum, grid, st); break;
    case PHI_P1: scan_dispatch<E, D, PHI_P1>(a, sum, grid, st); break;
    case PHI_P4: scan_dispatch<E, D, PHI_P4>(a, sum, grid, st); break;
    default: scan_dispatch<E, D, PHI_GEN>(a, sum, grid, st); break;
  }
}

hipError_t launch_scan(const ScanLaunch& a, bool sum, hipStream_t st) {
  if (a.k.M <= 0) return hipSuccess;
  const dim3 grid((unsigned)((a.k.M + 127) / 128), (unsigned)a.k.H);
  if (a.k.et == ET_BF16) {
    if (a.k.d == 128) scan_dispatch_mode<uint16_t, 128>(a, sum, grid, st);
    else scan_dispatch_mode<uint16_t, 64>(a, sum, grid, st);
  } else {
    if (a.k.d == 128) scan_dispatch_mode<float, 128>(a, sum, grid, st);
    else scan_dispatch_mode<float, 64>(a, sum, grid, st);
  }
  return hipGetLastError();
}

}  // namespace kvb
