// Sequential within-block admission (the KVB_POL_SEQUENTIAL variant).
//
// DensityKV paper-summary page, appendix E (within-block competition):
// candidates are gated one at a time, so every admitted candidate takes part
// in the densities the later candidates are judged against.  Step j offers
// each density head its j-th candidate c in the method's order; the head's
// live states x (bank states and candidates admitted at earlier steps) get
// rho'_x = rho_x + phi(x, c); with e = max(0, n + 1 - M) the step is feasible
// when every head has at most e crossed states (rho'_x > tau rho0_x), as the
// method's prefix is shared by the heads (per head with KVB_POL_HEAD_PREFIX).
// A feasible step admits c everywhere: the crossed state, else the densest
// (ties: lower token id) or the oldest, leaves when e = 1; survivors take
// rho'_x - phi(x, y) for the evicted y; c enters with its density among the
// states left.  Only growth from later blocks counts against a baseline, so
// the block's candidates have none until the block ends (they never cross)
// and then take their density in the bank.  An infeasible step changes
// nothing.
//
// Three kernels:
//   pair_phi_kernel  every head's pairwise interactions over its M + N states
//                    (bank slots, then candidates), from explicit differences
//   seq_walk_kernel  the walk: one wave per head; the layer's heads meet at one
//                    barrier per step for the shared decision
//   seq_gather_kernel  the final live set into the bank: admitted rows fill the
//                    freed slots, then append; values stay with their keys
#include "kvb_common.hpp"
#include "kvb_launch.hpp"

namespace kvb {

// ---------------------------------------------------------------------------
// pair interactions: P[h][x][y] = phi(|X_x - X_y|^2), 16 x 16 pairs per block
// ---------------------------------------------------------------------------
constexpr int PAIR_MAXD = 256;   // widest row: 256-wide descriptors ([K; V] at d = 128)

template <typename E, int MODE>
__global__ __launch_bounds__(256) void pair_phi_kernel(const E* __restrict__ bankX, const E* __restrict__ candX,
                                                       int M, int N, int dx, PhiConst pc, uint64_t active,
                                                       float* __restrict__ P) {
  const int h = blockIdx.z;
  if (!head_on(active, h)) return;
  const int S = M + N;
  const int x0 = blockIdx.y * 16, y0 = blockIdx.x * 16;
  // (odd row stride: the 16 rows of one column fall in 16 different banks)
  __shared__ float sx[16][PAIR_MAXD + 1];
  __shared__ float sy[16][PAIR_MAXD + 1];
  auto row = [&](int v) -> const E* {
    return v < M ? bankX + ((int64_t)h * M + v) * dx : candX + ((int64_t)h * N + (v - M)) * dx;
  };
  for (int i = threadIdx.x; i < 16 * dx; i += 256) {
    const int r = i / dx, k = i % dx;
    sx[r][k] = (x0 + r < S) ? Ops<E>::to_f32(row(x0 + r)[k]) : 0.0f;
    sy[r][k] = (y0 + r < S) ? Ops<E>::to_f32(row(y0 + r)[k]) : 0.0f;
  }
  __syncthreads();
  const int tx = threadIdx.x / 16, ty = threadIdx.x % 16;
  if (x0 + tx >= S || y0 + ty >= S) return;
  float d2 = 0.0f;
  for (int k = 0; k < dx; ++k) {
    const float df = sx[tx][k] - sy[ty][k];
    d2 = __builtin_fmaf(df, df, d2);
  }
  const float t = fmaxf(__builtin_fmaf(d2, pc.inv_s2, pc.eps), pc.eps);
  P[((int64_t)h * S + (x0 + tx)) * S + (y0 + ty)] = phi_of_t<MODE>(t, pc.neg_half_p);
}

// ---------------------------------------------------------------------------
// the walk
// ---------------------------------------------------------------------------
// State arrays are written and read back by the same wave across steps:
// loads and stores at device scope keep them out of the vector L1, so a
// lane always sees what another lane of its wave stored at an earlier step.
KVB_DEV uint64_t ld_rr(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
KVB_DEV void st_rr(uint64_t* p, float rho, float rho0) {
  const uint64_t v = (uint64_t)__float_as_uint(rho) | ((uint64_t)__float_as_uint(rho0) << 32);
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
KVB_DEV int ld_tok(const int32_t* p) {
  return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
KVB_DEV void st_tok(int32_t* p, int v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

// (key, index) maximum over the wave, fixed butterfly (ties: larger index,
// which never decides: keys carry the token id and are unique among live
// states)
KVB_DEV void wave_argmax(uint64_t& k, int& i) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint64_t ko = __shfl_xor(k, o);
    const int io = __shfl_xor(i, o);
    if (ko > k || (ko == k && io > i)) { k = ko; i = io; }
  }
}

constexpr int SEQ_MAXHPW = 4;   // heads per wave (64 heads over 16 waves)

__global__ __launch_bounds__(1024) void seq_walk_kernel(SeqLaunch a) {
  const int lane = lane_id(), w = wave_id();
  const int nw = blockDim.x / 64;
  const int S = a.M + a.N;
  const bool finite = __builtin_isfinite(a.tau);
  __shared__ int s_ok[2][KVB_SEQ_MAX_HEADS];
  // this wave's heads
  int hs[SEQ_MAXHPW];
  int nh = 0;
  if (a.per_head) {
    hs[nh++] = blockIdx.x;
  } else {
    for (int h = w; h < a.H && nh < SEQ_MAXHPW; h += nw) hs[nh++] = h;
  }
  int n_occ[SEQ_MAXHPW], n_adm[SEQ_MAXHPW], n_ev[SEQ_MAXHPW], n_md[SEQ_MAXHPW];
  // initial states: bank slots below the count, candidates not yet live
  for (int q = 0; q < nh; ++q) {
    const int h = hs[q];
    n_occ[q] = head_on(a.active, h) ? a.cnt[h] : 0;
    n_adm[q] = n_ev[q] = n_md[q] = 0;
    if (!head_on(a.active, h)) continue;
    uint64_t* rr = a.st_rr + (int64_t)h * S;
    int32_t* tk = a.st_tok + (int64_t)h * S;
    for (int x = lane; x < S; x += 64) {
      if (x < a.M) {
        const bool live = x < n_occ[q];
        st_rr(rr + x, live ? a.rho[(int64_t)h * a.M + x] : 0.0f, live ? a.rho0[(int64_t)h * a.M + x] : 0.0f);
        st_tok(tk + x, live ? a.bank_tok[(int64_t)h * a.M + x] : -1);
      } else {
        st_rr(rr + x, 0.0f, 0.0f);
        st_tok(tk + x, -1);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  for (int j = 0; j < a.N; ++j) {
    // ---- offer: projected densities, crossings, eviction candidates ----
    bool feas[SEQ_MAXHPW], mand[SEQ_MAXHPW];
    int yv[SEQ_MAXHPW], cx[SEQ_MAXHPW];
    float Sc[SEQ_MAXHPW];
    for (int q = 0; q < nh; ++q) {
      const int h = hs[q];
      feas[q] = true;
      yv[q] = -1;
      cx[q] = -1;
      Sc[q] = 0.0f;
      if (!head_on(a.active, h)) continue;
      const int c = a.order[(int64_t)h * a.N + j];
      if ((unsigned)c >= (unsigned)a.N) continue;
      cx[q] = a.M + c;
      const float* Pc = a.P + ((int64_t)h * S + cx[q]) * S;
      const uint64_t* rr = a.st_rr + (int64_t)h * S;
      const int32_t* tk = a.st_tok + (int64_t)h * S;
      const bool gated = !(a.fill && n_occ[q] + 1 <= a.M);
      const int e = gated ? max(0, n_occ[q] + 1 - a.M) : 0;
      int ncross = 0, cidx = -1, didx = -1, oidx = -1;
      uint64_t dkey = 0, okey = 0;
      float sum = 0.0f;
      for (int x = lane; x < S; x += 64) {
        const int tok = ld_tok(tk + x);
        if (tok < 0) continue;
        const uint64_t v = ld_rr(rr + x);
        const float rho = __uint_as_float((uint32_t)v), rho0 = __uint_as_float((uint32_t)(v >> 32));
        const float p = Pc[x];
        const float proj = rho + p;
        sum += p;
        if (gated && finite && proj > a.tau * rho0) {
          ++ncross;
          cidx = max(cidx, x);
        }
        const uint64_t t = (uint64_t)(0xFFFFFFFFu - (uint32_t)tok);
        const uint64_t dk = ((uint64_t)float_key(proj) << 32) | t;
        if (didx < 0 || dk > dkey) { dkey = dk; didx = x; }
        if (oidx < 0 || t > okey) { okey = t; oidx = x; }
      }
      ncross = wave_sum_i(ncross);
      for (int o = 32; o >= 1; o >>= 1) cidx = max(cidx, __shfl_xor(cidx, o));
      sum = wave_sum(sum);
      wave_argmax(dkey, didx);
      wave_argmax(okey, oidx);
      feas[q] = ncross <= e;
      Sc[q] = sum;
      mand[q] = false;
      if (e > 0) {
        if (a.evict_mode == 1) yv[q] = didx;                          // densest only
        else if (ncross > 0) yv[q] = cidx;                            // the crossed state
        else yv[q] = a.evict_mode == 2 ? oidx : didx;                 // oldest / densest
        mand[q] = ncross > 0 && a.evict_mode != 1;
      }
    }
    bool admit_all = true;
    if (!a.per_head) {
      for (int q = 0; q < nh; ++q)
        if (lane == 0) s_ok[j & 1][hs[q]] = feas[q] ? 1 : 0;
      __syncthreads();
      for (int h = lane; h < a.H; h += 64)
        if (head_on(a.active, h) && !s_ok[j & 1][h]) admit_all = false;
      admit_all = !__any(!admit_all);
    }
    // ---- admit: evict, fix survivors, the candidate's baseline ----
    for (int q = 0; q < nh; ++q) {
      const int h = hs[q];
      if (cx[q] < 0) continue;
      const bool adm = a.per_head ? feas[q] : admit_all;
      if (!adm) continue;
      const int y = yv[q];
      const float* Pc = a.P + ((int64_t)h * S + cx[q]) * S;
      const float* Py = y >= 0 ? a.P + ((int64_t)h * S + y) * S : nullptr;
      uint64_t* rr = a.st_rr + (int64_t)h * S;
      int32_t* tk = a.st_tok + (int64_t)h * S;
      for (int x = lane; x < S; x += 64) {
        const int tok = ld_tok(tk + x);
        if (tok < 0 || x == y) continue;
        const uint64_t v = ld_rr(rr + x);
        const float proj = __uint_as_float((uint32_t)v) + Pc[x];
        const float r = y >= 0 ? proj - Py[x] : proj;
        st_rr(rr + x, r, __uint_as_float((uint32_t)(v >> 32)));
      }
      if (lane == 0) {
        const int c = cx[q] - a.M;
        const float rc = y >= 0 ? Sc[q] - Pc[y] : Sc[q];
        if (y >= 0) st_tok(tk + y, -1);
        // no baseline until the block ends: +inf never crosses
        st_rr(rr + cx[q], rc, __builtin_inff());
        st_tok(tk + cx[q], a.cand_tok[c]);
        a.log[(int64_t)h * a.N + n_adm[q]] = c;
      }
      ++n_adm[q];
      if (y >= 0) {
        ++n_ev[q];
        --n_occ[q];
      }
      if (mand[q]) ++n_md[q];
      ++n_occ[q];
      __builtin_amdgcn_s_waitcnt(0);
    }
  }
  for (int q = 0; q < nh; ++q) {
    const int h = hs[q];
    if (!head_on(a.active, h) || lane != 0) continue;
    a.n_adm[h] = n_adm[q];
    a.n_ev[h] = n_ev[q];
    a.n_mand[h] = n_md[q];
    a.kstar[h * a.kstar_hs] = n_adm[q];
  }
}

// ---------------------------------------------------------------------------
// gather: survivors keep their slots (densities from the walk), admitted
// candidates still live fill the freed slots in ascending order, then append
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void seq_gather_kernel(SeqGather g) {
  const int h = blockIdx.x;
  if (!head_on(g.active, h)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int M = g.M, N = g.N, S = M + N;
  const int n0 = g.cnt[h];
  const int64_t hb = (int64_t)h * M;
  const uint64_t* rr = g.st_rr + (int64_t)h * S;
  const int32_t* tk = g.st_tok + (int64_t)h * S;
  __shared__ int wsum[16];
  __shared__ int s_base;
  // freed slots (ascending) into the free list; survivors' densities
  if (tid == 0) s_base = 0;
  __syncthreads();
  for (int base = 0; base < n0; base += 1024) {
    const int b = base + tid;
    const bool live = b < n0;
    bool dead = false;
    if (live) {
      const int tok = ld_tok(tk + b);
      dead = tok < 0;
      if (!dead) {
        const uint64_t v = ld_rr(rr + b);
        const float rho = __uint_as_float((uint32_t)v);
        g.rho[hb + b] = rho;
        if (g.refresh) g.rho0[hb + b] = rho;
      }
    }
    const uint64_t bal = __ballot(live && dead);
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int pe = __popcll(bal & lt);
    if (lane == 0) wsum[w] = __popcll(bal);
    __syncthreads();
    int off = s_base;
    for (int k = 0; k < w; ++k) off += wsum[k];
    if (live && dead) g.freel[hb + off + pe] = b;
    __syncthreads();
    if (tid == 0) {
      int t = 0;
      for (int k = 0; k < 16; ++k) t += wsum[k];
      s_base += t;
    }
    __syncthreads();
  }
  const int nfree = s_base;
  __syncthreads();
  // admitted candidates still live, in admission order
  const int A = g.n_adm[h];
  if (tid == 0) s_base = 0;
  __syncthreads();
  for (int base = 0; base < A; base += 1024) {
    const int i = base + tid;
    const bool in = i < A;
    int c = -1;
    bool alive = false;
    if (in) {
      c = g.log[(int64_t)h * N + i];
      alive = (unsigned)c < (unsigned)N && ld_tok(tk + M + c) >= 0;
    }
    const uint64_t bal = __ballot(in && alive);
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int pe = __popcll(bal & lt);
    if (lane == 0) wsum[w] = __popcll(bal);
    __syncthreads();
    int off = s_base;
    for (int k = 0; k < w; ++k) off += wsum[k];
    if (in && alive) g.alive[(int64_t)h * N + off + pe] = c;
    __syncthreads();
    if (tid == 0) {
      int t = 0;
      for (int k = 0; k < 16; ++k) t += wsum[k];
      s_base += t;
    }
    __syncthreads();
  }
  const int nalive = s_base;
  // rows: each admitted candidate still live moves K, V (and its descriptor)
  const int esz = g.et == ET_BF16 ? 2 : 4;
  const int cpr = g.d * esz / 16, cprx = g.dx * esz / 16;
  const int per = 2 * cpr + (g.bankX ? cprx : 0);
  for (int u = tid; u < nalive * per; u += 1024) {
    const int jj = u / per, part = u % per;
    const int c = g.alive[(int64_t)h * N + jj];
    const int slot = jj < nfree ? g.freel[hb + jj] : n0 + (jj - nfree);
    if ((unsigned)slot >= (unsigned)M) {
      atomicOr(g.status, DEV_EVICT);
      continue;
    }
    const char* src;
    char* dst;
    int chunk;
    if (part < cpr) {
      src = (const char*)g.candK + ((int64_t)h * N + c) * g.d * esz;
      dst = (char*)g.bankK + (hb + slot) * g.d * esz;
      chunk = part;
    } else if (part < 2 * cpr) {
      src = (const char*)g.candV + ((int64_t)h * N + c) * g.d * esz;
      dst = (char*)g.bankV + (hb + slot) * g.d * esz;
      chunk = part - cpr;
    } else {
      src = (const char*)g.candX + ((int64_t)h * N + c) * g.dx * esz;
      dst = (char*)g.bankX + (hb + slot) * g.dx * esz;
      chunk = part - 2 * cpr;
    }
    *reinterpret_cast<u32x4_t*>(dst + chunk * 16) = *reinterpret_cast<const u32x4_t*>(src + chunk * 16);
    if (part == 0) {
      // the block's candidates take their baselines together: their density
      // in the bank at the end of the walk
      const uint64_t v = ld_rr(rr + M + c);
      g.rho[hb + slot] = __uint_as_float((uint32_t)v);
      g.rho0[hb + slot] = __uint_as_float((uint32_t)v);
      g.bank_tok[hb + slot] = g.cand_tok[c];
    }
  }
  if (tid == 0) {
    const int nn = n0 - nfree + nalive;
    if (nn > M || nalive < nfree) atomicOr(g.status, DEV_EVICT);
    g.count[h] = min(nn, M);
  }
}

hipError_t launch_sequential(const SeqLaunch& a, const SeqGather& g, const void* bankX, const void* candX, int dx,
                             const PhiConst& pc, int phi_mode, hipStream_t st) {
  if (dx < 1 || dx > PAIR_MAXD) return hipErrorInvalidValue;
  const int S = a.M + a.N;
  const dim3 pgrid((unsigned)((S + 15) / 16), (unsigned)((S + 15) / 16), (unsigned)a.H);
#define KVB_PAIR(E, MODE)                                                                                     \
  hipLaunchKernelGGL((pair_phi_kernel<E, MODE>), pgrid, dim3(256), 0, st, (const E*)bankX, (const E*)candX, a.M, \
                     a.N, dx, pc, a.active, a.P)
#define KVB_PAIR_E(E)                                   \
  switch (phi_mode) {                                   \
    case PHI_P2: KVB_PAIR(E, PHI_P2); break;            \
    case PHI_P0: KVB_PAIR(E, PHI_P0); break;            \
    case PHI_P1: KVB_PAIR(E, PHI_P1); break;            \
    case PHI_P4: KVB_PAIR(E, PHI_P4); break;            \
    default: KVB_PAIR(E, PHI_GEN); break;               \
  }
  if (g.et == ET_BF16) {
    KVB_PAIR_E(uint16_t)
  } else {
    KVB_PAIR_E(float)
  }
#undef KVB_PAIR_E
#undef KVB_PAIR
  if (a.per_head)
    hipLaunchKernelGGL(seq_walk_kernel, dim3((unsigned)a.H), dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL(seq_walk_kernel, dim3(1), dim3(64 * (a.H < 16 ? a.H : 16)), 0, st, a);
  hipLaunchKernelGGL(seq_gather_kernel, dim3((unsigned)a.H), dim3(1024), 0, st, g);
  return hipGetLastError();
}

}  // namespace kvb
