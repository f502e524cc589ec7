// Ordering, prefix feasibility, eviction selection, compaction/gather and
// segment tables for the per-head token banks.
//
// DensityKV paper-summary page, Method ("Online Density-Constrained Bank
// Update") and appendix B.1 ("Online Bank Update"): candidates are taken in
// ascending mean-normalised disturbance; one prefix length is shared by the
// heads of a layer and must be admissible for every head; the states that
// cross their growth bound are evicted first, then the densest, until the
// capacity is released; admitted states keep their exact values and set
// their baselines together.  Forcing-KV notes page, sections 3.3-3.5: static
// heads keep [sink, transition frame, chunk]; dynamic heads keep the BottomK
// segments in token order.
#include "kvb_common.hpp"
#include "kvb_launch.hpp"

namespace kvb {

enum : uint32_t { DEV_NONFINITE = 1u, DEV_COUNT = 2u, DEV_SEGOVF = 4u, DEV_EVICT = 8u };

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

// up to four int32 arrays zeroed by one launch
struct ZeroSet {
  int32_t* p[4];
  int64_t n[4];
};
__global__ void zero_i32x4_kernel(ZeroSet z) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (i < z.n[k]) { z.p[k][i] = 0; return; }
    i -= z.n[k];
  }
}

hipError_t launch_zero_i32(int32_t* const* ptrs, const int64_t* lens, int count, hipStream_t st) {
  ZeroSet z{};
  int64_t tot = 0;
  for (int k = 0; k < 4; ++k) {
    z.p[k] = k < count ? ptrs[k] : nullptr;
    z.n[k] = (k < count && ptrs[k]) ? lens[k] : 0;
    tot += z.n[k];
  }
  if (tot <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_i32x4_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st, z);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// mean-normalised disturbance: delta = D / mean_c D (0 if bank empty or mean 0)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void delta_kernel(const float* __restrict__ D, const int32_t* __restrict__ count,
                                                     uint64_t on, int n, float* __restrict__ delta) {
  const int h = blockIdx.x;
  if (!head_on(on, h)) return;
  __shared__ float red[16];
  const float* Dh = D + (int64_t)h * n;
  // fixed-order partial sums: thread i adds elements i, i + 1024, ...
  float s = 0.0f;
  for (int i = threadIdx.x; i < n; i += 1024) s += Dh[i];
  s = wave_sum(s);
  if (lane_id() == 0) red[wave_id()] = s;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) tot += red[k];
  const float mean = tot / (float)n;
  const bool zero = count[h] <= 0 || !(mean > 0.0f);
  for (int i = threadIdx.x; i < n; i += 1024) delta[(int64_t)h * n + i] = zero ? 0.0f : Dh[i] / mean;
}

hipError_t launch_delta(const float* D, const int32_t* count, uint64_t on, int H, int n, float* delta,
                        hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(delta_kernel, dim3(H), dim3(1024), 0, st, D, count, on, n, delta);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// sort: key = float_key(score) << 32 | tie (tie = token id or item index),
// ascending; value = index.  Blocks of 2048 are sorted in LDS (bitonic), then
// sorted runs are merged pairwise by rank (binary search in the other run).
// ---------------------------------------------------------------------------
constexpr int SORT_BS = 2048;

KVB_DEV uint64_t sort_key(const float* score, const int32_t* tie, int64_t tie_hstride, int h, int i,
                          int64_t score_hstride) {
  // no score: the tie key alone (source order, by token id)
  const uint32_t hi = score ? float_key(score[(int64_t)h * score_hstride + i]) : 0u;
  const uint32_t lo = tie ? (uint32_t)tie[(int64_t)h * tie_hstride + i] : (uint32_t)i;
  return ((uint64_t)hi << 32) | lo;
}

__global__ __launch_bounds__(1024) void block_sort_kernel(const float* __restrict__ score, int64_t score_hstride,
                                                         const int32_t* __restrict__ tie, int64_t tie_hstride,
                                                         uint64_t on, int n,
                                                         uint64_t* __restrict__ kout, int32_t* __restrict__ vout,
                                                         int32_t* __restrict__ final_out, int64_t final_hstride) {
  const int h = blockIdx.y;
  if (!head_on(on, h)) return;
  __shared__ uint64_t sk[SORT_BS];
  __shared__ int32_t sv[SORT_BS];
  const int base = blockIdx.x * SORT_BS;
  for (int i = threadIdx.x; i < SORT_BS; i += 1024) {
    const int g = base + i;
    if (g < n) {
      sk[i] = sort_key(score, tie, tie_hstride, h, g, score_hstride);
      sv[i] = g;
    } else {
      sk[i] = ~0ull;
      sv[i] = -1;
    }
  }
  __syncthreads();
  // bitonic network: one compare-exchange per thread and step
  const int p = threadIdx.x;
  for (int k = 2; k <= SORT_BS; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      const int i = (p / j) * 2 * j + (p % j);
      const int l = i + j;
      const bool up = ((i & k) == 0);
      const uint64_t a = sk[i], b = sk[l];
      if ((a > b) == up) {
        sk[i] = b; sk[l] = a;
        const int32_t t = sv[i]; sv[i] = sv[l]; sv[l] = t;
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < SORT_BS; i += 1024) {
    const int g = base + i;
    if (g < n) {
      if (final_out) final_out[(int64_t)h * final_hstride + g] = sv[i];
      else {
        kout[(int64_t)h * n + g] = sk[i];
        vout[(int64_t)h * n + g] = sv[i];
      }
    }
  }
}

__global__ __launch_bounds__(256) void merge_kernel(const uint64_t* __restrict__ kin, const int32_t* __restrict__ vin,
                                                    uint64_t on, int n, int L,
                                                    uint64_t* __restrict__ kout, int32_t* __restrict__ vout,
                                                    int32_t* __restrict__ final_out, int64_t final_hstride) {
  const int h = blockIdx.y;
  if (!head_on(on, h)) return;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int64_t hb = (int64_t)h * n;
  const int pair0 = (i / (2 * L)) * (2 * L);
  const int a0 = pair0, a1 = min(n, pair0 + L);
  const int b0 = a1, b1 = min(n, pair0 + 2 * L);
  const uint64_t key = kin[hb + i];
  int lo, hi, pos;
  if (i < a1) {   // element of run A: count B elements < key
    lo = b0; hi = b1;
    while (lo < hi) { const int m = (lo + hi) >> 1; if (kin[hb + m] < key) lo = m + 1; else hi = m; }
    pos = pair0 + (i - a0) + (lo - b0);
  } else {        // element of run B: count A elements < key
    lo = a0; hi = a1;
    while (lo < hi) { const int m = (lo + hi) >> 1; if (kin[hb + m] < key) lo = m + 1; else hi = m; }
    pos = pair0 + (i - b0) + (lo - a0);
  }
  if (final_out) final_out[(int64_t)h * final_hstride + pos] = vin[hb + i];
  else {
    kout[hb + pos] = key;
    vout[hb + pos] = vin[hb + i];
  }
}

hipError_t launch_sort(const float* score, int64_t score_hstride, const int32_t* tie, int64_t tie_hstride,
                       uint64_t on, int H, int n, uint64_t* k0, uint64_t* k1, int32_t* v0, int32_t* v1,
                       int32_t* out, int64_t out_hstride, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int nb = (n + SORT_BS - 1) / SORT_BS;
  const bool single = nb == 1;
  hipLaunchKernelGGL(block_sort_kernel, dim3(nb, H), dim3(SORT_BS / 2), 0, st, score, score_hstride, tie, tie_hstride, on,
                     n, k0, v0, single ? out : nullptr, out_hstride);
  if (single) return hipGetLastError();
  uint64_t* ka = k0; uint64_t* kb = k1;
  int32_t* va = v0; int32_t* vb = v1;
  for (int L = SORT_BS; L < n; L <<= 1) {
    const bool last = 2 * L >= n;
    hipLaunchKernelGGL(merge_kernel, dim3((n + 255) / 256, H), dim3(256), 0, st, ka, va, on, n, L, kb, vb,
                       last ? out : nullptr, out_hstride);
    uint64_t* tk = ka; ka = kb; kb = tk;
    int32_t* tv = va; va = vb; vb = tv;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// per-frame rank of a Forcing-KV segment score (frames hold a handful of
// segments: a direct count per item)
// ---------------------------------------------------------------------------
__global__ void frame_rank_kernel(const float* __restrict__ score, int items, int nseg, float* __restrict__ rank) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= items) return;
  const int f0 = (i / nseg) * nseg;
  const float s = score[i];
  int r = 0;
  for (int j = f0; j < f0 + nseg; ++j) {
    const float sj = score[j];
    r += (sj < s || (sj == s && j < i)) ? 1 : 0;
  }
  rank[i] = (float)r;
}

hipError_t launch_frame_rank(const float* score, int items, int nseg, float* rank, hipStream_t st) {
  if (items <= 0) return hipSuccess;
  hipLaunchKernelGGL(frame_rank_kernel, dim3((items + 255) / 256), dim3(256), 0, st, score, items, nseg, rank);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// shared prefix length k*
// ---------------------------------------------------------------------------
__global__ void hist_kernel(const int32_t* __restrict__ t, const int32_t* __restrict__ count,
                            uint64_t active, int M, int kmax, int32_t* __restrict__ hist) {
  const int h = blockIdx.y;
  if (!head_on(active, h)) return;
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= count[h]) return;
  int v = t[(int64_t)h * M + b];
  v = v < 0 ? 0 : v;
  // states that never cross within kmax do not enter any |V_h(k)|; skipping
  // them avoids serialising most atomics on one bin
  if (v <= kmax) atomicAdd(&hist[(int64_t)h * (kmax + 2) + v], 1);
}

__global__ __launch_bounds__(1024) void cumsum_kernel(int32_t* __restrict__ hist, uint64_t active,
                                                      int len) {
  const int h = blockIdx.x;
  if (!head_on(active, h)) return;
  __shared__ int32_t ws[16];
  int32_t* p = hist + (int64_t)h * len;
  // thread t scans the contiguous chunk [t * per, (t + 1) * per)
  const int per = (len + 1023) / 1024;
  const int b0 = min(len, (int)threadIdx.x * per), b1 = min(len, b0 + per);
  int32_t s = 0;
  for (int i = b0; i < b1; ++i) s += p[i];
  // exclusive prefix of the chunk sums: wave scan, then across waves
  int32_t inc = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t v = __shfl_up(inc, o);
    if (lane_id() >= o) inc += v;
  }
  if (lane_id() == 63) ws[wave_id()] = inc;
  __syncthreads();
  int32_t off = 0;
  for (int k = 0; k < wave_id(); ++k) off += ws[k];
  int32_t run = off + inc - s;
  for (int i = b0; i < b1; ++i) {
    run += p[i];
    p[i] = run;
  }
}

// head h admits the first k candidates: |V_h(k)| <= e_h(k), or (fill
// variant) the k fit below capacity with no density check
KVB_DEV bool head_feasible(const int32_t* cum, int n, int M, int kmax, int fill, int h, int k) {
  if (k == 0 || (fill && n + k <= M)) return true;
  return cum[(int64_t)h * (kmax + 2) + k] <= max(0, n + k - M);
}

// shared prefix: the largest k feasible for every density head
__global__ void feasible_kernel(const int32_t* __restrict__ cum, const int32_t* __restrict__ count,
                                uint64_t active, int H, int M, int kmax, int fill,
                                int32_t* __restrict__ kstar) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k > kmax) return;
  bool ok = true;
  for (int h = 0; h < H && ok; ++h)
    if (head_on(active, h)) ok = head_feasible(cum, count[h], M, kmax, fill, h, k);
  if (ok) atomicMax(kstar, k);
}

// per-head prefix: kstar[h] = the largest k feasible for head h
__global__ void feasible_head_kernel(const int32_t* __restrict__ cum, const int32_t* __restrict__ count,
                                     uint64_t active, int M, int kmax, int fill, int32_t* __restrict__ kstar) {
  const int h = blockIdx.y;
  if (!head_on(active, h)) return;
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k > kmax) return;
  if (head_feasible(cum, count[h], M, kmax, fill, h, k)) atomicMax(kstar + h, k);
}

// expects hist and kstar zeroed by the caller
hipError_t launch_kstar(const SelectLaunch& a, hipStream_t st) {
  if (a.M > 0)
    hipLaunchKernelGGL(hist_kernel, dim3((a.M + 255) / 256, a.H), dim3(256), 0, st, a.t, a.count, a.active, a.M,
                       a.kmax, a.hist);
  hipLaunchKernelGGL(cumsum_kernel, dim3(a.H), dim3(1024), 0, st, a.hist, a.active, a.kmax + 2);
  if (a.kstar_hs)
    hipLaunchKernelGGL(feasible_head_kernel, dim3((a.kmax + 1 + 255) / 256, a.H), dim3(256), 0, st, a.hist, a.count,
                       a.active, a.M, a.kmax, a.fill, a.kstar);
  else
    hipLaunchKernelGGL(feasible_kernel, dim3((a.kmax + 1 + 255) / 256), dim3(256), 0, st, a.hist, a.count,
                       a.active, a.H, a.M, a.kmax, a.fill, a.kstar);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// eviction: crossed states plus the r = e - |V| largest keys
// (projected density desc, token asc) among the rest, by an MSB-first radix
// select over 64-bit keys; then ballot/prefix-sum compaction of the evicted
// and surviving slots, both in ascending slot order.
// ---------------------------------------------------------------------------
// larger key = evicted first: (projected density desc, token asc), or the
// token alone (oldest first) for source-order completion
KVB_DEV uint64_t evict_key(float rp, int32_t tok, bool oldest) {
  const uint64_t t = (uint64_t)(0xFFFFFFFFu - (uint32_t)tok);
  return oldest ? t : (((uint64_t)float_key(rp) << 32) | t);
}

__global__ __launch_bounds__(1024) void evict_kernel(SelectLaunch a) {
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int M = a.M;
  const int64_t hb = (int64_t)h * M;
  if (!head_on(a.active, h)) return;
  const int n = a.count[h];
  const int ks = a.kstar[h * a.kstar_hs];
  const int e = ks > 0 ? max(0, n + ks - M) : 0;
  // crossed states (t_b <= k*): counted unless the prefix fits below capacity
  // in the fill variant; evicted first unless the eviction is densest-only
  const bool gated = ks > 0 && !(a.fill && n + ks <= M);
  const bool oldest = a.evict_mode == 2;
  const bool force = a.evict_mode != 1;
  __shared__ int hist[256];
  __shared__ int s_nm;
  __shared__ uint64_t s_prefix, s_mask;
  __shared__ int s_rem;
  __shared__ int wsum[16];
  __shared__ int s_base_e, s_base_s;
  if (tid == 0) { s_nm = 0; s_prefix = 0; s_mask = 0; s_base_e = 0; s_base_s = 0; }
  __syncthreads();
  int nm_local = 0;
  for (int b = tid; b < n; b += 1024) nm_local += (gated && a.t[hb + b] <= ks) ? 1 : 0;
  atomicAdd(&s_nm, nm_local);
  __syncthreads();
  const int nm_crossed = s_nm;
  const int nm = force ? nm_crossed : 0;   // forced evictions
  int r = e - nm;
  if (r < 0) {
    if (tid == 0) atomicOr(a.status, DEV_EVICT);
    r = 0;
  }
  if (tid == 0) s_rem = r;
  __syncthreads();
  // radix select of the r-th largest key among non-crossed states; none to
  // pick (r = 0) or all of them (r = n - nm) need no select
  if (r > 0 && r < n - nm) {
    __shared__ int wsc[4];
    __shared__ int s_sel;
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      for (int i = tid; i < 256; i += 1024) hist[i] = 0;
      __syncthreads();
      const uint64_t pre = s_prefix, msk = s_mask;
      for (int b = tid; b < n; b += 1024) {
        if (force && gated && a.t[hb + b] <= ks) continue;
        const uint64_t key = evict_key(a.rhoP[hb + b], a.bank_tok[hb + b], oldest);
        if ((key & msk) == pre) atomicAdd(&hist[(key >> shift) & 0xFF], 1);
      }
      __syncthreads();
      // suffix counts S(d) = #keys with digit >= d: thread t < 256 takes digit
      // 255 - t and scans in t; the selected digit has S(d) >= rem > S(d+1)
      const int rem = s_rem;
      const int d = 255 - tid;
      int c = 0, inc = 0;
      if (tid < 256) {
        c = hist[d];
        inc = c;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int v = __shfl_up(inc, o);
          if (lane >= o) inc += v;
        }
        if (lane == 63) wsc[w] = inc;
      }
      __syncthreads();
      if (tid < 256) {
        int off = 0;
        for (int k = 0; k < w; ++k) off += wsc[k];
        const int S = off + inc;
        if (S >= rem && S - c < rem) { s_sel = d; s_rem = rem - (S - c); }
      }
      __syncthreads();
      if (tid == 0) {
        s_prefix = pre | ((uint64_t)s_sel << shift);
        s_mask = msk | (0xFFull << shift);
      }
      __syncthreads();
    }
  }
  // keys >= thr are evicted among the non-crossed states (all of them when
  // r covers every such state)
  const uint64_t thr = (r >= n - nm) ? 0ull : s_prefix;
  // admitted states' densities: sum over the survivors directly when they are
  // fewer than the evicted states, else D(c) minus the evicted interactions
  const bool direct = (n - e) < e;
  // compaction in ascending slot order
  for (int base = 0; base < n; base += 1024) {
    const int b = base + tid;
    bool ev = false, live = b < n;
    if (live) {
      const bool mand = force && gated && a.t[hb + b] <= ks;
      ev = mand || (r > 0 && evict_key(a.rhoP[hb + b], a.bank_tok[hb + b], oldest) >= thr);
      a.evict[hb + b] = ev ? 1 : 0;
    }
    const uint64_t be = __ballot(live && ev);
    const uint64_t bs = __ballot(live && !ev);
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int pe = __popcll(be & lt), ps = __popcll(bs & lt);
    if (lane == 0) wsum[w] = (__popcll(be) << 16) | __popcll(bs);
    __syncthreads();
    int oe = 0, os = 0;
    for (int j = 0; j < w; ++j) { oe += wsum[j] >> 16; os += wsum[j] & 0xFFFF; }
    const int be0 = s_base_e, bs0 = s_base_s;
    if (live && ev) {
      a.evl[hb + be0 + oe + pe] = b;
      if (!direct) a.fixl[hb + be0 + oe + pe] = b;
    }
    if (live && !ev) {
      a.surv[hb + bs0 + os + ps] = b;
      if (direct) a.fixl[hb + bs0 + os + ps] = b;
    }
    __syncthreads();
    if (tid == 0) {
      int te = 0, ts = 0;
      for (int j = 0; j < 16; ++j) { te += wsum[j] >> 16; ts += wsum[j] & 0xFFFF; }
      s_base_e += te; s_base_s += ts;
    }
    __syncthreads();
  }
  for (int b = n + tid; b < M; b += 1024) a.evict[hb + b] = 0;
  if (tid == 0) {
    a.n_ev[h] = s_base_e;
    a.n_surv[h] = s_base_s;
    a.n_mand[h] = nm_crossed;
    a.n_fix[h] = direct ? s_base_s : s_base_e;
    a.fmode[h] = direct ? 1 : 0;
    if (s_base_e != e) atomicOr(a.status, DEV_EVICT);
  }
}

hipError_t launch_evict(const SelectLaunch& a, hipStream_t st) {
  hipLaunchKernelGGL(evict_kernel, dim3(a.H), dim3(1024), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// apply: survivors' density update, gather of admitted K/V rows into freed
// slots (then appended after the old occupancy), baselines of admitted rows
// ---------------------------------------------------------------------------
__global__ void apply_surv_kernel(ApplyLaunch a) {
  const int h = blockIdx.y;
  if (!head_on(a.active, h)) return;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= a.n_surv[h]) return;
  const int64_t hb = (int64_t)h * a.M;
  const int slot = a.surv[hb + i];
  const float r = a.rhoP[hb + slot] - a.acc_surv[hb + i];
  a.rho[hb + slot] = r;
  if (a.refresh) a.rho0[hb + slot] = r;
}

// 8 rows per 256-thread block; each row moves K and V (16-byte chunks)
template <int CPR>
__global__ __launch_bounds__(256) void apply_adm_kernel(ApplyLaunch a) {
  const int h = blockIdx.y;
  if (!head_on(a.active, h)) return;
  const int ks = a.kstar[h * a.kstar_hs];
  constexpr int RPB = 256 / (2 * CPR);
  const int j = blockIdx.x * RPB + threadIdx.x / (2 * CPR);
  if (j >= ks) return;
  const int part = (threadIdx.x % (2 * CPR)) / CPR;   // 0 = K, 1 = V
  const int c = threadIdx.x % CPR;
  const int64_t hb = (int64_t)h * a.M;
  const int ne = a.n_ev[h];
  const int nold = a.n_surv[h] + ne;
  const int slot = j < ne ? a.evl[hb + j] : nold + (j - ne);
  const int cand = a.order[(int64_t)h * a.N + j];
  if ((unsigned)slot >= (unsigned)a.M || (unsigned)cand >= (unsigned)a.N) return;
  const int esz = a.et == ET_BF16 ? 2 : 4;
  const int64_t rowb = (int64_t)a.d * esz;
  const char* src = (const char*)(part ? a.candV : a.candK) + ((int64_t)h * a.N + cand) * rowb;
  char* dst = (char*)(part ? a.bankV : a.bankK) + (hb + slot) * rowb;
  *reinterpret_cast<u32x4_t*>(dst + c * 16) = *reinterpret_cast<const u32x4_t*>(src + c * 16);
  if (threadIdx.x % (2 * CPR) == 0) {
    const int64_t hk = (int64_t)h * a.kmax + j;
    const float r = a.fmode[h] ? a.acc_adm_ev[hk] + a.acc_adm_adm[hk]
                               : (a.D[(int64_t)h * a.N + cand] - a.acc_adm_ev[hk]) + a.acc_adm_adm[hk];
    a.rho[hb + slot] = r;
    a.rho0[hb + slot] = r;
    a.bank_tok[hb + slot] = a.cand_tok[cand];
  }
}

__global__ void commit_count_kernel(ApplyLaunch a) {
  const int h = threadIdx.x;
  if (h >= a.H || !head_on(a.active, h)) return;
  a.count[h] = a.n_surv[h] + a.kstar[h * a.kstar_hs];
}

hipError_t launch_apply(const ApplyLaunch& a, hipStream_t st) {
  if (a.M > 0)
    hipLaunchKernelGGL(apply_surv_kernel, dim3((a.M + 255) / 256, a.H), dim3(256), 0, st, a);
  const int cpr = a.d * (a.et == ET_BF16 ? 2 : 4) / 16;
  if (a.kmax > 0) {
    if (cpr == 16)
      hipLaunchKernelGGL((apply_adm_kernel<16>), dim3((a.kmax + 7) / 8, a.H), dim3(256), 0, st, a);
    else if (cpr == 8)
      hipLaunchKernelGGL((apply_adm_kernel<8>), dim3((a.kmax + 15) / 16, a.H), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((apply_adm_kernel<32>), dim3((a.kmax + 3) / 4, a.H), dim3(256), 0, st, a);
  }
  hipLaunchKernelGGL(commit_count_kernel, dim3(1), dim3(64), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// segment tables consumed by chunk attention
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void segments_kernel(SegLaunch a) {
  const int h = blockIdx.x;
  const int esz = a.et == ET_BF16 ? 2 : 4;
  const int64_t rowb = (int64_t)a.d * esz;
  SegEntry* out = a.segs + (int64_t)h * a.seg_cap;
  extern __shared__ uint32_t bits[];
  __shared__ int s_n;
  const uint8_t lab = a.label[h];
  if (threadIdx.x == 0) s_n = 0;
  __syncthreads();
  auto push = [&](const void* kb, const void* vb, int64_t head_rows, int64_t row0, int len) {
    if (len <= 0) return;
    const int i = s_n;
    if (i >= a.seg_cap) { atomicOr(a.status, DEV_SEGOVF); return; }
    out[i].k = (const char*)kb + ((int64_t)h * head_rows + row0) * rowb;
    out[i].v = (const char*)vb + ((int64_t)h * head_rows + row0) * rowb;
    out[i].len = len;
    out[i].pad = 0;
    s_n = i + 1;
  };
  if (lab == 2) {
    const int words = (a.items + 31) / 32;
    for (int i = threadIdx.x; i < words; i += 64) bits[i] = 0u;
    __syncthreads();
    for (int j = threadIdx.x; j < a.keep; j += 64) {
      const int it = a.dyn_order[(int64_t)h * a.dyn_order_hstride + j];
      if ((unsigned)it < (unsigned)a.items) atomicOr(&bits[it >> 5], 1u << (it & 31));
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    push(a.sink_k, a.sink_v, a.sink_len, 0, a.sink_len);
    if (lab == 0) {
      push(a.bankK, a.bankV, a.M, 0, a.count[h]);
      if (a.win_len > 0) {
        const int first = min(a.win_len, a.win_cap - a.win_start);
        push(a.win_k, a.win_v, a.win_cap, a.win_start, first);
        push(a.win_k, a.win_v, a.win_cap, 0, a.win_len - first);
      }
    } else if (lab == 1) {
      if (a.N >= a.F) push(a.candK, a.candV, a.N, a.N - a.F, a.F);
    } else {
      int it = 0;
      while (it < a.items) {
        if (bits[it >> 5] & (1u << (it & 31))) {
          int end = it + 1;
          while (end < a.items && (bits[end >> 5] & (1u << (end & 31)))) ++end;
          push(a.candK, a.candV, a.N, (int64_t)it * a.seg_len, (end - it) * a.seg_len);
          it = end;
        } else {
          ++it;
        }
      }
    }
    push(a.chunk_k, a.chunk_v, a.chunk_len, 0, a.chunk_len);
    a.nseg[h] = s_n;
  }
}

hipError_t launch_segments(const SegLaunch& a, hipStream_t st) {
  const size_t shm = (size_t)((a.items + 31) / 32 + 1) * 4;
  hipLaunchKernelGGL(segments_kernel, dim3(a.H), dim3(64), shm, st, a);
  return hipGetLastError();
}

}  // namespace kvb
