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

// the clears of zero_i32x4_kernel in every block, and in block 0 the count
// clamp of the update's prologue
__global__ void zero_clamp_kernel(ZeroSet z, CountClamp cc) {
  if (blockIdx.x == 0 && (int)threadIdx.x < cc.H && head_on(cc.active, threadIdx.x)) {
    const int h = threadIdx.x;
    const int n = cc.count[h];
    const int c = min(max(n, 0), cc.M);
    cc.cnt[h] = c;
    if (c != n) atomicOr(cc.status, DEV_COUNT);
  }
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (i < z.n[k]) { z.p[k][i] = 0; return; }
    i -= z.n[k];
  }
}

hipError_t launch_zero_i32_clamp(int32_t* const* ptrs, const int64_t* lens, int count, const CountClamp& cc,
                                 hipStream_t st) {
  ZeroSet z{};
  int64_t tot = 0;
  for (int k = 0; k < 4; ++k) {
    z.p[k] = k < count ? ptrs[k] : nullptr;
    z.n[k] = (k < count && ptrs[k]) ? lens[k] : 0;
    tot += z.n[k];
  }
  const int64_t blocks = (tot + 255) / 256 > 0 ? (tot + 255) / 256 : 1;
  hipLaunchKernelGGL(zero_clamp_kernel, dim3((unsigned)blocks), dim3(256), 0, st, z, cc);
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
// ascending; value = index.  Blocks of 2048 are sorted by a bitonic network
// whose steps between elements less than 128 apart run in registers (lane
// shuffles within a wave, no barrier) and the rest through LDS.  Sorted
// runs are then merged pairwise by rank: an element's place is its index in
// its own run plus the number of keys before it in the other run (keys
// equal to it count from the first run only, so places never collide).
// ---------------------------------------------------------------------------
constexpr int SORT_BS = 2048;

KVB_DEV uint64_t sort_key(const float* score, const int32_t* tie, int64_t tie_hstride, int h, int i,
                          int64_t score_hstride) {
  // no score: the tie key alone (source order, by token id)
  const uint32_t hi = score ? float_key(score[(int64_t)h * score_hstride + i]) : 0u;
  const uint32_t lo = tie ? (uint32_t)tie[(int64_t)h * tie_hstride + i] : (uint32_t)i;
  return ((uint64_t)hi << 32) | lo;
}

// the value of lane (lane ^ m), m a power of two below 64 known at compile
// time: lane moves within a quad for m < 4, swizzles within 32 lanes below
// 32, a permute across the halves for 32
KVB_DEV int lane_xor(int v, int m) {
  switch (m) {
    case 1: return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);   // quad_perm (1, 0, 3, 2)
    case 2: return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);   // quad_perm (2, 3, 0, 1)
    case 4: return __builtin_amdgcn_ds_swizzle(v, (4 << 10) | 0x1F);
    case 8: return __builtin_amdgcn_ds_swizzle(v, (8 << 10) | 0x1F);
    case 16: return __builtin_amdgcn_ds_swizzle(v, (16 << 10) | 0x1F);
    default: return __shfl_xor(v, m);
  }
}
KVB_DEV uint64_t lane_xor_u64(uint64_t v, int m) {
  const uint32_t lo = (uint32_t)lane_xor((int)(uint32_t)v, m);
  const uint32_t hi = (uint32_t)lane_xor((int)(uint32_t)(v >> 32), m);
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
  // thread t holds elements 2t and 2t + 1
  const int t = threadIdx.x;
  uint64_t k[2];
  int32_t v[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int g = base + 2 * t + b;
    k[b] = g < n ? sort_key(score, tie, tie_hstride, h, g, score_hstride) : ~0ull;
    v[b] = g < n ? g : -1;
  }
#pragma unroll
  for (int kk = 2; kk <= SORT_BS; kk <<= 1) {
    int j = kk >> 1;
    if (j >= 128) {
      // steps across waves: one compare-exchange per thread and step in LDS
      sk[2 * t] = k[0];
      sk[2 * t + 1] = k[1];
      sv[2 * t] = v[0];
      sv[2 * t + 1] = v[1];
      __syncthreads();
#pragma unroll
      for (; j >= 128; j >>= 1) {
        const int i = (t / j) * 2 * j + (t % j);
        const int l = i + j;
        const bool up = ((i & kk) == 0);
        const uint64_t a = sk[i], c = sk[l];
        if ((a > c) == up) {
          sk[i] = c;
          sk[l] = a;
          const int32_t tv = sv[i];
          sv[i] = sv[l];
          sv[l] = tv;
        }
        __syncthreads();
      }
      k[0] = sk[2 * t];
      k[1] = sk[2 * t + 1];
      v[0] = sv[2 * t];
      v[1] = sv[2 * t + 1];
    }
    // steps within a wave: element 2t + b meets 2(t ^ j/2) + b (j >= 2), or
    // its neighbour in the same thread (j = 1); the lower index of a pair
    // keeps the smaller key when its kk bit is clear
#pragma unroll
    for (; j >= 2; j >>= 1) {
      const bool keep_min = (((2 * t) & j) == 0) == (((2 * t) & kk) == 0);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const uint64_t pk = lane_xor_u64(k[b], j >> 1);
        const int32_t pv = lane_xor(v[b], j >> 1);
        const bool lt = pk < k[b];
        const uint64_t mn = lt ? pk : k[b], mx = lt ? k[b] : pk;
        const uint64_t nk = keep_min ? mn : mx;
        v[b] = nk != k[b] ? pv : v[b];
        k[b] = nk;
      }
    }
    {
      const bool up = ((2 * t) & kk) == 0;
      const bool sw = (k[0] > k[1]) == up;
      const uint64_t k0 = sw ? k[1] : k[0], k1 = sw ? k[0] : k[1];
      const int32_t v0 = sw ? v[1] : v[0], v1 = sw ? v[0] : v[1];
      k[0] = k0;
      k[1] = k1;
      v[0] = v0;
      v[1] = v1;
    }
  }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int g = base + 2 * t + b;
    if (g < n) {
      if (final_out) final_out[(int64_t)h * final_hstride + g] = v[b];
      else {
        kout[(int64_t)h * n + g] = k[b];
        vout[(int64_t)h * n + g] = v[b];
      }
    }
  }
}

// number of keys in run[0, len) before key: smaller, or (before_equal) equal
KVB_DEV int run_rank(const uint64_t* run, int len, uint64_t key, bool before_equal) {
  int lo = 0, hi = len;
  while (lo < hi) {
    const int m = (lo + hi) >> 1;
    const uint64_t x = run[m];
    if (x < key || (before_equal && x == key)) lo = m + 1;
    else hi = m;
  }
  return lo;
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
  int pos;
  if (i < a1) pos = pair0 + (i - a0) + run_rank(kin + hb + b0, b1 - b0, key, false);   // run A: B's smaller keys
  else pos = pair0 + (i - b0) + run_rank(kin + hb + a0, a1 - a0, key, true);           // run B: A's keys up to key
  if (final_out) final_out[(int64_t)h * final_hstride + pos] = vin[hb + i];
  else {
    kout[hb + pos] = key;
    vout[hb + pos] = vin[hb + i];
  }
}

// small n (<= 1024): every item's rank is the number of keys before it
// (smaller, or equal and at a lower index)
__global__ __launch_bounds__(1024) void rank_sort_kernel(const float* __restrict__ score, int64_t score_hstride,
                                                        const int32_t* __restrict__ tie, int64_t tie_hstride,
                                                        uint64_t on, int n, int32_t* __restrict__ out,
                                                        int64_t out_hstride, int64_t score_ls, int64_t out_ls) {
  const int h = blockIdx.x;
  if (!head_on(on, h)) return;
  // layer blockIdx.y of a batch of layers (strides 0 for one layer)
  score += blockIdx.y * score_ls;
  out += blockIdx.y * out_ls;
  __shared__ uint64_t sk[1024];
  const int i = threadIdx.x;
  if (i < n) sk[i] = sort_key(score, tie, tie_hstride, h, i, score_hstride);
  __syncthreads();
  if (i >= n) return;
  const uint64_t key = sk[i];
  int r = 0;
  for (int j = 0; j < n; ++j) r += (sk[j] < key || (sk[j] == key && j < i)) ? 1 : 0;
  out[(int64_t)h * out_hstride + r] = i;
}

hipError_t launch_sort(const float* score, int64_t score_hstride, const int32_t* tie, int64_t tie_hstride,
                       uint64_t on, int H, int n, uint64_t* k0, uint64_t* k1, int32_t* v0, int32_t* v1,
                       int32_t* out, int64_t out_hstride, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (n <= 1024) {
    hipLaunchKernelGGL(rank_sort_kernel, dim3(H), dim3(1024), 0, st, score, score_hstride, tie, tie_hstride, on, n,
                       out, out_hstride, (int64_t)0, (int64_t)0);
    return hipGetLastError();
  }
  const int nb = (n + SORT_BS - 1) / SORT_BS;
  const bool single = nb == 1;
  hipLaunchKernelGGL(block_sort_kernel, dim3(nb, H), dim3(SORT_BS / 2), 0, st, score, score_hstride, tie, tie_hstride, on,
                     n, k0, v0, single ? out : nullptr, out_hstride);
  if (single) return hipGetLastError();
  uint64_t* ka = k0; uint64_t* kb = k1;
  int32_t* va = v0; int32_t* vb = v1;
  for (int L = SORT_BS; L < n; L <<= 1) {
    const bool last = 2 * (int64_t)L >= n;
    hipLaunchKernelGGL(merge_kernel, dim3((n + 255) / 256, H), dim3(256), 0, st, ka, va, on, n, L, kb, vb,
                       last ? out : nullptr, out_hstride);
    uint64_t* tk = ka; ka = kb; kb = tk;
    int32_t* tv = va; va = vb; vb = tv;
  }
  return hipGetLastError();
}

// the rank sort of up to 1,024 items for each of nlayers layers (layer l's
// scores and order at + l score_ls, + l out_ls)
hipError_t launch_rank_sort_layers(const float* score, int64_t score_hstride, int64_t score_ls, uint64_t on, int H,
                                   int n, int nlayers, int32_t* out, int64_t out_hstride, int64_t out_ls,
                                   hipStream_t st) {
  if (n <= 0 || nlayers <= 0) return hipSuccess;
  hipLaunchKernelGGL(rank_sort_kernel, dim3(H, nlayers), dim3(1024), 0, st, score, score_hstride, nullptr, (int64_t)0,
                     on, n, out, out_hstride, score_ls, out_ls);
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

// Eviction in three launches, so that the per-state passes run on many
// work-groups per head:
//   evict_select_kernel  (one block per head) the counts, and the threshold
//                        key of the r-th largest key when a partial
//                        completion is needed (8-bit MSB-first radix select,
//                        ended once every key of the selected bin is taken:
//                        the threshold is then that bin's smallest key);
//                        the crossed count at k* is read from the crossing-
//                        time prefix sums, so the common cases pass over no
//                        state at all
//   evict_flags_kernel   (256 states per block) the eviction flag of every
//                        slot and each block's evicted / surviving counts
//   evict_write_kernel   (256 states per block) the block's offset from the
//                        counts before it, then ballot compaction of the
//                        evicted and surviving slots in ascending slot order
struct EvSel {        // per head, written by evict_select_kernel
  uint64_t thr;       // completion threshold: keys >= thr are evicted
  int32_t n, e, r, nm, nm_crossed, mode;   // mode: 0 no completion, 1 all non-crossed, 2 keys >= thr
};
static_assert(sizeof(EvSel) <= 32, "per-head eviction plan slot");

KVB_DEV bool evict_flag(const SelectLaunch& a, const EvSel& q, int64_t hb, int b, int ks) {
  const bool gated = ks > 0 && !(a.fill && q.n + ks <= a.M) && !a.skip_cross;
  const bool force = a.evict_mode != 1;
  if (force && gated && a.t[hb + b] <= ks) return true;
  if (q.mode == 1) return true;
  if (q.mode == 2) return evict_key(a.rhoP[hb + b], a.bank_tok[hb + b], a.evict_mode == 2) >= q.thr;
  return false;
}

constexpr int EV_KPT = 16;   // keys per thread held in registers by the eviction select

__global__ __launch_bounds__(1024) void evict_select_kernel(SelectLaunch a) {
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
  // |V_h(k*)| from the prefix sums of the crossing-time histogram (not
  // computed when the whole bank is replaced without a crossing scan)
  const int nm_crossed = a.skip_cross ? -1 : (gated ? a.hist[(int64_t)h * (a.kmax + 2) + ks] : 0);
  const int nm = (force && !a.skip_cross) ? nm_crossed : 0;
  int r = e - nm;
  if (r < 0) {
    if (tid == 0) atomicOr(a.status, DEV_EVICT);
    r = 0;
  }
  // none to pick (r = 0) or all of them (r = n - nm): no select
  const int mode = r == 0 ? 0 : (r >= n - nm ? 1 : 2);
  __shared__ int hist[256];
  __shared__ uint64_t s_prefix, s_mask;
  __shared__ int s_rem;
  __shared__ int wsc[4];
  __shared__ int s_sel, s_cnt;
  __shared__ unsigned long long s_min;
  if (mode == 2) {
    if (tid == 0) { s_prefix = 0; s_mask = 0; s_rem = r; }
    // Up to EV_KPT keys per thread are read once into registers (all their
    // loads in flight together); the passes then bin registers.  Larger
    // banks read the keys from memory at every pass.
    const bool inreg = n <= EV_KPT * 1024;
    uint64_t kr[EV_KPT];
    uint32_t live = 0;
    if (inreg) {
#pragma unroll
      for (int i = 0; i < EV_KPT; ++i) {
        const int b = tid + 1024 * i;
        kr[i] = 0;
        if (b < n && !(force && gated && !a.skip_cross && a.t[hb + b] <= ks)) {
          kr[i] = evict_key(a.rhoP[hb + b], a.bank_tok[hb + b], oldest);
          live |= 1u << i;
        }
      }
    }
    __syncthreads();
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      for (int i = tid; i < 256; i += 1024) hist[i] = 0;
      __syncthreads();
      const uint64_t pre = s_prefix, msk = s_mask;
      if (inreg) {
#pragma unroll
        for (int i = 0; i < EV_KPT; ++i)
          if (((live >> i) & 1u) && (kr[i] & msk) == pre) atomicAdd(&hist[(kr[i] >> shift) & 0xFF], 1);
      } else {
        for (int b = tid; b < n; b += 1024) {
          if (force && gated && !a.skip_cross && a.t[hb + b] <= ks) continue;
          const uint64_t key = evict_key(a.rhoP[hb + b], a.bank_tok[hb + b], oldest);
          if ((key & msk) == pre) atomicAdd(&hist[(key >> shift) & 0xFF], 1);
        }
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
        if (S >= rem && S - c < rem) { s_sel = d; s_rem = rem - (S - c); s_cnt = c; }
      }
      __syncthreads();
      if (tid == 0) {
        s_prefix = pre | ((uint64_t)s_sel << shift);
        s_mask = msk | (0xFFull << shift);
        s_min = ~0ull;
      }
      __syncthreads();
      if (s_cnt == s_rem) {
        // every key of the selected bin is taken (always so once the bin
        // holds a single key): the threshold is the bin's smallest key
        const uint64_t pre2 = s_prefix, msk2 = s_mask;
        unsigned long long mn = ~0ull;
        if (inreg) {
#pragma unroll
          for (int i = 0; i < EV_KPT; ++i)
            if (((live >> i) & 1u) && (kr[i] & msk2) == pre2) mn = kr[i] < mn ? kr[i] : mn;
        } else {
          for (int b = tid; b < n; b += 1024) {
            if (force && gated && !a.skip_cross && a.t[hb + b] <= ks) continue;
            const uint64_t key = evict_key(a.rhoP[hb + b], a.bank_tok[hb + b], oldest);
            if ((key & msk2) == pre2) mn = key < mn ? key : mn;
          }
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
          const unsigned long long v = __shfl_xor(mn, o);
          mn = v < mn ? v : mn;
        }
        if (lane == 0 && mn != ~0ull) atomicMin(&s_min, mn);
        __syncthreads();
        if (tid == 0) s_prefix = s_min;
        __syncthreads();
        break;
      }
    }
  }
  if (tid == 0) {
    EvSel q;
    q.thr = mode == 2 ? s_prefix : 0ull;
    q.n = n; q.e = e; q.r = r; q.nm = nm; q.nm_crossed = nm_crossed; q.mode = mode;
    reinterpret_cast<EvSel*>(a.evsel)[h] = q;
  }
}

__global__ __launch_bounds__(256) void evict_flags_kernel(SelectLaunch a) {
  const int h = blockIdx.y;
  if (!head_on(a.active, h)) return;
  const int64_t hb = (int64_t)h * a.M;
  const EvSel q = reinterpret_cast<const EvSel*>(a.evsel)[h];
  const int ks = a.kstar[h * a.kstar_hs];
  const int b = blockIdx.x * 256 + threadIdx.x;
  const bool live = b < q.n;
  const bool ev = live && evict_flag(a, q, hb, b, ks);
  if (b < a.M) a.evict[hb + b] = ev ? 1 : 0;
  __shared__ int cnt[2];
  if (threadIdx.x == 0) { cnt[0] = 0; cnt[1] = 0; }
  __syncthreads();
  const uint64_t be = __ballot(ev), bs = __ballot(live && !ev);
  if (lane_id() == 0) {
    atomicAdd(&cnt[0], __popcll(be));
    atomicAdd(&cnt[1], __popcll(bs));
  }
  __syncthreads();
  if (threadIdx.x == 0) a.evblk[(int64_t)h * gridDim.x + blockIdx.x] = (cnt[0] << 16) | cnt[1];
}

__global__ __launch_bounds__(256) void evict_write_kernel(SelectLaunch a) {
  const int h = blockIdx.y;
  if (!head_on(a.active, h)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t hb = (int64_t)h * a.M;
  const EvSel q = reinterpret_cast<const EvSel*>(a.evsel)[h];
  const int nblk = gridDim.x, blk = blockIdx.x;
  const int32_t* bc = a.evblk + (int64_t)h * nblk;
  const bool direct = (q.n - q.e) < q.e;
  // offsets of this block: the counts of the blocks before it; the last
  // block also writes the totals
  __shared__ int s_oe, s_os, s_we[4], s_ws[4];
  if (w == 0) {
    int oe = 0, os = 0, te = 0, ts = 0;
    for (int i = lane; i < nblk; i += 64) {
      const int v = bc[i];
      if (i < blk) { oe += v >> 16; os += v & 0xFFFF; }
      te += v >> 16;
      ts += v & 0xFFFF;
    }
    oe = wave_sum_i(oe);
    os = wave_sum_i(os);
    te = wave_sum_i(te);
    ts = wave_sum_i(ts);
    if (lane == 0) {
      s_oe = oe;
      s_os = os;
      if (blk == nblk - 1) {
        a.n_ev[h] = te;
        a.n_surv[h] = ts;
        a.n_mand[h] = q.nm_crossed;
        a.n_fix[h] = direct ? ts : te;
        a.fmode[h] = direct ? 1 : 0;
        if (te != q.e) atomicOr(a.status, DEV_EVICT);
      }
    }
  }
  const int b = blk * 256 + tid;
  const bool live = b < q.n;
  const bool ev = live && a.evict[hb + b];
  const uint64_t be = __ballot(ev), bs = __ballot(live && !ev);
  if (lane == 0) { s_we[w] = __popcll(be); s_ws[w] = __popcll(bs); }
  __syncthreads();
  int oe = s_oe, os = s_os;
  for (int k = 0; k < w; ++k) { oe += s_we[k]; os += s_ws[k]; }
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  if (ev) {
    const int j = oe + __popcll(be & lt);
    a.evl[hb + j] = b;
    if (!direct) a.fixl[hb + j] = b;
  }
  if (live && !ev) {
    const int j = os + __popcll(bs & lt);
    a.surv[hb + j] = b;
    if (direct) a.fixl[hb + j] = b;
  }
}

hipError_t launch_evict(const SelectLaunch& a, hipStream_t st) {
  hipLaunchKernelGGL(evict_select_kernel, dim3(a.H), dim3(1024), 0, st, a);
  const unsigned nblk = (unsigned)((a.M + 255) / 256);
  if (nblk == 0) return hipGetLastError();
  hipLaunchKernelGGL(evict_flags_kernel, dim3(nblk, a.H), dim3(256), 0, st, a);
  hipLaunchKernelGGL(evict_write_kernel, dim3(nblk, a.H), dim3(256), 0, st, a);
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

// Gather of admitted rows.  TPR threads per row, each moving U 16-byte
// chunks: chunk r + TPR i of the row's K chunks followed by its V chunks, so
// that each load and store instruction covers whole consecutive 16 TPR-byte
// pieces of a row and every thread keeps U loads in flight.
template <int CPR>
__global__ __launch_bounds__(256) void apply_adm_kernel(ApplyLaunch a) {
  constexpr int U = 4;
  constexpr int TPR = 2 * CPR / U;   // threads per row
  constexpr int RPB = 256 / TPR;     // rows per block
  static_assert(CPR % U == 0 && 256 % TPR == 0, "gather shape");
  const int h = blockIdx.y;
  if (!head_on(a.active, h)) return;
  const int ks = a.kstar[h * a.kstar_hs];
  const int j = blockIdx.x * RPB + threadIdx.x / TPR;
  if (j >= ks) return;
  const int r = threadIdx.x % TPR;
  const int64_t hb = (int64_t)h * a.M;
  const int ne = a.n_ev[h];
  const int nold = a.n_surv[h] + ne;
  const int slot = j < ne ? a.evl[hb + j] : nold + (j - ne);
  const int cand = a.order[(int64_t)h * a.N + j];
  if ((unsigned)slot >= (unsigned)a.M || (unsigned)cand >= (unsigned)a.N) return;
  const int64_t rowb = (int64_t)CPR * 16;
  const char* srcK = (const char*)a.candK + ((int64_t)h * a.N + cand) * rowb;
  const char* srcV = (const char*)a.candV + ((int64_t)h * a.N + cand) * rowb;
  char* dstK = (char*)a.bankK + (hb + slot) * rowb;
  char* dstV = (char*)a.bankV + (hb + slot) * rowb;
  u32x4_t v[U];
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const int c = r + TPR * i;   // < 2 CPR
    const char* src = c < CPR ? srcK + c * 16 : srcV + (c - CPR) * 16;
    v[i] = *reinterpret_cast<const u32x4_t*>(src);
  }
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const int c = r + TPR * i;
    char* dst = c < CPR ? dstK + c * 16 : dstV + (c - CPR) * 16;
    *reinterpret_cast<u32x4_t*>(dst) = v[i];
  }
  if (r == 0) {
    const int64_t hk = (int64_t)h * a.kmax + j;
    const float rr = a.fmode[h] ? a.acc_adm_ev[hk] + a.acc_adm_adm[hk]
                                : (a.D[(int64_t)h * a.N + cand] - a.acc_adm_ev[hk]) + a.acc_adm_adm[hk];
    a.rho[hb + slot] = rr;
    a.rho0[hb + slot] = rr;
    a.bank_tok[hb + slot] = a.cand_tok[cand];
  }
}

// descriptor rows of the admitted candidates, into the slots apply_adm_kernel
// gives their keys (16-byte chunks)
__global__ __launch_bounds__(256) void apply_adm_x_kernel(ApplyLaunch a) {
  const int h = blockIdx.y;
  if (!head_on(a.active, h)) return;
  const int ks = a.kstar[h * a.kstar_hs];
  const int esz = a.et == ET_BF16 ? 2 : 4;
  const int cpr = a.dx * esz / 16;
  const int u = blockIdx.x * 256 + threadIdx.x;
  const int j = u / cpr, c = u % cpr;
  if (j >= ks) return;
  const int64_t hb = (int64_t)h * a.M;
  const int ne = a.n_ev[h];
  const int nold = a.n_surv[h] + ne;
  const int slot = j < ne ? a.evl[hb + j] : nold + (j - ne);
  const int cand = a.order[(int64_t)h * a.N + j];
  if ((unsigned)slot >= (unsigned)a.M || (unsigned)cand >= (unsigned)a.N) return;
  const int64_t rowb = (int64_t)a.dx * esz;
  const char* src = (const char*)a.candX + ((int64_t)h * a.N + cand) * rowb;
  char* dst = (char*)a.bankX + (hb + slot) * rowb;
  *reinterpret_cast<u32x4_t*>(dst + c * 16) = *reinterpret_cast<const u32x4_t*>(src + c * 16);
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
    // rows per block: 256 / (2 cpr / 4)
    if (cpr == 16)
      hipLaunchKernelGGL((apply_adm_kernel<16>), dim3((a.kmax + 31) / 32, a.H), dim3(256), 0, st, a);
    else if (cpr == 8)
      hipLaunchKernelGGL((apply_adm_kernel<8>), dim3((a.kmax + 63) / 64, a.H), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((apply_adm_kernel<32>), dim3((a.kmax + 15) / 16, a.H), dim3(256), 0, st, a);
  }
  if (a.bankX && a.candX && a.kmax > 0) {
    const int cprx = a.dx * (a.et == ET_BF16 ? 2 : 4) / 16;
    hipLaunchKernelGGL(apply_adm_x_kernel, dim3((unsigned)(((int64_t)a.kmax * cprx + 255) / 256), a.H), dim3(256), 0,
                       st, a);
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
      // the committed count, clamped (no update ran when N = 0)
      const int n = a.count[h];
      const int nc = min(max(n, 0), a.M);
      if (nc != n) atomicOr(a.status, DEV_COUNT);
      push(a.bankK, a.bankV, a.M, 0, nc);
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
