// Chunk attention over the ragged per-head retained KV.
//
// DensityKV card page, Figure 2: the current queries read the retained
// history (sink, per-head bank, local window) through the backbone's native
// attention; Forcing-KV notes page, section 3.3: the chunk attends to its own
// keys without a mask.  O_h = softmax(Q_h K_h^T * scale) V_h, where K_h/V_h
// is the concatenation of the head's segments (order irrelevant).
//
// bf16 path: flash-style online softmax.  Work-group = 8 waves x 32 queries;
// KV tiles of 64 keys staged in LDS, double buffered: K and V row-major with
// XOR-swizzled 16-byte chunks, copied straight from global memory to LDS;
// V^T fragments come from the transposing LDS read.  The next tile's copies
// are in flight while the current tile is multiplied.  Scores are computed transposed (S^T = K Q^T, 16x16x32
// MFMA) so every lane holds keys of a single query; P^T feeds
// O^T = V^T P^T directly as the B operand.  The running maximum is only
// moved when a tile raises it by more than 2^8 (exact: numerator and
// denominator share the stale maximum).
#include <type_traits>

#include "kvb_common.hpp"
#include "kvb_launch.hpp"

namespace kvb {

// Eight waves of 32 queries share each K/V tile in LDS: half the L2 -> LDS
// traffic per flop of four waves, which matters because the chip runs this
// kernel at its power limit (one work-group per CU, two waves per SIMD).
constexpr int ATT_NW = 8;            // waves per work-group
constexpr int ATT_NT = 64 * ATT_NW;  // threads per work-group
constexpr int ATT_TK = 64;           // keys per tile
constexpr int ATT_QW = 32;           // queries per wave
constexpr int ATT_QB = 32 * ATT_NW;  // queries per work-group
constexpr int ATT_MAXSEG = 256;     // segments cached in LDS
constexpr float ATT_RESCALE_LOG2 = 8.0f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

KVB_DEV uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

// XOR swizzle of the 16-byte chunks of a 64-row K or V tile in LDS.  With
// 16 chunks per row (d = 128) the chunk of row r is XORed with
// s(r) = ((r2 ^ r3) << 3) | (r1 r0 << 1) | r2: any 8 (or 16) aligned rows
// take distinct values, so the 16-byte K fragment reads (one chunk of
// consecutive rows) are conflict-free, and any 4 (or 8) aligned rows take
// distinct chunk pairs, so the transposing V reads (two adjacent chunks of
// 4 consecutive rows per 16 lanes) are too.  d = 64 keeps the 3 low bits.
template <int CPR> KVB_DEV int att_swz(int r) {
  const int base = ((r & 3) << 1) | ((r >> 2) & 1);
  if constexpr (CPR == 16) return base | ((((r >> 2) ^ (r >> 3)) & 1) << 3);
  else return base;
}

// LDS transpose read (gfx950): within each 16-lane group, lane 16G + i
// receives element i & 3 of the 8 bytes addressed by lanes 16G + 4j + (i >> 2),
// j = 0..3, as its elements j
KVB_DEV s16x4_t lds_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)p);
}

// Global -> LDS copies of 16 bytes per lane, written as inline assembly so
// that the compiler does not track them (its own tracking of copies through
// the builtins costs about a tenth of the attention time here).  The kernel
// orders them itself: s_waitcnt vmcnt(0) and a barrier before a copied tile
// is read.  M0 holds the wave's LDS destination (lane l writes 16 bytes at
// M0 + 16 l) and is declared clobbered, so the compiler reloads any value of
// its own after the statement.  No outputs: the data goes to LDS only.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
KVB_DEV void lds_copy_buf(i32x4_t rsrc, uint32_t voff, int soff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 1\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(m0), "v"(voff), "s"(rsrc),
               "s"(soff)
               : "memory", "m0");
}
KVB_DEV void lds_copy_glb(const void* g, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 1\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(g) : "memory", "m0");
}
// LDS byte address of p (wave-uniform)
KVB_DEV uint32_t lds_addr(const void* p) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)p);
}
// buffer resource on [base, base + nbytes): stride 0, raw buffer
KVB_DEV i32x4_t buf_rsrc(const void* base, int nbytes) {
  const uint64_t b = (uint64_t)base;
  i32x4_t r;
  r[0] = (int)(uint32_t)b;
  r[1] = (int)((uint32_t)(b >> 32) & 0xffffu);
  r[2] = nbytes;
  r[3] = 0x00020000;
  return r;
}

// O[off .. off + 3] = v * inv, as fp32 or bf16
KVB_DEV void attn_store(void* O, int out_f32, int64_t off, f32x4_t v, float inv) {
  if (out_f32) {
    const float4 r = {v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv};
    *reinterpret_cast<float4*>((float*)O + off) = r;
  } else {
    uint2 r;
    r.x = pack_bf16x2(v[0] * inv, v[1] * inv);
    r.y = pack_bf16x2(v[2] * inv, v[3] * inv);
    *reinterpret_cast<uint2*>((uint16_t*)O + off) = r;
  }
}

template <int D>
__global__ __launch_bounds__(ATT_NT, 2) void attn_bf16_kernel(const uint16_t* __restrict__ Q, void* __restrict__ O,
                                                           const SegEntry* __restrict__ segs,
                                                           const int32_t* __restrict__ nseg_p, int seg_cap, int Lq,
                                                           float scale_log2, int out_f32, int nqt, int H,
                                                           int rounds, int Ir, f32x4_t* __restrict__ part,
                                                           int32_t* __restrict__ pflag) {
  using Op = Ops<uint16_t>;
  constexpr int NKS = D / 32;             // k-steps for S^T
  constexpr int NDB = D / 16;             // d blocks for O^T
  constexpr int CPR = D / 8;              // 16-byte chunks per key row
  constexpr int KPASS = ATT_TK * CPR / ATT_NT;   // chunks copied per thread and tile (each of K, V)
  // two buffer sets as distinct LDS objects: the direct-to-LDS copy of the
  // next tile is then known not to alias the reads of the current one
  __shared__ __attribute__((aligned(16))) uint16_t sK0[ATT_TK * D];
  __shared__ __attribute__((aligned(16))) uint16_t sK1[ATT_TK * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV0[ATT_TK * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV1[ATT_TK * D];
  __shared__ int s_pre[ATT_MAXSEG + 1];
  __shared__ const void* s_k[ATT_MAXSEG];
  __shared__ const void* s_v[ATT_MAXSEG];

  const int G = gridDim.x;
  const int bl = xcd_remap(blockIdx.x, G);   // head-major items, one XCD per range
  const int lane = lane_id(), w = wave_id();
  const int g = lane >> 4;
  const int wu = __builtin_amdgcn_readfirstlane(w);   // the wave index as a uniform value
  const int tid = threadIdx.x;

  // ---- work plan ----
  // Items are (head, 256-query tile), head-major.  Without a partial buffer
  // the grid has one work-group per item.  With one, the grid is one
  // work-group per slot: `rounds` rounds of whole items, then the Ir items
  // left over are balanced over all G work-groups.  Each of those keeps a
  // main piece, key tiles [0, T), in the work-group of its own index (so
  // the work-groups of a head sweep its keys together, as in the plain
  // grid).  The tails [T, n) of the longer items fill slots: first the
  // G - Ir spare work-groups (room T each), then the work-groups whose own
  // item is shorter than T (room T - n), in head order.  A slot takes
  // consecutive tails of one head (the same tail keys, read from L2 after
  // the first), each costing its length plus one tile of start-up.  T is
  // the smallest length at or above the even share for which every tail
  // finds a slot; every work-group derives the same plan from the segment
  // lengths.  Split items leave fp32 partials that attn_merge_kernel adds.
  __shared__ int s_nt[ATT_MAX_HEADS];
  __shared__ int s_T, s_whole;
  const int base = rounds * G;          // first left-over item
  const int h0 = base / nqt;
  // left-over items of head hh: [first_of(hh), (hh + 1) nqt)
  auto first_of = [&](int hh) -> int { return max(hh * nqt, base); };
  // Tail fill for cut tc.  Slot groups in order: g = 0, the spare
  // work-groups; g = 1 + hh, the left-over items of head hh when it is
  // shorter than tc.  Returns whether every tail is placed; with a target
  // slot (tg, tj) also its tails: items [*first, *first + *cnt) of head *th.
  auto fill = [&](int tc, int tg, int tj, int* th, int* first, int* cnt) -> bool {
    int gi = 0, used = 0;
    // (heads before h0 have no left-over item: their groups are empty)
    auto gcount = [&](int g) -> int {
      if (g == 0) return G - Ir;
      const int hh = g - 1;
      return hh >= h0 && s_nt[hh] < tc ? (hh + 1) * nqt - first_of(hh) : 0;
    };
    auto groom = [&](int g) -> int { return g == 0 ? tc : tc - s_nt[g - 1]; };
    for (int hh = h0; hh < H; ++hh) {
      const int r = s_nt[hh] - tc;
      if (r <= 0) continue;
      int rem = (hh + 1) * nqt - first_of(hh), it = first_of(hh);
      while (rem > 0) {
        if (gi > H) return false;
        const int m = gcount(gi) - used;
        const int k = groom(gi) / (r + 1);
        if (m <= 0 || k <= 0) {
          ++gi;
          used = 0;
          continue;
        }
        const int take = min((rem + k - 1) / k, m);
        if (tg == gi && tj >= used && tj < used + take) {
          *th = hh;
          *first = it + (tj - used) * k;
          *cnt = min(k, rem - (tj - used) * k);
          return true;
        }
        const int placed = min(rem, take * k);
        rem -= placed;
        it += placed;
        used += take;
        if (used >= gcount(gi)) {
          ++gi;
          used = 0;
        }
      }
    }
    return tg < 0;
  };
  int T = 0;
  int bli = bl;   // this work-group's left-over item (when below Ir)
  if (Ir > 0) {
    // tiles per head: one wave per head, its lanes reading the segment
    // lengths in parallel
    for (int hh = h0 + wu; hh < H; hh += ATT_NW) {
      const int ns = min(nseg_p[hh], min(seg_cap, ATT_MAXSEG));
      int len = 0;
      for (int sg = lane; sg < ns; sg += 64) len += segs[(int64_t)hh * seg_cap + sg].len;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) len += __shfl_xor(len, o);
      if (lane == 0) s_nt[hh] = (len + ATT_TK - 1) / ATT_TK;
    }
    __syncthreads();
    if (w == 0) {
      int64_t work = 0;
      int ntmax = 0, ntmin = 1 << 30;
      for (int hh = h0; hh < H; ++hh) {
        work += (int64_t)((hh + 1) * nqt - first_of(hh)) * s_nt[hh];
        ntmax = max(ntmax, s_nt[hh]);
        ntmin = min(ntmin, s_nt[hh]);
      }
      // Left-over items of one length that fill at least four fifths of
      // the slots run whole (cut T = the longest item): at the chip's power
      // limit the idle slots cost less than the split's partials, merge and
      // tail re-reads (480P layer-chunk, 228 items on 256 slots: 0.613 ->
      // 0.601 ms).  Items of different lengths are always balanced.
      const bool whole = ntmin == ntmax && 5 * Ir >= 4 * G;
      const int tlo = max(1, (int)((work + G - 1) / G));
      int dh, df, dc;
      const bool ok = !whole && fill(tlo + lane, -1, 0, &dh, &df, &dc);   // candidate cuts, one per lane
      const uint64_t msk = __ballot(ok);
      if (lane == 0) {
        s_T = msk ? tlo + (int)__builtin_ctzll(msk) : ntmax;
        s_whole = whole;
      }
    }
    __syncthreads();
    T = __builtin_amdgcn_readfirstlane(s_T);
    // whole left-over items sit where a grid of one work-group per item
    // puts them: the first Ir dispatches, Ir / 8 per XCD (each XCD's L2
    // then serves as many items as in that grid); the other work-groups
    // have no piece
    if (__builtin_amdgcn_readfirstlane(s_whole)) bli = (int)blockIdx.x < Ir ? xcd_remap(blockIdx.x, Ir) : Ir;
  }

  // per-piece state (set by `piece` below)
  int h = -1, nseg = 0, Lkv = 0, q0 = 0, t_beg = 0, t_end = 0;
  s16x8_t qf[2][NKS];
  f32x4_t o[NDB][2];
  float m_run[2];
  // softmax denominators, accumulated by MFMA from the same bf16 weights as
  // the numerator (ones x P^T: every row of L holds the query's sum)
  f32x4_t L[2];
  const s16x8_t ones = {0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80};

  // Tile addressing.  A tile inside one segment (all but a handful per head)
  // is one base pointer plus the row offset; a tile that straddles segments
  // or the end resolves each row on its own (rows past the end re-read the
  // last row: their scores are masked to -inf, their values get weight 0).
  // The current segment's bounds and bases are kept in scalar registers;
  // the LDS segment table is read only when a tile leaves the segment.
  int ucur = 0, ulo = 0, uhi = -1;
  const void* ubk = nullptr;
  const void* ubv = nullptr;
  // byte offsets (inside a 64-row tile) of the source chunks this lane copies
  // to LDS slots (row, lane % CPR): the same for K and V, fixed for the kernel
  uint32_t koff[KPASS];
#pragma unroll
  for (int i = 0; i < KPASS; ++i) {
    const int sl = (w * KPASS + i) * 64 + lane;
    const int r = sl / CPR, c = sl % CPR;
    koff[i] = (uint32_t)(r * D + (c ^ att_swz<CPR>(r)) * 8) * 2u;
  }
  auto uniform_ptr = [](const void* p) -> const void* {
    // (readfirstlane returns int: widen through uint32_t, never by sign)
    const uint64_t v = (uint64_t)p;
    const uint32_t vh = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    const uint32_t vl = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    return (const void*)(((uint64_t)vh << 32) | (uint64_t)vl);
  };
  auto fetch = [&](int kbase, uint16_t* sKn, uint16_t* sVn) __attribute__((always_inline)) {
    if (kbase < ulo || kbase + ATT_TK > uhi) {
      if (kbase < ulo) ucur = 0;   // a new pass over the tiles
      while (ucur + 1 < nseg && __builtin_amdgcn_readfirstlane(s_pre[ucur + 1]) <= kbase) ++ucur;
      ulo = __builtin_amdgcn_readfirstlane(s_pre[ucur]);
      uhi = __builtin_amdgcn_readfirstlane(s_pre[ucur + 1]);
      ubk = uniform_ptr(s_k[ucur]);
      ubv = uniform_ptr(s_v[ucur]);
    }
    if (kbase + ATT_TK <= uhi) {
      // whole tile inside one segment: buffer resources on the segment
      // (uniform base, per-lane offsets fixed for the kernel)
      const int nbytes = (uhi - ulo) * D * 2;
      const i32x4_t rk = buf_rsrc(ubk, nbytes), rvs = buf_rsrc(ubv, nbytes);
      const int soff = (kbase - ulo) * D * 2;
#pragma unroll
      for (int i = 0; i < KPASS; ++i) {
        lds_copy_buf(rk, koff[i], soff, lds_addr(sKn + (wu * KPASS + i) * 64 * 8));
        lds_copy_buf(rvs, koff[i], soff, lds_addr(sVn + (wu * KPASS + i) * 64 * 8));
      }
    } else {
      // each row finds its segment from the tile's first one (ucur holds
      // kbase) on, once for its K and V rows
#pragma unroll
      for (int i = 0; i < KPASS; ++i) {
        const int sl = (wu * KPASS + i) * 64 + lane;
        const int r = sl / CPR, c = sl % CPR;
        const int j = min(kbase + r, Lkv - 1);
        int sg = ucur;
        while (sg + 1 < nseg && s_pre[sg + 1] <= j) ++sg;
        const int64_t ro = (int64_t)(j - s_pre[sg]) * D + (c ^ att_swz<CPR>(r)) * 8;
        lds_copy_glb((const uint16_t*)s_k[sg] + ro, lds_addr(sKn + (wu * KPASS + i) * 64 * 8));
        lds_copy_glb((const uint16_t*)s_v[sg] + ro, lds_addr(sVn + (wu * KPASS + i) * 64 * 8));
      }
    }
  };

  // element offsets of this lane's K fragments (row 16kb + (lane & 15) of a
  // tile, chunk 4k + g): the swizzle of row 16kb + x equals that of x
  int kread[NKS];
#pragma unroll
  for (int k = 0; k < NKS; ++k) {
    const int r = lane & 15;
    kread[k] = r * D + (((4 * k + g) ^ att_swz<CPR>(r)) * 8);
  }
  // element offsets of this lane's 8-byte V pieces for the transposing reads:
  // lane 16G + a reads row 4G + (a >> 2) (+ 32 hk, + 16 for the upper half),
  // d = 16 db + 4 (a & 3) .. + 3; the read then hands lane 16G + i the values
  // V[4G + j][16 db + i], j = 0..3 (the A operand of O^T = V^T P^T)
  int vread[NDB];
  {
    const int a = lane & 15;
    const int r = 4 * g + (a >> 2);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      vread[db] = r * D + (((2 * db + ((a & 3) >> 1)) ^ att_swz<CPR>(r)) * 8) + (a & 1) * 4;
  }

  // Softmax modes of one tile.  FIRST: the tile's maximum becomes the
  // query's reference m (first tile of the fast pass).  FAST: weights
  // 2^(s c - m) against that fixed reference, no maximum taken: exact
  // whenever they stay finite (fp32 and bf16 reach 2^127), which the pass
  // checks at the end.  SAFE: the reference follows the running maximum,
  // moved only when a tile raises it by more than 2^8 (numerator and
  // denominator are rescaled together).  IDLE: a wave whose queries all
  // lie past Lq only copies its share of the next tile and meets the
  // barrier.
  constexpr int FIRST = 0, FAST = 1, SAFE = 2, IDLE = 3;
  auto step = [&](auto mode_c, int tile, const uint16_t* sKc, const uint16_t* sVc, uint16_t* sKn,
                  uint16_t* sVn) __attribute__((always_inline)) {
    constexpr int mode = decltype(mode_c)::value;
    const int kbase = tile * ATT_TK;
    const bool more = tile + 1 < t_end;
    if (more) fetch(kbase + ATT_TK, sKn, sVn);
    if constexpr (mode == IDLE) {
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      return;
    }

    // ---- S^T = K Q^T ----
    // MFMA issue at raised wave priority: the SIMD's other wave, between its
    // own products, then gets the vector ALU for its softmax.  Fragments of
    // key block kb + 2 are read while block kb is multiplied.
    __builtin_amdgcn_s_setprio(1);
    f32x4_t s[4][2];
    s16x8_t kf[2][NKS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int k = 0; k < NKS; ++k) kf[kb][k] = Op::load(sKc + 16 * kb * D + kread[k]);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      s[kb][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < NKS; ++k) {
        s[kb][0] = Op::mma16(kf[kb & 1][k], qf[0][k], s[kb][0]);
        s[kb][1] = Op::mma16(kf[kb & 1][k], qf[1][k], s[kb][1]);
      }
      if (kb + 2 < 4) {
#pragma unroll
        for (int k = 0; k < NKS; ++k) kf[kb & 1][k] = Op::load(sKc + 16 * (kb + 2) * D + kread[k]);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * NKS, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * NKS, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, NKS, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * NKS, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, NKS, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * NKS, 0);
    __builtin_amdgcn_s_setprio(0);
    // ---- softmax (log2 domain), lane owns query 16qb + (lane & 15) ----
    if (kbase + ATT_TK > Lkv) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kbase + 16 * kb + 4 * g + i >= Lkv) { s[kb][0][i] = -__builtin_inff(); s[kb][1][i] = -__builtin_inff(); }
    }
    if constexpr (mode != FAST) {
      float mt[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float mx = s[0][qb][0];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kb][qb][i]);
        const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
        const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
        mt[qb] = mx * scale_log2;
      }
      if constexpr (mode == FIRST) {
        m_run[0] = mt[0];
        m_run[1] = mt[1];
      } else {
        const bool grow = (mt[0] > m_run[0] + ATT_RESCALE_LOG2) || (mt[1] > m_run[1] + ATT_RESCALE_LOG2);
        if (__any(grow)) {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            const float mnew = fmaxf(m_run[qb], mt[qb]);
            const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - mnew);
            m_run[qb] = mnew;
            L[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) o[db][qb] *= alpha;
          }
        }
      }
    }
    uint32_t pk[2][4][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float nm = -m_run[qb];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][i], scale_log2, nm));
        pk[qb][kb][0] = pack_bf16x2(p[0], p[1]);
        pk[qb][kb][1] = pack_bf16x2(p[2], p[3]);
      }
    }
    // ---- O^T += V^T P^T ----
    // B operand element j of lane 16G + i: key 32hk + 4G + j (j < 4) or
    // 32hk + 16 + 4G + (j - 4); the transposing V reads follow that order
#pragma unroll
    for (int hk = 0; hk < 2; ++hk) {
      u32x4_t b0 = {pk[0][2 * hk][0], pk[0][2 * hk][1], pk[0][2 * hk + 1][0], pk[0][2 * hk + 1][1]};
      u32x4_t b1 = {pk[1][2 * hk][0], pk[1][2 * hk][1], pk[1][2 * hk + 1][0], pk[1][2 * hk + 1][1]};
      const s16x8_t bb0 = __builtin_bit_cast(s16x8_t, b0);
      const s16x8_t bb1 = __builtin_bit_cast(s16x8_t, b1);
      L[0] = Op::mma16(ones, bb0, L[0]);
      L[1] = Op::mma16(ones, bb1, L[1]);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint16_t* vp = sVc + 32 * hk * D + vread[db];
        const s16x4_t lo = lds_tr16(vp);
        const s16x4_t hi = lds_tr16(vp + 16 * D);
        const s16x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[db][0] = Op::mma16(a, bb0, o[db][0]);
        o[db][1] = Op::mma16(a, bb1, o[db][1]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // next K and V tiles resident in LDS
    __syncthreads();
  };
  auto reset = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) o[db][qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run[0] = m_run[1] = -__builtin_inff();
    L[0] = L[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (t_beg < t_end) fetch(t_beg * ATT_TK, sK0, sV0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  };

  // One piece: key tiles [t0, t1) of item (head, query tile).  slot < 0:
  // the whole item, normalised into O; slot 0 / 1: the main piece / the
  // tail of left-over item ir, stored unnormalised with its reference and
  // denominator.  flag: the main piece (or whole left-over item) records
  // whether the item was split.
  auto piece = [&](int item, int t0, int t1, int slot, int ir) __attribute__((always_inline)) {
    const int hn = item / nqt, qt = item % nqt;
    if (hn != h) {
      // every wave's last table read came before the previous barrier.
      // Wave 0 reads the head's table 64 entries at a time (one load
      // latency, not one per segment) and scans the lengths into offsets.
      h = hn;
      nseg = min(nseg_p[h], min(seg_cap, ATT_MAXSEG));
      if (w == 0) {
        int carry = 0;
        for (int s0 = 0; s0 < nseg; s0 += 64) {
          const int sg = s0 + lane;
          int len = 0;
          if (sg < nseg) {
            const SegEntry e = segs[(int64_t)h * seg_cap + sg];
            s_k[sg] = e.k;
            s_v[sg] = e.v;
            len = e.len;
          }
          int x = len;   // inclusive scan over the wave
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o);
            if (lane >= o) x += y;
          }
          if (sg < nseg) s_pre[sg] = carry + x - len;
          carry += __shfl(x, 63);
        }
        if (lane == 0) s_pre[nseg] = carry;
      }
      __syncthreads();
      Lkv = __builtin_amdgcn_readfirstlane(s_pre[nseg]);
    }
    ucur = 0;
    ulo = 0;
    uhi = -1;   // the next fetch seeks its segment
    const int ntile = (Lkv + ATT_TK - 1) / ATT_TK;
    t_beg = t0;
    t_end = min(t1, ntile);

    // query fragments (B operand of S^T = K Q^T)
    q0 = qt * ATT_QB + w * ATT_QW;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int q = q0 + 16 * qb + (lane & 15);
      const uint16_t* qp = Q + ((int64_t)h * Lq + (q < Lq ? q : 0)) * D;
#pragma unroll
      for (int k = 0; k < NKS; ++k) {
        if (q < Lq) qf[qb][k] = Op::load(qp + Op::off16(k, lane));
        else qf[qb][k] = s16x8_t{};
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): query fragments resident before the tiles

    // fast pass (tile t in buffer set (t - t0) & 1).  A wave with no query
    // below Lq (the padding of a head's last query tile) takes the same
    // barriers and its share of the copies, in a loop of its own: the chip
    // holds this kernel at its power limit, and the skipped products leave
    // that power to the work that counts (480P layer-chunk: 0.608 -> 0.602 ms).
    auto fast_pass = [&](auto first_c, auto fast_c) __attribute__((always_inline)) {
      reset();
      if (t_beg < t_end) step(first_c, t_beg, sK0, sV0, sK1, sV1);
      for (int tile = t_beg + 1; tile < t_end; tile += 2) {
        step(fast_c, tile, sK1, sV1, sK0, sV0);
        if (tile + 1 < t_end) step(fast_c, tile + 1, sK0, sV0, sK1, sV1);
      }
    };
    auto safe_pass = [&](auto safe_c) __attribute__((always_inline)) {
      reset();
      for (int tile = t_beg; tile < t_end; tile += 2) {
        step(safe_c, tile, sK0, sV0, sK1, sV1);
        if (tile + 1 < t_end) step(safe_c, tile + 1, sK1, sV1, sK0, sV0);
      }
    };
    const bool idle = qt * ATT_QB + wu * ATT_QW >= Lq;   // (wu: the wave index as a uniform value)
    if (idle) fast_pass(std::integral_constant<int, IDLE>{}, std::integral_constant<int, IDLE>{});
    else fast_pass(std::integral_constant<int, FIRST>{}, std::integral_constant<int, FAST>{});
    // a non-finite numerator or denominator anywhere in the work-group (a
    // query whose scores rose by about 2^127 past its first tile's): redo the
    // piece's tiles with the running-maximum pass (an idle wave's sums are
    // the zeros of reset)
    float chk = L[0][0] + L[1][0];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) chk += (o[db][qb][0] + o[db][qb][1]) + (o[db][qb][2] + o[db][qb][3]);
    if (__syncthreads_or(!__builtin_isfinite(chk))) {
      if (idle) safe_pass(std::integral_constant<int, IDLE>{});
      else safe_pass(std::integral_constant<int, SAFE>{});
    }

    if (slot >= 0) {
      // ---- partial: lane's o (NDB x 2 vectors), then {m0, m1, L0, L1} ----
      f32x4_t* pp = part + (((int64_t)ir * 2 + slot) * ATT_NW + w) * (2 * NDB + 1) * 64 + lane;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) pp[(2 * db + qb) * 64] = o[db][qb];
      pp[2 * NDB * 64] = f32x4_t{m_run[0], m_run[1], L[0][0], L[1][0]};
      if (slot == 0 && tid == 0) pflag[ir] = 1;
      return;
    }
    if (ir >= 0 && tid == 0) pflag[ir] = 0;
    // ---- normalise and store: lane holds O[q][16db + 4g + i] ----
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float l = L[qb][0];
      const float inv = l > 0.f ? 1.0f / l : 0.0f;
      const int q = q0 + 16 * qb + (lane & 15);
      if (q < Lq) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          attn_store(O, out_f32, ((int64_t)h * Lq + q) * D + 16 * db + 4 * g, o[db][qb], inv);
      }
    }
  };

  // this work-group's tail range: items [tl_first, tl_first + tl_cnt) of
  // one head, key tiles [T, tl_nt)
  int tl_first = 0, tl_cnt = 0, tl_nt = 0;
  if (Ir > 0) {
    int tg = -1, tj = 0;
    if (bli >= Ir) {
      tg = 0;
      tj = bli - Ir;
    } else {
      const int hh = (base + bli) / nqt;
      if (s_nt[hh] < T) {
        tg = 1 + hh;
        tj = base + bli - first_of(hh);
      }
    }
    int th = 0;
    if (tg >= 0 && fill(T, tg, tj, &th, &tl_first, &tl_cnt)) tl_nt = s_nt[th];
    else tl_cnt = 0;
  }
  // pieces in order: whole items of each round, then the main piece (or the
  // whole left-over item), then the tails; one call site keeps one copy of
  // the tile loop
  const int npieces = rounds + (Ir > 0 ? (bli < Ir ? 1 : 0) + tl_cnt : 0);
  for (int pc = 0; pc < npieces; ++pc) {
    int item, t0 = 0, t1 = 1 << 30, slot = -1, ir = -1;
    const int pt = pc - rounds - (bli < Ir ? 1 : 0);   // tail index (when >= 0)
    if (pc < rounds) {
      item = pc * G + bl;
    } else if (pt < 0) {
      item = base + bli;
      ir = bli;
      const int nt = s_nt[item / nqt];
      if (nt > T) {
        t1 = T;
        slot = 0;
      }
    } else {
      item = tl_first + pt;
      ir = item - base;
      t0 = T;
      t1 = tl_nt;
      slot = 1;
    }
    piece(item, t0, t1, slot, ir);
  }
}

// Merge of the two pieces of a split item: weights against the larger of
// the two references, o = (o0 a0 + o1 a1) / (L0 a0 + L1 a1).  One
// work-group per left-over item, lanes laid out as in attn_bf16_kernel.
template <int D>
__global__ __launch_bounds__(ATT_NT) void attn_merge_kernel(void* __restrict__ O, const f32x4_t* __restrict__ part,
                                                         const int32_t* __restrict__ pflag, int base, int nqt,
                                                         int Lq, int out_f32) {
  constexpr int NDB = D / 16;
  const int ir = blockIdx.x;
  if (pflag[ir] == 0) return;
  const int item = base + ir, h = item / nqt, qt = item % nqt;
  const int lane = lane_id(), w = wave_id(), g = lane >> 4;
  const f32x4_t* p0 = part + (((int64_t)ir * 2 + 0) * ATT_NW + w) * (2 * NDB + 1) * 64 + lane;
  const f32x4_t* p1 = p0 + ATT_NW * (2 * NDB + 1) * 64;
  const f32x4_t s0 = p0[2 * NDB * 64], s1 = p1[2 * NDB * 64];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float m0 = s0[qb], m1 = s1[qb];
    const float mx = fmaxf(m0, m1);
    const float a0 = mx == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m0 - mx);
    const float a1 = mx == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m1 - mx);
    const float l = s0[2 + qb] * a0 + s1[2 + qb] * a1;
    const float inv = l > 0.f ? 1.0f / l : 0.0f;
    const int q = qt * ATT_QB + w * ATT_QW + 16 * qb + (lane & 15);
    if (q < Lq) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const f32x4_t v0 = p0[(2 * db + qb) * 64], v1 = p1[(2 * db + qb) * 64];
        const f32x4_t v = {v0[0] * a0 + v1[0] * a1, v0[1] * a0 + v1[1] * a1, v0[2] * a0 + v1[2] * a1,
                           v0[3] * a0 + v1[3] * a1};
        attn_store(O, out_f32, ((int64_t)h * Lq + q) * D + 16 * db + 4 * g, v, inv);
      }
    }
  }
}

// fp32 path (small shapes): one thread per (head, query), online softmax
template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(const float* __restrict__ Q, float* __restrict__ O,
                                                      const SegEntry* __restrict__ segs,
                                                      const int32_t* __restrict__ nseg_p, int seg_cap, int Lq,
                                                      float scale) {
  const int h = blockIdx.y;
  const int q = blockIdx.x * 64 + threadIdx.x;
  if (q >= Lq) return;
  const float* qp = Q + ((int64_t)h * Lq + q) * D;
  float qv[D];
#pragma unroll
  for (int i = 0; i < D; ++i) qv[i] = qp[i];
  float acc[D];
#pragma unroll
  for (int i = 0; i < D; ++i) acc[i] = 0.f;
  float m = -__builtin_inff(), l = 0.f;
  const int ns = min(nseg_p[h], seg_cap);
  for (int s = 0; s < ns; ++s) {
    const SegEntry e = segs[(int64_t)h * seg_cap + s];
    const float* kp = (const float*)e.k;
    const float* vp = (const float*)e.v;
    for (int j = 0; j < e.len; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < D; ++i) dot = __builtin_fmaf(qv[i], kp[(int64_t)j * D + i], dot);
      dot *= scale;
      const float mn = fmaxf(m, dot);
      const float a = expf(m - mn);
      const float p = expf(dot - mn);
      l = l * a + p;
#pragma unroll
      for (int i = 0; i < D; ++i) acc[i] = __builtin_fmaf(p, vp[(int64_t)j * D + i], acc[i] * a);
      m = mn;
    }
  }
  const float inv = l > 0.f ? 1.0f / l : 0.0f;
  float* op = O + ((int64_t)h * Lq + q) * D;
#pragma unroll
  for (int i = 0; i < D; ++i) op[i] = acc[i] * inv;
}

// Balanced-grid plan of a bf16 launch: G work-groups (one per slot, two per
// compute unit at the kernel's register use), `rounds` rounds of whole
// items, Ir left-over items whose partials need `bytes` of workspace; `use`
// says whether the balanced grid is taken at all.
AttnPlan attention_plan(int H, int d, int Lq, int et) {
  AttnPlan p{};
  if (et != ET_BF16 || Lq <= 0 || H <= 0) return p;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  const int items = ((Lq + ATT_QB - 1) / ATT_QB) * H;
  p.G = (8 / ATT_NW) * cus;    // two waves per SIMD
  p.rounds = items / p.G;
  p.Ir = items % p.G;
  // Balance whenever a round is left over.  The work-groups derive the split
  // from the segment lengths on the device, so heads of different lengths
  // (static and dynamic Forcing-KV heads) are balanced too, and a plan that
  // gains nothing falls back to whole items (T = the longest item).  Measured:
  // equal time on the 480P layer (228 items on 256 slots) and on 1080P, 9 %
  // faster on the hybrid 480P layer (7,800- and 18,720-key heads).
  if (p.Ir == 0) {
    p.use = false;
    return p;
  }
  p.use = true;
  const int64_t per_item = 2LL * ATT_NW * (2 * (d / 16) + 1) * 64 * 16;   // two pieces, every wave, float4 per lane
  p.flag_bytes = ((int64_t)p.Ir * 4 + 255) / 256 * 256;
  p.bytes = p.flag_bytes + p.Ir * per_item;
  return p;
}

hipError_t launch_attention(const AttnLaunch& a, hipStream_t st) {
  if (a.Lq <= 0 || a.H <= 0) return hipSuccess;
  if (a.et == ET_BF16) {
    const float sl2 = a.scale * 1.4426950408889634f;
    const int nqt = (a.Lq + ATT_QB - 1) / ATT_QB;
    const int items = nqt * a.H;
    // balanced grid when a workspace is given (and there is a round to fill)
    AttnPlan p = attention_plan(a.H, a.d, a.Lq, a.et);
    const bool bal = p.use && a.ws != nullptr && a.ws_bytes >= (size_t)p.bytes;
    int G = items, rounds = 1, Ir = 0;
    int32_t* flag = nullptr;
    f32x4_t* part = nullptr;
    if (bal) {
      G = p.G;
      rounds = p.rounds;
      Ir = p.Ir;
      if (Ir > 0) {
        flag = (int32_t*)a.ws;
        part = (f32x4_t*)((char*)a.ws + p.flag_bytes);
      }
    }
    if (a.d == 128)
      hipLaunchKernelGGL((attn_bf16_kernel<128>), dim3((unsigned)G), dim3(ATT_NT), 0, st, (const uint16_t*)a.Q, a.O,
                         a.segs, a.nseg, a.seg_cap, a.Lq, sl2, a.out_f32, nqt, a.H, rounds, Ir, part, flag);
    else
      hipLaunchKernelGGL((attn_bf16_kernel<64>), dim3((unsigned)G), dim3(ATT_NT), 0, st, (const uint16_t*)a.Q, a.O,
                         a.segs, a.nseg, a.seg_cap, a.Lq, sl2, a.out_f32, nqt, a.H, rounds, Ir, part, flag);
    if (Ir > 0) {
      if (a.d == 128)
        hipLaunchKernelGGL((attn_merge_kernel<128>), dim3((unsigned)Ir), dim3(ATT_NT), 0, st, a.O, part, flag,
                           rounds * G, nqt, a.Lq, a.out_f32);
      else
        hipLaunchKernelGGL((attn_merge_kernel<64>), dim3((unsigned)Ir), dim3(ATT_NT), 0, st, a.O, part, flag,
                           rounds * G, nqt, a.Lq, a.out_f32);
    }
  } else {
    const dim3 grid((unsigned)((a.Lq + 63) / 64), (unsigned)a.H);
    if (a.d == 128)
      hipLaunchKernelGGL((attn_f32_kernel<128>), grid, dim3(64), 0, st, (const float*)a.Q, (float*)a.O, a.segs,
                         a.nseg, a.seg_cap, a.Lq, a.scale);
    else
      hipLaunchKernelGGL((attn_f32_kernel<64>), grid, dim3(64), 0, st, (const float*)a.Q, (float*)a.O, a.segs,
                         a.nseg, a.seg_cap, a.Lq, a.scale);
  }
  return hipGetLastError();
}

}  // namespace kvb
