// Gram-based Soft-Riesz kernels: key norms, fused pairwise-interaction row
// sums (disturbance and density fix-ups) and the ordered crossing scan.
//
// DensityKV paper-summary page, Method ("Soft-Riesz Density", "Online
// Density-Constrained Bank Update") and appendix B.1: the interaction of two
// post-RoPE keys is a softened inverse power of their squared distance; the
// exact update touches bank x candidate pairs, admitted x evicted pairs and
// admitted x admitted pairs.
//
// Squared distances come from 32x32 MFMA dot products with fp32
// accumulation.  One extra k-step multiplies the column key's squared norm
// (split exactly into three bf16 parts) by -1/2, so the MFMA returns
// R = x.y - |y|^2/2 and the softened distance is
//   t = eps + |x - y|^2 / sigma^2 = fma(R, -2/sigma^2, |x|^2/sigma^2 + eps),
// leaving fma, max, the reciprocal/power and one add per pair on the VALU.
#include "kvb_common.hpp"
#include "kvb_launch.hpp"

namespace kvb {

// Norm augmentation.  Every key row carries a 16-byte augmentation row
// written by norms_kernel:
//   bf16 keys: (h, m, l, -1/2, -1/2, -1/2, 0, 0), |k|^2 = h + m + l exactly
//              (three bf16 parts), used as the y side of one extra k-step;
//   fp32 keys: (|k|^2, -1/2, 0, 0).
// The x side of that k-step is built in registers from the x row's own
// augmentation: (-1/2, -1/2, -1/2, xh, xm, xl, 0, 0) (bf16) or -1/2 / |x|^2
// (fp32, one element per k-slice), so the MFMA accumulates
//   R = x.y - |x|^2/2 - |y|^2/2 = -|x - y|^2 / 2.
template <typename E> struct Aug;
template <> struct Aug<uint16_t> {
  KVB_DEV static s16x8_t xfrag(u32x4_t a, int lane) {
    if (lane >> 5) return s16x8_t{};
    const u32x4_t r = {0xBF00BF00u, 0xBF00u | (a[0] << 16), (a[0] >> 16) | (a[1] << 16), 0u};
    return __builtin_bit_cast(s16x8_t, r);
  }
  // y side: the stored row (the upper k-slice pairs with zeros on the x side)
  KVB_DEV static s16x8_t yfrag(const u32x4_t& a, int) { return __builtin_bit_cast(s16x8_t, a); }
  // direct form: stored rows are (h', m', l', 1, 1, 1, 1, 1) with h' + m' + l'
  // = |k|^2 / sigma^2; the x side is (1, 1, 1, xh', xm', xl', eh, em) and, in
  // the upper k-slice, eps's third part against the last 1, so the norm step
  // adds |y|^2/sigma^2 + |x|^2/sigma^2 + eps exactly
  KVB_DEV static s16x8_t xfrag_direct(u32x4_t a, int lane, u32x4_t e) {
    const u32x4_t r = (lane >> 5) ? u32x4_t{0u, 0u, 0u, e[2] << 16}
                                  : u32x4_t{0x3F803F80u, 0x3F80u | (a[0] << 16), (a[0] >> 16) | (a[1] << 16),
                                            e[0] | (e[1] << 16)};
    return __builtin_bit_cast(s16x8_t, r);
  }
  // bf16 parts (hi, mid, lo) of eps, exact for any float
  KVB_DEV static u32x4_t eps_parts(float eps) {
    const uint16_t hi = f32_to_bf16(eps);
    const float r1 = eps - bf16_to_f32(hi);
    const uint16_t mid = f32_to_bf16(r1);
    const uint16_t lo = f32_to_bf16(r1 - bf16_to_f32(mid));
    return u32x4_t{hi, mid, lo, 0u};
  }
  // x * s for a power of two s: exact in bf16 (keys are far from the
  // exponent limits)
  KVB_DEV static s16x8_t scale(s16x8_t x, float sc) {
    s16x8_t r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (short)f32_to_bf16(bf16_to_f32((uint16_t)x[j]) * sc);
    return r;
  }
};
template <> struct Aug<float> {
  KVB_DEV static float xfrag(u32x4_t a, int lane) { return (lane >> 5) ? __uint_as_float(a[0]) : -0.5f; }
  KVB_DEV static float yfrag(const u32x4_t& a, int lane) { return __uint_as_float((lane >> 5) ? a[1] : a[0]); }
};

template <bool B> struct BoolTag { static constexpr bool value = B; };

// 256-wide bf16 rows (the [K; V] descriptors of d = 128 heads): a 512-byte
// row spans the 64 LDS banks twice, so the chunk swizzle r & 7 (8 rows on 8
// distinct 16-byte bank groups) repeats every 8 rows
template <> struct Tile<uint16_t, 256> {
  static constexpr int EPC = 8;
  static constexpr int CPR = 32;
  KVB_DEV static int swz(int r) { return r & 7; }
  KVB_DEV static int at(int r, int e) { return r * 256 + (((e / EPC) ^ swz(r)) * EPC) + e % EPC; }
  // (as in the general tile: the chunk bits of f and e are disjoint)
  KVB_DEV static int at_step(int a0, int f) { return a0 ^ f; }
};
// rows after which Tile<E, D>'s swizzle repeats
template <typename E, int D> constexpr int swz_period() {
  if constexpr (sizeof(E) != 2) return 1;
  else if constexpr (D == 256) return 8;
  else return 16;
}

// Stages TC key rows (gathered by virtual index) and their augmentation rows
// into LDS with direct-to-LDS loads.  NT threads in NW waves; copy i of wave
// w fills tile rows (i NW + w) RPI .. + RPI - 1 (one contiguous KiB of LDS),
// lane l taking row + l / CPR and LDS chunk l % CPR.  The rows of one lane
// differ by multiples of NW RPI, a multiple of the swizzle's period, so the
// lane's source chunk offset is the same for every copy.  Wave 0 copies the
// augmentation rows and records each row's index (-1 when absent) in sV
// when given.
//
// Indices come in two steps so that reading an index list never stalls the
// copies in flight: index() keeps the raw list entries of a tile (plain
// loads, nothing computed from them), issue() turns them into row indices
// one tile later.  raw(c) reads list position c (clamped by the caller);
// fix(c, raw) returns the virtual row index of position c or -1.  Absent
// rows copy row `fb` (any existing row).
template <typename E, int D, int TC, int NT = 256>
struct DmaTile {
  using T = Tile<E, D>;
  static constexpr int NW = NT / 64;
  static constexpr int RPI = 64 / T::CPR;           // rows per copy
  static constexpr int PASSW = TC / (RPI * NW);     // copies per wave and tile
  static_assert(TC == 64 && PASSW * RPI * NW == TC, "tile shape");
  static_assert((NW * RPI) % swz_period<E, D>() == 0, "the swizzle must repeat across a lane's copies");
  int vi[PASSW];
  int va;
  // Per-lane offsets are recomputed from an opaque lane id at each use: kept
  // live across the loop they would cost registers the MFMA loop needs.
  template <typename F>
  KVB_DEV void index(int tile, F raw) {
    const unsigned lane = (unsigned)opaque_i(lane_id());
    const int w = __builtin_amdgcn_readfirstlane(wave_id());
    const int r0 = (int)(lane / T::CPR);
#pragma unroll
    for (int i = 0; i < PASSW; ++i) vi[i] = raw(tile * TC + (i * NW + w) * RPI + r0);
    va = w == 0 ? raw(tile * TC + (int)lane) : 0;
  }
  template <typename G>
  KVB_DEV void issue(int tile, G fix, const HeadKeys<E, D>& hk, E* sY, u32x4_t* sA, int* sV, int fb) const {
    const unsigned lane = (unsigned)opaque_i(lane_id());
    const int w = __builtin_amdgcn_readfirstlane(wave_id());
    const int r0 = (int)(lane / T::CPR), c = (int)(lane % T::CPR);
    const int eoff = (c ^ T::swz(w * RPI + r0)) * T::EPC;
#pragma unroll
    for (int i = 0; i < PASSW; ++i) {
      const int r = (i * NW + w) * RPI + r0;
      const int v = fix(tile * TC + r, vi[i]);
      dma16(hk.row(v >= 0 ? v : fb) + eoff, sY + (i * NW + w) * RPI * D);
    }
    if (w == 0) {
      const int v = fix(tile * TC + (int)lane, va);
      if (sV != nullptr) sV[lane] = v;
      dma16(hk.aug(v >= 0 ? v : fb), sA);
    }
  }
};

// ---------------------------------------------------------------------------
// squared norms: one group of CPR lanes per row, 16-byte chunks
// ---------------------------------------------------------------------------
// With a status word, a live row of a checked head (bit h of chk) whose
// squared norm is not finite sets DEV_NONFINITE: every row of the second set
// is live, and row b of the first set's head h is live when b < the clamped
// count cntA[h] (rowsA rows per head).
template <typename E, int CPR>
__global__ __launch_bounds__(256) void norms_kernel(const E* __restrict__ keysA, int64_t nA, float* __restrict__ outA,
                                                    u32x4_t* __restrict__ augA, const E* __restrict__ keysB,
                                                    int64_t nB, float* __restrict__ outB, u32x4_t* __restrict__ augB,
                                                    int d, float scale, int direct, NormCheck chk) {
  constexpr int EPC = 16 / sizeof(E);
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t row = gid / CPR;
  const int c = (int)(gid % CPR);
  // rows [0, nA) from the first key set, then [nA, nA + nB) from the second
  const bool first = row < nA;
  const E* keys = first ? keysA : keysB;
  float* out = first ? outA : outB;
  u32x4_t* aug = first ? augA : augB;
  if (!first) row -= nA;
  const int64_t nrows = first ? nA : nB;
  float s = 0.0f;
  if (row < nrows) {
    const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(keys + row * d + c * EPC);
    const E* e = reinterpret_cast<const E*>(&raw);
#pragma unroll
    for (int j = 0; j < EPC; ++j) {
      const float x = Ops<E>::to_f32(e[j]);
      s = __builtin_fmaf(x, x, s);
    }
  }
#pragma unroll
  for (int o = CPR / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  if (row < nrows && c == 0) {
    if (chk.status != nullptr && !isfinite(s)) {
      const int rph = first ? chk.rowsA : chk.rowsB;
      const int h = (int)(row / rph), b = (int)(row % rph);
      bool live = head_on(chk.active, h);
      if (live && first) live = b < min(max(chk.cntA[h], 0), rph);
      if (live) atomicOr(chk.status, DEV_NONFINITE);
    }
    out[row] = s * scale;
    u32x4_t a = {0u, 0u, 0u, 0u};
    if constexpr (sizeof(E) == 2) {
      const float q = direct ? s * scale : s;       // scale is a power of two in the direct form
      const uint16_t hi = f32_to_bf16(q);
      const float r1 = q - bf16_to_f32(hi);
      const uint16_t mid = f32_to_bf16(r1);
      const uint16_t lo = f32_to_bf16(r1 - bf16_to_f32(mid));
      a[0] = (uint32_t)hi | ((uint32_t)mid << 16);
      if (direct) {
        a[1] = (uint32_t)lo | (0x3F80u << 16);    // bf16(1)
        a[2] = 0x3F803F80u;
        a[3] = 0x3F803F80u;
      } else {
        a[1] = (uint32_t)lo | (0xBF00u << 16);    // bf16(-1/2)
        a[2] = 0xBF00BF00u;
      }
    } else {
      a[0] = __float_as_uint(s);
      a[1] = __float_as_uint(-0.5f);
    }
    aug[row] = a;
  }
}

hipError_t launch_norms(const void* keysA, int rowsA, float* outA, void* augA, const void* keysB, int rowsB,
                        float* outB, void* augB, int et, int H, int d, float scale, bool direct, hipStream_t st,
                        NormCheck chk) {
  const int64_t nA = keysA ? (int64_t)H * rowsA : 0, nB = keysB ? (int64_t)H * rowsB : 0;
  if (nA + nB == 0) return hipSuccess;
  chk.rowsA = rowsA > 0 ? rowsA : 1;
  chk.rowsB = rowsB > 0 ? rowsB : 1;
  if (chk.cntA == nullptr) chk.status = nullptr;
  const int esz = et == ET_BF16 ? 2 : 4;
  const int cpr = d * esz / 16;
  const dim3 grid((unsigned)(((nA + nB) * cpr + 255) / 256));
  if (et == ET_BF16) {
    const uint16_t* a = (const uint16_t*)keysA;
    const uint16_t* b = (const uint16_t*)keysB;
    if (cpr == 8)
      hipLaunchKernelGGL((norms_kernel<uint16_t, 8>), grid, dim3(256), 0, st, a, nA, outA, (u32x4_t*)augA, b, nB, outB,
                         (u32x4_t*)augB, d, scale, (int)direct, chk);
    else if (cpr == 32)
      hipLaunchKernelGGL((norms_kernel<uint16_t, 32>), grid, dim3(256), 0, st, a, nA, outA, (u32x4_t*)augA, b, nB,
                         outB, (u32x4_t*)augB, d, scale, (int)direct, chk);
    else
      hipLaunchKernelGGL((norms_kernel<uint16_t, 16>), grid, dim3(256), 0, st, a, nA, outA, (u32x4_t*)augA, b, nB, outB,
                         (u32x4_t*)augB, d, scale, (int)direct, chk);
  } else {
    const float* a = (const float*)keysA;
    const float* b = (const float*)keysB;
    if (cpr == 16)
      hipLaunchKernelGGL((norms_kernel<float, 16>), grid, dim3(256), 0, st, a, nA, outA, (u32x4_t*)augA, b, nB, outB,
                         (u32x4_t*)augB, d, scale, 0, chk);
    else
      hipLaunchKernelGGL((norms_kernel<float, 32>), grid, dim3(256), 0, st, a, nA, outA, (u32x4_t*)augA, b, nB, outB,
                         (u32x4_t*)augB, d, scale, 0, chk);
  }
  return hipGetLastError();
}


// ---------------------------------------------------------------------------
// gram row sums: out[i] = sum_{j in cols} phi(row_i, col_j).
// Work-group: 8 waves x 32 rows (A operand in registers, at most 128 VGPRs
// so that four waves share each SIMD); column tiles of 64 (two 32-column
// subtiles, B operand) staged through LDS, double buffered.  The two
// subtiles' MFMA chains are independent, so the interactions of one overlap
// the products of the other.  Lane (h = lane>>5, n = lane&31) accumulates
// rows 8(i>>2) + 4h + (i&3) against column n; a final butterfly over n sums
// the columns.
// ---------------------------------------------------------------------------
constexpr int GRAM_NT = 512;      // threads per work-group
constexpr int GRAM_ROWS = 256;    // rows per work-group (32 per wave)
// The admitted x admitted variant (self-excluding index list) keeps the
// column-sum terms live besides the row sums: more registers than four waves
// per SIMD leave, so it runs four-wave work-groups of 128 rows, three waves
// per SIMD.
constexpr int SYM_NT = 256;
static_assert(SYM_NT / 2 == GRAM_ROW_BLOCK, "rows per work-group of the symmetric self-Gram");
template <bool SELF, bool CLIST> constexpr int gram_nt() { return (SELF && CLIST) ? SYM_NT : GRAM_NT; }
// waves per SIMD the register budget is sized for: 256-wide rows (bf16
// descriptors) hold twice the row fragments and run two
template <int D, bool SELF, bool CLIST> constexpr int gram_wpe() { return D > 128 ? 2 : ((SELF && CLIST) ? 3 : 4); }

template <typename E, int D, int MODE, bool SELF, bool CLIST, bool DIRECT>
__global__ __launch_bounds__((gram_nt<SELF, CLIST>()), (gram_wpe<D, SELF, CLIST>())) void gram_kernel(KeySpace<E> ks, VList rows, VList cols,
                                                         float* __restrict__ out, int64_t out_hstride,
                                                         int64_t split_stride, PhiConst pc, uint64_t active,
                                                         float* __restrict__ colsum, int64_t col_ld) {
  using O = Ops<E>;
  using A = Aug<E>;
  using T = Tile<E, D>;
  constexpr int TC = 64;
  constexpr int NK = D / O::K32;
  __shared__ __attribute__((aligned(16))) E sY0[TC * D];
  __shared__ __attribute__((aligned(16))) E sY1[TC * D];
  __shared__ __attribute__((aligned(16))) u32x4_t sA0[TC];
  __shared__ __attribute__((aligned(16))) u32x4_t sA1[TC];
  __shared__ int sV0[TC];
  __shared__ int sV1[TC];
  // symmetric self-Gram (rows and columns the same list, colsum given): a
  // work-group takes only the column tiles from its own row block on; the
  // diagonal block adds row sums, the tiles right of it also column sums,
  // which stand for the mirrored pairs of the later rows
  constexpr int NT = gram_nt<SELF, CLIST>();
  constexpr int ROWS = NT / 2;   // 32 rows per wave
  __shared__ float sColP[SELF ? NT / 64 : 1][SELF ? 2 : 1][SELF ? 64 : 1];

  // XCD-aware order: logical items (head, split, row tile), head-major
  const int R = gridDim.x, S = gridDim.z;
  const int lin = xcd_remap(blockIdx.x + R * (blockIdx.y + gridDim.y * blockIdx.z), R * gridDim.y * S);
  const int h = lin / (S * R);
  const int zs = (lin / R) % S;
  if (!head_on(active, h)) return;
  const HeadKeys<E, D> hk(ks, h);
  const int nrows = vlist_count(rows, h);
  const int r0 = (lin % R) * ROWS;
  if (r0 >= nrows) return;
  const int ncols = vlist_count(cols, h);
  const int ntiles = (ncols + TC - 1) / TC;
  const bool sym = SELF && colsum != nullptr;
  const int tb = sym ? r0 / TC : 0;                  // first column tile of this work-group
  const int tdiag = tb + ROWS / TC;             // first tile right of the diagonal block
  const int per = (max(ntiles - tb, 0) + (int)gridDim.z - 1) / (int)gridDim.z;
  const int t0 = tb + zs * per;
  const int t1 = min(ntiles, t0 + per);
  const int fb = ks.M > 0 ? 0 : ks.M;   // an existing row: bank slot 0, else candidate 0

  const int lane = lane_id(), w = wave_id();
  const int hh = lane >> 5, nn = lane & 31;
  const int wrow = r0 + w * 32;
  if (t0 >= t1) {
    // no column tile in this split (an empty column list, say): the partial
    // row sums are zero, and no row fragment needs loading
    if (lane < 32 && wrow + lane < nrows)
      out[(int64_t)h * out_hstride + (int64_t)zs * split_stride + wrow + lane] = 0.0f;
    return;
  }

  typename O::frag xf[NK];
  typename O::frag xa;
  {
    const int r = wrow + nn;
    int v = r < nrows ? vlist_at(rows, h, r) : -1;
    v = hk.ok(v) ? v : -1;
    const E* xp = hk.row(v >= 0 ? v : fb);
#pragma unroll
    for (int k = 0; k < NK; ++k) xf[k] = v >= 0 ? O::load(xp + O::off32(k, lane)) : typename O::frag{};
    if constexpr (DIRECT) {
      // x' = x * (-2/sigma^2) (exact): the MFMA then returns t itself
#pragma unroll
      for (int k = 0; k < NK; ++k) xf[k] = A::scale(xf[k], pc.c2);
      xa = v >= 0 ? A::xfrag_direct(gload16(hk.aug(v)), lane, A::eps_parts(pc.eps)) : typename O::frag{};
    } else {
      xa = v >= 0 ? A::xfrag(gload16(hk.aug(v)), lane) : typename O::frag{};
    }
  }
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;

  using LD = DmaTile<E, D, TC, NT>;
  LD ld;
  // list position c -> raw entry (a plain load for index lists, the position
  // itself for ranges) -> virtual row index (-1 past the end)
  const int32_t* cidx = CLIST ? cols.idx + (int64_t)h * cols.idx_hstride : nullptr;
  auto raw = [&](int c) -> int { return CLIST ? cidx[min(c, ncols - 1)] : c; };
  auto fix = [&](int c, int e) -> int {
    const int v = CLIST ? e + cols.add : cols.base + e;
    return (c < ncols && hk.ok(v)) ? v : -1;
  };
  // Full tiles (every position below ncols) take a fast path: no clamp and
  // no check per row.  A range tile that lies in one key set (bank or
  // candidates) is consecutive rows: one uniform base plus this lane's row
  // offset.  An index-list tile reads its entries with per-lane offsets
  // fixed for the kernel.  The lane's row of copy i is (i NW + w) RPI + rl.
  // Per-lane parts: kept live in the variants without self-exclusion; the
  // self-excluding variants recompute them from an opaque lane id at each
  // use (kept live there they cost registers the MFMA loop needs).
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const unsigned ln_keep = (unsigned)lane;
  auto lane_part = [&]() -> unsigned { return SELF ? (unsigned)opaque_i(lane_id()) : ln_keep; };
  auto full = [&](int tile) -> bool {
    if ((tile + 1) * TC > ncols) return false;
    if constexpr (CLIST) return true;
    const int vlo = cols.base + tile * TC;   // one key set for the whole tile
    return (vlo + TC <= (int)hk.M || vlo >= (int)hk.M) && vlo + TC <= (int)hk.lim;
  };
  // (range columns read no list: their positions are computed when a
  // partial tile is issued, and a full tile needs none)
  auto load_index = [&](int tile) {
    if constexpr (CLIST) {
      if (full(tile)) {
        const int rl = (int)(lane_part() / T::CPR);
        const int32_t* ip = cidx + tile * TC + wu * LD::RPI + rl;
#pragma unroll
        for (int i = 0; i < LD::PASSW; ++i) ld.vi[i] = ip[i * LD::NW * LD::RPI];
        ld.va = wu == 0 ? cidx[tile * TC + lane] : 0;
      } else {
        ld.index(tile, raw);
      }
    }
  };
  auto load_issue = [&](int tile, E* nY, u32x4_t* nA, int* nV) {
    if (full(tile)) {
      const unsigned ln = lane_part();
      const int rl = (int)(ln / T::CPR);
      const int eoff = ((int)(ln % T::CPR) ^ T::swz(wu * LD::RPI + rl)) * T::EPC;
      if constexpr (CLIST) {
#pragma unroll
        for (int i = 0; i < LD::PASSW; ++i)
          dma16(hk.row(ld.vi[i] + cols.add) + eoff, nY + (i * LD::NW + wu) * LD::RPI * D);
      } else {
        const int vlo = cols.base + tile * TC;
        const E* base = hk.row(vlo) + (int64_t)(wu * LD::RPI + rl) * D + eoff;
#pragma unroll
        for (int i = 0; i < LD::PASSW; ++i)
          dma16(base + (int64_t)i * LD::NW * LD::RPI * D, nY + (i * LD::NW + wu) * LD::RPI * D);
      }
      if (wu == 0) {
        const int v = CLIST ? ld.va + cols.add : cols.base + tile * TC + lane;
        nV[lane] = v;
        dma16(hk.aug(v), nA);
      }
    } else {
      if constexpr (!CLIST) ld.index(tile, raw);
      ld.issue(tile, fix, hk, nY, nA, nV, fb);
    }
  };
  // PLAIN (direct form, every column of the tile present): t needs no clamp
  auto step = [&](auto plain_tag, int tile, const E* cY, const u32x4_t* cA, const int* cV, E* nY, u32x4_t* nA,
                  int* nV) {
    constexpr bool PLAIN = decltype(plain_tag)::value;
    if (tile + 1 < t1) {
      // the next set was last read before the previous barrier
      load_issue(tile + 1, nY, nA, nV);
      if (tile + 2 < t1) load_index(tile + 2);
    }
    // both subtiles' products first: two independent chains, interleaved
    // so that each fragment read and each product has the other chain's
    // product to hide behind
    // column fragment k of subtile sub: sub 32 D + at(n, off32(k, lane)),
    // stepped from one start offset (the swizzle repeats every 32 rows);
    // the start is rebuilt per tile so the compiler does not keep a register
    // per fragment live across the loop
    // (fp32 tiles have no swizzle: their offsets fold into immediates as is)
    const int y0 = sizeof(E) == 2 ? opaque_i(T::at(nn, O::off32(0, lane))) : 0;
    auto yoff = [&](int sub, int k) -> int {
      if constexpr (sizeof(E) == 2) return 32 * sub * D + T::at_step(y0, O::off32(k, 0));
      else return T::at(32 * sub + nn, O::off32(k, lane));
    };
    f32x16_t cc[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int i = 0; i < 16; ++i) cc[sub][i] = 0.0f;
#pragma unroll
    for (int k = 0; k < NK; ++k)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) cc[sub] = O::mma32(xf[k], O::load(cY + yoff(sub, k)), cc[sub]);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) cc[sub] = O::mma32(xa, A::yfrag(cA[32 * sub + nn], lane), cc[sub]);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int yv = cV[32 * sub + nn];
      // an absent column clamps t to +inf, where every phi mode but p = 0 is 0
      const float lo = opaque(yv >= 0 ? pc.eps : __builtin_inff());
      // self-exclusion (rows and columns are the same list): a pair is its
      // own partner exactly when the list positions coincide, which needs
      // the subtile's column range to be the wave's row range
      const bool diag = SELF && (tile * TC + 32 * sub) == wrow;
      // column sums (symmetric self-Gram, right of the diagonal block). Rows
      // and columns are one list, so such a tile only exists for a full row
      // block: no padding row enters these sums.
      float cs = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float t;
        if constexpr (DIRECT) {
          t = PLAIN ? cc[sub][i] : fmaxf(cc[sub][i], lo);
        } else {
          t = __builtin_fmaf(cc[sub][i], pc.c2, pc.eps);
          t = fmaxf(t, lo);
        }
        float f = phi_of_t<MODE>(t, pc.neg_half_p);
        if constexpr (MODE == PHI_P0) f = yv >= 0 ? f : 0.0f;
        if constexpr (SELF) {
          if (diag) f = (nn == 8 * (i >> 2) + 4 * hh + (i & 3)) ? 0.0f : f;
        }
        acc[i] += f;
        if constexpr (SELF) cs += f;
      }
      if constexpr (SELF) {
        if (sym && tile >= tdiag) sColP[w][hh][32 * sub + nn] = cs;
      }
    }
    if constexpr (SELF) {
      if (sym && tile >= tdiag) {
        // the tile's column sums over the work-group's rows, one slice per row block
        __syncthreads();
        if ((int)threadIdx.x < TC) {
          float cs = 0.0f;
#pragma unroll
          for (int ww = 0; ww < NT / 64; ++ww) cs += sColP[ww][0][threadIdx.x] + sColP[ww][1][threadIdx.x];
          const int c = tile * TC + (int)threadIdx.x;
          const int b = r0 / ROWS;
          if (c < ncols) colsum[h * sym_head_floats(col_ld) + sym_col_off(col_ld, b) + (c - (b + 1) * ROWS)] = cs;
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // next tile resident in LDS
    __syncthreads();
  };
  // Ordered form (direct form, p = 2, no self-exclusion): the products of
  // a tile are issued in a fixed order, each column fragment read two
  // products ahead, and the interactions of subtile 0 are spread between
  // the products of subtile 1 (two per product, from the third on, once its
  // last product has had two products' time to finish); subtile 1's
  // interactions follow.  Sums are taken in the same order as in `step`,
  // so results are bit-identical.  Measured on the 480P layer-chunk:
  // scoring 0.832 -> 0.820 ms.
  constexpr bool ORDERED = DIRECT && !SELF && MODE == PHI_P2 && sizeof(E) == 2;
  // acc += phi(max(c, lo)) (CLAMP) or phi(c)
  auto phi_acc = [&](auto clamp_tag, const f32x16_t& c, float lo) __attribute__((always_inline)) {
    constexpr bool CLAMP = decltype(clamp_tag)::value;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float t = CLAMP ? fmaxf(c[i], lo) : c[i];
      acc[i] += __builtin_amdgcn_rcpf(t);
    }
  };
  auto ostep = [&](auto plain_tag, int tile, const E* cY, const u32x4_t* cA, const int* cV, E* nY, u32x4_t* nA,
                   int* nV) __attribute__((always_inline)) {
    constexpr bool PLAIN = decltype(plain_tag)::value;
    if (tile + 1 < t1) {
      load_issue(tile + 1, nY, nA, nV);
      if (tile + 2 < t1) load_index(tile + 2);
    }
    const int y0 = opaque_i(T::at(nn, O::off32(0, lane)));
    // absent columns clamp t to +inf (phi 0); full tiles need no clamp
    float lo0 = pc.eps, lo1 = pc.eps;
    if constexpr (!PLAIN) {
      lo0 = opaque(cV[nn] >= 0 ? pc.eps : __builtin_inff());
      lo1 = opaque(cV[32 + nn] >= 0 ? pc.eps : __builtin_inff());
    }
    // products in order: subtile 0 (NK k-steps, then the norm step), then
    // subtile 1; product j's column fragment is read at product j - 2
    constexpr int NP = 2 * (NK + 1);
    constexpr int PF = 2;
    auto bfrag = [&](int j) -> typename O::frag {
      const int sub = j / (NK + 1), k = j % (NK + 1);
      if (k < NK) return O::load(cY + 32 * sub * D + T::at_step(y0, O::off32(k, 0)));
      return A::yfrag(cA[32 * sub + nn], lane);
    };
    f32x16_t c0, c1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      c0[i] = 0.0f;
      c1[i] = 0.0f;
    }
    typename O::frag fb[PF + 1];
#pragma unroll
    for (int j = 0; j < PF; ++j) fb[j] = bfrag(j);
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      __builtin_amdgcn_sched_barrier(0);
      if (j + PF < NP) fb[(j + PF) % (PF + 1)] = bfrag(j + PF);
      const int k = j % (NK + 1);
      if (j < NK + 1) c0 = O::mma32(k < NK ? xf[k] : xa, fb[j % (PF + 1)], c0);
      else c1 = O::mma32(k < NK ? xf[k] : xa, fb[j % (PF + 1)], c1);
      if (j >= NK + 2) {
        const int i0 = 16 * (j - NK - 2) / NK, i1 = 16 * (j - NK - 1) / NK;
#pragma unroll
        for (int i = i0; i < i1; ++i) {
          const float t = PLAIN ? c0[i] : fmaxf(c0[i], lo0);
          acc[i] += __builtin_amdgcn_rcpf(t);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    phi_acc(BoolTag<!PLAIN>{}, c1, lo1);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // next tile resident in LDS
    __syncthreads();
  };
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): row fragments resident
  if (t0 < t1) {
    load_index(t0);
    load_issue(t0, sY0, sA0, sV0);
    if (t0 + 1 < t1) load_index(t0 + 1);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  // only the last tile of the column list can be ragged
  const int tfull = DIRECT ? min(t1, ncols / TC) : t0;
  int tile = t0;
  if constexpr (ORDERED) {
    for (; tile + 1 < tfull; tile += 2) {
      ostep(BoolTag<true>{}, tile, sY0, sA0, sV0, sY1, sA1, sV1);
      ostep(BoolTag<true>{}, tile + 1, sY1, sA1, sV1, sY0, sA0, sV0);
    }
    for (; tile < t1; ++tile) {
      if (((tile - t0) & 1) == 0) ostep(BoolTag<false>{}, tile, sY0, sA0, sV0, sY1, sA1, sV1);
      else ostep(BoolTag<false>{}, tile, sY1, sA1, sV1, sY0, sA0, sV0);
    }
  } else {
    for (; tile + 1 < tfull; tile += 2) {
      step(BoolTag<true>{}, tile, sY0, sA0, sV0, sY1, sA1, sV1);
      step(BoolTag<true>{}, tile + 1, sY1, sA1, sV1, sY0, sA0, sV0);
    }
    for (; tile < t1; ++tile) {
      if (((tile - t0) & 1) == 0) step(BoolTag<false>{}, tile, sY0, sA0, sV0, sY1, sA1, sV1);
      else step(BoolTag<false>{}, tile, sY1, sA1, sV1, sY0, sA0, sV0);
    }
  }
  // sum over the 32 columns held by the half-wave
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float v = acc[i];
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 8);
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 1);
    acc[i] = v;
  }
  if (nn == 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = wrow + 8 * (i >> 2) + 4 * hh + (i & 3);
      if (r < nrows) out[(int64_t)h * out_hstride + (int64_t)zs * split_stride + r] = acc[i];
    }
  }
}

template <typename E>
static KeySpace<E> key_space(const KeysDesc& k) {
  return KeySpace<E>{(const E*)k.bankK, (const E*)k.candK, k.bankN, k.candN, (const u32x4_t*)k.bankA,
                     (const u32x4_t*)k.candA, k.M, k.N, k.d};
}

template <typename E, int D, int MODE, bool DIRECT>
static void gram_dispatch_self(const GramLaunch& g, dim3 grid, hipStream_t st) {
  const KeySpace<E> ks = key_space<E>(g.k);
  // self-exclusion only arises with both sides the same index list
  if (g.self_excl && g.cols.idx) {
    grid.x = (unsigned)((g.rows.n + SYM_NT / 2 - 1) / (SYM_NT / 2));
    hipLaunchKernelGGL((gram_kernel<E, D, MODE, true, true, DIRECT>), grid, dim3(SYM_NT), 0, st, ks, g.rows, g.cols,
                       g.out, g.out_hstride, g.split_stride, g.pc, g.active, g.colsum, g.col_ld);
  } else if (g.self_excl)
    hipLaunchKernelGGL((gram_kernel<E, D, MODE, true, false, DIRECT>), grid, dim3(GRAM_NT), 0, st, ks, g.rows, g.cols,
                       g.out, g.out_hstride, g.split_stride, g.pc, g.active, g.colsum, g.col_ld);
  else if (g.cols.idx)
    hipLaunchKernelGGL((gram_kernel<E, D, MODE, false, true, DIRECT>), grid, dim3(GRAM_NT), 0, st, ks, g.rows, g.cols,
                       g.out, g.out_hstride, g.split_stride, g.pc, g.active, g.colsum, g.col_ld);
  else
    hipLaunchKernelGGL((gram_kernel<E, D, MODE, false, false, DIRECT>), grid, dim3(GRAM_NT), 0, st, ks, g.rows, g.cols,
                       g.out, g.out_hstride, g.split_stride, g.pc, g.active, g.colsum, g.col_ld);
}

template <typename E, int D>
static void gram_dispatch_mode(const GramLaunch& g, dim3 grid, hipStream_t st) {
  switch (g.phi_mode) {
    case PHI_P2:
      if constexpr (sizeof(E) == 2) {
        if (g.pc.direct) { gram_dispatch_self<E, D, PHI_P2, true>(g, grid, st); break; }
      }
      gram_dispatch_self<E, D, PHI_P2, false>(g, grid, st);
      break;
    case PHI_P0: gram_dispatch_self<E, D, PHI_P0, false>(g, grid, st); break;
    case PHI_P1: gram_dispatch_self<E, D, PHI_P1, false>(g, grid, st); break;
    case PHI_P4: gram_dispatch_self<E, D, PHI_P4, false>(g, grid, st); break;
    default: gram_dispatch_self<E, D, PHI_GEN, false>(g, grid, st); break;
  }
}

hipError_t launch_gram(const GramLaunch& g, hipStream_t st) {
  if (g.rows.n <= 0) return hipSuccess;
  const dim3 grid((unsigned)((g.rows.n + GRAM_ROWS - 1) / GRAM_ROWS), (unsigned)g.k.H,
                  (unsigned)(g.splits > 0 ? g.splits : 1));
  if (g.k.et == ET_BF16) {
    if (g.k.d == 256) gram_dispatch_mode<uint16_t, 256>(g, grid, st);
    else if (g.k.d == 128) gram_dispatch_mode<uint16_t, 128>(g, grid, st);
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

// Four lanes per column: lane q sums a quarter of the blocks in order, and the
// quarters are added as (q0 + q1) + (q2 + q3), a fixed order.
__global__ void sym_combine_kernel(float* __restrict__ dst, int64_t dst_hstride, const float* __restrict__ colsum,
                                   int64_t col_ld, int nblocks, VList rows, uint64_t active) {
  const int h = blockIdx.y;
  if (!head_on(active, h)) return;
  const int j = blockIdx.x * (blockDim.x / 4) + (int)(threadIdx.x >> 2);
  const int q = (int)(threadIdx.x & 3);
  if (j >= vlist_count(rows, h)) return;   // the column's four lanes leave together
  const int jb = min(j / GRAM_ROW_BLOCK, nblocks);
  const int per = (jb + 3) / 4;
  const int b0 = min(q * per, jb), b1 = min(b0 + per, jb);
  const float* ch = colsum + h * sym_head_floats(col_ld);
  float s = 0.0f;
  for (int b = b0; b < b1; ++b) s += ch[sym_col_off(col_ld, b) + (j - (b + 1) * GRAM_ROW_BLOCK)];
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  if (q == 0) dst[(int64_t)h * dst_hstride + j] += s;
}

hipError_t launch_sym_combine(float* dst, int64_t dst_hstride, const float* colsum, int64_t col_ld, int nblocks,
                              VList rows, uint64_t active, int H, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(sym_combine_kernel, dim3((n + 63) / 64, H), dim3(256), 0, st, dst, dst_hstride, colsum, col_ld,
                     nblocks, rows, active);
  return hipGetLastError();
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
// (A = candidates from LDS, B = bank rows in registers, plus the norm
// augmentation step) gives lane l the 16 values of bank row (l & 31).  The
// candidates are placed in LDS so that lane half h = l >> 5 holds positions
// 16h .. 16h + 15 of the subtile in order.  The canonical running sum is
//   first half:  carry + P0(i),      second half:  (carry + tot0) + P1(i),
// with P the sequential sums inside a half and tot0, tot1 the half totals
// (exchanged between the two lanes of a row); the carry advances to
// (carry + tot0) + tot1.  This value is monotone in k, identical in the scan
// and the sum pass, and its subtile-boundary values are the checkpoints.
//
// scan pass: t_b = smallest k with S_b(k) > tau * rho0_b (kmax+1 if none).
// sum pass:  rhoP_b = S_b(k*) starting from the nearest checkpoint.
// ---------------------------------------------------------------------------
template <typename E, int D, int MODE, bool SUM, bool DIRECT>
__global__ __launch_bounds__(256, (D > 128 ? 2 : 4)) void scan_kernel(KeySpace<E> ks, const float* __restrict__ rho,
                                                   const float* __restrict__ rho0, const int32_t* __restrict__ count,
                                                   const int32_t* __restrict__ order, uint64_t active,
                                                   int kmax, float tau, int cps, int ncp, float* __restrict__ cp,
                                                   int32_t* __restrict__ t_out, const int32_t* __restrict__ kstar_p,
                                                   int kstar_hs, int keep_crossed, float* __restrict__ rhoP,
                                                   PhiConst pc) {
  using O = Ops<E>;
  using A = Aug<E>;
  using T = Tile<E, D>;
  constexpr int TC = 64;               // candidates per LDS stage (two subtiles)
  constexpr int NK = D / O::K32;
  __shared__ __attribute__((aligned(16))) E sC0[TC * D];
  __shared__ __attribute__((aligned(16))) E sC1[TC * D];
  __shared__ __attribute__((aligned(16))) u32x4_t sA0[TC];
  __shared__ __attribute__((aligned(16))) u32x4_t sA1[TC];

  const int R = gridDim.x;
  const int lin = xcd_remap(blockIdx.x + R * blockIdx.y, R * gridDim.y);
  const int h = lin / R;
  if (!head_on(active, h)) return;
  const HeadKeys<E, D> hk(ks, h);
  const int M = ks.M;
  const int n = count[h];
  const int b0 = (lin % R) * 128;
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
    kst = kstar_p[h * kstar_hs];
    // crossed rows (t_b <= k*) are evicted and their projected density is
    // unused, unless the policy lets crossed rows survive
    need = valid && kst > 0 && (keep_crossed || t_out[hb] > kst);
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
  typename O::frag ba;
  {
    const E* bp = ks.bankK + hb * D;
#pragma unroll
    for (int k = 0; k < NK; ++k) bf[k] = valid ? O::load(bp + O::off32(k, lane)) : typename O::frag{};
    if constexpr (DIRECT) {
#pragma unroll
      for (int k = 0; k < NK; ++k) bf[k] = A::scale(bf[k], pc.c2);
      ba = valid ? A::xfrag_direct(gload16(ks.bankA + hb), lane, A::eps_parts(pc.eps)) : typename O::frag{};
    } else {
      ba = valid ? A::xfrag(gload16(ks.bankA + hb), lane) : typename O::frag{};
    }
  }

  const int st_begin = sub_begin / 2, st_end = (sub_end + 1) / 2;
  DmaTile<E, D, TC> ld;
  // position j of the order -> raw entry -> virtual row index (-1 past kmax)
  const int32_t* ord = order + (int64_t)h * ks.N;
  // LDS row r of a stage (subtile r / 32, MFMA row rho = r % 32 = 8q + 4h + r')
  // holds order position 32 (r / 32) + 16 h + 4 q + r': the MFMA output then
  // gives lane half h the 16 consecutive positions 16 h .. 16 h + 15
  auto pos_of = [](int c) -> int {
    const int rho = c & 31;
    return (c & ~31) + 16 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3);
  };
  auto raw = [&](int c) -> int { return ord[min(pos_of(c), kmax - 1)]; };
  auto fix = [&](int c, int e) -> int {
    return (pos_of(c) < kmax && (unsigned)e < (unsigned)ks.N) ? M + e : -1;
  };
  // candidates are always present in a stage's used positions; rows past
  // kmax copy a fallback row and are masked below
  const int fb = M;                      // candidate 0 (N > 0 whenever kmax > 0)
  // Full stages (every position below kmax): each row is candidate ord[j]
  // and needs neither clamp nor check, so a copy address is one multiply-add
  // on the list entry.  For bf16 keys the order position of a lane's copy i
  // is 64 stage + jp + joff(i), with jp fixed for the kernel: copies of one
  // lane are NW RPI = 16 (or 32) rows apart, and pos_of moves a row only
  // inside its group of 32.
  using LD = DmaTile<E, D, TC>;
  constexpr bool FASTG = sizeof(E) == 2 && (LD::NW * LD::RPI == 16 || LD::NW * LD::RPI == 32);
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int jp = pos_of(wu * LD::RPI + lane / T::CPR);
  auto joff = [](int i) -> int { return LD::NW * LD::RPI == 16 ? 32 * (i >> 1) + 8 * (i & 1) : 32 * i; };
  auto full = [&](int stg) -> bool { return (stg + 1) * TC <= kmax; };
  auto index_fast = [&](int stg) {
    const int32_t* op = ord + stg * TC + jp;
#pragma unroll
    for (int i = 0; i < LD::PASSW; ++i) ld.vi[i] = op[joff(i)];
    ld.va = wu == 0 ? raw(stg * TC + lane) : 0;
  };
  const E* cand0 = hk.cand + (int64_t)M * D;   // candidate row 0
  auto issue_fast = [&](int stg, E* nC, u32x4_t* nA) {
    const int eoff = ((lane % T::CPR) ^ T::swz(wu * LD::RPI + lane / T::CPR)) * T::EPC;
#pragma unroll
    for (int i = 0; i < LD::PASSW; ++i)
      dma16(cand0 + (int64_t)(uint32_t)ld.vi[i] * D + eoff, nC + (i * LD::NW + wu) * LD::RPI * D);
    if (wu == 0) {
      const int v = fix(stg * TC + lane, ld.va);
      dma16(hk.aug(v >= 0 ? v : fb), nA);
    }
  };
  auto load_index = [&](int stg) {
    if (FASTG && full(stg)) index_fast(stg);
    else ld.index(stg, raw);
  };
  auto load_issue = [&](int stg, E* nC, u32x4_t* nA) {
    if (FASTG && full(stg)) issue_fast(stg, nC, nA);
    else ld.issue(stg, fix, hk, nC, nA, nullptr, fb);
  };
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): bank fragments resident
  if (st_begin < st_end) {
    load_index(st_begin);
    load_issue(st_begin, sC0, sA0);
    if (st_begin + 1 < st_end) load_index(st_begin + 1);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  // one stage (returns false once every row of the work-group has crossed);
  // the two buffer sets are distinct LDS objects, so the copy in flight is
  // known not to alias the reads of the current stage
  auto step = [&](int stg, const E* cC, const u32x4_t* cA, E* nC, u32x4_t* nA) -> bool {
    const bool more = stg + 1 < st_end;
    if (more) {
      // the next set was last read before the previous barrier
      load_issue(stg + 1, nC, nA);
      if (stg + 2 < st_end) load_index(stg + 2);
    }
    // a wave whose rows have all crossed skips the stage, unless crossed
    // rows may survive: the scan then keeps their running sums (checkpoints)
    const bool wave_busy = (!SUM && keep_crossed) || __any(!done);
    if (wave_busy) {
      // both subtiles' products first (independent MFMA chains), then the
      // interactions and prefix sums of each in order
      // candidate fragment k of subtile half: 32 half D + at(n, off32(k,
      // lane)), stepped from one start offset rebuilt per stage (kept live
      // across the walk, one register per fragment would spill)
      // (fp32 tiles have no swizzle: their offsets fold into immediates)
      const int c0 = sizeof(E) == 2 ? opaque_i(T::at(lane & 31, O::off32(0, lane))) : 0;
      auto coff = [&](int half, int k) -> int {
        if constexpr (sizeof(E) == 2) return 32 * half * D + T::at_step(c0, O::off32(k, 0));
        else return T::at(32 * half + (lane & 31), O::off32(k, lane));
      };
      // the two halves' chains interleaved (each fragment read and product
      // has the other chain's product to hide behind)
      f32x16_t accs[2];
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int i = 0; i < 16; ++i) accs[half][i] = 0.0f;
#pragma unroll
      for (int k = 0; k < NK; ++k)
#pragma unroll
        for (int half = 0; half < 2; ++half) accs[half] = O::mma32(O::load(cC + coff(half, k)), bf[k], accs[half]);
#pragma unroll
      for (int half = 0; half < 2; ++half)
        accs[half] = O::mma32(A::yfrag(cA[32 * half + (lane & 31)], lane), ba, accs[half]);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int sub = 2 * stg + half;
        if (sub < sub_begin || sub >= sub_end) continue;
        if constexpr (!SUM) {
          if (sub % cps == 0 && sub > 0 && valid) cp[((int64_t)h * ncp + sub / cps) * M + b] = carry;
        }
        const f32x16_t acc = accs[half];
        // lane (row b, half hh) holds candidates pos0 + 16 hh + i, i = 0..15
        float v[16];
        const int pos0 = 32 * sub;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          // direct form: the MFMA returned t (no clamp needed, eps >= 1e-2);
          // positions past kmax hold a stand-in row and are zeroed below
          float t = acc[i];
          if constexpr (!DIRECT) {
            t = __builtin_fmaf(acc[i], pc.c2, pc.eps);
            t = fmaxf(t, pc.eps);
          }
          v[i] = phi_of_t<MODE>(t, pc.neg_half_p);
        }
        if (pos0 + 32 > kmax) {   // last subtile: drop positions past kmax
#pragma unroll
          for (int i = 0; i < 16; ++i) v[i] = (pos0 + 16 * hh + i < kmax) ? v[i] : 0.0f;
        }
        // sequential half sums, exchanged between the two lanes of a row:
        // after the swap every lane holds tot0 (first half) and tot1
        float tot = v[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) tot += v[i];
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tot), __float_as_uint(tot), false, false);
        const float tot0 = __uint_as_float(sw[0]), tot1 = __uint_as_float(sw[1]);
        const float mid = carry + tot0;             // S at the end of the first half
        const float s_end = mid + tot1;
        const float base = hh ? mid : carry;        // S before this lane's first candidate
        if constexpr (!SUM) {
          const bool cross = !done && (s_end > thr);
          // rows cross once; the exact position search runs only in waves where
          // some row crosses in this subtile (both lanes of a row agree)
          if (__any(cross)) {
            int first = 64;
            if (cross) {
              float P = 0.0f;
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                P = (i == 0) ? v[0] : P + v[i];
                if (base + P > thr && first == 64) first = 16 * hh + i;
              }
            }
            const auto fs = __builtin_amdgcn_permlane32_swap((unsigned)first, (unsigned)first, false, false);
            first = min((int)fs[0], (int)fs[1]);
            if (cross) t_b = pos0 + first + 1;
          }
          // a crossed row's running sum stops unless crossed rows may survive
          // (the sum pass then resumes them from their checkpoints too)
          if (!done || keep_crossed) carry = s_end;
          done = done || cross;
        } else {
          if (sub < sub_end - 1) {
            carry = s_end;
          } else {
            const int j = (kst - 1) - pos0;         // position of the last admitted candidate
            const int jh = j >> 4, jj = j & 15;
            float P = 0.0f, PP = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              PP = (i == 0) ? v[0] : PP + v[i];
              if (i == jj) P = PP;
            }
            const float S = base + P;               // meaningful in the lanes with hh == jh
            const auto ss = __builtin_amdgcn_permlane32_swap(__float_as_uint(S), __float_as_uint(S), false, false);
            carry = __uint_as_float(jh ? ss[1] : ss[0]);
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // next stage resident in LDS
    if constexpr (!SUM) {
      // every row of the work-group crossed: later checkpoints are never
      // read (the sum pass skips rows with t_b <= k*); checked every fourth
      // stage to keep one plain barrier per stage
      if ((stg & 3) == 3 && !keep_crossed) return __syncthreads_or(!done) != 0;
      __syncthreads();
      return true;
    } else {
      __syncthreads();
      return true;
    }
  };
  for (int stg = st_begin; stg < st_end; stg += 2) {
    if (!step(stg, sC0, sA0, sC1, sA1)) break;
    if (stg + 1 < st_end && !step(stg + 1, sC1, sA1, sC0, sA0)) break;
  }
  if (valid && hh == 0) {
    if constexpr (SUM) rhoP[hb] = need ? carry : r_b;
    else t_out[hb] = t_b;
  }
}

template <typename E, int D, int MODE, bool DIRECT>
static void scan_dispatch(const ScanLaunch& a, bool sum, dim3 grid, hipStream_t st) {
  const KeySpace<E> ks = key_space<E>(a.k);
  if (sum)
    hipLaunchKernelGGL((scan_kernel<E, D, MODE, true, DIRECT>), grid, dim3(256), 0, st, ks, a.rho, a.rho0, a.count,
                       a.order, a.active, a.kmax, a.tau, a.cps, a.ncp, a.cp, a.t_out, a.kstar, a.kstar_hs,
                       a.keep_crossed, a.rhoP, a.pc);
  else
    hipLaunchKernelGGL((scan_kernel<E, D, MODE, false, DIRECT>), grid, dim3(256), 0, st, ks, a.rho, a.rho0, a.count,
                       a.order, a.active, a.kmax, a.tau, a.cps, a.ncp, a.cp, a.t_out, a.kstar, a.kstar_hs,
                       a.keep_crossed, a.rhoP, a.pc);
}

template <typename E, int D>
static void scan_dispatch_mode(const ScanLaunch& a, bool sum, dim3 grid, hipStream_t st) {
  switch (a.phi_mode) {
    case PHI_P2:
      if constexpr (sizeof(E) == 2) {
        if (a.pc.direct) { scan_dispatch<E, D, PHI_P2, true>(a, sum, grid, st); break; }
      }
      scan_dispatch<E, D, PHI_P2, false>(a, sum, grid, st);
      break;
    case PHI_P0: scan_dispatch<E, D, PHI_P0, false>(a, sum, grid, st); break;
    case PHI_P1: scan_dispatch<E, D, PHI_P1, false>(a, sum, grid, st); break;
    case PHI_P4: scan_dispatch<E, D, PHI_P4, false>(a, sum, grid, st); break;
    default: scan_dispatch<E, D, PHI_GEN, false>(a, sum, grid, st); break;
  }
}

hipError_t launch_scan(const ScanLaunch& a, bool sum, hipStream_t st) {
  if (a.k.M <= 0) return hipSuccess;
  const dim3 grid((unsigned)((a.k.M + 127) / 128), (unsigned)a.k.H);
  if (a.k.et == ET_BF16) {
    if (a.k.d == 256) scan_dispatch_mode<uint16_t, 256>(a, sum, grid, st);
    else if (a.k.d == 128) scan_dispatch_mode<uint16_t, 128>(a, sum, grid, st);
    else scan_dispatch_mode<uint16_t, 64>(a, sum, grid, st);
  } else {
    if (a.k.d == 128) scan_dispatch_mode<float, 128>(a, sum, grid, st);
    else scan_dispatch_mode<float, 64>(a, sum, grid, st);
  }
  return hipGetLastError();
}

}  // namespace kvb
