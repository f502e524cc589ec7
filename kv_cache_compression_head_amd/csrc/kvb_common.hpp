// Shared device helpers for the kvbank HIP kernels (gfx950 / CDNA4 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define KVB_DEV __device__ __forceinline__

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

namespace kvb {

constexpr int WAVE = 64;

KVB_DEV bool head_on(uint64_t mask, int h) { return (mask >> h) & 1ull; }
KVB_DEV int lane_id() { return threadIdx.x & 63; }
KVB_DEV int wave_id() { return threadIdx.x >> 6; }

KVB_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
KVB_DEV uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// MFMA operand traits.  For a Gram product X Y^T both operands are read the
// same way from row-major [row][d] storage: a lane supplies a slice of the d
// (contraction) axis of one row.  16x16 tiles: row = lane & 15, slice group =
// lane >> 4.  32x32 tiles: row = lane & 31, slice group = lane >> 5.
// Output: 16x16 -> acc[i] = C[4*(lane>>4) + i][lane & 15];
//         32x32 -> acc[i] = C[8*(i>>2) + 4*(lane>>5) + (i&3)][lane & 31].
// ---------------------------------------------------------------------------
template <typename E> struct Ops;

template <> struct Ops<uint16_t> {   // bf16 storage
  using frag = s16x8_t;
  static constexpr int K16 = 32;   // contraction per 16x16 MFMA
  static constexpr int K32 = 16;   // contraction per 32x32 MFMA
  KVB_DEV static int off16(int ks, int lane) { return ks * 32 + (lane >> 4) * 8; }
  KVB_DEV static int off32(int ks, int lane) { return ks * 16 + (lane >> 5) * 8; }
  KVB_DEV static frag load(const uint16_t* p) { return *reinterpret_cast<const s16x8_t*>(p); }
  KVB_DEV static f32x4_t mma16(frag a, frag b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  KVB_DEV static f32x16_t mma32(frag a, frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  KVB_DEV static float to_f32(uint16_t v) { return bf16_to_f32(v); }
  static constexpr int PAD = 8;      // LDS row padding (elements): 16 bytes
};

template <> struct Ops<float> {      // fp32 storage
  using frag = float;
  static constexpr int K16 = 4;
  static constexpr int K32 = 2;
  KVB_DEV static int off16(int ks, int lane) { return ks * 4 + (lane >> 4); }
  KVB_DEV static int off32(int ks, int lane) { return ks * 2 + (lane >> 5); }
  KVB_DEV static frag load(const float* p) { return *p; }
  KVB_DEV static f32x4_t mma16(frag a, frag b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  KVB_DEV static f32x16_t mma32(frag a, frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  KVB_DEV static float to_f32(float v) { return v; }
  static constexpr int PAD = 4;      // 16 bytes
};

// ---------------------------------------------------------------------------
// Soft-Riesz interaction phi(d2) = (eps + d2 / sigma^2)^(-p/2).
// The caller folds the norms: t = eps + (|x|^2 + |y|^2 - 2 x.y) / sigma^2
// computed as fma(dot, -2/sigma^2, xs + ys) with xs = |x|^2/sigma^2 + eps and
// ys = |y|^2/sigma^2, then clamped to t >= eps (d2 >= 0).
// ---------------------------------------------------------------------------
enum PhiMode { PHI_P2 = 0, PHI_P0 = 1, PHI_P1 = 2, PHI_P4 = 3, PHI_GEN = 4 };

struct PhiConst {
  float c2;       // -2 / sigma^2
  float inv_s2;   // 1 / sigma^2
  float eps;
  float neg_half_p;
  // "direct" form: sigma^2 is a power of two (so x * -2/sigma^2 and the
  // scaled norms are exact in bf16 parts) and eps >= 1e-2 (so rounding can
  // never bring t = eps + d2/sigma^2 near zero): the MFMA then returns t
  // itself and the clamp is needed only on ragged tiles
  int32_t direct;
};

template <int MODE> KVB_DEV float phi_of_t(float t, float neg_half_p) {
  if constexpr (MODE == PHI_P2) return __builtin_amdgcn_rcpf(t);
  else if constexpr (MODE == PHI_P0) return 1.0f;
  else if constexpr (MODE == PHI_P1) return __builtin_amdgcn_rsqf(t);
  else if constexpr (MODE == PHI_P4) { float r = __builtin_amdgcn_rcpf(t); return r * r; }
  else return __builtin_amdgcn_exp2f(neg_half_p * __builtin_amdgcn_logf(t));
}

template <int MODE> KVB_DEV float phi_pair(float dot, float us, const PhiConst& pc) {
  float t = __builtin_fmaf(dot, pc.c2, us);
  t = fmaxf(t, pc.eps);
  return phi_of_t<MODE>(t, pc.neg_half_p);
}

// ---------------------------------------------------------------------------
// Row lists.  A "virtual" key index v addresses bank slot v when v < M and
// candidate row v - M otherwise.  A list yields, for head h and position i,
// idx ? idx[h * idx_hstride + i] + add : base + i, with count
// cnt ? min(cnt[h * cnt_hstride] + cnt_add, n) : n.
// ---------------------------------------------------------------------------
struct VList {
  const int32_t* idx;
  const int32_t* cnt;
  int32_t idx_hstride;
  int32_t cnt_hstride;
  int32_t add;
  int32_t base;
  int32_t n;        // upper bound (also the count when cnt is null)
  int32_t cnt_add;
};

KVB_DEV int vlist_count(const VList& L, int h) {
  if (!L.cnt) return L.n;
  int c = L.cnt[(int64_t)h * L.cnt_hstride] + L.cnt_add;
  c = c < 0 ? 0 : c;
  return c < L.n ? c : L.n;
}
KVB_DEV int vlist_at(const VList& L, int h, int i) {
  return L.idx ? L.idx[(int64_t)h * L.idx_hstride + i] + L.add : L.base + i;
}

// Keys of one layer in two buffers: bank [H][M][d] and candidates [H][N][d],
// with their scaled squared norms (|k|^2 / sigma^2) in [H][M] and [H][N] and
// a 16-byte "augmentation" row per key holding |k|^2 split exactly into
// bf16 parts (hi, mid, lo) (bf16 keys) or as one float (fp32 keys); an extra
// MFMA k-step against (-1/2, -1/2, -1/2) then yields k.x - |k|^2 / 2.
template <typename E> struct KeySpace {
  const E* bankK;
  const E* candK;
  const float* bankN;
  const float* candN;
  const u32x4_t* bankA;
  const u32x4_t* candA;
  int32_t M;
  int32_t N;
  int32_t d;
  KVB_DEV const E* row(int h, int v) const {
    return v < M ? bankK + ((int64_t)h * M + v) * d : candK + ((int64_t)h * N + (v - M)) * d;
  }
  KVB_DEV bool ok(int v) const { return v >= 0 && v < M + N; }
  KVB_DEV float nrm(int h, int v) const {
    return v < M ? bankN[(int64_t)h * M + v] : candN[(int64_t)h * N + (v - M)];
  }
  KVB_DEV const u32x4_t* aug(int h, int v) const {
    return v < M ? bankA + ((int64_t)h * M + v) : candA + ((int64_t)h * N + (v - M));
  }
};

// Per-head view of a KeySpace with compile-time row length: row addresses are
// one select and one shift from two per-head bases.
template <typename E, int D> struct HeadKeys {
  const E* bank;      // bankK + h*M*D
  const E* cand;      // candK + (h*N - M)*D  (indexed by the virtual index)
  const u32x4_t* abank;
  const u32x4_t* acand;
  uint32_t lim;       // M + N
  uint32_t M;
  KVB_DEV HeadKeys(const KeySpace<E>& ks, int h)
      : bank(ks.bankK + (int64_t)h * ks.M * D), cand(ks.candK + ((int64_t)h * ks.N - ks.M) * D),
        abank(ks.bankA + (int64_t)h * ks.M), acand(ks.candA + ((int64_t)h * ks.N - ks.M)),
        lim((uint32_t)(ks.M + ks.N)), M((uint32_t)ks.M) {}
  KVB_DEV bool ok(int v) const { return (uint32_t)v < lim; }
  KVB_DEV const E* row(int v) const { return ((uint32_t)v < M ? bank : cand) + (int64_t)(uint32_t)v * D; }
  KVB_DEV const u32x4_t* aug(int v) const { return ((uint32_t)v < M ? abank : acand) + (uint32_t)v; }
};

// LDS key tiles: rows of D elements with no padding; the 16-byte chunks of
// row r are XOR-swizzled so that the 16 rows read by one quarter-wave hit 16
// different 16-byte bank groups.
template <typename E, int D> struct Tile {
  static constexpr int EPC = 16 / (int)sizeof(E);   // elements per chunk
  static constexpr int CPR = D / EPC;               // chunks per row
  KVB_DEV static int swz(int r) {
    if constexpr (sizeof(E) == 2) {
      if constexpr (CPR == 16) return r & 15;
      else return (r >> 1) & 7;
    } else {
      return 0;
    }
  }
  // element offset of element e of row r (e is a fragment start)
  KVB_DEV static int at(int r, int e) { return r * D + (((e / EPC) ^ swz(r)) * EPC) + e % EPC; }
  // at(r, e + f) from a0 = at(r, e), for a fragment step f whose chunk bits
  // are disjoint from e's (f = off32(k, 0) against e = off32(0, lane)): the
  // swizzle is an XOR on the chunk index and the row base has no bits below
  // D, so stepping along the row is an XOR of the start offset
  KVB_DEV static int at_step(int a0, int f) { return a0 ^ f; }
};

// 16-byte global -> LDS copy that bypasses registers: lane l of the wave
// writes 16 bytes at lds + 16 l
KVB_DEV void dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// value the optimiser cannot see through (keeps a clamp a single max)
KVB_DEV float opaque(float x) {
  asm volatile("" : "+v"(x));
  return x;
}
// same for an integer: values derived from it are recomputed where used
// instead of being hoisted out of a loop and kept in registers
KVB_DEV int opaque_i(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Work-groups are dealt round-robin to the 8 XCDs of the chip (dispatch
// index p runs on XCD p % 8).  Remap so that XCD x processes one contiguous
// range of the W logical work items: items that share data (same head) then
// share one XCD's L2.  The map is a bijection for any W.
constexpr int NUM_XCD = 8;
KVB_DEV int xcd_remap(int p, int W) {
  const int x = p % NUM_XCD, j = p / NUM_XCD;
  const int q = W / NUM_XCD, rem = W % NUM_XCD;
  return x * q + (x < rem ? x : rem) + j;
}

// 16-byte load through the global address space (generic pointers that are
// known to point to device memory; keeps the load off the LDS counter)
KVB_DEV u32x4_t gload16(const void* p) {
  typedef __attribute__((address_space(1))) const u32x4_t gvec;
  return *(gvec*)(p);
}

// order-preserving map of a float to an unsigned key (ascending floats ->
// ascending keys; -0 and +0 differ, NaN not expected)
KVB_DEV uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// wave reductions (deterministic fixed-order butterflies)
// ---------------------------------------------------------------------------
KVB_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
KVB_DEV int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace kvb
