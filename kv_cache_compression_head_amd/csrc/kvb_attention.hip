// Chunk attention over the ragged per-head retained KV.
//
// DensityKV card page, Figure 2: the current queries read the retained
// history (sink, per-head bank, local window) through the backbone's native
// attention; Forcing-KV notes page, section 3.3: the chunk attends to its own
// keys without a mask.  O_h = softmax(Q_h K_h^T * scale) V_h, where K_h/V_h
// is the concatenation of the head's segments (order irrelevant).
//
// bf16 path: flash-style online softmax.  Work-group = 4 waves x 32 queries;
// KV tiles of 64 keys staged in LDS (K row-major, V transposed).  Scores are
// computed transposed (S^T = K Q^T, 16x16x32 MFMA) so that every lane holds
// keys of a single query; P^T feeds O^T = V^T P^T directly as the B operand.
#include "kvb_common.hpp"
#include "kvb_launch.hpp"

namespace kvb {

constexpr int ATT_TK = 64;          // keys per tile
constexpr int ATT_QW = 32;          // queries per wave
constexpr int ATT_MAXSEG = 256;     // segments cached in LDS

struct SegCache {
  const SegEntry* segs;
  int n;
};

// locate virtual key j: segment index via the LDS prefix table
KVB_DEV int seg_find(const int* pre, int n, int j) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int m = (lo + hi + 1) >> 1;
    if (pre[m] <= j) lo = m; else hi = m - 1;
  }
  return lo;
}

template <int D>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(const uint16_t* __restrict__ Q, void* __restrict__ O,
                                                           const SegEntry* __restrict__ segs,
                                                           const int32_t* __restrict__ nseg_p, int seg_cap, int Lq,
                                                           float scale_log2, int out_f32, int nqt) {
  using Op = Ops<uint16_t>;
  constexpr int LDK = D + 8;              // K row stride (elements)
  constexpr int LDV = ATT_TK + 8;         // V^T row stride (elements)
  constexpr int NKS = D / 32;             // k-steps for S^T
  constexpr int NDB = D / 16;             // d blocks for O^T
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) uint16_t sK[ATT_TK * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sV[D * LDV];
  __shared__ int s_pre[ATT_MAXSEG + 1];
  __shared__ const void* s_k[ATT_MAXSEG];
  __shared__ const void* s_v[ATT_MAXSEG];

  const int bid = blockIdx.x;
  const int h = bid / nqt;
  const int qt = bid % nqt;
  const int lane = lane_id(), w = wave_id();
  const int g = lane >> 4;
  const int tid = threadIdx.x;

  int nseg = nseg_p[h];
  nseg = nseg < ATT_MAXSEG ? nseg : ATT_MAXSEG;
  if (tid == 0) {
    int acc = 0;
    for (int s = 0; s < nseg; ++s) {
      const SegEntry e = segs[(int64_t)h * seg_cap + s];
      s_pre[s] = acc;
      s_k[s] = e.k;
      s_v[s] = e.v;
      acc += e.len;
    }
    s_pre[nseg] = acc;
  }
  __syncthreads();
  const int Lkv = s_pre[nseg];

  // query fragments (B operand of S^T = K Q^T)
  const int q0 = qt * 128 + w * ATT_QW;
  s16x8_t qf[2][NKS];
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

  f32x4_t o[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) o[db][qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-__builtin_inff(), -__builtin_inff()};
  float l_run[2] = {0.f, 0.f};

  const int ntile = (Lkv + ATT_TK - 1) / ATT_TK;
  for (int tile = 0; tile < ntile; ++tile) {
    const int kbase = tile * ATT_TK;
    // ---- stage K (row-major) and V (transposed) ----
    {
      // K: rows r = tid / CPR + (256 / CPR) * i
#pragma unroll
      for (int i = 0; i < ATT_TK * CPR / 256; ++i) {
        const int r = tid / CPR + (256 / CPR) * i;
        const int c = tid % CPR;
        const int j = kbase + r;
        u32x4_t val = {0u, 0u, 0u, 0u};
        if (j < Lkv) {
          const int s = seg_find(s_pre, nseg, j);
          const uint16_t* p = (const uint16_t*)s_k[s] + (int64_t)(j - s_pre[s]) * D + c * 8;
          val = *reinterpret_cast<const u32x4_t*>(p);
        }
        *reinterpret_cast<u32x4_t*>(sK + r * LDK + c * 8) = val;
      }
      // V: thread covers keys 4kg..4kg+3 and d 8dc..8dc+7
      if (tid < 16 * CPR) {
        const int kg = tid / CPR, dc = tid % CPR;
        uint16_t vv[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = kbase + 4 * kg + i;
          u32x4_t val = {0u, 0u, 0u, 0u};
          if (j < Lkv) {
            const int s = seg_find(s_pre, nseg, j);
            const uint16_t* p = (const uint16_t*)s_v[s] + (int64_t)(j - s_pre[s]) * D + dc * 8;
            val = *reinterpret_cast<const u32x4_t*>(p);
          }
          const uint16_t* e = reinterpret_cast<const uint16_t*>(&val);
#pragma unroll
          for (int x = 0; x < 8; ++x) vv[i][x] = e[x];
        }
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const uint32_t lo = (uint32_t)vv[0][x] | ((uint32_t)vv[1][x] << 16);
          const uint32_t hi = (uint32_t)vv[2][x] | ((uint32_t)vv[3][x] << 16);
          uint2 pk; pk.x = lo; pk.y = hi;
          *reinterpret_cast<uint2*>(sV + (8 * dc + x) * LDV + 4 * kg) = pk;
        }
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T ----
    f32x4_t s[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      s[kb][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const uint16_t* kp = sK + (16 * kb + (lane & 15)) * LDK;
#pragma unroll
      for (int k = 0; k < NKS; ++k) {
        const s16x8_t a = Op::load(kp + Op::off16(k, lane));
        s[kb][0] = Op::mma16(a, qf[0][k], s[kb][0]);
        s[kb][1] = Op::mma16(a, qf[1][k], s[kb][1]);
      }
    }
    // ---- online softmax (log2 domain), lane owns query 16qb + (lane & 15) ----
    const bool partial = kbase + ATT_TK > Lkv;
    s16x4_t pk[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = s[kb][qb][i] * scale_log2;
          if (partial && kbase + 16 * kb + 4 * g + i >= Lkv) v = -__builtin_inff();
          s[kb][qb][i] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m_run[qb], mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - mnew);
      m_run[qb] = mnew;
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = __builtin_amdgcn_exp2f(s[kb][qb][i] - mnew);
          ls += p[i];
        }
        s16x4_t v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (short)f32_to_bf16(p[i]);
        pk[qb][kb] = v;
      }
      l_run[qb] = l_run[qb] * alpha + ls;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db][qb] *= alpha;
    }
    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int hk = 0; hk < 2; ++hk) {
      s16x8_t b0, b1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        b0[i] = pk[0][2 * hk][i]; b0[4 + i] = pk[0][2 * hk + 1][i];
        b1[i] = pk[1][2 * hk][i]; b1[4 + i] = pk[1][2 * hk + 1][i];
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint16_t* vp = sV + (16 * db + (lane & 15)) * LDV + 32 * hk + 4 * g;
        const uint2 lo = *reinterpret_cast<const uint2*>(vp);
        const uint2 hi = *reinterpret_cast<const uint2*>(vp + 16);
        u32x4_t raw = {lo.x, lo.y, hi.x, hi.y};
        const s16x8_t a = __builtin_bit_cast(s16x8_t, raw);
        o[db][0] = Op::mma16(a, b0, o[db][0]);
        o[db][1] = Op::mma16(a, b1, o[db][1]);
      }
    }
    __syncthreads();
  }

  // ---- normalise and store: lane holds O[q][16db + 4g + i] ----
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float l = l_run[qb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const float inv = l > 0.f ? 1.0f / l : 0.0f;
    const int q = q0 + 16 * qb + (lane & 15);
    if (q < Lq) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d0 = 16 * db + 4 * g;
        const int64_t off = ((int64_t)h * Lq + q) * D + d0;
        if (out_f32) {
          float4 v = {o[db][qb][0] * inv, o[db][qb][1] * inv, o[db][qb][2] * inv, o[db][qb][3] * inv};
          *reinterpret_cast<float4*>((float*)O + off) = v;
        } else {
          uint2 pkv;
          pkv.x = (uint32_t)f32_to_bf16(o[db][qb][0] * inv) | ((uint32_t)f32_to_bf16(o[db][qb][1] * inv) << 16);
          pkv.y = (uint32_t)f32_to_bf16(o[db][qb][2] * inv) | ((uint32_t)f32_to_bf16(o[db][qb][3] * inv) << 16);
          *reinterpret_cast<uint2*>((uint16_t*)O + off) = pkv;
        }
      }
    }
  }
}

// fp32 reference-precision path (small shapes): one thread per (head, query)
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
  const int ns = nseg_p[h];
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

hipError_t launch_attention(const AttnLaunch& a, hipStream_t st) {
  if (a.Lq <= 0 || a.H <= 0) return hipSuccess;
  if (a.et == ET_BF16) {
    const int nqt = (a.Lq + 127) / 128;
    const float sl2 = a.scale * 1.4426950408889634f;
    const dim3 grid((unsigned)(nqt * a.H));
    if (a.d == 128)
      hipLaunchKernelGGL((attn_bf16_kernel<128>), grid, dim3(256), 0, st, (const uint16_t*)a.Q, a.O, a.segs, a.nseg,
                         a.seg_cap, a.Lq, sl2, a.out_f32, nqt);
    else
      hipLaunchKernelGGL((attn_bf16_kernel<64>), grid, dim3(256), 0, st, (const uint16_t*)a.Q, a.O, a.segs, a.nseg,
                         a.seg_cap, a.Lq, sl2, a.out_f32, nqt);
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
