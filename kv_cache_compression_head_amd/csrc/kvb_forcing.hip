// Forcing-KV dynamic-head segment similarity.
//
// Forcing-KV notes page, section 3.4 and the section 3.5 sketch: each history
// frame is cut into contiguous segments; a segment scores the mean over its
// tokens of the cosine similarity between the token's key in frame t and in
// frame t+1 (the last history frame pairs with the first frame of the new
// chunk); a token's key concatenates all dynamic heads, so one score list is
// shared by the dynamic heads of the layer.  HBM-bound streaming reduction:
// every key of the chain is read once.
#include "kvb_common.hpp"
#include "kvb_launch.hpp"

namespace kvb {


#ifndef COS_ROWS_NF
#define COS_ROWS_NF 4
#endif
#ifndef COS_ROWS_NH
#define COS_ROWS_NH 8
#endif

struct CosArgs {
  const void* hist; const void* nxt;
  int32_t H, d, F, T, nxt_rows, ndyn;
  int32_t dyn_heads[64];
  float* cosbuf;
  int64_t hist_ls, nxt_ls;   // layer strides (elements); layer = blockIdx.z
};

// One wave per (token position p, group of U cosines).  The wave's lanes
// hold the token's features over the dynamic heads as 16-byte chunks (chunk
// lane + 64 k, k < KC).  Group g computes the cosines of frame pairs
// (t, t + 1) for t in [g U, g U + U): it loads its U + 1 frames at once
// (one frame shared with the next group) before reducing any of them, so
// every wave keeps (U + 1) KC loads in flight and the token's frames are
// spread over several waves; the kernel is bound by HBM, not by the
// reductions.
template <typename E, int KC>
__global__ __launch_bounds__(256) void cos_kernel(CosArgs a) {
  constexpr int EPC = 16 / sizeof(E);
  constexpr int U = KC >= 16 ? 1 : 16 / KC;   // cosines per wave
  const int lane = lane_id();
  const int p = blockIdx.x * 4 + wave_id();
  if (p >= a.F) return;
  const int t0 = blockIdx.y * U;              // first frame of the group
  const int layer = blockIdx.z;
  const E* hist = (const E*)a.hist + layer * a.hist_ls;
  const E* nxt = (const E*)a.nxt + layer * a.nxt_ls;
  float* cosbuf = a.cosbuf + (int64_t)layer * a.T * a.F;
  const int cpr = a.d / EPC;
  const int nch = a.ndyn * cpr;
  // element offsets of this lane's chunks: frame 0 of the history, and the
  // first row of the next chunk
  int64_t hoff[KC], noff[KC];
  bool ok[KC];
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    const int c = lane + 64 * k;
    ok[k] = c < nch;
    const int hd = ok[k] ? a.dyn_heads[c / cpr] : 0;
    const int cc = ok[k] ? c % cpr : 0;
    hoff[k] = ((int64_t)hd * a.T * a.F + p) * a.d + cc * EPC;
    noff[k] = ((int64_t)hd * a.nxt_rows + p) * a.d + cc * EPC;
  }
  const int64_t fstride = (int64_t)a.F * a.d;
  u32x4_t fr[U + 1][KC];
#pragma unroll
  for (int u = 0; u <= U; ++u) {
    const int t = t0 + u;
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      fr[u][k] = u32x4_t{0u, 0u, 0u, 0u};
      if (ok[k] && t <= a.T) {
        const E* src = t < a.T ? hist + hoff[k] + t * fstride : nxt + noff[k];
        fr[u][k] = *reinterpret_cast<const u32x4_t*>(src);
      }
    }
  }
  float nprev = 0.f;
#pragma unroll
  for (int u = 0; u <= U; ++u) {
    const int t = t0 + u;
    if (t > a.T) break;
    float nn = 0.f, dot = 0.f;
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      const E* e = reinterpret_cast<const E*>(&fr[u][k]);
      const E* f = reinterpret_cast<const E*>(&fr[u > 0 ? u - 1 : 0][k]);
#pragma unroll
      for (int j = 0; j < EPC; ++j) {
        const float x = Ops<E>::to_f32(e[j]);
        nn = __builtin_fmaf(x, x, nn);
        if (u > 0) dot = __builtin_fmaf(x, Ops<E>::to_f32(f[j]), dot);
      }
    }
    nn = wave_sum(nn);
    if (u > 0) {
      dot = wave_sum(dot);
      const float den = fmaxf(sqrtf(nprev) * sqrtf(nn), 1e-8f);
      if (lane == 0) cosbuf[(int64_t)(t - 1) * a.F + p] = dot / den;
    }
    nprev = nn;
  }
}

// Row-group form for up to NH dynamic heads: CPR lanes hold one token's
// key row of one head (16 bytes each), so every load instruction of a wave
// reads 64 / CPR consecutive token rows of one head, one contiguous piece.
// A work-group takes 4 (64 / CPR) consecutive tokens and NF consecutive
// frames (NF - 1 frame pairs; the last frame is shared with the next
// group), and issues all NF x NH loads of a lane before reducing any of
// them.  Per lane the heads' partial sums are added in head order, then the
// CPR lanes of the row are added by a butterfly.
template <typename E, int CPR, int NH, int NF>
__global__ __launch_bounds__(256) void cos_rows_kernel(CosArgs a) {
  constexpr int EPC = 16 / sizeof(E);
  constexpr int TPW = 64 / CPR;   // tokens per wave
  const int lane = lane_id(), w = wave_id();
  const int c = lane % CPR;
  const int p = (blockIdx.x * 4 + w) * TPW + lane / CPR;
  const bool okp = p < a.F;
  const int t0 = blockIdx.y * (NF - 1);   // first frame of the group
  const int layer = blockIdx.z;
  const E* hist = (const E*)a.hist + layer * a.hist_ls;
  const E* nxt = (const E*)a.nxt + layer * a.nxt_ls;
  float* cosbuf = a.cosbuf + (int64_t)layer * a.T * a.F;
  u32x4_t fr[NF][NH];
#pragma unroll
  for (int u = 0; u < NF; ++u) {
    const int t = t0 + u;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      fr[u][h] = u32x4_t{0u, 0u, 0u, 0u};
      if (h < a.ndyn && okp && t <= a.T) {
        const int hd = a.dyn_heads[h];
        const E* src = t < a.T ? hist + (((int64_t)hd * a.T + t) * a.F + p) * a.d + c * EPC
                               : nxt + ((int64_t)hd * a.nxt_rows + p) * a.d + c * EPC;
        fr[u][h] = *reinterpret_cast<const u32x4_t*>(src);
      }
    }
  }
  float nprev = 0.f;
#pragma unroll
  for (int u = 0; u < NF; ++u) {
    const int t = t0 + u;
    float nn = 0.f, dot = 0.f;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const E* e = reinterpret_cast<const E*>(&fr[u][h]);
      const E* f = reinterpret_cast<const E*>(&fr[u > 0 ? u - 1 : 0][h]);
#pragma unroll
      for (int j = 0; j < EPC; ++j) {
        const float x = Ops<E>::to_f32(e[j]);
        nn = __builtin_fmaf(x, x, nn);
        if (u > 0) dot = __builtin_fmaf(x, Ops<E>::to_f32(f[j]), dot);
      }
    }
#pragma unroll
    for (int o = CPR / 2; o >= 1; o >>= 1) {
      nn += __shfl_xor(nn, o);
      if (u > 0) dot += __shfl_xor(dot, o);
    }
    if (u > 0 && c == 0 && okp && t <= a.T) {
      const float den = fmaxf(sqrtf(nprev) * sqrtf(nn), 1e-8f);
      cosbuf[(int64_t)(t - 1) * a.F + p] = dot / den;
    }
    nprev = nn;
  }
}

// segment means: one work-group per (frame, segment) item, fixed-order sum
__global__ __launch_bounds__(256) void segmean_kernel(const float* __restrict__ cosbuf, int F, int seg_len, int ndyn,
                                                      CosArgs a, float* __restrict__ scores, int64_t shs,
                                                      int64_t score_ls) {
  const int item = blockIdx.x;
  const int layer = blockIdx.y;
  const int nseg = F / seg_len;
  const int t = item / nseg, j = item % nseg;
  const float* src = cosbuf + (int64_t)layer * a.T * F + (int64_t)t * F + (int64_t)j * seg_len;
  scores += layer * score_ls;
  __shared__ float red[256];
  float s = 0.f;
  for (int i = threadIdx.x; i < seg_len; i += 256) s += src[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o >= 1; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if ((int)threadIdx.x < ndyn) scores[(int64_t)a.dyn_heads[threadIdx.x] * shs + item] = red[0] / (float)seg_len;
}

hipError_t launch_segment_cosine(const CosLaunch& c, hipStream_t st) {
  if (c.ndyn <= 0 || c.T <= 0) return hipSuccess;
  CosArgs a;
  a.hist = c.hist; a.nxt = c.nxt; a.H = c.H; a.d = c.d; a.F = c.F; a.T = c.T; a.nxt_rows = c.nxt_rows;
  a.ndyn = c.ndyn;
  for (int i = 0; i < 64; ++i) a.dyn_heads[i] = c.dyn_heads[i];
  a.cosbuf = c.cosbuf;
  a.hist_ls = c.nlayers > 1 ? c.hist_ls : 0;
  a.nxt_ls = c.nlayers > 1 ? c.nxt_ls : 0;
  const unsigned nl = (unsigned)(c.nlayers > 1 ? c.nlayers : 1);
  const int cpr = c.d * (c.et == ET_BF16 ? 2 : 4) / 16;
  if (c.ndyn <= COS_ROWS_NH && (cpr == 8 || cpr == 16 || cpr == 32)) {
    constexpr int NF = COS_ROWS_NF;
    const dim3 g((unsigned)((c.F + 4 * (64 / cpr) - 1) / (4 * (64 / cpr))), (unsigned)((c.T + NF - 2) / (NF - 1)),
                 nl);
#define KVB_COSR(E)                                                                                           \
  if (cpr == 8) hipLaunchKernelGGL((cos_rows_kernel<E, 8, COS_ROWS_NH, NF>), g, dim3(256), 0, st, a);        \
  else if (cpr == 16) hipLaunchKernelGGL((cos_rows_kernel<E, 16, COS_ROWS_NH, NF>), g, dim3(256), 0, st, a); \
  else hipLaunchKernelGGL((cos_rows_kernel<E, 32, COS_ROWS_NH, NF>), g, dim3(256), 0, st, a);
    if (c.et == ET_BF16) {
      KVB_COSR(uint16_t)
    } else {
      KVB_COSR(float)
    }
#undef KVB_COSR
  } else {
  const int kc = (c.ndyn * cpr + 63) / 64;   // <= 16 (checked on the host)
  const int kcp = kc <= 1 ? 1 : kc <= 2 ? 2 : kc <= 4 ? 4 : kc <= 8 ? 8 : 16;
  const int U = kcp >= 16 ? 1 : 16 / kcp;   // cosines per wave, as in the kernel
  const dim3 grid((unsigned)((c.F + 3) / 4), (unsigned)((c.T + U - 1) / U), nl);
#define KVB_COS(E)                                                                                 \
  if (kcp == 1) hipLaunchKernelGGL((cos_kernel<E, 1>), grid, dim3(256), 0, st, a);                 \
  else if (kcp == 2) hipLaunchKernelGGL((cos_kernel<E, 2>), grid, dim3(256), 0, st, a);            \
  else if (kcp == 4) hipLaunchKernelGGL((cos_kernel<E, 4>), grid, dim3(256), 0, st, a);            \
  else if (kcp == 8) hipLaunchKernelGGL((cos_kernel<E, 8>), grid, dim3(256), 0, st, a);            \
  else hipLaunchKernelGGL((cos_kernel<E, 16>), grid, dim3(256), 0, st, a);
  if (c.et == ET_BF16) {
    KVB_COS(uint16_t)
  } else {
    KVB_COS(float)
  }
#undef KVB_COS
  }
  const int items = c.T * (c.F / c.seg_len);
  hipLaunchKernelGGL(segmean_kernel, dim3(items, nl), dim3(256), 0, st, c.cosbuf, c.F, c.seg_len, c.ndyn, a, c.scores,
                     c.score_hstride, nl > 1 ? c.score_ls : 0);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Offline head profiling (Forcing-KV notes page, section 3.2).  The mass of a
// region is attention with one-hot values: O[q][r] = sum of query q's softmax
// weights on region r's keys.  The profile points every segment's values at
// a block of one-hot rows for its region, runs the attention kernels, and
// sums O[.][0..3] over the queries.
// ---------------------------------------------------------------------------
template <typename E>
__global__ void onehot_fill_kernel(E* __restrict__ ind, int64_t rows, int d) {
  // ind [4][rows][d]: block r holds rows with a one in column r
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= 4 * rows * d) return;
  const int c = (int)(i % d);
  const int r = (int)(i / (rows * d));
  if constexpr (sizeof(E) == 2) ind[i] = c == r ? (uint16_t)0x3F80 : (uint16_t)0;
  else ind[i] = c == r ? 1.0f : 0.0f;
}

__global__ void profile_segs_kernel(const SegEntry* __restrict__ segs, const int32_t* __restrict__ nseg,
                                    const int32_t* __restrict__ region, int H, int seg_cap, int64_t max_len,
                                    const char* ind, int64_t block_bytes, SegEntry* __restrict__ out,
                                    int32_t* __restrict__ bad) {
  const int h = blockIdx.x;
  if (h >= H) return;
  const int ns = min(nseg[h], seg_cap);
  for (int s = threadIdx.x; s < ns; s += blockDim.x) {
    const int64_t e = (int64_t)h * seg_cap + s;
    SegEntry x = segs[e];
    const int r = region[e];
    const bool ok = (unsigned)r < 4u && x.len <= max_len;
    if (!ok) {
      atomicOr(&bad[h], 1);
      x.len = 0;                          // nothing read past the one-hot block
    }
    x.v = ind + (int64_t)(ok ? r : 0) * block_bytes;
    out[e] = x;
  }
}

__global__ __launch_bounds__(256) void profile_reduce_kernel(const float* __restrict__ O, int Lq, int d, float alpha,
                                                             const int32_t* __restrict__ bad,
                                                             float* __restrict__ mass, float* __restrict__ score,
                                                             uint8_t* __restrict__ label) {
  const int h = blockIdx.x;
  __shared__ double red[4][256];
  double m[4] = {0.0, 0.0, 0.0, 0.0};
  for (int q = threadIdx.x; q < Lq; q += 256) {
    const float* o = O + ((int64_t)h * Lq + q) * d;
#pragma unroll
    for (int r = 0; r < 4; ++r) m[r] += (double)o[r];
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) red[r][threadIdx.x] = m[r];
  __syncthreads();
  for (int o = 128; o >= 1; o >>= 1) {
    if ((int)threadIdx.x < o) {
#pragma unroll
      for (int r = 0; r < 4; ++r) red[r][threadIdx.x] += red[r][threadIdx.x + o];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double tot = red[0][0] + red[1][0] + red[2][0] + red[3][0];
    const double sc = (red[3][0] + red[2][0]) / (tot - red[1][0]);
    const bool ok = bad[h] == 0;
    if (mass) {
#pragma unroll
      for (int r = 0; r < 4; ++r) mass[h * 4 + r] = (float)red[r][0];
    }
    score[h] = ok ? (float)sc : __builtin_nanf("");
    // static (1) when the score exceeds alpha, dynamic (2) otherwise; 0xFF when invalid
    label[h] = ok ? (sc > (double)alpha ? 1 : 2) : 0xFF;
  }
}

hipError_t launch_head_profile(const ProfileLaunch& p, hipStream_t st) {
  const int esz = p.a.et == ET_BF16 ? 2 : 4;
  const int64_t n = 4 * (int64_t)p.max_len * p.a.d;
  const int64_t block_bytes = (int64_t)p.max_len * p.a.d * esz;
  if (n > 0) {
    if (p.a.et == ET_BF16)
      hipLaunchKernelGGL(onehot_fill_kernel<uint16_t>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                         (uint16_t*)p.ind, (int64_t)p.max_len, p.a.d);
    else
      hipLaunchKernelGGL(onehot_fill_kernel<float>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                         (float*)p.ind, (int64_t)p.max_len, p.a.d);
  }
  hipError_t e = launch_fill_i32(p.bad, p.a.H, 0, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(profile_segs_kernel, dim3(p.a.H), dim3(64), 0, st, p.a.segs, p.a.nseg, p.region, p.a.H,
                     p.a.seg_cap, (int64_t)p.max_len, (const char*)p.ind, block_bytes, p.segs_out, p.bad);
  AttnLaunch a = p.a;
  a.segs = p.segs_out;
  a.O = p.O;
  a.out_f32 = 1;
  a.ws = nullptr;
  a.ws_bytes = 0;
  e = launch_attention(a, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(profile_reduce_kernel, dim3(p.a.H), dim3(256), 0, st, p.O, p.a.Lq, p.a.d, p.alpha, p.bad,
                     p.mass, p.score, p.label);
  return hipGetLastError();
}

}  // namespace kvb
