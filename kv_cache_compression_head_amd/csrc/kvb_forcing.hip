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

constexpr int COS_MAXC = 16;   // 16-byte chunks per lane (<= 64 heads x 16 chunks)

struct CosArgs {
  const void* hist; const void* nxt;
  int32_t H, d, F, T, nxt_rows, ndyn;
  int32_t dyn_heads[64];
  float* cosbuf;
};

// one wave per token position p: walks frames 0..T, keeping the previous
// frame's chunks in registers
template <typename E>
__global__ __launch_bounds__(256) void cos_kernel(CosArgs a) {
  constexpr int EPC = 16 / sizeof(E);
  const int lane = lane_id();
  const int p = blockIdx.x * 4 + wave_id();
  if (p >= a.F) return;
  const int cpr = a.d / EPC;
  const int nch = a.ndyn * cpr;
  u32x4_t prev[COS_MAXC];
  float nprev = 0.f;
  for (int t = 0; t <= a.T; ++t) {
    float nn = 0.f, dot = 0.f;
#pragma unroll
    for (int k = 0; k < COS_MAXC; ++k) {
      const int c = lane + 64 * k;
      if (64 * k >= nch) break;
      u32x4_t cur = {0u, 0u, 0u, 0u};
      if (c < nch) {
        const int hd = a.dyn_heads[c / cpr];
        const int cc = c % cpr;
        const E* base;
        if (t < a.T) base = (const E*)a.hist + (((int64_t)hd * a.T * a.F) + (int64_t)t * a.F + p) * a.d;
        else base = (const E*)a.nxt + ((int64_t)hd * a.nxt_rows + p) * a.d;
        cur = *reinterpret_cast<const u32x4_t*>(base + cc * EPC);
      }
      const E* e = reinterpret_cast<const E*>(&cur);
      const E* f = reinterpret_cast<const E*>(&prev[k]);
#pragma unroll
      for (int j = 0; j < EPC; ++j) {
        const float x = Ops<E>::to_f32(e[j]);
        nn = __builtin_fmaf(x, x, nn);
        if (t > 0) dot = __builtin_fmaf(x, Ops<E>::to_f32(f[j]), dot);
      }
      prev[k] = cur;
    }
    nn = wave_sum(nn);
    if (t > 0) {
      dot = wave_sum(dot);
      const float den = fmaxf(sqrtf(nprev) * sqrtf(nn), 1e-8f);
      if (lane == 0) a.cosbuf[(int64_t)(t - 1) * a.F + p] = dot / den;
    }
    nprev = nn;
  }
}

// segment means: one work-group per (frame, segment) item, fixed-order sum
__global__ __launch_bounds__(256) void segmean_kernel(const float* __restrict__ cosbuf, int F, int seg_len, int ndyn,
                                                      CosArgs a, float* __restrict__ scores, int64_t shs) {
  const int item = blockIdx.x;
  const int nseg = F / seg_len;
  const int t = item / nseg, j = item % nseg;
  const float* src = cosbuf + (int64_t)t * F + (int64_t)j * seg_len;
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
  const dim3 grid((unsigned)((c.F + 3) / 4));
  if (c.et == ET_BF16) hipLaunchKernelGGL(cos_kernel<uint16_t>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(cos_kernel<float>, grid, dim3(256), 0, st, a);
  const int items = c.T * (c.F / c.seg_len);
  hipLaunchKernelGGL(segmean_kernel, dim3(items), dim3(256), 0, st, c.cosbuf, c.F, c.seg_len, c.ndyn, a, c.scores,
                     c.score_hstride);
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
