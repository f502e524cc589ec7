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

}  // namespace kvb
