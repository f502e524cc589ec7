// Memory-key write path: rows that leave the local window become bank
// candidates, and the arriving rows take their ring slots.
//
// DensityKV paper summary, supplementary "Post-RoPE Attention Geometry": the
// backbones zero the temporal rotary coordinate of non-local memory keys and
// keep their spatial coordinates, and the bank stores those post-RoPE keys.
// Method, "Online Density-Constrained Bank Update": the candidates are the
// frames that leave the window.  A key written into the window at temporal
// coordinate t therefore enters the bank with each temporal rotary pair
// (x_2i, x_2i+1), i < n_t, turned by -t * base^(-i / n_t); the spatial pairs
// and the value are copied bit for bit.  Pair layout (a reading): interleaved
// pairs, n_t = d/2 - 2 floor(d/6) temporal pairs first.
//
// One thread per 16-byte chunk of one row of one head: it reads the chunk of
// K and of V from the ring, writes the candidate chunks, then writes the
// arriving rows' chunks into the same slot.  HBM-bound streaming copy; only
// chunks that hold temporal pairs do arithmetic (angles in double, so that
// coordinates of a few dozen radians lose nothing to range reduction).
#include "kvb_common.hpp"
#include "kvb_launch.hpp"

namespace kvb {

template <typename E>
__global__ __launch_bounds__(256) void window_advance_kernel(WindowLaunch a) {
  constexpr int EPC = 16 / (int)sizeof(E);   // elements per chunk
  const int cpr = a.d / EPC;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)a.H * a.n_rows * cpr;
  if (idx >= total) return;
  const int c = (int)(idx % cpr);
  const int64_t hr = idx / cpr;
  const int r = (int)(hr % a.n_rows);
  const int h = (int)(hr / a.n_rows);
  const int slot = (int)(((int64_t)a.start + r) % a.cap);
  const int64_t src = ((int64_t)h * a.cap + slot) * a.d + (int64_t)c * EPC;
  const int64_t dst = ((int64_t)h * a.n_rows + r) * a.d + (int64_t)c * EPC;
  u32x4_t kc = *reinterpret_cast<const u32x4_t*>((const E*)a.ring_k + src);
  const u32x4_t vc = *reinterpret_cast<const u32x4_t*>((const E*)a.ring_v + src);
  const int nt = a.d / 2 - 2 * (a.d / 6);
  const int p0 = c * EPC / 2;                // first pair of the chunk
  if (p0 < nt) {
    const double t = (double)(a.t_first + r / a.F);
    E* e = reinterpret_cast<E*>(&kc);
#pragma unroll
    for (int j = 0; j < EPC / 2; ++j) {
      const int i = p0 + j;
      if (i < nt) {
        const double w = exp2(-(double)i / (double)nt * a.log2_base);
        double s, co;
        sincos(-t * w, &s, &co);
        const double x = (double)Ops<E>::to_f32(e[2 * j]);
        const double y = (double)Ops<E>::to_f32(e[2 * j + 1]);
        const float xr = (float)(co * x - s * y);
        const float yr = (float)(s * x + co * y);
        if constexpr (sizeof(E) == 2) {
          e[2 * j] = f32_to_bf16(xr);
          e[2 * j + 1] = f32_to_bf16(yr);
        } else {
          e[2 * j] = xr;
          e[2 * j + 1] = yr;
        }
      }
    }
  }
  *reinterpret_cast<u32x4_t*>((E*)a.cand_k + dst) = kc;
  *reinterpret_cast<u32x4_t*>((E*)a.cand_v + dst) = vc;
  if (a.new_k) {
    *reinterpret_cast<u32x4_t*>((E*)a.ring_k + src) = *reinterpret_cast<const u32x4_t*>((const E*)a.new_k + dst);
    *reinterpret_cast<u32x4_t*>((E*)a.ring_v + src) = *reinterpret_cast<const u32x4_t*>((const E*)a.new_v + dst);
  }
}

hipError_t launch_window_advance(const WindowLaunch& a, hipStream_t st) {
  const int epc = a.et == ET_BF16 ? 8 : 4;
  const int64_t total = (int64_t)a.H * a.n_rows * (a.d / epc);
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (a.et == ET_BF16) hipLaunchKernelGGL(window_advance_kernel<uint16_t>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(window_advance_kernel<float>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvb
