// C-ABI of the kvbank library: argument checks, workspace layout and the
// launch sequence of one layer's scoring, bank update and chunk attention.
// Every check runs on the host before the first launch.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "kvb_launch.hpp"
#include "../../include/kvbank.h"

using namespace kvb;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return KVB_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

#define REQ_PTR(p, a, name)                                                         \
  do {                                                                              \
    if (!(p)) return fail(KVB_EINVAL, "%s is NULL", name);                          \
    if (!aligned((p), (a))) return fail(KVB_EINVAL, "%s is not %d-byte aligned", name, (int)(a)); \
  } while (0)

#define HIPCHK(expr)                                                                \
  do {                                                                              \
    hipError_t e_ = (expr);                                                         \
    if (e_ != hipSuccess) return fail(KVB_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

struct Heads {
  uint64_t dens = 0, stat = 0, dyn = 0;
  int ndyn = 0;
  int dyn_list[64];
};

int check_layer(const kvb_layer_desc* L, int32_t N, Heads* hd) {
  if (!L) return fail(KVB_EINVAL, "layer descriptor is NULL");
  if (L->H < 1 || L->H > KVB_MAX_HEADS) return fail(KVB_ESHAPE, "H=%d outside [1, %d]", L->H, KVB_MAX_HEADS);
  if (L->d != 64 && L->d != 128) return fail(KVB_ESHAPE, "d=%d (supported: 64, 128)", L->d);
  if (L->dtype != KVB_BF16 && L->dtype != KVB_F32) return fail(KVB_EDTYPE, "dtype=%d", L->dtype);
  if (L->frame_tokens <= 0) return fail(KVB_ESHAPE, "frame_tokens=%d", L->frame_tokens);
  if (L->M < 0) return fail(KVB_ESHAPE, "M=%d", L->M);
  if (N < 0) return fail(KVB_ESHAPE, "N=%d", N);
  if ((int64_t)N + (int64_t)L->M >= (int64_t)1 << 30) return fail(KVB_ESHAPE, "N + M too large");
  if (!L->label) return fail(KVB_EINVAL, "label is NULL");
  for (int h = 0; h < L->H; ++h) {
    const uint8_t lab = L->label[h];
    if (lab == KVB_HEAD_DENSITY) hd->dens |= 1ull << h;
    else if (lab == KVB_HEAD_STATIC) hd->stat |= 1ull << h;
    else if (lab == KVB_HEAD_DYNAMIC) {
      hd->dyn |= 1ull << h;
      hd->dyn_list[hd->ndyn++] = h;
    } else return fail(KVB_EPARAM, "label[%d]=%d (0 density, 1 static, 2 dynamic)", h, (int)lab);
  }
  const kvb_params& P = L->params;
  if (hd->dens) {
    if (L->M <= 0) return fail(KVB_ESHAPE, "density heads need M > 0");
    if (!(P.tau >= 1.0f)) return fail(KVB_EPARAM, "tau=%g must be >= 1", (double)P.tau);
    if (!(P.sigma > 0.0f) || !isfinite(P.sigma)) return fail(KVB_EPARAM, "sigma=%g must be > 0", (double)P.sigma);
    if (!(P.p >= 0.0f) || !isfinite(P.p)) return fail(KVB_EPARAM, "p=%g must be >= 0", (double)P.p);
    if (P.p > 0.0f && (!(P.eps > 0.0f) || !isfinite(P.eps)))
      return fail(KVB_EPARAM, "eps=%g must be > 0 when p > 0", (double)P.eps);
  }
  if (P.policy & ~KVB_POL_ALL) return fail(KVB_EPARAM, "policy=%#x has unknown bits", P.policy);
  if ((P.policy & KVB_POL_EVICT_DENSEST) && (P.policy & KVB_POL_EVICT_OLDEST))
    return fail(KVB_EPARAM, "policy: EVICT_DENSEST and EVICT_OLDEST exclude each other");
  if (hd->dyn) {
    if (P.seg_len <= 0 || L->frame_tokens % P.seg_len != 0)
      return fail(KVB_EPARAM, "seg_len=%d must divide frame_tokens=%d", P.seg_len, L->frame_tokens);
    if (!(P.retention >= 0.0 && P.retention <= 1.0)) return fail(KVB_EPARAM, "retention=%g not in [0,1]", P.retention);
  }
  if ((hd->dyn || hd->stat) && N % L->frame_tokens != 0)
    return fail(KVB_ESHAPE, "Forcing-KV heads need N (%d) to be a multiple of frame_tokens (%d)", N, L->frame_tokens);
  if (L->desc_dim != 0) {
    if (L->desc_dim != 64 && L->desc_dim != 128 && !(L->desc_dim == 256 && L->dtype == KVB_BF16))
      return fail(KVB_ESHAPE, "desc_dim=%d (supported: 0 = the keys, 64, 128; 256 for bf16)", L->desc_dim);
    if (hd->dyn || hd->stat) return fail(KVB_EPARAM, "density descriptors apply to density-only layers");
  }
  return KVB_OK;
}

int phi_mode_of(float p) {
  if (p == 2.0f) return PHI_P2;
  if (p == 0.0f) return PHI_P0;
  if (p == 1.0f) return PHI_P1;
  if (p == 4.0f) return PHI_P4;
  return PHI_GEN;
}

PhiConst phi_const(const kvb_params& P) {
  PhiConst c;
  c.inv_s2 = 1.0f / (P.sigma * P.sigma);
  c.c2 = -2.0f * c.inv_s2;
  c.eps = P.p > 0.0f ? P.eps : 0.0f;
  c.neg_half_p = -0.5f * P.p;
  int e2 = 0;
  const float s2 = P.sigma * P.sigma;
  c.direct = (P.p == 2.0f && frexpf(c.inv_s2, &e2) == 0.5f && c.inv_s2 * s2 == 1.0f && c.eps >= 1e-2f) ? 1 : 0;
  return c;
}

constexpr int SCAN_SUB = 32;      // candidates per scan subtile
constexpr int MAX_SPLITS = 8;

struct Layout {
  size_t normB, normC, augB, augC, k0, k1, v0, v1, t, cp, hist, rhoP, evict, surv, evl, fixl, nsurv, nfix,
      fmode, cnt, evsel, evblk, accS, accAE, accAA, colAA, cos, split, seqP, seqRR, seqTok, seqLog, seqAdm, seqFree,
      seqAlive, total;
  int kmax, cps, ncp;
};

size_t bump(size_t* off, size_t bytes) {
  const size_t at = *off;
  *off += (bytes + 255) & ~(size_t)255;
  return at;
}

Layout layout_of(const kvb_layer_desc* L, int32_t N) {
  Layout o{};
  const int64_t H = L->H, M = L->M;
  o.kmax = (int)(N < L->M ? N : L->M);
  const int64_t nsub = (o.kmax + SCAN_SUB - 1) / SCAN_SUB;
  o.cps = 8;
  while ((nsub + o.cps - 1) / o.cps > 256) o.cps *= 2;
  o.ncp = (int)((nsub + o.cps - 1) / o.cps) + 1;
  size_t off = 0;
  o.normB = bump(&off, H * M * 4);
  o.normC = bump(&off, H * N * 4);
  o.augB = bump(&off, H * M * 16);
  o.augC = bump(&off, H * N * 16);
  o.k0 = bump(&off, H * N * 8);
  o.k1 = bump(&off, H * N * 8);
  o.v0 = bump(&off, H * N * 4);
  o.v1 = bump(&off, H * N * 4);
  o.t = bump(&off, H * M * 4);
  o.cp = bump(&off, H * (int64_t)o.ncp * M * 4);
  o.hist = bump(&off, H * (int64_t)(o.kmax + 2) * 4);
  o.rhoP = bump(&off, H * M * 4);
  o.evict = bump(&off, H * M);
  o.surv = bump(&off, H * M * 4);
  o.evl = bump(&off, H * M * 4);
  o.fixl = bump(&off, H * M * 4);
  o.nsurv = bump(&off, H * 4);
  o.nfix = bump(&off, H * 4);
  o.fmode = bump(&off, H * 4);
  o.cnt = bump(&off, H * 4);
  o.evsel = bump(&off, H * 32);
  o.evblk = bump(&off, H * ((M + 255) / 256) * 4);
  o.accS = bump(&off, H * M * 4);
  o.accAE = bump(&off, H * (int64_t)o.kmax * 4);
  o.accAA = bump(&off, H * (int64_t)o.kmax * 4);
  // column-sum slices of the symmetric admitted x admitted Gram
  o.colAA = bump(&off, H * sym_head_floats(o.kmax) * 4);
  o.cos = bump(&off, (int64_t)N * 4);
  o.split = bump(&off, H * (int64_t)MAX_SPLITS * (N > L->M ? N : L->M) * 4);
  if (L->params.policy & KVB_POL_SEQUENTIAL) {
    // sequential admission: every head's pair interactions over its M + N states
    const int64_t S = M + N;
    o.seqP = bump(&off, H * S * S * 4);
    o.seqRR = bump(&off, H * S * 8);
    o.seqTok = bump(&off, H * S * 4);
    o.seqLog = bump(&off, H * (int64_t)N * 4);
    o.seqAdm = bump(&off, H * 4);
    o.seqFree = bump(&off, H * M * 4);
    o.seqAlive = bump(&off, H * (int64_t)N * 4);
  }
  o.total = off;
  return o;
}

template <typename T> T* at(void* ws, size_t off) { return reinterpret_cast<T*>((char*)ws + off); }

int check_bank(const kvb_bank* B, const kvb_layer_desc* L) {
  if (!B) return fail(KVB_EINVAL, "bank is NULL");
  REQ_PTR(B->K, 16, "bank.K");
  REQ_PTR(B->V, 16, "bank.V");
  REQ_PTR(B->tok, 4, "bank.tok");
  REQ_PTR(B->rho0, 4, "bank.rho0");
  REQ_PTR(B->rho, 4, "bank.rho");
  REQ_PTR(B->count, 4, "bank.count");
  if (L->desc_dim) REQ_PTR(B->X, 16, "bank.X (desc_dim > 0)");
  return KVB_OK;
}

// The density's rows: the keys, or the descriptor arrays when desc_dim > 0
struct DensRows {
  const void* bank;
  const void* cand;
  int dim;
};
int density_rows(const kvb_layer_desc* L, const kvb_bank* B, const void* cand_k, const kvb_kv_layout* lay,
                 DensRows* r) {
  if (!L->desc_dim) {
    *r = DensRows{B->K, cand_k, L->d};
    return KVB_OK;
  }
  if (!lay) return fail(KVB_EINVAL, "layout is NULL (desc_dim > 0 needs layout.cand_x)");
  REQ_PTR(lay->cand_x, 16, "layout.cand_x (desc_dim > 0)");
  *r = DensRows{B->X, lay->cand_x, L->desc_dim};
  return KVB_OK;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return KVB_OK;
  if (ws_bytes < need) return fail(KVB_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  REQ_PTR(ws, 16, "ws");
  return KVB_OK;
}

// Column splits for a gram launch.  Work-groups cost the same (one column
// range each), so the time is about rounds * columns-per-work-group, where a
// round is one work-group per slot (two per compute unit at the kernel's
// register use); pick the split count (up to MAX_SPLITS) that minimises it.
int choose_splits(int H, int rows, int ncols) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  const int64_t slots = 2LL * cus;
  const int64_t wgs = (int64_t)H * ((rows + 255) / 256);
  const int64_t tiles = (ncols + 63) / 64;
  int best = 1;
  int64_t best_cost = INT64_MAX;
  for (int s = 1; s <= MAX_SPLITS && s <= tiles; ++s) {
    const int64_t cost = ((wgs * s + slots - 1) / slots) * ((tiles + s - 1) / s);
    if (cost < best_cost) { best_cost = cost; best = s; }
  }
  return best;
}

// The symmetric self-Gram: row block b takes the tiles from 4b on, so the
// work-groups are uneven; the cost of s splits is the larger of the longest
// work-group and the average load per slot.
int choose_splits_sym(int H, int n) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  const int64_t slots = 3LL * cus;   // three four-wave work-groups per CU in this variant
  const int64_t tiles = (n + 63) / 64;
  const int blocks = (n + GRAM_ROW_BLOCK - 1) / GRAM_ROW_BLOCK;
  int best = 1;
  int64_t best_cost = INT64_MAX;
  for (int s = 1; s <= MAX_SPLITS && s <= tiles; ++s) {
    int64_t total = 0, longest = 0;
    for (int b = 0; b < blocks; ++b) {
      const int64_t t = (tiles - (int64_t)b * (GRAM_ROW_BLOCK / 64) + s - 1) / s;
      total += t * s;
      longest = t > longest ? t : longest;
    }
    const int64_t avg = (H * total + slots - 1) / slots;
    const int64_t cost = longest > avg ? longest : avg;
    if (cost < best_cost) { best_cost = cost; best = s; }
  }
  return best;
}

// one gram launch over rows_ub rows and at most cols_ub columns, with the
// column range split over work-groups when the row tiles alone cannot fill
// the device; split partials are summed in a fixed order
hipError_t run_gram(GramLaunch g, int H, int rows_ub, int cols_ub, float* dst, int64_t dst_hstride, float* split,
                    int64_t split_n, hipStream_t st) {
  g.splits = g.colsum ? choose_splits_sym(H, rows_ub) : choose_splits(H, rows_ub, cols_ub);
  if (g.splits > 1) {
    g.out = split;
    g.out_hstride = (int64_t)MAX_SPLITS * split_n;
    g.split_stride = split_n;
  } else {
    g.out = dst;
    g.out_hstride = dst_hstride;
    g.split_stride = 0;
  }
  hipError_t e = launch_gram(g, st);
  if (e != hipSuccess || g.splits == 1) return e;
  return launch_sum_splits(split, (int64_t)MAX_SPLITS * split_n, split_n, g.splits, dst, dst_hstride, H, rows_ub, st);
}

// ---------------------------------------------------------------------------
// Scratch of chunk_attention_noalloc: the balanced grid's partials and flags
// in a file-scope device array, one copy per GPU, held until the process
// ends.  Host code never uses the array's name as an address: the device
// address comes from hipGetSymbolAddress, once per device, and is kept here.
// ---------------------------------------------------------------------------
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)72 << 20;
constexpr int NOALLOC_MAX_DEVICES = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[NOALLOC_MAX_DEVICES] = {};

// the current device's address of `scratch` (looked up on the first call on
// that device, with the device current)
int scratch_on_current_device(void** out) {
  int dev = 0;
  HIPCHK(hipGetDevice(&dev));
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return fail(KVB_EHIP, "device %d beyond the scratch table", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    HIPCHK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(KVB_EHIP, "hipGetSymbolAddress returned NULL for the scratch array");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KVB_OK;
}

}  // namespace

extern "C" {

const char* kvb_last_error(void) { return g_err; }

#ifndef KVB_SOURCE_HASH
#define KVB_SOURCE_HASH "unknown"
#endif
const char* kvb_source_hash(void) { return KVB_SOURCE_HASH; }

int kvbank_workspace_size(const kvb_layer_desc* L, int32_t N, size_t* bytes) {
  Heads hd;
  int rc = check_layer(L, N, &hd);
  if (rc) return rc;
  if (!bytes) return fail(KVB_EINVAL, "bytes is NULL");
  *bytes = layout_of(L, N).total;
  return ok();
}

int kvbank_score(const kvb_layer_desc* L, const kvb_bank* bank, const void* cand_k, const int32_t* cand_tok,
                 int32_t N, const kvb_kv_layout* lay, float* out_D, float* out_score, int32_t* out_order, void* ws,
                 size_t ws_bytes, kvb_stream_t stream) {
  Heads hd;
  int rc = check_layer(L, N, &hd);
  if (rc) return rc;
  if (N == 0 || !(hd.dens || hd.dyn)) return ok();
  const Layout lo = layout_of(L, N);
  if ((rc = check_ws(ws, ws_bytes, lo.total))) return rc;
  REQ_PTR(cand_k, 16, "cand_k");
  REQ_PTR(out_score, 4, "out_score");
  REQ_PTR(out_order, 4, "out_order");
  if (hd.dens) {
    if ((rc = check_bank(bank, L))) return rc;
    REQ_PTR(cand_tok, 4, "cand_tok");
    REQ_PTR(out_D, 4, "out_D");
  }
  if (hd.dyn) {
    // the cosine kernel holds one token's features of every dynamic head in
    // one wave: at most 1,024 16-byte chunks (64 lanes x 16)
    const int chunks = hd.ndyn * (L->d * (L->dtype == KVB_BF16 ? 2 : 4) / 16);
    if (chunks > 1024)
      return fail(KVB_ESHAPE, "%d dynamic heads of d=%d %s exceed the cosine kernel's 16 KB per token", hd.ndyn,
                  L->d, L->dtype == KVB_BF16 ? "bf16" : "fp32");
    if (!lay) return fail(KVB_EINVAL, "layout is NULL (needed by dynamic heads)");
    REQ_PTR(lay->chunk_k, 16, "layout.chunk_k");
    if (lay->chunk_len < L->frame_tokens) return fail(KVB_ESHAPE, "chunk_len < frame_tokens");
  }
  hipStream_t st = (hipStream_t)stream;
  const int H = L->H, M = L->M, d = L->d, et = L->dtype;
  const PhiConst pc = phi_const(L->params);
  if (hd.dens) {
    DensRows dr{};
    if ((rc = density_rows(L, bank, cand_k, lay, &dr))) return rc;
    float* nB = at<float>(ws, lo.normB);
    float* nC = at<float>(ws, lo.normC);
    void* aB = at<void>(ws, lo.augB);
    void* aC = at<void>(ws, lo.augC);
    HIPCHK(launch_norms(dr.bank, M, nB, aB, dr.cand, N, nC, aC, et, H, dr.dim, pc.inv_s2, et == ET_BF16 && pc.direct,
                        st));
    GramLaunch g{};
    g.k = KeysDesc{dr.bank, dr.cand, nB, nC, aB, aC, M, N, dr.dim, H, et};
    g.rows = VList{nullptr, nullptr, 0, 0, 0, M, N, 0};
    g.cols = VList{nullptr, bank->count, 0, 1, 0, 0, M, 0};
    g.pc = pc;
    g.phi_mode = phi_mode_of(L->params.p);
    g.active = hd.dens;
    g.splits = choose_splits(H, N, M);
    if (g.splits > 1) {
      g.out = at<float>(ws, lo.split);
      g.out_hstride = (int64_t)MAX_SPLITS * N;
      g.split_stride = N;
    } else {
      g.out = out_D;
      g.out_hstride = N;
      g.split_stride = 0;
    }
    HIPCHK(launch_gram(g, st));
    if (g.splits > 1)
      HIPCHK(launch_sum_splits(g.out, (int64_t)MAX_SPLITS * N, N, g.splits, out_D, N, H, N, st));
    HIPCHK(launch_delta(out_D, bank->count, hd.dens, H, N, out_score, st));
    // order: ascending (delta, token id), or token id alone (source order)
    const float* key = (L->params.policy & KVB_POL_SOURCE_ORDER) ? nullptr : out_score;
    HIPCHK(launch_sort(key, N, cand_tok, 0, hd.dens, H, N, at<uint64_t>(ws, lo.k0), at<uint64_t>(ws, lo.k1),
                       at<int32_t>(ws, lo.v0), at<int32_t>(ws, lo.v1), out_order, N, st));
  }
  if (hd.dyn) {
    const int F = L->frame_tokens, T = N / F, seg = L->params.seg_len;
    CosLaunch c{};
    c.hist = cand_k; c.nxt = lay->chunk_k; c.et = et; c.H = H; c.d = d; c.F = F; c.T = T; c.seg_len = seg;
    c.nxt_rows = lay->chunk_len; c.ndyn = hd.ndyn;
    for (int i = 0; i < hd.ndyn; ++i) c.dyn_heads[i] = hd.dyn_list[i];
    c.cosbuf = at<float>(ws, lo.cos); c.scores = out_score; c.score_hstride = N;
    HIPCHK(launch_segment_cosine(c, st));
    const int items = T * (F / seg);
    if (L->params.policy & KVB_POL_FRAME_BOTTOMK) {
      // per-frame BottomK: items sorted by their rank inside their frame (then
      // by index), so that the first T floor(r n) are every frame's lowest
      float* rank = at<float>(ws, lo.cos);   // the cosine scratch is free again
      HIPCHK(launch_frame_rank(out_score + (int64_t)hd.dyn_list[0] * N, items, F / seg, rank, st));
      HIPCHK(launch_sort(rank, 0, nullptr, 0, hd.dyn, H, items, at<uint64_t>(ws, lo.k0), at<uint64_t>(ws, lo.k1),
                         at<int32_t>(ws, lo.v0), at<int32_t>(ws, lo.v1), out_order, N, st));
    } else {
      HIPCHK(launch_sort(out_score, N, nullptr, 0, hd.dyn, H, items, at<uint64_t>(ws, lo.k0),
                         at<uint64_t>(ws, lo.k1), at<int32_t>(ws, lo.v0), at<int32_t>(ws, lo.v1), out_order, N, st));
    }
  }
  return ok();
}

// Forcing-KV segment scoring of several layers that share one descriptor:
// the cosines, the segment means and the BottomK order of every layer in
// one launch each.
static int check_score_layers(const kvb_layer_desc* L, int32_t nlayers, int32_t N, Heads* hd) {
  int rc = check_layer(L, N, hd);
  if (rc) return rc;
  if (nlayers < 0 || nlayers > 65535) return fail(KVB_ESHAPE, "nlayers=%d outside [0, 65535]", nlayers);
  if (hd->dens) return fail(KVB_EPARAM, "kvbank_score_layers takes Forcing-KV layers only (no density heads)");
  if (L->params.policy & KVB_POL_FRAME_BOTTOMK)
    return fail(KVB_EPARAM, "kvbank_score_layers orders the items of the whole history (no KVB_POL_FRAME_BOTTOMK)");
  if (hd->dyn) {
    const int items = N / L->params.seg_len;
    if (items > 1024) return fail(KVB_EPARAM, "%d items per layer (at most 1,024)", items);
    const int chunks = hd->ndyn * (L->d * (L->dtype == KVB_BF16 ? 2 : 4) / 16);
    if (chunks > 1024)
      return fail(KVB_ESHAPE, "%d dynamic heads of d=%d %s exceed the cosine kernel's 16 KB per token", hd->ndyn,
                  L->d, L->dtype == KVB_BF16 ? "bf16" : "fp32");
  }
  return KVB_OK;
}

int kvbank_score_layers_workspace_size(const kvb_layer_desc* L, int32_t nlayers, int32_t N, size_t* bytes) {
  Heads hd;
  int rc = check_score_layers(L, nlayers, N, &hd);
  if (rc) return rc;
  if (!bytes) return fail(KVB_EINVAL, "bytes is NULL");
  // the cosine of every token and frame pair of every layer
  *bytes = hd.dyn ? (((size_t)nlayers * (size_t)N * 4 + 255) & ~(size_t)255) : 0;
  return ok();
}

int kvbank_score_layers(const kvb_layer_desc* L, int32_t nlayers, const void* cand_k, int64_t cand_layer_stride,
                        const void* chunk_k, int64_t chunk_layer_stride, int32_t chunk_len, int32_t N,
                        float* out_score, int32_t* out_order, void* ws, size_t ws_bytes, kvb_stream_t stream) {
  Heads hd;
  int rc = check_score_layers(L, nlayers, N, &hd);
  if (rc) return rc;
  if (N == 0 || nlayers == 0 || !hd.dyn) return ok();
  const int H = L->H, d = L->d, F = L->frame_tokens;
  REQ_PTR(cand_k, 16, "cand_k");
  REQ_PTR(chunk_k, 16, "chunk_k");
  REQ_PTR(out_score, 4, "out_score");
  REQ_PTR(out_order, 4, "out_order");
  if (chunk_len < F) return fail(KVB_ESHAPE, "chunk_len=%d < frame_tokens=%d", chunk_len, F);
  const int64_t esz = L->dtype == KVB_BF16 ? 2 : 4;
  if (cand_layer_stride < (int64_t)H * N * d || (cand_layer_stride * esz) % 16 != 0)
    return fail(KVB_ESHAPE, "cand_layer_stride=%lld (at least H N d, 16-byte multiple)", (long long)cand_layer_stride);
  if (chunk_layer_stride < (int64_t)H * chunk_len * d || (chunk_layer_stride * esz) % 16 != 0)
    return fail(KVB_ESHAPE, "chunk_layer_stride=%lld (at least H chunk_len d, 16-byte multiple)",
                (long long)chunk_layer_stride);
  size_t need = 0;
  if ((rc = kvbank_score_layers_workspace_size(L, nlayers, N, &need))) return rc;
  if ((rc = check_ws(ws, ws_bytes, need))) return rc;
  hipStream_t st = (hipStream_t)stream;
  const int T = N / F, seg = L->params.seg_len, items = N / seg;
  CosLaunch c{};
  c.hist = cand_k; c.nxt = chunk_k; c.et = L->dtype; c.H = H; c.d = d; c.F = F; c.T = T; c.seg_len = seg;
  c.nxt_rows = chunk_len; c.ndyn = hd.ndyn;
  for (int i = 0; i < hd.ndyn; ++i) c.dyn_heads[i] = hd.dyn_list[i];
  c.cosbuf = (float*)ws; c.scores = out_score; c.score_hstride = N;
  c.nlayers = nlayers; c.hist_ls = cand_layer_stride; c.nxt_ls = chunk_layer_stride; c.score_ls = (int64_t)H * N;
  HIPCHK(launch_segment_cosine(c, st));
  HIPCHK(launch_rank_sort_layers(out_score, N, (int64_t)H * N, hd.dyn, H, items, nlayers, out_order, N,
                                 (int64_t)H * N, st));
  return ok();
}

int kvbank_update(const kvb_layer_desc* L, kvb_bank* bank, const void* cand_k, const void* cand_v,
                  const int32_t* cand_tok, int32_t N, const float* D, const int32_t* order,
                  const kvb_kv_layout* lay, kvb_update_out* out, void* ws, size_t ws_bytes, kvb_stream_t stream) {
  Heads hd;
  int rc = check_layer(L, N, &hd);
  if (rc) return rc;
  const Layout lo = layout_of(L, N);
  if ((rc = check_ws(ws, ws_bytes, lo.total))) return rc;
  if (!lay) return fail(KVB_EINVAL, "layout is NULL");
  if (!out) return fail(KVB_EINVAL, "update output is NULL");
  REQ_PTR(out->k_star, 4, "out.k_star");
  REQ_PTR(out->n_mandatory, 4, "out.n_mandatory");
  REQ_PTR(out->n_evicted, 4, "out.n_evicted");
  REQ_PTR(out->status, 4, "out.status");
  REQ_PTR(out->segs, 8, "out.segs");
  REQ_PTR(out->nseg, 4, "out.nseg");
  if (out->t_cross && !aligned(out->t_cross, 4)) return fail(KVB_EINVAL, "out.t_cross is not 4-byte aligned");
  if (out->rho_proj && !aligned(out->rho_proj, 4)) return fail(KVB_EINVAL, "out.rho_proj is not 4-byte aligned");
  if (out->seg_cap > KVB_MAX_SEGMENTS) return fail(KVB_ESHAPE, "seg_cap=%d > %d", out->seg_cap, KVB_MAX_SEGMENTS);
  const int H = L->H, M = L->M, d = L->d, et = L->dtype, F = L->frame_tokens;
  const int has_sink = lay->sink_len > 0, has_chunk = lay->chunk_len > 0;
  if (lay->sink_len < 0 || lay->chunk_len < 0 || lay->win_len < 0 || lay->win_cap < 0)
    return fail(KVB_ESHAPE, "negative layout length");
  if (has_sink) { REQ_PTR(lay->sink_k, 16, "layout.sink_k"); REQ_PTR(lay->sink_v, 16, "layout.sink_v"); }
  if (has_chunk) { REQ_PTR(lay->chunk_k, 16, "layout.chunk_k"); REQ_PTR(lay->chunk_v, 16, "layout.chunk_v"); }
  if (lay->win_len > 0) {
    REQ_PTR(lay->win_k, 16, "layout.win_k");
    REQ_PTR(lay->win_v, 16, "layout.win_v");
    if (lay->win_len > lay->win_cap || lay->win_start < 0 || lay->win_start >= lay->win_cap)
      return fail(KVB_ESHAPE, "window ring: start=%d len=%d cap=%d", lay->win_start, lay->win_len, lay->win_cap);
  }
  int items = 0, keep = 0;
  if (hd.dyn) {
    items = (N / F) * (F / L->params.seg_len);
    if (L->params.policy & KVB_POL_FRAME_BOTTOMK) {
      const int nseg = F / L->params.seg_len;
      keep = (N / F) * (int)floor(L->params.retention * (double)nseg);
    } else {
      keep = (int)floor(L->params.retention * (double)items);
    }
  }
  {
    int need = 0;
    if (hd.dens) need = 4 + (lay->win_len > 0 ? 1 : 0);
    if (hd.stat) need = need > 3 ? need : 3;
    if (hd.dyn) need = need > 2 + keep ? need : 2 + keep;
    if (out->seg_cap < need) return fail(KVB_ESHAPE, "seg_cap=%d < %d needed", out->seg_cap, need);
  }
  if (hd.dens) {
    if ((rc = check_bank(bank, L))) return rc;
    if (N > 0) {
      REQ_PTR(cand_k, 16, "cand_k");
      REQ_PTR(cand_v, 16, "cand_v");
      REQ_PTR(cand_tok, 4, "cand_tok");
      REQ_PTR(D, 4, "D");
      REQ_PTR(order, 4, "order");
    }
  }
  if (hd.dyn && N > 0) REQ_PTR(order, 4, "order");
  if ((hd.stat || hd.dyn) && N > 0) { REQ_PTR(cand_k, 16, "cand_k"); REQ_PTR(cand_v, 16, "cand_v"); }

  hipStream_t st = (hipStream_t)stream;
  const PhiConst pc = phi_const(L->params);
  const int pm = phi_mode_of(L->params.p);
  const uint32_t pol = hd.dens ? L->params.policy : 0u;
  const int ks_hs = (pol & KVB_POL_HEAD_PREFIX) ? 1 : 0;
  {
    // outputs, and the crossing-time histogram when the density path runs
    const bool dens_run = hd.dens && N > 0;
    int32_t* zp[4] = {out->n_mandatory, out->n_evicted, out->k_star,
                      dens_run ? at<int32_t>(ws, lo.hist) : nullptr};
    const int64_t zn[4] = {H, H, ks_hs ? H : 1, (int64_t)H * (lo.kmax + 2)};
    if (dens_run) {
      // the update reads the bank's occupancy only through this clamped copy
      const CountClamp cc{bank->count, at<int32_t>(ws, lo.cnt), out->status, hd.dens, H, M};
      HIPCHK(launch_zero_i32_clamp(zp, zn, 4, cc, st));
    } else {
      HIPCHK(launch_zero_i32(zp, zn, 4, st));
    }
  }
  DensRows dr{};
  if (hd.dens && N > 0 && (rc = density_rows(L, bank, cand_k, lay, &dr))) return rc;
  if (hd.dens && N > 0 && (pol & KVB_POL_SEQUENTIAL)) {
    SeqLaunch q{};
    q.H = H; q.M = M; q.N = N; q.active = hd.dens; q.P = at<float>(ws, lo.seqP); q.cnt = at<int32_t>(ws, lo.cnt);
    q.rho = bank->rho; q.rho0 = bank->rho0; q.bank_tok = bank->tok; q.cand_tok = cand_tok; q.order = order;
    q.tau = L->params.tau; q.fill = (pol & KVB_POL_FILL_BELOW_CAP) ? 1 : 0;
    q.evict_mode = (pol & KVB_POL_EVICT_DENSEST) ? 1 : (pol & KVB_POL_EVICT_OLDEST) ? 2 : 0;
    q.per_head = ks_hs;
    q.st_rr = at<uint64_t>(ws, lo.seqRR); q.st_tok = at<int32_t>(ws, lo.seqTok); q.log = at<int32_t>(ws, lo.seqLog);
    q.n_adm = at<int32_t>(ws, lo.seqAdm); q.kstar = out->k_star; q.kstar_hs = ks_hs; q.n_ev = out->n_evicted;
    q.n_mand = out->n_mandatory; q.status = out->status;
    SeqGather g{};
    g.H = H; g.M = M; g.N = N; g.d = d; g.dx = d; g.et = et; g.active = hd.dens; g.cnt = q.cnt; g.st_rr = q.st_rr;
    g.st_tok = q.st_tok; g.log = q.log; g.n_adm = q.n_adm; g.freel = at<int32_t>(ws, lo.seqFree);
    g.alive = at<int32_t>(ws, lo.seqAlive); g.refresh = (pol & KVB_POL_REFRESH_BASELINE) ? 1 : 0;
    g.rho = bank->rho; g.rho0 = bank->rho0; g.bank_tok = bank->tok; g.count = bank->count;
    g.bankK = bank->K; g.bankV = bank->V; g.candK = cand_k; g.candV = cand_v;
    g.bankX = L->desc_dim ? bank->X : nullptr; g.candX = L->desc_dim ? lay->cand_x : nullptr; g.dx = dr.dim;
    g.cand_tok = cand_tok; g.status = out->status;
    HIPCHK(launch_sequential(q, g, dr.bank, dr.cand, dr.dim, pc, pm, st));
  } else if (hd.dens && N > 0) {
    const int kmax = lo.kmax;
    const int32_t* cnt = at<int32_t>(ws, lo.cnt);
    float* nB = at<float>(ws, lo.normB);
    float* nC = at<float>(ws, lo.normC);
    void* aB = at<void>(ws, lo.augB);
    void* aC = at<void>(ws, lo.augC);
    HIPCHK(launch_norms(dr.bank, M, nB, aB, dr.cand, N, nC, aC, et, H, dr.dim, pc.inv_s2, et == ET_BF16 && pc.direct,
                        st, NormCheck{out->status, cnt, hd.dens, 0, 0}));
    const KeysDesc kd{dr.bank, dr.cand, nB, nC, aB, aC, M, N, dr.dim, H, et};
    ScanLaunch s{};
    s.k = kd; s.rho = bank->rho; s.rho0 = bank->rho0; s.count = cnt; s.order = order;
    s.active = hd.dens; s.kmax = kmax; s.tau = L->params.tau; s.cps = lo.cps; s.ncp = lo.ncp;
    s.cp = at<float>(ws, lo.cp); s.kstar = out->k_star; s.kstar_hs = ks_hs;
    // crossed states survive with densest-only eviction, and below capacity
    // in the fill variant: their running sums and rho' are then needed
    s.keep_crossed = (pol & (KVB_POL_EVICT_DENSEST | KVB_POL_FILL_BELOW_CAP)) ? 1 : 0;
    s.t_out = out->t_cross ? out->t_cross : at<int32_t>(ws, lo.t);
    s.rhoP = out->rho_proj ? out->rho_proj : at<float>(ws, lo.rhoP);
    s.pc = pc; s.phi_mode = pm;
    // With min(N, M) = M every density head can admit k = M: e(M) = n covers
    // any crossed set, so k* = M and the whole bank leaves whatever crossed.
    // Unless the per-state diagnostics are asked for, the crossing scan, the
    // prefix search and the rho' pass decide nothing here and are skipped
    // (n_mandatory is then -1).
    const bool replace_all = kmax == M && !out->t_cross && !out->rho_proj;
    if (!replace_all) HIPCHK(launch_scan(s, false, st));
    SelectLaunch sel{};
    sel.H = H; sel.M = M; sel.kmax = kmax; sel.active = hd.dens; sel.count = cnt;
    sel.t = s.t_out; sel.hist = at<int32_t>(ws, lo.hist); sel.kstar = out->k_star; sel.rhoP = s.rhoP;
    sel.kstar_hs = ks_hs;
    sel.fill = (pol & KVB_POL_FILL_BELOW_CAP) ? 1 : 0;
    sel.evict_mode = (pol & KVB_POL_EVICT_DENSEST) ? 1 : (pol & KVB_POL_EVICT_OLDEST) ? 2 : 0;
    sel.bank_tok = bank->tok; sel.evict = at<uint8_t>(ws, lo.evict); sel.surv = at<int32_t>(ws, lo.surv);
    sel.evl = at<int32_t>(ws, lo.evl); sel.n_surv = at<int32_t>(ws, lo.nsurv); sel.n_ev = out->n_evicted;
    sel.n_mand = out->n_mandatory; sel.status = out->status;
    sel.fixl = at<int32_t>(ws, lo.fixl); sel.n_fix = at<int32_t>(ws, lo.nfix); sel.fmode = at<int32_t>(ws, lo.fmode);
    sel.evsel = at<void>(ws, lo.evsel); sel.evblk = at<int32_t>(ws, lo.evblk);
    sel.skip_cross = replace_all ? 1 : 0;
    if (replace_all) {
      HIPCHK(launch_fill_i32(out->k_star, ks_hs ? H : 1, kmax, st));
    } else {
      HIPCHK(launch_kstar(sel, st));
      HIPCHK(launch_scan(s, true, st));
    }
    HIPCHK(launch_evict(sel, st));
    // density fix-ups: survivors x evicted, admitted x evicted, admitted x admitted
    GramLaunch g{};
    g.k = kd; g.pc = pc; g.phi_mode = pm; g.splits = 1; g.split_stride = 0; g.active = hd.dens;
    const VList evl{sel.evl, sel.n_ev, M, 1, 0, 0, M, 0};
    const VList fxl{sel.fixl, sel.n_fix, M, 1, 0, 0, M, 0};
    const VList srv{sel.surv, sel.n_surv, M, 1, 0, 0, M, 0};
    const VList adm{order, out->k_star, N, ks_hs, M, 0, kmax, 0};
    float* split = at<float>(ws, lo.split);
    const int64_t sstride = (N > M ? N : M);
    g.rows = srv; g.cols = evl; g.self_excl = 0;
    HIPCHK(run_gram(g, H, M, kmax, at<float>(ws, lo.accS), M, split, sstride, st));
    g.rows = adm; g.cols = fxl;
    HIPCHK(run_gram(g, H, kmax, M, at<float>(ws, lo.accAE), kmax, split, sstride, st));
    // admitted x admitted is symmetric: each unordered pair once, the
    // mirrored half through column sums added back in order
    g.rows = adm; g.cols = adm; g.self_excl = 1;
    g.colsum = at<float>(ws, lo.colAA); g.col_ld = kmax;
    HIPCHK(run_gram(g, H, kmax, kmax, at<float>(ws, lo.accAA), kmax, split, sstride, st));
    HIPCHK(launch_sym_combine(at<float>(ws, lo.accAA), kmax, g.colsum, kmax,
                              (kmax + GRAM_ROW_BLOCK - 1) / GRAM_ROW_BLOCK, adm, hd.dens, H, kmax, st));
    g.colsum = nullptr;
    ApplyLaunch ap{};
    ap.H = H; ap.M = M; ap.N = N; ap.d = d; ap.et = et; ap.kmax = kmax; ap.active = hd.dens;
    ap.bankK = bank->K; ap.bankV = bank->V; ap.bank_tok = bank->tok; ap.rho0 = bank->rho0; ap.rho = bank->rho;
    ap.count = bank->count; ap.candK = cand_k; ap.candV = cand_v; ap.cand_tok = cand_tok; ap.order = order;
    ap.bankX = L->desc_dim ? bank->X : nullptr; ap.candX = L->desc_dim ? lay->cand_x : nullptr; ap.dx = L->desc_dim;
    ap.D = D; ap.kstar = out->k_star; ap.kstar_hs = ks_hs;
    ap.refresh = (pol & KVB_POL_REFRESH_BASELINE) ? 1 : 0; ap.surv = sel.surv; ap.n_surv = sel.n_surv; ap.evl = sel.evl;
    ap.n_ev = sel.n_ev; ap.rhoP = s.rhoP; ap.acc_surv = at<float>(ws, lo.accS);
    ap.acc_adm_ev = at<float>(ws, lo.accAE); ap.acc_adm_adm = at<float>(ws, lo.accAA); ap.fmode = sel.fmode;
    HIPCHK(launch_apply(ap, st));
  }
  SegLaunch sg{};
  sg.H = H; sg.d = d; sg.et = et; sg.M = M; sg.N = N; sg.F = F;
  for (int h = 0; h < H; ++h) sg.label[h] = L->label[h];
  sg.sink_k = lay->sink_k; sg.sink_v = lay->sink_v; sg.sink_len = lay->sink_len;
  sg.win_k = lay->win_k; sg.win_v = lay->win_v; sg.win_cap = lay->win_cap; sg.win_start = lay->win_start;
  sg.win_len = lay->win_len;
  sg.chunk_k = lay->chunk_k; sg.chunk_v = lay->chunk_v; sg.chunk_len = lay->chunk_len;
  sg.bankK = hd.dens ? bank->K : nullptr; sg.bankV = hd.dens ? bank->V : nullptr;
  sg.count = hd.dens ? bank->count : nullptr;
  sg.candK = cand_k; sg.candV = cand_v;
  sg.dyn_order = order; sg.dyn_order_hstride = N;
  sg.seg_len = hd.dyn ? L->params.seg_len : 1; sg.items = items; sg.keep = keep;
  sg.segs = reinterpret_cast<SegEntry*>(out->segs); sg.nseg = out->nseg; sg.seg_cap = out->seg_cap;
  sg.status = out->status;
  HIPCHK(launch_segments(sg, st));
  return ok();
}

int chunk_attention(const kvb_attn_desc* A, const void* Q, const kvb_segment* segs, const int32_t* nseg, void* O,
                    void* ws, size_t ws_bytes, kvb_stream_t stream) {
  if (!A) return fail(KVB_EINVAL, "attention descriptor is NULL");
  if (A->H < 1 || A->H > KVB_MAX_HEADS) return fail(KVB_ESHAPE, "H=%d", A->H);
  if (A->d != 64 && A->d != 128) return fail(KVB_ESHAPE, "d=%d (supported: 64, 128)", A->d);
  if (A->dtype != KVB_BF16 && A->dtype != KVB_F32) return fail(KVB_EDTYPE, "dtype=%d", A->dtype);
  if (A->Lq < 0) return fail(KVB_ESHAPE, "Lq=%d", A->Lq);
  if (A->seg_cap < 1 || A->seg_cap > KVB_MAX_SEGMENTS) return fail(KVB_ESHAPE, "seg_cap=%d", A->seg_cap);
  if (A->Lq == 0) return ok();
  REQ_PTR(Q, 16, "Q");
  REQ_PTR(O, 16, "O");
  REQ_PTR(segs, 8, "segs");
  REQ_PTR(nseg, 4, "nseg");
  AttnLaunch a{};
  a.H = A->H; a.d = A->d; a.Lq = A->Lq; a.et = A->dtype; a.out_f32 = A->dtype == KVB_F32 ? 1 : (A->out_f32 ? 1 : 0);
  a.scale = A->scale > 0.0f ? A->scale : 1.0f / sqrtf((float)A->d);
  a.Q = Q; a.O = O; a.segs = reinterpret_cast<const SegEntry*>(segs); a.nseg = nseg; a.seg_cap = A->seg_cap;
  if (ws) {
    const AttnPlan p = attention_plan(A->H, A->d, A->Lq, A->dtype);
    if (int rc = check_ws(ws, ws_bytes, (size_t)p.bytes)) return rc;
    a.ws = ws;
    a.ws_bytes = ws_bytes;
  }
  HIPCHK(launch_attention(a, (hipStream_t)stream));
  return ok();
}

int chunk_attention_noalloc(const kvb_attn_desc* A, const void* Q, const kvb_segment* segs, const int32_t* nseg,
                            void* O, kvb_stream_t stream) {
  if (!A) return fail(KVB_EINVAL, "attention descriptor is NULL");
  if (A->H < 1 || A->H > KVB_MAX_HEADS) return fail(KVB_ESHAPE, "H=%d", A->H);
  if (A->d != 64 && A->d != 128) return fail(KVB_ESHAPE, "d=%d (supported: 64, 128)", A->d);
  if (A->dtype != KVB_BF16 && A->dtype != KVB_F32) return fail(KVB_EDTYPE, "dtype=%d", A->dtype);
  if (A->Lq < 0) return fail(KVB_ESHAPE, "Lq=%d", A->Lq);
  if (A->seg_cap < 1 || A->seg_cap > KVB_MAX_SEGMENTS) return fail(KVB_ESHAPE, "seg_cap=%d", A->seg_cap);
  if (A->Lq == 0) return ok();
  REQ_PTR(Q, 16, "Q");
  REQ_PTR(O, 16, "O");
  REQ_PTR(segs, 8, "segs");
  REQ_PTR(nseg, 4, "nseg");
  AttnLaunch a{};
  a.H = A->H; a.d = A->d; a.Lq = A->Lq; a.et = A->dtype; a.out_f32 = A->dtype == KVB_F32 ? 1 : (A->out_f32 ? 1 : 0);
  a.scale = A->scale > 0.0f ? A->scale : 1.0f / sqrtf((float)A->d);
  a.Q = Q; a.O = O; a.segs = reinterpret_cast<const SegEntry*>(segs); a.nseg = nseg; a.seg_cap = A->seg_cap;
  const AttnPlan p = attention_plan(A->H, A->d, A->Lq, A->dtype);
  if (p.use) {
    if ((size_t)p.bytes > NOALLOC_SCRATCH_BYTES)
      return fail(KVB_EWORKSPACE, "the balanced grid needs %lld bytes of scratch, more than the %zu of "
                  "chunk_attention_noalloc's static array", (long long)p.bytes, NOALLOC_SCRATCH_BYTES);
    void* ptr = nullptr;
    if (int rc = scratch_on_current_device(&ptr)) return rc;
    a.ws = ptr;
    a.ws_bytes = NOALLOC_SCRATCH_BYTES;
  }
  HIPCHK(launch_attention(a, (hipStream_t)stream));
  return ok();
}

// workspace of forcing_head_profile: one-hot blocks, segment table, O, flags
struct ProfileLayout { int64_t ind, segs, O, bad, total; };
static ProfileLayout profile_layout(const kvb_attn_desc* A, int32_t max_len) {
  ProfileLayout p{};
  int64_t off = 0;
  const int esz = A->dtype == KVB_BF16 ? 2 : 4;
  auto bump = [&](int64_t bytes) { const int64_t o = off; off += (bytes + 255) / 256 * 256; return o; };
  p.ind = bump(4LL * max_len * A->d * esz);
  p.segs = bump((int64_t)A->H * A->seg_cap * (int64_t)sizeof(SegEntry));
  p.O = bump((int64_t)A->H * A->Lq * A->d * 4);
  p.bad = bump((int64_t)A->H * 4);
  p.total = off;
  return p;
}

static int check_profile_desc(const kvb_attn_desc* A, int32_t max_len) {
  if (!A) return fail(KVB_EINVAL, "attention descriptor is NULL");
  if (A->H < 1 || A->H > KVB_MAX_HEADS) return fail(KVB_ESHAPE, "H=%d", A->H);
  if (A->d != 64 && A->d != 128) return fail(KVB_ESHAPE, "d=%d (supported: 64, 128)", A->d);
  if (A->dtype != KVB_BF16 && A->dtype != KVB_F32) return fail(KVB_EDTYPE, "dtype=%d", A->dtype);
  if (A->Lq < 1) return fail(KVB_ESHAPE, "Lq=%d", A->Lq);
  if (A->seg_cap < 1 || A->seg_cap > KVB_MAX_SEGMENTS) return fail(KVB_ESHAPE, "seg_cap=%d", A->seg_cap);
  if (max_len < 0) return fail(KVB_ESHAPE, "max_len=%d", max_len);
  return KVB_OK;
}

int forcing_head_profile_workspace_size(const kvb_attn_desc* A, int32_t max_len, size_t* bytes) {
  if (int rc = check_profile_desc(A, max_len)) return rc;
  if (!bytes) return fail(KVB_EINVAL, "bytes is NULL");
  *bytes = (size_t)profile_layout(A, max_len).total;
  return ok();
}

int forcing_head_profile(const kvb_attn_desc* A, const void* Q, const kvb_segment* segs, const int32_t* nseg,
                         const int32_t* region, int32_t max_len, float alpha, float* out_mass, float* out_score,
                         uint8_t* out_label, void* ws, size_t ws_bytes, kvb_stream_t stream) {
  if (int rc = check_profile_desc(A, max_len)) return rc;
  if (!(alpha >= 0.0f && alpha <= 1.0f)) return fail(KVB_EPARAM, "alpha=%g not in [0,1]", (double)alpha);
  const ProfileLayout lo = profile_layout(A, max_len);
  if (int rc = check_ws(ws, ws_bytes, (size_t)lo.total)) return rc;
  REQ_PTR(Q, 16, "Q");
  REQ_PTR(segs, 8, "segs");
  REQ_PTR(nseg, 4, "nseg");
  REQ_PTR(region, 4, "region");
  REQ_PTR(out_score, 4, "out_score");
  REQ_PTR(out_label, 1, "out_label");
  if (out_mass && !aligned(out_mass, 4)) return fail(KVB_EINVAL, "out_mass is not 4-byte aligned");
  ProfileLaunch p{};
  p.a.H = A->H; p.a.d = A->d; p.a.Lq = A->Lq; p.a.et = A->dtype; p.a.out_f32 = 1;
  p.a.scale = A->scale > 0.0f ? A->scale : 1.0f / sqrtf((float)A->d);
  p.a.Q = Q; p.a.segs = reinterpret_cast<const SegEntry*>(segs); p.a.nseg = nseg; p.a.seg_cap = A->seg_cap;
  p.region = region; p.max_len = max_len; p.alpha = alpha;
  p.ind = at<void>(ws, lo.ind); p.segs_out = at<SegEntry>(ws, lo.segs); p.O = at<float>(ws, lo.O);
  p.bad = at<int32_t>(ws, lo.bad); p.mass = out_mass; p.score = out_score; p.label = out_label;
  HIPCHK(launch_head_profile(p, (hipStream_t)stream));
  return ok();
}

int kvbank_window_advance(const kvb_layer_desc* L, void* ring_k, void* ring_v, int32_t ring_cap, int32_t start,
                          int32_t n_rows, int32_t t_first, float rope_base, const void* new_k, const void* new_v,
                          void* cand_k, void* cand_v, kvb_stream_t stream) {
  if (!L) return fail(KVB_EINVAL, "layer descriptor is NULL");
  if (L->H < 1 || L->H > KVB_MAX_HEADS) return fail(KVB_ESHAPE, "H=%d", L->H);
  if (L->d != 64 && L->d != 128) return fail(KVB_ESHAPE, "d=%d (supported: 64, 128)", L->d);
  if (L->dtype != KVB_BF16 && L->dtype != KVB_F32) return fail(KVB_EDTYPE, "dtype=%d", L->dtype);
  if (L->frame_tokens <= 0) return fail(KVB_ESHAPE, "frame_tokens=%d", L->frame_tokens);
  if (!(rope_base > 1.0f) || !isfinite(rope_base)) return fail(KVB_EPARAM, "rope_base=%g", (double)rope_base);
  if (n_rows < 0 || ring_cap < 0 || n_rows > ring_cap || n_rows % L->frame_tokens != 0)
    return fail(KVB_ESHAPE, "n_rows=%d ring_cap=%d frame_tokens=%d", n_rows, ring_cap, L->frame_tokens);
  if (n_rows == 0) return ok();
  if (start < 0 || start >= ring_cap) return fail(KVB_ESHAPE, "start=%d ring_cap=%d", start, ring_cap);
  if ((new_k == nullptr) != (new_v == nullptr)) return fail(KVB_EINVAL, "new_k and new_v: both or neither");
  REQ_PTR(ring_k, 16, "ring_k");
  REQ_PTR(ring_v, 16, "ring_v");
  REQ_PTR(cand_k, 16, "cand_k");
  REQ_PTR(cand_v, 16, "cand_v");
  if (new_k) { REQ_PTR(new_k, 16, "new_k"); REQ_PTR(new_v, 16, "new_v"); }
  WindowLaunch w{};
  w.ring_k = ring_k; w.ring_v = ring_v; w.cap = ring_cap; w.start = start; w.n_rows = n_rows;
  w.F = L->frame_tokens; w.t_first = t_first; w.H = L->H; w.d = L->d; w.et = L->dtype;
  w.log2_base = log2((double)rope_base);
  w.new_k = new_k; w.new_v = new_v; w.cand_k = cand_k; w.cand_v = cand_v;
  HIPCHK(launch_window_advance(w, (hipStream_t)stream));
  return ok();
}

static_assert(KVB_MAX_HEADS <= ATT_MAX_HEADS, "attention plan holds every head");

int chunk_attention_workspace_size(const kvb_attn_desc* A, size_t* bytes) {
  if (!A || !bytes) return fail(KVB_EINVAL, "NULL argument");
  if (A->H < 1 || A->H > KVB_MAX_HEADS) return fail(KVB_ESHAPE, "H=%d", A->H);
  if (A->d != 64 && A->d != 128) return fail(KVB_ESHAPE, "d=%d (supported: 64, 128)", A->d);
  if (A->Lq < 0) return fail(KVB_ESHAPE, "Lq=%d", A->Lq);
  *bytes = (size_t)attention_plan(A->H, A->d, A->Lq, A->dtype).bytes;
  return ok();
}

}  // extern "C"
