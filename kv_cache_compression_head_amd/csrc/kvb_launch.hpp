// Internal launch interface between the C-ABI layer and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "kvb_common.hpp"

namespace kvb {

enum ElemType { ET_BF16 = 0, ET_F32 = 1 };

// device status bits (the C ABI's KVB_DEV_* values)
enum : uint32_t { DEV_NONFINITE = 1u, DEV_COUNT = 2u, DEV_SEGOVF = 4u, DEV_EVICT = 8u };

struct KeysDesc {            // one layer's keys in two buffers (see KeySpace)
  const void* bankK;
  const void* candK;
  const float* bankN;
  const float* candN;
  const void* bankA;         // 16 bytes per row
  const void* candA;
  int32_t M, N, d, H;
  int32_t et;
};

// out[r] = |k_r|^2 * scale and aug[r] = the augmentation row of key r (exact
// split of |k_r|^2, or of |k_r|^2 * scale in the direct form), for two key
// sets [H][rowsA][d] and [H][rowsB][d] in one launch (a null set is skipped)
// Optional check of the keys: with status set, a live row of a head in
// active whose squared norm is not finite ORs DEV_NONFINITE into *status
// (rows of the first set are live below the clamped count cntA[h]; every row
// of the second set is live)
struct NormCheck {
  uint32_t* status;
  const int32_t* cntA;
  uint64_t active;
  int32_t rowsA, rowsB;   // filled in by launch_norms
};
hipError_t launch_norms(const void* keysA, int rowsA, float* outA, void* augA, const void* keysB, int rowsB,
                        float* outB, void* augB, int et, int H, int d, float scale, bool direct, hipStream_t s,
                        NormCheck chk = NormCheck{nullptr, nullptr, 0, 0, 0});

// out[h*out_hstride + split*split_stride + i] = sum_{j in cols} phi(row_i, col_j)
struct GramLaunch {
  KeysDesc k;
  VList rows, cols;
  float* out;
  int64_t out_hstride;
  int64_t split_stride;
  int32_t splits;
  int32_t self_excl;
  PhiConst pc;
  int32_t phi_mode;
  uint64_t active;        // bit h: head computed
  // symmetric self-Gram (self_excl, rows == cols): column-sum slices in the
  // triangular layout below, for a list bounded by col_ld entries; null
  // computes every ordered pair
  float* colsum;
  int64_t col_ld;
};
hipError_t launch_gram(const GramLaunch& g, hipStream_t s);
// dst[h][j] += sum over row blocks b < j / 128 of the column sum of block b at
// column j, in a fixed order, for j below the row list's count (the symmetric
// self-Gram's mirrored pairs)
hipError_t launch_sym_combine(float* dst, int64_t dst_hstride, const float* colsum, int64_t col_ld, int nblocks,
                              VList rows, uint64_t active, int H, int n, hipStream_t s);
constexpr int GRAM_ROW_BLOCK = 128;   // rows per work-group of the symmetric self-Gram
// Triangular column-sum layout for a list bounded by n: row block b keeps only
// the columns right of its diagonal block, [(b+1) 128, n), and the blocks are
// packed one after another, so block b starts at sum_{b'<b} (n - (b'+1) 128).
// Column c of block b is at sym_col_off(n, b) + c - (b+1) 128; one head holds
// sym_head_floats(n) floats.
__host__ __device__ inline int64_t sym_col_off(int64_t n, int b) {
  return (int64_t)b * n - (int64_t)(GRAM_ROW_BLOCK / 2) * b * (b + 1);
}
__host__ __device__ inline int64_t sym_head_floats(int64_t n) {
  const int nb = (int)((n + GRAM_ROW_BLOCK - 1) / GRAM_ROW_BLOCK);
  return nb > 1 ? sym_col_off(n, nb - 1) : 0;
}

// sum split partials in order: dst[h*dst_hstride+i] = sum_s src[h*src_hstride + s*split_stride + i]
hipError_t launch_sum_splits(const float* src, int64_t src_hstride, int64_t split_stride, int splits,
                             float* dst, int64_t dst_hstride, int H, int n, hipStream_t s);

struct ScanLaunch {
  KeysDesc k;
  const float* rho;       // [H][M] current density
  const float* rho0;      // [H][M]
  const int32_t* count;   // [H]
  const int32_t* order;   // [H][N] candidate permutation
  uint64_t active;        // bit h: density head
  int32_t kmax;
  float tau;              // may be +inf
  int32_t cps;            // subtiles per checkpoint
  int32_t ncp;            // checkpoints per row
  float* cp;              // [H][ncp][M]
  int32_t* t_out;         // [H][M] (scan)
  const int32_t* kstar;   // device: [1] shared prefix, or [H] per head (sum)
  int32_t kstar_hs;       // head stride of kstar: 0 shared, 1 per head
  int32_t keep_crossed;   // 1: crossed rows may survive (their running sums and rho' are needed)
  float* rhoP;            // [H][M] (sum)
  PhiConst pc;
  int32_t phi_mode;
};
hipError_t launch_scan(const ScanLaunch& a, bool sum_mode, hipStream_t s);

// ---- selection / bookkeeping ----------------------------------------------
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);
// zero count (<= 4) int32 arrays of the given lengths in one launch (null entries skipped)
hipError_t launch_zero_i32(int32_t* const* ptrs, const int64_t* lens, int count, hipStream_t s);
// the same clears, and besides cnt[h] = min(max(count[h], 0), M) for the
// heads in active, with DEV_COUNT ORed into *status when a count was clamped
struct CountClamp {
  const int32_t* count;
  int32_t* cnt;
  uint32_t* status;
  uint64_t active;
  int32_t H, M;
};
hipError_t launch_zero_i32_clamp(int32_t* const* ptrs, const int64_t* lens, int count, const CountClamp& cc,
                                 hipStream_t s);

// keys for sorting: key = float_key(score[h][i]) << 32 | tie[i]; value = i
hipError_t launch_rank_sort_layers(const float* score, int64_t score_hstride, int64_t score_ls, uint64_t on, int H,
                                   int n, int nlayers, int32_t* out, int64_t out_hstride, int64_t out_ls,
                                   hipStream_t st);
hipError_t launch_sort(const float* score, int64_t score_hstride, const int32_t* tie, int64_t tie_hstride,
                       uint64_t head_on, int H, int n, uint64_t* kbuf0, uint64_t* kbuf1,
                       int32_t* vbuf0, int32_t* vbuf1, int32_t* out_order, int64_t out_hstride,
                       hipStream_t s);

// rank[i] = position of item i inside its frame of nseg items, ascending by
// (score, index), as a float sort key
hipError_t launch_frame_rank(const float* score, int items, int nseg, float* rank, hipStream_t s);

// per head: mean of D over n, delta = D / mean (0 if bank empty or mean 0)
hipError_t launch_delta(const float* D, const int32_t* count, uint64_t head_on, int H, int n,
                        float* delta, hipStream_t s);

struct SelectLaunch {
  int32_t H, M, kmax;
  uint64_t active;           // bit h: density head
  const int32_t* count;      // [H] bank occupancy
  const int32_t* t;          // [H][M] crossing times
  int32_t* hist;             // [H][kmax+2] scratch, becomes |V_h(k)|
  int32_t* kstar;            // device: [1] shared prefix, or [H] per head
  int32_t kstar_hs;          // 0 shared, 1 per head (each head its own largest feasible k)
  int32_t fill;              // 1: no density gating while n + k <= M
  int32_t evict_mode;        // 0 crossed then densest, 1 densest only, 2 crossed then oldest
  const float* rhoP;         // [H][M]
  const int32_t* bank_tok;   // [H][M]
  uint8_t* evict;            // [H][M]
  int32_t* surv;             // [H][M] survivor slots (ascending)
  int32_t* evl;              // [H][M] evicted slots (ascending)
  int32_t* n_surv;           // [H]
  int32_t* n_ev;             // [H]
  int32_t* n_mand;           // [H]
  uint32_t* status;          // device status word
  int32_t* fixl;             // [H][M] column list of the admitted-state fix-up
  int32_t* n_fix;            // [H]
  int32_t* fmode;            // [H] 1: fixl = survivors (direct sum), 0: fixl = evicted (subtract)
  int32_t skip_cross;        // 1: no crossing scan ran (k* = M replaces the whole bank); n_mand = -1
  void* evsel;               // [H] per-head eviction plan (32 bytes each), scratch
  int32_t* evblk;            // [H][ceil(M / 256)] per-block evicted / surviving counts, scratch
};
hipError_t launch_kstar(const SelectLaunch& a, hipStream_t s);
hipError_t launch_evict(const SelectLaunch& a, hipStream_t s);

struct ApplyLaunch {
  int32_t H, M, N, d, et, kmax;
  uint64_t active;
  void* bankK; void* bankV;
  int32_t* bank_tok; float* rho0; float* rho; int32_t* count;
  const void* candK; const void* candV; const int32_t* cand_tok;
  const int32_t* order;       // [H][N]
  const float* D;             // [H][N]
  const int32_t* kstar; int32_t kstar_hs;
  int32_t refresh;            // 1: every live state's baseline becomes its new density
  const int32_t* surv; const int32_t* n_surv;
  const int32_t* evl; const int32_t* n_ev;
  const float* rhoP;          // [H][M]
  const float* acc_surv;      // [H][M] sum over evicted for survivors (by survivor position)
  const float* acc_adm_ev;    // [H][kmax] sum over fixl for admitted
  const int32_t* fmode;       // [H]
  const float* acc_adm_adm;   // [H][kmax] sum over other admitted for admitted
  void* bankX; const void* candX; int32_t dx;   // density descriptors moved with K and V (null: none)
};
hipError_t launch_apply(const ApplyLaunch& a, hipStream_t s);

// ---- sequential within-block admission --------------------------------------
constexpr int KVB_SEQ_MAX_HEADS = 64;
struct SeqLaunch {
  int32_t H, M, N;
  uint64_t active;            // bit h: density head
  float* P;                   // [H][M+N][M+N] pair interactions (bank slots, then candidates)
  const int32_t* cnt;         // [H] clamped occupancy before the block
  const float* rho; const float* rho0; const int32_t* bank_tok;   // bank [H][M]
  const int32_t* cand_tok;    // [N]
  const int32_t* order;       // [H][N]
  float tau;
  int32_t fill, evict_mode, per_head;
  uint64_t* st_rr;            // [H][M+N] (rho, rho0) of each state
  int32_t* st_tok;            // [H][M+N] token id of live states, -1 otherwise
  int32_t* log;               // [H][N] admitted candidates in admission order
  int32_t* n_adm;             // [H]
  int32_t* kstar;             // out: admissions ([1] shared, [H] per head)
  int32_t kstar_hs;
  int32_t* n_ev;              // out [H]: evictions during the walk
  int32_t* n_mand;            // out [H]: of them, crossed states
  uint32_t* status;
};
struct SeqGather {
  int32_t H, M, N, d, dx, et;
  uint64_t active;
  const int32_t* cnt;
  const uint64_t* st_rr; const int32_t* st_tok;
  const int32_t* log; const int32_t* n_adm;
  int32_t* freel;             // [H][M] scratch
  int32_t* alive;             // [H][N] scratch
  int32_t refresh;
  float* rho; float* rho0; int32_t* bank_tok; int32_t* count;
  void* bankK; void* bankV; void* bankX;          // bankX may be null (descriptors are the keys)
  const void* candK; const void* candV; const void* candX;
  const int32_t* cand_tok;
  uint32_t* status;
};
hipError_t launch_sequential(const SeqLaunch& a, const SeqGather& g, const void* bankX, const void* candX, int dx,
                             const PhiConst& pc, int phi_mode, hipStream_t s);

// ---- segment tables ---------------------------------------------------------
struct SegEntry { const void* k; const void* v; int32_t len; int32_t pad; };

struct SegLaunch {
  int32_t H, d, et, M, N, F;
  uint8_t label[64];
  const void* sink_k; const void* sink_v; int32_t sink_len;
  const void* win_k; const void* win_v; int32_t win_cap, win_start, win_len;
  const void* chunk_k; const void* chunk_v; int32_t chunk_len;
  const void* bankK; const void* bankV; const int32_t* count;
  const void* candK; const void* candV;
  const int32_t* dyn_order; int64_t dyn_order_hstride;  // item order (dynamic heads)
  int32_t seg_len, items, keep;
  SegEntry* segs; int32_t* nseg; int32_t seg_cap;
  uint32_t* status;
};
hipError_t launch_segments(const SegLaunch& a, hipStream_t s);

// ---- Forcing-KV segment similarity ------------------------------------------
struct CosLaunch {
  const void* hist;    // [H][T*F][d]
  const void* nxt;     // [H][>=F][d] (first F rows used)
  int32_t et, H, d, F, T, seg_len;
  int32_t nxt_rows;    // rows per head in nxt
  int32_t ndyn; int32_t dyn_heads[64];
  float* cosbuf;       // [T][F]
  float* scores;       // [H][N] (written for dynamic heads)
  int64_t score_hstride;
  // several layers in one launch (kvbank_score_layers): layer l reads
  // hist + l hist_ls, nxt + l nxt_ls (elements) and writes cosbuf + l T F,
  // scores + l score_ls; nlayers = 1 for one layer
  int32_t nlayers;
  int64_t hist_ls, nxt_ls, score_ls;
};
hipError_t launch_segment_cosine(const CosLaunch& a, hipStream_t s);

// ---- attention ----------------------------------------------------------------
struct AttnLaunch {
  int32_t H, d, Lq, et, out_f32;
  float scale;
  const void* Q; void* O;
  const SegEntry* segs; const int32_t* nseg; int32_t seg_cap;
  void* ws; size_t ws_bytes;   // optional: enables the balanced grid (partials of split items)
};
// ---- offline head profiling (Forcing-KV) ------------------------------------
struct ProfileLaunch {
  AttnLaunch a;             // queries, segment table (keys), shapes
  const int32_t* region;    // [H][seg_cap]: 0 other, 1 sink, 2 transition, 3 generate
  int32_t max_len;          // rows of each one-hot block (>= every segment length)
  float alpha;
  void* ind;                // workspace: [4][max_len][d] one-hot rows
  SegEntry* segs_out;       // workspace: [H][seg_cap]
  float* O;                 // workspace: [H][Lq][d] fp32
  int32_t* bad;             // workspace: [H]
  float* mass;              // optional [H][4]
  float* score;             // [H]
  uint8_t* label;           // [H]
};
hipError_t launch_head_profile(const ProfileLaunch& p, hipStream_t s);

// ---- memory-key write path (window ring advance) ---------------------------
struct WindowLaunch {
  void* ring_k; void* ring_v;       // [H][cap][d]
  int32_t cap, start, n_rows, F, t_first, H, d, et;
  double log2_base;                 // log2 of the rotary base
  const void* new_k; const void* new_v;   // [H][n_rows][d] or null
  void* cand_k; void* cand_v;             // [H][n_rows][d]
};
hipError_t launch_window_advance(const WindowLaunch& a, hipStream_t s);

struct AttnPlan { int G, rounds, Ir; bool use; int64_t flag_bytes, bytes; };
constexpr int ATT_MAX_HEADS = 64;   // per-head tile counts of the balanced grid's plan live in LDS
AttnPlan attention_plan(int H, int d, int Lq, int et);
hipError_t launch_attention(const AttnLaunch& a, hipStream_t s);

}  // namespace kvb
