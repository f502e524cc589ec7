/*
 * kvbank -- head-wise compressed KV cache for chunk-by-chunk autoregressive
 * video diffusion, one attention layer at a time, on AMD Instinct MI355X
 * (gfx950).  Plain C ABI: device pointers, sizes and a HIP stream; no
 * framework types.
 *
 * The operations follow two methods described on public pages:
 *
 *  - "DensityKV: Density-Guided KV Cache Compression for Long Video
 *    Generation" (paper summary): per-(layer, head) banks of exact K/V pairs,
 *    Soft-Riesz density of post-RoPE keys, candidates ordered by
 *    mean-normalised insertion disturbance, the largest prefix length that
 *    every head of the layer can admit under an insertion-relative density
 *    growth bound tau, eviction of crossed states then the densest
 *    (Method; appendix B.1; defaults in appendices D-E).
 *  - "Forcing-KV: Hybrid KV Cache Compression for Efficient Autoregressive
 *    Video Diffusion Models" (paper notes): static heads keep the sink frame,
 *    the transition frame and the current chunk (section 3.3); dynamic heads
 *    keep the least similar frame segments (section 3.4).
 *
 * Readings fixed where the pages are silent:
 *   phi(d2) = (eps + d2 / sigma^2)^(-p/2) with d2 the squared distance of
 *   post-RoPE keys; a state's density excludes itself and counts bank states
 *   only; delta(c) = D(c) / mean D with D(c) = sum over the bank of phi(c, b);
 *   candidates ordered by ascending (delta, token id) per head; a state
 *   crosses at prefix length k when rho_b + sum_{j<k} phi(b, c_j) > tau *
 *   rho0_b (strict); e(k) = max(0, n + k - M); k is feasible when every
 *   density head has |crossed| <= e(k), k <= min(N, M); k = 0 always
 *   feasible; eviction = crossed states, then the largest projected
 *   densities (ties: lower token id first); admitted states get rho0 = rho =
 *   their density in the new bank.  Forcing-KV: cos(a, b) = a.b /
 *   max(|a||b|, 1e-8) on keys concatenated over the dynamic heads; kept count
 *   floor(r * items) in double precision; ties to the lower item index.
 *
 * Ownership and execution: the caller allocates every buffer (bank,
 * candidates, outputs, workspace); the library never allocates or frees
 * device memory and keeps no state besides a thread-local error string.
 * Every call is asynchronous on the given stream and never synchronises;
 * buffers must stay alive until the stream has executed the work.  Host-side
 * checks run before any launch; a negative status means nothing was queued.
 * Device-side conditions never trap: they set bits in kvb_update_out.status.
 *
 * Layouts: all K/V/Q buffers are head-major [H][rows][d], contiguous, dtype
 * KVB_BF16 (uint16 bit patterns) or KVB_F32, 16-byte aligned.
 */
#ifndef KVBANK_H
#define KVBANK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t* kvb_stream_t;   /* same type as hipStream_t */

/* status codes (return values) */
#define KVB_OK          0
#define KVB_EINVAL     (-1)   /* null or misaligned (16 B) pointer */
#define KVB_ESHAPE     (-2)   /* bad H, d, M, N, F, segment capacity ... */
#define KVB_EDTYPE     (-3)   /* unsupported dtype */
#define KVB_EPARAM     (-4)   /* tau < 1 or NaN, sigma <= 0, eps <= 0 with p > 0, p < 0 or NaN, r not in [0,1],
                                 seg_len not dividing F, bad head label */
#define KVB_EWORKSPACE (-5)   /* workspace too small */
#define KVB_EHIP       (-6)   /* HIP runtime error at launch (message in kvb_last_error) */

/* device status bits (kvb_update_out.status).  None of these conditions
 * traps: the kernels read and write only inside each head's slices and go on.
 * A head's bank never holds more than M pairs (DensityKV paper summary,
 * appendix B.1, online bank update); a non-finite key has no Soft-Riesz
 * density (Method, Soft-Riesz density). */
#define KVB_DEV_NONFINITE 1u  /* a density head's live bank key or candidate key has a non-finite squared
                                 norm (NaN or Inf element, or overflow); its densities and decisions are
                                 then meaningless, but every access stays in bounds */
#define KVB_DEV_COUNT   2u    /* bank count[h] outside [0, M]: the update used min(max(count, 0), M) for
                                 every read, and the committed count is that clamped value plus k* minus
                                 the evictions */
#define KVB_DEV_SEGOVF  4u    /* segment table capacity exceeded (truncated) */
#define KVB_DEV_EVICT   8u    /* eviction count inconsistent with the crossed set */

/* element types */
#define KVB_BF16 0
#define KVB_F32  1

/* head labels */
#define KVB_HEAD_DENSITY 0    /* DensityKV bank */
#define KVB_HEAD_STATIC  1    /* Forcing-KV static head */
#define KVB_HEAD_DYNAMIC 2    /* Forcing-KV dynamic head */

#define KVB_MAX_HEADS 64
#define KVB_MAX_SEGMENTS 256  /* per head, attention side */

/* DensityKV policy variants (DensityKV paper summary, appendix E
 * ablations); 0 is the method: candidates by ascending (delta, token id),
 * frozen insertion baselines, crossed states evicted first then the densest,
 * one prefix length shared by the layer's density heads, density gating at
 * every occupancy. */
#define KVB_POL_SOURCE_ORDER     1u   /* candidates in source order: ascending token id */
#define KVB_POL_REFRESH_BASELINE 2u   /* after each update every state's baseline = its new density */
#define KVB_POL_EVICT_DENSEST    4u   /* evict the e highest projected densities, crossed or not */
#define KVB_POL_EVICT_OLDEST     8u   /* crossed states, then ascending token id (source-order completion) */
#define KVB_POL_HEAD_PREFIX     16u   /* each density head its own largest feasible prefix (k_star is [H]) */
#define KVB_POL_FILL_BELOW_CAP  32u   /* no density check, no eviction, for prefixes with n + k <= M */
/* Forcing-KV dynamic heads (notes page, section 3.4 as printed): BottomK
 * within each frame, floor(r * n) of its n = F / seg_len segments, instead of
 * one BottomK over all (frame, segment) items */
#define KVB_POL_FRAME_BOTTOMK   64u
/* DensityKV sequential within-block admission (paper summary, appendix E,
 * within-block competition): instead of the largest shared prefix, kvbank_update
 * walks the candidates in order and gates each one against the bank as it
 * stands, earlier admissions included.  Step j offers every density head its
 * j-th candidate c; with e = max(0, n + 1 - M) the step is feasible when each
 * head has at most e states x with rho_x + phi(x, c) > tau * rho0_x (decided
 * by the whole layer; per head with KVB_POL_HEAD_PREFIX; unchecked below
 * capacity with KVB_POL_FILL_BELOW_CAP).  A feasible step admits c, evicting
 * the crossed state, else the densest (ties: lower token) or, with
 * KVB_POL_EVICT_OLDEST, the oldest (KVB_POL_EVICT_DENSEST: the densest).
 * Only growth from later blocks counts against a baseline: the block's
 * admitted candidates cannot cross during the walk and take their density in
 * the bank as baseline when it ends.  Outputs: k_star = admitted
 * candidates, n_evicted = evictions during the walk (admitted candidates
 * included), n_mandatory = of them, crossed states; t_cross and rho_proj are
 * not written.  The workspace holds every head's (M + N)^2 pair interactions
 * in fp32. */
#define KVB_POL_SEQUENTIAL     128u
#define KVB_POL_ALL            255u

typedef struct kvb_params {
  float tau;          /* density growth bound, >= 1 (may be +inf) */
  float sigma;        /* Soft-Riesz bandwidth, > 0 */
  float eps;          /* softening, > 0 unless p == 0 */
  float p;            /* decay exponent, >= 0 */
  int32_t seg_len;    /* Forcing-KV segment length in tokens (divides F); used by dynamic heads */
  uint32_t policy;    /* OR of KVB_POL_*; EVICT_DENSEST and EVICT_OLDEST exclude each other */
  double retention;   /* Forcing-KV kept fraction r in [0, 1] */
} kvb_params;

typedef struct kvb_layer_desc {
  int32_t H;             /* heads, 1 .. KVB_MAX_HEADS */
  int32_t d;             /* head dim: 64 or 128 */
  int32_t M;             /* bank capacity per head (>= 0; > 0 when a density head exists) */
  int32_t dtype;         /* KVB_BF16 or KVB_F32 */
  int32_t frame_tokens;  /* F: tokens per latent frame */
  int32_t desc_dim;      /* density descriptor (DensityKV paper summary, appendix E, descriptor ablation):
                            0 = the post-RoPE keys themselves (the method); 64, 128 or (bf16 only) 256 =
                            separate rows of that dimension in bank->X and layout->cand_x (pre-RoPE keys,
                            or [K; V]: 128 wide when d = 64, 256 wide when d = 128).  Other widths are
                            KVB_ESHAPE.  Density-only layers (no Forcing-KV heads) */
  const uint8_t* label;  /* HOST pointer, H head labels */
  kvb_params params;
} kvb_layer_desc;

typedef struct kvb_bank {   /* device pointers, updated in place */
  void* K;          /* [H][M][d] */
  void* V;          /* [H][M][d] */
  int32_t* tok;     /* [H][M] token ids */
  float* rho0;      /* [H][M] frozen insertion baselines */
  float* rho;       /* [H][M] current densities (maintained incrementally) */
  int32_t* count;   /* [H] occupancy n_h; slots [0, n_h) are live */
  void* X;          /* [H][M][desc_dim] density descriptors, moved with K and V (desc_dim > 0; else unused) */
} kvb_bank;

typedef struct kvb_kv_layout {   /* device pointers of the non-bank KV of the layer */
  const void* sink_k; const void* sink_v; int32_t sink_len;    /* [H][sink_len][d] sink frame(s) */
  int32_t win_cap;                                            /* rows per head of the window ring */
  const void* win_k; const void* win_v;                       /* [H][win_cap][d] local window ring */
  int32_t win_start; int32_t win_len;                         /* live rows: win_len rows from win_start (mod cap) */
  const void* chunk_k; const void* chunk_v; int32_t chunk_len; /* [H][chunk_len][d] current chunk */
  int32_t reserved;
  const void* cand_x;   /* [H][N][desc_dim] the candidates' density descriptors (desc_dim > 0; else unused) */
} kvb_kv_layout;

typedef struct kvb_segment {   /* one contiguous run of retained rows of one head */
  const void* k;   /* device pointer to the first K row */
  const void* v;   /* device pointer to the first V row */
  int32_t len;     /* rows */
  int32_t reserved;
} kvb_segment;

typedef struct kvb_update_out {   /* device pointers written by kvbank_update */
  int32_t* k_star;        /* [1] shared admitted prefix length; [H] per head with KVB_POL_HEAD_PREFIX */
  int32_t* n_mandatory;   /* [H] states that crossed tau * rho0 at k*; -1 when min(N, M) = M and neither
                             t_cross nor rho_proj is given: every head can then admit k = M (the e(M) = n
                             evictions cover any crossed set), the whole bank is replaced whatever crossed,
                             and the crossing scan is skipped */
  int32_t* n_evicted;     /* [H] */
  uint32_t* status;       /* [1] OR of KVB_DEV_* bits (caller zeroes it) */
  kvb_segment* segs;      /* [H][seg_cap] segment table read by chunk_attention */
  int32_t* nseg;          /* [H] */
  int32_t seg_cap;        /* >= 5 for density heads, 3 for static, 2 + kept items for dynamic; <= 256 */
  int32_t reserved;
  int32_t* t_cross;       /* optional [H][M]: per bank slot, the smallest prefix length at which the
                             state crosses tau * rho0 (min(N, M) + 1 if never), for density heads */
  float* rho_proj;        /* optional [H][M]: projected density rho'(k*) per bank slot (rows that
                             crossed at k* keep their current density) */
} kvb_update_out;

typedef struct kvb_attn_desc {
  int32_t H, d, Lq, dtype;
  float scale;            /* softmax scale; <= 0 selects 1/sqrt(d) */
  int32_t seg_cap;        /* row stride (entries) of the segment table, <= KVB_MAX_SEGMENTS */
  int32_t out_f32;        /* 1: O is fp32; 0: O has the input dtype */
  int32_t reserved;
} kvb_attn_desc;

/* Workspace bytes needed by kvbank_score and kvbank_update for N
 * candidates per head.  Host only; no device work.  With kmax = min(N, M)
 * admissible candidates, the size grows as H * kmax^2 / 64 bytes (the column
 * sums of the symmetric admitted x admitted Gram) plus terms linear in N and
 * M: for example 61 MB at H = 12, M = 9,360, N = 23,400. */
int kvbank_workspace_size(const kvb_layer_desc* L, int32_t N, size_t* bytes);

/* Scoring (DensityKV Method, "Online Density-Constrained Bank Update";
 * Forcing-KV section 3.4).
 *   cand_k   [H][N][d]  post-RoPE candidate keys (density heads: the frames that
 *                        just left the local window; Forcing-KV heads: the history
 *                        frames in time order, N a multiple of F)
 *   cand_tok [N]         token ids, shared by the heads, unique
 *   lay                  needed by dynamic heads (the chunk's first frame pairs with
 *                        the last history frame); may be NULL without dynamic heads
 * Outputs (device, [H][N], row stride N):
 *   density heads: out_D = D(c), out_score = delta(c), out_order = candidate
 *                  indices sorted by ascending (delta, token id)
 *   dynamic heads: out_score[0:items] = segment scores (items = N / seg_len, item
 *                  i covers history rows [i*seg_len, (i+1)*seg_len)), out_order
 *                  = item indices sorted ascending by (score, index)
 *   static heads:  untouched
 * KVB_ESHAPE when one token's features over the dynamic heads exceed 16 KB
 * (more than 32 dynamic fp32 heads at d = 128).  The bank's count is read
 * clamped to [0, M]; kvbank_update reports an out-of-range count.
 * N = 0 is a no-op. */
int kvbank_score(const kvb_layer_desc* L, const kvb_bank* bank, const void* cand_k, const int32_t* cand_tok,
                 int32_t N, const kvb_kv_layout* lay, float* out_D, float* out_score, int32_t* out_order, void* ws,
                 size_t ws_bytes, kvb_stream_t stream);

/* Forcing-KV segment scoring of several layers in one call (Forcing-KV notes,
 * section 3.4 and the section 3.5 sketch: a layer's dynamic heads score each
 * history segment by the mean cosine between adjacent frames; the layers of
 * a model score independently).  For nlayers layers that share the
 * descriptor L and whose heads are all static or dynamic, this gives the
 * same outputs, bit for bit, as kvbank_score on each layer l with
 *   cand_k  + l * cand_layer_stride   [H][N][d] history keys of layer l
 *   chunk_k + l * chunk_layer_stride  [H][chunk_len][d] the chunk's keys
 *                                     (its first frame pairs with the last
 *                                     history frame)
 *   out_score + l * H * N, out_order + l * H * N   (as kvbank_score's)
 * (strides in elements, multiples of 16 bytes), with the cosines, the
 * segment means and the BottomK orders of all layers in one launch each: at
 * one layer the segment cosine reads too few bytes to reach the memory
 * bandwidth past a launch.  Static heads' rows are untouched.  Workspace:
 * kvbank_score_layers_workspace_size bytes (the per-token cosines).
 * KVB_EPARAM with density heads, with KVB_POL_FRAME_BOTTOMK or with more
 * than 1,024 items (N / seg_len) per layer; KVB_ESHAPE for strides shorter
 * than one layer, chunk_len < frame_tokens, or as kvbank_score.  N = 0,
 * nlayers = 0 or no dynamic head is a no-op. */
int kvbank_score_layers_workspace_size(const kvb_layer_desc* L, int32_t nlayers, int32_t N, size_t* bytes);
int kvbank_score_layers(const kvb_layer_desc* L, int32_t nlayers, const void* cand_k, int64_t cand_layer_stride,
                        const void* chunk_k, int64_t chunk_layer_stride, int32_t chunk_len, int32_t N,
                        float* out_score, int32_t* out_order, void* ws, size_t ws_bytes, kvb_stream_t stream);

/* Admission / eviction and segment table (DensityKV appendix B.1 "Online
 * Bank Update"; Forcing-KV sections 3.3-3.4).
 *   density heads: shared prefix k*, eviction set, exact K/V/token moves into
 *     the bank (freed slots first, then appended; live slots stay dense),
 *     density fix-ups; D and order are kvbank_score's outputs.
 *   static heads:  segments [sink, last F candidate rows, chunk]
 *   dynamic heads: keep floor(r * items) lowest-scoring items; segments [sink,
 *     kept runs in token order, chunk]
 *   density heads' segments: [sink, bank[0:n_h], window (<= 2 ring runs), chunk]
 * Writes out->k_star, n_mandatory, n_evicted, segs, nseg; ORs out->status. */
int kvbank_update(const kvb_layer_desc* L, kvb_bank* bank, const void* cand_k, const void* cand_v,
                  const int32_t* cand_tok, int32_t N, const float* D, const int32_t* order,
                  const kvb_kv_layout* lay, kvb_update_out* out, void* ws, size_t ws_bytes, kvb_stream_t stream);

/* Native attention of the chunk's queries over each head's segment table
 * (DensityKV card page Figure 2; Forcing-KV section 3.3):
 *   O_h = softmax(Q_h K_h^T * scale) V_h,  Q, O [H][Lq][d].
 * ws (device, optional, caller-owned, 256-byte aligned): with ws_bytes >=
 * chunk_attention_workspace_size(A) > 0, the bf16 path balances its work
 * over every slot of the GPU: items (head, 128-query tile) left over after
 * whole rounds are cut along the keys into a main piece and a tail, whose
 * fp32 partials (o, reference, denominator) a second kernel merges.  This is
 * taken whenever the items do not fill whole rounds (the size is 0 when they
 * do); the cut is derived on the device from the segment lengths, so heads
 * of different lengths are balanced too.  ws = NULL runs one work-group per
 * item.  Both give the same result up to rounding.
 * A too-small non-NULL workspace is KVB_EWORKSPACE.  Calls that share one
 * workspace must not overlap. */
int chunk_attention(const kvb_attn_desc* A, const void* Q, const kvb_segment* segs, const int32_t* nseg, void* O,
                    void* ws, size_t ws_bytes, kvb_stream_t stream);

/* chunk_attention for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments and result as chunk_attention, without the workspace: when
 * the balanced grid is taken (chunk_attention_workspace_size > 0) its
 * partials and flags live in a static device array of the library, 72 MiB
 * per GPU (enough for every plan on a 256-compute-unit device), kept until
 * the process ends; its address is looked up once per device, on the first
 * call made with that device current.  Nothing is allocated or freed, by the
 * library or by any routine it calls.  Every flag and partial a call reads is
 * written earlier in the same call, so nothing needs clearing.  Calls on one
 * GPU share the array: calls that overlap in time on one GPU (two streams,
 * or two host threads) race and must be serialised by the caller.  A plan
 * needing more than 72 MiB is KVB_EWORKSPACE (nothing is queued). */
int chunk_attention_noalloc(const kvb_attn_desc* A, const void* Q, const kvb_segment* segs, const int32_t* nseg,
                            void* O, kvb_stream_t stream);

/* Workspace bytes for chunk_attention's balanced grid (0: nothing to
 * balance, or the fp32 path).  Depends on the current device's compute-unit
 * count.  Host only; no device work. */
int chunk_attention_workspace_size(const kvb_attn_desc* A, size_t* bytes);

/* Memory-key write path (DensityKV paper summary, supplementary "Post-RoPE
 * Attention Geometry": memory keys carry temporal rotary coordinate 0 and keep
 * their spatial coordinates; Method, "Online Density-Constrained Bank
 * Update": the candidates are the frames that leave the local window).
 * The n_rows ring rows from position start (mod ring_cap) leave the window;
 * row r belongs to departing frame r / F (F = L->frame_tokens), whose keys
 * carry temporal coordinate t_first + r / F.
 *   ring_k, ring_v [H][ring_cap][d] device, L->dtype; updated in place when
 *                   new_k/new_v are given
 *   cand_k [H][n_rows][d]: the row's key with each temporal rotary pair
 *                   (x_2i, x_2i+1), i < n_t = d/2 - 2 floor(d/6), turned by
 *                   -t * rope_base^(-i / n_t) (interleaved pairs, temporal
 *                   first); the other elements copied bit for bit
 *   cand_v [H][n_rows][d]: the row's value, bit for bit
 *   new_k, new_v [H][n_rows][d] (optional, both or neither): written into the
 *                   departed slots after they are read (the arriving frames)
 * Device buffers are caller-owned; cand_* must not overlap ring_* or new_*.
 * n_rows = 0 is a no-op.  Errors: KVB_EINVAL null or misaligned (16 B)
 * pointer; KVB_ESHAPE n_rows > ring_cap, start outside [0, ring_cap),
 * n_rows not a multiple of F; KVB_EPARAM rope_base <= 1 or not finite. */
int kvbank_window_advance(const kvb_layer_desc* L, void* ring_k, void* ring_v, int32_t ring_cap, int32_t start,
                          int32_t n_rows, int32_t t_first, float rope_base, const void* new_k, const void* new_v,
                          void* cand_k, void* cand_v, kvb_stream_t stream);

/* Offline head profiling (Forcing-KV notes page, section 3.2).  Per head,
 * the sums over the chunk's Lq queries of their softmax(Q K^T * scale)
 * weights on each region of the head's key set: A_other, A_sink,
 * A_transition, A_generate; score = (A_generate + A_transition) /
 * (A_total - A_sink); the head is static when score > alpha (0.8 on the
 * page), else dynamic.
 *   A: H, d, Lq, dtype, scale and seg_cap as for chunk_attention
 *   Q [H][Lq][d]; segs/nseg: the head's key segments (v pointers unused)
 *   region [H][seg_cap] int32 device: 0 other history, 1 sink, 2 transition,
 *          3 generate (the chunk itself)
 *   max_len: at least every segment's length (sizes the workspace)
 *   out_mass [H][4] float device, optional: A_other, A_sink, A_transition,
 *          A_generate; out_score [H] float; out_label [H] uint8:
 *          KVB_HEAD_STATIC or KVB_HEAD_DYNAMIC.  A head with a segment
 *          longer than max_len or a region outside 0..3 gets score NaN and
 *          label 0xFF (nothing is read past the workspace).
 *   ws: forcing_head_profile_workspace_size bytes, caller-owned.
 * Runs the attention kernels with one-hot values (the mass of region r is
 * column r of the output).  Errors: as for chunk_attention, plus EPARAM for
 * alpha outside [0, 1]. */
int forcing_head_profile_workspace_size(const kvb_attn_desc* A, int32_t max_len, size_t* bytes);
int forcing_head_profile(const kvb_attn_desc* A, const void* Q, const kvb_segment* segs, const int32_t* nseg,
                         const int32_t* region, int32_t max_len, float alpha, float* out_mass, float* out_score,
                         uint8_t* out_label, void* ws, size_t ws_bytes, kvb_stream_t stream);

/* Message of the last non-OK status on this thread ("" if none). */
const char* kvb_last_error(void);

/* SHA-256 (64 hex digits) of the sources this library was built from, set
 * by the package's build script ("unknown" for another build).  A loader can
 * compare it with the sources beside the library and refuse a stale build.
 * Static string; no device work. */
const char* kvb_source_hash(void);

#ifdef __cplusplus
}
#endif

#endif /* KVBANK_H */
