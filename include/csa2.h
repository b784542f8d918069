/*
 * csa2.h — C ABI of the CSA2 (Compressed Sparse Attention 2) hot path with an
 * FP4 main-KV cache, for AMD Instinct MI355X (gfx950).
 *
 * The method (DeepSeek-V4.1-Flash, as described on the public pages):
 *  - every attention layer is statically Full, Reindex or Reuse and shares the
 *    main KV, the indexer K and the Top-K indices across layers
 *    (gkm0120.cn survey, section 2.2.2 mode table; aprilzz.com article,
 *    section "CSA2：在层的维度上共享缓存");
 *  - a Full layer scores every visible entry with the indexer and selects a new
 *    Top-512; in the decoder it also builds a candidate pool of at most 2048
 *    blocks x 8 positions that later Reindex layers score inside
 *    (gkm0120.cn section 2.2.3 "Hierarchical Sparse Indexer"; aprilzz.com CSA2
 *    section);
 *  - the main KV is stored as FP4 E2M1 with one E4M3 scale per 16 channels and
 *    no global scale (aprilzz.com section "FP4 KV 与部署层的几个改动");
 *  - every layer also runs a 128-token sliding-window attention
 *    (aprilzz.com section "把 prefill 砍掉一半").
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers owned by the caller, unless noted.
 *    The library never allocates device memory; scratch comes from a
 *    caller-provided workspace sized by the matching *_workspace_size call.
 *  - Work is enqueued asynchronously on the given stream (NULL = the null
 *    stream).  Kernel faults surface at the caller's next synchronisation.
 *  - Every argument is validated on the host BEFORE any HIP call; on a
 *    non-OK status nothing has been enqueued and csa2_last_error() returns a
 *    message (thread-local).  A failed launch returns CSA2_EHIP.
 *  - bf16 data is passed as raw 16-bit patterns (uint16_t).
 *  - Floating-point inputs must be finite.
 *  - Indices are int32: entry counts per sequence must be < 2^31.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_ABI_VERSION 3

typedef enum {
    CSA2_OK = 0,
    CSA2_EINVAL = 1,        /* bad pointer / size / layout argument               */
    CSA2_EUNSUPPORTED = 2,  /* valid but not implemented (e.g. H not a multiple of 16) */
    CSA2_EWORKSPACE = 3,    /* workspace missing or smaller than required          */
    CSA2_EMODE = 4,         /* layer-mode sequence error (Reuse before a selection) */
    CSA2_EHIP = 5           /* a HIP runtime call or kernel launch failed          */
} csa2_status;

typedef enum { CSA2_F32 = 0, CSA2_BF16 = 1 } csa2_dtype;

typedef enum { CSA2_FULL = 0, CSA2_REINDEX = 1, CSA2_REUSE = 2 } csa2_mode;

/* FP4 main-KV cache view.  Two byte planes:
 *   codes : one row of D/2 bytes per entry; byte i holds channel 2i in its low
 *           nibble and channel 2i+1 in its high nibble; nibble = sign<<3 | E2M1.
 *   scales: one row of D/16 E4M3FN bytes per entry (channels 16g..16g+15).
 * Entry (b, j) lives in physical row
 *   page_table == NULL : b * seq_stride + j
 *   page_table != NULL : page_table[b * max_pages + j / page_size] * page_size + j % page_size
 * page_size must be a multiple of 8 (an 8-entry pool block never straddles a page). */
typedef struct csa2_fp4_kv {
    uint8_t* codes;
    uint8_t* scales;
    const int32_t* page_table;
    int32_t page_size;
    int32_t max_pages;
    int64_t seq_stride;
    int32_t D;
} csa2_fp4_kv;

/* Indexer-K view: k[row][D_i] bf16, rows addressed exactly as in csa2_fp4_kv. */
typedef struct csa2_idx_k {
    const uint16_t* k;
    const int32_t* page_table;
    int32_t page_size;
    int32_t max_pages;
    int64_t seq_stride;
    int32_t D_i;
} csa2_idx_k;

int32_t csa2_abi_version(void);
/* Message describing the last non-OK status returned on this thread ("" if none). */
const char* csa2_last_error(void);
const char* csa2_status_string(csa2_status st);

/* ---------------------------------------------------------------------------
 * FP4 pack: x[rows][D] (fp32 or bf16) -> codes[rows][D/2], scales[rows][D/16].
 * Per 16-channel group: scale = E4M3FN nearest to amax/6 (ties to even,
 * saturating at 448); element = E2M1 nearest to |x|/scale (ties to the even
 * code, saturating at 6), sign copied; scale 0 encodes all magnitudes as 0.
 * D % 16 == 0.  rows may be 0 (no-op).
 * (aprilzz.com, section "FP4 KV 与部署层的几个改动"; OCP MX v1.0 E2M1; OFP8 E4M3.)
 */
csa2_status csa2_fp4_quantize(const void* x, csa2_dtype xt, int64_t rows, int32_t D, uint8_t* codes,
                              uint8_t* scales, hipStream_t stream);

/* FP4 unpack: y[rows][D] fp32 = (-1)^s * E2M1 * E4M3 scale (exact). */
csa2_status csa2_fp4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t D, float* y,
                                hipStream_t stream);

/* Per-step KV append: quantize x[B][D] and write row b at logical entry pos[b]
 * of sequence b of the cache view (contiguous or paged).  pos is a device
 * array; every pos[b] must address an allocated row. */
csa2_status csa2_fp4_append(const void* x, csa2_dtype xt, int32_t B, const int32_t* pos, const csa2_fp4_kv* kv,
                            hipStream_t stream);

/* Per-step append of one decode token per sequence, in one launch: everything
 * the layer stack reads about the new token.
 *   x       [B][D] fp32/bf16: main-KV latent of the new entry, FP4-quantised
 *           into logical entry pos[b] of sequence b of kv (as csa2_fp4_append)
 *   k_new   [B][D_i] bf16 or NULL: indexer key of the new entry, copied to
 *           entry pos[b] of the indexer-K view k
 *   swa_new [n_layers] host array of device pointers to [B][D] bf16 rows: each
 *           layer's window row of the new token, copied into the layer's window
 *           ring swa_kv[l] ([B][T][D] bf16) at row tok[b] mod T
 * pos and tok are device [B] int32: pos[b] the new entry's index (it must
 * address an allocated row of both views), tok[b] >= 0 the new token's
 * absolute position in its sequence (the window ring's row rule; see
 * csa2_swa_attn).  0 <= n_layers <= 32.  Alignment: x, k_new, k and every
 * window pointer 16 bytes, codes 8.  Rows are written in place; the caller
 * orders this call before the layers that read them (aprilzz.com, sections
 * "FP4 KV 与部署层的几个改动" and "把 prefill 砍掉一半"). */
typedef struct csa2_append_args {
    int32_t B;
    const void* x;
    csa2_dtype xt;
    const int32_t* pos;
    const csa2_fp4_kv* kv;
    const uint16_t* k_new;
    const csa2_idx_k* k;
    int32_t n_layers;
    const uint16_t* const* swa_new;
    uint16_t* const* swa_kv;
    int32_t T;
    const int32_t* tok;
} csa2_append_args;
csa2_status csa2_append_token(const csa2_append_args* a, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * SWA Bounded Replay: rebuild window rows from the last n tokens instead of
 * keeping them (gkm0120.cn section 2.1; aprilzz.com sections "把 prefill 砍掉一半"
 * and "FP4 KV 与部署层的几个改动"; aimodeling.com "第三层").  For every layer l
 * and sequence b, token i (0 <= i < n) of the replay has position
 * p = t_end[b] - n + 1 + i and its window row is
 *   swa_kv[l][b][p mod T][d] = bf16( sum_c h[l][b][i][c] * W[l][d][c] )
 * accumulated in fp32 and rounded to nearest-even once.  Positions p < 0 are
 * skipped; other ring rows are left as they are.
 *   h      [n_layers] host array of device [B][n][d_model] bf16 (layer inputs)
 *   W      [n_layers] host array of device [D][d_model] bf16 (output-major)
 *   swa_kv [n_layers] host array of device [B][T][D] bf16 rings (written)
 *   t_end  [B] device int32
 * 0 <= n <= T; d_model % 64 == 0; D % 16 == 0; 0 <= n_layers <= 48; h and W
 * 16-byte aligned, swa_kv 8-byte aligned.  B*n == 0 or n_layers == 0: no-op. */
typedef struct csa2_replay_args {
    int32_t B;
    int32_t n;
    int32_t d_model;
    int32_t D;
    int32_t T;
    const int32_t* t_end;
    int32_t n_layers;
    const uint16_t* const* h;
    const uint16_t* const* W;
    uint16_t* const* swa_kv;
} csa2_replay_args;
csa2_status csa2_swa_replay(const csa2_replay_args* a, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Full-mode indexer scoring (gkm0120.cn section 2.2.2; aprilzz.com CSA2 section).
 *   q_idx  [B][Q][H_i][D_i] bf16 indexer queries (row r = b*Q + q)
 *   k      indexer-K view of B sequences, shared by all heads and layers
 *   n_vis  [B][Q] int32: entries 0..n_vis-1 of sequence b are visible to row r
 *   scores [B*Q][n_max] fp32 out, or NULL: s_j = sum_h dot(q_h, k_j) for
 *          j < n_vis, -inf for n_vis <= j < n_max.  fp32 evaluation: qbar_c =
 *          sum_h q_hc (h ascending), then an FMA chain over channels
 *          ascending, from +0.
 *   block_max [B*Q][ceil(n_max/8)] fp32 out or NULL: max score of each aligned
 *          8-entry block (-inf when no entry of the block is visible).
 *          At least one of scores / block_max is given; block maxima alone
 *          are what a pool needs (its Top-K follows from the rescored pool).
 * D_i in {64, 128}; 1 <= H_i <= 64; n_vis[r] <= n_max.
 */
csa2_status csa2_index_full(const uint16_t* q_idx, int32_t B, int32_t Q, int32_t H_i, const csa2_idx_k* k,
                            const int32_t* n_vis, int32_t n_max, float* scores, float* block_max,
                            hipStream_t stream);

/* Reindex-mode scoring inside the pool (gkm0120.cn section 2.2.3).
 *   pool_blocks [B*Q][P] int32: ascending 8-entry block ids, -1 padded.
 *   pool_scores [B*Q][8P] fp32 out: position p scores entry
 *               pool_blocks[p/8]*8 + p%8, -inf if the block is -1 or the
 *               entry is not visible.  Same score definition as above. */
csa2_status csa2_index_reindex(const uint16_t* q_idx, int32_t B, int32_t Q, int32_t H_i, const csa2_idx_k* k,
                               const int32_t* n_vis, const int32_t* pool_blocks, int32_t P, float* pool_scores,
                               hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Top-K selection (aprilzz.com CSA2 section: "selects a new Top-512").
 *   scores [rows][n] fp32, -inf = invalid (never selected).
 *   Order: score descending, position ascending on ties.  The min(k, #valid)
 *   selected positions are written ascending to out_idx[rows][k], -1 padded.
 *   pool_blocks NULL, or [rows][n/8]: position p is reported as entry
 *   pool_blocks[p/8]*8 + p%8 (n must then be a multiple of 8).
 *   1 <= k <= 2048.  Workspace: csa2_topk_workspace_size(rows, n, k) bytes,
 *   device memory, contents need not be initialised.
 * Also builds the hierarchical pool: csa2_topk(block_max, rows, nblocks, 2048,
 * NULL, pool_blocks, ...). */
size_t csa2_topk_workspace_size(int32_t rows, int32_t n, int32_t k);
csa2_status csa2_topk(const float* scores, int32_t rows, int32_t n, int32_t k, const int32_t* pool_blocks,
                      int32_t* out_idx, void* ws, size_t ws_bytes, hipStream_t stream);

/* Allocation-free Top-K, for callers that cannot allocate device memory
 * (code under HIP graph capture, serving loops, harnesses that forbid
 * hipMalloc).  Same arguments and result as csa2_topk without the workspace:
 * rows longer than 32768 positions use a scratch array built into the library
 * (5,243,904 bytes per GPU, held until the process ends) that serves at most 64
 * rows; more rows return CSA2_EUNSUPPORTED with nothing enqueued.  The call
 * allocates nothing.  Every call on one GPU uses that GPU's single scratch
 * array: calls that overlap on one GPU (other streams, other threads) race
 * and must be ordered by the caller.  The scratch's counters are cleared by
 * a kernel each call (no memset node). */
csa2_status csa2_topk_noalloc(const float* scores, int32_t rows, int32_t n, int32_t k, const int32_t* pool_blocks,
                              int32_t* out_idx, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Sparse attention over the selected FP4 entries (partial, to be merged with
 * the window).  K = V = the dequantised latent entry (MQA over one latent).
 *   q    [B][Q][H][D] fp32 or bf16        idx [B][Q][K] int32 entry ids, -1 = none
 *   o    [B][Q][H][D] fp32 out, normalised over this key set
 *   lse  [B][Q][H]    fp32 out, natural-log sum of exp(sm_scale * q.k) (-inf if empty)
 * H % 16 == 0, H <= 64; D in {128, 256, 512}.  Workspace from
 * csa2_attn_workspace_size (may be 0).  codes must be 16-byte and scales
 * 4-byte aligned, and the cache must hold at least one row (row 0 is read, and
 * ignored, in place of missing entries).  Errors: CSA2_EINVAL for null or
 * misaligned pointers and out-of-range sizes, CSA2_EUNSUPPORTED for other H/D,
 * CSA2_EWORKSPACE for a short workspace; nothing is enqueued on error. */
size_t csa2_attn_workspace_size(int32_t B, int32_t Q, int32_t H, int32_t D);
csa2_status csa2_sparse_attn_fp4(const void* q, csa2_dtype qt, int32_t B, int32_t Q, int32_t H,
                                 const csa2_fp4_kv* kv, const int32_t* idx, int32_t K, float sm_scale, float* o,
                                 float* lse, void* ws, size_t ws_bytes, hipStream_t stream);

/* Sliding-window attention over the layer's own bf16 latent rows
 * (aprilzz.com section "把 prefill 砍掉一半": 128-token window in every layer).
 * Window ring: the layer's window row of token t (absolute position in its
 * sequence) lives in swa_kv[b][t mod T] -- the rule csa2_append_token and
 * csa2_swa_replay write by.
 *   swa_kv [B][T][D] bf16 ring; q_pos [B][Q] int32: the query token's absolute
 *   position p; keys = the rows of tokens max(0, p-window+1) .. p (the query
 *   token included).  1 <= window <= T, so no two tokens of a window share a
 *   row; p < 0 gives an empty window.
 *   merge == 0: write o/lse of this key set.  merge == 1: o/lse already hold a
 *   partial over a disjoint key set; combine both into one softmax (exact
 *   log-sum-exp merge) in place.
 * The window rows are converted to fp16 inside the kernel: values must satisfy
 * |v| < 65504 (smaller than 2^-14 lose precision as fp16 subnormals). */
csa2_status csa2_swa_attn(const void* q, csa2_dtype qt, int32_t B, int32_t Q, int32_t H, int32_t D,
                          const uint16_t* swa_kv, int32_t T, const int32_t* q_pos, int32_t window, float sm_scale,
                          int32_t merge, float* o, float* lse, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Layer-mode dispatcher (gkm0120.cn section 2.2.2; aprilzz.com CSA2 section).
 * One call runs one layer of a static pattern:
 *   FULL    : index_full over all visible entries -> Top-K -> idx;
 *             if build_pool, also block max -> Top-P blocks -> pool.
 *   REINDEX : index_reindex inside st->pool with this layer's q_idx -> Top-K -> idx.
 *   REUSE   : no indexer; attends with the latest idx.
 * then sparse attention over idx merged with the layer's SWA.
 * Returns CSA2_EMODE (nothing enqueued) for REUSE before any selection or
 * REINDEX before a pool exists in st. */
typedef struct csa2_layer_args {
    int32_t B, Q, H, H_i, K, P;
    /* per layer */
    const void* q;           /* [B][Q][H][D] main query */
    csa2_dtype qt;
    const uint16_t* q_idx;   /* [B][Q][H_i][D_i] indexer query (FULL/REINDEX), may be NULL for REUSE */
    const uint16_t* swa_kv;  /* [B][T][D] bf16 window ring (row t mod T holds token t) */
    int32_t T;
    const int32_t* q_pos;    /* [B][Q] absolute token position of each query row */
    int32_t window;          /* 1 <= window <= T */
    float sm_scale;
    float* o;                /* [B][Q][H][D] fp32 out */
    float* lse;              /* [B][Q][H] fp32 out */
    /* shared across the layers of a stack */
    const csa2_fp4_kv* kv;
    const csa2_idx_k* k;
    const int32_t* n_vis;    /* [B][Q] */
    int32_t n_max;
    int32_t build_pool;      /* FULL only */
    void* ws;
    size_t ws_bytes;
} csa2_layer_args;

typedef struct csa2_group_state {
    int32_t* idx;            /* [B*Q][K] device: latest selection */
    int32_t* pool;           /* [B*Q][P] device: pool blocks of the last pool-building FULL */
    int32_t has_idx;         /* host flags, maintained by csa2_layer_forward */
    int32_t has_pool;
    /* Host bookkeeping of the workspace's selection counters, maintained by
     * csa2_layer_forward (initialise all three to 0).  The counters sit at the
     * start of the workspace and depend only on B*Q; they are cleared once and
     * every later call leaves them cleared again.  A call re-clears them when
     * the workspace pointer or B*Q differs from the recorded ones, so one
     * state may move between workspaces and shapes (n_max, K, P may change
     * from call to call).  ws_clean is reset to 0 after an error status. */
    int32_t ws_clean;
    int32_t clean_rows;
    const void* clean_ws;
    /* Staged copy (maintained by csa2_layer_forward; initialise to 0): with
     * many query rows per sequence (Q >= 256, D = 512, H = 64, bf16 queries,
     * Q*K >= 2*n_max) a Full layer writes an fp16 copy of the FP4 entries by
     * logical position into the workspace (B*n_max*D*2 bytes, counted by
     * csa2_layer_workspace_size) and attends from it; later Reindex and Reuse
     * layers of the group read the same copy while has_stage is set and the
     * workspace, B*Q and n_max are the ones recorded.  Its values are the
     * cache's decode, so the outputs are bit for bit those of the FP4 path.
     * Clear has_stage, like has_idx, whenever the cache changes outside a Full
     * layer of the group. */
    int32_t has_stage;
    int32_t stage_n;
} csa2_group_state;

size_t csa2_layer_workspace_size(int32_t B, int32_t Q, int32_t H, int32_t D, int32_t n_max, int32_t K, int32_t P);
csa2_status csa2_layer_forward(csa2_mode mode, const csa2_layer_args* a, csa2_group_state* st,
                               hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
