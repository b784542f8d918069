// Internal interfaces shared by the kernels' translation units: the Top-K
// selector (whose first-digit histogram the Full-mode scan can build while it
// scores), the scan launcher with those histograms, and the attention
// launcher used by both the standalone entry points and the layer dispatcher.
#pragma once
#include <cstddef>

#include "common.h"

namespace csa2 {

constexpr int TOPK_KMAX = 2048;       // largest k
constexpr int TOPK_SMALL_N = 16384;   // one workgroup per row, 16 keys per thread
constexpr int TOPK_ONEWG_N = 32768;   // rows up to this length are selected by one workgroup (32 keys per thread)
constexpr int TOPK_CAP = 8192;        // candidates kept per row from the threshold bin
constexpr int NBINS1 = 2048;          // first digit: top 11 bits of the order-preserving key

// fp32 -> order-preserving unsigned key (-0 folded into +0); -inf -> 0 (invalid).
__device__ __forceinline__ uint32_t key32(float s) {
    if (s == -INFINITY) return 0u;
    const uint32_t u = __float_as_uint(s + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct TopkRowState {
    uint32_t n_sel;   // positions above the threshold bin (definitely selected)
    uint32_t n_cand;  // positions inside the threshold bin
    uint32_t valid;   // valid (finite) positions of the row
    uint32_t digit;   // the threshold bin
};
// n_sel and n_cand form one 8-byte word: a split workgroup reserves room in
// both lists with a single 64-bit atomic (workspaces are 16-byte aligned)
static_assert(sizeof(TopkRowState) == 16 && offsetof(TopkRowState, n_sel) == 0 &&
                  offsetof(TopkRowState, n_cand) == 4,
              "list counters must share one 8-byte word");

// One selection problem: rows x n scores -> rows x k indices.  The last five
// pointers are carved from a workspace by topk_carve.
struct TopkSeg {
    const float* scores;
    int32_t n, k;
    const int32_t* pool;   // NULL or [rows][n/8] position -> entry map
    int32_t* out;          // [rows][k]
    const int32_t* lim;    // NULL, or [rows]: positions >= ceil(lim[row] / lim_div) are invalid and unread
    int32_t lim_div;
    uint32_t* hist;        // [rows][NBINS1]
    TopkRowState* state;   // [rows]
    int* sel;              // [rows][TOPK_KMAX]
    uint32_t* ckey;        // [rows][TOPK_CAP]
    uint32_t* cpos;        // [rows][TOPK_CAP]
};

struct TopkSegs {
    TopkSeg seg[2];
    int32_t nseg;
    int32_t rows;
};

// Workspace of one large selection: its counters (row histograms and row
// states, which must be zero when the selection starts and are left zero by
// it) and its lists (no initial contents).  The two parts are carved
// separately so that a caller can keep the counters at a place that does not
// move when other sizes (n, k) change.
size_t topk_counter_bytes(int64_t rows);
size_t topk_list_bytes(int64_t rows);
size_t topk_large_ws_bytes(int64_t rows);  // both parts in one region (16-byte aligned)
void topk_carve(void* counters, void* lists, int64_t rows, TopkSeg* sg);
// zero the histograms and row states of every segment
void topk_launch_zero(const TopkSegs& segs, hipStream_t stream);
// build the first-digit histograms (not needed when the scan built them)
void topk_launch_hist(const TopkSegs& segs, hipStream_t stream);
// threshold split + candidate select + sorted output
void topk_launch_select(const TopkSegs& segs, hipStream_t stream);
// one workgroup per row (n <= TOPK_ONEWG_N); lim as in TopkSeg
void topk_launch_small(const float* scores, int rows, int n, int k, const int32_t* pool, int32_t* out,
                       hipStream_t stream, const int32_t* lim = nullptr, int lim_div = 1);

// Zero up to 6 ranges of 32-bit words in one launch.
struct ZeroRanges {
    uint32_t* ptr[6];
    int64_t count[6];
    int32_t n;
};
void launch_zero_ranges(const ZeroRanges& z, hipStream_t stream);

// Reindex-mode scan that also builds the first-digit histogram of the pool
// scores (hist/st may be NULL).
csa2_status index_reindex_hist(const uint16_t* q_idx, int32_t B, int32_t Q, int32_t H_i, const csa2_idx_k* k,
                               const int32_t* n_vis, const int32_t* pool_blocks, int32_t P, float* pool_scores,
                               uint32_t* hist, TopkRowState* st, hipStream_t stream);

// Full-mode scan that also builds the Top-K first-digit histograms of the
// entry scores (hist_e/st_e) and of the block maxima (hist_b/st_b; may be NULL).
csa2_status index_full_hist(const uint16_t* q_idx, int32_t B, int32_t Q, int32_t H_i, const csa2_idx_k* k,
                            const int32_t* n_vis, int32_t n_max, float* scores, float* block_max, uint32_t* hist_e,
                            TopkRowState* st_e, uint32_t* hist_b, TopkRowState* st_b, bool skip_invisible,
                            hipStream_t stream);

// Screened many-row Full selection (matrix-core screen, exact rescoring of the
// candidates, exact selection): the Top-K of every row into out[rows][K];
// scratch [rows][n_max] fp32 holds the exact scores of rows selected in full.
bool screen_applicable(int32_t B, int32_t Q, int32_t D_i, int32_t n_max, int32_t K);
size_t screen_ws_bytes(int32_t B, int32_t Q, int32_t n_max);
csa2_status screen_select(const uint16_t* q_idx, int32_t B, int32_t Q, int32_t H_i, const csa2_idx_k* k,
                          const int32_t* n_vis, int32_t n_max, int32_t K, void* ws, size_t ws_bytes, float* scratch,
                          int32_t* out, hipStream_t stream);

csa2_status attn_launch(const void* q, csa2_dtype qt, int32_t B, int32_t Q, int32_t H, int32_t D,
                        const csa2_fp4_kv* kv, const int32_t* idx, int32_t K, const uint16_t* swa, int32_t T,
                        const int32_t* q_pos, int32_t window, float sm_scale, int32_t merge, float* o, float* lse,
                        void* ws, size_t ws_bytes, hipStream_t stream, const char* what,
                        const uint16_t* k16 = nullptr, int64_t n_stage = 0);
size_t attn_workspace_bytes(int64_t rows, int H, int D);
// fp16 copy of a cache's entries by logical position, k16[b n_stage + j][D]
// for j < n_stage (zeros where the page table maps no page); the prefill
// attention of a group reads it instead of dequantising every selected entry
bool attn_stage_applicable(int32_t B, int32_t Q, int32_t H, int32_t D, int32_t K);
size_t attn_stage_bytes(int32_t B, int32_t Q, int32_t H, int32_t D, int32_t n_max, int32_t K);
csa2_status attn_stage_cache(const csa2_fp4_kv* kv, int32_t B, int64_t n_stage, uint16_t* k16, hipStream_t stream);

}  // namespace csa2
