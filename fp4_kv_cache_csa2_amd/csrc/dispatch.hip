// Layer-mode dispatcher: runs one layer of a static Full / Reindex / Reuse
// pattern over shared caches (gkm0120.cn survey, section 2.2.2 mode table;
// aprilzz.com V4.1 Flash article, section "CSA2：在层的维度上共享缓存").
//   Full    : indexer over every visible entry -> new Top-K (and, for a group
//             that holds Reindex layers, the pool of the best 8-entry blocks);
//   Reindex : indexer with the layer's own query, only inside the pool -> new Top-K;
//   Reuse   : no indexer; the latest Top-K is attended again.
// Every layer then attends with its own main query over the selected FP4
// entries and its own window rows in one fused kernel.
#include "internal.h"

namespace csa2 {
namespace {

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct LayerWs {
    size_t scores, block_max, pool_scores, topk, attn, total;
    size_t topk_bytes, attn_bytes;
};

LayerWs layer_ws(int64_t rows, int H, int D, int64_t n_max, int K, int P) {
    LayerWs w{};
    const int64_t nblocks = (n_max + 7) / 8;
    size_t off = 0;
    w.scores = off;
    off = align256(off + (size_t)(rows * n_max) * 4);
    w.block_max = off;
    off = align256(off + (size_t)(rows * nblocks) * 4);
    w.pool_scores = off;
    off = align256(off + (size_t)(rows * 8 * (int64_t)P) * 4);
    // two selections (entries, pool blocks) may run side by side
    const size_t tk = (n_max > TOPK_ONEWG_N || 8 * (int64_t)P > TOPK_ONEWG_N) ? 2 * topk_large_ws_bytes(rows) : 0;
    w.topk = off;
    w.topk_bytes = tk;
    off = align256(off + tk);
    w.attn = off;
    w.attn_bytes = attn_workspace_bytes(rows, H, D);
    off = align256(off + w.attn_bytes);
    w.total = off;
    return w;
}

}  // namespace
}  // namespace csa2

using namespace csa2;

extern "C" size_t csa2_layer_workspace_size(int32_t B, int32_t Q, int32_t H, int32_t D, int32_t n_max, int32_t K,
                                            int32_t P) {
    if (B <= 0 || Q <= 0 || n_max < 0 || K <= 0 || P < 0) return 0;
    return layer_ws((int64_t)B * Q, H, D, n_max, K, P).total;
}

extern "C" csa2_status csa2_layer_forward(csa2_mode mode, const csa2_layer_args* a, csa2_group_state* st,
                                          hipStream_t stream) {
    clear_error();
    CSA2_ARG(a != nullptr && st != nullptr, "layer_forward: null args or state");
    CSA2_ARG(mode == CSA2_FULL || mode == CSA2_REINDEX || mode == CSA2_REUSE, "layer_forward: bad mode %d",
             (int)mode);
    CSA2_ARG(a->B >= 0 && a->Q >= 0, "layer_forward: B=%d Q=%d", a->B, a->Q);
    CSA2_ARG(a->K >= 1 && a->K <= 2048, "layer_forward: K=%d must be in [1, 2048]", a->K);
    CSA2_ARG(a->kv != nullptr && a->k != nullptr, "layer_forward: null cache views");
    CSA2_ARG(st->idx != nullptr, "layer_forward: state has no idx buffer");
    const bool indexer = mode != CSA2_REUSE;
    const bool pool = (mode == CSA2_FULL && a->build_pool) || mode == CSA2_REINDEX;
    if (pool) {
        CSA2_ARG(a->P >= 1 && a->P <= 2048, "layer_forward: P=%d must be in [1, 2048]", a->P);
        CSA2_ARG(st->pool != nullptr, "layer_forward: state has no pool buffer");
    }
    CSA2_REQUIRE(mode != CSA2_REUSE || st->has_idx, CSA2_EMODE, "layer_forward: Reuse layer before any selection");
    CSA2_REQUIRE(mode != CSA2_REINDEX || st->has_pool, CSA2_EMODE,
                 "layer_forward: Reindex layer before a Full layer built a pool");
    if (indexer) CSA2_ARG(a->q_idx != nullptr && a->n_vis != nullptr, "layer_forward: null q_idx / n_vis");
    const int64_t rows = (int64_t)a->B * a->Q;
    if (rows == 0) return CSA2_OK;
    // the layout depends only on the shapes, never on the mode: every layer of a
    // group passes the same P and shares the workspace (and the zeroed Reindex
    // histogram kept in it)
    CSA2_ARG(a->P >= 0 && a->P <= 2048, "layer_forward: P=%d must be in [0, 2048]", a->P);
    const LayerWs w = layer_ws(rows, a->H, a->kv->D, a->n_max, a->K, a->P);
    CSA2_REQUIRE(a->ws != nullptr && a->ws_bytes >= w.total, CSA2_EWORKSPACE,
                 "layer_forward: workspace of %zu bytes required, %zu given", w.total,
                 a->ws ? a->ws_bytes : (size_t)0);
    CSA2_ARG(((uintptr_t)a->ws & 255) == 0, "layer_forward: workspace must be 256-byte aligned");
    char* ws = static_cast<char*>(a->ws);
    float* scores = reinterpret_cast<float*>(ws + w.scores);
    float* block_max = reinterpret_cast<float*>(ws + w.block_max);
    float* pool_scores = reinterpret_cast<float*>(ws + w.pool_scores);
    void* tk = ws + w.topk;
    (void)w.topk_bytes;
    void* aw = ws + w.attn;
    const int rows32 = (int)rows;
    csa2_status s = CSA2_OK;
    bool topk_ws_used = false;
    if (mode == CSA2_FULL) {
        // Top-K entries and pool blocks: large selections share the zero /
        // split / finish launches; their first-digit histograms come out of the scan
        const int32_t n = a->n_max, nb = (int32_t)((a->n_max + 7) / 8);
        const bool e_large = n > TOPK_ONEWG_N;
        const bool b_large = a->build_pool && nb > TOPK_ONEWG_N;  // implies e_large
        TopkSegs segs{};
        segs.rows = rows32;
        TopkSeg* se = nullptr;
        TopkSeg* sb = nullptr;
        if (e_large) {
            se = &segs.seg[segs.nseg++];
            *se = TopkSeg{scores, n, a->K, nullptr, st->idx, a->n_vis, 1};
            topk_carve(tk, rows, se);
        }
        if (b_large) {
            sb = &segs.seg[segs.nseg++];
            *sb = TopkSeg{block_max, nb, a->P, nullptr, st->pool, a->n_vis, 8};
            topk_carve(static_cast<char*>(tk) + topk_large_ws_bytes(rows), rows, sb);
        }
        // the histograms and row states must start at zero: cleared here once
        // per workspace, then left cleared by the finish pass of every call
        topk_ws_used = segs.nseg > 0;
        if (!st->ws_clean && segs.nseg) {
            ZeroRanges z{};
            for (int i = 0; i < segs.nseg; ++i) {
                z.ptr[z.n] = segs.seg[i].hist;
                z.count[z.n++] = rows * NBINS1;
                z.ptr[z.n] = reinterpret_cast<uint32_t*>(segs.seg[i].state);
                z.count[z.n++] = rows * (int64_t)(sizeof(TopkRowState) / 4);
            }
            launch_zero_ranges(z, stream);
        }
        // scores past a row's n_vis are neither written nor read.  Several query
        // rows per sequence: the scan shares each K block among them and the
        // first-digit histograms come from their own pass
        const bool multi = a->Q >= 2;
        s = index_full_hist(a->q_idx, a->B, a->Q, a->H_i, a->k, a->n_vis, n, scores,
                            a->build_pool ? block_max : nullptr, se && !multi ? se->hist : nullptr,
                            se && !multi ? se->state : nullptr, sb && !multi ? sb->hist : nullptr,
                            sb && !multi ? sb->state : nullptr, true, stream);
        if (s != CSA2_OK) return s;
        if (segs.nseg && multi) topk_launch_hist(segs, stream);
        if (segs.nseg) topk_launch_select(segs, stream);
        if (!e_large) topk_launch_small(scores, rows32, n, a->K, nullptr, st->idx, stream, a->n_vis, 1);
        if (a->build_pool && !b_large)
            topk_launch_small(block_max, rows32, nb, a->P, nullptr, st->pool, stream, a->n_vis, 8);
        s = launch_status("layer_forward");
    } else if (mode == CSA2_REINDEX) {
        // (the pool scores' first-digit histogram is built inside the select:
        // flushing it from the scan's many workgroups with contended atomics costs more)
        s = index_reindex_hist(a->q_idx, a->B, a->Q, a->H_i, a->k, a->n_vis, st->pool, a->P, pool_scores, nullptr,
                               nullptr, stream);
        if (s == CSA2_OK) {
            topk_launch_small(pool_scores, rows32, 8 * a->P, a->K, st->pool, st->idx, stream);
            s = launch_status("layer_forward");
        }
    }
    if (s != CSA2_OK) {
        st->ws_clean = 0;
        return s;
    }
    if (mode == CSA2_FULL) {
        if (topk_ws_used) st->ws_clean = 1;
        st->has_idx = 1;
        if (a->build_pool) st->has_pool = 1;
    } else if (mode == CSA2_REINDEX) {
        st->has_idx = 1;
    }
    return attn_launch(a->q, a->qt, a->B, a->Q, a->H, a->kv->D, a->kv, st->idx, a->K, a->swa_kv, a->T, a->q_slot,
                       a->window, a->sm_scale, 0, a->o, a->lse, aw, w.attn_bytes, stream, "layer_forward");
}
