// Indexer scoring: Full mode over every visible entry, Reindex mode over the
// hierarchical pool (gkm0120.cn survey sections 2.2.2-2.2.3; aprilzz.com V4.1
// Flash article, section "CSA2：在层的维度上共享缓存").
//
// Score of entry j for query row r: s_j = sum_h dot(q_h, k_j) with one bf16
// indexer-K vector per entry shared by all heads.  It is evaluated as
//   qbar_c = sum_h q_hc (fp32, h ascending)   then   s_j = FMA chain over c (fp32, c ascending)
// so every entry costs D_i FMAs and the scan is a pure HBM stream of the
// indexer K (2*D_i bytes per entry).  The chain order is part of the
// definition: the Top-K that follows is an integer result decided by these
// fp32 values, so it must be reproduced exactly, not approximately.
//
// Work decomposition: a 256-thread workgroup takes tiles of 256 entries.  The
// tile (64 KB at D_i = 128) is read with fully coalesced 16-byte loads and
// written to LDS with a 16-byte XOR swizzle; each thread then reads back one
// whole entry (conflict-free) and runs its FMA chain.  8 consecutive lanes hold
// an aligned 8-entry block, so the block max for the pool is three lane shuffles.
#include "common.h"

namespace csa2 {
namespace {

constexpr int TILE = 256;

struct IndexParams {
    const uint16_t* q_idx;     // [rows][H_i][DI]
    int32_t H_i, Q;
    const uint16_t* k;         // indexer K plane
    RowMap kmap;
    const int32_t* n_vis;      // [rows]
    int64_t n_pos;             // positions per row: n_max (Full) or 8P (Reindex)
    const int32_t* pool;       // [rows][P] (Reindex)
    int32_t P;
    float* scores;             // [rows][n_pos]
    float* block_max;          // [rows][ceil(n_pos/8)] or null (Full)
    int64_t tiles_per_row;
};

template <int DI, bool REINDEX>
__global__ __launch_bounds__(TILE, 2) void index_kernel(IndexParams p) {
    constexpr int CH = DI / 8;  // 16-byte chunks per entry
    __shared__ uint4 tile[TILE * CH];
    __shared__ int64_t rowtab[TILE];
    __shared__ float4 qbar_s[DI / 4];

    const int t = threadIdx.x;
    const int r = blockIdx.y;
    const int b = r / p.Q;
    const int64_t nv = min((int64_t)p.n_vis[r], p.kmap.capacity);

    // qbar_c = sum over heads, ascending, fp32
    if (t < DI) {
        const uint16_t* qr = p.q_idx + (int64_t)r * p.H_i * DI + t;
        float acc = 0.0f;
        for (int h = 0; h < p.H_i; ++h) acc = acc + __uint_as_float((uint32_t)qr[(int64_t)h * DI] << 16);
        reinterpret_cast<float*>(qbar_s)[t] = acc;
    }
    __syncthreads();

    const int64_t nblocks = (p.n_pos + 7) / 8;
    for (int64_t ti = blockIdx.x; ti < p.tiles_per_row; ti += gridDim.x) {
        const int64_t p0 = ti * TILE;
        // 1. physical row of every entry of the tile (-1 = not visible)
        const int64_t pos = p0 + t;
        int64_t j = -1;
        if (pos < p.n_pos) {
            if (REINDEX) {
                int32_t blk = p.pool[(int64_t)r * p.P + (pos >> 3)];
                if (blk >= 0) j = (int64_t)blk * 8 + (pos & 7);
            } else {
                j = pos;
            }
        }
        const bool valid = j >= 0 && j < nv;
        rowtab[t] = valid ? phys_row(p.kmap, b, j) : -1;
        __syncthreads();
        // 2. coalesced load of the tile into swizzled LDS
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int L = i * TILE + t;
            const int e = L / CH, c = L % CH;
            const int64_t row = rowtab[e];
            uint4 v = make_uint4(0, 0, 0, 0);
            if (row >= 0) v = *reinterpret_cast<const uint4*>(p.k + row * DI + c * 8);
            tile[e * CH + (c ^ (e & (CH - 1)))] = v;
        }
        __syncthreads();
        // 3. one entry per thread: sequential FMA chain over channels
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const uint4 v = tile[t * CH + (c ^ (t & (CH - 1)))];
            const float4 qa = qbar_s[2 * c], qb = qbar_s[2 * c + 1];  // same address in every lane: broadcast
            acc = fmaf(qa.x, bf16_lo(v.x), acc);
            acc = fmaf(qa.y, bf16_hi(v.x), acc);
            acc = fmaf(qa.z, bf16_lo(v.y), acc);
            acc = fmaf(qa.w, bf16_hi(v.y), acc);
            acc = fmaf(qb.x, bf16_lo(v.z), acc);
            acc = fmaf(qb.y, bf16_hi(v.z), acc);
            acc = fmaf(qb.z, bf16_lo(v.w), acc);
            acc = fmaf(qb.w, bf16_hi(v.w), acc);
        }
        const float s = valid ? acc : -INFINITY;
        if (pos < p.n_pos) p.scores[(int64_t)r * p.n_pos + pos] = s;
        if (!REINDEX && p.block_max != nullptr) {
            float m = s;
            m = fmaxf(m, __shfl_xor(m, 1));
            m = fmaxf(m, __shfl_xor(m, 2));
            m = fmaxf(m, __shfl_xor(m, 4));
            if ((t & 7) == 0 && (pos >> 3) < nblocks) p.block_max[(int64_t)r * nblocks + (pos >> 3)] = m;
        }
        // the next iteration rewrites rowtab/tile only after its own barrier
    }
}

csa2_status check_common(const char* what, const uint16_t* q_idx, int32_t B, int32_t Q, int32_t H_i,
                         const csa2_idx_k* k, const int32_t* n_vis, int64_t n_entries, RowMap* map) {
    CSA2_ARG(k != nullptr, "%s: null indexer-K view", what);
    CSA2_ARG(B >= 0 && Q >= 0, "%s: B=%d Q=%d must be >= 0", what, B, Q);
    CSA2_ARG((int64_t)B * Q <= 65535, "%s: B*Q=%lld rows exceeds 65535", what, (long long)B * Q);
    CSA2_ARG(H_i >= 1 && H_i <= 64, "%s: H_i=%d must be in [1, 64]", what, H_i);
    CSA2_REQUIRE(k->D_i == 64 || k->D_i == 128, CSA2_EUNSUPPORTED, "%s: D_i=%d (supported: 64, 128)", what, k->D_i);
    if ((int64_t)B * Q == 0) return CSA2_OK;
    CSA2_ARG(q_idx && k->k && n_vis, "%s: null pointer", what);
    CSA2_ARG(aligned(k->k, 16), "%s: indexer K must be 16-byte aligned", what);
    return make_rowmap(k->page_table, k->page_size, k->max_pages, k->seq_stride, n_entries, map, what);
}

csa2_status launch_index(IndexParams& p, int rows, int D_i, bool reindex, hipStream_t stream, const char* what) {
    p.tiles_per_row = (p.n_pos + TILE - 1) / TILE;
    if (p.tiles_per_row == 0 || rows == 0) return CSA2_OK;
    // enough workgroups to fill 256 CUs x 2 several times over; each loops over tiles
    int64_t gx = p.tiles_per_row;
    const int64_t target = 4096;
    if (gx * rows > target) gx = (target + rows - 1) / rows;
    if (gx < 1) gx = 1;
    dim3 grid((unsigned)gx, (unsigned)rows);
    if (D_i == 128) {
        if (reindex)
            index_kernel<128, true><<<grid, TILE, 0, stream>>>(p);
        else
            index_kernel<128, false><<<grid, TILE, 0, stream>>>(p);
    } else {
        if (reindex)
            index_kernel<64, true><<<grid, TILE, 0, stream>>>(p);
        else
            index_kernel<64, false><<<grid, TILE, 0, stream>>>(p);
    }
    return launch_status(what);
}

}  // namespace
}  // namespace csa2

using namespace csa2;

extern "C" csa2_status csa2_index_full(const uint16_t* q_idx, int32_t B, int32_t Q, int32_t H_i,
                                       const csa2_idx_k* k, const int32_t* n_vis, int32_t n_max, float* scores,
                                       float* block_max, hipStream_t stream) {
    clear_error();
    CSA2_ARG(n_max >= 0, "index_full: n_max=%d < 0", n_max);
    RowMap map;
    csa2_status st = check_common("index_full", q_idx, B, Q, H_i, k, n_vis, n_max, &map);
    if (st != CSA2_OK || (int64_t)B * Q == 0 || n_max == 0) return st;
    CSA2_ARG(scores != nullptr, "index_full: null scores");
    IndexParams p{};
    p.q_idx = q_idx;
    p.H_i = H_i;
    p.Q = Q;
    p.k = k->k;
    p.kmap = map;
    p.n_vis = n_vis;
    p.n_pos = n_max;
    p.scores = scores;
    p.block_max = block_max;
    return launch_index(p, B * Q, k->D_i, false, stream, "index_full");
}

extern "C" csa2_status csa2_index_reindex(const uint16_t* q_idx, int32_t B, int32_t Q, int32_t H_i,
                                          const csa2_idx_k* k, const int32_t* n_vis, const int32_t* pool_blocks,
                                          int32_t P, float* pool_scores, hipStream_t stream) {
    clear_error();
    CSA2_ARG(P >= 0 && P <= (1 << 27), "index_reindex: P=%d out of range", P);
    RowMap map;
    // the pool may name any block of the sequence; the view is checked for one page at least
    csa2_status st = check_common("index_reindex", q_idx, B, Q, H_i, k, n_vis, 1, &map);
    if (st != CSA2_OK || (int64_t)B * Q == 0 || P == 0) return st;
    CSA2_ARG(pool_blocks && pool_scores, "index_reindex: null pointer");
    IndexParams p{};
    p.q_idx = q_idx;
    p.H_i = H_i;
    p.Q = Q;
    p.k = k->k;
    p.kmap = map;
    p.n_vis = n_vis;
    p.n_pos = (int64_t)8 * P;
    p.pool = pool_blocks;
    p.P = P;
    p.scores = pool_scores;
    return launch_index(p, B * Q, k->D_i, true, stream, "index_reindex");
}
