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
// Work decomposition: every wavefront streams its own blocks of 64 entries
// (16 KB at D_i = 128) with no workgroup barrier in the loop.  A block is
// read with fully coalesced 16-byte loads into registers, written to the
// wave's private LDS tile with a 16-byte XOR swizzle, and read back one whole
// entry per lane (conflict-free); the loads of the wave's next block are in
// flight while the current one is scored.  8 consecutive lanes hold an
// aligned 8-entry block, so the block max for the pool is three lane shuffles.
#include "internal.h"

namespace csa2 {
namespace {

constexpr int WAVES = 4;      // wavefronts per workgroup
constexpr int EPB = 64;       // entries per wave block (one per lane)
constexpr int BM_STASH = 32;  // blocks per wave whose maxima are held back (the launch gives at most 32)

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
    int64_t blocks_per_row;    // ceil(n_pos / 64)
    int32_t skip_invisible;    // Full: blocks past n_vis are not written at all (their
                               // readers bound each row by n_vis); else they get -inf
    // optional first-digit histograms for the Top-K that follows (Full only)
    uint32_t* hist_e;          // [rows][NBINS1] of the entry scores
    TopkRowState* state_e;
    uint32_t* hist_b;          // [rows][NBINS1] of the block maxima
    TopkRowState* state_b;
};

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr uint32_t NOROW = 0xFFFFFFFFu;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Physical row of position pos of row r (NOROW: not visible).  A K plane
// holds fewer than 2^32 - 1 rows (it would exceed device memory otherwise).
template <bool REINDEX>
__device__ __forceinline__ uint32_t entry_row(const IndexParams& p, int r, int b, int64_t nv, int64_t pos) {
    if (pos >= p.n_pos) return NOROW;
    int64_t j = pos;
    if (REINDEX) {
        const int32_t blk = p.pool[(int64_t)r * p.P + (pos >> 3)];
        if (blk < 0) return NOROW;
        j = (int64_t)blk * 8 + (pos & 7);
    }
    if (j >= nv) return NOROW;
    return (uint32_t)phys_row(p.kmap, b, j);
}

// Issue the loads of one wave block into registers.  Load i of lane l covers
// 16-byte chunk c of entry e with i*64 + l = e*CH + c.
// A block whose 64 entries are all visible and lie in one run of the K plane:
// a contiguous plane, or pages of at least 64 entries (blocks are 64-aligned,
// so they never straddle such a page).
template <bool CONTIG>
__device__ __forceinline__ bool run_block(const IndexParams& p, int64_t nv, int64_t blk) {
    return (CONTIG || p.kmap.page_shift >= 6) && blk * EPB + EPB <= min(nv, p.n_pos);
}

// FAST: a run block (Full mode) takes the short path below; used by the
// multi-row kernel, where the per-load index arithmetic is a fifth of the VALU
// work, and by the paged single-row scan (the contiguous single-row scan keeps
// the one addressing it was tuned with).
template <int DI, bool REINDEX, bool CONTIG, bool FAST = false>
__device__ __forceinline__ void load_block(const IndexParams& p, int r, int b, int64_t nv, int64_t blk, int lane,
                                           uint32_t myrow, uint4 (&v)[DI / 8]) {
    constexpr int CH = DI / 8;
    const int64_t p0 = blk * EPB;
    if (FAST && !REINDEX && run_block<CONTIG>(p, nv, blk)) {
        // 64 entries in one run of 64 DI bf16, read at a wave-uniform base +
        // 16 lane + 1024 i (no per-load index arithmetic, shuffles or masking)
        const int64_t row0 = CONTIG ? (int64_t)b * p.kmap.seq_stride + p0 : phys_row(p.kmap, b, p0);
        const uint8_t* base = reinterpret_cast<const uint8_t*>(p.k + row0 * DI);
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + 16 * lane + 1024 * i));
            v[i] = make_uint4(x.x, x.y, x.z, x.w);
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int L = i * 64 + lane;
        const int e = L / CH, c = L % CH;
        // loads are unconditional (an invisible entry reads row 0 of the plane,
        // which always exists, and is zeroed after): no divergent branches
        bool ok;
        uint64_t row;
        if (CONTIG) {
            const int64_t pos = p0 + e;
            ok = pos < nv && pos < p.n_pos;
            row = ok ? (uint64_t)((int64_t)b * p.kmap.seq_stride + pos) : 0u;
        } else {
            const uint32_t r32 = (uint32_t)__shfl((int)myrow, e);
            ok = r32 != NOROW;
            row = ok ? (uint64_t)r32 : 0u;
        }
        // non-temporal: the K stream is read once (measured ~12% more HBM
        // throughput than default-cached loads on this access pattern)
        const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.k + row * DI + c * 8));
        // the mask is opaque to the compiler, so it keeps the load unconditional
        uint32_t m;
        asm volatile("v_mov_b32 %0, %1" : "=v"(m) : "v"(ok ? 0xFFFFFFFFu : 0u));
        v[i] = make_uint4(x.x & m, x.y & m, x.z & m, x.w & m);
    }
}

template <int DI, bool REINDEX, bool CONTIG>
__global__ __launch_bounds__(WAVES * 64, REINDEX ? 1 : 2) void index_kernel(IndexParams p) {
    constexpr int CH = DI / 8;  // 16-byte chunks per entry
    __shared__ uint4 tile[WAVES][EPB * CH];
    __shared__ float4 qbar_s[DI / 4];
    // 16-bit bin counters, two per word; a workgroup scores at most 65535
    // positions (the launch guarantees it), so a half never overflows
    __shared__ uint32_t hist_s[2][NBINS1 / 2];
    // Full mode: each wave's block maxima wait here and are written after its
    // last block (interleaved with the K stream, these small writes cost
    // several times their bytes in read bandwidth)
    __shared__ float bm_stash[WAVES][REINDEX ? 1 : BM_STASH * 8];

    const int t = threadIdx.x;
    const int lane = t & 63, w = t >> 6;
    const int r = blockIdx.y;
    const int b = r / p.Q;
    const int64_t nv = min((int64_t)p.n_vis[r], p.kmap.capacity);

    // the first block's row lookups and loads go out before the query sum:
    // neither depends on it, so their round trips overlap
    const int64_t stride = (int64_t)gridDim.x * WAVES;
    int64_t blk = (int64_t)blockIdx.x * WAVES + w;
    const int64_t blk_first = blk;
    const int64_t nbv = REINDEX ? p.blocks_per_row : (min(nv, p.n_pos) + EPB - 1) / EPB;
    // paged Full scan: run blocks skip the per-lane row lookups
    constexpr bool PFAST = !CONTIG && !REINDEX;
    bool full = PFAST && blk < nbv && run_block<CONTIG>(p, nv, blk);
    uint32_t row_next = (CONTIG || blk >= nbv || full) ? 0u : entry_row<REINDEX>(p, r, b, nv, blk * EPB + lane);
    uint4 v[CH];
    if (blk < nbv) load_block<DI, REINDEX, CONTIG, PFAST>(p, r, b, nv, blk, lane, row_next, v);

    // qbar_c = sum over heads, ascending, fp32
    if (t < DI) {
        const uint16_t* qr = p.q_idx + (int64_t)r * p.H_i * DI + t;
        float acc = 0.0f;
        for (int h = 0; h < p.H_i; ++h) acc = acc + __uint_as_float((uint32_t)qr[(int64_t)h * DI] << 16);
        reinterpret_cast<float*>(qbar_s)[t] = acc;
    }
    const bool hist = p.hist_e != nullptr;
    const bool hist_b = !REINDEX && p.hist_b != nullptr;
    if (hist || hist_b)
        for (int i = t; i < NBINS1; i += WAVES * 64) (&hist_s[0][0])[i] = 0u;
    __syncthreads();

    const int64_t nblocks8 = (p.n_pos + 7) / 8;
    uint4* my = tile[w];
    uint32_t n_valid = 0, n_valid_b = 0;  // lane counts for the histograms

    // (Full mode: only blocks holding a visible entry are read)
    int it = 0;  // this wave's blocks so far
    for (; blk < nbv; blk += stride, ++it) {
        const int64_t pos = blk * EPB + lane;
        const bool valid = CONTIG ? (pos < nv && pos < p.n_pos) : (full || row_next != NOROW);
        // An opaque zero, fresh every block: LDS addresses are recomputed each
        // block (two ALU ops each) instead of being hoisted into ~48 registers.
        int z;
        asm volatile("s_mov_b32 %0, 0" : "=s"(z));
        const int lz = lane + z;
        // stage the block in this wave's LDS tile
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int L = i * 64 + lz;
            const int e = L / CH, c = L % CH;
            my[e * CH + (c ^ (e & (CH - 1)))] = v[i];
        }
        wave_sync();
        // next block's loads fly while this one is scored
        const int64_t nxt = blk + stride;
        if (nxt < nbv) {
            full = PFAST && run_block<CONTIG>(p, nv, nxt);
            if (!CONTIG && !full) row_next = entry_row<REINDEX>(p, r, b, nv, nxt * EPB + lane);
            load_block<DI, REINDEX, CONTIG, PFAST>(p, r, b, nv, nxt, lane, row_next, v);
        }
        // one entry per lane: sequential FMA chain over channels.  qbar is
        // re-read from LDS (a broadcast) each block rather than held in 128
        // registers: the opaque zero keeps the compiler from hoisting it.
        const float4* qb_s = qbar_s + z;
        const uint4* mine = my + lz * CH;
        const int sw = lz & (CH - 1);
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const uint4 k4 = mine[c ^ sw];
            const float4 qa = qb_s[2 * c], qb = qb_s[2 * c + 1];  // same address in every lane: broadcast
            acc = fmaf(qa.x, bf16_lo(k4.x), acc);
            acc = fmaf(qa.y, bf16_hi(k4.x), acc);
            acc = fmaf(qa.z, bf16_lo(k4.y), acc);
            acc = fmaf(qa.w, bf16_hi(k4.y), acc);
            acc = fmaf(qb.x, bf16_lo(k4.z), acc);
            acc = fmaf(qb.y, bf16_hi(k4.z), acc);
            acc = fmaf(qb.z, bf16_lo(k4.w), acc);
            acc = fmaf(qb.w, bf16_hi(k4.w), acc);
        }
        wave_sync();  // the tile is rewritten by the next iteration
        const float s = valid ? acc : -INFINITY;
        if (p.scores != nullptr && pos < p.n_pos) p.scores[(int64_t)r * p.n_pos + pos] = s;
        if (hist && valid) {
            const uint32_t d = key32(s) >> 21;
            atomicAdd(&hist_s[0][d >> 1], 1u << (16 * (d & 1)));
            ++n_valid;
        }
        if (!REINDEX && p.block_max != nullptr) {
            float m = s;
            m = fmaxf(m, __shfl_xor(m, 1));
            m = fmaxf(m, __shfl_xor(m, 2));
            m = fmaxf(m, __shfl_xor(m, 4));
            if ((lane & 7) == 0 && (pos >> 3) < nblocks8) {
                if (it < BM_STASH)
                    bm_stash[w][REINDEX ? 0 : it * 8 + (lane >> 3)] = m;
                else
                    p.block_max[(int64_t)r * nblocks8 + (pos >> 3)] = m;
                if (hist_b && m != -INFINITY) {
                    const uint32_t d = key32(m) >> 21;
                    atomicAdd(&hist_s[1][d >> 1], 1u << (16 * (d & 1)));
                    ++n_valid_b;
                }
            }
        }
    }
    if (!REINDEX && p.block_max != nullptr) {
        wave_sync();
        // stashed maxima: block blk_first + j stride holds stash entries 8j..8j+7
        for (int i = lane; i < min(it, BM_STASH) * 8; i += 64) {
            const int64_t b8 = (blk_first + (int64_t)(i >> 3) * stride) * 8 + (i & 7);
            if (b8 < nblocks8) p.block_max[(int64_t)r * nblocks8 + b8] = bm_stash[w][REINDEX ? 0 : i];
        }
    }
    // blocks without a visible entry: -inf, unless the readers skip them
    if (!REINDEX && !p.skip_invisible) {
        for (; blk < p.blocks_per_row; blk += stride) {
            const int64_t pos = blk * EPB + lane;
            if (p.scores != nullptr && pos < p.n_pos) p.scores[(int64_t)r * p.n_pos + pos] = -INFINITY;
            if (p.block_max != nullptr && (lane & 7) == 0 && (pos >> 3) < nblocks8)
                p.block_max[(int64_t)r * nblocks8 + (pos >> 3)] = -INFINITY;
        }
    }
    if (hist || hist_b) {
        // valid counts: one atomic per wave; bins: only the non-empty ones
        for (int off = 32; off > 0; off >>= 1) {
            n_valid += __shfl_xor(n_valid, off);
            n_valid_b += __shfl_xor(n_valid_b, off);
        }
        if (hist && lane == 0 && n_valid) atomicAdd(&p.state_e[r].valid, n_valid);
        if (hist_b && lane == 0 && n_valid_b) atomicAdd(&p.state_b[r].valid, n_valid_b);
        __syncthreads();
        for (int i = t; i < NBINS1; i += WAVES * 64) {
            if (hist) {
                const uint32_t ce = (hist_s[0][i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
                if (ce) atomicAdd(&p.hist_e[(int64_t)r * NBINS1 + i], ce);
            }
            if (hist_b) {
                const uint32_t cb = (hist_s[1][i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
                if (cb) atomicAdd(&p.hist_b[(int64_t)r * NBINS1 + i], cb);
            }
        }
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

// Full-mode scoring of RB query rows of one sequence per workgroup (several
// query tokens of a sequence: multi-token decode, prefill).  Every K block is
// read from memory once for the RB rows; each lane runs RB independent FMA
// chains over its entry, each in the same channel order as the single-row
// kernel, so the scores are identical bit for bit.  No fused histograms.
template <int DI, bool CONTIG, int RB>
__global__ __launch_bounds__(WAVES * 64, 2) void index_multi_kernel(IndexParams p) {
    constexpr int CH = DI / 8;
    __shared__ uint4 tile[WAVES][EPB * CH];
    __shared__ float4 qbar_s[RB][DI / 4];

    const int t = threadIdx.x;
    const int lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int gps = (p.Q + RB - 1) / RB;  // row groups per sequence
    const int b = blockIdx.y / gps;
    const int q0 = (blockIdx.y % gps) * RB;
    const int nr = min(RB, p.Q - q0);
    const int r0 = b * p.Q + q0;
    int64_t nvr[RB];
    int64_t nvmax = 0;
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
        nvr[rr] = rr < nr ? min((int64_t)p.n_vis[r0 + rr], p.kmap.capacity) : 0;
        nvmax = max(nvmax, nvr[rr]);
    }
    // the first block's loads go out before the query sums
    const int64_t stride = (int64_t)gridDim.x * WAVES;
    int64_t blk = (int64_t)blockIdx.x * WAVES + w;
    const int64_t nbv = (min(nvmax, p.n_pos) + EPB - 1) / EPB;
    uint32_t row_next = (CONTIG || blk >= nbv) ? 0u : entry_row<false>(p, r0, b, nvmax, blk * EPB + lane);
    uint4 v[CH];
    if (blk < nbv) load_block<DI, false, CONTIG, true>(p, r0, b, nvmax, blk, lane, row_next, v);

    for (int i = t; i < RB * DI; i += WAVES * 64) {
        const int rr = i / DI, c = i % DI;
        float acc = 0.0f;
        if (rr < nr) {
            const uint16_t* qr = p.q_idx + (int64_t)(r0 + rr) * p.H_i * DI + c;
            for (int h = 0; h < p.H_i; ++h) acc = acc + __uint_as_float((uint32_t)qr[(int64_t)h * DI] << 16);
        }
        reinterpret_cast<float*>(qbar_s[rr])[c] = acc;
    }
    __syncthreads();

    const int64_t nblocks8 = (p.n_pos + 7) / 8;
    uint4* my = tile[w];
    for (; blk < nbv; blk += stride) {
        const int64_t pos = blk * EPB + lane;
        int z;
        asm volatile("s_mov_b32 %0, 0" : "=s"(z));
        const int lz = lane + z;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int L = i * 64 + lz;
            const int e = L / CH, c = L % CH;
            my[e * CH + (c ^ (e & (CH - 1)))] = v[i];
        }
        wave_sync();
        const int64_t nxt = blk + stride;
        if (nxt < nbv) {
            if (!CONTIG) row_next = entry_row<false>(p, r0, b, nvmax, nxt * EPB + lane);
            load_block<DI, false, CONTIG, true>(p, r0, b, nvmax, nxt, lane, row_next, v);
        }
        const uint4* mine = my + lz * CH;
        const int sw = lz & (CH - 1);
        float acc[RB];
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) acc[rr] = 0.0f;
        // (not fully unrolled: the query broadcasts of a few channels at a time
        // stay in registers, not all RB x DI of them)
#pragma unroll 2
        for (int c = 0; c < CH; ++c) {
            const uint4 k4 = mine[c ^ sw];
            const float kf[8] = {bf16_lo(k4.x), bf16_hi(k4.x), bf16_lo(k4.y), bf16_hi(k4.y),
                                 bf16_lo(k4.z), bf16_hi(k4.z), bf16_lo(k4.w), bf16_hi(k4.w)};
#pragma unroll
            for (int rr = 0; rr < RB; ++rr) {
                const float4 qa = qbar_s[rr][2 * c + z], qb = qbar_s[rr][2 * c + 1 + z];  // broadcasts
                acc[rr] = fmaf(qa.x, kf[0], acc[rr]);
                acc[rr] = fmaf(qa.y, kf[1], acc[rr]);
                acc[rr] = fmaf(qa.z, kf[2], acc[rr]);
                acc[rr] = fmaf(qa.w, kf[3], acc[rr]);
                acc[rr] = fmaf(qb.x, kf[4], acc[rr]);
                acc[rr] = fmaf(qb.y, kf[5], acc[rr]);
                acc[rr] = fmaf(qb.z, kf[6], acc[rr]);
                acc[rr] = fmaf(qb.w, kf[7], acc[rr]);
            }
        }
        wave_sync();
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) {
            if (rr >= nr) break;
            const int64_t r = r0 + rr;
            const float s = (pos < nvr[rr] && pos < p.n_pos) ? acc[rr] : -INFINITY;
            if (p.scores != nullptr && pos < p.n_pos) p.scores[r * p.n_pos + pos] = s;
            if (p.block_max != nullptr) {
                float m = s;
                m = fmaxf(m, __shfl_xor(m, 1));
                m = fmaxf(m, __shfl_xor(m, 2));
                m = fmaxf(m, __shfl_xor(m, 4));
                if ((lane & 7) == 0 && (pos >> 3) < nblocks8) p.block_max[r * nblocks8 + (pos >> 3)] = m;
            }
        }
    }
    if (!p.skip_invisible) {
        for (; blk < p.blocks_per_row; blk += stride) {
            const int64_t pos = blk * EPB + lane;
            for (int rr = 0; rr < nr; ++rr) {
                const int64_t r = r0 + rr;
                if (p.scores != nullptr && pos < p.n_pos) p.scores[r * p.n_pos + pos] = -INFINITY;
                if (p.block_max != nullptr && (lane & 7) == 0 && (pos >> 3) < nblocks8)
                    p.block_max[r * nblocks8 + (pos >> 3)] = -INFINITY;
            }
        }
    }
}

csa2_status launch_index(IndexParams& p, int rows, int D_i, bool reindex, hipStream_t stream, const char* what) {
    p.blocks_per_row = (p.n_pos + EPB - 1) / EPB;
    if (p.blocks_per_row == 0 || rows == 0) return CSA2_OK;
    // at least about two resident workgroups per CU on 256 CUs in total, and at
    // most 32 blocks per wave, so that the longest rows of a ragged batch are
    // spread over enough CUs (workgroups past a short row's end exit at once)
    int64_t gx = (p.blocks_per_row + WAVES - 1) / WAVES;
    const int64_t target = 512;
    const int64_t per_wave_cap = (p.blocks_per_row + WAVES * 32 - 1) / (WAVES * 32);
    if (gx * rows > target) gx = max((target + rows - 1) / rows, per_wave_cap);
    // with histograms, a workgroup may score at most 65535 positions (16-bit bins)
    const int64_t min_gx = (p.blocks_per_row + (65535 / (WAVES * EPB)) * WAVES - 1) / ((65535 / (WAVES * EPB)) * WAVES);
    if (gx < min_gx) gx = min_gx;
    if (gx < 1) gx = 1;
    const dim3 block(WAVES * 64);
    const bool contig = !reindex && p.kmap.page_table == nullptr;
    if (!reindex && p.hist_e == nullptr && p.hist_b == nullptr && p.Q >= 2) {
        // RB rows of a sequence per workgroup
        const int rb = p.Q >= 8 ? 8 : (p.Q >= 4 ? 4 : 2);
        const int groups = (rows / p.Q) * ((p.Q + rb - 1) / rb);
        int64_t gm = (p.blocks_per_row + WAVES - 1) / WAVES;
        if (gm * groups > target) gm = max((target + groups - 1) / groups, per_wave_cap);
        if (gm < 1) gm = 1;
        const dim3 grid_m((unsigned)gm, (unsigned)groups);
#define CSA2_IDXM(DD, RBV)                                                                 \
    if (D_i == DD && rb == RBV) {                                                          \
        if (contig)                                                                        \
            index_multi_kernel<DD, true, RBV><<<grid_m, block, 0, stream>>>(p);            \
        else                                                                               \
            index_multi_kernel<DD, false, RBV><<<grid_m, block, 0, stream>>>(p);           \
    }
        CSA2_IDXM(128, 8) CSA2_IDXM(128, 4) CSA2_IDXM(128, 2)
        CSA2_IDXM(64, 8) CSA2_IDXM(64, 4) CSA2_IDXM(64, 2)
#undef CSA2_IDXM
        return launch_status(what);
    }
    const dim3 grid((unsigned)gx, (unsigned)rows);
#define CSA2_IDX(DD)                                                                   \
    if (D_i == DD) {                                                                   \
        if (reindex)                                                                   \
            index_kernel<DD, true, false><<<grid, block, 0, stream>>>(p);              \
        else if (contig)                                                               \
            index_kernel<DD, false, true><<<grid, block, 0, stream>>>(p);              \
        else                                                                           \
            index_kernel<DD, false, false><<<grid, block, 0, stream>>>(p);             \
    }
    CSA2_IDX(128)
    CSA2_IDX(64)
#undef CSA2_IDX
    return launch_status(what);
}

}  // namespace
}  // namespace csa2

using namespace csa2;

csa2_status csa2::index_full_hist(const uint16_t* q_idx, int32_t B, int32_t Q, int32_t H_i, const csa2_idx_k* k,
                                  const int32_t* n_vis, int32_t n_max, float* scores, float* block_max,
                                  uint32_t* hist_e, TopkRowState* st_e, uint32_t* hist_b, TopkRowState* st_b,
                                  bool skip_invisible, hipStream_t stream) {
    CSA2_ARG(n_max >= 0, "index_full: n_max=%d < 0", n_max);
    RowMap map;
    csa2_status st = check_common("index_full", q_idx, B, Q, H_i, k, n_vis, n_max, &map);
    if (st != CSA2_OK || (int64_t)B * Q == 0 || n_max == 0) return st;
    // (the dispatcher may ask for the block maxima alone)
    CSA2_ARG(scores != nullptr || block_max != nullptr, "index_full: null scores and block maxima");
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
    p.hist_e = hist_e;
    p.state_e = st_e;
    p.hist_b = block_max ? hist_b : nullptr;
    p.state_b = st_b;
    p.skip_invisible = skip_invisible ? 1 : 0;
    return launch_index(p, B * Q, k->D_i, false, stream, "index_full");
}

extern "C" csa2_status csa2_index_full(const uint16_t* q_idx, int32_t B, int32_t Q, int32_t H_i,
                                       const csa2_idx_k* k, const int32_t* n_vis, int32_t n_max, float* scores,
                                       float* block_max, hipStream_t stream) {
    clear_error();
    return index_full_hist(q_idx, B, Q, H_i, k, n_vis, n_max, scores, block_max, nullptr, nullptr, nullptr, nullptr,
                           false, stream);
}

csa2_status csa2::index_reindex_hist(const uint16_t* q_idx, int32_t B, int32_t Q, int32_t H_i, const csa2_idx_k* k,
                                     const int32_t* n_vis, const int32_t* pool_blocks, int32_t P, float* pool_scores,
                                     uint32_t* hist, TopkRowState* st, hipStream_t stream) {
    CSA2_ARG(P >= 0 && P <= (1 << 27), "index_reindex: P=%d out of range", P);
    RowMap map;
    // the pool may name any block of the sequence; the view is checked for one page at least
    csa2_status s = check_common("index_reindex", q_idx, B, Q, H_i, k, n_vis, 1, &map);
    if (s != CSA2_OK || (int64_t)B * Q == 0 || P == 0) return s;
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
    p.hist_e = hist;
    p.state_e = st;
    return launch_index(p, B * Q, k->D_i, true, stream, "index_reindex");
}

extern "C" csa2_status csa2_index_reindex(const uint16_t* q_idx, int32_t B, int32_t Q, int32_t H_i,
                                          const csa2_idx_k* k, const int32_t* n_vis, const int32_t* pool_blocks,
                                          int32_t P, float* pool_scores, hipStream_t stream) {
    clear_error();
    return index_reindex_hist(q_idx, B, Q, H_i, k, n_vis, pool_blocks, P, pool_scores, nullptr, nullptr, stream);
}
