// Block-wide selection helpers shared by the Top-K kernels and the screened
// multi-query selection: a 1024-thread workgroup, a radix select over
// register-resident composite keys key32(score) << 32 | ~position, and the
// position-ordered output of a selection.
#pragma once
#include "internal.h"

namespace csa2 {
namespace {

constexpr int WG = 1024;     // single-row workgroup
constexpr int NW = WG / 64;  // its wavefronts

__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t pos) {
    return ((uint64_t)key << 32) | (uint64_t)(~pos);
}

// ---------------------------------------------------------------------------
// Block-wide helpers for a 1024-thread workgroup.
struct SelectLds {
    uint32_t hist[2][NBINS1];  // double-buffered: a pass zeroes the buffer of the pass after next
    uint32_t wsum[NW];
    uint32_t bin, above, total, nsel;
};

// Exclusive prefix sum over the threads of the block; *total gets the sum.
__device__ uint32_t block_excl_scan(uint32_t v, SelectLds& sh, uint32_t* total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const uint32_t x = wave_incl_scan(v);
    if (lane == 63) sh.wsum[wid] = x;
    __syncthreads();
    uint32_t base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint32_t ws = sh.wsum[w];
        base += (w < wid) ? ws : 0u;
        tot += ws;
    }
    *total = tot;
    __syncthreads();  // wsum may be rewritten by the next call
    return base + x - v;
}

// The bin d of hist[0..nb) with  above < need <= above + hist[d]  (above =
// sum of the bins above d): written to sh.bin / sh.above.  Two barriers.
__device__ void find_bin(const uint32_t* hist, SelectLds& sh, int nb, uint32_t need) {
    const int per = (nb + WG - 1) / WG;  // bins per thread, thread 0 owns the top bins
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    uint32_t local = 0;
    for (int i = 0; i < per; ++i) {
        const int bin = nb - 1 - (t * per + i);
        if (bin >= 0) local += hist[bin];
    }
    const uint32_t x = wave_incl_scan(local);
    if (lane == 63) sh.wsum[wid] = x;
    __syncthreads();
    uint32_t above = x - local;
#pragma unroll
    for (int w = 0; w < NW; ++w) above += (w < wid) ? sh.wsum[w] : 0u;
    for (int i = 0; i < per; ++i) {
        const int bin = nb - 1 - (t * per + i);
        if (bin < 0) break;
        const uint32_t h = hist[bin];
        if (above < need && need <= above + h) {
            sh.bin = (uint32_t)bin;
            sh.above = above;
        }
        above += h;
    }
    __syncthreads();
}

// Radix select over register-resident elements (key 0 = not in the set).
// On return, element (key, pos) is selected iff key != 0 and
// (composite & mask) >= prefix; exactly `need` elements qualify.
// Requires sh.hist[first_pass & 1] zeroed on entry; leaves both buffers zeroed.
template <int E, typename PosOf>
__device__ void select_regs_by(const uint32_t (&key)[E], PosOf pos_of, uint32_t need, int first_pass,
                            uint64_t& prefix, uint64_t& mask, SelectLds& sh) {
    const int shifts[6] = {53, 42, 32, 21, 10, 0};
    const int widths[6] = {11, 11, 10, 11, 11, 10};
    // the other buffer is zeroed while this pass counts
    for (int i = threadIdx.x; i < NBINS1; i += WG) sh.hist[(first_pass + 1) & 1][i] = 0u;
    for (int pass = first_pass; pass < 6; ++pass) {
        uint32_t* h = sh.hist[pass & 1];
        const int sh_ = shifts[pass], nb = 1 << widths[pass];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if (key[e] == 0u) continue;
            const uint64_t c = composite(key[e], pos_of(e));
            if ((c & mask) == prefix) atomicAdd(&h[(uint32_t)(c >> sh_) & (uint32_t)(nb - 1)], 1u);
        }
        __syncthreads();
        find_bin(h, sh, nb, need);
        const uint32_t d = sh.bin;
        need -= sh.above;
        prefix |= (uint64_t)d << sh_;
        mask |= (uint64_t)(nb - 1) << sh_;
        const bool done = h[d] == need;
        // every thread has read h[d] (after find_bin's last barrier read): clear
        // this buffer for the pass after next; the barrier inside the next
        // pass's find_bin orders it before that pass's atomics
        __syncthreads();
        for (int i = threadIdx.x; i < NBINS1; i += WG) h[i] = 0u;
        if (done) break;
    }
    __syncthreads();
}

// (positions in a register array)
template <int E>
__device__ void select_regs(const uint32_t (&key)[E], const uint32_t (&pos)[E], uint32_t need, int first_pass,
                            uint64_t& prefix, uint64_t& mask, SelectLds& sh) {
    select_regs_by<E>(key, [&](int e) { return pos[e]; }, need, first_pass, prefix, mask, sh);
}

__device__ __forceinline__ int32_t map_pos(int p, const int32_t* pool, int64_t row, int nblk) {
    return pool ? pool[row * nblk + (p >> 3)] * 8 + (p & 7) : p;
}

// Write the distinct positions sel[0..total) (each < n) to out[0..total) in
// ascending order, and -1 to out[total..k): a counting sort on the top 11 bits
// of the position, then each position's rank among the few in its bin.
__device__ void emit_sorted(const int* sel, int total, int n, int k, SelectLds& sh, int* tmp, int32_t* out,
                            const int32_t* pool, int64_t row) {
    const int t = threadIdx.x;
    int bits = 0;
    while (bits < 31 && (1 << bits) < n) ++bits;
    const int shift = bits > 11 ? bits - 11 : 0;
    uint32_t* cnt = sh.hist[0];
    uint32_t* start = sh.hist[1];
    for (int i = t; i < NBINS1; i += WG) cnt[i] = 0u;
    __syncthreads();
    int x[2];
    uint32_t slot[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int i = t + j * WG;
        x[j] = i < total ? sel[i] : 0;
        slot[j] = i < total ? atomicAdd(&cnt[x[j] >> shift], 1u) : 0u;
    }
    __syncthreads();
    const uint32_t c0 = cnt[2 * t], c1 = cnt[2 * t + 1];
    uint32_t tot;
    const uint32_t b0 = block_excl_scan(c0 + c1, sh, &tot);
    start[2 * t] = b0;
    start[2 * t + 1] = b0 + c0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j)
        if (t + j * WG < total) tmp[start[x[j] >> shift] + slot[j]] = x[j];
    __syncthreads();
    const int nblk = n / 8;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        if (t + j * WG >= total) continue;
        const uint32_t bn = (uint32_t)x[j] >> shift;
        const uint32_t s0 = start[bn], c = cnt[bn];
        uint32_t r = 0;
        for (uint32_t q = 0; q < c; ++q) r += tmp[s0 + q] < x[j];
        out[row * (int64_t)k + s0 + r] = map_pos(x[j], pool, row, nblk);
    }
    for (int i = total + t; i < k; i += WG) out[row * (int64_t)k + i] = -1;
}

// Slow general radix select over a row in global memory, restricted to the
// elements matching prefix/mask (used only when a threshold bin overflows the
// candidate buffer, e.g. long runs of equal scores).  Appends exactly `need`
// elements of that subset to sel[]: the positions above the subset (already in
// sel[]) are excluded from the final gather as well as from the passes.
__device__ void select_global_row(const float* s, int n, uint32_t need, uint64_t prefix, uint64_t mask,
                                  SelectLds& sh, int* sel) {
    const int shifts[6] = {53, 42, 32, 21, 10, 0};
    const int widths[6] = {11, 11, 10, 11, 11, 10};
    const uint64_t sub_prefix = prefix, sub_mask = mask;
    int pass = 0;
    while (pass < 6 && ((mask >> shifts[pass]) & 1u)) ++pass;  // skip decided digits
    uint32_t* h = sh.hist[0];
    for (; pass < 6; ++pass) {
        const int sh_ = shifts[pass], nb = 1 << widths[pass];
        for (int i = threadIdx.x; i < nb; i += WG) h[i] = 0u;
        __syncthreads();
        for (int i = threadIdx.x; i < n; i += WG) {
            const uint32_t k = key32(s[i]);
            if (k == 0u) continue;
            const uint64_t c = composite(k, (uint32_t)i);
            if ((c & mask) == prefix) atomicAdd(&h[(uint32_t)(c >> sh_) & (uint32_t)(nb - 1)], 1u);
        }
        __syncthreads();
        find_bin(h, sh, nb, need);
        const uint32_t d = sh.bin;
        need -= sh.above;
        prefix |= (uint64_t)d << sh_;
        mask |= (uint64_t)(nb - 1) << sh_;
        const bool done = h[d] == need;
        __syncthreads();
        if (done) break;
    }
    for (int i = threadIdx.x; i < n; i += WG) {
        const uint32_t k = key32(s[i]);
        if (k == 0u) continue;
        const uint64_t c = composite(k, (uint32_t)i);
        if ((c & sub_mask) == sub_prefix && (c & mask) >= prefix) sel[atomicAdd(&sh.nsel, 1u)] = i;
    }
    __syncthreads();
}

}  // namespace
}  // namespace csa2
