// Top-K selection by (score descending, position ascending), as a radix select
// over a 64-bit composite key  key32(score) << 32 | ~position.  All composites
// are distinct, so "the K largest composites" is exactly the selection and the
// result does not depend on thread scheduling (aprilzz.com V4.1 Flash article,
// section "CSA2：在层的维度上共享缓存": every Full layer selects a new Top-512;
// the same routine selects the 2048 pool blocks, gkm0120.cn section 2.2.3).
//
// key32 maps fp32 to an order-preserving unsigned integer (-0 folded into +0);
// -inf marks an invalid position and maps to 0, which is never selected.
// Digits of the composite: key bits 31..21, 20..10, 9..0, then the same on
// ~position; a pass stops refining as soon as its bin holds exactly the
// number of elements still needed.
//
// Two paths:
//  * n <= 32768 (Reindex pools, short contexts, prefill rows): one 1024-thread
//    workgroup per row holds 4, 8, 16 or 32 consecutive keys per thread (the
//    fewest that cover n, so that every wave holds keys) in registers,
//    narrows the
//    selection to the keys above a sampled lower bound, runs the passes with
//    an LDS histogram over those, and writes the selection in position order
//    with one block-wide prefix sum (no sort).
//  * larger n: a per-row 2048-bin histogram of the top 11 key bits (fused into
//    the Full-mode scan, or built by its own pass), then a grid-wide pass that
//    sends positions above the threshold bin straight to the selection and
//    positions inside it to a candidate list, then one workgroup per row that
//    selects among the candidates (or, if the bin overflowed the candidate
//    buffer, among the whole row) and writes the result in position order by a
//    counting sort on the positions' top bits.
// Several independent selections (the Top-K entries and the pool blocks of a
// Full layer) run in the same launches as separate segments.
#include <atomic>
#include <mutex>

#include "select.h"

namespace csa2 {
namespace {

constexpr int PWG = 256;        // threads of the grid-wide passes
constexpr int CHUNK = 4096;     // positions per workgroup in the histogram pass (16 per thread)
constexpr int CCHUNK = 16384;   // positions per workgroup in the split pass (64 per thread): few workgroups
                                // per row keep the two per-row list counters lightly contended
constexpr int LCAP = 4096;      // candidates a split workgroup can hold in LDS
constexpr int CWG = 1024;       // threads of the split pass: 16 positions each, four waves per SIMD to
                                // hide the latency of its short dependent chains

// positions of a row that may hold a valid score
__device__ __forceinline__ int row_limit(const TopkSeg& sg, int64_t row) {
    if (sg.lim == nullptr) return sg.n;
    const int64_t l = ((int64_t)max(sg.lim[row], 0) + sg.lim_div - 1) / sg.lim_div;
    return (int)min((int64_t)sg.n, l);
}

// ---------------------------------------------------------------------------
// Small path.
//
// A lower bound T on the k-th largest key first limits the selection to few
// keys: every thread's largest key m_t is one of its elements, so if at least
// ceil(k/16) threads of each of the 16 waves have m_t >= T, at least k
// elements are >= T.  T = the smallest over the waves of the wave's
// ceil(k/16)-th largest m_t (found bit by bit with ballots).  The keys in
// [T, kmax] then go into one 2048-bin histogram of (key - T) >> shift (shift
// chosen so that the range fits); the bin holding the k-th largest is found
// by a prefix sum, and the few keys in that bin are ranked among themselves by
// their composite (key, ~position) to give the exact threshold composite.
// Every selected element is >= T, so the result is that of a full radix
// select.  If T cannot be formed (k > 1024) or the threshold bin holds more
// than 64 keys (long runs of equal scores), a radix select over all keys runs.
constexpr int TIE_CAP = 64;                 // keys of the threshold bin ranked directly

// E_SMALL keys per thread: 4, 8, 16 or 32 (n up to 4096, 8192, 16384, 32768).
template <int E_SMALL>
__global__ __launch_bounds__(WG) void topk_small_kernel(const float* __restrict__ scores, int n, int k,
                                                        const int32_t* __restrict__ pool,
                                                        int32_t* __restrict__ out, const int32_t* __restrict__ lim,
                                                        int lim_div) {
    static_assert(E_SMALL <= 32, "selection flags are one 32-bit word per thread");
    __shared__ SelectLds sh;
    __shared__ int32_t pool_s[E_SMALL * WG / 8];  // the row's pool blocks (position -> entry map)
    __shared__ uint32_t tie_key[TIE_CAP], tie_pos[TIE_CAP];
    __shared__ uint32_t wave_t[NW], wave_m[NW];
    __shared__ uint32_t counts, tie_n;
    __shared__ uint64_t cstar_s;
    __shared__ int32_t out_s[TOPK_KMAX];  // the selection in position order, copied out coalesced
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int64_t row = blockIdx.x;
    const float* s = scores + row * (int64_t)n;
    const int nblk = n / 8;
    // positions at or past nl are invalid and never read
    const int nl = lim ? (int)min((int64_t)n, ((int64_t)max(lim[row], 0) + lim_div - 1) / lim_div) : n;
    if (pool)
        for (int i = t; i < nblk; i += WG) pool_s[i] = pool[row * nblk + i];
    for (int i = t; i < NBINS1; i += WG) sh.hist[0][i] = 0u;
    if (t == 0) {
        counts = 0u;
        tie_n = 0u;
    }
    uint32_t key[E_SMALL];
    // thread t owns positions E t .. E t + E - 1 (ordered output); read them as
    // 16-byte loads when the row is 16-byte aligned (strided scalar loads
    // thrash the vector cache and cost several microseconds here)
    if ((n & 3) == 0 && (((uintptr_t)s) & 15) == 0 && (t + 1) * E_SMALL <= nl) {
        const float4* s4 = reinterpret_cast<const float4*>(s) + t * (E_SMALL / 4);
#pragma unroll
        for (int e = 0; e < E_SMALL / 4; ++e) {
            const float4 v = s4[e];
            key[4 * e] = key32(v.x);
            key[4 * e + 1] = key32(v.y);
            key[4 * e + 2] = key32(v.z);
            key[4 * e + 3] = key32(v.w);
        }
    } else {
#pragma unroll
        for (int e = 0; e < E_SMALL; ++e) {
            const int i = t * E_SMALL + e;
            key[e] = i < nl ? key32(s[i]) : 0u;
        }
    }
    // ---- the bound T, the largest key and the number of valid keys
    const int c = (k + NW - 1) / NW;
    uint32_t mt = 0u, nv = 0u;
#pragma unroll
    for (int e = 0; e < E_SMALL; ++e) {
        mt = max(mt, key[e]);
        nv += key[e] != 0u;
    }
    if (c <= 64) {
        // largest V (a multiple of 2^16) with #{lanes: mt >= V} >= c: the top
        // 16 key bits bound the selection almost as tightly as all 32, in half
        // the ballot steps
        uint32_t v = 0u;
        for (int bit = 31; bit >= 16; --bit) {
            const uint32_t cand = v | (1u << bit);
            if (__popcll(__ballot(mt >= cand)) >= (uint32_t)c) v = cand;
        }
        if (lane == 0) wave_t[wid] = v;
    }
    const uint32_t wm = wave_umax(mt);
    nv = wave_sum(nv);
    if (lane == 0) {
        wave_m[wid] = wm;
        atomicAdd(&counts, nv);
    }
    __syncthreads();  // also publishes pool_s and the zeroed histogram
    const uint32_t valid = counts;
    const bool all = valid <= (uint32_t)k;
    uint32_t T = 0u, kmax = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) kmax = max(kmax, wave_m[w]);
    if (c <= 64) {
        T = wave_t[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) T = min(T, wave_t[w]);
    }
    // (a wave without valid keys gives T = 0; then every valid key, at least
    // k + 1 of them, is >= 1)
    bool fast = !all && c <= 64;
    if (T == 0u) T = 1u;
    uint32_t sft = 0, d = 0, need = 0, mb = 0;
    uint64_t cstar = 0;
    if (fast) {
        // ---- one histogram of the keys >= T over their range
        const uint32_t span = kmax - T;
        const int bits = span ? 32 - __clz((int)span) : 0;
        sft = bits > 11 ? (uint32_t)(bits - 11) : 0u;
#pragma unroll
        for (int e = 0; e < E_SMALL; ++e)
            if (key[e] >= T) atomicAdd(&sh.hist[0][(key[e] - T) >> sft], 1u);
        __syncthreads();
        find_bin(sh.hist[0], sh, NBINS1, (uint32_t)k);
        d = sh.bin;
        need = (uint32_t)k - sh.above;
        mb = sh.hist[0][d];
        if (mb != need) {
            if (mb <= (uint32_t)TIE_CAP) {
                // rank the threshold bin's keys by composite: the need-th largest
                // is the threshold
#pragma unroll
                for (int e = 0; e < E_SMALL; ++e)
                    if (key[e] >= T && ((key[e] - T) >> sft) == d) {
                        const uint32_t at = atomicAdd(&tie_n, 1u);
                        tie_key[at] = key[e];
                        tie_pos[at] = (uint32_t)(t * E_SMALL + e);
                    }
                __syncthreads();
                if (t < (int)mb) {
                    const uint64_t me = composite(tie_key[t], tie_pos[t]);
                    uint32_t rank = 0;
                    for (uint32_t j = 0; j < mb; ++j) rank += composite(tie_key[j], tie_pos[j]) > me;
                    if (rank == need - 1u) cstar_s = me;
                }
                __syncthreads();
                cstar = cstar_s;
            } else {
                fast = false;  // (block-uniform: mb comes from LDS)
            }
        }
    }
    uint64_t prefix = 0, mask = 0;
    if (!all && !fast) {
        __syncthreads();  // the histogram is reused by the radix select
        for (int i = t; i < NBINS1; i += WG) sh.hist[0][i] = 0u;
        __syncthreads();
        uint32_t pos[E_SMALL];
#pragma unroll
        for (int e = 0; e < E_SMALL; ++e) pos[e] = (uint32_t)(t * E_SMALL + e);
        select_regs<E_SMALL>(key, pos, (uint32_t)k, 0, prefix, mask, sh);
    }
    // ---- selected positions, written in position order.  Fast path: the
    // selected composites are exactly those >= one threshold -- the ranked
    // need-th composite of bin d, or when the whole bin is taken the bin's
    // lowest key with the smallest position part (bin d's keys start at
    // T + d 2^sft, which no overflow reaches: d 2^sft <= kmax - T)
    const uint64_t cthr = (fast && mb == need) ? (uint64_t)(T + (d << sft)) << 32 : cstar;
    uint32_t fs = 0;
#pragma unroll
    for (int e = 0; e < E_SMALL; ++e) {
        bool ok;
        if (all) {
            ok = key[e] != 0u;
        } else if (fast) {
            ok = composite(key[e], (uint32_t)(t * E_SMALL + e)) >= cthr;
        } else {
            ok = key[e] != 0u && (composite(key[e], (uint32_t)(t * E_SMALL + e)) & mask) >= prefix;
        }
        fs |= (uint32_t)ok << e;
    }
    uint32_t total;
    uint32_t o = block_excl_scan((uint32_t)__popc(fs), sh, &total);
    // selected positions into LDS at their output slots, then one coalesced
    // copy (padded with -1) instead of scattered per-key stores
#pragma unroll
    for (int e = 0; e < E_SMALL; ++e) {
        if ((fs >> e) & 1u) {
            const int p = t * E_SMALL + e;
            out_s[o++] = pool ? pool_s[p >> 3] * 8 + (p & 7) : p;
        }
    }
    __syncthreads();
    for (int i = t; i < k; i += WG) out[row * (int64_t)k + i] = i < (int)total ? out_s[i] : -1;
}

// ---------------------------------------------------------------------------
// Large path.
__global__ void topk_zero_kernel(TopkSegs segs) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int sgi = 0; sgi < segs.nseg; ++sgi) {
        const TopkSeg& sg = segs.seg[sgi];
        if (i < (int64_t)segs.rows * NBINS1) sg.hist[i] = 0u;
        if (i < segs.rows) sg.state[i] = TopkRowState{0u, 0u, 0u, 0u};
    }
}

__global__ __launch_bounds__(PWG) void topk_hist_kernel(TopkSegs segs) {
    __shared__ uint32_t h[NBINS1];
    const int sgi = blockIdx.y / segs.rows;
    const int64_t row = blockIdx.y % segs.rows;
    const TopkSeg& sg = segs.seg[sgi];
    const int lim = row_limit(sg, row);
    if ((int)blockIdx.x * CHUNK >= lim) return;
    const int t = threadIdx.x;
    for (int i = t; i < NBINS1; i += PWG) h[i] = 0u;
    __syncthreads();
    const float* s = sg.scores + row * (int64_t)sg.n;
    const int lo = blockIdx.x * CHUNK;
    const int hi = min(lim, lo + CHUNK);
    uint32_t cnt = 0;
    float v[CHUNK / PWG];
#pragma unroll
    for (int e = 0; e < CHUNK / PWG; ++e) {
        const int i = lo + e * PWG + t;
        v[e] = i < hi ? s[i] : -INFINITY;
    }
#pragma unroll
    for (int e = 0; e < CHUNK / PWG; ++e) {
        const uint32_t kk = key32(v[e]);
        if (kk != 0u) {
            atomicAdd(&h[kk >> 21], 1u);
            ++cnt;
        }
    }
    cnt = wave_sum(cnt);
    if ((t & 63) == 0 && cnt) atomicAdd(&sg.state[row].valid, cnt);
    __syncthreads();
    uint32_t* gh = sg.hist + row * NBINS1;
    for (int i = t; i < NBINS1; i += PWG)
        if (h[i]) atomicAdd(&gh[i], h[i]);
}

// Threshold bin of a row from its global histogram (NT threads, NBINS1 / NT
// bins each): hv holds bins i NT + t of the histogram, read by the caller with
// coalesced loads (issued before its own loads, so the search does not wait
// behind them); they are staged in LDS first.
template <int NT>
__device__ void row_threshold(const uint32_t (&hv)[NBINS1 / NT], uint32_t need, uint32_t* lh, uint32_t* scan,
                              uint32_t* d_out, uint32_t* above_out) {
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    constexpr int per = NBINS1 / NT;
#pragma unroll
    for (int i = 0; i < per; ++i) lh[i * NT + t] = hv[i];
    __syncthreads();
    uint32_t mine[per];
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) {
        mine[i] = lh[NBINS1 - 1 - (t * per + i)];
        local += mine[i];
    }
    const uint32_t x = wave_incl_scan(local);
    if (lane == 63) scan[wid] = x;
    __syncthreads();
    uint32_t base = 0;
    for (int w = 0; w < wid; ++w) base += scan[w];
    uint32_t above = base + x - local;
#pragma unroll
    for (int i = 0; i < per; ++i) {
        if (above < need && need <= above + mine[i]) {
            *d_out = (uint32_t)(NBINS1 - 1 - (t * per + i));
            *above_out = above;
        }
        above += mine[i];
    }
    __syncthreads();
}

// Threshold split of one chunk.  Positions above the threshold bin go to the
// row's selection list, positions inside it to the candidate list; both are
// gathered in LDS first, so each list costs one global atomic per workgroup.
// VEC: every segment's rows are 16-byte aligned with n a multiple of 4 (the
// launcher checks), so scores are read as 16-byte groups without a per-thread
// branch (a branch makes the compiler wait for every load at its join).
template <bool VEC>
__global__ __launch_bounds__(CWG) void topk_compact_kernel(TopkSegs segs) {
    __shared__ uint32_t scan[CWG / 64];
    __shared__ uint32_t sh[6];
    __shared__ int l_sel[TOPK_KMAX];
    __shared__ uint32_t l_ck[LCAP], l_cp[LCAP];
    uint32_t* lh = l_ck;  // the row histogram is staged here before the candidates arrive
    const int sgi = blockIdx.y / segs.rows;
    const int64_t row = blockIdx.y % segs.rows;
    const TopkSeg& sg = segs.seg[sgi];
    const int lim = row_limit(sg, row);
    if ((int)blockIdx.x * CCHUNK >= lim) return;
    const int t = threadIdx.x;
    const int lo = blockIdx.x * CCHUNK;
    const int hi = min(lim, lo + CCHUNK);
    const float* s = sg.scores + row * (int64_t)sg.n;
    // the row's valid count and histogram first: the threshold search needs
    // them before any score (loads complete in order)
    const uint32_t valid = sg.state[row].valid;
    uint32_t hv[NBINS1 / CWG];
#pragma unroll
    for (int i = 0; i < NBINS1 / CWG; ++i) hv[i] = sg.hist[row * NBINS1 + i * CWG + t];
    // every position of this thread is loaded before any is classified: one
    // memory round trip, overlapping the threshold search; round rd covers
    // positions lo + rd*CWG*16 + (e*CWG + t)*4 + j
    constexpr int ROUNDS = CCHUNK / (CWG * 16);
    float va[ROUNDS][16];
#pragma unroll
    for (int rd = 0; rd < ROUNDS; ++rd) {
        const int base = lo + rd * CWG * 16;
        if (VEC) {
            // a group starting below n lies inside the row (n and i are
            // multiples of 4); one starting at or past n reads the row's last
            // group instead, and every position at or past hi is masked
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = base + (e * CWG + t) * 4;
                const float4 f = *reinterpret_cast<const float4*>(s + min(i, sg.n - 4));
                va[rd][4 * e] = i < hi ? f.x : -INFINITY;
                va[rd][4 * e + 1] = i + 1 < hi ? f.y : -INFINITY;
                va[rd][4 * e + 2] = i + 2 < hi ? f.z : -INFINITY;
                va[rd][4 * e + 3] = i + 3 < hi ? f.w : -INFINITY;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = base + (e * CWG + t) * 4;  // 4 consecutive positions
#pragma unroll
                for (int j = 0; j < 4; ++j) va[rd][4 * e + j] = (i + j < hi) ? s[i + j] : -INFINITY;
            }
        }
    }
    // keep the loads here, ahead of the threshold search (a compiler barrier,
    // not a wait: the values are awaited where they are first used)
    asm volatile("" ::: "memory");
    if (t < 2) sh[2 + t] = 0u;
    const bool all = valid <= (uint32_t)sg.k;
    uint32_t d = 0;
    if (!all) {
        row_threshold<CWG>(hv, (uint32_t)sg.k, lh, scan, &sh[0], &sh[1]);
        d = sh[0];
        if (blockIdx.x == 0 && t == 0) sg.state[row].digit = d;
    }
    __syncthreads();  // sh[2..3] initialised; lh free for candidates
#pragma unroll
    for (int rd = 0; rd < ROUNDS; ++rd) {
        const float* v = va[rd];
        const int base = lo + rd * CWG * 16;
        // classify, then one packed LDS atomic per wave reserves the slots
        // (selected count in the low half, candidates in the high half: each
        // is at most CCHUNK = 16384 per workgroup)
        uint32_t kk[16];
        uint32_t fsel = 0, fcand = 0;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            kk[e] = key32(v[e]);
            const uint32_t dig = kk[e] >> 21;
            const bool ok = kk[e] != 0u;
            fsel |= (uint32_t)(ok && (all || dig > d)) << e;
            fcand |= (uint32_t)(ok && !all && dig == d) << e;
        }
        const uint32_t mine = (uint32_t)__popc(fsel) | ((uint32_t)__popc(fcand) << 16);
        // (each half sums to at most 64 x 16: no carry into the other)
        const uint32_t incl = wave_incl_scan(mine);
        uint32_t wbase = 0;
        if ((t & 63) == 63) wbase = atomicAdd(&sh[2], incl);
        wbase = (uint32_t)__builtin_amdgcn_readlane((int)wbase, 63);
        uint32_t at_s = (wbase & 0xFFFFu) + ((incl - mine) & 0xFFFFu);
        uint32_t at_c = (wbase >> 16) + ((incl - mine) >> 16);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int i = base + ((e >> 2) * CWG + t) * 4 + (e & 3);
            if ((fsel >> e) & 1u) l_sel[at_s++] = i;
            if ((fcand >> e) & 1u) {
                if (at_c < (uint32_t)LCAP) {
                    l_ck[at_c] = kk[e];
                    l_cp[at_c] = (uint32_t)i;
                }
                ++at_c;
            }
        }
    }
    __syncthreads();
    const uint32_t ns = sh[2] & 0xFFFFu, nc = sh[2] >> 16;
    if (t == 0) {
        // a local overflow pushes the row's count past the capacity: the finish
        // pass then selects from the whole row instead of the candidate list
        const uint32_t add = nc > (uint32_t)LCAP ? (uint32_t)TOPK_CAP + 1u : nc;
        // both lists reserved by one 64-bit atomic (n_sel low, n_cand high): the
        // row's workgroups queue on one counter once, not twice.  Neither half
        // carries into the other: n_sel stays <= k, n_cand below
        // (n / CCHUNK + 1) (TOPK_CAP + 1) < 2^32
        uint64_t both = 0;
        if (ns | add)
            both = atomicAdd(reinterpret_cast<unsigned long long*>(&sg.state[row].n_sel),
                             ((unsigned long long)add << 32) | ns);
        sh[4] = (uint32_t)both;
        sh[5] = (uint32_t)(both >> 32);
    }
    __syncthreads();
    int* sel = sg.sel + row * TOPK_KMAX + sh[4];
    for (uint32_t j = t; j < ns; j += CWG) sel[j] = l_sel[j];
    const uint32_t cb = sh[5];
    uint32_t* ck = sg.ckey + row * TOPK_CAP;
    uint32_t* cp = sg.cpos + row * TOPK_CAP;
    for (uint32_t j = t; j < nc && j < (uint32_t)LCAP && cb + j < (uint32_t)TOPK_CAP; j += CWG) {
        ck[cb + j] = l_ck[j];
        cp[cb + j] = l_cp[j];
    }
}

constexpr int E_CAND = TOPK_CAP / WG;  // candidates per thread in the finish kernel (8)

__global__ __launch_bounds__(WG) void topk_finish_kernel(TopkSegs segs) {
    __shared__ SelectLds sh;
    __shared__ int sel[TOPK_KMAX];
    __shared__ int tmp[TOPK_KMAX];
    const int sgi = blockIdx.x / segs.rows;
    const int64_t row = blockIdx.x % segs.rows;
    const TopkSeg& sg = segs.seg[sgi];
    const int t = threadIdx.x;
    const TopkRowState st = sg.state[row];
    const bool all = st.valid <= (uint32_t)sg.k;
    const bool from_list = !all && st.n_cand <= (uint32_t)TOPK_CAP;
    // the selected list and the candidates are loaded together, before any
    // wait: unconditional loads at clamped (in-bounds) indices, masked after,
    // so that no branch makes the compiler wait for one before issuing the other
    int selv[TOPK_KMAX / WG];
#pragma unroll
    for (int j = 0; j < TOPK_KMAX / WG; ++j) selv[j] = sg.sel[row * TOPK_KMAX + t + j * WG];
    uint32_t key[E_CAND], pos[E_CAND];
#pragma unroll
    for (int e = 0; e < E_CAND; ++e) {
        key[e] = sg.ckey[row * TOPK_CAP + e * WG + t];
        pos[e] = sg.cpos[row * TOPK_CAP + e * WG + t];
    }
#pragma unroll
    for (int j = 0; j < TOPK_KMAX / WG; ++j) {
        const int i = t + j * WG;
        sel[i] = i < (int)st.n_sel ? selv[j] : 0x7FFFFFFF;
    }
    for (int i = t; i < NBINS1; i += WG) sh.hist[1][i] = 0u;
    if (t == 0) sh.nsel = st.n_sel;
    __syncthreads();
    if (!all) {
        const uint32_t need = (uint32_t)sg.k - st.n_sel;
        uint64_t prefix = (uint64_t)st.digit << 53;
        uint64_t mask = (uint64_t)0x7FF << 53;
        if (from_list) {
#pragma unroll
            for (int e = 0; e < E_CAND; ++e) {
                const bool in = e * WG + t < (int)st.n_cand;
                key[e] = in ? key[e] : 0u;
                pos[e] = in ? pos[e] : 0u;
            }
            select_regs<E_CAND>(key, pos, need, 1, prefix, mask, sh);
#pragma unroll
            for (int e = 0; e < E_CAND; ++e)
                if (key[e] != 0u && (composite(key[e], pos[e]) & mask) >= prefix)
                    sel[atomicAdd(&sh.nsel, 1u)] = (int)pos[e];
            __syncthreads();
        } else {
            select_global_row(sg.scores + row * (int64_t)sg.n, row_limit(sg, row), need, prefix, mask, sh, sel);
        }
    }
    const uint32_t total = all ? st.valid : (uint32_t)sg.k;
    emit_sorted(sel, (int)total, sg.n, sg.k, sh, tmp, sg.out, sg.pool, row);
    // leave the row's histogram and state cleared for the next selection
    for (int i = t; i < NBINS1; i += WG) sg.hist[row * NBINS1 + i] = 0u;
    if (t == 0) sg.state[row] = TopkRowState{0u, 0u, 0u, 0u};
}

}  // namespace

size_t topk_counter_bytes(int64_t rows) {
    return ((size_t)rows * (NBINS1 * 4 + sizeof(TopkRowState)) + 15) & ~(size_t)15;
}
size_t topk_list_bytes(int64_t rows) { return (size_t)rows * (TOPK_KMAX * 4 + TOPK_CAP * 8); }
size_t topk_large_ws_bytes(int64_t rows) { return topk_counter_bytes(rows) + topk_list_bytes(rows) + 256; }

void topk_carve(void* counters, void* lists, int64_t rows, TopkSeg* sg) {
    char* c = static_cast<char*>(counters);
    sg->hist = reinterpret_cast<uint32_t*>(c);
    sg->state = reinterpret_cast<TopkRowState*>(c + (size_t)rows * NBINS1 * 4);
    char* w = static_cast<char*>(lists);
    sg->sel = reinterpret_cast<int*>(w);
    w += (size_t)rows * TOPK_KMAX * 4;
    sg->ckey = reinterpret_cast<uint32_t*>(w);
    w += (size_t)rows * TOPK_CAP * 4;
    sg->cpos = reinterpret_cast<uint32_t*>(w);
}

void topk_launch_zero(const TopkSegs& segs, hipStream_t stream) {
    const int64_t nz = (int64_t)segs.rows * NBINS1;
    topk_zero_kernel<<<(unsigned)((nz + 255) / 256), 256, 0, stream>>>(segs);
}

void topk_launch_hist(const TopkSegs& segs, hipStream_t stream) {
    int chunks = 0;
    for (int i = 0; i < segs.nseg; ++i) chunks = max(chunks, (segs.seg[i].n + CHUNK - 1) / CHUNK);
    topk_hist_kernel<<<dim3((unsigned)chunks, (unsigned)(segs.rows * segs.nseg)), PWG, 0, stream>>>(segs);
}

void topk_launch_select(const TopkSegs& segs, hipStream_t stream) {
    int chunks = 0;
    for (int i = 0; i < segs.nseg; ++i) chunks = max(chunks, (segs.seg[i].n + CCHUNK - 1) / CCHUNK);
    bool vec = true;
    for (int i = 0; i < segs.nseg; ++i)
        vec = vec && segs.seg[i].n >= 4 && (segs.seg[i].n & 3) == 0 && (((uintptr_t)segs.seg[i].scores) & 15) == 0;
    const dim3 grid((unsigned)chunks, (unsigned)(segs.rows * segs.nseg));
    if (vec)
        topk_compact_kernel<true><<<grid, CWG, 0, stream>>>(segs);
    else
        topk_compact_kernel<false><<<grid, CWG, 0, stream>>>(segs);
    topk_finish_kernel<<<(unsigned)(segs.rows * segs.nseg), WG, 0, stream>>>(segs);
}

void topk_launch_small(const float* scores, int rows, int n, int k, const int32_t* pool, int32_t* out,
                       hipStream_t stream, const int32_t* lim, int lim_div) {
    // short rows take fewer keys per thread so that every wave holds keys: a
    // wave without any gives the sampled bound T no strength (T = 1), and the
    // selection then falls back to the radix passes
    if (n <= TOPK_SMALL_N / 4)
        topk_small_kernel<TOPK_SMALL_N / 4 / WG><<<rows, WG, 0, stream>>>(scores, n, k, pool, out, lim, lim_div);
    else if (n <= TOPK_SMALL_N / 2)
        topk_small_kernel<TOPK_SMALL_N / 2 / WG><<<rows, WG, 0, stream>>>(scores, n, k, pool, out, lim, lim_div);
    else if (n <= TOPK_SMALL_N)
        topk_small_kernel<TOPK_SMALL_N / WG><<<rows, WG, 0, stream>>>(scores, n, k, pool, out, lim, lim_div);
    else
        topk_small_kernel<TOPK_ONEWG_N / WG><<<rows, WG, 0, stream>>>(scores, n, k, pool, out, lim, lim_div);
}

__global__ void zero_ranges_kernel(ZeroRanges z) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int r = 0; r < z.n; ++r)
        if (i < z.count[r]) z.ptr[r][i] = 0u;
}

void launch_zero_ranges(const ZeroRanges& z, hipStream_t stream) {
    int64_t mx = 0;
    for (int r = 0; r < z.n; ++r) mx = max(mx, z.count[r]);
    if (mx == 0) return;
    zero_ranges_kernel<<<(unsigned)((mx + 255) / 256), 256, 0, stream>>>(z);
}

// ---------------------------------------------------------------------------
// Allocation-free Top-K: the large path's workspace is a file-scope device
// array, one per GPU, holding the counters and lists of up to
// TOPK_NOALLOC_MAX_ROWS rows.  Host code reaches it only through the address
// hipGetSymbolAddress returns for the current device (the array's name in host
// code is not a device address).
constexpr int TOPK_NOALLOC_MAX_ROWS = 64;
constexpr size_t TOPK_NOALLOC_COUNTERS =
    ((size_t)TOPK_NOALLOC_MAX_ROWS * (NBINS1 * 4 + sizeof(TopkRowState)) + 255) & ~(size_t)255;
constexpr size_t TOPK_NOALLOC_BYTES =
    TOPK_NOALLOC_COUNTERS + (size_t)TOPK_NOALLOC_MAX_ROWS * (TOPK_KMAX * 4 + TOPK_CAP * 8);

static __device__ __align__(256) uint8_t scratch[TOPK_NOALLOC_BYTES];

constexpr int NOALLOC_MAX_DEVICES = 64;
static std::atomic<void*> g_scratch_ptr[NOALLOC_MAX_DEVICES];
static std::mutex g_scratch_mu;

// Device address of the current device's scratch array (resolved once per device).
static csa2_status scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    CSA2_REQUIRE(e == hipSuccess, CSA2_EHIP, "topk_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    CSA2_REQUIRE(dev >= 0 && dev < NOALLOC_MAX_DEVICES, CSA2_EUNSUPPORTED, "topk_noalloc: device %d out of range",
                 dev);
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            CSA2_REQUIRE(e == hipSuccess && p != nullptr, CSA2_EHIP, "topk_noalloc: hipGetSymbolAddress: %s",
                         hipGetErrorString(e));
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return CSA2_OK;
}

}  // namespace csa2

using namespace csa2;

extern "C" size_t csa2_topk_workspace_size(int32_t rows, int32_t n, int32_t k) {
    (void)k;
    if (rows <= 0 || n <= TOPK_ONEWG_N) return 0;
    return topk_large_ws_bytes(rows);
}

extern "C" csa2_status csa2_topk(const float* scores, int32_t rows, int32_t n, int32_t k,
                                 const int32_t* pool_blocks, int32_t* out_idx, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
    clear_error();
    CSA2_ARG(rows >= 0 && n >= 0, "topk: rows=%d n=%d must be >= 0", rows, n);
    CSA2_ARG(k >= 1 && k <= TOPK_KMAX, "topk: k=%d must be in [1, %d]", k, TOPK_KMAX);
    CSA2_ARG(pool_blocks == nullptr || n % 8 == 0, "topk: with a pool map n=%d must be a multiple of 8", n);
    CSA2_ARG(rows <= 65535, "topk: rows=%d exceeds 65535", rows);
    if (rows == 0) return CSA2_OK;
    CSA2_ARG(out_idx != nullptr, "topk: null out_idx");
    CSA2_ARG(n == 0 || scores != nullptr, "topk: null scores");
    if (n <= TOPK_ONEWG_N) {
        topk_launch_small(scores, rows, n, k, pool_blocks, out_idx, stream);
        return launch_status("topk");
    }
    const size_t need = topk_large_ws_bytes(rows);
    CSA2_REQUIRE(ws != nullptr && ws_bytes >= need, CSA2_EWORKSPACE,
                 "topk: workspace of %zu bytes required, %zu given", need, ws ? ws_bytes : (size_t)0);
    CSA2_ARG(aligned(ws, 16), "topk: workspace must be 16-byte aligned");
    TopkSegs segs{};
    segs.nseg = 1;
    segs.rows = rows;
    TopkSeg& sg = segs.seg[0];
    sg.scores = scores;
    sg.n = n;
    sg.k = k;
    sg.pool = pool_blocks;
    sg.out = out_idx;
    topk_carve(ws, static_cast<char*>(ws) + topk_counter_bytes(rows), rows, &sg);
    topk_launch_zero(segs, stream);
    topk_launch_hist(segs, stream);
    topk_launch_select(segs, stream);
    return launch_status("topk");
}

extern "C" csa2_status csa2_topk_noalloc(const float* scores, int32_t rows, int32_t n, int32_t k,
                                         const int32_t* pool_blocks, int32_t* out_idx, hipStream_t stream) {
    clear_error();
    CSA2_ARG(rows >= 0 && n >= 0, "topk_noalloc: rows=%d n=%d must be >= 0", rows, n);
    CSA2_ARG(k >= 1 && k <= TOPK_KMAX, "topk_noalloc: k=%d must be in [1, %d]", k, TOPK_KMAX);
    CSA2_ARG(pool_blocks == nullptr || n % 8 == 0, "topk_noalloc: with a pool map n=%d must be a multiple of 8", n);
    CSA2_ARG(rows <= 65535, "topk_noalloc: rows=%d exceeds 65535", rows);
    if (rows == 0) return CSA2_OK;
    CSA2_ARG(out_idx != nullptr, "topk_noalloc: null out_idx");
    CSA2_ARG(n == 0 || scores != nullptr, "topk_noalloc: null scores");
    if (n <= TOPK_ONEWG_N) {  // one workgroup per row: no scratch at all
        topk_launch_small(scores, rows, n, k, pool_blocks, out_idx, stream);
        return launch_status("topk_noalloc");
    }
    CSA2_REQUIRE(rows <= TOPK_NOALLOC_MAX_ROWS, CSA2_EUNSUPPORTED,
                 "topk_noalloc: rows=%d exceeds the %d rows its built-in scratch holds for n > %d "
                 "(use csa2_topk with a workspace)",
                 rows, TOPK_NOALLOC_MAX_ROWS, TOPK_ONEWG_N);
    void* base = nullptr;
    const csa2_status st = scratch_address(&base);
    if (st != CSA2_OK) return st;
    TopkSegs segs{};
    segs.nseg = 1;
    segs.rows = rows;
    TopkSeg& sg = segs.seg[0];
    sg.scores = scores;
    sg.n = n;
    sg.k = k;
    sg.pool = pool_blocks;
    sg.out = out_idx;
    topk_carve(base, static_cast<char*>(base) + TOPK_NOALLOC_COUNTERS, rows, &sg);
    // the counters must start at zero; the previous call on this GPU left
    // them cleared, but a failed or interrupted one may not have
    topk_launch_zero(segs, stream);
    topk_launch_hist(segs, stream);
    topk_launch_select(segs, stream);
    return launch_status("topk_noalloc");
}
