// Top-K selection by (score descending, position ascending), as a radix select
// over a 64-bit composite key  key32(score) << 32 | ~position.  All composites
// are distinct, so "the K largest composites" is exactly the selection and the
// result is independent of thread scheduling (aprilzz.com V4.1 Flash article,
// section "CSA2：在层的维度上共享缓存": every Full layer selects a new Top-512;
// the same routine selects the 2048 pool blocks, gkm0120.cn section 2.2.3).
//
// key32 maps fp32 to an order-preserving unsigned integer (-0 folded into +0);
// -inf marks an invalid position and maps to 0, which is never selected.
//
// Two paths:
//  * n <= 16384 (Reindex pools, short contexts): one 1024-thread workgroup per
//    row caches the row's keys in LDS and runs the whole radix select there.
//  * larger n: (1) zero the per-row state, (2) many workgroups per row build a
//    4096-bin histogram of the top 12 key bits, (3) the same grid splits the
//    row: positions above the threshold bin go straight to the selection,
//    positions inside it to a candidate list, (4) one workgroup per row
//    finishes the select on the candidates (or, if the bin overflows the
//    candidate buffer, on the whole row) and writes the sorted result.
#include "common.h"

namespace csa2 {
namespace {

constexpr int NBINS = 4096;     // widest digit: 12 bits
constexpr int WG = 1024;        // single-row workgroup
constexpr int KMAX = 2048;
constexpr int SMALL_N = 16384;  // rows cached in LDS
constexpr int CAP = 8192;       // candidate capacity per row
constexpr int CHUNK = 16384;    // positions per workgroup in the multi-workgroup passes
constexpr int PWG = 256;        // threads of the multi-workgroup passes

struct RowState {
    uint32_t valid;   // number of valid positions
    uint32_t n_sel;   // positions definitely selected (above the threshold bin)
    uint32_t n_cand;  // positions in the threshold bin
    uint32_t digit;   // threshold bin (top 12 bits)
};

__device__ __forceinline__ uint32_t key32(float s) {
    if (s == -INFINITY) return 0u;
    uint32_t u = __float_as_uint(s + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// Workgroup helpers (blockDim.x == WG)

// Finds the bin d (of nb) such that  above < need <= above + hist[d],  where
// above = sum of the bins above d.  Result in *d_out / *above_out (LDS).
__device__ void find_bin(const uint32_t* hist, int nb, uint32_t need, uint32_t* scan, uint32_t* d_out,
                         uint32_t* above_out) {
    const int t = threadIdx.x, nt = blockDim.x;
    const int per = nb / nt;  // bins per thread, descending bins: thread 0 owns the top
    uint32_t local = 0;
    for (int i = 0; i < per; ++i) local += hist[nb - 1 - (t * per + i)];
    scan[t] = local;
    __syncthreads();
    // inclusive Hillis-Steele scan over threads
    for (int off = 1; off < nt; off <<= 1) {
        uint32_t v = (t >= off) ? scan[t - off] : 0u;
        __syncthreads();
        scan[t] += v;
        __syncthreads();
    }
    uint32_t above = scan[t] - local;
    for (int i = 0; i < per; ++i) {
        const int bin = nb - 1 - (t * per + i);
        const uint32_t h = hist[bin];
        if (above < need && need <= above + h) {
            *d_out = (uint32_t)bin;
            *above_out = above;
        }
        above += h;
    }
    __syncthreads();
}

__device__ __forceinline__ void append_lds(int* list, uint32_t* count, int value) {
    uint32_t at = atomicAdd(count, 1u);
    list[at] = value;
}

// Source of (key, position) pairs for select_rows.
struct LdsKeys {  // keys cached in LDS, position = index
    const uint32_t* keys;
    int n;
    __device__ uint32_t key(int i) const { return keys[i]; }
    __device__ uint32_t pos(int i) const { return (uint32_t)i; }
};
struct LdsCands {  // candidate (key, position) pairs in LDS
    const uint32_t* keys;
    const uint32_t* pos_;
    int n;
    __device__ uint32_t key(int i) const { return keys[i]; }
    __device__ uint32_t pos(int i) const { return pos_[i]; }
};
struct GlobalRow {  // a whole row of scores in global memory
    const float* s;
    int n;
    __device__ uint32_t key(int i) const { return key32(s[i]); }
    __device__ uint32_t pos(int i) const { return (uint32_t)i; }
};

// Radix select of the `need` largest composites among the elements of src
// whose composite matches `prefix` on the bits of `mask` (need >= 1 and at
// most that many elements).  Digits: key bits 31..20, 19..10, 9..0, then the
// same on ~position.  Selected positions are appended to sel[] via *n_sel.
template <class Src>
__device__ void radix_select(const Src& src, uint32_t need, int first_pass, uint64_t prefix, uint64_t mask,
                             uint32_t* hist, uint32_t* scan, uint32_t* shared2, int* sel, uint32_t* n_sel) {
    const int t = threadIdx.x, nt = blockDim.x;
    const int shifts[6] = {52, 42, 32, 20, 10, 0};
    const int widths[6] = {12, 10, 10, 12, 10, 10};
    for (int pass = first_pass; pass < 6; ++pass) {
        const int sh = shifts[pass], wd = widths[pass], nb = 1 << wd;
        for (int i = t; i < nb; i += nt) hist[i] = 0u;
        __syncthreads();
        for (int i = t; i < src.n; i += nt) {
            const uint32_t k = src.key(i);
            if (k == 0u) continue;
            const uint64_t c = ((uint64_t)k << 32) | (uint64_t)(~src.pos(i));
            if ((c & mask) == prefix) atomicAdd(&hist[(uint32_t)(c >> sh) & (uint32_t)(nb - 1)], 1u);
        }
        __syncthreads();
        find_bin(hist, nb, need, scan, &shared2[0], &shared2[1]);
        const uint32_t d = shared2[0], above = shared2[1];
        need -= above;
        prefix |= (uint64_t)d << sh;
        mask |= (uint64_t)(nb - 1) << sh;
        const bool done = (hist[d] == need);
        __syncthreads();
        if (done) break;
    }
    // selected <=> composite restricted to the decided bits >= prefix
    for (int i = t; i < src.n; i += nt) {
        const uint32_t k = src.key(i);
        if (k == 0u) continue;
        const uint64_t c = ((uint64_t)k << 32) | (uint64_t)(~src.pos(i));
        if ((c & mask) >= prefix) append_lds(sel, n_sel, (int)src.pos(i));
    }
    __syncthreads();
}

// Bitonic sort of sel[0..KMAX) ascending (unused slots hold INT32_MAX).
__device__ void sort_sel(int* sel) {
    const int t = threadIdx.x;
    for (int size = 2; size <= KMAX; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = t; i < KMAX / 2; i += blockDim.x) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const bool up = ((lo & size) == 0);
                const int a = sel[lo], c = sel[hi];
                if ((a > c) == up) {
                    sel[lo] = c;
                    sel[hi] = a;
                }
            }
            __syncthreads();
        }
    }
}

__device__ void write_out(const int* sel, uint32_t total, int k, const int32_t* pool, int64_t row, int nblk,
                          int32_t* out) {
    for (int i = threadIdx.x; i < k; i += blockDim.x) {
        int v = -1;
        if ((uint32_t)i < total) {
            const int p = sel[i];
            v = pool ? pool[row * nblk + (p >> 3)] * 8 + (p & 7) : p;
        }
        out[row * (int64_t)k + i] = v;
    }
}

// ---------------------------------------------------------------------------
// Small path: one workgroup per row, keys cached in LDS.
__global__ __launch_bounds__(WG) void topk_small_kernel(const float* __restrict__ scores, int n, int k,
                                                        const int32_t* __restrict__ pool,
                                                        int32_t* __restrict__ out) {
    __shared__ uint32_t keys[SMALL_N];
    __shared__ uint32_t hist[NBINS];
    __shared__ uint32_t scan[WG];
    __shared__ int sel[KMAX];
    __shared__ uint32_t sh[4];
    const int t = threadIdx.x;
    const int64_t row = blockIdx.x;
    const float* s = scores + row * (int64_t)n;
    if (t == 0) {
        sh[2] = 0u;  // valid count
        sh[3] = 0u;  // n_sel
    }
    for (int i = t; i < KMAX; i += WG) sel[i] = 0x7FFFFFFF;
    __syncthreads();
    uint32_t cnt = 0;
    for (int i = t; i < n; i += WG) {
        const uint32_t kk = key32(s[i]);
        keys[i] = kk;
        cnt += (kk != 0u);
    }
    atomicAdd(&sh[2], cnt);
    __syncthreads();
    const uint32_t valid = sh[2];
    if (valid <= (uint32_t)k) {
        for (int i = t; i < n; i += WG)
            if (keys[i] != 0u) append_lds(sel, &sh[3], i);
        __syncthreads();
    } else {
        LdsKeys src{keys, n};
        radix_select(src, (uint32_t)k, 0, 0ull, 0ull, hist, scan, sh, sel, &sh[3]);
    }
    const uint32_t total = valid < (uint32_t)k ? valid : (uint32_t)k;
    sort_sel(sel);
    write_out(sel, total, k, pool, row, n / 8, out);
}

// ---------------------------------------------------------------------------
// Large path.
__global__ void topk_zero_kernel(uint32_t* __restrict__ hist, RowState* __restrict__ state, int rows) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < (int64_t)rows * NBINS) hist[i] = 0u;
    if (i < rows) state[i] = RowState{0u, 0u, 0u, 0u};
}

__global__ __launch_bounds__(PWG) void topk_hist_kernel(const float* __restrict__ scores, int n,
                                                       uint32_t* __restrict__ ghist, RowState* __restrict__ state) {
    __shared__ uint32_t h[NBINS];
    const int t = threadIdx.x;
    const int64_t row = blockIdx.y;
    for (int i = t; i < NBINS; i += PWG) h[i] = 0u;
    __syncthreads();
    const float* s = scores + row * (int64_t)n;
    const int lo = blockIdx.x * CHUNK;
    const int hi = min(n, lo + CHUNK);
    uint32_t cnt = 0;
    for (int i = lo + t; i < hi; i += PWG) {
        const uint32_t kk = key32(s[i]);
        if (kk != 0u) {
            atomicAdd(&h[kk >> 20], 1u);
            ++cnt;
        }
    }
    // wave reduce the valid count, one atomic per wave
    for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
    if ((t & 63) == 0 && cnt) atomicAdd(&state[row].valid, cnt);
    __syncthreads();
    uint32_t* gh = ghist + row * NBINS;
    for (int i = t; i < NBINS; i += PWG)
        if (h[i]) atomicAdd(&gh[i], h[i]);
}

// Threshold bin of a row from its global histogram (PWG threads; 16 bins each).
__device__ void row_threshold(const uint32_t* gh, uint32_t need, uint32_t* scan, uint32_t* d_out,
                              uint32_t* above_out) {
    const int t = threadIdx.x;
    constexpr int per = NBINS / PWG;
    uint32_t local = 0;
    uint32_t mine[per];
    for (int i = 0; i < per; ++i) {
        mine[i] = gh[NBINS - 1 - (t * per + i)];
        local += mine[i];
    }
    scan[t] = local;
    __syncthreads();
    for (int off = 1; off < PWG; off <<= 1) {
        uint32_t v = (t >= off) ? scan[t - off] : 0u;
        __syncthreads();
        scan[t] += v;
        __syncthreads();
    }
    uint32_t above = scan[t] - local;
    for (int i = 0; i < per; ++i) {
        if (above < need && need <= above + mine[i]) {
            *d_out = (uint32_t)(NBINS - 1 - (t * per + i));
            *above_out = above;
        }
        above += mine[i];
    }
    __syncthreads();
}

__device__ __forceinline__ uint32_t wave_append(bool pred, uint32_t* counter) {
    const uint64_t m = __ballot(pred);
    if (m == 0) return 0u;
    const int lane = threadIdx.x & 63;
    const int leader = __ffsll((unsigned long long)m) - 1;
    uint32_t base = 0;
    if (lane == leader) base = atomicAdd(counter, (uint32_t)__popcll(m));
    base = __shfl(base, leader);
    return base + (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
}

__global__ __launch_bounds__(PWG) void topk_compact_kernel(const float* __restrict__ scores, int n, int k,
                                                          const uint32_t* __restrict__ ghist,
                                                          RowState* __restrict__ state, int* __restrict__ gsel,
                                                          uint32_t* __restrict__ ckey, uint32_t* __restrict__ cpos) {
    __shared__ uint32_t scan[PWG];
    __shared__ uint32_t sh[2];
    const int t = threadIdx.x;
    const int64_t row = blockIdx.y;
    const uint32_t valid = state[row].valid;
    const bool all = valid <= (uint32_t)k;
    uint32_t d = 0;
    if (!all) {
        row_threshold(ghist + row * NBINS, (uint32_t)k, scan, &sh[0], &sh[1]);
        d = sh[0];
        if (blockIdx.x == 0 && t == 0) state[row].digit = d;
    }
    const float* s = scores + row * (int64_t)n;
    int* sel = gsel + row * KMAX;
    uint32_t* ck = ckey + row * CAP;
    uint32_t* cp = cpos + row * CAP;
    const int lo = blockIdx.x * CHUNK;
    const int hi = min(n, lo + CHUNK);
    // iterate in whole waves so the ballots see every lane
    for (int base = lo; base < hi; base += PWG) {
        const int i = base + t;
        const uint32_t kk = (i < hi) ? key32(s[i]) : 0u;
        const uint32_t dig = kk >> 20;
        const bool take = kk != 0u && (all || dig > d);
        const bool cand = kk != 0u && !all && dig == d;
        const uint32_t at = wave_append(take, &state[row].n_sel);
        if (take) sel[at] = i;
        const uint32_t ca = wave_append(cand, &state[row].n_cand);
        if (cand && ca < CAP) {
            ck[ca] = kk;
            cp[ca] = (uint32_t)i;
        }
    }
}

__global__ __launch_bounds__(WG) void topk_finish_kernel(const float* __restrict__ scores, int n, int k,
                                                         const int32_t* __restrict__ pool,
                                                         const RowState* __restrict__ state,
                                                         const int* __restrict__ gsel,
                                                         const uint32_t* __restrict__ ckey,
                                                         const uint32_t* __restrict__ cpos,
                                                         int32_t* __restrict__ out) {
    __shared__ uint32_t hist[NBINS];
    __shared__ uint32_t scan[WG];
    __shared__ int sel[KMAX];
    __shared__ uint32_t lk[CAP];
    __shared__ uint32_t lp[CAP];
    __shared__ uint32_t sh[4];
    const int t = threadIdx.x;
    const int64_t row = blockIdx.x;
    const RowState st = state[row];
    for (int i = t; i < KMAX; i += WG) sel[i] = (i < (int)st.n_sel) ? gsel[row * KMAX + i] : 0x7FFFFFFF;
    if (t == 0) sh[3] = st.n_sel;
    __syncthreads();
    const bool all = st.valid <= (uint32_t)k;
    if (!all) {
        const uint32_t need = (uint32_t)k - st.n_sel;
        const uint64_t prefix = (uint64_t)st.digit << 52;
        const uint64_t mask = (uint64_t)0xFFF << 52;
        if (st.n_cand <= (uint32_t)CAP) {
            for (int i = t; i < (int)st.n_cand; i += WG) {
                lk[i] = ckey[row * CAP + i];
                lp[i] = cpos[row * CAP + i];
            }
            __syncthreads();
            LdsCands src{lk, lp, (int)st.n_cand};
            radix_select(src, need, 1, prefix, mask, hist, scan, sh, sel, &sh[3]);
        } else {
            GlobalRow src{scores + row * (int64_t)n, n};
            radix_select(src, need, 1, prefix, mask, hist, scan, sh, sel, &sh[3]);
        }
    }
    const uint32_t total = all ? st.valid : (uint32_t)k;
    sort_sel(sel);
    write_out(sel, total, k, pool, row, n / 8, out);
}

size_t large_ws_bytes(int64_t rows) {
    return (size_t)rows * (NBINS * 4 + sizeof(RowState) + KMAX * 4 + CAP * 8) + 256;
}

}  // namespace
}  // namespace csa2

using namespace csa2;

extern "C" size_t csa2_topk_workspace_size(int32_t rows, int32_t n, int32_t k) {
    (void)k;
    if (rows <= 0 || n <= SMALL_N) return 0;
    return large_ws_bytes(rows);
}

extern "C" csa2_status csa2_topk(const float* scores, int32_t rows, int32_t n, int32_t k,
                                 const int32_t* pool_blocks, int32_t* out_idx, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
    clear_error();
    CSA2_ARG(rows >= 0 && n >= 0, "topk: rows=%d n=%d must be >= 0", rows, n);
    CSA2_ARG(k >= 1 && k <= KMAX, "topk: k=%d must be in [1, %d]", k, KMAX);
    CSA2_ARG(pool_blocks == nullptr || n % 8 == 0, "topk: with a pool map n=%d must be a multiple of 8", n);
    if (rows == 0) return CSA2_OK;
    CSA2_ARG(out_idx != nullptr, "topk: null out_idx");
    CSA2_ARG(n == 0 || scores != nullptr, "topk: null scores");
    if (n <= SMALL_N) {
        topk_small_kernel<<<rows, WG, 0, stream>>>(scores, n, k, pool_blocks, out_idx);
        return launch_status("topk");
    }
    const size_t need = large_ws_bytes(rows);
    CSA2_REQUIRE(ws != nullptr && ws_bytes >= need, CSA2_EWORKSPACE,
                 "topk: workspace of %zu bytes required, %zu given", need, ws ? ws_bytes : (size_t)0);
    CSA2_ARG(((uintptr_t)ws & 15) == 0, "topk: workspace must be 16-byte aligned");
    char* w = static_cast<char*>(ws);
    uint32_t* hist = reinterpret_cast<uint32_t*>(w);
    w += (size_t)rows * NBINS * 4;
    RowState* state = reinterpret_cast<RowState*>(w);
    w += (size_t)rows * sizeof(RowState);
    int* sel = reinterpret_cast<int*>(w);
    w += (size_t)rows * KMAX * 4;
    uint32_t* ckey = reinterpret_cast<uint32_t*>(w);
    w += (size_t)rows * CAP * 4;
    uint32_t* cpos = reinterpret_cast<uint32_t*>(w);
    const int64_t zero_n = (int64_t)rows * NBINS;
    topk_zero_kernel<<<(unsigned)((zero_n + 255) / 256), 256, 0, stream>>>(hist, state, rows);
    const dim3 grid((unsigned)((n + CHUNK - 1) / CHUNK), (unsigned)rows);
    topk_hist_kernel<<<grid, PWG, 0, stream>>>(scores, n, hist, state);
    topk_compact_kernel<<<grid, PWG, 0, stream>>>(scores, n, k, hist, state, sel, ckey, cpos);
    topk_finish_kernel<<<rows, WG, 0, stream>>>(scores, n, k, pool_blocks, state, sel, ckey, cpos, out_idx);
    return launch_status("topk");
}
