// Screened Full-mode selection for many query rows of a sequence (multi-token
// decode, prefill chunks): the Top-K of every row, bit for bit the one the
// exact scores define (aprilzz.com V4.1 Flash article, section
// "CSA2：在层的维度上共享缓存": every Full layer selects a new Top-512; score
// definition as in the indexer scan: qbar_c = sum_h q_hc, then an fp32 FMA
// chain over the channels in ascending order).
//
// Exact scores cost D_i FMAs per (row, entry) on the vector ALU, which bounds
// the many-row scan far below the HBM roof.  Instead:
//  1. approximate scores S~ = bf16(qbar) . k on the matrix cores (bf16 x bf16
//     products are exact in fp32, accumulated in fp32), with a bound
//     |S - S~| <= eps = 2^-8 ||qbar||_2 ||k||_2 for every entry (rounding qbar
//     to bf16 moves it by at most 2^-9 |qbar_c| per channel; the two fp32
//     accumulations of 128 terms add at most 2^-16 of sum |qbar_c k_c|; by
//     Cauchy-Schwarz sum |qbar_c k_c| <= ||qbar|| ||k||; the factor keeps a
//     margin of almost 2 over the sum of these terms);
//  2. per row, the lower bounds S~ - eps over aligned 16-entry blocks: the
//     K-th largest block bound tau is <= the K-th largest exact score, since
//     each of those K blocks holds an entry whose exact score is >= its bound;
//  3. candidates: the entries with S~ + eps >= tau -- every entry whose exact
//     score is >= tau, the exact Top-K among them;
//  4. exact scores of the candidates, then the exact selection by composite
//     key (score, position) among them.  A row with more candidates than the
//     buffer holds, or whose candidates do not hold K exact scores >= tau,
//     is scored and selected exactly in full instead.
#include "select.h"

namespace csa2 {
namespace {

constexpr int SC_DI = 128;                // indexer width the screen supports
constexpr int SC_TM = 128;                // query rows per screening workgroup (4 waves x 2 tiles of 16)
constexpr int SC_TN = 128;                // entries per screening workgroup (8 tiles of 16)
constexpr int SC_KROW = SC_DI / 8 + 2;    // 16-byte chunks per staged K row (2 of padding: no bank conflicts)
constexpr int SC_LCAP = 32;               // candidates per row a screening workgroup gathers in LDS
constexpr int SC_CAP = 4096;              // candidates kept per row (4 per selecting thread)
constexpr int SC_MAXN = TOPK_ONEWG_N;     // longest row the screen serves
constexpr float SC_EPS = 0x1p-8f;
constexpr float SC_UP = 1.0f + 0x1p-20f;  // rounds a computed norm up past its fp32 rounding

struct ScreenParams {
    const uint16_t* q_idx;  // [rows][H_i][128]
    int32_t H_i, Q, B;
    int64_t rows;
    const uint16_t* k;
    RowMap kmap;
    const int32_t* n_vis;   // [rows]
    int32_t n_max, nb16, K;
    uint16_t* qhi;          // [rows][128] bf16(qbar)
    float* qn;              // [rows] ||qbar||_2, rounded up
    float* lb;              // [rows][nb16] block lower bounds
    float* tau;             // [rows]
    uint32_t* ccnt;         // [rows] candidate counts
    int32_t* cand;          // [rows][SC_CAP]
    float* scratch;         // [rows][n_max] exact scores of a row selected in full
    int32_t* out;           // [rows][K]
};

__device__ __forceinline__ uint16_t bf16_rne(float x) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // NaN stays NaN
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float row4_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// key32 back to the float it encodes (nonzero keys)
__device__ __forceinline__ float key_float(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// qbar of a row, channel c (h ascending, fp32), as the indexer scan sums it
__device__ __forceinline__ float qbar_channel(const ScreenParams& p, int64_t r, int c) {
    const uint16_t* qr = p.q_idx + r * p.H_i * SC_DI + c;
    float acc = 0.0f;
    for (int h = 0; h < p.H_i; ++h) acc = acc + __uint_as_float((uint32_t)qr[(int64_t)h * SC_DI] << 16);
    return acc;
}

// ---- 0: bf16(qbar) and ||qbar||_2 of every row (one wave per row)
__global__ __launch_bounds__(256) void sc_prep_kernel(ScreenParams p) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + w;
    if (r >= p.rows) return;
    const float a = qbar_channel(p, r, 2 * lane), b = qbar_channel(p, r, 2 * lane + 1);
    reinterpret_cast<uint32_t*>(p.qhi + r * SC_DI)[lane] = (uint32_t)bf16_rne(a) | ((uint32_t)bf16_rne(b) << 16);
    float ss = fmaf(a, a, b * b);
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if (lane == 0) p.qn[r] = (ss < INFINITY) ? sqrtf(ss) * SC_UP : INFINITY;
}

// ---- 1 and 2: screening products of SC_TM rows x SC_TN entries of one
// sequence on the matrix cores.  PASS 1 writes the block lower bounds, PASS 2
// the candidates.  The K tile is staged in LDS (row (key) k at k * SC_KROW
// chunks), the A operand of v_mfma_f32_16x16x32_bf16 is entry (lane % 16),
// channels 32 blk + 8 (lane / 16) .. +7, the B operand row (lane % 16) of the
// wave's 16-row tile; the accumulator holds entries 4 (lane / 16) .. +3 of row
// (lane % 16).
template <int PASS>
__global__ __launch_bounds__(256, 2) void sc_gemm_kernel(ScreenParams p) {
    __shared__ uint4 kt[SC_TN * SC_KROW];
    __shared__ __attribute__((aligned(16))) float kns[SC_TN];
    __shared__ uint32_t nvmax_s;
    __shared__ uint32_t lc[PASS == 2 ? SC_TM : 1];
    __shared__ int32_t lcand[PASS == 2 ? SC_TM * SC_LCAP : 1];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6, c16 = lane & 15, g = lane >> 4;
    const int b = blockIdx.z;
    const int q0 = blockIdx.y * SC_TM;
    const int64_t e0 = (int64_t)blockIdx.x * SC_TN;

    // the lane's rows (two 16-row tiles per wave)
    int64_t rr[2];
    int nvr[2];
    bool rok[2];
    uint32_t nvl = 0;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int ql = q0 + 32 * w + 16 * rt + c16;
        rok[rt] = ql < p.Q;
        rr[rt] = (int64_t)b * p.Q + (rok[rt] ? ql : 0);
        nvr[rt] = rok[rt] ? min(max(p.n_vis[rr[rt]], 0), p.n_max) : 0;
        nvl = max(nvl, (uint32_t)nvr[rt]);
    }
    // B operands and the row constants load while the visible range is agreed on
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    bf16x8 qb[2][4];
    float qnr[2], taur[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const uint4* qp = reinterpret_cast<const uint4*>(p.qhi + rr[rt] * SC_DI);
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            const uint4 v = rok[rt] ? qp[4 * blk + g] : make_uint4(0u, 0u, 0u, 0u);
            qb[rt][blk] = __builtin_bit_cast(bf16x8, v);
        }
        qnr[rt] = p.qn[rr[rt]];
        taur[rt] = PASS == 2 ? p.tau[rr[rt]] : 0.0f;
    }
    if (t == 0) nvmax_s = 0u;
    if (PASS == 2 && t < SC_TM) lc[t] = 0u;
    __syncthreads();
    nvl = wave_umax(nvl);
    if (lane == 0) atomicMax(&nvmax_s, nvl);
    __syncthreads();
    const int64_t nvmax = nvmax_s;
    if (e0 >= nvmax) return;  // no row of this workgroup sees these entries

    // ---- stage the K tile (entries past every row's view read as zeros) and
    // the entries' norms: load i of thread t is chunk t % 16 of entry 16 i + t / 16
#pragma unroll
    for (int i = 0; i < SC_TN * 16 / 256; ++i) {
        const int el = 16 * i + (t >> 4), c = t & 15;
        const int64_t e = e0 + el;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (e < nvmax) v = *reinterpret_cast<const uint4*>(p.k + phys_row(p.kmap, b, e) * SC_DI + 8 * c);
        kt[el * SC_KROW + c] = v;
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
        float ss = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            ss = fmaf(bf16_lo(wv[j]), bf16_lo(wv[j]), ss);
            ss = fmaf(bf16_hi(wv[j]), bf16_hi(wv[j]), ss);
        }
        ss += __shfl_xor(ss, 1);
        ss += __shfl_xor(ss, 2);
        ss += __shfl_xor(ss, 4);
        ss += __shfl_xor(ss, 8);
        if (c == 0) kns[el] = (ss < INFINITY) ? sqrtf(ss) * SC_UP : INFINITY;
    }
    __syncthreads();

    float lbv[2][SC_TN / 16];
#pragma unroll
    for (int j = 0; j < SC_TN / 16; ++j) {
        f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            const bf16x8 a = __builtin_bit_cast(bf16x8, kt[(16 * j + c16) * SC_KROW + 4 * blk + g]);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[rt][blk], acc[rt], 0, 0, 0);
        }
        const float4 kn4 = *reinterpret_cast<const float4*>(&kns[16 * j + 4 * g]);
        const float knv[4] = {kn4.x, kn4.y, kn4.z, kn4.w};
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            float m = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t e = e0 + 16 * j + 4 * g + i;
                const bool valid = e < nvr[rt];
                const float eps = SC_EPS * qnr[rt] * knv[i];
                if (PASS == 1) {
                    const float lo = acc[rt][i] - eps;
                    if (valid && lo == lo) m = fmaxf(m, lo);  // (NaN: no bound)
                } else if (valid && !(acc[rt][i] + eps < taur[rt])) {  // (NaN: a candidate)
                    const int rl = 32 * w + 16 * rt + c16;
                    const uint32_t slot = atomicAdd(&lc[rl], 1u);
                    if (slot < (uint32_t)SC_LCAP) {
                        lcand[rl * SC_LCAP + slot] = (int32_t)e;
                    } else {
                        const uint32_t gs = atomicAdd(&p.ccnt[rr[rt]], 1u);
                        if (gs < (uint32_t)SC_CAP) p.cand[rr[rt] * SC_CAP + gs] = (int32_t)e;
                    }
                }
            }
            if (PASS == 1) lbv[rt][j] = row4_max(m);
        }
    }
    if (PASS == 1) {
        if (g == 0) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                if (!rok[rt]) continue;
#pragma unroll
                for (int j = 0; j < SC_TN / 16; ++j) {
                    const int64_t bi = e0 / 16 + j;
                    if (bi < p.nb16) p.lb[rr[rt] * p.nb16 + bi] = lbv[rt][j];
                }
            }
        }
    } else {
        __syncthreads();
        if (t < SC_TM && q0 + t < p.Q) {
            const uint32_t n = min(lc[t], (uint32_t)SC_LCAP);
            if (n) {
                const int64_t r = (int64_t)b * p.Q + q0 + t;
                const uint32_t base = atomicAdd(&p.ccnt[r], n);
                for (uint32_t i = 0; i < n && base + i < (uint32_t)SC_CAP; ++i)
                    p.cand[r * SC_CAP + base + i] = lcand[t * SC_LCAP + i];
            }
        }
    }
}

// ---- between the passes: tau = the K-th largest block lower bound of each
// row (-inf when the row has fewer than K blocks or bounds: every visible
// entry is then a candidate), four 8-bit radix passes over the keys; clears
// the row's candidate count.
constexpr int TAU_NT = 256;
__global__ __launch_bounds__(TAU_NT) void sc_tau_kernel(ScreenParams p) {
    __shared__ uint32_t h[256];
    __shared__ uint32_t wsum[TAU_NT / 64];
    __shared__ uint32_t s_d, s_need;
    const int64_t r = blockIdx.x;
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int nv = min(max(p.n_vis[r], 0), p.n_max);
    const int nb = (nv + 15) / 16;
    if (t == 0) p.ccnt[r] = 0u;
    constexpr int E = (SC_MAXN / 16 + TAU_NT - 1) / TAU_NT;
    uint32_t key[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = t + TAU_NT * e;
        key[e] = i < nb ? key32(p.lb[r * p.nb16 + i]) : 0u;
    }
    uint32_t prefix = 0, need = (uint32_t)p.K;
    bool ok = nb >= p.K;
    for (int pass = 0; pass < 4 && ok; ++pass) {
        const int sh = 24 - 8 * pass;
        h[t] = 0u;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (key[e] != 0u && (pass == 0 || (key[e] >> (sh + 8)) == (prefix >> (sh + 8))))
                atomicAdd(&h[(key[e] >> sh) & 255u], 1u);
        __syncthreads();
        // bins from the top: thread t holds bin 255 - t
        const uint32_t x = h[255 - t];
        const uint32_t incl = wave_incl_scan(x);
        if (lane == 63) wsum[wid] = incl;
        __syncthreads();
        uint32_t above = incl - x, total = 0;
#pragma unroll
        for (int v = 0; v < TAU_NT / 64; ++v) {
            above += (v < wid) ? wsum[v] : 0u;
            total += wsum[v];
        }
        if (above < need && need <= above + x) {
            s_d = (uint32_t)(255 - t);
            s_need = need - above;
        }
        __syncthreads();
        if (total < need) {
            ok = false;  // (block-uniform) fewer valid bounds than K
        } else {
            prefix |= s_d << sh;
            need = s_need;
        }
        __syncthreads();
    }
    if (t == 0) p.tau[r] = ok ? key_float(prefix) : -INFINITY;
}

// exact score of entry j of sequence b (the indexer scan's FMA chain).  qbar
// is read from LDS (broadcast) at an opaque offset, so that the compiler does
// not hoist all 128 values into registers across the caller's loop.
__device__ __forceinline__ float exact_score(const ScreenParams& p, int b, int64_t j, const float* qb) {
    const uint4* kr = reinterpret_cast<const uint4*>(p.k + phys_row(p.kmap, b, j) * SC_DI);
    int z;
    asm volatile("s_mov_b32 %0, 0" : "=s"(z));
    const float4* q4 = reinterpret_cast<const float4*>(qb) + z;
    float acc = 0.0f;
    // (the row in two halves of 64 channels: half the registers in flight)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        uint4 kv[SC_DI / 16];
#pragma unroll
        for (int c = 0; c < SC_DI / 16; ++c) kv[c] = kr[hf * (SC_DI / 16) + c];
#pragma unroll
        for (int c = 0; c < SC_DI / 16; ++c) {
            const int cc = hf * (SC_DI / 16) + c;
            const float4 qa = q4[2 * cc], qc = q4[2 * cc + 1];
            acc = fmaf(qa.x, bf16_lo(kv[c].x), acc);
            acc = fmaf(qa.y, bf16_hi(kv[c].x), acc);
            acc = fmaf(qa.z, bf16_lo(kv[c].y), acc);
            acc = fmaf(qa.w, bf16_hi(kv[c].y), acc);
            acc = fmaf(qc.x, bf16_lo(kv[c].z), acc);
            acc = fmaf(qc.y, bf16_hi(kv[c].z), acc);
            acc = fmaf(qc.z, bf16_lo(kv[c].w), acc);
            acc = fmaf(qc.w, bf16_hi(kv[c].w), acc);
        }
    }
    return acc;
}

// ---- 3: exact scores of the candidates and the exact selection (one
// workgroup per row).  Candidate scores are computed one entry per thread at
// a time into LDS, then taken into registers as keys (SC_CAP / WG per
// thread); the full fallback scores the row into its scratch and selects
// from there.
__global__ __launch_bounds__(WG) void sc_select_kernel(ScreenParams p) {
    __shared__ SelectLds sh;
    __shared__ int sel[TOPK_KMAX];
    __shared__ int tmp[TOPK_KMAX];
    __shared__ __attribute__((aligned(16))) float qb[SC_DI];
    __shared__ float cs[SC_CAP];
    __shared__ uint32_t s_valid, s_ge;
    const int64_t r = blockIdx.x;
    const int b = (int)(r / p.Q);
    const int t = threadIdx.x;
    const int nv = min(max(p.n_vis[r], 0), p.n_max);
    const uint32_t cnt = p.ccnt[r];
    const float tau = p.tau[r];
    if (t < SC_DI) qb[t] = qbar_channel(p, r, t);
    for (int i = t; i < NBINS1; i += WG) sh.hist[0][i] = 0u;
    if (t == 0) {
        sh.nsel = 0u;
        s_valid = 0u;
        s_ge = 0u;
    }
    __syncthreads();
    const uint32_t ktau = tau == -INFINITY ? 0u : key32(tau);
    const bool screened = cnt <= (uint32_t)SC_CAP;
    constexpr int EC = SC_CAP / WG;
    uint32_t key[EC], pos[EC];
    if (screened) {
#pragma unroll 1
        for (uint32_t i = t; i < cnt; i += WG) cs[i] = exact_score(p, b, p.cand[r * SC_CAP + i], qb);
        __syncthreads();
        uint32_t nvalid = 0, nge = 0;
#pragma unroll
        for (int e = 0; e < EC; ++e) {
            const uint32_t i = (uint32_t)(t + WG * e);
            key[e] = i < cnt ? key32(cs[i]) : 0u;
            pos[e] = i < cnt ? (uint32_t)p.cand[r * SC_CAP + i] : 0u;
            nvalid += key[e] != 0u;
            nge += key[e] != 0u && key[e] >= ktau;
        }
        nvalid = wave_sum(nvalid);
        nge = wave_sum(nge);
        if ((t & 63) == 0) {
            atomicAdd(&s_valid, nvalid);
            atomicAdd(&s_ge, nge);
        }
    }
    __syncthreads();
    // the candidates hold the answer when they hold K exact scores >= tau, or
    // (tau = -inf: every visible entry is a candidate) all visible entries
    const bool use = screened && (tau == -INFINITY ? cnt == (uint32_t)nv : s_ge >= (uint32_t)p.K);
    uint32_t total;
    if (use) {
        total = min((uint32_t)p.K, s_valid);
        if (s_valid > (uint32_t)p.K) {
            uint64_t prefix = 0, mask = 0;
            select_regs<EC>(key, pos, (uint32_t)p.K, 0, prefix, mask, sh);
#pragma unroll
            for (int e = 0; e < EC; ++e)
                if (key[e] != 0u && (composite(key[e], pos[e]) & mask) >= prefix) sel[atomicAdd(&sh.nsel, 1u)] = (int)pos[e];
        } else {
#pragma unroll
            for (int e = 0; e < EC; ++e)
                if (key[e] != 0u) sel[atomicAdd(&sh.nsel, 1u)] = (int)pos[e];
        }
        __syncthreads();
    } else {
        // every visible entry, exactly, into the row's scratch; the selection
        // then runs its radix passes over the scratch
        float* srow = p.scratch + r * p.n_max;
        uint32_t nval = 0;
#pragma unroll 1
        for (int j = t; j < nv; j += WG) {
            const float sc = exact_score(p, b, j, qb);
            srow[j] = sc;
            nval += key32(sc) != 0u;
        }
        nval = wave_sum(nval);
        if (t == 0) s_valid = 0u;
        __syncthreads();
        if ((t & 63) == 0) atomicAdd(&s_valid, nval);
        __syncthreads();
        total = min((uint32_t)p.K, s_valid);
        if (s_valid > (uint32_t)p.K) {
            select_global_row(srow, nv, (uint32_t)p.K, 0, 0, sh, sel);
        } else {
            for (int j = t; j < nv; j += WG)
                if (key32(srow[j]) != 0u) sel[atomicAdd(&sh.nsel, 1u)] = j;
            __syncthreads();
        }
    }
    emit_sorted(sel, (int)total, p.n_max, p.K, sh, tmp, p.out, nullptr, r);
}

inline size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

bool screen_applicable(int32_t B, int32_t Q, int32_t D_i, int32_t n_max, int32_t K) {
    const int64_t rows = (int64_t)B * Q;
    return Q >= 2 && rows >= 64 && D_i == SC_DI && n_max > 0 && n_max <= SC_MAXN && K >= 1 && K <= TOPK_KMAX;
}

size_t screen_ws_bytes(int32_t B, int32_t Q, int32_t n_max) {
    if (Q < 2 || n_max <= 0 || n_max > SC_MAXN) return 0;
    const int64_t rows = (int64_t)B * Q;
    const int64_t nb16 = (n_max + 15) / 16;
    return al256(rows * SC_DI * 2) + 3 * al256(rows * 4) + al256(rows * nb16 * 4) + al256(rows * SC_CAP * 4) + 256;
}

csa2_status screen_select(const uint16_t* q_idx, int32_t B, int32_t Q, int32_t H_i, const csa2_idx_k* k,
                          const int32_t* n_vis, int32_t n_max, int32_t K, void* ws, size_t ws_bytes, float* scratch,
                          int32_t* out, hipStream_t stream) {
    CSA2_ARG(screen_applicable(B, Q, k ? k->D_i : 0, n_max, K), "screen: unsupported shape");
    CSA2_ARG(q_idx && k && k->k && n_vis && out && ws && scratch, "screen: null pointer");
    CSA2_ARG(H_i >= 1 && H_i <= 64, "screen: H_i=%d", H_i);
    CSA2_REQUIRE(ws_bytes >= screen_ws_bytes(B, Q, n_max), CSA2_EWORKSPACE, "screen: workspace too small");
    ScreenParams p{};
    csa2_status st = make_rowmap(k->page_table, k->page_size, k->max_pages, k->seq_stride, n_max, &p.kmap, "screen");
    if (st != CSA2_OK) return st;
    const int64_t rows = (int64_t)B * Q;
    p.q_idx = q_idx;
    p.H_i = H_i;
    p.Q = Q;
    p.B = B;
    p.rows = rows;
    p.k = k->k;
    p.n_vis = n_vis;
    p.n_max = n_max;
    p.nb16 = (n_max + 15) / 16;
    p.K = K;
    char* w = static_cast<char*>(ws);
    w = reinterpret_cast<char*>(((uintptr_t)w + 255) & ~(uintptr_t)255);
    p.qhi = reinterpret_cast<uint16_t*>(w);
    w += al256(rows * SC_DI * 2);
    p.qn = reinterpret_cast<float*>(w);
    w += al256(rows * 4);
    p.tau = reinterpret_cast<float*>(w);
    w += al256(rows * 4);
    p.ccnt = reinterpret_cast<uint32_t*>(w);
    w += al256(rows * 4);
    p.lb = reinterpret_cast<float*>(w);
    w += al256(rows * (int64_t)p.nb16 * 4);
    p.cand = reinterpret_cast<int32_t*>(w);
    p.scratch = scratch;
    p.out = out;
    sc_prep_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, stream>>>(p);
    const dim3 grid((unsigned)((n_max + SC_TN - 1) / SC_TN), (unsigned)((Q + SC_TM - 1) / SC_TM), (unsigned)B);
    sc_gemm_kernel<1><<<grid, 256, 0, stream>>>(p);
    sc_tau_kernel<<<(unsigned)rows, TAU_NT, 0, stream>>>(p);
    sc_gemm_kernel<2><<<grid, 256, 0, stream>>>(p);
    sc_select_kernel<<<(unsigned)rows, WG, 0, stream>>>(p);
    return launch_status("screen");
}

}  // namespace csa2
