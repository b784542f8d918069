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
//     |S - S~| <= eps for every entry, S the exact score's fp32 chain.  With
//     T = sum_c |qbar_c k_c| <= ||qbar|| ||k|| (Cauchy-Schwarz) and u = 2^-8
//     the unit roundoff of bf16: rounding qbar to bf16 moves channel c by at
//     most u/(1+u) |qbar_c| < (2^-8 - 2^-16 + 2^-24) |qbar_c|, so the real
//     products move by less than (2^-8 - 2^-16 + 2^-24) T; the matrix cores'
//     fp32 sum of 128 products adds at most 2^-16 T (two units of 2^-24 per
//     addition, so that a truncating adder is covered), the exact chain of
//     128 FMAs at most 2^-17 T.  eps = (2^-8 + 2^-15) ||qbar|| ||k|| covers
//     the total, below 2^-8 + 2^-17 + 2^-24 of T, with the roundings of eps
//     and of S~ +- eps and the norms (rounded up) inside the margin.  Subnormal operands
//     or products, were they flushed, move a score by at most
//     2^-122 (||qbar|| + ||k||) + 2^-118: eps carries twice that as an
//     absolute term;
//     Each aligned group of four entries takes the eps of the largest of its
//     four norms (eps grows with the norm, so it bounds each of them), so that
//     the bounds cost one operation per group of four and row, not per entry;
//  2. per row, the lower bounds S~ - eps over aligned 16-entry blocks: the
//     K-th largest block bound tau is <= the K-th largest exact score, since
//     each of those K blocks holds an entry whose exact score is >= its bound;
//  3. candidates: the entries with S~ + eps >= tau -- every entry whose exact
//     score is >= tau, the exact Top-K among them;
//  4. exact scores of the candidates, then the exact selection by composite
//     key (score, position) among them (one wave per row).  A row with more candidates than the
//     buffer holds, or whose candidates do not hold K exact scores >= tau,
//     is scored and selected exactly in full instead.
#include "select.h"

namespace csa2 {
namespace {

constexpr int SC_DI = 128;                // indexer width the screen supports
constexpr int SC_TM = 128;                // query rows per screening workgroup (4 waves x 2 tiles of 16)
constexpr int SC_TN = 128;                // entries per staged sub-tile (8 MFMA tiles of 16)
constexpr int SC_SUB = 8;                 // sub-tiles per screening workgroup (1024 entries)
constexpr int SC_KROW = SC_DI / 8 + 2;    // 16-byte chunks per staged K row (2 of padding: no bank conflicts)
constexpr int SC_CAP = 4096;              // candidates kept per row
constexpr int SC_WCAP = 1024;             // candidates a one-wave selection holds (16 per lane)
constexpr int SC_MAXN = TOPK_ONEWG_N;     // longest row the screen serves (its position bitmap: 4 KB)
constexpr float SC_EPS = 0x1.02p-8f;      // relative part of the bound (times ||qbar|| ||k||): 2^-8 + 2^-15
constexpr float SC_EABS_N = 0x1p-121f;    // absolute part: times (||qbar|| + ||k||) ...
constexpr float SC_EABS = 0x1p-117f;      // ... plus this
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
    float* cscore;          // [rows][SC_CAP] exact scores of the candidates
    float* kn;              // [B][n_max] ||k||_2 of the entries, rounded up
    float* qbf;             // [rows][128] qbar in fp32 (the exact scores' query)
    uint2* seg;             // [rows][nwx] (first slot, count) of each screening workgroup's candidates
    int32_t nwx;            // screening workgroups along the entries
    uint32_t* slow;         // [0] rows queued for the workgroup selection, [1] rows taken, [2..] the rows
    float* scratch;         // [rows][n_max] exact scores of a row selected in full
    int32_t* out;           // [rows][K]
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

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

// the bound eps of one entry from the row's constants (qe, qa) and the
// entry's norm: eps = qe kn + 2^-121 kn + qa, with qe = (2^-8 + 2^-15) ||qbar||
// and qa = 2^-121 ||qbar|| + 2^-117 (both screening passes form L and U
// through these, so that they agree bit for bit)
__device__ __forceinline__ void row_eps(float qn, float& qe, float& qa) {
    qe = SC_EPS * qn;
    qa = fmaf(SC_EABS_N, qn, SC_EABS);
}
__device__ __forceinline__ float entry_eps(float qe, float qa, float kn) {
    return fmaf(qe, kn, fmaf(SC_EABS_N, kn, qa));
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// qbar of a row, channel c (h ascending, fp32), as the indexer scan sums it
__device__ __forceinline__ float qbar_channel(const ScreenParams& p, int64_t r, int c) {
    const uint16_t* qr = p.q_idx + r * p.H_i * SC_DI + c;
    float acc = 0.0f;
    for (int h = 0; h < p.H_i; ++h) acc = acc + __uint_as_float((uint32_t)qr[(int64_t)h * SC_DI] << 16);
    return acc;
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
    // (the row in two halves of 64 channels: half the registers in flight; a
    // rolled loop keeps the rescoring kernel within 128 registers, so that two
    // of its workgroups share a CU)
#pragma unroll 1
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

// ---- 0: bf16(qbar) and ||qbar||_2 of every row (one wave per row); clears
// the queue of rows for the workgroup selection
__global__ __launch_bounds__(256) void sc_prep_kernel(ScreenParams p) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (blockIdx.x == 0 && threadIdx.x < 2) p.slow[threadIdx.x] = 0u;
    const int64_t r = (int64_t)blockIdx.x * 4 + w;
    if (r >= p.rows) return;
    const float a = qbar_channel(p, r, 2 * lane), b = qbar_channel(p, r, 2 * lane + 1);
    reinterpret_cast<uint32_t*>(p.qhi + r * SC_DI)[lane] = (uint32_t)bf16_rne(a) | ((uint32_t)bf16_rne(b) << 16);
    reinterpret_cast<float2*>(p.qbf + r * SC_DI)[lane] = make_float2(a, b);
    float ss = fmaf(a, a, b * b);
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if (lane == 0) p.qn[r] = (ss < INFINITY) ? sqrtf(ss) * SC_UP : INFINITY;
}

// ---- 1 and 2: screening products of SC_TM rows x SC_SUB sub-tiles of SC_TN
// entries of one sequence on the matrix cores.  PASS 1 writes the block lower
// bounds and the entries' norms, PASS 2 the candidates (one global atomic per
// row and workgroup).  Sub-tiles are staged in two LDS buffers (row (entry) e
// at e * SC_KROW chunks): the next one's loads fly while the current one is
// multiplied.  The A operand of v_mfma_f32_16x16x32_bf16 is entry (lane % 16),
// channels 32 blk + 8 (lane / 16) .. +7, the B operand row (lane % 16) of the
// wave's 16-row tile; the accumulator holds entries 4 (lane / 16) .. +3 of
// row (lane % 16).  (kb, lbo, kno: restrict pointers, so that the compiler
// need not wait for a store before the next K load.)
template <int PASS, bool CONTIG>
__global__ __launch_bounds__(256, 2) void sc_gemm_kernel(ScreenParams p, const uint16_t* __restrict__ kb,
                                                         float* __restrict__ lbo, float* __restrict__ kno) {
    __shared__ uint4 kt[2][SC_TN * SC_KROW];
    __shared__ __attribute__((aligned(16))) float kns[2][SC_TN];
    __shared__ uint32_t nvmax_s;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6, c16 = lane & 15, g = lane >> 4;
    const int b = blockIdx.z;
    const int q0 = blockIdx.y * SC_TM;
    const int64_t ew = (int64_t)blockIdx.x * SC_TN * SC_SUB;

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
        const int nvl_r = p.n_vis[rr[rt]];  // (loads stay unconditional: rr is a valid row)
        nvr[rt] = rok[rt] ? min(max(nvl_r, 0), p.n_max) : 0;
        nvl = max(nvl, (uint32_t)nvr[rt]);
    }
    // B operands and the row constants load while the visible range is agreed on
    bf16x8 qb[2][4];
    float qe[2], qa[2], taur[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const uint4* qp = reinterpret_cast<const uint4*>(p.qhi + rr[rt] * SC_DI);
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            uint4 v = qp[4 * blk + g];
            if (!rok[rt]) v = make_uint4(0u, 0u, 0u, 0u);
            qb[rt][blk] = __builtin_bit_cast(bf16x8, v);
        }
        row_eps(p.qn[rr[rt]], qe[rt], qa[rt]);
        taur[rt] = PASS == 2 ? p.tau[rr[rt]] : 0.0f;
    }
    if (t == 0) nvmax_s = 0u;
    __syncthreads();
    nvl = wave_umax(nvl);
    if (lane == 0) atomicMax(&nvmax_s, nvl);
    __syncthreads();
    const int64_t nvmax = nvmax_s;
    if (ew >= nvmax) return;  // no row of this workgroup sees these entries
    const int nloc = (int)min((int64_t)SC_TN * SC_SUB, nvmax - ew);  // entries of this workgroup someone sees
    const int nsub = (nloc + SC_TN - 1) / SC_TN;

    // staging: load i of thread t is chunk t % 16 of entry 16 i + t / 16 of a
    // sub-tile, at a 32-bit offset from the workgroup's first entry; entries
    // nobody sees read the last seen entry (loads stay unconditional: a
    // conditional load makes the compiler wait for it at once) and are zeroed
    // when stored
    constexpr int NLD = SC_TN * 16 / 256;
    const uint16_t* kw = CONTIG ? kb + ((int64_t)b * p.kmap.seq_stride + ew) * SC_DI : kb;
    uint4 v[NLD];
    auto load = [&](int s) {
        if (CONTIG) {
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                const int el = min(s * SC_TN + 16 * i + (t >> 4), nloc - 1);
                v[i] = *reinterpret_cast<const uint4*>(kw + (uint32_t)el * SC_DI + 8 * (t & 15));
            }
        } else {
            int64_t row[NLD];  // all page lookups first, then all loads
#pragma unroll
            for (int i = 0; i < NLD; ++i) row[i] = phys_row(p.kmap, b, ew + min(s * SC_TN + 16 * i + (t >> 4), nloc - 1));
#pragma unroll
            for (int i = 0; i < NLD; ++i) v[i] = *reinterpret_cast<const uint4*>(kb + row[i] * SC_DI + 8 * (t & 15));
        }
    };
    auto store = [&](int s, int buf) {
        float knl[NLD];
        if (PASS == 2) {
            // norms from the first pass (the same workgroup coordinates wrote them)
            if (t < SC_TN) kns[buf][t] = s * SC_TN + t < nloc ? kno[(int64_t)b * p.n_max + ew + s * SC_TN + t] : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int el = 16 * i + (t >> 4), c = t & 15;
            if (s * SC_TN + el >= nloc) v[i] = make_uint4(0u, 0u, 0u, 0u);
            kt[buf][el * SC_KROW + c] = v[i];
            if (PASS == 1) {
                // ||k||^2 of the entry: bf16 pair dot products, then the 16 lanes
                // holding its chunks (one DPP row) summed
                typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
                const uint32_t wv[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
                float ss = 0.0f;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const bf16x2 x = __builtin_bit_cast(bf16x2, wv[jj]);
                    ss = __builtin_amdgcn_fdot2_f32_bf16(x, x, ss, false);
                }
                ss += __uint_as_float(dpp_src<0xB1>(__float_as_uint(ss)));
                ss += __uint_as_float(dpp_src<0x4E>(__float_as_uint(ss)));
                ss += __uint_as_float(dpp_src<0x141>(__float_as_uint(ss)));
                ss += __uint_as_float(dpp_src<0x140>(__float_as_uint(ss)));
                knl[i] = (ss < INFINITY) ? sqrtf(ss) * SC_UP : INFINITY;
            }
        }
        if (PASS == 1) {
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                const int el = 16 * i + (t >> 4);
                if ((t & 15) == 0) {
                    kns[buf][el] = knl[i];
                    // (every row tile writes the same values: the second pass of the
                    // same coordinates reads the entries its rows see)
                    if (s * SC_TN + el < nloc) kno[(int64_t)b * p.n_max + ew + s * SC_TN + el] = knl[i];
                }
            }
        }
    };
    load(0);
    store(0, 0);
    __syncthreads();

    uint32_t cm[2][SC_SUB];  // PASS 2: candidate bits of sub-tile s, bit 4j + i = entry 16j + 4g + i
#pragma unroll
    for (int s = 0; s < SC_SUB; ++s) {
        cm[0][s] = 0u;
        cm[1][s] = 0u;
        if (s < nsub) {
            const int buf = s & 1;
            if (s + 1 < nsub) load(s + 1);
            const int64_t es = ew + (int64_t)s * SC_TN;
            // entry 16 j + 4 g + i of the sub-tile is visible to row rt iff 16 j + i < lim4[rt]
            int lim4[2];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) lim4[rt] = (int)min(max((int64_t)nvr[rt] - es, (int64_t)0), (int64_t)SC_TN) - 4 * g;
            float lbv[2][SC_TN / 16];
#pragma unroll
            for (int j = 0; j < SC_TN / 16; ++j) {
                f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
                for (int blk = 0; blk < 4; ++blk) {
                    const bf16x8 a = __builtin_bit_cast(bf16x8, kt[buf][(16 * j + c16) * SC_KROW + 4 * blk + g]);
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt)
                        acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[rt][blk], acc[rt], 0, 0, 0);
                }
                // the largest norm of the lane's four entries 16 j + 4 g .. +3
                const float4 kn4 = *reinterpret_cast<const float4*>(&kns[buf][16 * j + 4 * g]);
                const float kn4m = fmaxf(fmaxf(kn4.x, kn4.y), fmaxf(kn4.z, kn4.w));
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    const float eps4 = entry_eps(qe[rt], qa[rt], kn4m);
                    if (PASS == 1) {
                        // the group's lower bound: its largest S~ less the group's eps
                        float m = -INFINITY;
#pragma unroll
                        for (int i = 0; i < 4; ++i) m = fmaxf(m, 16 * j + i < lim4[rt] ? acc[rt][i] : -INFINITY);
                        float lo = m - eps4;
                        lo = lo == lo ? lo : -INFINITY;  // (a NaN bound bounds nothing)
                        lbv[rt][j] = row4_max(lo);
                    } else {
                        // candidates: S~ >= tau - eps (NaN: a candidate)
                        const float t4 = taur[rt] - eps4;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const bool c = 16 * j + i < lim4[rt] && !(acc[rt][i] < t4);
                            cm[rt][s] |= (uint32_t)c << (4 * j + i);
                        }
                    }
                }
            }
            if (PASS == 1 && g == 0) {
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    if (!rok[rt]) continue;
#pragma unroll
                    for (int j = 0; j < SC_TN / 16; ++j) {
                        const int64_t bi = es / 16 + j;
                        if (bi < p.nb16) lbo[rr[rt] * p.nb16 + bi] = lbv[rt][j];
                    }
                }
            }
            // (the next sub-tile's LDS writes stay after this one's reads: hoisted
            // above them they would wait for its loads before the products)
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            if (s + 1 < nsub) store(s + 1, buf ^ 1);
            __syncthreads();
        }
    }
    if (PASS == 2) {
        // one atomic per row: the four lanes of a row (lane / 16 = 0..3) take
        // consecutive slots in lane order
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            uint32_t n = 0;
#pragma unroll
            for (int s = 0; s < SC_SUB; ++s) n += (uint32_t)__popc(cm[rt][s]);
            const uint32_t n0 = __shfl(n, c16), n1 = __shfl(n, c16 + 16), n2 = __shfl(n, c16 + 32),
                           n3 = __shfl(n, c16 + 48);
            const uint32_t total = n0 + n1 + n2 + n3;
            uint32_t base = 0;
            if (g == 0 && rok[rt]) {
                if (total) base = atomicAdd(&p.ccnt[rr[rt]], total);
                p.seg[rr[rt] * p.nwx + blockIdx.x] = make_uint2(base, total);
            }
            base = __shfl(base, c16);
            uint32_t at = base + (g > 0 ? n0 : 0u) + (g > 1 ? n1 : 0u) + (g > 2 ? n2 : 0u);
#pragma unroll
            for (int s = 0; s < SC_SUB; ++s) {
                uint32_t bits = cm[rt][s];
                while (bits) {
                    const int bit = __builtin_ctz(bits);
                    bits &= bits - 1u;
                    if (at < (uint32_t)SC_CAP)
                        p.cand[rr[rt] * SC_CAP + at] =
                            (int32_t)(ew + (int64_t)s * SC_TN + 16 * (bit >> 2) + 4 * g + (bit & 3));
                    ++at;
                }
            }
        }
    }
}

// ---- between the passes: tau = the K-th largest block lower bound of each
// row with its key's low 16 bits cleared (-inf when the row has fewer than K
// blocks or bounds: every visible entry is then a candidate), bit by bit over
// the top 16 key bits (one wave per row, SC_MAXN / 16 / 64 bounds per lane);
// clears the row's candidate count.  Any value at or below the K-th bound is
// a valid tau; the top 16 bits (a relative step of at most 2^-7) take half the
// bisection steps for about 3 % more candidates.
__global__ __launch_bounds__(256) void sc_tau_kernel(ScreenParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= p.rows) return;
    const int nv = min(max(p.n_vis[r], 0), p.n_max);
    const int nb = (nv + 15) / 16;
    if (lane == 0) p.ccnt[r] = 0u;
    constexpr int E = SC_MAXN / 16 / 64;
    uint32_t key[E];
    uint32_t nz = 0;
    float x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = p.lb[r * p.nb16 + min(lane + 64 * e, p.nb16 - 1)];  // (unconditional loads)
#pragma unroll
    for (int e = 0; e < E; ++e) {
        key[e] = lane + 64 * e < nb ? key32(x[e]) : 0u;
        nz += key[e] != 0u;
    }
    nz = wave_sum(nz);
    float tau = -INFINITY;
    if (nz >= (uint32_t)p.K) {
        uint32_t v = 0u;  // the largest v (low 16 bits clear) with #{key >= v} >= K
        for (int bit = 31; bit >= 16; --bit) {
            const uint32_t c = v | (1u << bit);
            uint32_t n = 0;
#pragma unroll
            for (int e = 0; e < E; ++e) n += key[e] >= c;
            if (wave_sum(n) >= (uint32_t)p.K) v = c;
        }
        tau = v ? key_float(v) : -INFINITY;
    }
    if (lane == 0) p.tau[r] = tau;
}

// ---- 3: exact scores of the candidates, by the screening workgroups'
// coordinates: the workgroup of rows q0..q0+127 and entries ew..ew+1023 takes
// the candidates the second pass found there (their K rows were just read by
// the same coordinates, so they come from this XCD's L2), with the rows'
// qbar staged in LDS; one candidate per thread at a time, the next one located
// while the current one is scored.
constexpr int RS_NT = 512;  // threads of the rescoring workgroup
__global__ __launch_bounds__(RS_NT, 4) void sc_rescore_kernel(ScreenParams p) {
    // (rows padded by 4 floats: lanes reading one channel of different rows hit
    // different banks)
    __shared__ __attribute__((aligned(16))) float qs[SC_TM][SC_DI + 4];
    __shared__ uint32_t cbase[SC_TM], cnum[SC_TM], cpre[SC_TM + 1];
    __shared__ uint32_t nvmax_s;
    const int t = threadIdx.x, lane = t & 63;
    const int b = blockIdx.z;
    const int q0 = blockIdx.y * SC_TM;
    const int64_t ew = (int64_t)blockIdx.x * SC_TN * SC_SUB;
    if (t == 0) nvmax_s = 0u;
    __syncthreads();
    // the same visible range as the screening passes (their early exit)
    uint32_t nvl = 0;
    if (t < SC_TM && q0 + t < p.Q) nvl = (uint32_t)min(max(p.n_vis[(int64_t)b * p.Q + q0 + t], 0), p.n_max);
    nvl = wave_umax(nvl);
    if (lane == 0) atomicMax(&nvmax_s, nvl);
    __syncthreads();
    if (ew >= (int64_t)nvmax_s) return;
    if (t < SC_TM) {
        uint2 sg = make_uint2(0u, 0u);
        if (q0 + t < p.Q) {
            const int64_t r = (int64_t)b * p.Q + q0 + t;
            sg = p.seg[r * p.nwx + blockIdx.x];
            const uint32_t cap = (uint32_t)SC_CAP;
            sg.y = sg.x < cap ? min(sg.y, cap - sg.x) : 0u;  // slots past the buffer are not kept
        }
        cbase[t] = sg.x;
        cnum[t] = sg.y;
    }
    // the rows' qbar (rows past Q: zeros, never used)
    for (int i = t; i < SC_TM * SC_DI / 4; i += RS_NT) {
        const int rl = i / (SC_DI / 4), c4 = i % (SC_DI / 4);
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (q0 + rl < p.Q) v = reinterpret_cast<const float4*>(p.qbf + ((int64_t)b * p.Q + q0 + rl) * SC_DI)[c4];
        *reinterpret_cast<float4*>(&qs[rl][4 * c4]) = v;
    }
    __syncthreads();
    if (t < 64) {
        // exclusive prefix of the counts (two per lane)
        const uint32_t a = cnum[2 * t], c = cnum[2 * t + 1];
        const uint32_t incl = wave_incl_scan(a + c);
        cpre[2 * t] = incl - a - c;
        cpre[2 * t + 1] = incl - c;
        if (t == 63) cpre[SC_TM] = incl;
    }
    __syncthreads();
    const uint32_t total = cpre[SC_TM];
    // flat index pi -> (row, slot, entry); the next one's lookup and entry load
    // are issued before the current one is scored
    auto locate = [&](uint32_t pi, int& rl, uint32_t& slot, int32_t& e) {
        int lo = 0, hi = SC_TM - 1;  // the last rl with cpre[rl] <= pi
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (cpre[mid] <= pi) lo = mid; else hi = mid - 1;
        }
        rl = lo;
        slot = cbase[rl] + (pi - cpre[rl]);
        e = p.cand[((int64_t)b * p.Q + q0 + rl) * SC_CAP + slot];
    };
    uint32_t pi = t;
    if (pi >= total) return;
    int rl;
    uint32_t slot;
    int32_t e;
    locate(pi, rl, slot, e);
#pragma unroll 1
    while (true) {
        const uint32_t pn = pi + RS_NT;
        int rl_n = 0;
        uint32_t slot_n = 0;
        int32_t e_n = 0;
        if (pn < total) locate(pn, rl_n, slot_n, e_n);
        const int64_t r = (int64_t)b * p.Q + q0 + rl;
        p.cscore[r * SC_CAP + slot] = exact_score(p, b, e, qs[rl]);
        if (pn >= total) break;
        pi = pn;
        rl = rl_n;
        slot = slot_n;
        e = e_n;
    }
}

// ---- 4: the exact selection among the scored candidates, one wave per row
// (up to SC_WCAP candidates, SC_WCAP / 64 per lane).  The K-th largest
// composite key is found bit by bit (the score key, then the position among
// equal scores), and the selected positions leave in ascending order through
// a per-wave bitmap of the row's positions.  Rows with more candidates, or
// whose candidates fail the count check, are queued for the workgroup
// selection.
constexpr int SC_WE = SC_WCAP / 64;
__global__ __launch_bounds__(256) void sc_select_wave_kernel(ScreenParams p) {
    __shared__ uint32_t bm[4][SC_MAXN / 32];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t r = (int64_t)blockIdx.x * 4 + w;
    if (r >= p.rows) return;
    const int nv = min(max(p.n_vis[r], 0), p.n_max);
    const uint32_t cnt = p.ccnt[r];
    const float tau = p.tau[r];
    if (cnt > (uint32_t)SC_WCAP) {
        if (lane == 0) p.slow[2 + atomicAdd(&p.slow[0], 1u)] = (uint32_t)r;
        return;
    }
    const uint32_t ktau = tau == -INFINITY ? 0u : key32(tau);
    // (loads unconditional: a slot past the count reads slot 0, masked after;
    // a conditional load would make the compiler wait for it at once)
    uint32_t key[SC_WE], pos[SC_WE];
    float sc[SC_WE];
#pragma unroll
    for (int e = 0; e < SC_WE; ++e) {
        const uint32_t i = (uint32_t)(lane + 64 * e);
        const uint32_t ic = i < cnt ? i : 0u;
        pos[e] = (uint32_t)p.cand[r * SC_CAP + ic];
        sc[e] = p.cscore[r * SC_CAP + ic];
    }
    uint32_t nval = 0, nge = 0;
#pragma unroll
    for (int e = 0; e < SC_WE; ++e) {
        key[e] = (uint32_t)(lane + 64 * e) < cnt ? key32(sc[e]) : 0u;
        nval += key[e] != 0u;
        nge += key[e] != 0u && key[e] >= ktau;
    }
    nval = wave_sum(nval);
    nge = wave_sum(nge);
    const bool ok = tau == -INFINITY ? cnt == (uint32_t)nv : nge >= (uint32_t)p.K;
    if (!ok) {
        if (lane == 0) p.slow[2 + atomicAdd(&p.slow[0], 1u)] = (uint32_t)r;
        return;
    }
    // threshold: score key v, and among keys == v the positions <= pv
    uint32_t v = 0u, pv = 0xFFFFFFFFu;
    const uint32_t K = (uint32_t)p.K;
    if (nval > K) {
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t c = v | (1u << bit);
            uint32_t n = 0;
#pragma unroll
            for (int e = 0; e < SC_WE; ++e) n += key[e] >= c;
            if (wave_sum(n) >= K) v = c;
        }
        uint32_t above = 0, eq = 0;
#pragma unroll
        for (int e = 0; e < SC_WE; ++e) {
            above += key[e] > v;
            eq += key[e] == v;
        }
        above = wave_sum(above);
        eq = wave_sum(eq);
        const uint32_t need = K - above;  // 1 <= need <= eq
        if (need < eq) {
            // the smallest pv with #{key == v, pos <= pv} >= need (bit by bit
            // from the top: keep a bit clear while enough positions lie below)
            pv = 0u;
            for (int bit = 31; bit >= 0; --bit) {
                const uint32_t c = pv | ((1u << bit) - 1u);
                uint32_t n = 0;
#pragma unroll
                for (int e = 0; e < SC_WE; ++e) n += key[e] == v && pos[e] <= c;
                if (wave_sum(n) < need) pv |= 1u << bit;
            }
        }
    }
    // selected positions into the bitmap, then out in ascending order
    uint32_t* bmw = bm[w];
    const int nwords = (p.n_max + 31) / 32;
    for (int i = lane; i < nwords; i += 64) bmw[i] = 0u;
    wave_lds_sync();
#pragma unroll
    for (int e = 0; e < SC_WE; ++e)
        if (key[e] != 0u && (key[e] > v || (key[e] == v && pos[e] <= pv)))
            atomicOr(&bmw[pos[e] >> 5], 1u << (pos[e] & 31));
    wave_lds_sync();
    // lane l owns words l * per .. l * per + per - 1
    const int per = (nwords + 63) / 64;
    uint32_t mine = 0;
    for (int i = 0; i < per; ++i) {
        const int wi = lane * per + i;
        if (wi < nwords) mine += (uint32_t)__popc(bmw[wi]);
    }
    const uint32_t incl = wave_incl_scan(mine);
    uint32_t at = incl - mine;
    const uint32_t total = __shfl(incl, 63);
    int32_t* orow = p.out + r * p.K;
    for (int i = 0; i < per; ++i) {
        const int wi = lane * per + i;
        if (wi >= nwords) break;
        uint32_t bits = bmw[wi];
        while (bits) {
            const int bit = __builtin_ctz(bits);
            bits &= bits - 1u;
            if (at < K) orow[at] = wi * 32 + bit;
            ++at;
        }
    }
    for (uint32_t i = total + lane; i < K; i += 64) orow[i] = -1;
}

// ---- 5: the queued rows, one workgroup at a time: up to SC_CAP scored
// candidates selected by radix passes, or (more candidates,
// or a failed count check) every visible entry scored into the row's scratch
// and selected from there.
__global__ __launch_bounds__(WG) void sc_select_wg_kernel(ScreenParams p) {
    __shared__ SelectLds sh;
    __shared__ int sel[TOPK_KMAX];
    __shared__ int tmp[TOPK_KMAX];
    __shared__ __attribute__((aligned(16))) float qb[SC_DI];
    __shared__ uint32_t s_valid, s_ge, s_row;
    const int t = threadIdx.x;
    const uint32_t queued = p.slow[0];
    for (;;) {
        __syncthreads();
        if (t == 0) s_row = atomicAdd(&p.slow[1], 1u);
        __syncthreads();
        const uint32_t qi = s_row;
        if (qi >= queued) break;
        const int64_t r = p.slow[2 + qi];
        const int b = (int)(r / p.Q);
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
            uint32_t nvalid = 0, nge = 0;
#pragma unroll
            for (int e = 0; e < EC; ++e) {
                const uint32_t i = (uint32_t)(t + WG * e);
                key[e] = i < cnt ? key32(p.cscore[r * SC_CAP + i]) : 0u;
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
        const bool use = screened && (tau == -INFINITY ? cnt == (uint32_t)nv : s_ge >= (uint32_t)p.K);
        uint32_t total;
        if (use) {
            total = min((uint32_t)p.K, s_valid);
            if (s_valid > (uint32_t)p.K) {
                uint64_t prefix = 0, mask = 0;
                select_regs<EC>(key, pos, (uint32_t)p.K, 0, prefix, mask, sh);
#pragma unroll
                for (int e = 0; e < EC; ++e)
                    if (key[e] != 0u && (composite(key[e], pos[e]) & mask) >= prefix)
                        sel[atomicAdd(&sh.nsel, 1u)] = (int)pos[e];
            } else {
#pragma unroll
                for (int e = 0; e < EC; ++e)
                    if (key[e] != 0u) sel[atomicAdd(&sh.nsel, 1u)] = (int)pos[e];
            }
            __syncthreads();
        } else {
            // every visible entry, exactly, into the row's scratch; the
            // selection then runs its radix passes over the scratch
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
    const int64_t nwx = (n_max + SC_TN * SC_SUB - 1) / (SC_TN * SC_SUB);
    return al256(rows * SC_DI * 2) + 3 * al256(rows * 4) + al256(rows * nb16 * 4) + 2 * al256(rows * SC_CAP * 4) +
           al256((rows + 2) * 4) + al256((int64_t)B * n_max * 4) + al256(rows * SC_DI * 4) + al256(rows * nwx * 8) +
           256;
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
    w += al256(rows * SC_CAP * 4);
    p.cscore = reinterpret_cast<float*>(w);
    w += al256(rows * SC_CAP * 4);
    p.slow = reinterpret_cast<uint32_t*>(w);
    w += al256((rows + 2) * 4);
    p.kn = reinterpret_cast<float*>(w);
    w += al256((int64_t)B * n_max * 4);
    p.qbf = reinterpret_cast<float*>(w);
    w += al256(rows * SC_DI * 4);
    p.nwx = (int32_t)((n_max + SC_TN * SC_SUB - 1) / (SC_TN * SC_SUB));
    p.seg = reinterpret_cast<uint2*>(w);
    p.scratch = scratch;
    p.out = out;
    const unsigned row_blocks = (unsigned)((rows + 3) / 4);
    sc_prep_kernel<<<row_blocks, 256, 0, stream>>>(p);
    const dim3 grid((unsigned)((n_max + SC_TN * SC_SUB - 1) / (SC_TN * SC_SUB)), (unsigned)((Q + SC_TM - 1) / SC_TM),
                    (unsigned)B);
    const bool contig = p.kmap.page_table == nullptr;
    if (contig)
        sc_gemm_kernel<1, true><<<grid, 256, 0, stream>>>(p, p.k, p.lb, p.kn);
    else
        sc_gemm_kernel<1, false><<<grid, 256, 0, stream>>>(p, p.k, p.lb, p.kn);
    sc_tau_kernel<<<row_blocks, 256, 0, stream>>>(p);
    if (contig)
        sc_gemm_kernel<2, true><<<grid, 256, 0, stream>>>(p, p.k, p.lb, p.kn);
    else
        sc_gemm_kernel<2, false><<<grid, 256, 0, stream>>>(p, p.k, p.lb, p.kn);
    sc_rescore_kernel<<<grid, RS_NT, 0, stream>>>(p);
    sc_select_wave_kernel<<<row_blocks, 256, 0, stream>>>(p);
    // the queued rows: a few workgroups take them in turn (none: they exit at once)
    sc_select_wg_kernel<<<(unsigned)(rows < 64 ? rows : 64), WG, 0, stream>>>(p);
    return launch_status("screen");
}

}  // namespace csa2
