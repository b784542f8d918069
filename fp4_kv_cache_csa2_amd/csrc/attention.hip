// Sparse FP4 attention + sliding-window attention with one softmax over the
// union of both key sets.  K = V = the latent key vector (one latent shared by
// all query heads).
//  * selected entries: FP4 E2M1 codes x E4M3 scale per 16 channels (aprilzz.com
//    V4.1 Flash article, section "FP4 KV 与部署层的几个改动"), gathered through
//    the Top-K index list;
//  * window: the layer's own bf16 latent rows of the last `window` tokens
//    (aprilzz.com, section "把 prefill 砍掉一半": 128-token SWA in every layer).
//
// One workgroup = one query row x a range of 16-key chunks; wave w owns query
// heads 16w..16w+15 (heads are the MFMA N dimension, keys the M dimension).
// Per chunk the workgroup gathers 16 keys once, dequantises them in registers
// (an E2M1 x E4M3 product has <= 6 significant bits, so it is exact in bf16
// and fp16) into two LDS tiles: K row-major bf16 for S^T = K Q^T
// (v_mfma_f32_16x16x32_bf16) and V^T fp16 for O^T = V^T P^T
// (v_mfma_f32_16x16x16_f16).  The S^T accumulator layout (lane holds keys
// 4g..4g+3 of head lane%16) is exactly the P^T operand layout of the second
// MFMA, so P never leaves registers.  Softmax is online (running max / sum in
// the log2 domain).  Few rows (decode) split the keys over several workgroups
// whose normalised partials (o, lse) are merged by a second kernel.
#include "internal.h"

namespace csa2 {
namespace {

constexpr int CHUNK_KEYS = 16;

struct AttnParams {
    const void* q;             // [rows][H][D]
    int32_t H, Q;
    // selected FP4 entries
    const uint8_t* codes;
    const uint8_t* scales;
    RowMap kvmap;
    const int32_t* idx;        // [rows][K]
    int32_t K, Kp;             // Kp = K rounded up to 16 (0 if no sparse part)
    // window
    const uint16_t* swa;       // [B][T][D]
    int32_t T;
    const int32_t* q_slot;     // [rows]
    int32_t window, Wp;        // Wp = window rounded up to 16 (0 if no window part)
    float scale_log2;          // sm_scale * log2(e)
    int32_t merge;
    float* o;                  // [rows][H][D]
    float* lse;                // [rows][H]
    int32_t nsplit, cps;       // splits per row, chunks per split
    float* part_o;             // [rows][nsplit][H][D]
    float* part_lse;           // [rows][nsplit][H]
};

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float e4m3_val(uint32_t code) {
    uint32_t e = (code >> 3) & 15, m = code & 7;
    if (e == 0) return (float)m * 0.001953125f;
    return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

__device__ __forceinline__ float e2m1_val(uint32_t code) {
    uint32_t mag = code & 7u;
    float a = (mag < 2u) ? 0.5f * (float)mag : __uint_as_float(((mag >> 1) + 126u) << 23 | (mag & 1u) << 22);
    return (code & 8u) ? -a : a;
}

// byte offset of V^T[d][key 4kq] inside the padded transposed tile
__device__ __forceinline__ int vt_off(int d, int kq) { return d * 32 + (d >> 3) * 16 + kq * 8; }

constexpr int MAX_CPS = 64;  // chunks per split (keys per workgroup <= 1024)

// Raw data of one dequantisation item (4 keys x 8 channels): FP4 code words and
// scale bytes, or 4 x 8 bf16 window channels.
struct RawItem {
    uint4 w[4];
};

template <int D>
__device__ __forceinline__ void load_item(const AttnParams& p, bool sparse, const int64_t* krow, int kq, int co,
                                          RawItem& raw) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t r = krow[4 * kq + i];
        if (r < 0) {
            raw.w[i] = make_uint4(0, 0, 0, 0);
        } else if (sparse) {
            raw.w[i].x = *reinterpret_cast<const uint32_t*>(p.codes + r * (D / 2) + co * 4);
            raw.w[i].y = p.scales[r * (D / 16) + (co >> 1)];
        } else {
            raw.w[i] = *reinterpret_cast<const uint4*>(p.swa + r * D + co * 8);
        }
    }
}

// Dequantise one item into the K tile (bf16, row-major, swizzled) and the V^T
// tile (fp16, transposed, padded).
template <int D>
__device__ __forceinline__ void store_item(bool sparse, const RawItem& raw, int kq, int co, uint4* ktile,
                                           uint8_t* vtile) {
    constexpr int CPR = D / 8;
    uint32_t kb16[4][4];
    uint16_t vh[8][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float v[8];
        if (sparse) {
            const uint32_t cw = raw.w[i].x;
            const float s = e4m3_val(raw.w[i].y);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = e2m1_val((cw >> (4 * e)) & 15u) * s;
        } else {
            const uint32_t wv[4] = {raw.w[i].x, raw.w[i].y, raw.w[i].z, raw.w[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[2 * e] = bf16_lo(wv[e]);
                v[2 * e + 1] = bf16_hi(wv[e]);
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            kb16[i][e] = (__float_as_uint(v[2 * e]) >> 16) | (__float_as_uint(v[2 * e + 1]) & 0xFFFF0000u);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const _Float16 h = (_Float16)v[e];
            vh[e][i] = *reinterpret_cast<const uint16_t*>(&h);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int key = 4 * kq + i;
        ktile[key * CPR + (co ^ (key & 15))] = make_uint4(kb16[i][0], kb16[i][1], kb16[i][2], kb16[i][3]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int d = 8 * co + e;
        *reinterpret_cast<uint2*>(vtile + vt_off(d, kq)) =
            make_uint2((uint32_t)vh[e][0] | ((uint32_t)vh[e][1] << 16), (uint32_t)vh[e][2] | ((uint32_t)vh[e][3] << 16));
    }
}

template <int D, bool QF32, int NW>
__global__ __launch_bounds__(64 * NW) void attn_kernel(AttnParams p) {
    constexpr int NBLK = D / 32;  // 32-channel blocks of the S MFMA
    constexpr int NDT = D / 16;   // 16-channel tiles of the O MFMA
    constexpr int CPR = D / 8;    // 16-byte chunks per bf16 key row
    constexpr int NT = 64 * NW;
    constexpr int ITEMS = 4 * CPR;                       // dequantisation items per chunk
    constexpr int IPT = (ITEMS + NT - 1) / NT;           // items per thread
    __shared__ uint4 ktile[CHUNK_KEYS * CPR];
    __shared__ __attribute__((aligned(16))) uint8_t vtile[D * 32 + (D / 8) * 16];
    __shared__ int64_t krow[MAX_CPS * CHUNK_KEYS];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int64_t row = blockIdx.y;
    const int split = blockIdx.x;
    const int b = (int)(row / p.Q);
    const int head = 16 * w + c16;

    const int nchunks = (p.Kp + p.Wp) / CHUNK_KEYS;
    const int c_lo = split * p.cps;
    const int c_hi = min(nchunks, c_lo + p.cps);
    const int slot = p.Wp ? p.q_slot[row] : 0;
    const int wlo = max(0, slot - p.window + 1);

    // ---- physical rows of every key of this split (-1: none)
    const int nk = max(0, c_hi - c_lo) * CHUNK_KEYS;
    for (int i = tid; i < nk; i += NT) {
        const int kpos = c_lo * CHUNK_KEYS + i;
        int64_t r = -1;
        if (kpos < p.Kp) {
            if (kpos < p.K) {
                const int32_t e = p.idx[row * p.K + kpos];
                if (e >= 0) r = phys_row(p.kvmap, b, e);
            }
        } else {
            const int t = wlo + (kpos - p.Kp);
            if (t <= slot && t < p.T) r = (int64_t)b * p.T + t;
        }
        krow[i] = r;
    }

    // ---- Q operand (B of S^T = K Q^T): Q[head][32*blk + 8g .. +8]
    bf16x8 qhi[NBLK];
    bf16x8 qlo[QF32 ? NBLK : 1];
    if (QF32) {
        const float* qr = static_cast<const float*>(p.q) + (row * p.H + head) * D;
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk) {
            const float4 a = *reinterpret_cast<const float4*>(qr + 32 * blk + 8 * g);
            const float4 c = *reinterpret_cast<const float4*>(qr + 32 * blk + 8 * g + 4);
            const float xs[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
            uint16_t hi[8], lo[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t h = f32_to_bf16_rne(xs[i]);
                hi[i] = (uint16_t)h;
                lo[i] = (uint16_t)f32_to_bf16_rne(xs[i] - __uint_as_float(h << 16));
            }
            qhi[blk] = *reinterpret_cast<const bf16x8*>(hi);
            qlo[QF32 ? blk : 0] = *reinterpret_cast<const bf16x8*>(lo);
        }
    } else {
        const uint16_t* qr = static_cast<const uint16_t*>(p.q) + (row * p.H + head) * D;
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk)
            qhi[blk] = *reinterpret_cast<const bf16x8*>(qr + 32 * blk + 8 * g);
    }
    __syncthreads();

    f32x4 oacc[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;

    RawItem raw[IPT];
    if (c_lo < c_hi) {
        const bool sp = c_lo * CHUNK_KEYS < p.Kp;
#pragma unroll
        for (int it = 0; it < IPT; ++it) {
            const int item = it * NT + tid;
            if (item < ITEMS) load_item<D>(p, sp, krow, item / CPR, item % CPR, raw[it]);
        }
    }
    for (int ch = c_lo; ch < c_hi; ++ch) {
        const int kb = ch * CHUNK_KEYS;
        const bool sparse = kb < p.Kp;
        const int64_t* kr = krow + (ch - c_lo) * CHUNK_KEYS;
        // ---- dequantise the prefetched chunk into the LDS tiles
#pragma unroll
        for (int it = 0; it < IPT; ++it) {
            const int item = it * NT + tid;
            if (item < ITEMS) store_item<D>(sparse, raw[it], item / CPR, item % CPR, ktile, vtile);
        }
        __syncthreads();
        // ---- the next chunk's loads fly during this chunk's MFMAs
        if (ch + 1 < c_hi) {
            const bool sp = (ch + 1) * CHUNK_KEYS < p.Kp;
#pragma unroll
            for (int it = 0; it < IPT; ++it) {
                const int item = it * NT + tid;
                if (item < ITEMS) load_item<D>(p, sp, kr + CHUNK_KEYS, item / CPR, item % CPR, raw[it]);
            }
        }
        // ---- S^T[key][head] = sum_d K[key][d] Q[head][d]
        f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk) {
            const uint4 a4 = ktile[c16 * CPR + ((4 * blk + g) ^ c16)];
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(&a4);
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qhi[blk], s, 0, 0, 0);
            if (QF32) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qlo[QF32 ? blk : 0], s, 0, 0, 0);
        }
        // ---- online softmax for head `head` over keys 4g..4g+3 of this chunk
        float z[4];
        float mloc = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            z[i] = (kr[4 * g + i] >= 0) ? s[i] * p.scale_log2 : -INFINITY;
            mloc = fmaxf(mloc, z[i]);
        }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        const float m_new = fmaxf(m_run, mloc);
        const float alpha = (m_new == -INFINITY) ? 1.0f : exp2f(m_run - m_new);
        float psum = 0.0f;
        uint16_t ph[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float pi = (z[i] == -INFINITY) ? 0.0f : exp2f(z[i] - m_new);
            const _Float16 h = (_Float16)pi;
            psum += (float)h;  // normalise by the weights the MFMA actually applies
            ph[i] = *reinterpret_cast<const uint16_t*>(&h);
        }
        psum += __shfl_xor(psum, 16);
        psum += __shfl_xor(psum, 32);
        l_run = l_run * alpha + psum;
        m_run = m_new;
        const f16x4 pb = *reinterpret_cast<const f16x4*>(ph);
        // ---- O^T[d][head] = alpha * O^T + sum_key V^T[d][key] P^T[key][head]
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const uint2 a2 = *reinterpret_cast<const uint2*>(vtile + vt_off(16 * dt + c16, g));
            const f16x4 a = *reinterpret_cast<const f16x4*>(&a2);
            f32x4 acc = oacc[dt] * alpha;
            oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, pb, acc, 0, 0, 0);
        }
        __syncthreads();
    }

    // ---- normalised partial (o, lse) of this workgroup's key range
    const float inv = (l_run > 0.0f) ? 1.0f / l_run : 0.0f;
    const float lse_cur = (l_run > 0.0f) ? (m_run + log2f(l_run)) * 0.69314718055994531f : -INFINITY;
    if (p.nsplit > 1) {
        float* po = p.part_o + ((row * p.nsplit + split) * p.H + head) * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
            *reinterpret_cast<float4*>(po + 16 * dt + 4 * g) =
                make_float4(oacc[dt][0] * inv, oacc[dt][1] * inv, oacc[dt][2] * inv, oacc[dt][3] * inv);
        if (g == 0) p.part_lse[(row * p.nsplit + split) * p.H + head] = lse_cur;
        return;
    }
    float* orow = p.o + (row * p.H + head) * D;
    float w_cur = 1.0f, w_old = 0.0f, lse_out = lse_cur;
    if (p.merge) {
        const float lse_old = p.lse[row * p.H + head];
        const float L = fmaxf(lse_old, lse_cur);
        if (L == -INFINITY) {
            w_cur = 0.0f;
            w_old = 0.0f;
            lse_out = -INFINITY;
        } else {
            w_old = expf(lse_old - L);
            w_cur = expf(lse_cur - L);
            const float tot = w_old + w_cur;
            w_old /= tot;
            w_cur /= tot;
            lse_out = L + logf(tot);
        }
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
        float4* dst = reinterpret_cast<float4*>(orow + 16 * dt + 4 * g);
        float4 r = make_float4(oacc[dt][0] * inv * w_cur, oacc[dt][1] * inv * w_cur, oacc[dt][2] * inv * w_cur,
                               oacc[dt][3] * inv * w_cur);
        if (p.merge && w_old != 0.0f) {
            const float4 old = *dst;
            r.x += w_old * old.x;
            r.y += w_old * old.y;
            r.z += w_old * old.z;
            r.w += w_old * old.w;
        }
        *dst = r;
    }
    if (g == 0) p.lse[row * p.H + head] = lse_out;
}

// Merge the split partials of one (row, head): exact log-sum-exp combination,
// optionally together with the (o, lse) already in the output.  All loads are
// issued before any arithmetic.
template <int NS>
__global__ __launch_bounds__(128) void attn_merge_kernel(const float* __restrict__ part_o,
                                                         const float* __restrict__ part_lse, int nsplit, int H, int D,
                                                         int merge, float* __restrict__ o, float* __restrict__ lse) {
    const int64_t row = blockIdx.x;
    const int h = blockIdx.y;
    const int c = threadIdx.x * 4;
    float ls[NS + 1];
    float4 ov[NS + 1];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        ls[s] = s < nsplit ? part_lse[(row * nsplit + s) * H + h] : -INFINITY;
        ov[s] = s < nsplit ? *reinterpret_cast<const float4*>(part_o + ((row * nsplit + s) * H + h) * D + c)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    ls[NS] = merge ? lse[row * H + h] : -INFINITY;
    ov[NS] = merge ? *reinterpret_cast<const float4*>(o + (row * H + h) * D + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    float L = -INFINITY;
#pragma unroll
    for (int s = 0; s <= NS; ++s) L = fmaxf(L, ls[s]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float tot = 0.0f;
    if (L != -INFINITY) {
#pragma unroll
        for (int s = 0; s <= NS; ++s) {
            const float wv = (ls[s] == -INFINITY) ? 0.0f : expf(ls[s] - L);
            acc.x += wv * ov[s].x;
            acc.y += wv * ov[s].y;
            acc.z += wv * ov[s].z;
            acc.w += wv * ov[s].w;
            tot += wv;
        }
    }
    const float inv = tot > 0.0f ? 1.0f / tot : 0.0f;
    __syncthreads();  // every thread has read the old o/lse before any is overwritten
    *reinterpret_cast<float4*>(o + (row * H + h) * D + c) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    if (threadIdx.x == 0) lse[row * H + h] = tot > 0.0f ? L + logf(tot) : -INFINITY;
}

constexpr int MAX_SPLIT = 16;

int choose_nsplit(int64_t rows, int nchunks) {
    if (nchunks <= 1) return 1;
    int64_t want = (512 + rows - 1) / rows;  // aim at >= 512 workgroups
    int64_t by_chunks = (nchunks + 1) / 2;   // at least two chunks per split
    int64_t s = want < by_chunks ? want : by_chunks;
    if (s > MAX_SPLIT) s = MAX_SPLIT;
    if (s < 1) s = 1;
    return (int)s;
}

size_t attn_ws_bytes(int64_t rows, int H, int D) {
    int64_t s = (512 + rows - 1) / rows;
    if (s > MAX_SPLIT) s = MAX_SPLIT;
    if (s <= 1) return 0;
    return (size_t)(rows * s * H) * (size_t)(D + 1) * 4 + 256;
}

}  // namespace

// Shared launcher of the sparse-only, window-only and fused calls.
csa2_status attn_launch(const void* q, csa2_dtype qt, int32_t B, int32_t Q, int32_t H, int32_t D,
                        const csa2_fp4_kv* kv, const int32_t* idx, int32_t K, const uint16_t* swa, int32_t T,
                        const int32_t* q_slot, int32_t window, float sm_scale, int32_t merge, float* o, float* lse,
                        void* ws, size_t ws_bytes, hipStream_t stream, const char* what) {
    CSA2_ARG(B >= 0 && Q >= 0, "%s: B=%d Q=%d must be >= 0", what, B, Q);
    CSA2_ARG((int64_t)B * Q <= 65535, "%s: B*Q=%lld rows exceeds 65535", what, (long long)B * Q);
    CSA2_ARG(qt == CSA2_F32 || qt == CSA2_BF16, "%s: bad q dtype %d", what, (int)qt);
    CSA2_REQUIRE(H >= 16 && H <= 64 && H % 16 == 0, CSA2_EUNSUPPORTED, "%s: H=%d (supported: 16, 32, 48, 64)", what,
                 H);
    CSA2_REQUIRE(D == 128 || D == 256 || D == 512, CSA2_EUNSUPPORTED, "%s: D=%d (supported: 128, 256, 512)", what, D);
    CSA2_ARG(K >= 0 && K <= 65536, "%s: K=%d out of range", what, K);
    CSA2_ARG(window >= 0 && window <= 65536, "%s: window=%d out of range", what, window);
    const int64_t rows = (int64_t)B * Q;
    if (rows == 0) return CSA2_OK;
    CSA2_ARG(q && o && lse, "%s: null q/o/lse", what);
    CSA2_ARG(aligned(q, 16) && aligned(o, 16), "%s: q and o must be 16-byte aligned", what);
    AttnParams p{};
    if (K > 0) {
        CSA2_ARG(kv && kv->codes && kv->scales && idx, "%s: null cache view or idx", what);
        CSA2_ARG(kv->D == D, "%s: cache D=%d differs from D=%d", what, kv->D, D);
        CSA2_ARG(aligned(kv->codes, 4), "%s: codes must be 4-byte aligned", what);
        csa2_status st = make_rowmap(kv->page_table, kv->page_size, kv->max_pages, kv->seq_stride, 1, &p.kvmap, what);
        if (st != CSA2_OK) return st;
        p.codes = kv->codes;
        p.scales = kv->scales;
    }
    if (window > 0) {
        CSA2_ARG(swa && q_slot && T > 0, "%s: null window rows / q_slot or T <= 0", what);
        CSA2_ARG(aligned(swa, 16), "%s: window rows must be 16-byte aligned", what);
    }
    p.q = q;
    p.H = H;
    p.Q = Q;
    p.idx = idx;
    p.K = K;
    p.Kp = (K + CHUNK_KEYS - 1) / CHUNK_KEYS * CHUNK_KEYS;
    p.swa = swa;
    p.T = T;
    p.q_slot = q_slot;
    p.window = window;
    p.Wp = (window + CHUNK_KEYS - 1) / CHUNK_KEYS * CHUNK_KEYS;
    p.scale_log2 = sm_scale * 1.4426950408889634f;
    p.merge = merge ? 1 : 0;
    p.o = o;
    p.lse = lse;
    const int nchunks = (p.Kp + p.Wp) / CHUNK_KEYS;
    p.nsplit = choose_nsplit(rows, nchunks);
    p.cps = nchunks > 0 ? (nchunks + p.nsplit - 1) / p.nsplit : 0;
    CSA2_REQUIRE(p.cps <= MAX_CPS, CSA2_EUNSUPPORTED, "%s: %d keys per query need more than %d splits", what,
                 nchunks * CHUNK_KEYS, MAX_SPLIT);
    if (p.nsplit > 1) {
        const size_t need = (size_t)(rows * p.nsplit * H) * (size_t)(D + 1) * 4;
        CSA2_REQUIRE(ws != nullptr && ws_bytes >= need, CSA2_EWORKSPACE,
                     "%s: workspace of %zu bytes required, %zu given", what, need, ws ? ws_bytes : (size_t)0);
        CSA2_ARG(((uintptr_t)ws & 15) == 0, "%s: workspace must be 16-byte aligned", what);
        p.part_o = static_cast<float*>(ws);
        p.part_lse = p.part_o + rows * p.nsplit * H * (int64_t)D;
    }
    const dim3 grid((unsigned)p.nsplit, (unsigned)rows);
    const dim3 block((unsigned)(4 * H));
    const bool f32 = qt == CSA2_F32;
    const int nw = H / 16;
#define CSA2_ATTN_NW(DD, F, NWV) \
    if (nw == NWV) attn_kernel<DD, F, NWV><<<grid, block, 0, stream>>>(p);
#define CSA2_ATTN(DD)                                                                                   \
    if (D == DD) {                                                                                      \
        if (f32) {                                                                                      \
            CSA2_ATTN_NW(DD, true, 1) CSA2_ATTN_NW(DD, true, 2) CSA2_ATTN_NW(DD, true, 3)               \
            CSA2_ATTN_NW(DD, true, 4)                                                                   \
        } else {                                                                                        \
            CSA2_ATTN_NW(DD, false, 1) CSA2_ATTN_NW(DD, false, 2) CSA2_ATTN_NW(DD, false, 3)            \
            CSA2_ATTN_NW(DD, false, 4)                                                                  \
        }                                                                                               \
    }
    CSA2_ATTN(128)
    CSA2_ATTN(256)
    CSA2_ATTN(512)
#undef CSA2_ATTN
#undef CSA2_ATTN_NW
    if (p.nsplit > 1) {
        const dim3 mg((unsigned)rows, (unsigned)H), mb((unsigned)(D / 4));
        if (p.nsplit <= 4)
            attn_merge_kernel<4><<<mg, mb, 0, stream>>>(p.part_o, p.part_lse, p.nsplit, H, D, p.merge, o, lse);
        else if (p.nsplit <= 8)
            attn_merge_kernel<8><<<mg, mb, 0, stream>>>(p.part_o, p.part_lse, p.nsplit, H, D, p.merge, o, lse);
        else
            attn_merge_kernel<MAX_SPLIT><<<mg, mb, 0, stream>>>(p.part_o, p.part_lse, p.nsplit, H, D, p.merge, o,
                                                                lse);
    }
    return launch_status(what);
}

size_t attn_workspace_bytes(int64_t rows, int H, int D) { return attn_ws_bytes(rows, H, D); }

}  // namespace csa2

using namespace csa2;

extern "C" size_t csa2_attn_workspace_size(int32_t B, int32_t Q, int32_t H, int32_t D) {
    if (B <= 0 || Q <= 0 || H <= 0 || D <= 0) return 0;
    return attn_ws_bytes((int64_t)B * Q, H, D);
}

extern "C" csa2_status csa2_sparse_attn_fp4(const void* q, csa2_dtype qt, int32_t B, int32_t Q, int32_t H,
                                            const csa2_fp4_kv* kv, const int32_t* idx, int32_t K, float sm_scale,
                                            float* o, float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
    clear_error();
    CSA2_ARG(kv != nullptr, "sparse_attn_fp4: null cache view");
    return attn_launch(q, qt, B, Q, H, kv->D, kv, idx, K, nullptr, 0, nullptr, 0, sm_scale, 0, o, lse, ws, ws_bytes,
                       stream, "sparse_attn_fp4");
}

extern "C" csa2_status csa2_swa_attn(const void* q, csa2_dtype qt, int32_t B, int32_t Q, int32_t H, int32_t D,
                                     const uint16_t* swa_kv, int32_t T, const int32_t* q_slot, int32_t window,
                                     float sm_scale, int32_t merge, float* o, float* lse, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
    clear_error();
    CSA2_ARG(window >= 1, "swa_attn: window=%d must be >= 1", window);
    return attn_launch(q, qt, B, Q, H, D, nullptr, nullptr, 0, swa_kv, T, q_slot, window, sm_scale, merge, o, lse, ws,
                       ws_bytes, stream, "swa_attn");
}
