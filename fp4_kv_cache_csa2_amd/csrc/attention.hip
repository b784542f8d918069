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
// Per chunk the workgroup gathers 16 keys once and dequantises them in
// registers into two fp16 LDS tiles: K row-major for S^T = K Q^T
// (v_mfma_f32_16x16x32_f16) and V^T for O^T = V^T P^T
// (v_mfma_f32_16x16x16_f16).  An E2M1 x E4M3 product has <= 6 significant
// bits and lies in [2^-10, 2688], so it is exact in fp16; the E2M1 values come
// from a byte-permute table.  The query is pre-scaled per head by a power of
// two so that its largest element sits in [2^14, 2^15) (exact), and the scale
// is folded into the logit scale.  The S^T accumulator layout (lane holds keys
// 4g..4g+3 of head lane%16) is exactly the P^T operand layout of the second
// MFMA, so P never leaves registers.  Softmax is online in the log2 domain with
// a lazy maximum: the running maximum moves (and O is rescaled) only when a
// chunk exceeds it by more than 2^8, so P <= 256 stays well inside fp16.  Few
// rows (decode) split the keys over several workgroups whose normalised
// partials (o, lse) are merged by a second kernel.
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
    // split partials, unnormalised: o in MFMA lane order per 16-head group,
    // [rows][nsplit][H/16][D/16][64 lanes][4]; running max (log2 domain) and sum
    float* part_o;
    float2* part_ml;           // [rows][nsplit][H]
    float* lse_prev;           // [rows][H]: the output's lse before a merge
};

// E2M1 magnitude x 2^8 -> high byte of its fp16 value (the low byte is 0):
// magnitudes 0, 0.5, 1, 1.5 | 2, 3, 4, 6, times 256
constexpr uint32_t F16HI_LO = 0x5E5C5800u, F16HI_HI = 0x66646260u;

// E4M3FN scale byte -> fp16 bits of scale x 2^-8, twice (exact: E4M3 and fp16
// share the mantissa alignment, so the byte shifted into the fp16 exponent /
// mantissa fields is the scale with its exponent bias off by 8; subnormal
// scales land on fp16 subnormals).
__device__ __forceinline__ uint32_t e4m3_f16x2_over256(uint32_t code) { return (code << 7) | (code << 23); }

// 8 FP4 codes (one 32-bit word, channel 2i in the low nibble of byte i) times
// the scale -> four fp16 pairs (channels 2i, 2i+1).  (E2M1 x 2^8) x (E4M3 x
// 2^-8) is exact: <= 6 significant bits in [2^-10, 2688].
__device__ __forceinline__ void fp4x8_to_f16(uint32_t w, uint32_t sc2, uint32_t (&out)[4]) {
    const uint32_t ev = w & 0x07070707u;         // magnitudes of channels 0, 2, 4, 6
    const uint32_t od = (w >> 4) & 0x07070707u;  // magnitudes of channels 1, 3, 5, 7
    const uint32_t hbe = __builtin_amdgcn_perm(F16HI_HI, F16HI_LO, ev) | ((w << 4) & 0x80808080u);
    const uint32_t hbo = __builtin_amdgcn_perm(F16HI_HI, F16HI_LO, od) | (w & 0x80808080u);
    const uint32_t sel[4] = {0x040C000Cu, 0x050C010Cu, 0x060C020Cu, 0x070C030Cu};
    const f16x2 sc = *reinterpret_cast<const f16x2*>(&sc2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t pr = __builtin_amdgcn_perm(hbo, hbe, sel[i]);
        const f16x2 v = *reinterpret_cast<const f16x2*>(&pr) * sc;
        out[i] = *reinterpret_cast<const uint32_t*>(&v);
    }
}

// byte offset of V^T[d][key 4kq] inside the padded transposed tile (rows of
// 16 keys x fp16 = 32 B, plus 16 B after every 8 rows against bank conflicts)
__device__ __forceinline__ int vt_off(int d, int kq) { return d * 32 + (d >> 3) * 16 + kq * 8; }
// the same for d = 16 dt + c16 (c16 < 16), split so that dt becomes an immediate offset
__device__ __forceinline__ int vt_base(int c16, int kq) { return c16 * 32 + (c16 >> 3) * 16 + kq * 8; }
constexpr int VT_DT = 16 * 32 + 2 * 16;  // bytes per 16 rows

constexpr int MAX_CPS = 64;  // chunks per split (keys per workgroup <= 1024)
constexpr int RING = 4;      // chunks whose raw bytes are in flight / staged in LDS at once
// (many rows, no key split: a 2-chunk ring lets two workgroups share a CU,
// so one's dequantisation and barriers overlap the other's MFMAs)
constexpr int RING_WIDE = 2;

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* global_void_ptr;

// Asynchronous global -> LDS copies (LDS DMA): lane l of the wave writes its
// 16 (4) bytes at lds_base + 16 l (4 l); the wave's vmcnt counts the copy until
// it lands.
__device__ __forceinline__ void dma16_to_lds(const void* src, void* lds_base) {
    __builtin_amdgcn_global_load_lds((global_void_ptr)(const_cast<void*>(src)), (lds_void_ptr)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void dma4_to_lds(const void* src, void* lds_base) {
    __builtin_amdgcn_global_load_lds((global_void_ptr)(const_cast<void*>(src)), (lds_void_ptr)lds_base, 4, 0, 0);
}

// Workgroup barrier for LDS traffic only.  __syncthreads() would also wait for
// every outstanding LDS copy (they count as vector memory), including the ring
// refills still in flight; here only this wave's LDS instructions are drained
// (lgkmcnt 0), copies the caller needs are waited for explicitly, and the
// compiler may not move memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt: no wait
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Raw bytes of one 16-key chunk in an LDS ring slot.  Selected entries: the
// FP4 code rows [16][D/2] then the scale rows [16][D/16]; window: the bf16
// rows [16][D].  Copies per chunk (one wave instruction each, spread over the
// waves round-robin): codes D/128 x 16 B/lane, scales ceil(D/256) x 4 B/lane;
// window D/32 x 16 B/lane.
template <int D>
struct Stage {
    static constexpr int SLOT = CHUNK_KEYS * 2 * D;
    static constexpr int SCALE_OFF = CHUNK_KEYS * D / 2;
    static constexpr int N_CODE = D / 128;
    static constexpr int N_SCALE = (D + 255) / 256;
    static constexpr int N_WIN = D / 32;
};

// A key without a row copies row 0 instead: its values are finite and its
// softmax weight is exactly 0, so it adds nothing.
template <int D, int NW>
__device__ __forceinline__ void stage_chunk(const AttnParams& p, bool sparse, const int64_t* kr, uint8_t* slot, int w,
                                            int lane) {
    using S = Stage<D>;
    if (sparse) {
        constexpr int PPK = D / 32;  // 16-byte pieces per code row
#pragma unroll
        for (int jj = 0; jj < (S::N_CODE + NW - 1) / NW; ++jj) {
            const int j = jj * NW + w;
            if (j >= S::N_CODE) break;
            const int piece = j * 64 + lane;
            const int64_t r = max(kr[piece / PPK], (int64_t)0);
            dma16_to_lds(p.codes + r * (D / 2) + (piece % PPK) * 16, slot + j * 1024);
        }
        constexpr int DPK = D / 64;  // 4-byte pieces per scale row
#pragma unroll
        for (int k = 0; k < S::N_SCALE; ++k) {
            if ((S::N_CODE + k) % NW != w) continue;
            const int piece = k * 64 + lane;  // lanes past the 16 rows land in the slot's unused tail
            const int64_t r = piece < CHUNK_KEYS * DPK ? max(kr[piece / DPK], (int64_t)0) : 0;
            dma4_to_lds(p.scales + r * (D / 16) + (piece % DPK) * 4, slot + S::SCALE_OFF + k * 256);
        }
    } else {
        constexpr int PPK = D / 8;  // 16-byte pieces per bf16 row
#pragma unroll
        for (int jj = 0; jj < (S::N_WIN + NW - 1) / NW; ++jj) {
            const int j = jj * NW + w;
            if (j >= S::N_WIN) break;
            const int piece = j * 64 + lane;
            const int64_t r = max(kr[piece / PPK], (int64_t)0);
            dma16_to_lds(reinterpret_cast<const uint8_t*>(p.swa) + r * (2 * D) + (piece % PPK) * 16,
                           slot + j * 1024);
        }
    }
}

// Dequantise one item (4 keys x 8 channels) from a staged chunk into the K tile
// (fp16, rows of D + 8 halves: the pad spreads the 16 rows of an MFMA operand
// read over all banks) and the V^T tile (fp16, transposed, padded).  Keys
// without a row hold row 0's finite values; their softmax weight is exactly 0.
// Window rows are bf16; their fp16 conversion is exact for 2^-14 <= |v| < 65504.
template <int D, bool SPARSE>
__device__ __forceinline__ void store_item(const uint8_t* slot, int kq, int co, uint4* ktile, uint8_t* vtile) {
    constexpr int KROW = D / 8 + 1;  // uint4 per K-tile row
    uint32_t kh[4][4];               // fp16 pairs: [key][channel pair]
    if (SPARSE) {
        uint32_t cw[4], sb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = 4 * kq + i;
            cw[i] = *reinterpret_cast<const uint32_t*>(slot + key * (D / 2) + co * 4);
            sb[i] = slot[Stage<D>::SCALE_OFF + key * (D / 16) + (co >> 1)];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) fp4x8_to_f16(cw[i], e4m3_f16x2_over256(sb[i]), kh[i]);
    } else {
        uint4 u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] = *reinterpret_cast<const uint4*>(slot + (4 * kq + i) * (2 * D) + co * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t wv[4] = {u[i].x, u[i].y, u[i].z, u[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const f16x2 v = f16x2{(_Float16)bf16_lo(wv[e]), (_Float16)bf16_hi(wv[e])};
                kh[i][e] = *reinterpret_cast<const uint32_t*>(&v);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        ktile[(4 * kq + i) * KROW + co] = make_uint4(kh[i][0], kh[i][1], kh[i][2], kh[i][3]);
    // V^T row d = 8co + e holds channel e of the 4 keys
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int d = 8 * co + e;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t x01 = __builtin_amdgcn_perm(kh[1][e >> 1], kh[0][e >> 1], sel);
        const uint32_t x23 = __builtin_amdgcn_perm(kh[3][e >> 1], kh[2][e >> 1], sel);
        *reinterpret_cast<uint2*>(vtile + vt_off(d, kq)) = make_uint2(x01, x23);
    }
}

template <int D, bool QF32, int NW, int RG = RING>
__global__ __launch_bounds__(64 * NW, RG == RING ? 1 : 2) void attn_kernel(AttnParams p) {
    constexpr int NBLK = D / 32;  // 32-channel blocks of the S MFMA
    constexpr int NDT = D / 16;   // 16-channel tiles of the O MFMA
    constexpr int CPR = D / 8;    // 16-byte chunks per fp16 key row
    constexpr int NT = 64 * NW;
    constexpr int ITEMS = 4 * CPR;  // dequantisation items per chunk
    using S = Stage<D>;
    __shared__ uint4 ktile[CHUNK_KEYS * (CPR + 1)];
    __shared__ __attribute__((aligned(16))) uint8_t vtile[D * 32 + (D / 8) * 16];
    __shared__ __attribute__((aligned(16))) uint8_t ring[RG * S::SLOT];
    __shared__ int64_t krow[MAX_CPS * CHUNK_KEYS];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c16 = lane & 15;
    const int64_t row = blockIdx.y;
    const int split = blockIdx.x;
    const int b = (int)(row / p.Q);
    const int head = 16 * w + c16;

    const int nchunks = (p.Kp + p.Wp) / CHUNK_KEYS;
    const int n_sp_chunks = p.Kp / CHUNK_KEYS;
    const int c_lo = split * p.cps;
    const int c_hi = min(nchunks, c_lo + p.cps);
    const int slot = p.Wp ? p.q_slot[row] : 0;
    const int wlo = max(0, slot - p.window + 1);

    // ---- the index loads go first: they head the longest chain (index ->
    // physical row -> copy -> dequantisation); the query loads follow and fly
    // while the rows are resolved and the first copies are issued
    const int nk = max(0, c_hi - c_lo) * CHUNK_KEYS;
    constexpr int KR_IT = (MAX_CPS * CHUNK_KEYS + NT - 1) / NT;  // key rows per thread at most
    int32_t kent[KR_IT];
#pragma unroll
    for (int j = 0; j < KR_IT; ++j) {
        const int i = tid + j * NT;
        const int kpos = c_lo * CHUNK_KEYS + i;
        kent[j] = (i < nk && kpos < p.K) ? p.idx[row * p.K + kpos] : -1;
    }
    float qf[QF32 ? NBLK : 1][8];
    uint4 qraw[QF32 ? 1 : NBLK];
    if (QF32) {
        const float* qr = static_cast<const float*>(p.q) + (row * p.H + head) * D;
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk) {
            const float4 a = *reinterpret_cast<const float4*>(qr + 32 * blk + 8 * g);
            const float4 c = *reinterpret_cast<const float4*>(qr + 32 * blk + 8 * g + 4);
            float* f = qf[QF32 ? blk : 0];
            f[0] = a.x, f[1] = a.y, f[2] = a.z, f[3] = a.w, f[4] = c.x, f[5] = c.y, f[6] = c.z, f[7] = c.w;
        }
    } else {
        const uint16_t* qr = static_cast<const uint16_t*>(p.q) + (row * p.H + head) * D;
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk) qraw[QF32 ? 0 : blk] = *reinterpret_cast<const uint4*>(qr + 32 * blk + 8 * g);
    }

    // ---- physical rows of every key of this split (-1: none)
#pragma unroll
    for (int j = 0; j < KR_IT; ++j) {
        const int i = tid + j * NT;
        if (i >= nk) break;
        const int kpos = c_lo * CHUNK_KEYS + i;
        int64_t r = -1;
        if (kpos < p.Kp) {
            if (kent[j] >= 0) r = phys_row(p.kvmap, b, kent[j]);
        } else {
            const int t = wlo + (kpos - p.Kp);
            if (t <= slot && t < p.T) r = (int64_t)b * p.T + t;
        }
        krow[i] = r;
    }
    // LDS barrier only: the query loads stay in flight (each chunk's wait
    // below is for all of this wave's loads, so they are complete before S)
    lds_barrier();

    // ---- raw bytes of the first RG chunks start flowing into the LDS ring
    const int c_pre = min(c_hi, c_lo + RG);
    for (int ch = c_lo; ch < c_pre; ++ch)
        stage_chunk<D, NW>(p, ch < n_sp_chunks, krow + (ch - c_lo) * CHUNK_KEYS, ring + ((ch - c_lo) % RG) * S::SLOT,
                           w, lane);

    // ---- Q operand (B of S^T = K Q^T): Q[head][32*blk + 8g .. +8] in fp16,
    // pre-scaled by 2^-qs; an fp32 query is split into hi + lo fp16 parts
    uint32_t qmax = 0;  // largest |q| as an fp32 bit pattern (monotone in |q|)
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
        if (QF32) {
#pragma unroll
            for (int e = 0; e < 8; ++e) qmax = max(qmax, __float_as_uint(qf[QF32 ? blk : 0][e]) & 0x7FFFFFFFu);
        } else {
            const uint4 u = qraw[QF32 ? 0 : blk];
            const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) qmax = max(qmax, max((wv[e] << 16) & 0x7FFF0000u, wv[e] & 0x7FFF0000u));
        }
    }
    qmax = max(qmax, (uint32_t)__shfl_xor((int)qmax, 16));
    qmax = max(qmax, (uint32_t)__shfl_xor((int)qmax, 32));
    // 2^-qs maps the largest element into [2^14, 2^15)
    const int qs = qmax == 0 ? 0 : min(113, max(-100, (int)(qmax >> 23) - 127 - 14));
    const float qscale = __uint_as_float((uint32_t)(127 - qs) << 23);
    const float zscale = p.scale_log2 * __uint_as_float((uint32_t)(127 + qs) << 23);
    f16x8 qhi[NBLK];
    f16x8 qlo[QF32 ? NBLK : 1];
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
        float x[8];
        if (QF32) {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = qf[QF32 ? blk : 0][e] * qscale;
        } else {
            const uint4 u = qraw[QF32 ? 0 : blk];
            const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[2 * e] = bf16_lo(wv[e]) * qscale;
                x[2 * e + 1] = bf16_hi(wv[e]) * qscale;
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const _Float16 h = (_Float16)x[e];
            qhi[blk][e] = h;
            if (QF32) qlo[QF32 ? blk : 0][e] = (_Float16)(x[e] - (float)h);
        }
    }

    f32x4 oacc[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;

    int c_issued = c_pre;  // chunks [c_lo, c_issued) have been issued
    const int vb = vt_base(c16, g);
    for (int ch = c_lo; ch < c_hi; ++ch) {
        const bool sparse = ch < n_sp_chunks;
        const int64_t* kr = krow + (ch - c_lo) * CHUNK_KEYS;
        const uint8_t* st = ring + ((ch - c_lo) % RG) * S::SLOT;
        // ---- the chunk's copies have landed (all of this wave's copies: the
        // compiler cannot tell ring slots apart and would wait for them anyway)
        __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
        lds_barrier();  // every wave's copies have landed; the tiles are free
        // ---- dequantise the staged chunk into the LDS tiles
        if (sparse) {
#pragma unroll
            for (int it = 0; it < (ITEMS + NT - 1) / NT; ++it) {
                const int item = it * NT + tid;
                if (item < ITEMS) store_item<D, true>(st, item / CPR, item % CPR, ktile, vtile);
            }
        } else {
#pragma unroll
            for (int it = 0; it < (ITEMS + NT - 1) / NT; ++it) {
                const int item = it * NT + tid;
                if (item < ITEMS) store_item<D, false>(st, item / CPR, item % CPR, ktile, vtile);
            }
        }
        lds_barrier();
        // ---- the ring slot is free again: refill it with chunk ch + RG
        if (c_issued < c_hi) {
            stage_chunk<D, NW>(p, c_issued < n_sp_chunks, krow + (c_issued - c_lo) * CHUNK_KEYS,
                               ring + ((c_issued - c_lo) % RG) * S::SLOT, w, lane);
            ++c_issued;
        }
        // ---- S^T[key][head] = sum_d K[key][d] Q[head][d]
        // four accumulator chains (a dependent MFMA waits for three others);
        // the operands of the next four blocks are read while these multiply
        f32x4 sacc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) sacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        uint4 kop[2][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) kop[0][j] = ktile[c16 * (CPR + 1) + 4 * j + g];
#pragma unroll
        for (int grp = 0; grp < NBLK / 4; ++grp) {
            if (grp + 1 < NBLK / 4) {
#pragma unroll
                for (int j = 0; j < 4; ++j) kop[(grp + 1) & 1][j] = ktile[c16 * (CPR + 1) + 4 * (4 * (grp + 1) + j) + g];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f16x8 a = *reinterpret_cast<const f16x8*>(&kop[grp & 1][j]);
                sacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qhi[4 * grp + j], sacc[j], 0, 0, 0);
                if (QF32) sacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qlo[QF32 ? 4 * grp + j : 0], sacc[j], 0, 0, 0);
            }
        }
        const f32x4 s = (sacc[0] + sacc[1]) + (sacc[2] + sacc[3]);
        // ---- online softmax for head `head` over keys 4g..4g+3 of this chunk
        float z[4];
        float mloc = -INFINITY;
        int64_t kv4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) kv4[i] = kr[4 * g + i];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            z[i] = (kv4[i] >= 0) ? s[i] * zscale : -INFINITY;
            mloc = fmaxf(mloc, z[i]);
        }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        // lazy maximum: move it only when this chunk exceeds it by more than 2^8
        // (nothing to rescale while nothing has been accumulated)
        float alpha = 1.0f;
        if (mloc > m_run + 8.0f) {
            if (l_run > 0.0f) alpha = exp2f(m_run - mloc);
            m_run = mloc;
        }
        if (__any(alpha != 1.0f)) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
        }
        float psum = 0.0f;
        f16x4 pb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // z - m_run <= 8: the hardware exp2 needs no range reduction
            const _Float16 h = (_Float16)((z[i] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(z[i] - m_run));
            psum += (float)h;  // normalise by the weights the MFMA actually applies
            pb[i] = h;
        }
        psum += __shfl_xor(psum, 16);
        psum += __shfl_xor(psum, 32);
        l_run = l_run * alpha + psum;
        // ---- O^T[d][head] += sum_key V^T[d][key] P^T[key][head]
        // operands read eight tiles ahead of the MFMAs that use them
        constexpr int PG = NDT < 8 ? NDT : 8;
        uint2 vop[2][PG];
#pragma unroll
        for (int j = 0; j < PG; ++j) vop[0][j] = *reinterpret_cast<const uint2*>(vtile + vb + VT_DT * j);
#pragma unroll
        for (int grp = 0; grp < NDT / PG; ++grp) {
            if (grp + 1 < NDT / PG) {
#pragma unroll
                for (int j = 0; j < PG; ++j)
                    vop[(grp + 1) & 1][j] = *reinterpret_cast<const uint2*>(vtile + vb + VT_DT * (PG * (grp + 1) + j));
            }
#pragma unroll
            for (int j = 0; j < PG; ++j) {
                const f16x4 a = *reinterpret_cast<const f16x4*>(&vop[grp & 1][j]);
                oacc[PG * grp + j] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, pb, oacc[PG * grp + j], 0, 0, 0);
            }
        }
    }

    if (p.nsplit > 1) {
        // ---- unnormalised partial of this key range, each lane's 4 x D/16
        // accumulators stored contiguously (full 1 KB per wave instruction)
        float* po = p.part_o + ((row * p.nsplit + split) * p.H + 16 * w) * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4*>(po + (dt * 64 + lane) * 4) = oacc[dt];
        if (g == 0) p.part_ml[(row * p.nsplit + split) * p.H + head] = make_float2(m_run, l_run);
        // snapshot of the lse to merge with: the merge kernel overwrites it
        if (p.merge && split == 0 && g == 0) p.lse_prev[row * p.H + head] = p.lse[row * p.H + head];
        return;
    }
    // ---- normalised output (o, lse) of this key set
    const float inv = (l_run > 0.0f) ? 1.0f / l_run : 0.0f;
    const float lse_cur = (l_run > 0.0f) ? (m_run + log2f(l_run)) * 0.69314718055994531f : -INFINITY;
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

// Merge the split partials: exact log-sum-exp combination, optionally together
// with the (o, lse) already in the output.  One workgroup = one row x one
// 16-head group x 4 of its 16-column tiles; thread = one lane-order float4
// (head 16 hg + lane % 16, columns 16 dt + 4 (lane / 16) .. +3).  Splits are
// taken NB at a time (all loads of a batch issued before any arithmetic) with
// a running maximum across batches.
template <int NB>
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ part_o,
                                                         const float2* __restrict__ part_ml,
                                                         const float* __restrict__ lse_prev, int nsplit, int H, int D,
                                                         int merge, float* __restrict__ o, float* __restrict__ lse) {
    const int64_t row = blockIdx.x;
    const int hg = blockIdx.y;
    const int t = threadIdx.x, lane = t & 63;
    const int dt = blockIdx.z * 4 + (t >> 6);
    const int h = 16 * hg + (lane & 15);
    const int c = 16 * dt + 4 * (lane >> 4);
    float* op = o + (row * H + h) * D + c;
    // the output's own partial: weight e^lse = 2^(lse log2 e), normalised o
    const float lse_old = merge ? lse_prev[row * H + h] : -INFINITY;
    const float4 o_old = merge ? *reinterpret_cast<const float4*>(op) : make_float4(0.f, 0.f, 0.f, 0.f);
    float M = lse_old * 1.4426950408889634f;
    f32x4 acc = f32x4{o_old.x, o_old.y, o_old.z, o_old.w};
    float den = M == -INFINITY ? 0.0f : 1.0f;
    if (M == -INFINITY) acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < nsplit; s0 += NB) {
        float2 ml[NB];
        f32x4 ov[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int s = s0 + j;
            ml[j] = s < nsplit ? part_ml[(row * nsplit + s) * H + h] : make_float2(-INFINITY, 0.0f);
            ov[j] = s < nsplit ? *reinterpret_cast<const f32x4*>(part_o + ((row * nsplit + s) * H + 16 * hg) * D +
                                                                 (dt * 64 + lane) * 4)
                               : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        float Mb = M;
#pragma unroll
        for (int j = 0; j < NB; ++j) Mb = fmaxf(Mb, ml[j].x);
        if (Mb == -INFINITY) continue;
        if (Mb != M) {
            const float r = (M == -INFINITY) ? 0.0f : exp2f(M - Mb);
            acc *= r;
            den *= r;
            M = Mb;
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const float wv = (ml[j].x == -INFINITY) ? 0.0f : exp2f(ml[j].x - M);
            acc += wv * ov[j];
            den += wv * ml[j].y;
        }
    }
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    // (each thread rewrites only the o it read; the old lse comes from a snapshot)
    *reinterpret_cast<float4*>(op) = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    if (dt == 0 && (lane >> 4) == 0)
        lse[row * H + h] = den > 0.0f ? (M + log2f(den)) * 0.69314718055994531f : -INFINITY;
}

constexpr int MAX_SPLIT = 64;

int choose_nsplit(int64_t rows, int nchunks) {
    if (nchunks <= 1) return 1;
    // one resident workgroup per CU (its LDS ring holds one): about 256
    // workgroups run in a single round, more only add rounds and partials
    int64_t want = (256 + rows - 1) / rows;
    int64_t by_chunks = (nchunks + 1) / 2;   // at least two chunks per split
    int64_t s = want < by_chunks ? want : by_chunks;
    if (s > MAX_SPLIT) s = MAX_SPLIT;
    if (s < 1) s = 1;
    return (int)s;
}

size_t attn_ws_bytes(int64_t rows, int H, int D) {
    int64_t s = (256 + rows - 1) / rows;
    if (s > MAX_SPLIT) s = MAX_SPLIT;
    if (s <= 1) return 0;
    return (size_t)(rows * s * H) * (size_t)(D + 2) * 4 + (size_t)(rows * H) * 4 + 256;
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
        CSA2_ARG(aligned(kv->codes, 16) && aligned(kv->scales, 4),
                 "%s: codes must be 16-byte and scales 4-byte aligned", what);
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
        const size_t need = (size_t)(rows * p.nsplit * H) * (size_t)(D + 2) * 4 + (size_t)(rows * H) * 4;
        CSA2_REQUIRE(ws != nullptr && ws_bytes >= need, CSA2_EWORKSPACE,
                     "%s: workspace of %zu bytes required, %zu given", what, need, ws ? ws_bytes : (size_t)0);
        CSA2_ARG(((uintptr_t)ws & 15) == 0, "%s: workspace must be 16-byte aligned", what);
        p.part_o = static_cast<float*>(ws);
        p.part_ml = reinterpret_cast<float2*>(p.part_o + rows * p.nsplit * H * (int64_t)D);
        p.lse_prev = reinterpret_cast<float*>(p.part_ml + rows * p.nsplit * H);
    }
    const dim3 grid((unsigned)p.nsplit, (unsigned)rows);
    const dim3 block((unsigned)(4 * H));
    const bool f32 = qt == CSA2_F32;
    const int nw = H / 16;
    const bool wide = p.nsplit == 1 && rows >= 512 && D == 512 && nw == 4;
    if (wide) {
        if (f32)
            attn_kernel<512, true, 4, RING_WIDE><<<grid, block, 0, stream>>>(p);
        else
            attn_kernel<512, false, 4, RING_WIDE><<<grid, block, 0, stream>>>(p);
    }
#define CSA2_ATTN_NW(DD, F, NWV) \
    if (!wide && nw == NWV) attn_kernel<DD, F, NWV><<<grid, block, 0, stream>>>(p);
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
        const dim3 mg((unsigned)rows, (unsigned)(H / 16), (unsigned)(D / 64)), mb(256);
        if (p.nsplit <= 4)
            attn_merge_kernel<4><<<mg, mb, 0, stream>>>(p.part_o, p.part_ml, p.lse_prev, p.nsplit, H, D, p.merge, o,
                                                         lse);
        else if (p.nsplit <= 8)
            attn_merge_kernel<8><<<mg, mb, 0, stream>>>(p.part_o, p.part_ml, p.lse_prev, p.nsplit, H, D, p.merge, o,
                                                         lse);
        else if (p.nsplit <= 16)
            attn_merge_kernel<16><<<mg, mb, 0, stream>>>(p.part_o, p.part_ml, p.lse_prev, p.nsplit, H, D,
                                                         p.merge, o, lse);
        else  // one batch up to 24 splits (decode at a few rows)
            attn_merge_kernel<24><<<mg, mb, 0, stream>>>(p.part_o, p.part_ml, p.lse_prev, p.nsplit, H, D,
                                                         p.merge, o, lse);
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
