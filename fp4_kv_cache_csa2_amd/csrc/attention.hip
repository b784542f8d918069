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
// registers into one fp16 LDS tile, K row-major: S^T = K Q^T reads it directly
// (v_mfma_f32_16x16x32_f16), O^T = V^T P^T (v_mfma_f32_16x16x16_f16) reads V^T
// out of the same tile with the transposing LDS read.  An E2M1 x E4M3 product
// has <= 6 significant bits and lies in [2^-10, 2688], so it is exact in fp16;
// the E2M1 values come from the hardware FP4 conversion.  The query is
// pre-scaled per head by a power of
// two so that its largest element sits in [2^14, 2^15) (exact), and the scale
// is folded into the logit scale.  The S^T accumulator layout (lane holds keys
// 4g..4g+3 of head lane%16) is exactly the P^T operand layout of the second
// MFMA, so P never leaves registers.  Softmax is online in the log2 domain with
// a lazy maximum: the running maximum moves (and O is rescaled) only when a
// chunk exceeds it by more than 2^8, so P <= 256 stays well inside fp16.  Few
// rows (decode) split the keys over several workgroups whose unnormalised
// partials are merged by a second kernel.  At D = 512, H = 64 with bf16
// queries a producer/consumer variant (attn_pc_kernel) runs instead, split or
// not: four waves dequantise while four multiply.
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
    // fp16 copy of the FP4 entries by logical position (k16[b n_stage + j][D]), or null
    const uint16_t* k16;
    int64_t n_stage;
    // window
    const uint16_t* swa;       // [B][T][D] ring: token t at row t mod T
    int32_t T;
    const int32_t* q_pos;      // [rows] absolute position of the query token
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

// E4M3FN scale byte -> fp16 bits of scale x 2^-8, twice (exact: E4M3 and fp16
// share the mantissa alignment, so the byte shifted into the fp16 exponent /
// mantissa fields is the scale with its exponent bias off by 8; subnormal
// scales land on fp16 subnormals).
__device__ __forceinline__ uint32_t e4m3_f16x2_over256(uint32_t code) { return (code << 7) | (code << 23); }

// 8 FP4 codes (one 32-bit word, channel 2i in the low nibble of byte i) times
// the scale -> four fp16 pairs (channels 2i, 2i+1).  gfx950's FP4 conversion
// turns byte i into (E2M1 x 2^8) of both its nibbles, low nibble first (its
// fp32 scale is applied as a power of two; checked exhaustively on all 256
// byte values); (E2M1 x 2^8) x (E4M3 x 2^-8) is exact in fp16: <= 6
// significant bits in [2^-10, 2688].
__device__ __forceinline__ void fp4x8_to_f16(uint32_t w, uint32_t sc2, uint32_t (&out)[4]) {
    const f16x2 sc = __builtin_bit_cast(f16x2, sc2);
#define CSA2_FP4B(I)                                                                                            \
    out[I] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, I)) * sc);
    CSA2_FP4B(0) CSA2_FP4B(1) CSA2_FP4B(2) CSA2_FP4B(3)
#undef CSA2_FP4B
}

// LDS layout of the fp16 K tile, chosen against bank conflicts (measured on
// gfx950: 64 banks of 4 bytes; a 64-bit access serves lanes 0-31 and 32-63 in
// one pass each, a 128-bit access lanes {0-7, 24-31}, {8-15, 16-23},
// {32-39, 56-63}, {40-47, 48-55}).  Row k (D fp16) at k (D/8 + 2) 16 bytes, 32
// bytes of padding per row.  The tile serves both products: S reads lane
// (cz, gz) at row cz, 16-byte chunk 4j + gz; PV reads V^T by the transposing
// 64-bit LDS read (see attn_pv) at rows 4gz + cz/4, byte 32dt + 8(cz % 4);
// the dequantisation writes lane co at chunk co of one row.  All three are
// conflict-free.
constexpr int KROW_PAD = 2;

constexpr int MAX_CPS = 64;  // chunks per split (keys per workgroup <= 1024)
constexpr int RING = 4;      // chunks whose raw bytes are in flight / staged in LDS at once

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

// Copies of one chunk in two steps: the rows each lane copies are read from
// the workgroup's row list first (chunk_rows), the copies are issued later
// (chunk_issue), so that no copy waits for its own LDS read.  A key without a
// row copies row 0 instead: its values are finite and its softmax weight is
// exactly 0, so it adds nothing.
template <int D, int NW>
struct ChunkRows {
    using S = Stage<D>;
    static constexpr int NC = (S::N_CODE + NW - 1) / NW;  // code copies per wave
    static constexpr int NWN = (S::N_WIN + NW - 1) / NW;  // window copies per wave
    static constexpr int N = NC + S::N_SCALE > NWN ? NC + S::N_SCALE : NWN;
    int64_t r[N];
};

template <int D, int NW>
__device__ __forceinline__ void chunk_rows(bool sparse, const int64_t* kr, int w, int lane, ChunkRows<D, NW>& cr) {
    using S = Stage<D>;
    using C = ChunkRows<D, NW>;
    if (sparse) {
        constexpr int PPK = D / 32;  // 16-byte pieces per code row
#pragma unroll
        for (int jj = 0; jj < C::NC; ++jj) {
            const int j = jj * NW + w;
            if (j >= S::N_CODE) break;
            cr.r[jj] = kr[(j * 64 + lane) / PPK];
        }
        constexpr int DPK = D / 64;  // 4-byte pieces per scale row
#pragma unroll
        for (int k = 0; k < S::N_SCALE; ++k) {
            if ((S::N_CODE + k) % NW != w) continue;
            const int piece = k * 64 + lane;  // lanes past the 16 rows land in the slot's unused tail
            cr.r[C::NC + k] = piece < CHUNK_KEYS * DPK ? kr[piece / DPK] : 0;
        }
    } else {
        constexpr int PPK = D / 8;  // 16-byte pieces per bf16 row
#pragma unroll
        for (int jj = 0; jj < C::NWN; ++jj) {
            const int j = jj * NW + w;
            if (j >= S::N_WIN) break;
            cr.r[jj] = kr[(j * 64 + lane) / PPK];
        }
    }
}

template <int D, int NW>
__device__ __forceinline__ void chunk_issue(const AttnParams& p, bool sparse, const ChunkRows<D, NW>& cr,
                                            uint8_t* slot, int w, int lane) {
    using S = Stage<D>;
    using C = ChunkRows<D, NW>;
    // An opaque zero, fresh every call: the per-lane byte offsets are
    // recomputed here instead of being kept (hoisted out of the chunk loop) as
    // 64-bit addresses, which spill; a spill reload waits for every copy in
    // flight, the ring's prefetch included.
    int z;
    asm volatile("s_mov_b32 %0, 0" : "=s"(z));
    const int lz = lane + z;
    if (sparse) {
        constexpr int PPK = D / 32;
#pragma unroll
        for (int jj = 0; jj < C::NC; ++jj) {
            const int j = jj * NW + w;
            if (j >= S::N_CODE) break;
            const int64_t r = max(cr.r[jj], (int64_t)0);
            dma16_to_lds(p.codes + r * (D / 2) + ((j * 64 + lz) % PPK) * 16, slot + j * 1024);
        }
        constexpr int DPK = D / 64;
#pragma unroll
        for (int k = 0; k < S::N_SCALE; ++k) {
            if ((S::N_CODE + k) % NW != w) continue;
            const int64_t r = max(cr.r[C::NC + k], (int64_t)0);
            dma4_to_lds(p.scales + r * (D / 16) + ((k * 64 + lz) % DPK) * 4, slot + S::SCALE_OFF + k * 256);
        }
    } else {
        constexpr int PPK = D / 8;
#pragma unroll
        for (int jj = 0; jj < C::NWN; ++jj) {
            const int j = jj * NW + w;
            if (j >= S::N_WIN) break;
            const int64_t r = max(cr.r[jj], (int64_t)0);
            dma16_to_lds(reinterpret_cast<const uint8_t*>(p.swa) + r * (2 * D) + ((j * 64 + lz) % PPK) * 16,
                         slot + j * 1024);
        }
    }
}

// One dequantisation item: 4 keys x 8 channels as fp16 pairs kh[key][pair].
// FP4: E2M1 values times the E4M3 scale (exact in fp16).  Window rows are
// bf16; their fp16 conversion is exact for 2^-14 <= |v| < 65504.
__device__ __forceinline__ void item_from_fp4(const uint32_t (&cw)[4], const uint32_t (&sb)[4], uint32_t (&kh)[4][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) fp4x8_to_f16(cw[i], e4m3_f16x2_over256(sb[i]), kh[i]);
}
__device__ __forceinline__ void item_from_bf16(const uint4 (&u)[4], uint32_t (&kh)[4][4]) {
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

// Write one item (keys 4kq..4kq+3, channels 8co..8co+7) into the K tile.
template <int D>
__device__ __forceinline__ void put_item(const uint32_t (&kh)[4][4], int kq, int co, uint4* ktile) {
    constexpr int KROW = D / 8 + KROW_PAD;  // uint4 per K-tile row
#pragma unroll
    for (int i = 0; i < 4; ++i)
        ktile[(4 * kq + i) * KROW + co] = make_uint4(kh[i][0], kh[i][1], kh[i][2], kh[i][3]);
}

// Dequantise one item from a staged chunk into the K tile.  Keys without a row
// hold row 0's finite values; their softmax weight is exactly 0.
template <int D, bool SPARSE>
__device__ __forceinline__ void store_item(const uint8_t* slot, int kq, int co, uint4* ktile) {
    uint32_t kh[4][4];  // fp16 pairs: [key][channel pair]
    if (SPARSE) {
        uint32_t cw[4], sb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = 4 * kq + i;
            cw[i] = *reinterpret_cast<const uint32_t*>(slot + key * (D / 2) + co * 4);
            sb[i] = slot[Stage<D>::SCALE_OFF + key * (D / 16) + (co >> 1)];
        }
        item_from_fp4(cw, sb, kh);
    } else {
        uint4 u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] = *reinterpret_cast<const uint4*>(slot + (4 * kq + i) * (2 * D) + co * 16);
        item_from_bf16(u, kh);
    }
    put_item<D>(kh, kq, co, ktile);
}

// max / sum over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48)
// by two row swaps on the VALU, without an LDS round trip.  Every lane ends
// with the same bits: each pairwise step is commutative.
__device__ __forceinline__ float rows_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ uint32_t rows_umax(uint32_t x) {
    const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = max((uint32_t)a[0], (uint32_t)a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return max((uint32_t)b[0], (uint32_t)b[1]);
}

// Q operand (B of S^T = K Q^T) of one lane: Q[head][32 blk + 8g .. +8] in
// fp16, pre-scaled by 2^-qs so that the head's largest element lies in
// [2^14, 2^15); an fp32 query is split into hi + lo fp16 parts.  Returns the
// logit scale sm_scale log2(e) 2^qs.
// Only blocks BLK0..BLK0+NB-1 are converted; the scale comes from all D channels.
template <int D, bool QF32, int NB = D / 32, int BLK0 = 0>
__device__ __forceinline__ float q_operand(const float (&qf)[QF32 ? D / 32 : 1][8], const uint4 (&qraw)[QF32 ? 1 : D / 32],
                                          float scale_log2, f16x8 (&qhi)[NB], f16x8 (&qlo)[QF32 ? NB : 1]) {
    constexpr int NBLK = D / 32;
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
    qmax = rows_umax(qmax);
    // 2^-qs maps the largest element into [2^14, 2^15)
    const int qs = qmax == 0 ? 0 : min(113, max(-100, (int)(qmax >> 23) - 127 - 14));
    const float qscale = __uint_as_float((uint32_t)(127 - qs) << 23);
#pragma unroll
    for (int bi = 0; bi < NB; ++bi) {
        const int blk = BLK0 + bi;
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
            qhi[bi][e] = h;
            if (QF32) qlo[QF32 ? bi : 0][e] = (_Float16)(x[e] - (float)h);
        }
    }
    return scale_log2 * __uint_as_float((uint32_t)(127 + qs) << 23);
}

// One 16-key chunk from the LDS tiles for the lane's head, in three steps:
// S^T = K Q^T (attn_scores), online softmax in the log2 domain with a lazy
// maximum (attn_weights), O^T += V^T P^T (attn_pv).  kr: the chunk's key rows
// (-1: none); cz, gz: lane % 16 and lane / 16, recomputed by the caller every
// chunk (so that no address lives across the chunk loop).
// (over the NB 32-channel blocks from blk0 only: a partial score)
template <int D, bool QF32, int NB = D / 32>
__device__ __forceinline__ f32x4 attn_scores(const uint4* ktile, int cz, int gz, const f16x8 (&qhi)[NB],
                                             const f16x8 (&qlo)[QF32 ? NB : 1], int blk0 = 0) {
    constexpr int NBLK = NB, CPR = D / 8;
    ktile += 4 * blk0;
    // S^T[key][head] = sum_d K[key][d] Q[head][d]: four accumulator chains (a
    // dependent MFMA waits for three others); the operands of the next four
    // blocks are read while these multiply
    f32x4 sacc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) sacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint4 kop[2][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) kop[0][j] = ktile[cz * (CPR + KROW_PAD) + 4 * j + gz];
#pragma unroll
    for (int grp = 0; grp < NBLK / 4; ++grp) {
        if (grp + 1 < NBLK / 4) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                kop[(grp + 1) & 1][j] = ktile[cz * (CPR + KROW_PAD) + 4 * (4 * (grp + 1) + j) + gz];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f16x8 a = *reinterpret_cast<const f16x8*>(&kop[grp & 1][j]);
            sacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qhi[4 * grp + j], sacc[j], 0, 0, 0);
            if (QF32) sacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qlo[QF32 ? 4 * grp + j : 0], sacc[j], 0, 0, 0);
        }
    }
    return (sacc[0] + sacc[1]) + (sacc[2] + sacc[3]);
}

// Softmax weights of keys 4gz..4gz+3 (scores s), with the running maximum and
// sum; rescales O when the maximum moves.  Returns P as the fp16 B operand.
template <int NDT>
__device__ __forceinline__ f16x4 attn_weights(const f32x4& s, const int64_t* kr, int gz, float zscale,
                                              f32x4 (&oacc)[NDT], float& m_run, float& l_run) {
    float z[4];
    float mloc = -INFINITY;
    int64_t kv4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) kv4[i] = kr[4 * gz + i];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        z[i] = (kv4[i] >= 0) ? s[i] * zscale : -INFINITY;
        mloc = fmaxf(mloc, z[i]);
    }
    mloc = rows_max(mloc);
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
    l_run = l_run * alpha + rows_sum(psum);
    return pb;
}

// O^T[d][head] += sum_key V^T[d][key] P^T[key][head].  The A operand of lane
// (cz, gz), V^T[16dt + cz][keys 4gz..4gz+3], comes from the K tile through the
// transposing LDS read: within each 16-lane group, lane j receives element
// j % 4 of the four fp16 that lane 4e + j / 4 addresses, for e = 0..3.  So
// lane (cz, gz) addresses row 4gz + cz / 4 at columns 16dt + 4(cz % 4) .. +3.
// (over the NDTP 16-channel tiles from dt0 only)
template <int D, int NDTP = D / 16>
__device__ __forceinline__ void attn_pv(const uint4* ktile, int cz, int gz, const f16x4& pb, f32x4 (&oacc)[NDTP],
                                        int dt0 = 0) {
    constexpr int NDT = NDTP, ROWB = (D / 8 + KROW_PAD) * 16;
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4* lds_s16x4;
    const uint8_t* base = reinterpret_cast<const uint8_t*>(ktile) + (4 * gz + (cz >> 2)) * ROWB + 8 * (cz & 3) + 32 * dt0;
    auto vread = [&](int dt) {
        return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(base + 32 * dt)));
    };
    // operands read eight tiles ahead of the MFMAs that use them
    constexpr int PG = NDT < 8 ? NDT : 8;
    f16x4 vop[2][PG];
#pragma unroll
    for (int j = 0; j < PG; ++j) vop[0][j] = vread(j);
#pragma unroll
    for (int grp = 0; grp < NDT / PG; ++grp) {
        if (grp + 1 < NDT / PG) {
#pragma unroll
            for (int j = 0; j < PG; ++j) vop[(grp + 1) & 1][j] = vread(PG * (grp + 1) + j);
        }
#pragma unroll
        for (int j = 0; j < PG; ++j)
            oacc[PG * grp + j] = __builtin_amdgcn_mfma_f32_16x16x16f16(vop[grp & 1][j], pb, oacc[PG * grp + j], 0, 0, 0);
    }
}

// Two chunks A, B at once (many rows): softmax weights of keys 4gz..4gz+3 of
// both, and one O^T += V^T P^T over their 32 keys with the K = 32 MFMA (the
// K = 16 form runs at half its rate).  K index 8gz + e of the product is key
// 4gz + e of chunk A for e < 4 and key 4gz + e - 4 of chunk B otherwise, in
// both operands: P is (pA, pB), V^T is the transposing read of tile A
// followed by that of tile B.
// Scheduling hint for a run of N MFMAs fed by LDS reads (R per MFMA): the
// reads of the first A MFMAs first, then each MFMA followed by the reads of
// the one A places later, so that A MFMAs' operands are in flight while the
// matrix core works (the default schedule waits for each operand just before
// its MFMA).
template <int N, int R, int A>
__device__ __forceinline__ void mfma_pipeline_hint() {
    __builtin_amdgcn_sched_group_barrier(0x100, R * A, 0);  // DS reads
#pragma unroll
    for (int i = 0; i < N; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        if (i + A < N) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
    }
}

template <int NDT>
__device__ __forceinline__ f16x8 attn_weights2(const f32x4& sa, const f32x4& sb, uint32_t mk, int gz, float zscale,
                                               f32x4 (&oacc)[NDT], float& m_run, float& l_run) {
    // mk: validity bits of A's keys (bits 0-15) and B's (bits 16-31)
    float z[8];
    float mloc = -INFINITY;
    const uint32_t ma = mk >> (4 * gz), mb = mk >> (16 + 4 * gz);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        z[i] = ((ma >> i) & 1u) ? sa[i] * zscale : -INFINITY;
        z[4 + i] = ((mb >> i) & 1u) ? sb[i] * zscale : -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) mloc = fmaxf(mloc, z[i]);
    mloc = rows_max(mloc);
    // lazy maximum: move it only when these keys exceed it by more than 2^8
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
    f16x8 pb;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const _Float16 h = (_Float16)((z[i] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(z[i] - m_run));
        psum += (float)h;
        pb[i] = h;
    }
    l_run = l_run * alpha + rows_sum(psum);
    return pb;
}

// S^T of two chunks A, B at once, their MFMAs interleaved (A block 0, B
// block 0, A block 1, ...) over four accumulator chains (A even blocks, B even,
// A odd, B odd: a dependent MFMA follows three others), each operand read
// eight MFMAs ahead of its use from a ring of eight registers.
template <int D, int AHEAD = 8>
__device__ __forceinline__ void attn_scores2(const uint4* ka, const uint4* kb, int cz, int gz,
                                             const f16x8 (&qhi)[D / 32], f32x4& sa, f32x4& sb) {
    constexpr int NM = 2 * (D / 32), CPR = D / 8;
    const int ro = cz * (CPR + KROW_PAD) + gz;
    f32x4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint4 op[AHEAD];
    auto rd = [&](int m) { return ((m & 1) ? kb : ka)[ro + 4 * (m >> 1)]; };
#pragma unroll
    for (int m = 0; m < AHEAD; ++m) op[m] = rd(m);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const f16x8 a = *reinterpret_cast<const f16x8*>(&op[m % AHEAD]);
        acc[m & 3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qhi[m >> 1], acc[m & 3], 0, 0, 0);
        if (m + AHEAD < NM) op[m % AHEAD] = rd(m + AHEAD);
    }
    sa = acc[0] + acc[2];
    sb = acc[1] + acc[3];
}

template <int D>
__device__ __forceinline__ void attn_pv2(const uint4* ka, const uint4* kb, int cz, int gz, const f16x8& pb,
                                         f32x4 (&oacc)[D / 16]) {
    constexpr int NDT = D / 16, ROWB = (D / 8 + KROW_PAD) * 16;
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4* lds_s16x4;
    const int off = (4 * gz + (cz >> 2)) * ROWB + 8 * (cz & 3);
    const uint8_t* ba = reinterpret_cast<const uint8_t*>(ka) + off;
    const uint8_t* bb = reinterpret_cast<const uint8_t*>(kb) + off;
    auto vread = [&](int dt) {
        const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(ba + 32 * dt));
        const s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(bb + 32 * dt));
        return __builtin_bit_cast(f16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // each operand read eight MFMAs ahead of its use, from a ring of eight
    constexpr int AHEAD = 8;
    f16x8 vop[AHEAD];
#pragma unroll
    for (int j = 0; j < AHEAD; ++j) vop[j] = vread(j);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
        oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop[dt % AHEAD], pb, oacc[dt], 0, 0, 0);
        if (dt + AHEAD < NDT) vop[dt % AHEAD] = vread(dt + AHEAD);
    }
    mfma_pipeline_hint<NDT, 2, AHEAD>();
}

template <int D, bool QF32>
__device__ __forceinline__ void attn_chunk(const uint4* ktile, const int64_t* kr, int cz, int gz,
                                           const f16x8 (&qhi)[D / 32], const f16x8 (&qlo)[QF32 ? D / 32 : 1],
                                           float zscale, f32x4 (&oacc)[D / 16], float& m_run, float& l_run) {
    const f32x4 s = attn_scores<D, QF32>(ktile, cz, gz, qhi, qlo);
    const f16x4 pb = attn_weights<D / 16>(s, kr, gz, zscale, oacc, m_run, l_run);
    attn_pv<D>(ktile, cz, gz, pb, oacc);
}

// Normalised output (o, lse) of one head's key set, merged with the (o, lse)
// already in the output when p.merge is set.
// (columns of the NDTP tiles from tile dt0; the lse only when write_lse)
template <int D, int NDTP = D / 16>
__device__ __forceinline__ void attn_store(const AttnParams& p, int64_t row, int head, int g,
                                           const f32x4 (&oacc)[NDTP], float m_run, float l_run, int dt0 = 0,
                                           bool write_lse = true) {
    constexpr int NDT = NDTP;
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
        float4* dst = reinterpret_cast<float4*>(orow + 16 * (dt0 + dt) + 4 * g);
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
    if (write_lse && g == 0) p.lse[row * p.H + head] = lse_out;
}

// Unnormalised partial of one key split (a wave's 16 heads): each lane's
// 4 x D/16 accumulators stored contiguously (full 1 KB per wave instruction),
// the running max and sum per head, and for split 0 a snapshot of the lse to
// merge with (the merge kernel overwrites it).
template <int D>
__device__ __forceinline__ void attn_store_partial(const AttnParams& p, int64_t row, int split, int w, int lane,
                                                   int head, const f32x4 (&oacc)[D / 16], float m_run, float l_run) {
    constexpr int NDT = D / 16;
    float* po = p.part_o + ((row * p.nsplit + split) * p.H + 16 * w) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4*>(po + (dt * 64 + lane) * 4) = oacc[dt];
    if ((lane >> 4) == 0) {
        p.part_ml[(row * p.nsplit + split) * p.H + head] = make_float2(m_run, l_run);
        if (p.merge && split == 0) p.lse_prev[row * p.H + head] = p.lse[row * p.H + head];
    }
}

template <int D, bool QF32, int NW>
__global__ __launch_bounds__(64 * NW, 1) void attn_kernel(AttnParams p) {
    constexpr int RG = RING;
    constexpr int NBLK = D / 32;  // 32-channel blocks of the S MFMA
    constexpr int NDT = D / 16;   // 16-channel tiles of the O MFMA
    constexpr int CPR = D / 8;    // 16-byte chunks per fp16 key row
    constexpr int NT = 64 * NW;
    constexpr int ITEMS = 4 * CPR;  // dequantisation items per chunk
    using S = Stage<D>;
    __shared__ uint4 ktile[CHUNK_KEYS * (CPR + KROW_PAD)];
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
    // window: tokens wlo..qp, token t in ring row t mod T
    const int qp = p.Wp ? p.q_pos[row] : -1;
    const int wlo = max(0, qp - p.window + 1);
    const int wrow0 = p.Wp ? wlo % p.T : 0;

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
            const int i_w = kpos - p.Kp;  // window key i: token wlo + i (window <= T: no row repeats)
            if (wlo + i_w <= qp) r = (int64_t)b * p.T + (wrow0 + i_w >= p.T ? wrow0 + i_w - p.T : wrow0 + i_w);
        }
        krow[i] = r;
    }
    // LDS barrier only: the query loads stay in flight (each chunk's wait
    // below is for all of this wave's loads, so they are complete before S)
    lds_barrier();

    // ---- raw bytes of the first RG chunks start flowing into the LDS ring
    const int c_pre = min(c_hi, c_lo + RG);
    for (int ch = c_lo; ch < c_pre; ++ch) {
        ChunkRows<D, NW> cr;
        chunk_rows<D, NW>(ch < n_sp_chunks, krow + (ch - c_lo) * CHUNK_KEYS, w, lane, cr);
        chunk_issue<D, NW>(p, ch < n_sp_chunks, cr, ring + ((ch - c_lo) % RG) * S::SLOT, w, lane);
    }

    // ---- Q operand in fp16 (pre-scaled by a power of two)
    f16x8 qhi[NBLK];
    f16x8 qlo[QF32 ? NBLK : 1];
    const float zscale = q_operand<D, QF32>(qf, qraw, p.scale_log2, qhi, qlo);

    f32x4 oacc[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;

    int c_issued = c_pre;  // chunks [c_lo, c_issued) have been issued
    for (int ch = c_lo; ch < c_hi; ++ch) {
        // An opaque zero, fresh every chunk: the per-thread LDS addresses below
        // are recomputed from it (a few ALU ops) instead of living across the
        // loop in ~20 registers, which would spill next to the 128 output
        // accumulators and 64 query registers (and every spill reload waits
        // for all copies in flight, the ring's prefetch included).
        int zz;
        asm volatile("s_mov_b32 %0, 0" : "=s"(zz));
        const int tz = tid + zz;
        const int lz = tz & 63, gz = lz >> 4, cz = lz & 15;
        const bool sparse = ch < n_sp_chunks;
        const int64_t* kr = krow + (ch - c_lo) * CHUNK_KEYS;
        const uint8_t* st = ring + ((ch - c_lo) % RG) * S::SLOT;
        // ---- rows of the chunk the refill below copies, read now: they have
        // arrived by the barriers, so the refill issues its copies at once
        const bool refill = c_issued < c_hi;
        const bool nsparse = c_issued < n_sp_chunks;
        ChunkRows<D, NW> nr;
        if (refill) chunk_rows<D, NW>(nsparse, krow + (c_issued - c_lo) * CHUNK_KEYS, w, lz, nr);
        // ---- the chunk's copies have landed (all of this wave's copies: the
        // compiler cannot tell ring slots apart and would wait for them anyway)
        __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
        lds_barrier();  // every wave's copies have landed; the tiles are free
        // ---- dequantise the staged chunk into the LDS tiles
        if (sparse) {
#pragma unroll
            for (int it = 0; it < (ITEMS + NT - 1) / NT; ++it) {
                const int item = it * NT + tz;
                if (item < ITEMS) store_item<D, true>(st, item / CPR, item % CPR, ktile);
            }
        } else {
#pragma unroll
            for (int it = 0; it < (ITEMS + NT - 1) / NT; ++it) {
                const int item = it * NT + tz;
                if (item < ITEMS) store_item<D, false>(st, item / CPR, item % CPR, ktile);
            }
        }
        lds_barrier();
        // ---- the ring slot is free again: refill it with chunk ch + RG
        if (refill) {
            chunk_issue<D, NW>(p, nsparse, nr, ring + ((c_issued - c_lo) % RG) * S::SLOT, w, lz);
            ++c_issued;
        }
        attn_chunk<D, QF32>(ktile, kr, cz, gz, qhi, qlo, zscale, oacc, m_run, l_run);
    }

    if (p.nsplit > 1)
        attn_store_partial<D>(p, row, split, w, lane, head, oacc, m_run, l_run);
    else
        attn_store<D>(p, row, head, g, oacc, m_run, l_run);
}

// ---- D = 512, H = 64 with bf16 queries: prefill (no key split) and decode
// (keys split over workgroups, partials as in attn_kernel).  One workgroup of
// eight waves per CU.  Waves 0-3 consume (wave w: heads 16w..16w+15); waves
// 4-7 produce: producer p copies keys 4p..4p+3 of each chunk global -> LDS,
// PC_RING chunks ahead, and dequantises exactly those keys into one of
// PC_TILES tile buffers.  A producer only reads the copies it issued itself,
// so it waits on its own vector-memory counter and never on another wave.
// The consumers take the chunks in pairs: S for both chunks, one softmax over
// their 32 keys and one PV product over them on the K = 32 MFMA, while the
// producers fill the other pair's buffers; one workgroup barrier per pair
// hands the buffers over.  An odd chunk count gets a padding chunk whose keys
// have no row (weight exactly 0).
constexpr int PC_RING = 4;
constexpr int PC_TILES = 4;  // two pairs of chunk tiles
constexpr int PC_CONS = 4;   // consumer waves (16 heads each)
constexpr int PC_D = 512;
constexpr int PC_NT = 512;  // 4 consumer + 4 producer waves

// copies one producer issues per chunk (codes + scales, or 4 window rows)
__device__ __forceinline__ int pc_copies(bool sparse) { return sparse ? 2 : 4; }

// wait until at most n (0..15) of this wave's vector-memory operations are in flight
__device__ __forceinline__ void wait_vm_at_most(int n) {
#define CSA2_VMW(N) \
    case N: __builtin_amdgcn_s_waitcnt((N) | (7 << 4) | (15 << 8)); break;
    switch (n) {
        CSA2_VMW(0) CSA2_VMW(1) CSA2_VMW(2) CSA2_VMW(3) CSA2_VMW(4) CSA2_VMW(5) CSA2_VMW(6) CSA2_VMW(7)
        CSA2_VMW(8) CSA2_VMW(9) CSA2_VMW(10) CSA2_VMW(11) CSA2_VMW(12) CSA2_VMW(13) CSA2_VMW(14)
        default: __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (15 << 8)); break;
    }
#undef CSA2_VMW
}

// the same for n up to 31 (vmcnt's two high bits sit at bits 14-15 of the
// s_waitcnt immediate)
__device__ __forceinline__ void wait_vm_at_most32(int n) {
#define CSA2_VMW(N) \
    case N: __builtin_amdgcn_s_waitcnt(((N) & 15) | (((N) >> 4) << 14) | (7 << 4) | (15 << 8)); break;
    switch (n) {
        CSA2_VMW(0) CSA2_VMW(1) CSA2_VMW(2) CSA2_VMW(3) CSA2_VMW(4) CSA2_VMW(5) CSA2_VMW(6) CSA2_VMW(7)
        CSA2_VMW(8) CSA2_VMW(9) CSA2_VMW(10) CSA2_VMW(11) CSA2_VMW(12) CSA2_VMW(13) CSA2_VMW(14) CSA2_VMW(15)
        CSA2_VMW(16) CSA2_VMW(17) CSA2_VMW(18) CSA2_VMW(19) CSA2_VMW(20) CSA2_VMW(21) CSA2_VMW(22) CSA2_VMW(23)
        CSA2_VMW(24) CSA2_VMW(25) CSA2_VMW(26) CSA2_VMW(27) CSA2_VMW(28) CSA2_VMW(29) CSA2_VMW(30)
        default: __builtin_amdgcn_s_waitcnt(15 | (1 << 14) | (1 << 15) | (7 << 4) | (15 << 8)); break;
    }
#undef CSA2_VMW
}

__device__ __forceinline__ uint32_t lds_addr(const void* ptr) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)ptr;
}

// Producer pw's copies of one chunk (kr: the chunk's 16 key rows) into its own
// quarter of a ring slot, bytes 4096 pw .. 4096 pw + 4095, whatever the kind:
// FP4 codes of keys 4pw..4pw+3 ([4][D/2]) from its start and their scales in
// the 256 bytes after them (key 4pw+i at +32 i; the upper half takes
// duplicate copies), or the four window rows ([4][2D]).  The producers do not
// wait for one another's ring reads, so no producer may copy into bytes that
// another one reads: a slot that changes kind (FP4 entries, then window rows,
// or back at a row's start) would otherwise have one producer's new copies
// land on another's unread ones.
constexpr int PC_QUARTER = 4096;
static_assert(4 * 2 * PC_D == PC_QUARTER && 4 * (PC_D / 2) + 256 <= PC_QUARTER, "a producer's quarter holds 4 window rows or 4 FP4 rows and their scales");
__device__ __forceinline__ void pc_issue(const AttnParams& p, bool sparse, const int64_t* kr, uint8_t* slot, int pw,
                                         int lane) {
    constexpr int D = PC_D;
    // an opaque zero, fresh every call: per-lane offsets are recomputed here
    // instead of being kept across the chunk loop as 64-bit addresses
    int z;
    asm volatile("s_mov_b32 %0, 0" : "=s"(z));
    const int lz = lane + z;
    const int64_t* k4 = kr + 4 * pw;
    if (sparse) {
        const int64_t rc = max(k4[lz >> 4], (int64_t)0);
        const int64_t rs = max(k4[(lz >> 3) & 3], (int64_t)0);
        dma16_to_lds(p.codes + rc * (D / 2) + (lz & 15) * 16, slot + pw * PC_QUARTER);
        dma4_to_lds(p.scales + rs * (D / 16) + (lz & 7) * 4, slot + pw * PC_QUARTER + 4 * (D / 2));
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t r = max(k4[i], (int64_t)0);
            dma16_to_lds(reinterpret_cast<const uint8_t*>(p.swa) + r * (2 * D) + lz * 16,
                         slot + pw * PC_QUARTER + i * (2 * D));
        }
    }
}

// Producer pw dequantises its keys 4pw..4pw+3 (channels 8co..8co+7) from a
// ring slot into a tile buffer.  The slot is read in one asm block with its
// own wait: the compiler cannot tell ring slots apart and would make these
// reads wait for every copy in flight.
template <bool SPARSE>
__device__ __forceinline__ void pc_store(const uint8_t* slot, int pw, int co, uint4* ktile) {
    constexpr int D = PC_D;
    uint32_t kh[4][4];
    if (SPARSE) {
        uint32_t cw[4], sb[4];
        const uint32_t ac = lds_addr(slot + pw * PC_QUARTER + co * 4);
        const uint32_t as = lds_addr(slot + pw * PC_QUARTER + 4 * (D / 2) + (co >> 1));
        asm volatile(
            "ds_read_b32 %0, %8\n"
            "ds_read_b32 %1, %8 offset:256\n"
            "ds_read_b32 %2, %8 offset:512\n"
            "ds_read_b32 %3, %8 offset:768\n"
            "ds_read_u8 %4, %9\n"
            "ds_read_u8 %5, %9 offset:32\n"
            "ds_read_u8 %6, %9 offset:64\n"
            "ds_read_u8 %7, %9 offset:96\n"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(cw[0]), "=&v"(cw[1]), "=&v"(cw[2]), "=&v"(cw[3]), "=&v"(sb[0]), "=&v"(sb[1]), "=&v"(sb[2]),
              "=&v"(sb[3])
            : "v"(ac), "v"(as)
            : "memory");
        item_from_fp4(cw, sb, kh);
    } else {
        typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
        u32x4_t r0, r1, r2, r3;
        const uint32_t a = lds_addr(slot + pw * PC_QUARTER + co * 16);
        asm volatile(
            "ds_read_b128 %0, %4\n"
            "ds_read_b128 %1, %4 offset:1024\n"
            "ds_read_b128 %2, %4 offset:2048\n"
            "ds_read_b128 %3, %4 offset:3072\n"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
            : "v"(a)
            : "memory");
        const uint4 u[4] = {make_uint4(r0.x, r0.y, r0.z, r0.w), make_uint4(r1.x, r1.y, r1.z, r1.w),
                            make_uint4(r2.x, r2.y, r2.z, r2.w), make_uint4(r3.x, r3.y, r3.z, r3.w)};
        item_from_bf16(u, kh);
    }
    // the tile writes of put_item, in one asm block for the same reason: the
    // compiler would make them wait for the copies in flight.  Key 4pw+i at
    // (4pw+i)(D/8+2)16 + 16co.
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    constexpr int KROWB = (D / 8 + KROW_PAD) * 16;
    static_assert(3 * KROWB < 65536, "ds offsets are 16-bit");
    const uint32_t ak = lds_addr(ktile) + (uint32_t)(4 * pw * KROWB + co * 16);
    const u32x4_t k0{kh[0][0], kh[0][1], kh[0][2], kh[0][3]}, k1{kh[1][0], kh[1][1], kh[1][2], kh[1][3]};
    const u32x4_t k2{kh[2][0], kh[2][1], kh[2][2], kh[2][3]}, k3{kh[3][0], kh[3][1], kh[3][2], kh[3][3]};
    asm volatile(
        "ds_write_b128 %0, %1\n"
        "ds_write_b128 %0, %2 offset:%c5\n"
        "ds_write_b128 %0, %3 offset:%c6\n"
        "ds_write_b128 %0, %4 offset:%c7"
        :
        : "v"(ak), "v"(k0), "v"(k1), "v"(k2), "v"(k3), "i"(KROWB), "i"(2 * KROWB), "i"(3 * KROWB)
        : "memory");
}

// Producer pw's four rows 4pw..4pw+3 of a tile that holds bf16 window rows
// as copied: converted to fp16 in place (lane l: channels 8l..8l+7).  Reads
// and writes in asm for the reason given at pc_store.
__device__ __forceinline__ void pc_convert_rows(uint4* ktile, int pw, int lane) {
    constexpr int D = PC_D;
    constexpr int KROWB = (D / 8 + KROW_PAD) * 16;
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    u32x4_t r0, r1, r2, r3;
    const uint32_t a = lds_addr(ktile) + (uint32_t)(4 * pw * KROWB + lane * 16);
    asm volatile(
        "ds_read_b128 %0, %4\n"
        "ds_read_b128 %1, %4 offset:%c5\n"
        "ds_read_b128 %2, %4 offset:%c6\n"
        "ds_read_b128 %3, %4 offset:%c7\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
        : "v"(a), "i"(KROWB), "i"(2 * KROWB), "i"(3 * KROWB)
        : "memory");
    const uint4 u[4] = {make_uint4(r0.x, r0.y, r0.z, r0.w), make_uint4(r1.x, r1.y, r1.z, r1.w),
                        make_uint4(r2.x, r2.y, r2.z, r2.w), make_uint4(r3.x, r3.y, r3.z, r3.w)};
    uint32_t kh[4][4];
    item_from_bf16(u, kh);
    const u32x4_t k0{kh[0][0], kh[0][1], kh[0][2], kh[0][3]}, k1{kh[1][0], kh[1][1], kh[1][2], kh[1][3]};
    const u32x4_t k2{kh[2][0], kh[2][1], kh[2][2], kh[2][3]}, k3{kh[3][0], kh[3][1], kh[3][2], kh[3][3]};
    asm volatile(
        "ds_write_b128 %0, %1\n"
        "ds_write_b128 %0, %2 offset:%c5\n"
        "ds_write_b128 %0, %3 offset:%c6\n"
        "ds_write_b128 %0, %4 offset:%c7"
        :
        : "v"(a), "v"(k0), "v"(k1), "v"(k2), "v"(k3), "i"(KROWB), "i"(2 * KROWB), "i"(3 * KROWB)
        : "memory");
}

// SPLIT: keys split over workgroups (partials merged afterwards); without it
// every workgroup takes its row's whole list.  NW consumer waves: 4 (wave w:
// heads 16w..16w+15), or 1 (heads 16z..16z+15 of grid z): a few decode rows
// split their heads over four workgroups as well as their keys, so that each
// workgroup loads a quarter of the query and writes a quarter of the partial.
template <bool SPLIT, int NW>
__global__ __launch_bounds__(64 * (NW + 4), 1) void attn_pc_kernel(AttnParams p) {
    constexpr int D = PC_D, NT = 64 * (NW + 4);
    constexpr int NBLK = D / 32, NDT = D / 16, CPR = D / 8;
    using S = Stage<D>;
    __shared__ uint4 ktile[PC_TILES][CHUNK_KEYS * (CPR + KROW_PAD)];
    __shared__ __attribute__((aligned(16))) uint8_t ring[PC_RING * S::SLOT];
    __shared__ int64_t krow[MAX_CPS * CHUNK_KEYS + CHUNK_KEYS];
    __shared__ uint32_t kval[MAX_CPS + 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool consumer = wv < NW;
    const int g = lane >> 4, c16 = lane & 15;
    const int64_t row = blockIdx.y;
    const int split = blockIdx.x;
    const int b = (int)(row / p.Q);
    const int hg = NW == 1 ? (int)blockIdx.z : wv;  // (consumers) head group
    const int head = 16 * hg + c16;
    const int nchunks = (p.Kp + p.Wp) / CHUNK_KEYS;
    // this workgroup's chunks: c_lo + c for local c in [0, nloc)
    const int c_lo = SPLIT ? split * p.cps : 0;
    const int nloc = SPLIT ? max(0, min(nchunks, c_lo + p.cps) - c_lo) : nchunks;
    // chunks are consumed in pairs; an odd count gets one padding chunk
    // whose keys have no row (finite copies of row 0, weight exactly 0)
    const int npad = nloc + (nloc & 1);
    const int n_sp = p.Kp / CHUNK_KEYS;
    const int qp = p.Wp ? p.q_pos[row] : -1;
    const int wlo = max(0, qp - p.window + 1);
    const int wrow0 = p.Wp ? wlo % p.T : 0;
    const int nk = nloc * CHUNK_KEYS;
    // a local chunk's kind (sparse or window); the padding chunk is copied as
    // the kind of the chunk after the range, or past the last chunk as the
    // last one's (either view is valid)
    auto sparse_chunk = [&](int c) {
        const int a = c_lo + c;
        return a < n_sp || (a >= nchunks && p.Wp == 0);
    };

    // ---- index loads first, then the consumers' query loads
    constexpr int KR_IT = (MAX_CPS * CHUNK_KEYS + CHUNK_KEYS + NT - 1) / NT;
    int32_t kent[KR_IT];
#pragma unroll
    for (int j = 0; j < KR_IT; ++j) {
        const int i = tid + j * NT;
        const int kpos = c_lo * CHUNK_KEYS + i;
        kent[j] = (i < nk && kpos < p.K) ? p.idx[row * p.K + kpos] : -1;
    }
    uint4 qraw[NBLK];
    if (consumer) {
        const uint16_t* qr = static_cast<const uint16_t*>(p.q) + (row * p.H + head) * D;
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk) qraw[blk] = *reinterpret_cast<const uint4*>(qr + 32 * blk + 8 * g);
    }
    // ---- physical rows of every key (-1: none), the padding chunk included
    // and one validity bit per key (bit k of kval[c]: key k of chunk c has a
    // row), from a wave ballot: the 16 keys of a chunk are 16 lanes of a wave
#pragma unroll
    for (int j = 0; j < KR_IT; ++j) {
        const int i = tid + j * NT;
        const int kpos = c_lo * CHUNK_KEYS + i;
        int64_t r = -1;
        if (i >= nk) {
        } else if (kpos < p.Kp) {
            if (kent[j] >= 0) r = phys_row(p.kvmap, b, kent[j]);
        } else {
            const int i_w = kpos - p.Kp;
            if (wlo + i_w <= qp) r = (int64_t)b * p.T + (wrow0 + i_w >= p.T ? wrow0 + i_w - p.T : wrow0 + i_w);
        }
        const uint64_t valid = __ballot(r >= 0);
        if (i < npad * CHUNK_KEYS) {
            krow[i] = r;
            if ((lane & 15) == 0) kval[i >> 4] = (uint32_t)(valid >> (lane & 48)) & 0xFFFFu;
        }
    }
    lds_barrier();

    f16x8 qhi[NBLK];
    f16x8 qlo[1];
    float zscale = 0.0f;
    f32x4 oacc[NDT];
    float m_run = -INFINITY, l_run = 0.0f;
    const int pw = wv - NW;
    int issued = 0;  // (producers) chunks whose copies this wave has issued
    // producer step for chunk c: wait for this wave's copies of it, dequantise
    // them into tile buffer c % PC_TILES, refill the freed ring slot
    auto produce = [&](int c) {
        int later = 0;
        for (int ch = c + 1; ch < issued; ++ch) later += pc_copies(sparse_chunk(ch));
        wait_vm_at_most(later);
        int zz;
        asm volatile("s_mov_b32 %0, 0" : "=s"(zz));
        const int co = lane + zz;
        const uint8_t* st = ring + (c % PC_RING) * S::SLOT;
        const int tb = c % PC_TILES;
        if (sparse_chunk(c))
            pc_store<true>(st, pw, co, ktile[tb]);
        else
            pc_store<false>(st, pw, co, ktile[tb]);
        if (issued < npad) {
            pc_issue(p, sparse_chunk(issued), krow + issued * CHUNK_KEYS, ring + (issued % PC_RING) * S::SLOT, pw,
                     lane);
            ++issued;
        }
    };
    if (consumer) {
        const float qf[1][8] = {};
        zscale = q_operand<D, false>(qf, qraw, p.scale_log2, qhi, qlo);
#pragma unroll
        for (int i = 0; i < NDT; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
        issued = min(npad, PC_RING);
        for (int ch = 0; ch < issued; ++ch)
            pc_issue(p, sparse_chunk(ch), krow + ch * CHUNK_KEYS, ring + ch * S::SLOT, pw, lane);
        if (npad > 0) {
            produce(0);
            produce(1);
        }
    }
    lds_barrier();

    // iteration j: consumers take chunks 2j, 2j+1 (tile buffers of one pair),
    // producers fill the other pair's buffers with chunks 2j+2, 2j+3
    for (int c = 0; c < npad; c += 2) {
        if (consumer) {
            int zz;
            asm volatile("s_mov_b32 %0, 0" : "=s"(zz));
            const int lz = lane + zz, cz = lz & 15, gz = lz >> 4;
            const uint4* ka = ktile[c % PC_TILES];
            const uint4* kb = ktile[(c + 1) % PC_TILES];
            f32x4 sa, sb;
            attn_scores2<D>(ka, kb, cz, gz, qhi, sa, sb);
            mfma_pipeline_hint<2 * NBLK, 1, 8>();
            const uint32_t mk = kval[c] | (kval[c + 1] << 16);
            const f16x8 pb = attn_weights2<NDT>(sa, sb, mk, gz, zscale, oacc, m_run, l_run);
            attn_pv2<D>(ka, kb, cz, gz, pb, oacc);
        } else if (c + 2 < npad) {
            produce(c + 2);
            produce(c + 3);
        }
        lds_barrier();
    }
    if (consumer) {
        if (SPLIT)
            attn_store_partial<D>(p, row, split, hg, lane, head, oacc, m_run, l_run);
        else
            attn_store<D>(p, row, head, g, oacc, m_run, l_run);
    }
}

// Many rows without a key split: one workgroup per CU takes the rows
// blockIdx.x, blockIdx.x + gridDim.x, ... in turn, so that a row's set-up and
// output overlap its neighbours' work instead of leaving the CU idle: the
// producers load the next row's key indices while the current row runs and,
// during its last chunk pair, turn them into key rows, issue the next row's
// first copies and dequantise its first pair; meanwhile the consumers store
// the current output and load the next row's query.  Chunks are numbered across rows (tile buffer
// and ring slot = running chunk number mod 4), so the next row's first pair
// lands in the buffers the current row's last pair does not use.  Producer pw
// sets up the rows of its own keys 4pw..4pw+3 of every chunk (it alone reads
// them) and one byte per chunk of the validity bits (byte pw of kvb[c]).
//
// STAGED: the selected entries come from an fp16 copy of the cache by logical
// position (p.k16, built once for a group of layers that share the cache and
// its selections, so that neither the many query rows of a prefill chunk nor
// the group's layers dequantise an entry again).  A producer then copies each
// of its keys as one 1 KB row global -> LDS straight into its row of one of
// eight tile buffers (no ring, no dequantisation), six chunks ahead of the
// consumers and across row boundaries; a window chunk's bf16 rows are
// converted to fp16 in place once they have landed.  The consumers are the
// same.
template <bool STAGED>
__global__ __launch_bounds__(PC_NT, 1) void attn_pcr_kernel(AttnParams p, int64_t rows) {
    constexpr int D = PC_D, NW = PC_CONS;
    constexpr int NBLK = D / 32, NDT = D / 16, CPR = D / 8;
    constexpr int KPL = (MAX_CPS + 1) * 4 / 64;  // (chunk, key) pairs per producer lane
    constexpr int NTILE = STAGED ? 8 : PC_TILES;  // tile buffers (a power of two)
    using S = Stage<D>;
    __shared__ uint4 ktile[NTILE][CHUNK_KEYS * (CPR + KROW_PAD)];
    __shared__ __attribute__((aligned(16))) uint8_t ring[STAGED ? 16 : PC_RING * S::SLOT];
    __shared__ int64_t krow[2][MAX_CPS * CHUNK_KEYS + CHUNK_KEYS];
    __shared__ uint32_t kvb[2][MAX_CPS + 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t G = gridDim.x;
    const int nchunks = (p.Kp + p.Wp) / CHUNK_KEYS;
    const int npad = nchunks + (nchunks & 1);
    const int n_sp = p.Kp / CHUNK_KEYS;
    int64_t row = blockIdx.x;

    if (wv < NW) {
        // ---------------------------------------------------------- consumers
        const int g = lane >> 4, c16 = lane & 15;
        const int head = 16 * wv + c16;
        auto load_q = [&](int64_t r, uint4(&qraw)[NBLK]) {
            const uint16_t* qr = static_cast<const uint16_t*>(p.q) + (r * p.H + head) * D;
#pragma unroll
            for (int blk = 0; blk < NBLK; ++blk) qraw[blk] = *reinterpret_cast<const uint4*>(qr + 32 * blk + 8 * g);
        };
        // validity bits of chunk c: producer pw's four keys in byte pw
        auto bits16 = [](uint32_t x) {
            return (x & 0xFu) | ((x >> 4) & 0xF0u) | ((x >> 8) & 0xF00u) | ((x >> 12) & 0xF000u);
        };
        f16x8 qhi[NBLK];
        f16x8 qlo[1];
        const float qf[1][8] = {};
        float zscale;
        {
            uint4 qraw[NBLK];
            load_q(row, qraw);
            zscale = q_operand<D, false>(qf, qraw, p.scale_log2, qhi, qlo);
        }
        f32x4 oacc[NDT];
#pragma unroll
        for (int i = 0; i < NDT; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        float m_run = -INFINITY, l_run = 0.0f;
        int gb = 0, buf = 0;  // running number of this row's chunk 0; key-row buffer
        lds_barrier();
        for (;;) {
            const uint32_t* kv = kvb[buf];
            auto pair = [&](int c, f32x4& sa, f32x4& sb) {
                int zz;
                asm volatile("s_mov_b32 %0, 0" : "=s"(zz));
                const int lz = lane + zz, cz = lz & 15, gz = lz >> 4;
                attn_scores2<D, 6>(ktile[(gb + c) & (NTILE - 1)], ktile[(gb + c + 1) & (NTILE - 1)], cz, gz, qhi, sa,
                                   sb);
                mfma_pipeline_hint<2 * NBLK, 1, 6>();
                (void)gz;
            };
            auto finish = [&](int c, const f32x4& sa, const f32x4& sb) {
                int zz;
                asm volatile("s_mov_b32 %0, 0" : "=s"(zz));
                const int lz = lane + zz, cz = lz & 15, gz = lz >> 4;
                const uint32_t mk = bits16(kv[c]) | (bits16(kv[c + 1]) << 16);
                const f16x8 pb = attn_weights2<NDT>(sa, sb, mk, gz, zscale, oacc, m_run, l_run);
                attn_pv2<D>(ktile[(gb + c) & (NTILE - 1)], ktile[(gb + c + 1) & (NTILE - 1)], cz, gz, pb, oacc);
            };
            for (int c = 0; c < npad - 2; c += 2) {
                f32x4 sa, sb;
                pair(c, sa, sb);
                finish(c, sa, sb);
                lds_barrier();
            }
            // last pair, this row's output, then the next row's query (its
            // load overlaps the producers' set-up of the next row)
            const bool more = row + G < rows;
            f32x4 sa, sb;
            pair(npad - 2, sa, sb);
            finish(npad - 2, sa, sb);
            attn_store<D>(p, row, head, g, oacc, m_run, l_run);
            if (!more) {
                lds_barrier();
                break;
            }
            // an opaque zero after the stores: the compiler may not clear the
            // accumulators early (two live copies of them do not fit)
            float z0;
            asm volatile("v_mov_b32 %0, 0" : "=v"(z0)::"memory");
            {
                uint4 qraw[NBLK];
                load_q(row + G, qraw);
                zscale = q_operand<D, false>(qf, qraw, p.scale_log2, qhi, qlo);
            }
#pragma unroll
            for (int i = 0; i < NDT; ++i) oacc[i] = f32x4{z0, z0, z0, z0};
            m_run = -INFINITY;
            l_run = 0.0f;
            row += G;
            gb += npad;
            buf ^= 1;
            lds_barrier();
        }
    } else if constexpr (STAGED) {
        // ---------------------------------------------------------- producers
        const int pw = wv - NW;
        constexpr int KROWB = (CPR + KROW_PAD) * 16;
        const int64_t row0 = blockIdx.x;
        const int64_t nloc = (rows - row0 + G - 1) / G;  // rows of this workgroup (>= 1)
        const int64_t total = nloc * npad;               // its chunks, numbered across its rows
        int32_t kent[KPL];
        auto load_idx = [&](int64_t r) {
#pragma unroll
            for (int j = 0; j < KPL; ++j) {
                const int t = lane + 64 * j;
                const int kpos = (t >> 2) * CHUNK_KEYS + 4 * pw + (t & 3);
                kent[j] = (kpos < p.K && (t >> 2) < npad) ? p.idx[r * p.K + kpos] : -1;
            }
        };
        // rows of the staged copy / window ring for row r into krow[bf],
        // validity bits into byte pw of kvb[bf]
        auto set_rows = [&](int64_t r, int bf) {
            const int b = (int)(r / p.Q);
            const int qp = p.Wp ? p.q_pos[r] : -1;
            const int wlo = max(0, qp - p.window + 1);
            const int wrow0 = p.Wp ? wlo % p.T : 0;
#pragma unroll
            for (int j = 0; j < KPL; ++j) {
                const int t = lane + 64 * j;
                const int c = t >> 2;
                const int kpos = c * CHUNK_KEYS + 4 * pw + (t & 3);
                int64_t rr = -1;
                if (c >= nchunks) {
                } else if (kpos < p.Kp) {
                    if (kent[j] >= 0) rr = (int64_t)b * p.n_stage + kent[j];
                } else {
                    const int i_w = kpos - p.Kp;
                    if (wlo + i_w <= qp)
                        rr = (int64_t)b * p.T + (wrow0 + i_w >= p.T ? wrow0 + i_w - p.T : wrow0 + i_w);
                }
                const uint64_t valid = __ballot(rr >= 0);
                if (c < npad) {
                    krow[bf][kpos] = rr;
                    if ((t & 3) == 0)
                        reinterpret_cast<uint8_t*>(kvb[bf])[4 * c + pw] = (uint8_t)((valid >> (lane & 60)) & 0xFu);
                }
            }
        };
        auto sparse_chunk = [&](int c) { return c < n_sp || (c >= nchunks && p.Wp == 0); };
        // chunks are issued in order: vis of them so far, the next being
        // chunk is_c of this workgroup's row is_k, into tile vis % NTILE
        int64_t vis = 0;
        int is_k = 0, is_c = 0;
        auto issue_next = [&]() {
            const bool sp = sparse_chunk(is_c);
            const int64_t* k4 = krow[is_k & 1] + is_c * CHUNK_KEYS + 4 * pw;
            uint8_t* tb = reinterpret_cast<uint8_t*>(ktile[vis & (NTILE - 1)]) + 4 * pw * KROWB;
            const uint8_t* base = sp ? reinterpret_cast<const uint8_t*>(p.k16) : reinterpret_cast<const uint8_t*>(p.swa);
            int z;
            asm volatile("s_mov_b32 %0, 0" : "=s"(z));
            const int lz = lane + z;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // a key without a row copies row 0: finite values, weight exactly 0
                const int64_t r = max(k4[i], (int64_t)0);
                dma16_to_lds(base + r * (2 * D) + lz * 16, tb + i * KROWB);
            }
            ++vis;
            if (++is_c == npad) {
                is_c = 0;
                ++is_k;
            }
        };
        // issue up to chunk lim_v - 1, never past row lim_k (whose key rows
        // are the newest set up)
        auto issue_upto = [&](int64_t lim_v, int lim_k) {
            while (vis < lim_v && vis < total && is_k <= lim_k) issue_next();
        };
        // chunk v (chunk c of its row) landed in its tile, converted if a window chunk
        auto produce = [&](int64_t v, int c) {
            wait_vm_at_most32(4 * (int)(vis - v - 1));
            if (!sparse_chunk(c)) pc_convert_rows(ktile[v & (NTILE - 1)], pw, lane);
        };
        load_idx(row0);
        set_rows(row0, 0);
        if (nloc > 1) {
            load_idx(row0 + G);
            set_rows(row0 + G, 1);
        }
        if (nloc > 2) load_idx(row0 + 2 * G);
        issue_upto(NTILE - 2, 1);
        produce(0, 0);
        produce(1, 1);
        lds_barrier();
        for (int k = 0;; ++k) {
            // the row after next's key rows (the buffer of the row before, all
            // of whose chunks have been issued) and the index list after that
            if (k >= 1 && k + 1 < nloc) {
                set_rows(row0 + (k + 1) * G, (k + 1) & 1);
                if (k + 2 < nloc) load_idx(row0 + (k + 2) * G);
            }
            for (int c = 0; c < npad; c += 2) {
                // the consumers take chunks v, v + 1; the tiles of v - 2 and
                // v - 1 are free again
                const int64_t v = (int64_t)k * npad + c;
                issue_upto(v + NTILE, k + 1);
                if (v + 2 < total) {
                    const int cn = c + 2 < npad ? c + 2 : 0;
                    produce(v + 2, cn);
                    produce(v + 3, cn + 1);
                }
                lds_barrier();
            }
            if (k + 1 >= nloc) break;
        }
    } else {
        // ---------------------------------------------------------- producers
        const int pw = wv - NW;
        // (chunk, key) pair t = lane + 64 j of this producer: chunk t / 4,
        // key 4 pw + t % 4 of it, position 16 (t / 4) + 4 pw + t % 4
        int32_t kent[KPL];
        auto load_idx = [&](int64_t r) {
#pragma unroll
            for (int j = 0; j < KPL; ++j) {
                const int t = lane + 64 * j;
                const int kpos = (t >> 2) * CHUNK_KEYS + 4 * pw + (t & 3);
                kent[j] = (kpos < p.K && (t >> 2) < npad) ? p.idx[r * p.K + kpos] : -1;
            }
        };
        // key rows of row r into krow[bf], validity bits into byte pw of kvb[bf]
        auto set_rows = [&](int64_t r, int bf) {
            const int b = (int)(r / p.Q);
            const int qp = p.Wp ? p.q_pos[r] : -1;
            const int wlo = max(0, qp - p.window + 1);
            const int wrow0 = p.Wp ? wlo % p.T : 0;
#pragma unroll
            for (int j = 0; j < KPL; ++j) {
                const int t = lane + 64 * j;
                const int c = t >> 2;
                const int kpos = c * CHUNK_KEYS + 4 * pw + (t & 3);
                int64_t rr = -1;
                if (c >= nchunks) {
                } else if (kpos < p.Kp) {
                    if (kent[j] >= 0) rr = phys_row(p.kvmap, b, kent[j]);
                } else {
                    const int i_w = kpos - p.Kp;
                    if (wlo + i_w <= qp)
                        rr = (int64_t)b * p.T + (wrow0 + i_w >= p.T ? wrow0 + i_w - p.T : wrow0 + i_w);
                }
                const uint64_t valid = __ballot(rr >= 0);
                if (c < npad) {
                    krow[bf][kpos] = rr;
                    if ((t & 3) == 0)
                        reinterpret_cast<uint8_t*>(kvb[bf])[4 * c + pw] = (uint8_t)((valid >> (lane & 60)) & 0xFu);
                }
            }
        };
        int gb = 0, buf = 0, issued = 0;
        auto sparse_chunk = [&](int c) { return c < n_sp || (c >= nchunks && p.Wp == 0); };
        auto issue = [&](int c) {
            pc_issue(p, sparse_chunk(c), krow[buf] + c * CHUNK_KEYS, ring + ((gb + c) % PC_RING) * S::SLOT, pw, lane);
        };
        auto produce = [&](int c) {
            int later = 0;
            for (int ch = c + 1; ch < issued; ++ch) later += pc_copies(sparse_chunk(ch));
            wait_vm_at_most(later);
            int zz;
            asm volatile("s_mov_b32 %0, 0" : "=s"(zz));
            const int co = lane + zz;
            const uint8_t* st = ring + ((gb + c) % PC_RING) * S::SLOT;
            uint4* kt = ktile[(gb + c) & 3];
            if (sparse_chunk(c))
                pc_store<true>(st, pw, co, kt);
            else
                pc_store<false>(st, pw, co, kt);
            if (issued < npad) {
                issue(issued);
                ++issued;
            }
        };
        // a row's first copies and first pair
        auto start_row = [&]() {
            issued = min(npad, PC_RING);
            for (int ch = 0; ch < issued; ++ch) issue(ch);
            produce(0);
            produce(1);
        };
        load_idx(row);
        set_rows(row, 0);
        if (row + G < rows) load_idx(row + G);
        start_row();
        lds_barrier();
        for (;;) {
            for (int c = 0; c < npad - 2; c += 2) {
                produce(c + 2);
                produce(c + 3);
                lds_barrier();
            }
            if (row + G >= rows) {
                lds_barrier();
                break;
            }
            row += G;
            gb += npad;
            buf ^= 1;
            set_rows(row, buf);
            if (row + G < rows) load_idx(row + G);
            start_row();
            lds_barrier();
        }
    }
}

// Merge the split partials: exact log-sum-exp combination, optionally together
// with the (o, lse) already in the output.  One workgroup (one wave: many
// small workgroups spread the loads over all CUs) = one row x one 16-head
// group x one of its 16-column tiles; thread = one lane-order float4
// (head 16 hg + lane % 16, columns 16 dt + 4 (lane / 16) .. +3).  Splits are
// taken NB at a time (all loads of a batch issued before any arithmetic) with
// a running maximum across batches.
template <int NB>
__global__ __launch_bounds__(64) void attn_merge_kernel(const float* __restrict__ part_o,
                                                         const float2* __restrict__ part_ml,
                                                         const float* __restrict__ lse_prev, int nsplit, int H, int D,
                                                         int merge, float* __restrict__ o, float* __restrict__ lse) {
    const int64_t row = blockIdx.x;
    const int hg = blockIdx.y;
    const int t = threadIdx.x, lane = t & 63;
    const int dt = blockIdx.z;
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

// compute units of the current device (cached per device)
// fp16 copy of a cache's entries by logical position: one wave per entry,
// lane l decodes channels 8l..8l+7 (four code bytes and their scale) with the
// producers' arithmetic (bit for bit the tile they would write); an entry
// without a page, or past the sequence's addressable capacity, is zero.
__global__ __launch_bounds__(256) void stage_cache_kernel(const uint8_t* __restrict__ codes,
                                                          const uint8_t* __restrict__ scales, RowMap map,
                                                          int64_t nrows, int64_t n_stage, uint16_t* __restrict__ k16) {
    constexpr int D = PC_D;
    const int64_t e = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (e >= nrows) return;
    const int b = (int)(e / n_stage);
    const int64_t j = e - (int64_t)b * n_stage;
    const int64_t r = j < map.capacity ? phys_row(map, b, j) : -1;
    uint32_t o[4] = {0u, 0u, 0u, 0u};
    if (r >= 0) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + r * (D / 2) + lane * 4);
        const uint32_t sc = scales[r * (D / 16) + (lane >> 1)];
        fp4x8_to_f16(w, e4m3_f16x2_over256(sc), o);
    }
    reinterpret_cast<uint4*>(k16 + e * D)[lane] = make_uint4(o[0], o[1], o[2], o[3]);
}

int device_cus() {
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

int choose_nsplit(int64_t rows, int nchunks) {
    if (nchunks <= 1) return 1;
    // one resident workgroup per CU (its LDS ring holds one): about 256
    // workgroups run in a single round, more only add rounds and partials
    int64_t want = (256 + rows - 1) / rows;
    // at least RING chunks per split: a workgroup has RING chunks in flight, so
    // a shorter split costs the same time and only adds partials to write and
    // merge (measured at 4 and 8 decode rows)
    int64_t by_chunks = (nchunks + RING - 1) / RING;
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
                        const int32_t* q_pos, int32_t window, float sm_scale, int32_t merge, float* o, float* lse,
                        void* ws, size_t ws_bytes, hipStream_t stream, const char* what, const uint16_t* k16,
                        int64_t n_stage) {
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
        CSA2_ARG(swa && q_pos && T > 0, "%s: null window rows / q_pos or T <= 0", what);
        CSA2_ARG(window <= T, "%s: window=%d exceeds the ring's T=%d rows", what, window, T);
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
    p.q_pos = q_pos;
    p.window = window;
    p.Wp = (window + CHUNK_KEYS - 1) / CHUNK_KEYS * CHUNK_KEYS;
    p.scale_log2 = sm_scale * 1.4426950408889634f;
    p.merge = merge ? 1 : 0;
    p.o = o;
    p.lse = lse;
    const int nchunks = (p.Kp + p.Wp) / CHUNK_KEYS;
    p.nsplit = choose_nsplit(rows, nchunks);
    {
        // a split decode launch of the producer/consumer kernel (D = 512,
        // H = 64, bf16 queries) also splits the heads over four workgroups
        // when all of them fit in one round over the CUs: with a few more
        // rows than that allows, fewer key splits (at least two) make it fit
        const int64_t hw = H / 16;
        if (D == 512 && hw == 4 && qt == CSA2_BF16 && p.nsplit > 1 && rows * p.nsplit * hw > 256 &&
            256 / (rows * hw) >= 2)
            p.nsplit = (int)(256 / (rows * hw));
    }
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
    // D = 512, H = 64, bf16 queries: the producer/consumer kernel, with or
    // without a key split (the fp32 query's extra 64 registers do not fit);
    // the split instance is separate so that the prefill one keeps its
    // registers for the unsplit loop
    const bool wide = D == 512 && nw == 4 && !f32;
    // few rows: the head groups split over workgroups too, while every
    // workgroup still fits in one round over the CUs (one per CU)
    const bool hsplit = wide && p.nsplit > 1 && rows * p.nsplit * nw <= 256;
    if (hsplit) attn_pc_kernel<true, 1><<<dim3(grid.x, grid.y, (unsigned)nw), dim3(64 * 5), 0, stream>>>(p);
    if (wide && p.nsplit > 1 && !hsplit) attn_pc_kernel<true, PC_CONS><<<grid, dim3(PC_NT), 0, stream>>>(p);
    // many rows: one persistent workgroup per CU walks over them
    const int64_t ncu = device_cus();
    // an fp16 copy of the entries (a prefill group): the staged persistent kernel
    const bool staged = wide && p.nsplit == 1 && nchunks >= 2 && k16 != nullptr && K > 0;
    if (staged) {
        p.k16 = k16;
        p.n_stage = n_stage;
        attn_pcr_kernel<true><<<dim3((unsigned)(rows < ncu ? rows : ncu)), dim3(PC_NT), 0, stream>>>(p, rows);
    }
    const bool persist = !staged && wide && p.nsplit == 1 && rows > ncu && nchunks >= 2;
    if (persist) attn_pcr_kernel<false><<<dim3((unsigned)ncu), dim3(PC_NT), 0, stream>>>(p, rows);
    if (wide && p.nsplit == 1 && !persist && !staged)
        attn_pc_kernel<false, PC_CONS><<<grid, dim3(PC_NT), 0, stream>>>(p);
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
        const dim3 mg((unsigned)rows, (unsigned)(H / 16), (unsigned)(D / 16)), mb(64);
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

// Staging pays when a sequence's entries are selected several times per layer
// on average (many query rows of one sequence: a prefill chunk) and the
// persistent kernel applies (D = 512, H = 64, at least a round of rows).
bool attn_stage_applicable(int32_t B, int32_t Q, int32_t H, int32_t D, int32_t K) {
    (void)B;
    return D == PC_D && H == 16 * PC_CONS && K > 0 && Q >= 256;
}

size_t attn_stage_bytes(int32_t B, int32_t Q, int32_t H, int32_t D, int32_t n_max, int32_t K) {
    if (!attn_stage_applicable(B, Q, H, D, K) || n_max <= 0 || (int64_t)Q * K < 2 * (int64_t)n_max) return 0;
    return (size_t)B * (size_t)n_max * (size_t)D * 2;
}

csa2_status attn_stage_cache(const csa2_fp4_kv* kv, int32_t B, int64_t n_stage, uint16_t* k16, hipStream_t stream) {
    const char* what = "layer_forward (staging)";
    CSA2_ARG(kv && kv->codes && kv->scales && k16, "%s: null cache view or staging buffer", what);
    CSA2_REQUIRE(kv->D == PC_D, CSA2_EUNSUPPORTED, "%s: D=%d (staging supports 512)", what, kv->D);
    CSA2_ARG(B > 0 && n_stage > 0, "%s: B=%d n=%lld", what, B, (long long)n_stage);
    CSA2_ARG(aligned(kv->codes, 4) && aligned(k16, 16), "%s: codes must be 4-byte, the copy 16-byte aligned", what);
    RowMap m{};
    csa2_status st = make_rowmap(kv->page_table, kv->page_size, kv->max_pages, kv->seq_stride, 1, &m, what);
    if (st != CSA2_OK) return st;
    const int64_t nrows = (int64_t)B * n_stage;
    stage_cache_kernel<<<dim3((unsigned)((nrows + 3) / 4)), dim3(256), 0, stream>>>(kv->codes, kv->scales, m, nrows,
                                                                                   n_stage, k16);
    return launch_status(what);
}

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
                                     const uint16_t* swa_kv, int32_t T, const int32_t* q_pos, int32_t window,
                                     float sm_scale, int32_t merge, float* o, float* lse, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
    clear_error();
    CSA2_ARG(window >= 1, "swa_attn: window=%d must be >= 1", window);
    return attn_launch(q, qt, B, Q, H, D, nullptr, nullptr, 0, swa_kv, T, q_pos, window, sm_scale, merge, o, lse, ws,
                       ws_bytes, stream, "swa_attn");
}
