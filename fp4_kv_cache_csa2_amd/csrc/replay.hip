// SWA Bounded Replay: a layer's missing 128-token window is rebuilt from its
// last tokens instead of being persisted (gkm0120.cn survey, section 2.1;
// aprilzz.com V4.1 Flash article, sections "把 prefill 砍掉一半" and
// "FP4 KV 与部署层的几个改动"; aimodeling.com, "第三层").  Each layer's window
// row of token p is its window projection of the layer input at p,
// kv_p = bf16(h_p W^T), stored in ring row p mod T.
//
// One launch covers every layer (grid z).  Per layer this is a bf16 GEMM
// C^T[D][M] = W[D][d_model] . h[M][d_model]^T (M = B x n tokens) on
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation; computing C^T puts four
// consecutive output columns of one token in each lane, stored as 8 bytes.
// Workgroup tile: 256 output columns x 128 tokens, 8 waves of 64 x 64, one
// workgroup per CU.  Each k-step copies one 128-byte line (64 channels) of
// every W and h row of the tile global -> LDS by LDS DMA (whole-line requests
// move about 1.4x the bytes per second of half-line ones here) through a
// 3-deep ring of separate LDS arrays (two k-steps in flight while one is
// multiplied); 16-byte chunks are XOR-swizzled so that each 16-lane operand
// read hits 16 distinct bank groups.  The tile is as large as the LDS ring
// allows: every workgroup pulls its rows through its CU's path from L2, so
// bytes per CU, not HBM, bound this kernel at these sizes.
#include "internal.h"

namespace csa2 {
namespace {

constexpr int RP_MAX_LAYERS = 48;
constexpr int RP_TN = 256;     // output columns (D, rows of W) per workgroup
constexpr int RP_TM = 128;     // tokens (rows of h) per workgroup
constexpr int RP_KS = 64;      // channels per k-step: one 128-byte line of every row
constexpr int RP_NST = 3;      // ring depth (two k-steps in flight while one is multiplied)
constexpr int RP_WAVES = 8;    // 4 x 2 waves of 64 x 64
constexpr int RP_STAGE = (RP_TN + RP_TM) * RP_KS * 2;  // 48 KB per k-step
constexpr int RP_H_OFF = RP_TN * RP_KS * 2;            // h rows after the W rows
constexpr int RP_NJ = RP_STAGE / 1024 / RP_WAVES;      // DMA instructions per wave per k-step (6)

struct ReplayParams {
    int32_t M, n, dm, D, T;
    int32_t n_tiles, m_tiles, n_layers;
    const int32_t* t_end;
    const uint16_t* h[RP_MAX_LAYERS];
    const uint16_t* W[RP_MAX_LAYERS];
    uint16_t* ring[RP_MAX_LAYERS];
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void rp_dma16(const void* src, void* lds_base) {
    __builtin_amdgcn_global_load_lds((gbl_ptr_t)(const_cast<void*>(src)), (lds_ptr_t)lds_base, 16, 0, 0);
}

// LDS-only workgroup barrier (this wave's LDS instructions drained; the DMA
// copies the caller needs have been waited for explicitly).
__device__ __forceinline__ void rp_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// wait until at most N of this wave's vector-memory operations are in flight
template <int N>
__device__ __forceinline__ void rp_wait_vm() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)p;
}

// The eight MFMA operands of one 32-channel half k-step: four W rows and four
// h rows 2 KB apart.  Written as one asm block that also waits for the reads:
// the compiler cannot tell the ring slots apart and would otherwise make every
// read wait for all LDS copies still in flight.
__device__ __forceinline__ void read_operands(uint32_t aw, uint32_t ah, bf16x8 (&wa)[4], bf16x8 (&hb)[4]) {
    u32x4 r0, r1, r2, r3, r4, r5, r6, r7;
    asm volatile(
        "ds_read_b128 %0, %8\n"
        "ds_read_b128 %1, %8 offset:2048\n"
        "ds_read_b128 %2, %8 offset:4096\n"
        "ds_read_b128 %3, %8 offset:6144\n"
        "ds_read_b128 %4, %9\n"
        "ds_read_b128 %5, %9 offset:2048\n"
        "ds_read_b128 %6, %9 offset:4096\n"
        "ds_read_b128 %7, %9 offset:6144\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
        : "v"(aw), "v"(ah)
        : "memory");
    wa[0] = __builtin_bit_cast(bf16x8, r0);
    wa[1] = __builtin_bit_cast(bf16x8, r1);
    wa[2] = __builtin_bit_cast(bf16x8, r2);
    wa[3] = __builtin_bit_cast(bf16x8, r3);
    hb[0] = __builtin_bit_cast(bf16x8, r4);
    hb[1] = __builtin_bit_cast(bf16x8, r5);
    hb[2] = __builtin_bit_cast(bf16x8, r6);
    hb[3] = __builtin_bit_cast(bf16x8, r7);
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__global__ __launch_bounds__(64 * RP_WAVES, 1) void swa_replay_kernel(ReplayParams p) {
    // ring of k-steps: [W tile 256 x 64 | h tile 128 x 64] bf16, one 128-byte
    // row each, 16-byte chunks swizzled
    __shared__ __attribute__((aligned(16))) uint8_t st0[RP_STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st1[RP_STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st2[RP_STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // workgroups are dealt to the 8 XCDs round-robin by id; renumber them so
    // that each XCD runs a contiguous range of tiles (column tile fastest, then
    // token tile, then layer): the workgroups sharing an h tile, and mostly
    // those sharing a layer's W, then meet in the same L2
    const int G = p.n_tiles * p.m_tiles * p.n_layers;
    const int xcd = blockIdx.x % 8, k = blockIdx.x / 8;
    const int per = G / 8, rem = G % 8;
    const int lin = xcd * per + min(xcd, rem) + k;
    const int nt = lin % p.n_tiles, mt = (lin / p.n_tiles) % p.m_tiles, layer = lin / (p.n_tiles * p.m_tiles);
    const int n0 = nt * RP_TN, m0 = mt * RP_TM;
    const uint16_t* __restrict__ Wl = p.W[layer];
    const uint16_t* __restrict__ hl = p.h[layer];

    // ---- this lane's DMA sources: wave w copies 16-byte chunk positions
    // (6w + j) * 64 + lane of the 3072 in a k-step (2048 of W, then 1024 of h);
    // position (r, c') holds channel chunk c = c' ^ ((r / 2) % 8) of row r
    const char* src[RP_NJ];
#pragma unroll
    for (int j = 0; j < RP_NJ; ++j) {
        const int q = (RP_NJ * w + j) * 64 + lane;
        const bool is_h = q >= RP_TN * 8;
        const int pos = is_h ? q - RP_TN * 8 : q;
        const int r = pos >> 3, c = (pos & 7) ^ ((r >> 1) & 7);
        const int64_t grow = is_h ? min(m0 + r, p.M - 1) : min(n0 + r, p.D - 1);
        src[j] = reinterpret_cast<const char*>(is_h ? hl : Wl) + (grow * p.dm + 8 * c) * 2;
    }
    const int dst_off = RP_NJ * w * 1024;  // + j * 1024

    const int nk = p.dm / RP_KS;
    auto issue = [&](int ks, uint8_t* buf) {
        const int64_t kb = (int64_t)ks * RP_KS * 2;
#pragma unroll
        for (int j = 0; j < RP_NJ; ++j) rp_dma16(src[j] + kb, buf + dst_off + j * 1024);
    };

    // ---- operand reads: lane (c16, g) reads rows 16a + c16 of its wave's W
    // band and h band, channel chunk 4 kh + g of half k-step kh
    const int c16 = lane & 15, g = lane >> 4;
    const int wn = w & 3, wm = w >> 2;
    const int rw = (wn * 64 + c16) * 128, rh = RP_H_OFF + (wm * 64 + c16) * 128;
    const int ch0 = (g ^ (c16 >> 1)) << 4, ch1 = ((4 + g) ^ (c16 >> 1)) << 4;

    f32x4 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    bf16x8 wa0[4], hb0[4], wa1[4], hb1[4];
    auto multiply = [&](const bf16x8 (&wa)[4], const bf16x8 (&hb)[4]) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[a], hb[b], acc[a][b], 0, 0, 0);
    };

    // ---- prologue: two k-steps in flight.  Exactly two are always in flight
    // (past the end the last one is copied again into a slot that is never
    // read), so every wait below is the same unconditional one
    issue(0, st0);
    issue(min(1, nk - 1), st1);
    auto trip = [&](int k0) {
#pragma unroll
        for (int u = 0; u < RP_NST; ++u) {
            const int ks = k0 + u;
            if (ks < nk) {
                uint8_t* cur = u == 0 ? st0 : u == 1 ? st1 : st2;
                rp_wait_vm<RP_NJ>();  // this wave's copies of ks landed (ks + 1 may fly)
                rp_barrier();         // every wave's copies of ks landed; slot of ks - 1 free
                issue(min(ks + 2, nk - 1), u == 0 ? st2 : u == 1 ? st0 : st1);
                const uint32_t base = lds_addr(cur);
                read_operands(base + rw + ch0, base + rh + ch0, wa0, hb0);
                multiply(wa0, hb0);
                read_operands(base + rw + ch1, base + rh + ch1, wa1, hb1);
                multiply(wa1, hb1);
            }
        }
    };
    for (int k0 = 0; k0 < nk; k0 += RP_NST) trip(k0);
    rp_wait_vm<0>();  // no copy may land in LDS after the workgroup ends

    // ---- epilogue: acc[a][b][i] = C^T[n0 + 64wn + 16a + 4g + i][m0 + 64wm + 16b + c16]
    uint16_t* __restrict__ ring = p.ring[layer];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int m = m0 + wm * 64 + 16 * b + c16;
        if (m >= p.M) continue;
        const int seq = m / p.n, i = m - seq * p.n;
        const int64_t pos = (int64_t)p.t_end[seq] - p.n + 1 + i;
        if (pos < 0) continue;
        uint16_t* row = ring + ((int64_t)seq * p.T + pos % p.T) * p.D;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int col = n0 + wn * 64 + 16 * a + 4 * g;
            if (col >= p.D) continue;
            const f32x4 v = acc[a][b];
            uint2 o;
            o.x = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
            o.y = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
            *reinterpret_cast<uint2*>(row + col) = o;
        }
    }
}

}  // namespace
}  // namespace csa2

using namespace csa2;

extern "C" csa2_status csa2_swa_replay(const csa2_replay_args* a, hipStream_t stream) {
    clear_error();
    CSA2_ARG(a != nullptr, "swa_replay: null args");
    CSA2_ARG(a->B >= 0 && a->n >= 0, "swa_replay: B=%d n=%d must be >= 0", a->B, a->n);
    CSA2_ARG(a->T > 0 && a->n <= a->T, "swa_replay: n=%d must be in [0, T=%d]", a->n, a->T);
    CSA2_ARG(a->d_model > 0 && a->d_model % 64 == 0, "swa_replay: d_model=%d must be a positive multiple of 64",
             a->d_model);
    CSA2_ARG(a->D > 0 && a->D % 16 == 0, "swa_replay: D=%d must be a positive multiple of 16", a->D);
    CSA2_ARG(a->n_layers >= 0 && a->n_layers <= RP_MAX_LAYERS, "swa_replay: n_layers=%d out of [0, %d]", a->n_layers,
             RP_MAX_LAYERS);
    const int64_t M = (int64_t)a->B * a->n;
    if (M == 0 || a->n_layers == 0) return CSA2_OK;
    CSA2_ARG(M <= INT32_MAX, "swa_replay: B x n = %lld too large", (long long)M);
    CSA2_ARG(a->t_end && a->h && a->W && a->swa_kv, "swa_replay: null pointer");
    ReplayParams p{};
    for (int l = 0; l < a->n_layers; ++l) {
        CSA2_ARG(a->h[l] && a->W[l] && a->swa_kv[l], "swa_replay: null pointer for layer %d", l);
        CSA2_ARG(aligned(a->h[l], 16) && aligned(a->W[l], 16) && aligned(a->swa_kv[l], 8),
                 "swa_replay: layer %d: h and W must be 16-byte, swa_kv 8-byte aligned", l);
        p.h[l] = a->h[l];
        p.W[l] = a->W[l];
        p.ring[l] = a->swa_kv[l];
    }
    p.M = (int32_t)M;
    p.n = a->n;
    p.dm = a->d_model;
    p.D = a->D;
    p.T = a->T;
    p.t_end = a->t_end;
    p.n_tiles = (a->D + RP_TN - 1) / RP_TN;
    p.m_tiles = (int32_t)((M + RP_TM - 1) / RP_TM);
    p.n_layers = a->n_layers;
    const int64_t G = (int64_t)p.n_tiles * p.m_tiles * p.n_layers;
    CSA2_ARG(G <= INT32_MAX, "swa_replay: %lld tiles", (long long)G);
    swa_replay_kernel<<<(unsigned)G, 64 * RP_WAVES, 0, stream>>>(p);
    return launch_status("swa_replay");
}
