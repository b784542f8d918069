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
// Workgroup tile: 128 output columns x 128 tokens, 4 waves of 64 x 64.  The
// operand tiles (32 channels deep) stream global -> LDS by LDS DMA through a
// 4-deep ring of separate LDS arrays (three k-steps in flight while one is
// multiplied); 16-byte chunks are XOR-swizzled so that each 16-lane operand
// read hits 16 distinct bank groups.
#include "internal.h"

namespace csa2 {
namespace {

constexpr int RP_MAX_LAYERS = 48;
constexpr int RP_TILE = 128;   // output columns (D) and tokens (M) per workgroup
constexpr int RP_KS = 32;      // channels per k-step (one MFMA deep)
constexpr int RP_NST = 4;      // ring depth
constexpr int RP_HALF = RP_TILE * RP_KS * 2;  // bytes of one operand tile per k-step (8 KB)

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

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__global__ __launch_bounds__(256, 2) void swa_replay_kernel(ReplayParams p) {
    // ring of k-steps: [W tile 128 x 32 | h tile 128 x 32] bf16, swizzled chunks
    __shared__ __attribute__((aligned(16))) uint8_t st0[2 * RP_HALF];
    __shared__ __attribute__((aligned(16))) uint8_t st1[2 * RP_HALF];
    __shared__ __attribute__((aligned(16))) uint8_t st2[2 * RP_HALF];
    __shared__ __attribute__((aligned(16))) uint8_t st3[2 * RP_HALF];

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
    const int n0 = nt * RP_TILE, m0 = mt * RP_TILE;
    const uint16_t* __restrict__ Wl = p.W[layer];
    const uint16_t* __restrict__ hl = p.h[layer];

    // ---- this lane's four DMA sources per k-step: wave w copies 16-byte chunk
    // positions (4w + j) * 64 + lane of the 1024 in a k-step (W tile first)
    const char* src[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int q = (4 * w + j) * 64 + lane;
        const bool is_h = q >= 512;
        const int pos = q & 511;
        const int r = pos >> 2, c = (pos & 3) ^ ((r >> 2) & 3);
        const int64_t grow = is_h ? min(m0 + r, p.M - 1) : min(n0 + r, p.D - 1);
        src[j] = reinterpret_cast<const char*>(is_h ? hl : Wl) + (grow * p.dm + 8 * c) * 2;
    }
    const int dst_off = (4 * w) % 8 * 1024 + (w >= 2 ? RP_HALF : 0);  // + j * 1024

    const int nk = p.dm / RP_KS;
    auto issue = [&](int ks, uint8_t* buf) {
        const int64_t kb = (int64_t)ks * RP_KS * 2;
#pragma unroll
        for (int j = 0; j < 4; ++j) rp_dma16(src[j] + kb, buf + dst_off + j * 1024);
    };

    // ---- operand reads: lane (c16, g) reads row 16a + c16 of its wave's band,
    // channels 8g..8g+7 of the k-step, at chunk g ^ (c16 / 4)
    const int c16 = lane & 15, g = lane >> 4;
    const int wn = w & 1, wm = w >> 1;
    const int rd_w = (wn * 64 + c16) * 64 + ((g ^ (c16 >> 2)) << 4);
    const int rd_h = RP_HALF + (wm * 64 + c16) * 64 + ((g ^ (c16 >> 2)) << 4);

    f32x4 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    bf16x8 wa[4], hb[4];
    auto read_ops = [&](const uint8_t* buf) {
#pragma unroll
        for (int a = 0; a < 4; ++a) wa[a] = *reinterpret_cast<const bf16x8*>(buf + rd_w + a * 1024);
#pragma unroll
        for (int b = 0; b < 4; ++b) hb[b] = *reinterpret_cast<const bf16x8*>(buf + rd_h + b * 1024);
    };
    auto multiply = [&]() {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[a], hb[b], acc[a][b], 0, 0, 0);
    };

    // ---- prologue: k-steps 0..2 in flight.  Exactly three k-steps are always
    // in flight (past the end the last one is copied again into a slot that is
    // never read), so every wait below is the same unconditional vmcnt(8)
    issue(0, st0);
    issue(min(1, nk - 1), st1);
    issue(min(2, nk - 1), st2);
    // ---- four k-steps per trip so that every ring slot is a distinct LDS
    // object at each use; the first trip is peeled so that the copies in
    // flight at the loop head are in the same order on every path (the
    // compiler then sees that a slot's operands do not wait on later refills)
    auto trip = [&](int k0) {
#pragma unroll
        for (int u = 0; u < RP_NST; ++u) {
            const int ks = k0 + u;
            if (ks < nk) {
                rp_wait_vm<8>();  // this wave's copies of ks landed (ks+1, ks+2 may fly)
                rp_barrier();     // every wave's copies of ks landed; slot of ks-1 free
                // operands first: the refill issued next cannot alias them
                read_ops(u == 0 ? st0 : u == 1 ? st1 : u == 2 ? st2 : st3);
                issue(min(ks + 3, nk - 1), u == 0 ? st3 : u == 1 ? st0 : u == 2 ? st1 : st2);
                multiply();
            }
        }
    };
    trip(0);
    for (int k0 = RP_NST; k0 < nk; k0 += RP_NST) trip(k0);
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
    CSA2_ARG(a->d_model > 0 && a->d_model % 32 == 0, "swa_replay: d_model=%d must be a positive multiple of 32",
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
    p.n_tiles = (a->D + RP_TILE - 1) / RP_TILE;
    p.m_tiles = (int32_t)((M + RP_TILE - 1) / RP_TILE);
    p.n_layers = a->n_layers;
    const int64_t G = (int64_t)p.n_tiles * p.m_tiles * p.n_layers;
    CSA2_ARG(G <= INT32_MAX, "swa_replay: %lld tiles", (long long)G);
    swa_replay_kernel<<<(unsigned)G, 256, 0, stream>>>(p);
    return launch_status("swa_replay");
}
