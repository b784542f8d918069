// FP4 main-KV codec: E2M1 elements with one E4M3FN scale per 16 channels and
// no global scale (aprilzz.com V4.1 Flash article, section
// "FP4 KV 与部署层的几个改动"; element and scale formats per OCP MX v1.0 /
// OFP8).  One thread owns one 16-channel group: 64 B of fp32 in, 8 B of codes
// and 1 B of scale out, so a wavefront streams 4 KB in / 576 B out with
// contiguous, aligned accesses.
#include "common.h"

namespace csa2 {
namespace {

// E4M3FN code of the value nearest to amax/6, ties to even, saturating at 448.
// q = amax/6 is rounded to fp32 first; that rounding can land on an E4M3
// rounding boundary only if amax/6 is exactly on it (6 x any boundary fits in
// fp32), so rounding q again to 3 mantissa bits gives the exactly rounded result.
__device__ __forceinline__ uint32_t e4m3_scale_code(float amax) {
    float q = __fdiv_rn(amax, 6.0f);
    if (q >= 448.0f) return 0x7E;
    if (q < 0.015625f) {  // below 2^-6: subnormal grid of step 2^-9 (8 steps reach 2^-6 = code 0x08)
        return (uint32_t)rintf(q * 512.0f);
    }
    uint32_t u = __float_as_uint(q);
    int e = (int)(u >> 23) - 127;  // -6 .. 8
    uint32_t man = u & 0x7FFFFFu;
    uint32_t top = man >> 20, rem = man & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (top & 1u))) ++top;
    if (top == 8) { top = 0; ++e; }
    uint32_t code = ((uint32_t)(e + 7) << 3) | top;
    return code > 0x7Eu ? 0x7Eu : code;
}

__device__ __forceinline__ float e4m3_value(uint32_t code) {
    uint32_t e = (code >> 3) & 15, m = code & 7;
    if (e == 0) return (float)m * 0.001953125f;  // m/8 * 2^-6
    return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// E2M1 magnitude code of |x| on the grid {0,.5,1,1.5,2,3,4,6} x s, ties to the
// even code.  Every threshold m*s is exact in fp32 (<= 7 significant bits).
__device__ __forceinline__ uint32_t e2m1_mag(float a, float s) {
    return (uint32_t)(a > 0.25f * s) + (uint32_t)(a >= 0.75f * s) + (uint32_t)(a > 1.25f * s) +
           (uint32_t)(a >= 1.75f * s) + (uint32_t)(a > 2.5f * s) + (uint32_t)(a >= 3.5f * s) +
           (uint32_t)(a > 5.0f * s);
}

template <bool BF16>
__device__ __forceinline__ void load_group(const void* x, int64_t g, float v[16]) {
    if (BF16) {
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + g * 16);
        uint4 a = p[0], b = p[1];
        uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[2 * i] = bf16_lo(w[i]);
            v[2 * i + 1] = bf16_hi(w[i]);
        }
    } else {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + g * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float4 t = p[i];
            v[4 * i] = t.x;
            v[4 * i + 1] = t.y;
            v[4 * i + 2] = t.z;
            v[4 * i + 3] = t.w;
        }
    }
}

// Quantise one 16-channel group: returns the 8 code bytes, writes the scale.
__device__ __forceinline__ uint2 quantize_group(const float v[16], uint8_t* scale_out) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
    uint32_t sc = e4m3_scale_code(amax);
    float s = e4m3_value(sc);
    *scale_out = (uint8_t)sc;
    uint32_t w[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        uint32_t mag = (s == 0.0f) ? 0u : e2m1_mag(fabsf(v[i]), s);
        uint32_t code = ((__float_as_uint(v[i]) >> 31) << 3) | mag;
        w[i / 8] |= code << (4 * (i % 8));
    }
    return make_uint2(w[0], w[1]);
}

template <bool BF16>
__global__ __launch_bounds__(256) void fp4_quantize_kernel(const void* __restrict__ x, int64_t groups,
                                                           uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
    int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= groups) return;
    float v[16];
    load_group<BF16>(x, g, v);
    uint8_t sc;
    uint2 c = quantize_group(v, &sc);
    reinterpret_cast<uint2*>(codes)[g] = c;
    scales[g] = sc;
}

__global__ __launch_bounds__(256) void fp4_dequantize_kernel(const uint8_t* __restrict__ codes,
                                                             const uint8_t* __restrict__ scales, int64_t groups,
                                                             float* __restrict__ y) {
    int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= groups) return;
    uint2 c = reinterpret_cast<const uint2*>(codes)[g];
    float s = e4m3_value(scales[g]);
    uint32_t w[2] = {c.x, c.y};
    float out[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        uint32_t code = (w[i / 8] >> (4 * (i % 8))) & 15u;
        uint32_t mag = code & 7u;
        // E2M1: exponent field 0 -> m * 0.5; else 2^(e-1) * (1 + m/2)
        float a = (mag < 2u) ? 0.5f * (float)mag : __uint_as_float(((mag >> 1) + 126u) << 23 | (mag & 1u) << 22);
        float v = a * s;
        out[i] = (code & 8u) ? -v : v;
    }
    float4* yo = reinterpret_cast<float4*>(y + g * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) yo[i] = make_float4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
}

// Append: row b of x -> logical entry pos[b] of sequence b.
template <bool BF16>
__global__ __launch_bounds__(64) void fp4_append_kernel(const void* __restrict__ x, int32_t D,
                                                        const int32_t* __restrict__ pos, RowMap map,
                                                        uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
    int b = blockIdx.x;
    int64_t row = phys_row(map, b, pos[b]);
    int gpr = D / 16;
    for (int gi = threadIdx.x; gi < gpr; gi += blockDim.x) {
        float v[16];
        load_group<BF16>(x, (int64_t)b * gpr + gi, v);
        uint8_t sc;
        uint2 c = quantize_group(v, &sc);
        reinterpret_cast<uint2*>(codes + row * (D / 2))[gi] = c;
        scales[row * gpr + gi] = sc;
    }
}

constexpr int APPEND_MAX_LAYERS = 32;

struct AppendParams {
    const void* x;
    int32_t D, D_i, B, n_layers, T;
    const int32_t* pos;
    const int32_t* tok;
    RowMap kvmap, kmap;
    uint8_t* codes;
    uint8_t* scales;
    const uint16_t* k_new;
    uint16_t* k;
    const uint16_t* swa_new[APPEND_MAX_LAYERS];
    uint16_t* swa_kv[APPEND_MAX_LAYERS];
};

// Workgroup (b, role): role 0 quantises the FP4 entry, role 1 copies the
// indexer key, role 2 + l copies layer l's window row.
template <bool BF16>
__global__ __launch_bounds__(64) void append_token_kernel(AppendParams p) {
    const int b = blockIdx.x, role = blockIdx.y, t = threadIdx.x;
    if (role == 0) {
        const int64_t row = phys_row(p.kvmap, b, p.pos[b]);
        const int gpr = p.D / 16;
        for (int gi = t; gi < gpr; gi += blockDim.x) {
            float v[16];
            load_group<BF16>(p.x, (int64_t)b * gpr + gi, v);
            uint8_t sc;
            const uint2 c = quantize_group(v, &sc);
            reinterpret_cast<uint2*>(p.codes + row * (p.D / 2))[gi] = c;
            p.scales[row * gpr + gi] = sc;
        }
    } else if (role == 1) {
        if (p.k_new == nullptr) return;
        const int64_t row = phys_row(p.kmap, b, p.pos[b]);
        const uint4* src = reinterpret_cast<const uint4*>(p.k_new + (int64_t)b * p.D_i);
        uint4* dst = reinterpret_cast<uint4*>(p.k + row * p.D_i);
        for (int i = t; i < p.D_i / 8; i += blockDim.x) dst[i] = src[i];
    } else {
        const int l = role - 2;
        const uint4* src = reinterpret_cast<const uint4*>(p.swa_new[l] + (int64_t)b * p.D);
        // window ring: token t in row t mod T (a negative position names no token)
        const int tk = p.tok[b];
        if (tk < 0) return;
        const int t_row = tk % p.T;
        uint4* dst = reinterpret_cast<uint4*>(p.swa_kv[l] + ((int64_t)b * p.T + t_row) * p.D);
        for (int i = t; i < p.D / 8; i += blockDim.x) dst[i] = src[i];
    }
}

}  // namespace
}  // namespace csa2

using namespace csa2;

extern "C" csa2_status csa2_append_token(const csa2_append_args* a, hipStream_t stream) {
    clear_error();
    CSA2_ARG(a != nullptr && a->kv != nullptr, "append_token: null args or cache view");
    CSA2_ARG(a->B >= 0, "append_token: B=%d < 0", a->B);
    CSA2_ARG(a->kv->D > 0 && a->kv->D % 16 == 0, "append_token: D=%d must be a positive multiple of 16", a->kv->D);
    CSA2_ARG(a->xt == CSA2_F32 || a->xt == CSA2_BF16, "append_token: bad dtype %d", (int)a->xt);
    CSA2_ARG(a->n_layers >= 0 && a->n_layers <= APPEND_MAX_LAYERS, "append_token: n_layers=%d out of [0, %d]",
             a->n_layers, APPEND_MAX_LAYERS);
    if (a->B == 0) return CSA2_OK;
    CSA2_ARG(a->x && a->pos && a->kv->codes && a->kv->scales, "append_token: null pointer");
    CSA2_ARG(aligned(a->x, 16) && aligned(a->kv->codes, 8), "append_token: x must be 16-byte and codes 8-byte aligned");
    AppendParams p{};
    csa2_status st = make_rowmap(a->kv->page_table, a->kv->page_size, a->kv->max_pages, a->kv->seq_stride, 1,
                                 &p.kvmap, "append_token");
    if (st != CSA2_OK) return st;
    p.x = a->x;
    p.D = a->kv->D;
    p.B = a->B;
    p.pos = a->pos;
    p.codes = a->kv->codes;
    p.scales = a->kv->scales;
    if (a->k_new != nullptr) {
        CSA2_ARG(a->k != nullptr && a->k->k != nullptr, "append_token: k_new given without an indexer-K view");
        CSA2_ARG(a->k->D_i > 0 && a->k->D_i % 8 == 0, "append_token: D_i=%d must be a positive multiple of 8",
                 a->k->D_i);
        CSA2_ARG(aligned(a->k_new, 16) && aligned(a->k->k, 16), "append_token: k_new and k must be 16-byte aligned");
        st = make_rowmap(a->k->page_table, a->k->page_size, a->k->max_pages, a->k->seq_stride, 1, &p.kmap,
                         "append_token");
        if (st != CSA2_OK) return st;
        p.k_new = a->k_new;
        p.k = const_cast<uint16_t*>(a->k->k);
        p.D_i = a->k->D_i;
    }
    if (a->n_layers > 0) {
        CSA2_ARG(a->swa_new && a->swa_kv && a->tok && a->T > 0, "append_token: null window arrays / tok or T <= 0");
        for (int l = 0; l < a->n_layers; ++l) {
            CSA2_ARG(a->swa_new[l] && a->swa_kv[l], "append_token: null window row pointer of layer %d", l);
            CSA2_ARG(aligned(a->swa_new[l], 16) && aligned(a->swa_kv[l], 16),
                     "append_token: window rows of layer %d must be 16-byte aligned", l);
            p.swa_new[l] = a->swa_new[l];
            p.swa_kv[l] = a->swa_kv[l];
        }
        p.n_layers = a->n_layers;
        p.T = a->T;
        p.tok = a->tok;
    }
    const dim3 grid((unsigned)a->B, (unsigned)(2 + a->n_layers));
    if (a->xt == CSA2_BF16)
        append_token_kernel<true><<<grid, 64, 0, stream>>>(p);
    else
        append_token_kernel<false><<<grid, 64, 0, stream>>>(p);
    return launch_status("append_token");
}

extern "C" csa2_status csa2_fp4_quantize(const void* x, csa2_dtype xt, int64_t rows, int32_t D, uint8_t* codes,
                                         uint8_t* scales, hipStream_t stream) {
    clear_error();
    CSA2_ARG(rows >= 0, "fp4_quantize: rows=%lld < 0", (long long)rows);
    CSA2_ARG(D > 0 && D % 16 == 0, "fp4_quantize: D=%d must be a positive multiple of 16", D);
    CSA2_ARG(xt == CSA2_F32 || xt == CSA2_BF16, "fp4_quantize: bad dtype %d", (int)xt);
    if (rows == 0) return CSA2_OK;
    CSA2_ARG(x && codes && scales, "fp4_quantize: null pointer");
    CSA2_ARG(aligned(x, 16) && aligned(codes, 8), "fp4_quantize: x must be 16-byte and codes 8-byte aligned");
    int64_t groups = rows * (D / 16);
    dim3 grid((unsigned)((groups + 255) / 256));
    if (xt == CSA2_BF16)
        fp4_quantize_kernel<true><<<grid, 256, 0, stream>>>(x, groups, codes, scales);
    else
        fp4_quantize_kernel<false><<<grid, 256, 0, stream>>>(x, groups, codes, scales);
    return launch_status("fp4_quantize");
}

extern "C" csa2_status csa2_fp4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t D,
                                           float* y, hipStream_t stream) {
    clear_error();
    CSA2_ARG(rows >= 0, "fp4_dequantize: rows=%lld < 0", (long long)rows);
    CSA2_ARG(D > 0 && D % 16 == 0, "fp4_dequantize: D=%d must be a positive multiple of 16", D);
    if (rows == 0) return CSA2_OK;
    CSA2_ARG(codes && scales && y, "fp4_dequantize: null pointer");
    CSA2_ARG(aligned(codes, 8) && aligned(y, 16), "fp4_dequantize: codes must be 8-byte and y 16-byte aligned");
    int64_t groups = rows * (D / 16);
    fp4_dequantize_kernel<<<dim3((unsigned)((groups + 255) / 256)), 256, 0, stream>>>(codes, scales, groups, y);
    return launch_status("fp4_dequantize");
}

extern "C" csa2_status csa2_fp4_append(const void* x, csa2_dtype xt, int32_t B, const int32_t* pos,
                                       const csa2_fp4_kv* kv, hipStream_t stream) {
    clear_error();
    CSA2_ARG(kv != nullptr, "fp4_append: null cache view");
    CSA2_ARG(B >= 0, "fp4_append: B=%d < 0", B);
    CSA2_ARG(kv->D > 0 && kv->D % 16 == 0, "fp4_append: D=%d must be a positive multiple of 16", kv->D);
    CSA2_ARG(xt == CSA2_F32 || xt == CSA2_BF16, "fp4_append: bad dtype %d", (int)xt);
    if (B == 0) return CSA2_OK;
    CSA2_ARG(x && pos && kv->codes && kv->scales, "fp4_append: null pointer");
    CSA2_ARG(aligned(x, 16) && aligned(kv->codes, 8), "fp4_append: x must be 16-byte and codes 8-byte aligned");
    RowMap map;
    csa2_status st = make_rowmap(kv->page_table, kv->page_size, kv->max_pages, kv->seq_stride, 1, &map, "fp4_append");
    if (st != CSA2_OK) return st;
    if (xt == CSA2_BF16)
        fp4_append_kernel<true><<<B, 64, 0, stream>>>(x, kv->D, pos, map, kv->codes, kv->scales);
    else
        fp4_append_kernel<false><<<B, 64, 0, stream>>>(x, kv->D, pos, map, kv->codes, kv->scales);
    return launch_status("fp4_append");
}
