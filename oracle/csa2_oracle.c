/*
 * CSA2 reference oracle: plain, slow, obviously-correct CPU implementation of
 * what the CSA2 decode/prefill hot path computes.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no code, header, table or constant
 * with the HIP library: every definition below is written out again from
 * the sources cited next to it.
 *
 * Sources (the pages):
 *  [P2] aigc.cn "DeepSeek 发布 V4.1-Flash：552B MoE 多模态模型，KV 缓存压缩至前代四分之一",
 *       paragraph on KV-cache compression (CSA2 modes, hierarchical indexer, FP4 cache).
 *  [P3] gkm0120.cn "DeepSeek-V4.1-Flash 技术调研报告", section 2.2.2 (Full / Reindex /
 *       Reuse table) and section 2.2.3 (Hierarchical Sparse Indexer).
 *  [P4] aprilzz.com "DeepSeek V4.1 Flash 发布：KV cache 降到 890 字节/token…", sections
 *       "把 prefill 砍掉一半" (128-token SWA), "CSA2：在层的维度上共享缓存" (modes,
 *       Top-512, pool of 2048 blocks x 8), "FP4 KV 与部署层的几个改动" (E2M1 + one
 *       E4M3 scale per 16 channels, no global scale).
 *  [OCP-MX]  OCP Microscaling Formats (MX) Specification v1.0, FP4 E2M1 element type.
 *  [OCP-FP8] OCP 8-bit Floating Point Specification (OFP8), E4M3 encoding.
 *
 * Where the pages leave a step open, the reading taken is stated next to the
 * code and listed in the design notes:
 *  - Indexer score: s_j = sum over indexer heads h of dot(q_h, k_j), with one
 *    indexer-K vector per entry shared by all heads.  fp32 evaluation order:
 *    qbar_c = sum_h q_hc (h ascending, from +0), then s_j = fp32 FMA chain over
 *    channels c ascending, from +0.
 *  - Top-K order: score descending, entry index ascending on ties; output
 *    ascending entry index, -1 padded; -inf marks an invisible entry.
 *  - Pool: aligned 8-entry blocks ranked by the max score in the block; the
 *    best 2048 blocks (same tie rule) form the pool.
 *  - FP4 scale = RNE_E4M3FN(amax / 6) saturating at 448; element = nearest E2M1
 *    value of |x| / scale with ties to the even code; sign copied.
 *  - Attention: one softmax over the union of the selected entries and the SWA
 *    window, K = V = the latent, scale given by the caller; fp64 throughout.
 *
 * Everything here is fp64 unless the step itself is defined in fp32 (the
 * indexer score, whose fp32 rounding decides the integer Top-K result).
 *
 * Parity unpinned (fixed by these readings, not by the pages): the score's
 * lack of ReLU, head weights or scale, and its fp32 evaluation order (equal to
 * the per-head sums in exact arithmetic; its rounding decides near-ties); the
 * block-max pool rule; the attention scale 1/sqrt(D) without RoPE, sink or
 * de-duplication; the replayed window projection beyond one matrix product.
 * The tests pin everything the mathematics and the format specifications fix.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Number formats                                                           */
/* ------------------------------------------------------------------------ */

/* bf16 bit pattern -> float (exact: bf16 is the top half of an fp32). */
static float bf16_to_float(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* [OCP-FP8] E4M3 (the "FN" variant: no infinities, S.1111.111 is NaN).
 * Sign bit 7, exponent bits 6..3 with bias 7, mantissa bits 2..0.
 * Exponent field 0 encodes subnormals m/8 * 2^-6. */
double oracle_e4m3fn_decode(uint8_t code) {
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/* Round a non-negative real to the nearest finite E4M3FN value, ties to the
 * even code (mantissa LSB 0).  Brute force over all 127 non-negative finite
 * codes, so values above the largest finite value (448) go to 448:
 * the scale saturates rather than overflowing. */
uint8_t oracle_e4m3fn_round(double q) {
    /* Saturation stated outright: far above 448 the fp64 differences below
     * absorb 448 and every candidate would look equally distant. */
    if (q >= 448.0) return 0x7E;
    int best = 0;
    double best_err = fabs(q - oracle_e4m3fn_decode(0));
    for (int code = 1; code <= 0x7E; ++code) {
        double err = fabs(q - oracle_e4m3fn_decode((uint8_t)code));
        if (err < best_err || (err == best_err && (code & 1) == 0 && (best & 1) == 1)) {
            best = code;
            best_err = err;
        }
    }
    return (uint8_t)best;
}

/* [OCP-MX] FP4 E2M1 magnitude (3 bits): exponent bits 2..1 with bias 1,
 * mantissa bit 0; exponent 0 is subnormal (m * 0.5). */
double oracle_e2m1_magnitude(int mag) {
    int e = (mag >> 1) & 3;
    int m = mag & 1;
    if (e == 0) return 0.5 * (double)m;
    return ldexp(1.0 + 0.5 * (double)m, e - 1);
}

/* Nearest E2M1 magnitude code to a non-negative real, ties to the even code. */
static int e2m1_round_magnitude(double q) {
    if (q >= 6.0) return 7; /* saturate at the largest magnitude, 6 */
    int best = 0;
    double best_err = fabs(q - oracle_e2m1_magnitude(0));
    for (int mag = 1; mag < 8; ++mag) {
        double err = fabs(q - oracle_e2m1_magnitude(mag));
        if (err < best_err || (err == best_err && (mag & 1) == 0 && (best & 1) == 1)) {
            best = mag;
            best_err = err;
        }
    }
    return best;
}

/* ------------------------------------------------------------------------ */
/* FP4 main-KV codec  [P4 "FP4 KV 与部署层的几个改动"; P2; P3 2.2.1]          */
/* ------------------------------------------------------------------------ */

/* Encode rows x[rows][D] (fp32) into
 *   codes[rows][D/2]: byte i holds channel 2i in the low nibble and 2i+1 in
 *                     the high nibble; nibble = sign<<3 | E2M1 magnitude;
 *   scales[rows][D/16]: one E4M3FN byte per 16 consecutive channels.
 * No global (per-tensor) scale.  D must be a multiple of 16. */
void oracle_fp4_encode(const float* x, int64_t rows, int32_t D, uint8_t* codes, uint8_t* scales) {
    for (int64_t r = 0; r < rows; ++r) {
        const float* xr = x + r * D;
        for (int g = 0; g < D / 16; ++g) {
            double amax = 0.0;
            for (int c = 0; c < 16; ++c) {
                double a = fabs((double)xr[16 * g + c]);
                if (a > amax) amax = a;
            }
            uint8_t sc = oracle_e4m3fn_round(amax / 6.0);
            double s = oracle_e4m3fn_decode(sc);
            scales[r * (D / 16) + g] = sc;
            for (int c = 0; c < 16; ++c) {
                float v = xr[16 * g + c];
                int mag = (s == 0.0) ? 0 : e2m1_round_magnitude(fabs((double)v) / s);
                int code = (signbit(v) ? 8 : 0) | mag;
                int ch = 16 * g + c;
                uint8_t* byte = &codes[r * (D / 2) + ch / 2];
                if (ch % 2 == 0)
                    *byte = (uint8_t)((*byte & 0xF0) | code);
                else
                    *byte = (uint8_t)((*byte & 0x0F) | (code << 4));
            }
        }
    }
}

/* Decode one channel of one entry: (-1)^sign * E2M1 * E4M3 scale. */
static double fp4_value(const uint8_t* codes_row, const uint8_t* scales_row, int ch) {
    uint8_t byte = codes_row[ch / 2];
    int code = (ch % 2 == 0) ? (byte & 15) : (byte >> 4);
    double v = oracle_e2m1_magnitude(code & 7) * oracle_e4m3fn_decode(scales_row[ch / 16]);
    return (code & 8) ? -v : v;
}

void oracle_fp4_decode(const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t D, double* y) {
    for (int64_t r = 0; r < rows; ++r)
        for (int ch = 0; ch < D; ++ch)
            y[r * D + ch] = fp4_value(codes + r * (D / 2), scales + r * (D / 16), ch);
}

/* ------------------------------------------------------------------------ */
/* Indexer scoring  [P3 2.2.2; P4 "CSA2：在层的维度上共享缓存"]                 */
/* ------------------------------------------------------------------------ */

/* qbar_c = sum over heads h (ascending, fp32, from +0) of q_idx[h][c]. */
static void head_sum(const uint16_t* q_idx, int32_t H_i, int32_t D_i, float* qbar) {
    for (int c = 0; c < D_i; ++c) {
        float acc = 0.0f;
        for (int h = 0; h < H_i; ++h) acc = acc + bf16_to_float(q_idx[h * D_i + c]);
        qbar[c] = acc;
    }
}

/* fp32 FMA chain over channels ascending, from +0. */
static float score_entry(const float* qbar, const uint16_t* k_row, int32_t D_i) {
    float acc = 0.0f;
    for (int c = 0; c < D_i; ++c) acc = fmaf(qbar[c], bf16_to_float(k_row[c]), acc);
    return acc;
}

/* Full-mode scoring of one query row over one sequence's indexer K
 * (logical order, K[n][D_i] bf16 bits).  Entries j >= n_vis are invisible
 * and get -inf. */
void oracle_index_scores(const uint16_t* q_idx, int32_t H_i, int32_t D_i, const uint16_t* K, int64_t n,
                         int64_t n_vis, float* scores) {
    float* qbar = (float*)malloc(sizeof(float) * D_i);
    head_sum(q_idx, H_i, D_i, qbar);
    for (int64_t j = 0; j < n; ++j)
        scores[j] = (j < n_vis) ? score_entry(qbar, K + j * D_i, D_i) : -INFINITY;
    free(qbar);
}

/* Reindex-mode scoring [P3 2.2.3; P4]: the same score, evaluated only at the
 * pool positions.  Position p maps to entry pool[p/8]*8 + p%8; a -1 block or
 * an entry >= n_vis is invalid (-inf). */
void oracle_reindex_scores(const uint16_t* q_idx, int32_t H_i, int32_t D_i, const uint16_t* K, int64_t n_vis,
                           const int32_t* pool, int32_t P, float* pool_scores) {
    float* qbar = (float*)malloc(sizeof(float) * D_i);
    head_sum(q_idx, H_i, D_i, qbar);
    for (int64_t p = 0; p < 8LL * P; ++p) {
        int32_t blk = pool[p / 8];
        int64_t j = (int64_t)blk * 8 + p % 8;
        pool_scores[p] = (blk >= 0 && j < n_vis) ? score_entry(qbar, K + j * D_i, D_i) : -INFINITY;
    }
    free(qbar);
}

/* Block max over aligned groups of 8 entries (-inf if none is visible). */
void oracle_block_max(const float* scores, int64_t n, float* block_max) {
    int64_t nb = (n + 7) / 8;
    for (int64_t b = 0; b < nb; ++b) {
        float m = -INFINITY;
        for (int64_t j = 8 * b; j < n && j < 8 * b + 8; ++j)
            if (scores[j] > m) m = scores[j];
        block_max[b] = m;
    }
}

/* ------------------------------------------------------------------------ */
/* Top-K selection  [P4 "CSA2：在层的维度上共享缓存": a new Top-512 per Full]   */
/* ------------------------------------------------------------------------ */

typedef struct {
    float s;
    int64_t j;
} scored;

static int by_score_desc_index_asc(const void* a, const void* b) {
    const scored* x = (const scored*)a;
    const scored* y = (const scored*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->j < y->j) ? -1 : (x->j > y->j);
}

static int int64_asc(const void* a, const void* b) {
    int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
    return (x < y) ? -1 : (x > y);
}

/* Full sort of the valid (non -inf) entries by (score desc, index asc); the
 * first min(k, valid) are selected and written in ascending index order,
 * the rest of out[k] is -1.  If map != NULL, position p stands for entry
 * map[p/8]*8 + p%8 (a pool); ties are still broken by position, which is
 * the same as by entry because pool blocks are ascending. */
void oracle_topk(const float* scores, int64_t n, int32_t k, const int32_t* map, int32_t* out) {
    scored* v = (scored*)malloc(sizeof(scored) * (size_t)(n > 0 ? n : 1));
    int64_t m = 0;
    for (int64_t j = 0; j < n; ++j)
        if (scores[j] != -INFINITY) {
            v[m].s = scores[j];
            v[m].j = j;
            ++m;
        }
    qsort(v, (size_t)m, sizeof(scored), by_score_desc_index_asc);
    int64_t take = m < k ? m : k;
    int64_t* sel = (int64_t*)malloc(sizeof(int64_t) * (size_t)(take > 0 ? take : 1));
    for (int64_t i = 0; i < take; ++i) sel[i] = v[i].j;
    qsort(sel, (size_t)take, sizeof(int64_t), int64_asc);
    for (int32_t i = 0; i < k; ++i) {
        if (i < take) {
            int64_t p = sel[i];
            out[i] = map ? (int32_t)((int64_t)map[p / 8] * 8 + p % 8) : (int32_t)p;
        } else {
            out[i] = -1;
        }
    }
    free(sel);
    free(v);
}

/* ------------------------------------------------------------------------ */
/* Attention over selected FP4 entries plus the sliding window               */
/* [P4 "把 prefill 砍掉一半": 128-token SWA in every layer;                     */
/*  P4 "CSA2…": each layer keeps its own main Q and SWA KV]                   */
/* ------------------------------------------------------------------------ */

/* One query row, H heads of width D (q[H][D], values as fp64).
 * Key set = { decoded FP4 entry idx[i] : i < K, idx[i] >= 0 }
 *         u { window token t : max(0, q_pos-window+1) <= t <= q_pos }
 *           (omitted when swa == NULL).  The window is the 128 most recent
 *           tokens including the query token itself [P4 "把 prefill 砍掉一半"];
 *           the layer's window rows are kept in a ring swa[T][D] in which
 *           token t occupies row t mod T -- the row a rebuilt (replayed)
 *           window is written to, below -- so window <= T is required (no
 *           two tokens of one window share a row).
 * K = V = the key vector.  For each head: z = sm_scale * q.key,
 * o = sum softmax(z) * key, lse = log sum exp(z) (natural log).
 * An empty key set gives o = 0, lse = -inf. */
void oracle_attention(const double* q, int32_t H, int32_t D, const uint8_t* codes, const uint8_t* scales,
                      const int32_t* idx, int32_t K, const double* swa, int32_t T, int32_t q_pos, int32_t window,
                      double sm_scale, double* o, double* lse) {
    int32_t lo = q_pos - window + 1;
    if (lo < 0) lo = 0;
    int32_t n_swa = (swa != NULL && window > 0 && q_pos >= 0) ? (q_pos - lo + 1) : 0;
    int32_t n_keys = 0;
    for (int32_t i = 0; i < K; ++i)
        if (idx != NULL && idx[i] >= 0) ++n_keys;
    n_keys += n_swa;

    double* keys = (double*)malloc(sizeof(double) * (size_t)(n_keys > 0 ? n_keys : 1) * D);
    int32_t r = 0;
    for (int32_t i = 0; i < K; ++i)
        if (idx != NULL && idx[i] >= 0) {
            const uint8_t* cr = codes + (int64_t)idx[i] * (D / 2);
            const uint8_t* sr = scales + (int64_t)idx[i] * (D / 16);
            for (int c = 0; c < D; ++c) keys[(int64_t)r * D + c] = fp4_value(cr, sr, c);
            ++r;
        }
    for (int32_t t = lo; t < lo + n_swa; ++t, ++r) {
        const int64_t row = t % T; /* the ring row of token t */
        for (int c = 0; c < D; ++c) keys[(int64_t)r * D + c] = swa[row * D + c];
    }

    double* z = (double*)malloc(sizeof(double) * (size_t)(n_keys > 0 ? n_keys : 1));
    for (int32_t h = 0; h < H; ++h) {
        const double* qh = q + (int64_t)h * D;
        double* oh = o + (int64_t)h * D;
        for (int c = 0; c < D; ++c) oh[c] = 0.0;
        if (n_keys == 0) {
            lse[h] = -INFINITY;
            continue;
        }
        double m = -INFINITY;
        for (int32_t i = 0; i < n_keys; ++i) {
            double dot = 0.0;
            for (int c = 0; c < D; ++c) dot += qh[c] * keys[(int64_t)i * D + c];
            z[i] = sm_scale * dot;
            if (z[i] > m) m = z[i];
        }
        double l = 0.0;
        for (int32_t i = 0; i < n_keys; ++i) {
            double p = exp(z[i] - m);
            l += p;
            for (int c = 0; c < D; ++c) oh[c] += p * keys[(int64_t)i * D + c];
        }
        for (int c = 0; c < D; ++c) oh[c] /= l;
        lse[h] = m + log(l);
    }
    free(z);
    free(keys);
}

/* ------------------------------------------------------------------------ */
/* SWA Bounded Replay                                                        */
/* ------------------------------------------------------------------------ */

/* fp64 -> bf16 bit pattern, round to nearest, ties to even, in one step (no
 * intermediate fp32 rounding).  bf16 = 1 sign, 8 exponent (bias 127), 7
 * fraction bits; below 2^-126 the spacing stays 2^-133 (subnormals);
 * magnitudes that round past the largest finite value become infinity. */
uint16_t oracle_bf16_round(double v) {
    const uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v)) return 0x7FC0u;
    double a = fabs(v);
    if (isinf(a)) return sign | 0x7F80u;
    if (a == 0.0) return sign;
    int e = ilogb(a);                 /* 2^e <= a < 2^(e+1) */
    if (e < -126) e = -126;           /* subnormal range: fixed spacing */
    const int q = e - 7;              /* spacing of bf16 values near a */
    const double r = rint(ldexp(a, -q)); /* default rounding mode: nearest, ties to even */
    const double y = ldexp(r, q);
    if (y >= ldexp(1.0, 128)) return sign | 0x7F80u;
    const float f = (float)y;         /* exact: y has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(sign | ((u >> 16) & 0x7FFFu));
}

/* Rebuild a layer's window rows by replaying its last n tokens.  Reading
 * (the pages state only that the missing window state is rebuilt from the
 * last n_win = 128 tokens [P4 "把 prefill 砍掉一半", "FP4 KV 与部署层的几个改动"]):
 * the window row of token p is the layer's window projection of its input at
 * p, kv_p[d] = sum_c h_p[c] * W[d][c] (W output-major [D][d_model]), rounded
 * once to bf16.  h[n][d_model] holds the inputs of positions
 * t_end-n+1 .. t_end in order; token p goes to ring row p mod T.  Rows of the
 * ring that no replayed token maps to are left as they are. */
void oracle_swa_replay(const uint16_t* h, const uint16_t* W, int32_t n, int32_t dm, int32_t D, int64_t t_end,
                       int32_t T, uint16_t* ring) {
    for (int32_t i = 0; i < n; ++i) {
        const int64_t p = t_end - n + 1 + i;
        const int64_t slot = p % T;
        for (int32_t d = 0; d < D; ++d) {
            double acc = 0.0; /* each product is exact in fp64 (8 + 8 significant bits) */
            for (int32_t c = 0; c < dm; ++c)
                acc += (double)bf16_to_float(h[(int64_t)i * dm + c]) * (double)bf16_to_float(W[(int64_t)d * dm + c]);
            ring[slot * D + d] = oracle_bf16_round(acc);
        }
    }
}
