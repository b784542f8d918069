/* Memory- and UB-check driver for the oracle (test infrastructure only).
 *
 * Built together with csa2_oracle.c under gcc's AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_oracle_sanitized.py, it calls every
 * exported oracle function on small inputs that reach their edge cases: empty
 * and short rows, rows with fewer finite scores than k, every score equal,
 * pools with missing blocks and a partly visible last block, attention with no
 * selected key, a window starting at token 0, and the window replay wrapping
 * its ring.  It checks a few results that follow from the definitions (counts,
 * -1 padding, orderings) and exits non-zero on the first mismatch; the
 * sanitizers abort on any out-of-bounds access, leak or undefined operation.
 * The inputs are fixed bit patterns from a small xorshift generator: this file
 * holds none of the method's arithmetic. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_e4m3fn_decode(uint8_t code);
uint8_t oracle_e4m3fn_round(double q);
double oracle_e2m1_magnitude(int mag);
void oracle_fp4_encode(const float* x, int64_t rows, int32_t D, uint8_t* codes, uint8_t* scales);
void oracle_fp4_decode(const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t D, double* y);
void oracle_index_scores(const uint16_t* q_idx, int32_t H_i, int32_t D_i, const uint16_t* K, int64_t n,
                         int64_t n_vis, float* scores);
void oracle_reindex_scores(const uint16_t* q_idx, int32_t H_i, int32_t D_i, const uint16_t* K, int64_t n_vis,
                           const int32_t* pool, int32_t P, float* pool_scores);
void oracle_block_max(const float* scores, int64_t n, float* block_max);
void oracle_topk(const float* scores, int64_t n, int32_t k, const int32_t* map, int32_t* out);
void oracle_attention(const double* q, int32_t H, int32_t D, const uint8_t* codes, const uint8_t* scales,
                      const int32_t* idx, int32_t K, const double* swa, int32_t T, int32_t q_pos, int32_t window,
                      double sm_scale, double* o, double* lse);
uint16_t oracle_bf16_round(double v);
void oracle_swa_replay(const uint16_t* h, const uint16_t* W, int32_t n, int32_t dm, int32_t D, int64_t t_end,
                       int32_t T, uint16_t* ring);

static uint32_t rng = 2463534242u;
static uint32_t next_u32(void) {
    rng ^= rng << 13;
    rng ^= rng >> 17;
    rng ^= rng << 5;
    return rng;
}
/* a finite bf16 bit pattern of magnitude about 2^-4 .. 2^3 */
static uint16_t some_bf16(void) {
    const uint32_t r = next_u32();
    return (uint16_t)(((r & 1u) << 15) | ((123u + (r >> 1) % 8u) << 7) | ((r >> 8) & 0x7Fu));
}

static int fails = 0;
#define CHECK(c, ...)                      \
    do {                                   \
        if (!(c)) {                        \
            fprintf(stderr, __VA_ARGS__);  \
            fprintf(stderr, "\n");         \
            ++fails;                       \
        }                                  \
    } while (0)

static void check_formats(void) {
    for (int c = 0; c < 256; ++c) {
        const double v = oracle_e4m3fn_decode((uint8_t)c);
        if (!isnan(v)) CHECK(oracle_e4m3fn_round(fabs(v)) == (c & 0x7F), "e4m3 round trip of 0x%02x", c);
    }
    for (int m = 0; m < 8; ++m) CHECK(oracle_e2m1_magnitude(m) >= 0.0, "e2m1 magnitude %d", m);
    const int32_t D = 64;
    const int64_t rows = 5;
    float x[5 * 64];
    for (int i = 0; i < rows * D; ++i) x[i] = (float)((int)(next_u32() % 2001) - 1000) / 37.0f;
    for (int i = 0; i < D; ++i) x[i] = 0.0f;                  /* an all-zero row */
    for (int i = 0; i < D; ++i) x[D + i] = ldexpf(1.0f, -140); /* subnormal inputs */
    x[2 * D] = 1e30f;                                         /* saturation */
    uint8_t codes[5 * 32], scales[5 * 4];
    double y[5 * 64];
    oracle_fp4_encode(x, rows, D, codes, scales);
    oracle_fp4_decode(codes, scales, rows, D, y);
    for (int i = 0; i < D; ++i) CHECK(y[i] == 0.0, "zero row decodes to %g", y[i]);
    for (int i = 0; i < rows * D; ++i) CHECK(isfinite(y[i]), "decode %d not finite", i);
    oracle_fp4_encode(x, 0, D, codes, scales); /* no rows */
}

static void check_scores_and_topk(void) {
    const int32_t H_i = 3, D_i = 16;
    const int64_t n = 70;
    uint16_t q[3 * 16], K[70 * 16];
    for (int i = 0; i < H_i * D_i; ++i) q[i] = some_bf16();
    for (int i = 0; i < n * D_i; ++i) K[i] = some_bf16();
    float s[70];
    oracle_index_scores(q, H_i, D_i, K, n, 61, s);
    for (int64_t j = 61; j < n; ++j) CHECK(s[j] == -INFINITY, "invisible entry %lld scored", (long long)j);
    oracle_index_scores(q, H_i, D_i, K, 0, 0, s); /* empty row */

    float bm[9];
    oracle_index_scores(q, H_i, D_i, K, n, 61, s);
    oracle_block_max(s, n, bm);
    CHECK(bm[8] == -INFINITY, "block past the visible entries");

    int32_t out[80];
    /* k larger than the finite scores: the tail is -1 */
    oracle_topk(s, n, 64, NULL, out);
    for (int i = 0; i < 64; ++i) CHECK((i < 61) == (out[i] >= 0), "topk slot %d = %d", i, out[i]);
    /* every score equal: the lowest positions, ascending */
    float flat[70];
    for (int i = 0; i < n; ++i) flat[i] = 0.5f;
    oracle_topk(flat, n, 10, NULL, out);
    for (int i = 0; i < 10; ++i) CHECK(out[i] == i, "equal scores: slot %d = %d", i, out[i]);
    oracle_topk(flat, 0, 5, NULL, out); /* empty row */
    for (int i = 0; i < 5; ++i) CHECK(out[i] == -1, "empty row slot %d", i);

    /* pool: blocks 3, -1, 7 (entries 56..60 visible of block 7) */
    const int32_t P = 3;
    int32_t pool[3] = {3, -1, 7};
    float ps[24];
    oracle_reindex_scores(q, H_i, D_i, K, 61, pool, P, ps);
    for (int p = 8; p < 16; ++p) CHECK(ps[p] == -INFINITY, "missing block scored at %d", p);
    for (int p = 21; p < 24; ++p) CHECK(ps[p] == -INFINITY, "invisible pool entry scored at %d", p);
    /* positions map through the pool's blocks: entries of blocks 3 and 7 only */
    oracle_topk(ps, 24, 12, pool, out);
    for (int i = 0; i < 12; ++i)
        if (out[i] >= 0) CHECK((out[i] >= 24 && out[i] < 32) || (out[i] >= 56 && out[i] < 61), "pool pick %d", out[i]);
    for (int i = 1; i < 12; ++i)
        if (out[i] >= 0) CHECK(out[i] > out[i - 1], "pool picks not ascending at %d", i);
}

static void check_attention(void) {
    const int32_t H = 2, D = 32, T = 8;
    const int64_t n = 20;
    float x[20 * 32];
    for (int i = 0; i < n * D; ++i) x[i] = (float)((int)(next_u32() % 301) - 150) / 41.0f;
    uint8_t codes[20 * 16], scales[20 * 2];
    oracle_fp4_encode(x, n, D, codes, scales);
    double q[2 * 32], swa[8 * 32], o[2 * 32], lse[2];
    for (int i = 0; i < H * D; ++i) q[i] = (double)((int)(next_u32() % 201) - 100) / 50.0;
    for (int i = 0; i < T * D; ++i) swa[i] = (double)((int)(next_u32() % 201) - 100) / 50.0;
    int32_t idx[6] = {4, -1, 19, 0, -1, 7};
    oracle_attention(q, H, D, codes, scales, idx, 6, swa, T, 5, 4, 0.2, o, lse);
    for (int i = 0; i < H * D; ++i) CHECK(isfinite(o[i]), "attention output %d", i);
    /* no selected key, window starting at token 0 */
    int32_t none[3] = {-1, -1, -1};
    oracle_attention(q, H, D, codes, scales, none, 3, swa, T, 0, 4, 0.2, o, lse);
    for (int h = 0; h < H; ++h) CHECK(isfinite(lse[h]), "one window key: lse %d", h);
    /* nothing at all */
    oracle_attention(q, H, D, codes, scales, none, 3, NULL, T, -1, 0, 0.2, o, lse);
    for (int h = 0; h < H; ++h) CHECK(lse[h] == -INFINITY, "no keys: lse %d = %g", h, lse[h]);
}

static void check_replay(void) {
    const int32_t n = 5, dm = 24, D = 8, T = 4;
    uint16_t h[5 * 24], W[8 * 24], ring[4 * 8];
    for (int i = 0; i < n * dm; ++i) h[i] = some_bf16();
    for (int i = 0; i < D * dm; ++i) W[i] = some_bf16();
    memset(ring, 0xFF, sizeof ring);
    oracle_swa_replay(h, W, n, dm, D, 9, T, ring); /* tokens 5..9: the ring wraps */
    CHECK(oracle_bf16_round(1.0) == 0x3F80, "bf16 round of 1.0");
}

int main(void) {
    check_formats();
    check_scores_and_topk();
    check_attention();
    check_replay();
    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    printf("oracle sanitizer driver: all checks passed\n");
    return 0;
}
