/*
 * Driver for the sanitizer build of the CPU oracle (moe_oracle.c, test infrastructure).
 * Built with -fsanitize=address,undefined -fno-sanitize-recover=all; it calls every exported
 * oracle function on small inputs, including the edge cases (empty batch, invalid rows,
 * tails that are not a multiple of the unrolling, capacity overflow), and checks properties
 * that hold for any correct result.  Any out-of-bounds access or undefined behaviour aborts
 * the process; a failed property exits with status 2.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_gate_logits(const float* x, const float* w, const int32_t* row_valid, int64_t G, int64_t E,
                        int64_t H, float* logits);
double oracle_exp(double x);
double oracle_sigmoid(double l);
void oracle_select_softmax(const float* logits, const int32_t* row_valid, int64_t G, int E, int k,
                           int renormalize, int32_t* ids, float* weights);
void oracle_select_grouped(const float* logits, const float* bias, const int32_t* row_valid, int64_t G,
                           int E, int n_group, int topk_group, int group_topn, int k, int renormalize,
                           int32_t* ids, float* weights);
void oracle_dispatch(const int32_t* ids, int64_t G, int k, const int32_t* phys_of, const int32_t* n_rep,
                     int max_rep, int E, int p0, int El, int align, int64_t cap, int32_t* counts,
                     int64_t* seg_offsets, int32_t* sorted_pair, int32_t* pair_row, int64_t* num_rows,
                     int32_t* error_flag);
double oracle_e4m3_value(uint8_t c);
void oracle_e4m3_decode(const uint8_t* q, int64_t n, double* out);

static int failures = 0;
#define EXPECT(c)                                                         \
    do {                                                                  \
        if (!(c)) {                                                       \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
            ++failures;                                                   \
        }                                                                 \
    } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {  /* splitmix64, upper half */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return (uint32_t)((z ^ (z >> 31)) >> 32);
}
static float frnd(void) { return (float)((double)rnd() / 4294967296.0 * 2.0 - 1.0); }

static void check_exp(void) {
    const double xs[] = {0.0, 1.0, -1.0, 0.5, -20.0, 30.0, 700.0, -700.0, 1e-300};
    for (size_t i = 0; i < sizeof xs / sizeof xs[0]; ++i) {
        const double a = oracle_exp(xs[i]), b = exp(xs[i]);
        EXPECT(fabs(a - b) <= 4e-16 * b);
    }
    EXPECT(isnan(oracle_exp(NAN)));
    EXPECT(isinf(oracle_exp(800.0)));
    EXPECT(oracle_exp(-800.0) == 0.0);
    EXPECT(fabs(oracle_sigmoid(0.0) - 0.5) < 1e-17);
}

static void check_gate(int64_t G, int64_t E, int64_t H) {
    float* x = malloc(sizeof(float) * (size_t)(G * H + 1));
    float* w = malloc(sizeof(float) * (size_t)(E * H + 1));
    float* out = malloc(sizeof(float) * (size_t)(G * E + 1));
    int32_t* valid = malloc(sizeof(int32_t) * (size_t)(G + 1));
    for (int64_t i = 0; i < G * H; ++i) x[i] = frnd();
    for (int64_t i = 0; i < E * H; ++i) w[i] = frnd();
    for (int64_t g = 0; g < G; ++g) valid[g] = (g % 3) != 1;
    oracle_gate_logits(x, w, valid, G, E, H, out);
    for (int64_t g = 0; g < G; ++g)
        for (int64_t e = 0; e < E; ++e) {
            double d = 0.0, m = 0.0;
            for (int64_t h = 0; h < H; ++h) {
                d += (double)x[g * H + h] * w[e * H + h];
                m += fabs((double)x[g * H + h] * w[e * H + h]);
            }
            if (!valid[g]) EXPECT(out[g * E + e] == 0.0f);
            else EXPECT(fabs(out[g * E + e] - d) <= (double)H * 0x1p-24 * m + 1e-30);
        }
    oracle_gate_logits(x, w, NULL, 0, E, H, out);  /* empty batch */
    free(x); free(w); free(out); free(valid);
}

static void check_ids(const int32_t* ids, const int32_t* valid, int64_t G, int E, int k) {
    for (int64_t g = 0; g < G; ++g)
        for (int j = 0; j < k; ++j) {
            const int32_t id = ids[g * k + j];
            if (valid && !valid[g]) { EXPECT(id == -1); continue; }
            EXPECT(id >= 0 && id < E);
            for (int i = 0; i < j; ++i) EXPECT(ids[g * k + i] != id);
        }
}

static void check_select(void) {
    enum { G = 11, E = 24, NG = 4, K = 5 };
    float logits[G * E], bias[E], wts[G * K];
    int32_t ids[G * K], valid[G];
    for (int i = 0; i < G * E; ++i) logits[i] = 3.0f * frnd();
    for (int e = 0; e < E; ++e) bias[e] = 0.1f * frnd();
    for (int g = 0; g < G; ++g) valid[g] = g != 4;
    logits[2 * E + 7] = logits[2 * E + 9];  /* a tie */
    for (int renorm = 0; renorm <= 1; ++renorm) {
        oracle_select_softmax(logits, valid, G, E, K, renorm, ids, wts);
        check_ids(ids, valid, G, E, K);
        for (int g = 0; g < G; ++g) {
            double s = 0.0;
            for (int j = 0; j < K; ++j) {
                EXPECT(wts[g * K + j] >= 0.0f);
                if (j) EXPECT(wts[g * K + j] <= wts[g * K + j - 1]);
                s += wts[g * K + j];
            }
            if (!valid[g]) EXPECT(s == 0.0);
            else if (renorm) EXPECT(fabs(s - 1.0) < 1e-6);
            else EXPECT(s > 0.0 && s <= 1.0 + 1e-6);
        }
        oracle_select_grouped(logits, bias, valid, G, E, NG, 2, 2, K, renorm, ids, wts);
        check_ids(ids, valid, G, E, K);
        for (int g = 0; g < G; ++g) {
            if (!valid[g]) continue;
            int groups[NG] = {0};
            for (int j = 0; j < K; ++j) groups[ids[g * K + j] / (E / NG)] = 1;
            EXPECT(groups[0] + groups[1] + groups[2] + groups[3] <= 2);
        }
        oracle_select_grouped(logits, NULL, NULL, G, E, NG, NG, 1, K, renorm, ids, wts);
        check_ids(ids, NULL, G, E, K);
    }
    oracle_select_softmax(logits, NULL, 0, E, K, 1, ids, wts);  /* empty batch */
    oracle_select_grouped(logits, bias, NULL, 0, E, NG, 2, 2, K, 1, ids, wts);
}

static void check_dispatch(int64_t G, int k, int align, int64_t cap) {
    enum { E = 8, MAXREP = 2, P = 12, P0 = 3, EL = 5 };
    /* experts 0..3 have two replicas (slots e and 8+e), 4..7 one (slot e) */
    int32_t phys_of[E * MAXREP], n_rep[E];
    for (int e = 0; e < E; ++e) {
        n_rep[e] = e < 4 ? 2 : 1;
        phys_of[e * MAXREP] = e;
        phys_of[e * MAXREP + 1] = e < 4 ? 8 + e : -1;
    }
    const int64_t np = G * k;
    int32_t* ids = malloc(sizeof(int32_t) * (size_t)(np + 1));
    int32_t* pair_row = malloc(sizeof(int32_t) * (size_t)(np + 1));
    int32_t* sorted = malloc(sizeof(int32_t) * (size_t)(cap + 1));
    for (int64_t f = 0; f < np; ++f) ids[f] = (f % 7 == 3) ? -1 : (int32_t)(rnd() % E);
    int32_t counts[EL], err = -1;
    int64_t seg[EL + 1], rows = -1;
    for (int64_t r = 0; r < cap; ++r) sorted[r] = -7;
    oracle_dispatch(ids, G, k, phys_of, n_rep, MAXREP, E, P0, EL, align, cap, counts, seg, sorted, pair_row,
                    &rows, &err);
    (void)P;
    EXPECT(seg[0] == 0 && rows == seg[EL]);
    EXPECT(err == (rows > cap));
    int64_t local = 0, stored = 0;
    for (int e = 0; e < EL; ++e) {
        EXPECT(seg[e + 1] - seg[e] >= counts[e] && seg[e + 1] - seg[e] < counts[e] + align);
        EXPECT((seg[e + 1] - seg[e]) % align == 0);
        local += counts[e];
    }
    for (int64_t f = 0; f < np; ++f) {
        if (pair_row[f] < 0) continue;
        EXPECT(pair_row[f] < cap && sorted[pair_row[f]] == f);
        ++stored;
    }
    EXPECT(stored <= local);
    if (!err) EXPECT(stored == local);
    free(ids); free(pair_row); free(sorted);
}

static void check_e4m3(void) {
    uint8_t q[256];
    double v[256];
    for (int i = 0; i < 256; ++i) q[i] = (uint8_t)i;
    oracle_e4m3_decode(q, 256, v);
    for (int i = 0; i < 256; ++i) {
        if ((i & 0x7F) == 0x7F) { EXPECT(isnan(v[i])); continue; }
        EXPECT(fabs(v[i]) <= 448.0);
        EXPECT(v[i] == oracle_e4m3_value((uint8_t)i));
        EXPECT(v[i ^ 0x80] == -v[i]);
    }
    EXPECT(v[0x7E] == 448.0 && v[0x01] == 0x1p-9 && v[0x08] == 0x1p-6);
}

int main(void) {
    check_exp();
    check_gate(7, 13, 37);
    check_gate(3, 8, 1);
    check_gate(1, 1, 64);
    check_select();
    check_dispatch(0, 4, 4, 16);
    check_dispatch(9, 2, 1, 64);
    check_dispatch(40, 3, 4, 200);
    check_dispatch(40, 3, 16, 24);  /* overflows the capacity */
    check_e4m3();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 2;
    }
    printf("oracle sanitizer driver: ok\n");
    return 0;
}
