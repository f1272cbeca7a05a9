/*
 * CPU oracle for the single-rank MoE hot path -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously-correct C.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark load this library; the product path never does.
 * It shares no code, header, table or constant with the HIP library.
 *
 * Built with -O2 -ffp-contract=off (no fast-math, no flush-to-zero), so every
 * floating-point operation below happens exactly as written.
 *
 * The pages this follows are the SGLang walkthrough "SGLang 源码完全拆解(十七):
 * DP Attention 与专家并行" (called "the SGLang page" below) and the vLLM walkthrough
 * "vLLM 源码完全拆解(二十七): Dual Batch Overlap" ("the vLLM page").  Neither defines
 * the routing arithmetic; the readings taken here are listed with each function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ gate logits
 * Router logits logits[g,e] = sum_h x[g,h] * w[e,h] (op_gate of the SGLang page, section
 * "operations 与 yield").  The pages fix no precision or order; the reading taken is the
 * plain dot product in fp32 as one chain of fused multiply-adds in ascending h:
 *     acc = +0
 *     for h = 0 .. H-1:  acc = fmaf(x[g,h], w[e,h], acc)
 *     logits[g,e] = acc
 * so that the integer routing decision made from these logits can be reproduced bit for
 * bit.  Rows with row_valid[g] == 0 get logits 0.  The loops visit eight experts per h
 * step; each accumulator keeps its own ascending chain, so this is the definition above,
 * unchanged.
 */
void oracle_gate_logits(const float* x, const float* w, const int32_t* row_valid,
                        int64_t G, int64_t E, int64_t H, float* logits) {
    #pragma omp parallel for schedule(dynamic, 4)
    for (int64_t g = 0; g < G; ++g) {
        const float* xr = x + g * H;
        if (row_valid && !row_valid[g]) {
            for (int64_t e = 0; e < E; ++e) logits[g * E + e] = 0.0f;
            continue;
        }
        for (int64_t e0 = 0; e0 < E; e0 += 8) {
            int64_t ne = (E - e0) < 8 ? (E - e0) : 8;
            float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            for (int64_t h = 0; h < H; ++h)
                for (int64_t j = 0; j < ne; ++j)
                    acc[j] = fmaf(xr[h], w[(e0 + j) * H + h], acc[j]);
            for (int64_t j = 0; j < ne; ++j) logits[g * E + e0 + j] = acc[j];
        }
    }
}

/* ------------------------------------------------------------------ defined exp
 * The grouped-sigmoid selection compares sigma(l) + bias in fp64; to make that
 * integer decision reproducible on any machine, exp is not taken from a libm but
 * defined here by the classical Cody-Waite method:
 *   n  = round-to-nearest-even(x * (1/ln 2))
 *   r  = (x - n*LN2_HI) - n*LN2_LO            (two fused steps)
 *   p  = sum_{i=0..13} r^i / i!              (Horner, fused steps, 1/i! as 1.0/i!)
 *   exp(x) = p * 2^n
 * |r| <= ln2/2 bounds the truncated Taylor tail by ~4e-18, below half an ulp of 1.
 * LN2_HI carries 32 significant bits so n*LN2_HI is exact for |n| < 2^21.
 */
static const double O_INV_LN2 = 0x1.71547652b82fep+0;
static const double O_LN2_HI = 0x1.62e42fee00000p-1;
static const double O_LN2_LO = 0x1.a39ef35793c76p-33;

double oracle_exp(double x) {
    if (x != x) return x;
    if (x > 709.8) return INFINITY;
    if (x < -745.2) return 0.0;
    double n = nearbyint(x * O_INV_LN2);
    double r = fma(-n, O_LN2_HI, x);
    r = fma(-n, O_LN2_LO, r);
    double fact = 1.0;
    double coef[14];
    for (int i = 0; i < 14; ++i) {
        if (i > 0) fact *= (double)i;
        coef[i] = 1.0 / fact;
    }
    double p = coef[13];
    for (int i = 12; i >= 0; --i) p = fma(p, r, coef[i]);
    return ldexp(p, (int)n);
}

/* sigma(l) = 1 / (1 + exp(-l)) in fp64 */
double oracle_sigmoid(double l) { return 1.0 / (1.0 + oracle_exp(-l)); }

/* ------------------------------------------------------------------ top-k helper
 * Pick the k largest of key[0..n-1] among entries with allow[i] != 0.
 * Ties go to the lower index; the picks come out in descending key order.
 */
static void topk_desc(const double* key, const unsigned char* allow, int n, int k, int* out) {
    unsigned char* taken = (unsigned char*)calloc((size_t)n, 1);
    for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int i = 0; i < n; ++i) {
            if ((allow && !allow[i]) || taken[i]) continue;
            if (best < 0 || key[i] > key[best]) best = i;
        }
        out[j] = best;
        if (best >= 0) taken[best] = 1;
    }
    free(taken);
}

/* ------------------------------------------------------------------ softmax top-k
 * TopKOutput (topk_ids, topk_weights) of the SGLang page, section "normal dispatch
 * 的调用链".  Reading: the k experts with the largest logits (softmax is monotone,
 * so no exp enters the choice), ties to the lower id, slots in descending order;
 * weight = softmax(logits)[id] over all E experts in fp64, optionally divided by
 * the sum over the k picks.  Rows with row_valid == 0 get id -1 and weight 0
 * (pad rows carry no expert load: vLLM page, section "Pad 到最大，而非各扫门前雪";
 * -1 marks an empty slot: vLLM page, section "第 2 段：接收结果与挂 recv hook").
 */
void oracle_select_softmax(const float* logits, const int32_t* row_valid, int64_t G, int E,
                           int k, int renormalize, int32_t* ids, float* weights) {
    #pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < G; ++g) {
        if (row_valid && !row_valid[g]) {
            for (int j = 0; j < k; ++j) { ids[g * k + j] = -1; weights[g * k + j] = 0.0f; }
            continue;
        }
        double* key = (double*)malloc(sizeof(double) * (size_t)E);
        int* pick = (int*)malloc(sizeof(int) * (size_t)k);
        double mx = -INFINITY;
        for (int e = 0; e < E; ++e) {
            key[e] = (double)logits[g * E + e];
            if (key[e] > mx) mx = key[e];
        }
        double den = 0.0;
        for (int e = 0; e < E; ++e) den += exp(key[e] - mx);
        topk_desc(key, NULL, E, k, pick);
        double sel = 0.0;
        for (int j = 0; j < k; ++j) sel += exp(key[pick[j]] - mx) / den;
        for (int j = 0; j < k; ++j) {
            double p = exp(key[pick[j]] - mx) / den;
            ids[g * k + j] = pick[j];
            weights[g * k + j] = (float)(renormalize ? p / sel : p);
        }
        free(key);
        free(pick);
    }
}

/* ------------------------------------------------------------------ grouped sigmoid top-k
 * DeepSeek-V3-style routing with the load-balancing correction bias that the
 * SGLang page names in section "推理时怎么“选副本”" (the "fake" dispatch zeroes it).
 * The group rule itself is not on the pages; the reading is the DeepSeek-V3 report's:
 *   s_e   = sigma(l_e)                     (fp64, defined exp above)
 *   key_e = s_e + bias_e                   (fp64)
 *   experts are split into n_group contiguous groups of E/n_group;
 *   group score = sum of its group_topn largest keys, added largest first;
 *   keep the topk_group best groups (ties to the lower group);
 *   pick the k largest keys inside the kept groups (ties to the lower id),
 *   slots in descending key order;
 *   weight_j = s_{id_j} (bias excluded), divided by sum_j s_{id_j} when renormalize.
 * Rows with row_valid == 0 get id -1 and weight 0.
 */
void oracle_select_grouped(const float* logits, const float* bias, const int32_t* row_valid,
                           int64_t G, int E, int n_group, int topk_group, int group_topn,
                           int k, int renormalize, int32_t* ids, float* weights) {
    const int per = E / n_group;
    #pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < G; ++g) {
        if (row_valid && !row_valid[g]) {
            for (int j = 0; j < k; ++j) { ids[g * k + j] = -1; weights[g * k + j] = 0.0f; }
            continue;
        }
        double* s = (double*)malloc(sizeof(double) * (size_t)E);
        double* key = (double*)malloc(sizeof(double) * (size_t)E);
        double* gscore = (double*)malloc(sizeof(double) * (size_t)n_group);
        int* tmp = (int*)malloc(sizeof(int) * (size_t)(per > k ? per : k) + sizeof(int) * (size_t)n_group);
        int* gpick = tmp + (per > k ? per : k);
        unsigned char* allow = (unsigned char*)calloc((size_t)E, 1);
        for (int e = 0; e < E; ++e) {
            s[e] = oracle_sigmoid((double)logits[g * E + e]);
            key[e] = s[e] + (bias ? (double)bias[e] : 0.0);
        }
        for (int q = 0; q < n_group; ++q) {
            topk_desc(key + q * per, NULL, per, group_topn, tmp);
            double acc = 0.0;
            for (int j = 0; j < group_topn; ++j) acc += key[q * per + tmp[j]];
            gscore[q] = acc;
        }
        topk_desc(gscore, NULL, n_group, topk_group, gpick);
        for (int j = 0; j < topk_group; ++j)
            for (int e = gpick[j] * per; e < (gpick[j] + 1) * per; ++e) allow[e] = 1;
        topk_desc(key, allow, E, k, tmp);
        double sum = 0.0;
        for (int j = 0; j < k; ++j) sum += s[tmp[j]];
        for (int j = 0; j < k; ++j) {
            ids[g * k + j] = tmp[j];
            weights[g * k + j] = (float)(renormalize ? s[tmp[j]] / sum : s[tmp[j]]);
        }
        free(s); free(key); free(gscore); free(tmp); free(allow);
    }
}

/* ------------------------------------------------------------------ dispatch plan
 * The per-expert counts of get_dispatch_layout, the expert_alignment rounding and
 * the "handle" that tells combine where every pair went (SGLang page, section
 * "normal dispatch 的调用链"), computed for one rank's slots [p0, p0+E_l).
 *   physical slot of pair f = g*k + j with logical id l:
 *       p = phys_of[l][g mod n_rep[l]]   (the same choice on every rank: the
 *       rank-invariant pick of section "推理时怎么“选副本”")
 *   local iff p0 <= p < p0 + E_l; e = p - p0
 *   counts[e]            = number of local pairs on slot e
 *   seg_offsets[0] = 0,  seg_offsets[e+1] = seg_offsets[e] + roundup(counts[e], align)
 *   inside a segment pairs keep ascending f (a stable counting sort)
 *   sorted_pair[row] = f, alignment pad rows = -1; pair_row[f] = row or -1
 *   num_rows = seg_offsets[E_l]
 * Rows at or beyond cap are not stored: their pairs get pair_row = -1 and
 * error_flag = 1 (the fixed-capacity overflow of the low-latency buffers).
 */
void oracle_dispatch(const int32_t* ids, int64_t G, int k, const int32_t* phys_of,
                     const int32_t* n_rep, int max_rep, int E, int p0, int El, int align,
                     int64_t cap, int32_t* counts, int64_t* seg_offsets, int32_t* sorted_pair,
                     int32_t* pair_row, int64_t* num_rows, int32_t* error_flag) {
    const int64_t P = G * (int64_t)k;
    int32_t* slot = (int32_t*)malloc(sizeof(int32_t) * (size_t)(P > 0 ? P : 1));
    for (int e = 0; e < El; ++e) counts[e] = 0;
    for (int64_t f = 0; f < P; ++f) {
        slot[f] = -1;
        int32_t l = ids[f];
        if (l < 0 || l >= E) continue;
        int64_t g = f / k;
        int32_t p = phys_of[(int64_t)l * max_rep + (g % n_rep[l])];
        if (p >= p0 && p < p0 + El) {
            slot[f] = p - p0;
            counts[p - p0] += 1;
        }
    }
    seg_offsets[0] = 0;
    for (int e = 0; e < El; ++e) {
        int64_t padded = ((int64_t)counts[e] + align - 1) / align * align;
        seg_offsets[e + 1] = seg_offsets[e] + padded;
    }
    *num_rows = seg_offsets[El];
    *error_flag = seg_offsets[El] > cap ? 1 : 0;
    int64_t* fill = (int64_t*)malloc(sizeof(int64_t) * (size_t)(El > 0 ? El : 1));
    for (int e = 0; e < El; ++e) fill[e] = seg_offsets[e];
    for (int64_t f = 0; f < P; ++f) {
        pair_row[f] = -1;
        if (slot[f] < 0) continue;
        int64_t row = fill[slot[f]]++;
        if (row < cap) {
            sorted_pair[row] = (int32_t)f;
            pair_row[f] = (int32_t)row;
        }
    }
    for (int e = 0; e < El; ++e)
        for (int64_t row = seg_offsets[e] + counts[e]; row < seg_offsets[e + 1]; ++row)
            if (row < cap) sorted_pair[row] = -1;
    free(fill);
    free(slot);
}

/* ------------------------------------------------------------------ OCP e4m3fn decode
 * sign | 4-bit exponent (bias 7) | 3-bit mantissa; exponent field 0 is subnormal
 * (m/8 * 2^-6); 0x7F / 0xFF are NaN; there are no infinities.
 */
double oracle_e4m3_value(uint8_t c) {
    int sgn = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp(8.0 + m, e - 10);
    return sgn ? -v : v;
}

void oracle_e4m3_decode(const uint8_t* q, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_value(q[i]);
}
