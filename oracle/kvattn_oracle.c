/*
 * kvattn oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU implementation of decode-step attention over a
 * paged KV cache.  Only the tests, the smoke check and the bench's CPU
 * baseline may load it; the library never does.  It shares no code with the
 * HIP path: it knows nothing of prefix trees, packs, splits, tiles or merges
 * of partial results on the GPU side.
 *
 * What it computes (PAT review, "core formula" section):
 *     out = softmax(q K^T / sqrt(d)) V
 * for a single-token query q against the KV cache accumulated so far.  The
 * cache holds the current token too: the decode step appends K_t, V_t to the
 * cache before attending over [K_1 .. K_t] (short-term-memory concept page,
 * "technical principle": the autoregressive KV-cache step).
 *
 * Paged layout (same concept page, PagedAttention section): a request's token
 * t lives in physical block block_tables[b][t / 16], slot t % 16.  Pools are
 * [n_blocks][Hkv][16][D] bf16.  GQA: query head h reads KV head h / (Hq/Hkv)
 * (the GQA/MQA note on the concept page names the scheme; the contiguous
 * grouping is the plain reading).
 *
 * Arithmetic: bf16 -> double is exact; dot products, exp, sums in double;
 * two-pass softmax (max first, then exp and sums), not the online update.
 *
 * Parity pins: every function here is pinned by tests/test_oracle_pins.py
 * (brute force at 50 digits, torch float64 SDPA, closed forms, invariants,
 * a hand-derived golden case).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_to_f64(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Attention for one (query b, query head h) over tokens [t0, t1) of b.
 * Returns the partial triple in natural-log units:
 *   m   = max_t s_t,  l = sum_t exp(s_t - m),  acc = sum_t exp(s_t - m) V_t
 * with s_t = scale * (q . K_t).  `s` is scratch of at least (t1 - t0) doubles. */
static void partial_row(int32_t Hq, int32_t Hkv, int32_t D, int32_t bs, int32_t max_blocks,
                        const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                        const int32_t* block_tables, int64_t b, int64_t h, int64_t t0, int64_t t1,
                        double scale, double* s, double* m_out, double* l_out, double* acc) {
    const int64_t G = Hq / Hkv;
    const int64_t g = h / G;
    const uint16_t* qrow = q + (b * Hq + h) * D;
    double m = -INFINITY;
    for (int64_t t = t0; t < t1; ++t) {
        int64_t blk = block_tables[b * max_blocks + t / bs];
        int64_t o = t % bs;
        const uint16_t* krow = k_cache + ((blk * Hkv + g) * bs + o) * D;
        double dot = 0.0;
        for (int64_t i = 0; i < D; ++i) dot += bf16_to_f64(qrow[i]) * bf16_to_f64(krow[i]);
        s[t - t0] = dot * scale;
        if (s[t - t0] > m) m = s[t - t0];
    }
    double l = 0.0;
    for (int64_t i = 0; i < D; ++i) acc[i] = 0.0;
    for (int64_t t = t0; t < t1; ++t) {
        int64_t blk = block_tables[b * max_blocks + t / bs];
        int64_t o = t % bs;
        const uint16_t* vrow = v_cache + ((blk * Hkv + g) * bs + o) * D;
        double e = exp(s[t - t0] - m);
        l += e;
        for (int64_t i = 0; i < D; ++i) acc[i] += e * bf16_to_f64(vrow[i]);
    }
    *m_out = m;
    *l_out = l;
}

/*
 * out[r][:] = attention of row rows[r] (= b * Hq + h) over all seq_lens[b]
 * tokens of query b, in double.  scale <= 0 selects 1/sqrt(D).
 * Returns 0, or -1 on an invalid argument (seq_len < 1, bad head split).
 */
int kvattn_oracle_decode_rows(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t bs, int32_t max_blocks,
                              const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                              const int32_t* block_tables, const int32_t* seq_lens, double scale,
                              int64_t n_rows, const int64_t* rows, double* out) {
    if (Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || bs <= 0) return -1;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t b = rows[r] / Hq;
        if (b < 0 || b >= B || seq_lens[b] < 1 || seq_lens[b] > (int64_t)max_blocks * bs) return -1;
    }
    int bad = 0;
#pragma omp parallel
    {
        double* s = NULL;
        int64_t cap = 0;
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_rows; ++r) {
            int64_t b = rows[r] / Hq, h = rows[r] % Hq;
            int64_t T = seq_lens[b];
            if (T > cap) {
                free(s);
                cap = T;
                s = (double*)malloc((size_t)cap * sizeof(double));
            }
            if (!s) {
                bad = 1;
                continue;
            }
            double m, l;
            double* o = out + r * D;
            partial_row(Hq, Hkv, D, bs, max_blocks, q, k_cache, v_cache, block_tables, b, h, 0, T, scale, s,
                        &m, &l, o);
            for (int64_t i = 0; i < D; ++i) o[i] /= l;
        }
        free(s);
    }
    return bad ? -1 : 0;
}

/* The partial triple (m, l, acc[D]) of one row over tokens [t0, t1); natural-log units. */
int kvattn_oracle_partial(int32_t Hq, int32_t Hkv, int32_t D, int32_t bs, int32_t max_blocks,
                          const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                          const int32_t* block_tables, int64_t b, int64_t h, int64_t t0, int64_t t1,
                          double scale, double* m, double* l, double* acc) {
    if (t1 <= t0 || Hkv <= 0 || Hq % Hkv != 0) return -1;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
    double* s = (double*)malloc((size_t)(t1 - t0) * sizeof(double));
    if (!s) return -1;
    partial_row(Hq, Hkv, D, bs, max_blocks, q, k_cache, v_cache, block_tables, b, h, t0, t1, scale, s, m, l,
                acc);
    free(s);
    return 0;
}

/*
 * Combine n partial triples of one row with the online-softmax rule (PAT
 * review, merge stage: per-query partial results of several workgroups are
 * merged by an online softmax):
 *   M = max_i m_i,  w_i = exp(m_i - M),  out = sum_i w_i acc_i / sum_i w_i l_i
 */
int kvattn_oracle_merge(int32_t n, int32_t D, const double* m, const double* l, const double* acc, double* out) {
    if (n < 1) return -1;
    double M = -INFINITY;
    for (int32_t i = 0; i < n; ++i)
        if (m[i] > M) M = m[i];
    double L = 0.0;
    for (int32_t k = 0; k < D; ++k) out[k] = 0.0;
    for (int32_t i = 0; i < n; ++i) {
        double w = exp(m[i] - M);
        L += w * l[i];
        for (int32_t k = 0; k < D; ++k) out[k] += w * acc[(int64_t)i * D + k];
    }
    for (int32_t k = 0; k < D; ++k) out[k] /= L;
    return 0;
}

/* OpenMP threads the oracle's parallel loops use. */
int kvattn_oracle_threads(void) { return omp_get_max_threads(); }

/* Set the OpenMP threads of later calls (n >= 1); the timing of the CPU baseline
 * uses it to run on one core as well as on all of them. */
void kvattn_oracle_set_threads(int32_t n) {
    if (n >= 1) omp_set_num_threads(n);
}
