/*
 * Seeded synthetic value generator shared by the tests, the bench and the
 * oracle's callers.  It holds none of the attention arithmetic: it only turns
 * (seed, tag, element index) into a bf16 number drawn from N(0, 1).
 *
 * Definition (counter based, so any sub-range can be regenerated alone):
 *   key      = splitmix64_mix(seed * 2^8 + tag)
 *   bits(c)  = splitmix64_mix(key + (c + 1) * 0x9E3779B97F4A7C15)
 *              -- the c-th output of SplitMix64 (Steele, Lea, Flood 2014)
 *              started from state `key`
 *   u(c)     = ((bits(c) >> 11) + 1) * 2^-53          in (0, 1]
 *   pair p   = elements 2p and 2p+1, Box-Muller (1958) on u(2p), u(2p+1):
 *              r = sqrt(-2 ln u(2p)),  th = 2 pi u(2p+1)
 *              z(2p) = r cos th,  z(2p+1) = r sin th
 *   value    = bf16 round-to-nearest-even of (float) z
 *
 * Built with gcc (OpenMP); loaded through ctypes by workloads/__init__.py.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t tag) {
    return mix64(seed * 256ULL + tag + 0x9E3779B97F4A7C15ULL);
}

static inline double uniform01(uint64_t key, uint64_t c) {
    uint64_t b = mix64(key + (c + 1ULL) * 0x9E3779B97F4A7C15ULL);
    return (double)((b >> 11) + 1ULL) * (1.0 / 9007199254740992.0);
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static inline double normal_at(uint64_t key, uint64_t i) {
    uint64_t p = i >> 1;
    double u1 = uniform01(key, 2 * p), u2 = uniform01(key, 2 * p + 1);
    double r = sqrt(-2.0 * log(u1));
    double th = 6.283185307179586476925286766559 * u2;
    return (i & 1) ? r * sin(th) : r * cos(th);
}

/* out[k] = bf16 N(0,1) value of element (start + k) of stream (seed, tag). */
void kvgen_normal_bf16(uint64_t seed, uint64_t tag, uint64_t start, uint64_t count, uint16_t* out) {
    const uint64_t key = stream_key(seed, tag);
    int64_t n = (int64_t)count;
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < n; ++k) out[k] = f32_to_bf16_rne((float)normal_at(key, start + (uint64_t)k));
}

/* Gathered variant: out[k] = value of element idx[k]. */
void kvgen_normal_bf16_gather(uint64_t seed, uint64_t tag, const uint64_t* idx, uint64_t count, uint16_t* out) {
    const uint64_t key = stream_key(seed, tag);
    int64_t n = (int64_t)count;
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < n; ++k) out[k] = f32_to_bf16_rne((float)normal_at(key, idx[k]));
}

/*
 * Fill a paged pool laid out [n_blocks][n_heads][block_size][head_dim]:
 * element e gets the stream value of index e, and token slots o >= valid[blk]
 * of a block get the bf16 quiet NaN 0x7FC0 (they hold no token).
 */
void kvgen_fill_pool(uint64_t seed, uint64_t tag, int64_t n_blocks, int64_t n_heads, int64_t block_size,
                     int64_t head_dim, const int32_t* valid, uint16_t* out) {
    const uint64_t key = stream_key(seed, tag);
    const int64_t per_block = n_heads * block_size * head_dim;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t b = 0; b < n_blocks; ++b) {
        uint16_t* dst = out + b * per_block;
        const int64_t v = valid ? valid[b] : block_size;
        for (int64_t h = 0; h < n_heads; ++h)
            for (int64_t o = 0; o < block_size; ++o) {
                int64_t base = ((b * n_heads + h) * block_size + o) * head_dim;
                uint16_t* row = dst + (h * block_size + o) * head_dim;
                if (o >= v) {
                    for (int64_t i = 0; i < head_dim; ++i) row[i] = 0x7FC0u;
                } else {
                    for (int64_t i = 0; i < head_dim; ++i)
                        row[i] = f32_to_bf16_rne((float)normal_at(key, (uint64_t)(base + i)));
                }
            }
    }
}
