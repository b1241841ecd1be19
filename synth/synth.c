/* Host implementation of the seeded synthetic-input generator.  The
 * definition is stated in synth.h; synth_dev.hip implements the same
 * definition on the device for inputs that are too large to build on the
 * host.  Built with -ffp-contract=off: the only float operation is one
 * multiply per element. */
#include "synth.h"

#include <pthread.h>
#include <stddef.h>
#include <stdlib.h>

#define GOLDEN 0x9E3779B97F4A7C15ull

uint64_t synth_mix64(uint64_t z) {
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ull;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBull;
    z ^= z >> 31;
    return z;
}

uint64_t synth_word(uint64_t key, uint64_t n) { return synth_mix64(key + (n + 1) * GOLDEN); }

uint64_t synth_key(uint64_t seed, uint64_t tensor) { return synth_word(seed, tensor); }

static float normal_at(uint64_t key, uint64_t e, float scale) {
    int64_t s = 0;
    for (int j = 0; j < 4; ++j) {
        uint64_t w = synth_word(key, 4 * e + (uint64_t)j);
        s += (int64_t)(w & 0xFFFFF);
        s += (int64_t)((w >> 20) & 0xFFFFF);
        s += (int64_t)((w >> 40) & 0xFFFFF);
    }
    int32_t z = (int32_t)(s - 6 * (int64_t)0xFFFFF);
    return (float)z * scale;
}

static float sigma_scale(float sigma) {
    /* sigma * 2^-20, exact (power-of-two scaling of a normal float). */
    return sigma * (1.0f / 1048576.0f);
}

typedef struct {
    uint64_t key;
    int64_t first, begin, end;
    float scale;
    float* out;
} normal_job;

static void* normal_worker(void* p) {
    normal_job* j = (normal_job*)p;
    for (int64_t i = j->begin; i < j->end; ++i)
        j->out[i] = normal_at(j->key, (uint64_t)(j->first + i), j->scale);
    return NULL;
}

void synth_normal_f32(uint64_t seed, uint64_t tensor, int64_t first, int64_t count, float sigma,
                      float* out, int threads) {
    if (count <= 0) return;
    uint64_t key = synth_key(seed, tensor);
    float scale = sigma_scale(sigma);
    if (threads < 1) threads = 1;
    if (threads > 64) threads = 64;
    if (count < 65536) threads = 1;
    normal_job jobs[64];
    pthread_t tid[64];
    int64_t per = (count + threads - 1) / threads;
    int started = 0;
    for (int t = 0; t < threads; ++t) {
        int64_t b = (int64_t)t * per, e = b + per;
        if (e > count) e = count;
        if (b >= e) break;
        jobs[t] = (normal_job){key, first, b, e, scale, out};
        if (threads == 1) {
            normal_worker(&jobs[t]);
        } else if (pthread_create(&tid[started], NULL, normal_worker, &jobs[t]) == 0) {
            ++started;
        } else {
            normal_worker(&jobs[t]);
        }
    }
    for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
}

typedef struct {
    uint64_t key;
    int64_t k;
    const int64_t* rows;
    int64_t begin, end;
    float scale;
    float* out;
} rows_job;

static void* rows_worker(void* p) {
    rows_job* j = (rows_job*)p;
    for (int64_t i = j->begin; i < j->end; ++i) {
        uint64_t base = (uint64_t)j->rows[i] * (uint64_t)j->k;
        for (int64_t c = 0; c < j->k; ++c)
            j->out[i * j->k + c] = normal_at(j->key, base + (uint64_t)c, j->scale);
    }
    return NULL;
}

void synth_normal_rows_f32(uint64_t seed, uint64_t tensor, int64_t k, const int64_t* rows,
                           int64_t n_rows, float sigma, float* out, int threads) {
    if (n_rows <= 0 || k <= 0) return;
    uint64_t key = synth_key(seed, tensor);
    float scale = sigma_scale(sigma);
    if (threads < 1) threads = 1;
    if (threads > 64) threads = 64;
    if (threads > n_rows) threads = (int)n_rows;
    rows_job jobs[64];
    pthread_t tid[64];
    int64_t per = (n_rows + threads - 1) / threads;
    int started = 0;
    for (int t = 0; t < threads; ++t) {
        int64_t b = (int64_t)t * per, e = b + per;
        if (e > n_rows) e = n_rows;
        if (b >= e) break;
        jobs[t] = (rows_job){key, k, rows, b, e, scale, out};
        if (threads == 1) {
            rows_worker(&jobs[t]);
        } else if (pthread_create(&tid[started], NULL, rows_worker, &jobs[t]) == 0) {
            ++started;
        } else {
            rows_worker(&jobs[t]);
        }
    }
    for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
}

void synth_int8(uint64_t seed, uint64_t tensor, int64_t first, int64_t count, int8_t* out) {
    uint64_t key = synth_key(seed, tensor);
    for (int64_t i = 0; i < count; ++i)
        out[i] = (int8_t)((int)(synth_word(key, (uint64_t)(first + i)) % 255u) - 127);
}

void synth_f16_scale(uint64_t seed, uint64_t tensor, int64_t first, int64_t count, uint16_t* out) {
    uint64_t key = synth_key(seed, tensor);
    for (int64_t i = 0; i < count; ++i) {
        uint64_t w = synth_word(key, (uint64_t)(first + i));
        uint16_t e = (uint16_t)(3u + (uint16_t)((w >> 32) % 4u));
        out[i] = (uint16_t)((e << 10) | (uint16_t)(w & 0x3FFu));
    }
}

void synth_choose(uint64_t seed, uint64_t tensor, int64_t n, int64_t m, int64_t* out) {
    /* Partial Fisher-Yates over an implicit identity permutation; the
     * swapped entries are kept in a small open list so that no O(n) array
     * is needed beyond the output. */
    if (m > n) m = n;
    uint64_t key = synth_key(seed, tensor);
    /* perm values are materialized lazily: value(i) = i unless displaced. */
    int64_t cap = 2 * m + 2;
    int64_t* slot_idx = (int64_t*)malloc(sizeof(int64_t) * (size_t)cap);
    int64_t* slot_val = (int64_t*)malloc(sizeof(int64_t) * (size_t)cap);
    if (!slot_idx || !slot_val) {
        free(slot_idx);
        free(slot_val);
        return;
    }
    int64_t used = 0;
#define GETV(pos, dst)                                                   \
    do {                                                                 \
        int64_t _v = (pos);                                              \
        for (int64_t _s = 0; _s < used; ++_s)                            \
            if (slot_idx[_s] == (pos)) { _v = slot_val[_s]; break; }     \
        (dst) = _v;                                                      \
    } while (0)
#define SETV(pos, val)                                                   \
    do {                                                                 \
        int64_t _s = 0;                                                  \
        for (; _s < used; ++_s)                                          \
            if (slot_idx[_s] == (pos)) break;                            \
        if (_s == used) { slot_idx[used] = (pos); ++used; }              \
        slot_val[_s] = (val);                                            \
    } while (0)
    for (int64_t i = 0; i < m; ++i) {
        uint64_t r = synth_word(key, (uint64_t)i) % (uint64_t)(n - i);
        int64_t j = i + (int64_t)r;
        int64_t vi, vj;
        GETV(i, vi);
        GETV(j, vj);
        SETV(i, vj);
        SETV(j, vi);
        out[i] = vj;
    }
#undef GETV
#undef SETV
    free(slot_idx);
    free(slot_val);
}
