/*
 * synthgen.c -- seeded, counter-based synthetic matrix generator.
 *
 * This module fills host buffers with the synthetic inputs that both the
 * GPU path and the CPU oracle consume.  It contains none of the matrix
 * product's arithmetic; it only draws numbers.
 *
 * Every element is a pure function of (seed, stream, logical index), where
 * the logical index of element (r, c) of a rows x cols matrix is r*cols + c.
 * The leading dimension of the destination buffer therefore never changes
 * the values, and any sub-range of rows can be regenerated on its own.
 *
 * Bit source: the SplitMix64 output function (Steele, Lea and Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014), applied to the
 * Weyl sequence key + (c + 1) * 0x9E3779B97F4A7C15, i.e. word c of a
 * SplitMix64 stream started at `key`.  The per-(seed, stream) key is itself
 * a SplitMix64 word, so distinct streams start far apart.
 *
 * Distributions (one 64-bit word per element unless noted):
 *   SYNTH_NORMAL      N(0,1): Box-Muller (1958), cosine branch, computed in
 *                     double from words 2i and 2i+1, then rounded to fp32.
 *   SYNTH_UNIFORM_PM1 U[-1,1): top 24 bits * 2^-23 - 1 (exact in fp32).
 *   SYNTH_SMALLINT    integers in [-4, 4]: (word mod 9) - 4.
 *   SYNTH_UNIFORM01   U[0,1): top 24 bits * 2^-24 (exact in fp32).
 *
 * Build: gcc -O2 -fPIC -shared -pthread synthgen.c -lm
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>

#define SYNTH_NORMAL 0
#define SYNTH_UNIFORM_PM1 1
#define SYNTH_SMALLINT 2
#define SYNTH_UNIFORM01 3

static const uint64_t WEYL = 0x9E3779B97F4A7C15ULL;

/* SplitMix64 output (finalising) function. */
static inline uint64_t sm64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* Word c of the SplitMix64 sequence whose state starts at `key`. */
static inline uint64_t sm64_word(uint64_t key, uint64_t c) {
    return sm64_mix(key + (c + 1) * WEYL);
}

uint64_t synth_key(uint64_t seed, uint64_t stream) {
    return sm64_word(sm64_word(0, seed), stream);
}

uint64_t synth_word(uint64_t seed, uint64_t stream, uint64_t c) {
    return sm64_word(synth_key(seed, stream), c);
}

static inline float draw(uint64_t key, uint64_t idx, int dist) {
    switch (dist) {
    case SYNTH_NORMAL: {
        uint64_t w0 = sm64_word(key, 2 * idx);
        uint64_t w1 = sm64_word(key, 2 * idx + 1);
        double u1 = (double)((w0 >> 11) + 1) * 0x1.0p-53; /* (0, 1] */
        double u2 = (double)(w1 >> 11) * 0x1.0p-53;       /* [0, 1) */
        double r = sqrt(-2.0 * log(u1));
        return (float)(r * cos(6.283185307179586476925286766559 * u2));
    }
    case SYNTH_UNIFORM_PM1:
        return (float)((double)(sm64_word(key, idx) >> 40) * 0x1.0p-23 - 1.0);
    case SYNTH_SMALLINT:
        return (float)((int)(sm64_word(key, idx) % 9u) - 4);
    default: /* SYNTH_UNIFORM01 */
        return (float)((double)(sm64_word(key, idx) >> 40) * 0x1.0p-24);
    }
}

typedef struct {
    float *out;
    int64_t rows, cols, ld, r0, r1;
    uint64_t key;
    int dist;
} fill_job;

static void *fill_rows(void *arg) {
    fill_job *j = (fill_job *)arg;
    for (int64_t r = j->r0; r < j->r1; ++r) {
        float *row = j->out + r * j->ld;
        uint64_t base = (uint64_t)r * (uint64_t)j->cols;
        for (int64_t c = 0; c < j->cols; ++c)
            row[c] = draw(j->key, base + (uint64_t)c, j->dist);
    }
    return 0;
}

/*
 * Fill out[r*ld + c] for 0 <= r < rows, 0 <= c < cols.  Entries with
 * c >= cols (row padding) are left untouched.  Returns 0, or -1 on bad
 * arguments.  nthreads <= 1 runs on the calling thread.
 */
int synth_fill_f32(float *out, int64_t rows, int64_t cols, int64_t ld,
                   uint64_t seed, uint64_t stream, int dist, int nthreads) {
    if (rows < 0 || cols < 0 || ld < cols || dist < 0 || dist > 3) return -1;
    if (rows == 0 || cols == 0) return 0;
    if (!out) return -1;
    uint64_t key = synth_key(seed, stream);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > rows) nthreads = (int)rows;
    fill_job jobs[256];
    pthread_t tid[256];
    int64_t chunk = (rows + nthreads - 1) / nthreads;
    int launched = 0;
    for (int t = 0; t < nthreads; ++t) {
        int64_t r0 = t * chunk, r1 = r0 + chunk < rows ? r0 + chunk : rows;
        if (r0 >= r1) break;
        jobs[t] = (fill_job){out, rows, cols, ld, r0, r1, key, dist};
        if (t == nthreads - 1 || pthread_create(&tid[t], 0, fill_rows, &jobs[t]) != 0) {
            fill_rows(&jobs[t]);
            tid[t] = 0;
        }
        launched = t + 1;
    }
    for (int t = 0; t < launched; ++t)
        if (tid[t]) pthread_join(tid[t], 0);
    return 0;
}
