/*
 * Seeded, counter-based input generator for the selective-scan workloads.
 *
 * This module holds none of the scan's arithmetic: it only turns (seed, stream, index) into
 * pseudo-random numbers, so that the HIP path and the fp64 oracle can be fed bit-identical
 * inputs, and any slice of a tensor can be regenerated on its own.
 *
 * Definitions (all integer arithmetic is mod 2^64):
 *   mix64(z)  : the SplitMix64 output function (Steele, Lea & Flood, "Fast splittable
 *               pseudorandom number generators", OOPSLA 2014), with the 0xBF58476D1CE4E5B9 /
 *               0x94D049BB133111EB multipliers and 30/27/31 shifts.
 *   GAMMA     : 0x9E3779B97F4A7C15, the SplitMix64 increment.
 *   base(s,j) : mix64(s + GAMMA * (j + 1))                   one key per (seed, tensor stream)
 *   word(s,j,i): mix64(base(s,j) + GAMMA * (i + 1))           i-th output of that SplitMix64 stream
 *   unit(w)   : (w >> 11) * 2^-53                              in [0, 1)
 *   normal(i) : Box-Muller (1958) on the pair of words 2i, 2i+1:
 *               u1 = ((word(2i) >> 11) + 1) * 2^-53  in (0, 1],  u2 = unit(word(2i+1)),
 *               sqrt(-2 ln u1) * cos(2 pi u2), in fp64
 *   uniform(i): lo + (hi - lo) * unit(word(i)), in fp64
 * fp64 values are rounded to fp32 with round-to-nearest-even (the C conversion), and fp32 to
 * bf16 with round-to-nearest-even on the bit pattern (the generator never produces NaN/Inf).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t stream_base(uint64_t seed, uint64_t stream) {
    return mix64(seed + GAMMA * (stream + 1));
}

static inline uint64_t word_at(uint64_t base, uint64_t i) { return mix64(base + GAMMA * (i + 1)); }

static inline double unit53(uint64_t w) { return (double)(w >> 11) * 0x1.0p-53; }

static inline double normal_at(uint64_t base, uint64_t i) {
    double u1 = (double)((word_at(base, 2 * i) >> 11) + 1) * 0x1.0p-53;
    double u2 = unit53(word_at(base, 2 * i + 1));
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t bits;
    memcpy(&bits, &f, 4);
    uint32_t rounding = 0x7FFFu + ((bits >> 16) & 1u);
    return (uint16_t)((bits + rounding) >> 16);
}

enum { DIST_NORMAL = 0, DIST_UNIFORM = 1 };
enum { OUT_F32 = 0, OUT_BF16 = 1, OUT_F64 = 2 };

typedef struct {
    uint64_t base;
    int dist, out_kind;
    double lo, hi;
    int64_t offset, begin, end;
    void* out;
} gen_job;

static void* gen_worker(void* arg) {
    const gen_job* j = (const gen_job*)arg;
    for (int64_t k = j->begin; k < j->end; ++k) {
        uint64_t i = (uint64_t)(j->offset + k);
        double v = (j->dist == DIST_NORMAL) ? normal_at(j->base, i)
                                            : j->lo + (j->hi - j->lo) * unit53(word_at(j->base, i));
        if (j->out_kind == OUT_F64) {
            ((double*)j->out)[k] = v;
        } else if (j->out_kind == OUT_F32) {
            ((float*)j->out)[k] = (float)v;
        } else {
            ((uint16_t*)j->out)[k] = f32_to_bf16_rne((float)v);
        }
    }
    return NULL;
}

#define MAX_THREADS 64

/* Fill out[0..count) with values offset..offset+count-1 of stream (seed, stream).
 * dist: 0 normal(0,1), 1 uniform[lo,hi). out_kind: 0 fp32, 1 bf16 bits (uint16), 2 fp64.
 * Returns 0, or -1 on a bad argument. */
int ssm_gen_fill(uint64_t seed, uint64_t stream, int dist, double lo, double hi, int64_t offset,
                 int64_t count, int out_kind, void* out, int nthreads) {
    if (count < 0 || offset < 0 || (count > 0 && out == NULL)) return -1;
    if (dist != DIST_NORMAL && dist != DIST_UNIFORM) return -1;
    if (out_kind < OUT_F32 || out_kind > OUT_F64) return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > MAX_THREADS) nthreads = MAX_THREADS;
    if (count < 65536) nthreads = 1;
    gen_job jobs[MAX_THREADS];
    pthread_t tids[MAX_THREADS];
    uint64_t base = stream_base(seed, stream);
    int64_t per = (count + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].base = base;
        jobs[t].dist = dist;
        jobs[t].out_kind = out_kind;
        jobs[t].lo = lo;
        jobs[t].hi = hi;
        jobs[t].offset = offset;
        jobs[t].begin = per * t < count ? per * t : count;
        jobs[t].end = per * (t + 1) < count ? per * (t + 1) : count;
        jobs[t].out = out;
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tids[t], NULL, gen_worker, &jobs[t]) != 0) break;
        started = t;
    }
    gen_worker(&jobs[0]);
    for (int t = 1; t <= started; ++t) pthread_join(tids[t], NULL);
    for (int t = started + 1; t < nthreads; ++t) gen_worker(&jobs[t]);
    return 0;
}

/* Raw 64-bit words, for pinning the stream definition. */
void ssm_gen_words(uint64_t seed, uint64_t stream, int64_t offset, int64_t count, uint64_t* out) {
    uint64_t base = stream_base(seed, stream);
    for (int64_t k = 0; k < count; ++k) out[k] = word_at(base, (uint64_t)(offset + k));
}
