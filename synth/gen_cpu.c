/* Host (C, OpenMP) twin of the seeded generator defined in gen.py: SplitMix64
 * stream per tensor, Irwin-Hall(4) of the four 16-bit fields, v = mean + z*scale
 * in binary64 (no fusion), rounded to binary32, then to bfloat16 for bf16 tensors.
 * Compiled with -ffp-contract=off. Holds no arithmetic of the decode method. */
#include <stdint.h>
#include <stddef.h>

#define G_INC 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t synth_stream_key(uint64_t seed, uint64_t tid) {
    return mix64(mix64(seed + G_INC) + (tid + 1) * G_INC);
}

static inline double draw(uint64_t key, uint64_t i, double mean, double scale) {
    uint64_t w = mix64(key + (i + 1) * G_INC);
    int64_t s = (int64_t)(w & 0xFFFF) + (int64_t)((w >> 16) & 0xFFFF) +
                (int64_t)((w >> 32) & 0xFFFF) + (int64_t)(w >> 48);
    double t = (double)(s - 131070) * scale;
    return mean + t;
}

static inline uint16_t bf16_rne(float f) {
    union { float f; uint32_t u; } c;
    c.f = f;
    uint32_t u = c.u;
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

/* dst[j] = value(index = start + j) for j < n; dtype 0 = f32, 1 = bf16 bits. */
void synth_fill_flat(void* dst, int dtype, uint64_t n, uint64_t start,
                     uint64_t seed, uint64_t tid, double mean, double scale) {
    uint64_t key = synth_stream_key(seed, tid);
    if (dtype == 0) {
        float* o = (float*)dst;
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < (int64_t)n; ++j) o[j] = (float)draw(key, start + (uint64_t)j, mean, scale);
    } else {
        uint16_t* o = (uint16_t*)dst;
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < (int64_t)n; ++j) o[j] = bf16_rne((float)draw(key, start + (uint64_t)j, mean, scale));
    }
}

/* Stored values (binary32, or bfloat16 for dtype 1) widened exactly to binary64. */
void synth_fill_flat_f64(double* dst, int dtype, uint64_t n, uint64_t start,
                         uint64_t seed, uint64_t tid, double mean, double scale) {
    uint64_t key = synth_stream_key(seed, tid);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < (int64_t)n; ++j) {
        float f = (float)draw(key, start + (uint64_t)j, mean, scale);
        if (dtype == 1) {
            union { float f; uint32_t u; } c;
            c.u = (uint32_t)bf16_rne(f) << 16;
            f = c.f;
        }
        dst[j] = (double)f;
    }
}

/* Cache slab [n_bg][n_slots][head_dim] holding slots slot0..slot0+n_slots-1 of heads
 * bg0..bg0+n_bg-1: element index = ((bg * pitch) + slot) * head_dim + d. */
void synth_fill_cache(void* dst, int dtype, uint64_t bg0, uint64_t n_bg, uint64_t slot0,
                      uint64_t n_slots, uint64_t head_dim, uint64_t pitch,
                      uint64_t seed, uint64_t tid, double mean, double scale) {
    uint64_t key = synth_stream_key(seed, tid);
    int64_t total = (int64_t)(n_bg * n_slots * head_dim);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < total; ++j) {
        uint64_t d = (uint64_t)j % head_dim;
        uint64_t r = (uint64_t)j / head_dim;
        uint64_t slot = slot0 + r % n_slots;
        uint64_t bg = bg0 + r / n_slots;
        uint64_t idx = (bg * pitch + slot) * head_dim + d;
        double v = draw(key, idx, mean, scale);
        if (dtype == 0) ((float*)dst)[j] = (float)v;
        else ((uint16_t*)dst)[j] = bf16_rne((float)v);
    }
}
