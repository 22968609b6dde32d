/*
 * workloads/gen.c -- seeded, counter-based synthetic input generator.
 *
 * This file produces the numbers that both sides of a parity check consume: the
 * fp64 CPU oracle and the HIP path.  It holds none of the attention arithmetic:
 * it only turns (seed, stream id, element index) into a normal or uniform variate,
 * rounds it to binary32 / bfloat16, and adds the fixed structure terms the
 * synthetic workloads carry (chain blocks and repeated subunit blocks in the bias).
 *
 * Generator definition (every value is a pure function of its counter, so any
 * slice of any tensor can be produced independently and in parallel):
 *   mix64(z)        SplitMix64 output function (Steele, Lea & Flood, "Fast
 *                   splittable pseudorandom number generators", OOPSLA 2014).
 *   key(seed, tid)  mix64(mix64(seed) ^ (tid * 0xD1B54A32D192ED03)).
 *   word(key, c)    mix64(key + (c + 1) * 0x9E3779B97F4A7C15).
 *   normal(key, e)  Box-Muller on the word of pair c = e / 2:
 *                   u1 = (hi32 + 0.5) / 2^32, u2 = (lo32 + 0.5) / 2^32,
 *                   r = sqrt(-2 ln u1); even e -> r cos(2 pi u2), odd e -> r sin(2 pi u2).
 *   uniform(key, c) ((word >> 11) + 0.5) / 2^53, in (0, 1).
 * Values are formed in double, rounded once to binary32 (round to nearest even),
 * and, for bfloat16 tensors, rounded once more from binary32 to bfloat16 (RNE).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define WL_GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t wl_stream_key(uint64_t seed, uint64_t tid)
{
    return mix64(mix64(seed) ^ (tid * 0xD1B54A32D192ED03ULL));
}

uint64_t wl_word(uint64_t key, uint64_t ctr)
{
    return mix64(key + (ctr + 1) * WL_GOLDEN);
}

double wl_normal(uint64_t key, uint64_t e)
{
    const double two_pi = 6.283185307179586476925286766559;
    uint64_t w = wl_word(key, e >> 1);
    double u1 = ((double)(w >> 32) + 0.5) * (1.0 / 4294967296.0);
    double u2 = ((double)(w & 0xFFFFFFFFULL) + 0.5) * (1.0 / 4294967296.0);
    double r = sqrt(-2.0 * log(u1));
    return (e & 1) ? r * sin(two_pi * u2) : r * cos(two_pi * u2);
}

double wl_uniform(uint64_t key, uint64_t ctr)
{
    return ((double)(wl_word(key, ctr) >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

/* binary32 -> bfloat16, round to nearest even; NaN stays a quiet NaN. */
uint16_t wl_f32_to_bf16_one(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
        return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

void wl_f32_to_bf16(const float *in, uint16_t *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = wl_f32_to_bf16_one(in[i]);
}

/* out[n] = binary32(sigma * normal(key(seed, tid), start + n)) */
void wl_normal_f32(uint64_t seed, uint64_t tid, int64_t start, int64_t count, double sigma,
                   float *out)
{
    const uint64_t key = wl_stream_key(seed, tid);
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < count; ++n)
        out[n] = (float)(sigma * wl_normal(key, (uint64_t)(start + n)));
}

/* same values, rounded once more to bfloat16 */
void wl_normal_bf16(uint64_t seed, uint64_t tid, int64_t start, int64_t count, double sigma,
                    uint16_t *out)
{
    const uint64_t key = wl_stream_key(seed, tid);
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < count; ++n)
        out[n] = wl_f32_to_bf16_one((float)(sigma * wl_normal(key, (uint64_t)(start + n))));
}

/*
 * Pair bias [B,H,N,N] (k innermost):
 *   sigma * normal(key(seed, tid), flat index)
 *   + chain_add            if chain != NULL and chain[j] == chain[k]
 *   + pattern_h[j%L][k%L]  if L > 0, j/L == k/L and j/L < n_blocks, where
 *                          pattern_h[a][c] = normal(key(seed, pat_tid), (h*L + a)*L + c)
 * The sum is formed in double and rounded once (to binary32, then to bfloat16 when
 * out_bf16 is non-NULL).  Exactly one of out_f32 / out_bf16 is non-NULL.
 */
void wl_bias(uint64_t seed, uint64_t tid, int64_t B, int64_t H, int64_t N, double sigma,
             const int32_t *chain, double chain_add,
             int64_t L, int64_t n_blocks, uint64_t pat_tid,
             float *out_f32, uint16_t *out_bf16)
{
    const uint64_t key = wl_stream_key(seed, tid);
    const uint64_t pkey = wl_stream_key(seed, pat_tid);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t bh = 0; bh < B * H; ++bh) {
        for (int64_t j = 0; j < N; ++j) {
            const int64_t h = bh % H;
            const int64_t row = (bh * N + j) * N;
            for (int64_t kk = 0; kk < N; ++kk) {
                double x = sigma * wl_normal(key, (uint64_t)(row + kk));
                if (chain && chain[j] == chain[kk])
                    x += chain_add;
                if (L > 0 && j / L == kk / L && j / L < n_blocks) {
                    const int64_t a = j % L, c = kk % L;
                    x += wl_normal(pkey, (uint64_t)((h * L + a) * L + c));
                }
                const float f = (float)x;
                if (out_bf16)
                    out_bf16[row + kk] = wl_f32_to_bf16_one(f);
                else
                    out_f32[row + kk] = f;
            }
        }
    }
}
