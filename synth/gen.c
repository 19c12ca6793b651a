/*
 * gen.c -- seeded synthetic inputs shaped like the windows of a diffusion LLM
 * layer.  Shared by the oracle side and the GPU side of the tests and the
 * benchmark; holds none of the drift-detection arithmetic.
 *
 * Random numbers are counter based: element i of stream s under seed S is
 * splitmix64 (Steele, Lea & Flood 2014) of a key mixed from (S, s, i), so any
 * slice can be generated independently and in parallel.  Normals use the
 * Box-Muller transform in fp64; values are rounded to the storage type once
 * (bf16: round to nearest even).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static uint64_t smix(uint64_t z)
{
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static uint64_t rkey(uint64_t seed, uint64_t stream, uint64_t i)
{
    return smix(smix(seed ^ smix(stream * 0xD1B54A32D192ED03ull)) ^ (i * 0x9E3779B97F4A7C15ull));
}

/* uniform in (0, 1) */
static double uni(uint64_t seed, uint64_t stream, uint64_t i)
{
    return ((double)(rkey(seed, stream, i) >> 11) + 0.5) * 0x1p-53;
}

static double gauss(uint64_t seed, uint64_t stream, uint64_t i)
{
    double u1 = uni(seed, stream, 2 * i), u2 = uni(seed, stream, 2 * i + 1);
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

/* Student-t with nu = 3: Z / sqrt(chi2_3 / 3) from four independent normals */
static double student3(uint64_t seed, uint64_t stream, uint64_t i)
{
    double z = gauss(seed, stream, 4 * i);
    double a = gauss(seed, stream, 4 * i + 1), b = gauss(seed, stream, 4 * i + 2),
           c = gauss(seed, stream, 4 * i + 3);
    return z / sqrt((a * a + b * b + c * c) / 3.0);
}

static uint16_t to_bf16(double v)
{
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static double from_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double get(const void* p, int bf16, size_t i)
{
    return bf16 ? from_bf16(((const uint16_t*)p)[i]) : (double)((const float*)p)[i];
}

static void put(void* p, int bf16, size_t i, double v)
{
    if (bf16) ((uint16_t*)p)[i] = to_bf16(v);
    else      ((float*)p)[i] = (float)v;
}

/* out[i] = scale * N(0,1) for i in [0, count), element index offset+i */
void synth_normal(uint64_t seed, uint64_t stream, uint64_t offset, int64_t count, double scale,
                  int bf16, void* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        put(out, bf16, (size_t)i, scale * gauss(seed, stream, offset + (uint64_t)i));
}

/* out[i] = lo + (hi - lo) * U(0,1) as fp32, element index offset+i */
void synth_uniform(uint64_t seed, uint64_t stream, uint64_t offset, int64_t count, double lo,
                   double hi, float* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        out[i] = (float)(lo + (hi - lo) * uni(seed, stream, offset + (uint64_t)i));
}

/* Planted directions: M unit directions u_m (normalised N(0,I) draws), labels
 * uniform in [0, M), h_j = u_{label_j} + noise * N(0,I).  fp32 output. */
void synth_planted(uint64_t seed, int N, int d, int M, double noise, float* out, int32_t* labels)
{
    double* u = (double*)malloc(sizeof(double) * (size_t)M * d);
    for (int m = 0; m < M; ++m) {
        double ss = 0.0;
        for (int e = 0; e < d; ++e) {
            double g = gauss(seed, 5, (uint64_t)m * d + e);
            u[(size_t)m * d + e] = g;
            ss += g * g;
        }
        double inv = 1.0 / sqrt(ss);
        for (int e = 0; e < d; ++e) u[(size_t)m * d + e] *= inv;
    }
    for (int j = 0; j < N; ++j) {
        int lab = (int)(uni(seed, 6, (uint64_t)j) * M);
        if (lab >= M) lab = M - 1;
        labels[j] = lab;
        for (int e = 0; e < d; ++e)
            out[(size_t)j * d + e] =
                (float)(u[(size_t)lab * d + e] + noise * gauss(seed, 1, (uint64_t)j * d + e));
    }
    free(u);
}

/* The first `count` entries of a seeded Fisher-Yates permutation of [0, N),
 * sorted ascending: the rows a drift step perturbs in window w. */
void synth_pick_rows(uint64_t seed, uint64_t stream, int w, int N, int count, int32_t* rows)
{
    int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
    for (int i = 0; i < N; ++i) perm[i] = i;
    for (int i = 0; i < count && i < N - 1; ++i) {
        uint64_t r = rkey(seed, stream, ((uint64_t)w << 32) | (uint64_t)i);
        int j = i + (int)(r % (uint64_t)(N - i));
        int32_t t = perm[i];
        perm[i] = perm[j];
        perm[j] = t;
    }
    for (int i = 0; i < count; ++i) rows[i] = perm[i];
    free(perm);
    /* ascending */
    for (int i = 1; i < count; ++i) {
        int32_t x = rows[i];
        int p = i;
        while (p > 0 && rows[p - 1] > x) { rows[p] = rows[p - 1]; --p; }
        rows[p] = x;
    }
}

/* data[w][row][0:len] += sigma * noise for every row in rows[w][0:nrows];
 * kind 0 = Gaussian, 1 = Student-t (nu = 3).  The noise of (w, row, e) is
 * element (((w0 + w) * N + row) * len + e) of the stream, so a slice of
 * windows starting at global window w0 sees the same noise as the whole. */
void synth_add_noise_rows(uint64_t seed, uint64_t stream, int w0, int W, int N, int len,
                          int nrows, const int32_t* rows, double sigma, int kind, int bf16,
                          void* data)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < (int64_t)W * nrows; ++t) {
        int w = (int)(t / nrows);
        int row = rows[t];
        size_t base = ((size_t)w * N + (size_t)row) * (size_t)len;
        uint64_t gbase = ((uint64_t)(w0 + w) * (uint64_t)N + (uint64_t)row) * (uint64_t)len;
        for (int e = 0; e < len; ++e) {
            uint64_t ix = gbase + (uint64_t)e;
            double z = kind == 1 ? student3(seed, stream, ix) : gauss(seed, stream, ix);
            put(data, bf16, base + e, get(data, bf16, base + e) + sigma * z);
        }
    }
}

/* Rotate each listed row by theta inside the plane of h and a random
 * direction u orthogonal to h (Gram-Schmidt of a Gaussian draw):
 * h' = cos(theta) h + sin(theta) ||h|| u. */
void synth_rotate_rows(uint64_t seed, uint64_t stream, int w0, int W, int N, int len, int nrows,
                       const int32_t* rows, double theta, int bf16, void* data)
{
#pragma omp parallel
    {
        double* h = (double*)malloc(sizeof(double) * (size_t)len);
        double* g = (double*)malloc(sizeof(double) * (size_t)len);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < (int64_t)W * nrows; ++t) {
            int w = (int)(t / nrows);
            int row = rows[t];
            size_t base = ((size_t)w * N + (size_t)row) * (size_t)len;
            double hh = 0.0;
            for (int e = 0; e < len; ++e) { h[e] = get(data, bf16, base + e); hh += h[e] * h[e]; }
            double hn = sqrt(hh);
            if (!(hn > 0.0)) continue;
            uint64_t gbase = ((uint64_t)(w0 + w) * (uint64_t)N + (uint64_t)row) * (uint64_t)len;
            double gh = 0.0;
            for (int e = 0; e < len; ++e) {
                g[e] = gauss(seed, stream, gbase + (uint64_t)e);
                gh += g[e] * h[e] / hn;
            }
            double gg = 0.0;
            for (int e = 0; e < len; ++e) { g[e] -= gh * h[e] / hn; gg += g[e] * g[e]; }
            double gn = sqrt(gg);
            if (!(gn > 0.0)) continue;
            double c = cos(theta), s = sin(theta);
            for (int e = 0; e < len; ++e) put(data, bf16, base + e, c * h[e] + s * hn * g[e] / gn);
        }
        free(h);
        free(g);
    }
}
