/*
 * Seeded synthetic inputs for the MoE layer: counter-based Gaussian draws.
 *
 * This file holds no part of the layer's arithmetic.  It is the one module
 * that both the CPU oracle's tests and the GPU path's tests/bench take their
 * inputs from, so that the two sides see byte-identical tensors.
 *
 * Generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC'11), written from the published round
 * function: two 32x32->64 multiplies per round, key bumped by the Weyl
 * constants, 10 rounds.  Key = (low 32 bits of seed, tensor id) with the
 * seed's high 32 bits folded into counter word 3; counter words 0..1 = the
 * 64-bit index of the draw pair.
 *
 * One Philox block (4 words) gives two 53-bit uniforms u1 in (0,1] and u2 in
 * [0,1); Box-Muller turns them into two standard normals
 *   z0 = sqrt(-2 ln u1) cos(2 pi u2),  z1 = sqrt(-2 ln u1) sin(2 pi u2).
 * Element i of a tensor takes z0 of pair i/2 when i is even, z1 when odd, so
 * any slice of any tensor can be produced on its own.  The value is scaled by
 * sigma in fp64, then rounded to nearest-even fp32, and (for bf16 output)
 * rounded again to nearest-even bf16.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static void philox4x32_10(uint32_t ctr[4], uint32_t k0, uint32_t k1) {
    for (int r = 0; r < 10; ++r) {
        uint64_t p0 = (uint64_t)PHILOX_M0 * ctr[0];
        uint64_t p1 = (uint64_t)PHILOX_M1 * ctr[2];
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ ctr[1] ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ ctr[3] ^ k1;
        uint32_t n3 = lo0;
        ctr[0] = n0; ctr[1] = n1; ctr[2] = n2; ctr[3] = n3;
        k0 += PHILOX_W0;
        k1 += PHILOX_W1;
    }
}

/* Raw Philox output block for (seed, tensor id, counter). Exposed for the
 * known-answer test of the generator itself. */
void synth_philox_block(uint32_t k0, uint32_t k1, const uint32_t ctr_in[4], uint32_t out[4]) {
    uint32_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
    philox4x32_10(c, k0, k1);
    memcpy(out, c, sizeof(c));
}

static void normal_pair(uint64_t seed, uint32_t tensor_id, uint64_t pair, double* z0, double* z1) {
    uint32_t c[4] = {(uint32_t)pair, (uint32_t)(pair >> 32), 0u, (uint32_t)(seed >> 32)};
    philox4x32_10(c, (uint32_t)seed, tensor_id);
    uint64_t a = ((uint64_t)c[0] << 32) | c[1];
    uint64_t b = ((uint64_t)c[2] << 32) | c[3];
    double u1 = ((double)(a >> 11) + 1.0) * (1.0 / 9007199254740992.0); /* (0,1] */
    double u2 = (double)(b >> 11) * (1.0 / 9007199254740992.0);         /* [0,1) */
    double r = sqrt(-2.0 * log(u1));
    double th = 6.283185307179586476925286766559 * u2;
    *z0 = r * cos(th);
    *z1 = r * sin(th);
}

static uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* Standard-normal draw of elements [first, first+n) of tensor `tensor_id`,
 * scaled by sigma.  dtype 0: fp32 into out (float*); dtype 1: bf16 bit
 * patterns into out (uint16_t*).  When `add` is non-null (fp64, length n), it
 * is added to sigma*z before rounding (used to shift token vectors). */
void synth_normal(uint64_t seed, uint32_t tensor_id, uint64_t first, uint64_t n,
                  double sigma, const double* add, int dtype, void* out, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (n == 0) return;
    /* Work over draw pairs so both Box-Muller outputs are used. */
    const int64_t p0 = (int64_t)(first >> 1), p1 = (int64_t)((first + n - 1) >> 1);
#pragma omp parallel for num_threads(nthreads) schedule(static, 2048)
    for (int64_t p = p0; p <= p1; ++p) {
        double z[2];
        normal_pair(seed, tensor_id, (uint64_t)p, &z[0], &z[1]);
        for (int h = 0; h < 2; ++h) {
            uint64_t i = 2 * (uint64_t)p + (uint64_t)h;
            if (i < first || i >= first + n) continue;
            uint64_t j = i - first;
            double v = sigma * z[h];
            if (add) v += add[j];
            float f = (float)v;
            if (dtype == 0) ((float*)out)[j] = f;
            else ((uint16_t*)out)[j] = f32_to_bf16_rne(f);
        }
    }
}

/* Same as synth_normal, but element j of the output is element
 * first + (j / row_len) * row_stride + (j % row_len) of the tensor, i.e. a
 * strided block of rows; used to draw a few rows of a large tensor. */
void synth_normal_rows(uint64_t seed, uint32_t tensor_id, uint64_t first, uint64_t nrows,
                       uint64_t row_len, uint64_t row_stride, double sigma, const double* add_row,
                       int dtype, void* out, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    const int64_t nn = (int64_t)(nrows * row_len);
#pragma omp parallel for num_threads(nthreads) schedule(static, 4096)
    for (int64_t j = 0; j < nn; ++j) {
        uint64_t r = (uint64_t)j / row_len, c = (uint64_t)j % row_len;
        uint64_t i = first + r * row_stride + c;
        double z0, z1;
        normal_pair(seed, tensor_id, i >> 1, &z0, &z1);
        double v = sigma * ((i & 1u) ? z1 : z0);
        if (add_row) v += add_row[c];
        float f = (float)v;
        if (dtype == 0) ((float*)out)[j] = f;
        else ((uint16_t*)out)[j] = f32_to_bf16_rne(f);
    }
}

/* Raw 32-bit draws (word 0 of each Philox block, counter = index). */
void synth_u32(uint64_t seed, uint32_t tensor_id, uint64_t first, uint64_t n, uint32_t* out) {
    for (uint64_t j = 0; j < n; ++j) {
        uint64_t i = first + j;
        uint32_t c[4] = {(uint32_t)i, (uint32_t)(i >> 32), 0u, (uint32_t)(seed >> 32)};
        philox4x32_10(c, (uint32_t)seed, tensor_id);
        out[j] = c[0];
    }
}
