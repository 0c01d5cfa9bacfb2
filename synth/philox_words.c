/* Philox-4x32-10 raw output words for the synthetic-input streams.
 *
 * Fills r0[i], r1[i] with the two 64-bit words of block (first + i) of the
 * stream keyed by (k0, k1): counter (idx mod 2^32, idx div 2^32, 0, 0),
 * r0 = x0 | x1 << 32, r1 = x2 | x3 << 32.  Philox-4x32-10 as defined by
 * Salmon et al., "Parallel random numbers: as easy as 1, 2, 3" (SC'11).
 * Integer-only, so the Python twin in philox.py produces identical words. */
#include <stdint.h>

static inline void philox_block(uint64_t idx, uint32_t k0, uint32_t k1,
                                uint64_t *w0, uint64_t *w1) {
  uint32_t c0 = (uint32_t)idx, c1 = (uint32_t)(idx >> 32), c2 = 0, c3 = 0;
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    uint32_t n1 = (uint32_t)p1;
    uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    uint32_t n3 = (uint32_t)p0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  *w0 = (uint64_t)c0 | ((uint64_t)c1 << 32);
  *w1 = (uint64_t)c2 | ((uint64_t)c3 << 32);
}

void synth_philox_words(uint64_t first, int64_t n, uint32_t k0, uint32_t k1,
                        uint64_t *r0, uint64_t *r1) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) philox_block(first + (uint64_t)i, k0, k1, r0 + i, r1 + i);
}

/* Standard normals of the stream: out[2i], out[2i+1] are the Box-Muller pair
 * of block (first + i): u = ((r >> 11) + 1/2) * 2^-53 for r = r0, r1;
 * rad = sqrt(-2 ln u0); out = (rad cos 2 pi u1, rad sin 2 pi u1), each scaled
 * by std in double and rounded once to float.  n_out may be odd (the last
 * block then contributes only its first value). */
#include <math.h>
void synth_normals_f32(uint64_t first, int64_t n_out, uint32_t k0, uint32_t k1,
                       double std, float *out) {
  const int64_t n_pairs = (n_out + 1) / 2;
  const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n_pairs; ++i) {
    uint64_t w0, w1;
    philox_block(first + (uint64_t)i, k0, k1, &w0, &w1);
    double u0 = ((double)(w0 >> 11) + 0.5) * 0x1.0p-53;
    double u1 = ((double)(w1 >> 11) + 0.5) * 0x1.0p-53;
    double rad = sqrt(-2.0 * log(u0));
    double ang = two_pi * u1;
    out[2 * i] = (float)(std * (rad * cos(ang)));
    if (2 * i + 1 < n_out) out[2 * i + 1] = (float)(std * (rad * sin(ang)));
  }
}
