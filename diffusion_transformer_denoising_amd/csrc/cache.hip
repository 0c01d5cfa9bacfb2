// cache.hip -- the three bandwidth-bound kernels of block caching across
// denoise steps (page "Disaggregated Diffusion Pipeline", section "GLM-Image
// distributed mode": Cache-DiT with first/last block counts, a residual
// difference threshold and TaylorSeer extrapolation).  All three stream float
// [n] buffers once with 16-byte accesses; n is a multiple of 4.
#include "device.h"
#include "kernels.h"

namespace dit {

// Probe of a step.  For every i: p = x - h0 goes to probe, and h0 takes x (so
// h0 holds h_fn afterwards, the base the middle residual is measured from).
// With ref, workgroup w also writes sum |p - ref| and sum |ref| over its
// elements (float terms, double sums) to partials[2w], partials[2w + 1]; the
// grid-stride order is fixed by n and the grid, so the sums are deterministic.
__global__ __launch_bounds__(256) void cache_probe_kernel(const float *__restrict__ x,
                                                          float *__restrict__ h0,
                                                          float *__restrict__ probe,
                                                          const float *__restrict__ ref,
                                                          int64_t n4, double *__restrict__ partials) {
  double a = 0.0, b = 0.0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const f32x4 xv = reinterpret_cast<const f32x4 *>(x)[i];
    const f32x4 hv = reinterpret_cast<const f32x4 *>(h0)[i];
    f32x4 p;
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = xv[e] - hv[e];
    reinterpret_cast<f32x4 *>(probe)[i] = p;
    reinterpret_cast<f32x4 *>(h0)[i] = xv;
    if (ref) {
      const f32x4 r = reinterpret_cast<const f32x4 *>(ref)[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a += (double)fabsf(p[e] - r[e]);
        b += (double)fabsf(r[e]);
      }
    }
  }
  if (!ref) return;
  // wave sums by xor butterflies, then the four waves through LDS
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    a += __shfl_xor(a, o);
    b += __shfl_xor(b, o);
  }
  __shared__ double sa[4], sb[4];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sa[wave] = a;
    sb[wave] = b;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    partials[2 * blockIdx.x] = (sa[0] + sa[1]) + (sa[2] + sa[3]);
    partials[2 * blockIdx.x + 1] = (sb[0] + sb[1]) + (sb[2] + sb[3]);
  }
}

int cache_probe_groups(int64_t n) {
  const int64_t want = (n / 4 + 255) / 256;
  return (int)(want < CACHE_PROBE_MAX_WG ? (want > 0 ? want : 1) : CACHE_PROBE_MAX_WG);
}

hipError_t launch_cache_probe(const float *x, float *h0, float *probe, const float *ref, int64_t n,
                              double *partials, hipStream_t s) {
  if (n <= 0 || (n & 3)) return hipErrorInvalidValue;
  dit_launch(cache_probe_kernel, cache_probe_groups(n), 256, s, x, h0, probe, ref, n / 4, partials);
  return hipGetLastError();
}

// Cached step: x += T_0 + c1 T_1 + c2 T_2 over the nf factors in hand
// (factor q at tf + q n).
__global__ __launch_bounds__(256) void cache_apply_kernel(float *__restrict__ x,
                                                          const float *__restrict__ tf, int64_t n,
                                                          int nf, float c1, float c2) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n / 4) return;
  f32x4 xv = reinterpret_cast<f32x4 *>(x)[i];
  const f32x4 t0 = reinterpret_cast<const f32x4 *>(tf)[i];
  f32x4 m = t0;
  if (nf > 1) {
    const f32x4 t1 = reinterpret_cast<const f32x4 *>(tf + n)[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) m[e] += c1 * t1[e];
  }
  if (nf > 2) {
    const f32x4 t2 = reinterpret_cast<const f32x4 *>(tf + 2 * n)[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) m[e] += c2 * t2[e];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) xv[e] += m[e];
  reinterpret_cast<f32x4 *>(x)[i] = xv;
}

hipError_t launch_cache_apply(float *x, const float *tf, int64_t n, int nf, float c1, float c2,
                              hipStream_t s) {
  if (n <= 0 || (n & 3) || nf < 1 || nf > 3) return hipErrorInvalidValue;
  const int64_t threads = n / 4;
  dit_launch(cache_apply_kernel, (unsigned)((threads + 255) / 256), 256, s, x, tf, n, nf, c1, c2);
  return hipGetLastError();
}

// Full step: M = x - hf, then the factors in place: T_0 = M and, while the
// older factor exists, T_q = (new T_{q-1} - old T_{q-1}) / gap, for the nnew
// factors kept (nnew <= nold + 1, nnew <= 3).
__global__ __launch_bounds__(256) void cache_update_kernel(const float *__restrict__ x,
                                                           const float *__restrict__ hf,
                                                           float *__restrict__ tf, int64_t n,
                                                           int nnew, float gap) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n / 4) return;
  const f32x4 xv = reinterpret_cast<const f32x4 *>(x)[i];
  const f32x4 hv = reinterpret_cast<const f32x4 *>(hf)[i];
  f32x4 cur;
#pragma unroll
  for (int e = 0; e < 4; ++e) cur[e] = xv[e] - hv[e];
  for (int q = 0; q < nnew; ++q) {
    f32x4 *slot = reinterpret_cast<f32x4 *>(tf + q * n) + i;
    const f32x4 old = *slot;  // factor q of the previous full step
    *slot = cur;
    if (q + 1 < nnew) {
#pragma unroll
      for (int e = 0; e < 4; ++e) cur[e] = (cur[e] - old[e]) / gap;
    }
  }
}

hipError_t launch_cache_update(const float *x, const float *hf, float *tf, int64_t n, int nnew,
                               float gap, hipStream_t s) {
  if (n <= 0 || (n & 3) || nnew < 1 || nnew > 3 || !(gap >= 1.0f)) return hipErrorInvalidValue;
  const int64_t threads = n / 4;
  dit_launch(cache_update_kernel, (unsigned)((threads + 255) / 256), 256, s, x, hf, tf, n, nnew, gap);
  return hipGetLastError();
}

}  // namespace dit
