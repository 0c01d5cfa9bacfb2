// pointwise.hip -- the bandwidth-bound kernels of the denoise step:
// LayerNorm + adaLN modulation, rotary embedding, patchify, fused
// unpatchify + Euler update, and the small time-embedding path.
#include "device.h"
#include "kernels.h"

namespace dit {

// ---------------------------------------------------------------------------
// LayerNorm + modulation.  One wave per row: the row is held in registers
// (NV float4 per lane, NV = ceil(D / 256), fixed per instantiation so the
// loads are issued together without per-chunk branches), mean and variance
// are two wave reductions over the held values (two-pass), then
// y = (x - mu) * rstd * (1 + scale) + shift is written in the element type.
// Rows up to 20 * 256 = 5120 wide.
// ---------------------------------------------------------------------------
constexpr int LN_MAXV = 20;

template <typename T, int NV>
__global__ __launch_bounds__(256) void ln_mod_kernel(const float *__restrict__ x, int rows, int D,
                                                     float eps, const float *__restrict__ shift,
                                                     const float *__restrict__ scale,
                                                     T *__restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float *xr = x + (int64_t)row * D;
  const int nv = D >> 2;  // float4 count
  // Narrow rows: the modulation vectors go out with the row (read after the
  // reductions, each group's load would be another memory round trip before
  // its store).  Wide rows (more than 8 float4 per lane) read them in the
  // store loop instead: held from the start they would take 8 NV more
  // registers and leave two waves per SIMD at width 5120, too few rows in
  // flight to cover the memory latency.
  constexpr bool EARLY = NV <= 8;
  f32x4 v[NV], sh[EARLY ? NV : 1], sc[EARLY ? NV : 1];
  if (EARLY && shift) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = lane + i * 64;
      if (c < nv) {
        sh[EARLY ? i : 0] = *reinterpret_cast<const f32x4 *>(shift + 4 * c);
        sc[EARLY ? i : 0] = *reinterpret_cast<const f32x4 *>(scale + 4 * c);
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + i * 64;
    v[i] = c < nv ? *reinterpret_cast<const f32x4 *>(xr + 4 * c) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    s += (v[i][0] + v[i][1]) + (v[i][2] + v[i][3]);
  }
  const float mu = wave_sum(s) / (float)D;
  float q = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + i * 64;
    if (c < nv) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float d = v[i][e] - mu;
        q += d * d;
      }
    }
  }
  const float var = wave_sum(q) / (float)D;
  const float rstd = 1.0f / sqrtf(var + eps);
  T *yr = y + (int64_t)row * D;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + i * 64;
    if (c < nv) {
      f32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = (v[i][e] - mu) * rstd;
      if (shift) {
        f32x4 shv, scv;
        if constexpr (EARLY) {
          shv = sh[EARLY ? i : 0];
          scv = sc[EARLY ? i : 0];
        } else {
          shv = *reinterpret_cast<const f32x4 *>(shift + 4 * c);
          scv = *reinterpret_cast<const f32x4 *>(scale + 4 * c);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = o[e] * (1.0f + scv[e]) + shv[e];
      }
      if constexpr (sizeof(T) == 2) {
        bf16x4 b;
#pragma unroll
        for (int e = 0; e < 4; ++e) b[e] = (bf16)o[e];
        *reinterpret_cast<bf16x4 *>(yr + 4 * c) = b;
      } else {
        *reinterpret_cast<f32x4 *>(yr + 4 * c) = o;
      }
    }
  }
}

// launch the instantiation with NV == nvl (NV = 1 .. LN_MAXV)
template <typename T, int NV = 1>
static void launch_ln_t(int nvl, dim3 grid, hipStream_t s, const float *x, int rows, int D, float eps,
                        const float *shift, const float *scale, T *y) {
  if (nvl == NV) {
    dit_launch(ln_mod_kernel<T, NV>, grid, 256, s, x, rows, D, eps, shift, scale, y);
  } else if constexpr (NV < LN_MAXV) {
    launch_ln_t<T, NV + 1>(nvl, grid, s, x, rows, D, eps, shift, scale, y);
  }
}

hipError_t launch_ln_modulate(DType dt, const float *x, int rows, int D, float eps,
                              const float *shift, const float *scale, void *y, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (D % 4 != 0 || D > LN_MAXV * 256) return hipErrorInvalidValue;
  dim3 grid((rows + 3) / 4);
  const int nvl = (D / 4 + 63) / 64;
  if (dt == DT_BF16)
    launch_ln_t<bf16>(nvl, grid, s, x, rows, D, eps, shift, scale, static_cast<bf16 *>(y));
  else
    launch_ln_t<float>(nvl, grid, s, x, rows, D, eps, shift, scale, static_cast<float *>(y));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Rotary tables (the rotation itself runs in the QKV projection's epilogue).
// Tables in double precision, rounded once: column j < rf/2 belongs to axis f
// (pair j), then rh/2 columns of axis h, then rw/2 of axis w; the angle is
// pos_axis * theta^(-2 j_axis / r_axis).
__global__ void rope_table_kernel(float *cos_t, float *sin_t, int gf, int gh, int gw, int half_d,
                                  int rf, int rh, int rw, double theta) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t S = (int64_t)gf * gh * gw;
  if (idx >= S * half_d) return;
  const int j = (int)(idx % half_d);
  const int64_t tok = idx / half_d;
  const int pw = (int)(tok % gw);
  const int ph = (int)((tok / gw) % gh);
  const int pf = (int)(tok / ((int64_t)gw * gh));
  int pos, jj, width;
  if (j < rf / 2) {
    pos = pf; jj = j; width = rf;
  } else if (j < (rf + rh) / 2) {
    pos = ph; jj = j - rf / 2; width = rh;
  } else {
    pos = pw; jj = j - (rf + rh) / 2; width = rw;
  }
  const double phi = (double)pos * pow(theta, -2.0 * jj / (double)width);
  cos_t[idx] = (float)cos(phi);
  sin_t[idx] = (float)sin(phi);
}

hipError_t launch_rope_tables(float *cos_t, float *sin_t, int gf, int gh, int gw, int head_dim,
                              int rf, int rh, int rw, float theta, hipStream_t s) {
  const int64_t total = (int64_t)gf * gh * gw * (head_dim / 2);
  if (total <= 0) return hipSuccess;
  dim3 grid((unsigned)((total + 255) / 256));
  dit_launch(rope_table_kernel, grid, 256, s, cos_t, sin_t, gf, gh, gw, head_dim / 2, rf, rh, rw,
                                         (double)theta);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Patchify: token n = (f'*H' + h')*W' + w', element e = ((c*pf + i)*ph + j)*pw + k
// holds X[c, f'*pf + i, h'*ph + j, w'*pw + k].  One thread per output element.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void patchify_kernel(const float *__restrict__ X,
                                                       T *__restrict__ out, int C, int F, int H,
                                                       int W, int pf, int ph, int pw) {
  const int gh = H / ph, gw = W / pw;
  const int P = C * pf * ph * pw;
  const int64_t total = (int64_t)(F / pf) * gh * gw * P;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int e = (int)(idx % P);
  const int64_t n = idx / P;
  const int k = e % pw, j = (e / pw) % ph, i = (e / (pw * ph)) % pf, c = e / (pw * ph * pf);
  const int w_ = (int)(n % gw), h_ = (int)((n / gw) % gh), f_ = (int)(n / ((int64_t)gw * gh));
  const int64_t src = (((int64_t)c * F + f_ * pf + i) * H + h_ * ph + j) * W + w_ * pw + k;
  out[idx] = from_f32<T>(X[src]);
}

hipError_t launch_patchify(DType dt, const float *X, void *patches, int C, int F, int H, int W,
                           int pf, int ph, int pw, hipStream_t s) {
  const int64_t total = (int64_t)C * F * H * W;
  if (total <= 0) return hipSuccess;
  dim3 grid((unsigned)((total + 255) / 256));
  if (dt == DT_BF16)
    dit_launch(patchify_kernel<bf16>, grid, 256, s, X, static_cast<bf16 *>(patches), C, F, H, W, pf,
                                               ph, pw);
  else
    dit_launch(patchify_kernel<float>, grid, 256, s, X, static_cast<float *>(patches), C, F, H, W, pf,
                                                ph, pw);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fused unpatchify + Euler: one thread per latent element (c, f, h, w), which
// reads its velocity from token/element of the patch layout, updates X in
// place and optionally writes the velocity in latent layout.  With guidance
// the velocity is combined from the two branches' tokens first
// (v_neg + g (v_pos - v_neg); page "Support New Diffusion Models - SGLang
// Documentation", sections 1 and 2: guidance_scale, positive and negative
// condition kwargs).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void unpatchify_euler_kernel(const float *__restrict__ u,
                                                               const float *__restrict__ u_neg,
                                                               float g, float *__restrict__ X,
                                                               float *__restrict__ v_out,
                                                               float dt, int C, int F, int H,
                                                               int W, int pf, int ph, int pw) {
  const int64_t total = (int64_t)C * F * H * W;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int w = (int)(idx % W);
  const int h = (int)((idx / W) % H);
  const int f = (int)((idx / ((int64_t)W * H)) % F);
  const int c = (int)(idx / ((int64_t)W * H * F));
  const int gh = H / ph, gw = W / pw;
  const int P = C * pf * ph * pw;
  const int64_t n = ((int64_t)(f / pf) * gh + h / ph) * gw + w / pw;
  const int e = ((c * pf + f % pf) * ph + h % ph) * pw + w % pw;
  float v = u[n * P + e];
  if (u_neg) {
    const float vn = u_neg[n * P + e];
    v = vn + g * (v - vn);
  }
  X[idx] = X[idx] + dt * v;
  if (v_out) v_out[idx] = v;
}

hipError_t launch_unpatchify_euler(const float *u, const float *u_neg, float g, float *X,
                                   float *v_out, float dt, int C, int F, int H, int W, int pf,
                                   int ph, int pw, hipStream_t s) {
  const int64_t total = (int64_t)C * F * H * W;
  if (total <= 0) return hipSuccess;
  dim3 grid((unsigned)((total + 255) / 256));
  dit_launch(unpatchify_euler_kernel, grid, 256, s, u, u_neg, g, X, v_out, dt, C, F, H, W, pf, ph, pw);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void euler_kernel(float *__restrict__ X,
                                                    const float *__restrict__ v, int64_t n,
                                                    float dt) {
  const int64_t i4 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i4 + 3 < n) {
    f32x4 x = *reinterpret_cast<f32x4 *>(X + i4);
    const f32x4 vv = *reinterpret_cast<const f32x4 *>(v + i4);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = x[e] + dt * vv[e];
    *reinterpret_cast<f32x4 *>(X + i4) = x;
  } else {
    for (int64_t i = i4; i < n; ++i) X[i] = X[i] + dt * v[i];
  }
}

hipError_t launch_euler(float *X, const float *v, int64_t n, float dt, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t threads = (n + 3) / 4;
  dim3 grid((unsigned)((threads + 255) / 256));
  dit_launch(euler_kernel, grid, 256, s, X, v, n, dt);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Time path.
// ---------------------------------------------------------------------------
// One wave per output: the wave walks the weight row in 16-byte pieces.  The
// input vector is staged once per workgroup in LDS: x (SiLU applied when
// asked) or, with x == NULL, the timestep sinusoid of width K computed in
// double: [cos(t w_j), sin(t w_j)], w_j = 10000^(-j / (K/2)).
// Fan-out epilogue: with nfan > 0, fan_out[f * N + n] = y[n] + fan[f][n] for
// every f < nfan (fan is a device table of T [N] rows), which builds the
// per-block and head modulation vectors in the same launch.
constexpr int GEMV_MAXK = 8192;

template <typename T>
__global__ __launch_bounds__(256) void gemv_kernel(const T *__restrict__ W, const T *__restrict__ b,
                                                   const float *__restrict__ x, double t,
                                                   float *__restrict__ y, int N, int K,
                                                   int silu_in, const void *const *__restrict__ fan,
                                                   int nfan, float *__restrict__ fan_out) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int PRE = 4;  // weight pieces per lane read before the input is staged
  __shared__ float xs[GEMV_MAXK];
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  const bool live = n < N;
  // Everything that does not depend on the input goes out first (the fan-out
  // row's pointer, the first PRE pieces of the weight row, the bias, the
  // fan-out value), so that its memory latency overlaps the staging instead
  // of following it.  Buffer loads (zero past the range, no branch) and a
  // load through a selected pointer keep the compiler from waiting for them
  // where they are issued.
  const T *fp = W;  // fan-out row f = lane (rows past 64 are read at the end)
  if (live && lane < nfan) fp = static_cast<const T *>(fan[lane]) + n;
  const T *wr = W + (int64_t)(live ? n : 0) * K;
  const auto wrs = make_rsrc(W, (uint32_t)((int64_t)N * K * sizeof(T)));
  const uint32_t wrow = (uint32_t)((int64_t)n * K * sizeof(T));
  U128 pre[PRE];
#pragma unroll
  for (int i = 0; i < PRE; ++i) {
    const int k0 = (lane + i * 64) * VEC;
    pre[i] = buf_load16(wrs, live && k0 < K ? wrow + (uint32_t)(k0 * sizeof(T)) : OOB);
  }
  const auto brs = make_rsrc(b ? static_cast<const void *>(b) : static_cast<const void *>(W),
                             b ? (uint32_t)(N * sizeof(T)) : 0u);
  const uint32_t bbits =
      sizeof(T) == 2 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(brs, n * 2, 0, 0) << 16
                     : (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(brs, n * 4, 0, 0);
  const T fv = *fp;
  if (x) {
    for (int k = threadIdx.x; k < K; k += 256) xs[k] = silu_in ? silu(x[k]) : x[k];
  } else {
    const int half = K / 2;
    for (int j = threadIdx.x; j < half; j += 256) {
      const double a = t * pow(10000.0, -(double)j / (double)half);
      xs[j] = (float)cos(a);
      xs[half + j] = (float)sin(a);
    }
  }
  __syncthreads();
  if (!live) return;
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < PRE; ++i) {
    const int k0 = (lane + i * 64) * VEC;
    if (k0 < K) {
      const T *w = reinterpret_cast<const T *>(&pre[i]);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc += to_f32(w[e]) * xs[k0 + e];
    }
  }
  for (int k0 = (lane + PRE * 64) * VEC; k0 < K; k0 += 64 * VEC) {
    U128 raw = *reinterpret_cast<const U128 *>(wr + k0);
    const T *w = reinterpret_cast<const T *>(&raw);
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc += to_f32(w[e]) * xs[k0 + e];
  }
  const float yv = wave_sum(acc) + __uint_as_float(bbits);  // in every lane
  if (lane == 0) y[n] = yv;
  for (int f = lane; f < nfan; f += 64)
    fan_out[(int64_t)f * N + n] =
        yv + to_f32(f == lane ? fv : static_cast<const T *>(fan[f])[n]);
}

hipError_t launch_gemv(DType dt, const void *W, const void *b, const float *x, float t, float *y,
                       int N, int K, bool silu_in, const void *const *fan, int nfan, float *fan_out,
                       hipStream_t s) {
  if (K > GEMV_MAXK || (!x && (K & 1)) || (nfan > 0 && (!fan || !fan_out))) return hipErrorInvalidValue;
  // 32-bit buffer offsets over the weight matrix
  if ((int64_t)N * K * (dt == DT_BF16 ? 2 : 4) >= (int64_t)OOB) return hipErrorInvalidValue;
  dim3 grid((N + 3) / 4);
  if (dt == DT_BF16)
    dit_launch(gemv_kernel<bf16>, grid, 256, s, static_cast<const bf16 *>(W), static_cast<const bf16 *>(b),
                                           x, (double)t, y, N, K, silu_in, fan, nfan, fan_out);
  else
    dit_launch(gemv_kernel<float>, grid, 256, s, static_cast<const float *>(W), static_cast<const float *>(b),
                                            x, (double)t, y, N, K, silu_in, fan, nfan, fan_out);
  return hipGetLastError();
}

}  // namespace dit
