// kernels.h -- host-side launchers of the DiT kernels (internal to libdit.so).
// Every launcher validates nothing: the C ABI layer checks shapes first.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

// Kernel launches.  When a start event is pending in launch_timing() (the
// profiler sets one before a timed launch), the next dit_launch records it at
// the kernel's own dispatch and the stop event at its completion, through
// hipExtLaunchKernelGGL, rather than as two separate commands around it;
// otherwise it is a plain launch.
struct LaunchTiming {
  hipEvent_t start = nullptr, stop = nullptr;
};
LaunchTiming &launch_timing();  // per host thread

template <typename F, typename... Args>
inline void dit_launch(F kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
  LaunchTiming &t = launch_timing();
  if (t.start) {
    const hipEvent_t a = t.start, b = t.stop;
    t = LaunchTiming{};
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, a, b, 0, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
  }
}

enum DType { DT_F32 = 0, DT_BF16 = 1 };

// GEMM  C[M, N] = A[M, K] * W[N, K]^T + bias[N], followed by one epilogue.
enum Epilogue {
  EPI_STORE = 0,     // out T [M, ldo]            = C
  EPI_GELU = 1,      // out T [M, ldo]            = gelu_tanh(C)
  EPI_RESIDUAL = 2,  // out float [M, ldo]       += gate[col] * C  (gate NULL: 1)
  EPI_STORE_F32 = 3, // out float [M, ldo]        = C
  EPI_SPLIT = 4,     // column segment s = col / seg_width goes to seg_ptr[s]:
                     // row-major [M, seg_ld] or, when seg_trans[s], transposed
                     // [seg_width, seg_ld] (element (row, c) at c * seg_ld + row;
                     // rows are written in runs of 8, so seg_ld must cover M
                     // rounded up to 8); segments flagged seg_rope get the
                     // interleaved rotary rotation with the given tables
};

struct GemmArgs {
  const void *A;
  int64_t lda;
  const void *W;
  int64_t ldw;
  int M, N, K;
  const void *bias;  // T [N] or NULL
  void *out;
  int64_t ldo;
  const float *gate;  // EPI_RESIDUAL
  int seg_width;      // EPI_SPLIT (a multiple of 32)
  void *seg_ptr[3];
  int64_t seg_ld[3];
  int seg_trans[3];
  int seg_rope[3];    // rotate (2j, 2j+1) column pairs of this segment
  const float *rope_cos, *rope_sin;  // [M, rope_half_d] tables, per head
  int rope_half_d;
  // Several sequences stacked along M (the two branches of a guided step):
  // with seg_rows > 0, row r is token r % seg_rows of sequence r / seg_rows;
  // its RoPE table row is r % seg_rows, and a transposed segment stores it at
  // column (r / seg_rows) * seg_bstride + r % seg_rows (seg_rows a multiple
  // of 8).  seg_rows = 0: one sequence, row r at column r.
  int seg_rows;
  int64_t seg_bstride;
  // Grouped launch: `groups` independent problems with the same A and shape;
  // group g uses W = gw[g] and bias = gbias[g] (device tables) and writes split
  // segment s at seg_ptr[s] + g * seg_gstride[s] elements.  groups <= 1: none.
  int groups;
  const void *const *gw;
  const void *const *gbias;
  int64_t seg_gstride[3];
};
// tile: 0 automatic, 1 256x256 (4 waves), 2 128x128, 3 64x64, 4 256x256 (8 waves)
// (bf16); fp32 uses 64x64.
hipError_t launch_gemm(DType dt, Epilogue epi, const GemmArgs &a, hipStream_t s, int tile = 0);
// Operand byte offsets are 32-bit: (rows + 256) * ld * element size < 2^31.
bool gemm_offsets_fit(DType dt, int64_t M, int64_t lda, int64_t N, int64_t ldw);

// Flash attention over heads: o = softmax(q k^T * scale) v, non-causal.
// q [sq, ldq], k [sk, ldk], vt [heads*head_dim, ldv] (values transposed),
// o [sq, ldo]; head h occupies columns h*head_dim .. of q, k and o.
struct AttnArgs {
  const void *q;
  int64_t ldq;
  const void *k;
  int64_t ldk;
  const void *vt;
  int64_t ldv;
  void *o;
  int64_t ldo;
  int sq, sk, heads, head_dim;
  float scale_log2;  // log2(e) / sqrt(head_dim)
  // batch > 1: independent problems on grid.z, problem z at q + z * bq, k +
  // z * bk, vt + z * bvt and o + z * bo (elements); batch <= 1: one problem
  int batch;
  int64_t bq, bk, bvt, bo;
};
hipError_t launch_attention(DType dt, const AttnArgs &a, hipStream_t s);

// y[r, :] = LN(x[r, :]) * (1 + scale) + shift  (plain LN when shift == scale == NULL)
hipError_t launch_ln_modulate(DType dt, const float *x, int rows, int D, float eps,
                              const float *shift, const float *scale, void *y, hipStream_t s);

// cos/sin [S, head_dim/2] for the patch grid (gf, gh, gw) and split (rf, rh, rw).
hipError_t launch_rope_tables(float *cos_t, float *sin_t, int gf, int gh, int gw, int head_dim,
                              int rf, int rh, int rw, float theta, hipStream_t s);

// patches T [S, P] from latents X float [C, F, H, W].
hipError_t launch_patchify(DType dt, const float *X, void *patches, int C, int F, int H, int W,
                           int pf, int ph, int pw, hipStream_t s);

// X += dt * unpatchify(v), v_out (nullable) = unpatchify(v), with the velocity
// tokens v = u (float [S, P]) or, when u_neg is given, the guided
// v = u_neg + g * (u - u_neg).
hipError_t launch_unpatchify_euler(const float *u, const float *u_neg, float g, float *X,
                                   float *v_out, float dt, int C, int F, int H, int W, int pf,
                                   int ph, int pw, hipStream_t s);

// X[i] += dt * v[i], i < n.
hipError_t launch_euler(float *X, const float *v, int64_t n, float dt, hipStream_t s);

// y[n] = sum_k W[n, k] * in[k] + b[n], in = act(x) (act = SiLU when silu_in,
// else identity) or, with x == NULL, the timestep sinusoid of width K:
// [cos(t w_j), sin(t w_j)], w_j = 10000^(-j / (K/2)).  With nfan > 0 also
// fan_out[f, n] = y[n] + fan[f][n], f < nfan, fan a device table of T [N] rows.
hipError_t launch_gemv(DType dt, const void *W, const void *b, const float *x, float t, float *y,
                       int N, int K, bool silu_in, const void *const *fan, int nfan, float *fan_out,
                       hipStream_t s);

// Block caching across steps (float [n] buffers, n a multiple of 4).
// Probe: probe = x - h0, then h0 = x; with ref (nullable) workgroup w writes
// sum |probe - ref| and sum |ref| to partials[2w], partials[2w + 1], over
// cache_probe_groups(n) <= CACHE_PROBE_MAX_WG workgroups.
constexpr int CACHE_PROBE_MAX_WG = 2048;
int cache_probe_groups(int64_t n);
hipError_t launch_cache_probe(const float *x, float *h0, float *probe, const float *ref, int64_t n,
                              double *partials, hipStream_t s);
// x += T_0 + c1 T_1 + c2 T_2 over the first nf (1..3) factors, factor q at tf + q n.
hipError_t launch_cache_apply(float *x, const float *tf, int64_t n, int nf, float c1, float c2,
                              hipStream_t s);
// After a full step: T_0 = x - hf and T_q = (new T_{q-1} - old T_{q-1}) / gap for
// q < nnew (1..3), in place.
hipError_t launch_cache_update(const float *x, const float *hf, float *tf, int64_t n, int nnew,
                               float gap, hipStream_t s);

}  // namespace dit
