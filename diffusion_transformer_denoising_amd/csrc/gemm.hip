// gemm.hip -- MFMA GEMM with fused epilogues for the DiT projections.
//
// C[M, N] = A[M, K] * W[N, K]^T + bias, both operands K-contiguous (the
// row-major [out, in] weight layout), fp32 accumulation on the matrix cores,
// then one of the epilogues of kernels.h applied in registers: bias, GELU,
// gate * (.) added into the fp32 residual stream, fp32 store, or a split
// store that routes column segments to separate buffers (optionally
// transposed, which is how the attention values are laid out).
//
// Tiling: a 256-thread workgroup (4 waves as 2 x 2) owns a BM x BN output
// tile; each wave owns (BM/2) x (BN/2) as 32x32 MFMA tiles.  The K loop
// stages 128-byte slices of A and W rows through LDS (one 16-byte pad per row
// so the fragment reads of 16 consecutive rows hit distinct banks) and
// prefetches the next slice into registers while the current one feeds the
// MFMAs, so one barrier per K step suffices.
#include <cmath>

#include "device.h"
#include "kernels.h"

namespace dit {

template <typename T>
__device__ __forceinline__ typename Frag<T>::type lds_frag(const T *p) {
  typedef typename Frag<T>::type F;
  if constexpr (sizeof(T) == 2) {
    return *reinterpret_cast<const F *>(p);
  } else {
    F f;
    f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
    f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
    f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
    return f;
  }
}

template <typename T, int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs p) {
  constexpr int BK = 128 / sizeof(T);   // elements in a 128-byte row slice
  constexpr int VEC = 16 / sizeof(T);   // elements per 16-byte move
  constexpr int ROW = BK + VEC;         // LDS row stride (elements), 16-byte pad
  constexpr int CHUNKS = BK / 16;       // MFMA k-chunks per slice
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int LA = BM * 8 / 256;      // 16-byte loads per thread for A
  constexpr int LW = BN * 8 / 256;
  typedef typename Frag<T>::type F;

  __shared__ __attribute__((aligned(16))) T lds[2][(BM + BN) * ROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const T *A = static_cast<const T *>(p.A);
  const T *W = static_cast<const T *>(p.W);
  const int M = p.M, N = p.N, K = p.K;

  U128 ra[LA], rw[LW];
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int c = tid + i * 256, r = c >> 3, kk = (c & 7) * VEC;
      const int gm = m0 + r, gk = k0 + kk;
      if (gm < M && gk < K)
        ra[i] = *reinterpret_cast<const U128 *>(A + (int64_t)gm * p.lda + gk);
      else
        ra[i] = U128{{0u, 0u, 0u, 0u}};
    }
#pragma unroll
    for (int i = 0; i < LW; ++i) {
      const int c = tid + i * 256, r = c >> 3, kk = (c & 7) * VEC;
      const int gn = n0 + r, gk = k0 + kk;
      if (gn < N && gk < K)
        rw[i] = *reinterpret_cast<const U128 *>(W + (int64_t)gn * p.ldw + gk);
      else
        rw[i] = U128{{0u, 0u, 0u, 0u}};
    }
  };
  auto sstore = [&](int buf) {
    T *base = lds[buf];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int c = tid + i * 256, r = c >> 3, kk = (c & 7) * VEC;
      *reinterpret_cast<U128 *>(base + r * ROW + kk) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < LW; ++i) {
      const int c = tid + i * 256, r = c >> 3, kk = (c & 7) * VEC;
      *reinterpret_cast<U128 *>(base + (BM + r) * ROW + kk) = rw[i];
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

  const int KT = (K + BK - 1) / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
    const T *base = lds[cur];
#pragma unroll
    for (int ch = 0; ch < CHUNKS; ++ch) {
      const int kk = ch * 16 + (lane >> 5) * 8;
      F af[TM], wf[TN];
#pragma unroll
      for (int a = 0; a < TM; ++a)
        af[a] = lds_frag<T>(base + (wm * WM + a * 32 + (lane & 31)) * ROW + kk);
#pragma unroll
      for (int b = 0; b < TN; ++b)
        wf[b] = lds_frag<T>(base + (BM + wn * WN + b * 32 + (lane & 31)) * ROW + kk);
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b) mma32(af[a], wf[b], acc[a][b]);
    }
    if (kt + 1 < KT) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds column (lane & 31), rows j*8 + (lane>>5)*4 + i
  const T *bias = static_cast<const T *>(p.bias);
#pragma unroll
  for (int b = 0; b < TN; ++b) {
    const int col = n0 + wn * WN + b * 32 + (lane & 31);
    if (col >= N) continue;
    const float bv = bias ? to_f32(bias[col]) : 0.0f;
    float gv = 1.0f;
    if constexpr (EPI == EPI_RESIDUAL) gv = p.gate ? p.gate[col] : 1.0f;
    int seg = 0, sc = col;
    if constexpr (EPI == EPI_SPLIT) {
      seg = col / p.seg_width;
      sc = col - seg * p.seg_width;
    }
#pragma unroll
    for (int a = 0; a < TM; ++a) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row0 = m0 + wm * WM + a * 32 + j * 8 + (lane >> 5) * 4;
        if constexpr (EPI == EPI_SPLIT) {
          if (p.seg_trans[seg]) {
            T *dst = static_cast<T *>(p.seg_ptr[seg]) + (int64_t)sc * p.seg_ld[seg] + row0;
            if (row0 + 3 < M) {
              if constexpr (sizeof(T) == 2) {
                bf16x4 v4;
#pragma unroll
                for (int i = 0; i < 4; ++i) v4[i] = (bf16)(acc[a][b][j * 4 + i] + bv);
                *reinterpret_cast<bf16x4 *>(dst) = v4;
              } else {
                f32x4 v4;
#pragma unroll
                for (int i = 0; i < 4; ++i) v4[i] = acc[a][b][j * 4 + i] + bv;
                *reinterpret_cast<f32x4 *>(dst) = v4;
              }
            } else {
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (row0 + i < M) dst[i] = from_f32<T>(acc[a][b][j * 4 + i] + bv);
            }
            continue;
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = row0 + i;
          if (row >= M) continue;
          const float v = acc[a][b][j * 4 + i] + bv;
          if constexpr (EPI == EPI_STORE) {
            static_cast<T *>(p.out)[(int64_t)row * p.ldo + col] = from_f32<T>(v);
          } else if constexpr (EPI == EPI_GELU) {
            static_cast<T *>(p.out)[(int64_t)row * p.ldo + col] = from_f32<T>(gelu_tanh(v));
          } else if constexpr (EPI == EPI_RESIDUAL) {
            float *o = static_cast<float *>(p.out) + (int64_t)row * p.ldo + col;
            *o = *o + gv * v;
          } else if constexpr (EPI == EPI_STORE_F32) {
            static_cast<float *>(p.out)[(int64_t)row * p.ldo + col] = v;
          } else {
            static_cast<T *>(p.seg_ptr[seg])[(int64_t)row * p.seg_ld[seg] + sc] = from_f32<T>(v);
          }
        }
      }
    }
  }
}

template <typename T, int BM, int BN>
static hipError_t launch_t(Epilogue epi, const GemmArgs &a, hipStream_t s) {
  dim3 grid((a.N + BN - 1) / BN, (a.M + BM - 1) / BM);
  switch (epi) {
    case EPI_STORE: gemm_kernel<T, BM, BN, EPI_STORE><<<grid, 256, 0, s>>>(a); break;
    case EPI_GELU: gemm_kernel<T, BM, BN, EPI_GELU><<<grid, 256, 0, s>>>(a); break;
    case EPI_RESIDUAL: gemm_kernel<T, BM, BN, EPI_RESIDUAL><<<grid, 256, 0, s>>>(a); break;
    case EPI_STORE_F32: gemm_kernel<T, BM, BN, EPI_STORE_F32><<<grid, 256, 0, s>>>(a); break;
    case EPI_SPLIT: gemm_kernel<T, BM, BN, EPI_SPLIT><<<grid, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Tile choice: estimated time = (rounds of workgroups over the chip) x (tile
// area / relative efficiency of that tile), with workgroups per CU set by LDS.
static int pick_tile(int M, int N) {
  struct C { int id, bm, bn, per_cu; double eff; };
  const C cand[] = {{1, 256, 256, 1, 1.0}, {2, 128, 128, 2, 0.55}, {3, 64, 64, 4, 0.25}};
  int best = 3;
  double best_t = 1e300;
  for (const C &c : cand) {
    const double tiles = (double)((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
    const double rounds = std::ceil(tiles / (256.0 * c.per_cu));
    const double t = rounds * c.per_cu * (double)c.bm * c.bn / c.eff;
    if (t < best_t) { best_t = t; best = c.id; }
  }
  return best;
}

hipError_t launch_gemm(DType dt, Epilogue epi, const GemmArgs &a, hipStream_t s, int tile) {
  if (a.M <= 0 || a.N <= 0 || a.K <= 0) return hipSuccess;
  if (dt == DT_BF16) {
    if (tile == 0) tile = pick_tile(a.M, a.N);
    switch (tile) {
      case 1: return launch_t<bf16, 256, 256>(epi, a, s);
      case 2: return launch_t<bf16, 128, 128>(epi, a, s);
      default: return launch_t<bf16, 64, 64>(epi, a, s);
    }
  }
  return launch_t<float, 64, 64>(epi, a, s);
}

}  // namespace dit
