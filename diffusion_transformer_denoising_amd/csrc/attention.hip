// attention.hip -- flash attention on the matrix cores (self- and cross-attention).
//
// o_h = softmax(q_h k_h^T / sqrt(d)) v_h per head, non-causal, computed in one
// pass over key tiles with an online softmax, so the S x S score matrix never
// exists in memory.
//
// Formulation.  Each wave owns 32 queries and computes transposed products:
//   S^T[keys x queries]  = K * Q^T     (A = K rows from LDS, B = Q in registers)
//   O^T[dims x queries] += V^T * P^T   (A = V^T rows from LDS, B = P from the
//                                       S^T accumulators, no data movement)
// In the 32x32 accumulator layout a lane holds one column, so every lane owns
// exactly one query: its running max, running sum and rescale factor live in
// that lane, and a row reduction is an in-lane loop plus one exchange with the
// lane 32 apart (the other half of the keys).
//
// P as the B operand: the S^T accumulator of key tile mt gives lane half h the
// keys mt*32 + j*8 + h*4 + i.  Chunk c of the P.V contraction (16 keys) feeds
// accumulator elements j in {2(c%2), 2(c%2)+1}, i = 0..3 straight in as the
// fragment; that fixes the order of keys inside the chunk, and the V^T
// fragment is read from LDS in the same order (two 4-key runs per lane).
//
// Scores are kept in the log2 domain (scale folded with log2 e) so the
// exponentials are single v_exp_f32 instructions.  Keys past the end of the
// last tile are masked to -inf; values there are zero-filled in LDS.
#include "device.h"
#include "kernels.h"

namespace dit {

constexpr int ATT_BQ = 128;  // queries per workgroup (4 waves x 32)
constexpr int ATT_BK = 64;   // keys per tile

template <typename T>
__device__ __forceinline__ typename Frag<T>::type load8(const T *p) {
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

// 4 consecutive elements from LDS into fragment slots [s, s + 4).
template <typename T>
__device__ __forceinline__ void load4_into(typename Frag<T>::type &f, int s, const T *p) {
  if constexpr (sizeof(T) == 2) {
    bf16x4 v = *reinterpret_cast<const bf16x4 *>(p);
    f[s] = v[0]; f[s + 1] = v[1]; f[s + 2] = v[2]; f[s + 3] = v[3];
  } else {
    f32x4 v = *reinterpret_cast<const f32x4 *>(p);
    f[s] = v[0]; f[s + 1] = v[1]; f[s + 2] = v[2]; f[s + 3] = v[3];
  }
}

template <typename T, int HD>
__global__ __launch_bounds__(256) void attention_kernel(AttnArgs p) {
  typedef typename Frag<T>::type F;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int KROW = HD + VEC;          // K tile row stride (16-byte pad)
  constexpr int VROW = ATT_BK + 4;        // V^T tile row stride (elements)
  constexpr int QCH = HD / 16;            // k-chunks of the QK^T contraction
  constexpr int DT = HD / 32;             // 32-row dim tiles of O^T
  constexpr int KCH = HD / VEC;           // 16-byte chunks per K row
  constexpr int K_LOADS = ATT_BK * KCH / 256;
  constexpr int VCH = ATT_BK / VEC;       // 16-byte chunks per V^T row
  constexpr int V_LOADS = HD * VCH / 256;
  static_assert(K_LOADS >= 1 && V_LOADS >= 1, "tile too small for 256 threads");

  __shared__ __attribute__((aligned(16))) T ks[ATT_BK * KROW];
  __shared__ __attribute__((aligned(16))) T vs[HD * VROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int head = blockIdx.y;
  const int q0 = blockIdx.x * ATT_BQ + wave * 32;
  const int sq = p.sq, sk = p.sk;
  const T *Q = static_cast<const T *>(p.q) + head * HD;
  const T *Kg = static_cast<const T *>(p.k) + head * HD;
  const T *Vt = static_cast<const T *>(p.vt) + (int64_t)head * HD * p.ldv;

  // Q fragments stay in registers for the whole key loop.
  F qf[QCH];
  {
    const int qi = q0 + l32;
#pragma unroll
    for (int c = 0; c < QCH; ++c) {
      if (qi < sq) {
        qf[c] = load8<T>(Q + (int64_t)qi * p.ldq + c * 16 + half * 8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[c][e] = (T)0.0f;
      }
    }
  }

  f32x16 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[t][e] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  U128 rk[K_LOADS], rv[V_LOADS];
  auto gload = [&](int t0) {
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
      const int c = tid + i * 256, r = c / KCH, cc = (c % KCH) * VEC;
      if (t0 + r < sk)
        rk[i] = *reinterpret_cast<const U128 *>(Kg + (int64_t)(t0 + r) * p.ldk + cc);
      else
        rk[i] = U128{{0u, 0u, 0u, 0u}};
    }
#pragma unroll
    for (int i = 0; i < V_LOADS; ++i) {
      const int c = tid + i * 256, r = c / VCH, key = t0 + (c % VCH) * VEC;
      U128 v = *reinterpret_cast<const U128 *>(Vt + (int64_t)r * p.ldv + key);
      if (key + VEC > sk) {  // zero values past the last key
        T *e = reinterpret_cast<T *>(&v);
#pragma unroll
        for (int x = 0; x < VEC; ++x)
          if (key + x >= sk) e[x] = (T)0.0f;
      }
      rv[i] = v;
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
      const int c = tid + i * 256, r = c / KCH, cc = (c % KCH) * VEC;
      *reinterpret_cast<U128 *>(ks + r * KROW + cc) = rk[i];
    }
#pragma unroll
    for (int i = 0; i < V_LOADS; ++i) {
      const int c = tid + i * 256, r = c / VCH, cc = (c % VCH) * VEC;
      // VROW keeps rows 8-byte aligned only: store as two 8-byte halves.
      uint2 *dst = reinterpret_cast<uint2 *>(vs + r * VROW + cc);
      dst[0] = make_uint2(rv[i].w[0], rv[i].w[1]);
      dst[1] = make_uint2(rv[i].w[2], rv[i].w[3]);
    }
  };

  const int n_tiles = (sk + ATT_BK - 1) / ATT_BK;
  gload(0);
  for (int it = 0; it < n_tiles; ++it) {
    const int t0 = it * ATT_BK;
    __syncthreads();  // previous tile fully consumed
    sstore();
    __syncthreads();
    if (it + 1 < n_tiles) gload(t0 + ATT_BK);

    // ---- S^T = K Q^T for two 32-key tiles
    f32x16 s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[mt][e] = 0.0f;
#pragma unroll
    for (int c = 0; c < QCH; ++c) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        F kf = load8<T>(ks + (mt * 32 + l32) * KROW + c * 16 + half * 8);
        mma32(kf, qf[c], s[mt]);
      }
    }

    // ---- online softmax (log2 domain), one query per lane
    float mx = -INFINITY;
    const bool tail = (t0 + ATT_BK > sk);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float v = s[mt][e] * p.scale_log2;
        if (tail) {
          const int key = t0 + mt * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
          if (key >= sk) v = -INFINITY;
        }
        s[mt][e] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    float psum = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = fast_exp2(s[mt][e] - m_new);
        s[mt][e] = pe;
        psum += pe;
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[t][e] *= alpha;

    // ---- O^T += V^T P^T over four 16-key chunks
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int mt = c >> 1, j0 = (c & 1) * 2;
      F pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = (T)s[mt][j0 * 4 + e];
      const int key_a = mt * 32 + j0 * 8 + half * 4;
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        F vf;
        const T *row = vs + (t * 32 + l32) * VROW;
        load4_into<T>(vf, 0, row + key_a);
        load4_into<T>(vf, 4, row + key_a + 8);
        mma32(vf, pf, o[t]);
      }
    }
  }

  // ---- normalise and store: lane owns query q0 + l32, dims t*32 + j*8 + half*4 + i
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  const int qi = q0 + l32;
  if (qi < sq) {
    T *O = static_cast<T *>(p.o) + (int64_t)qi * p.ldo + head * HD;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        T *dst = O + t * 32 + j * 8 + half * 4;
        if constexpr (sizeof(T) == 2) {
          bf16x4 v4;
#pragma unroll
          for (int i = 0; i < 4; ++i) v4[i] = (bf16)(o[t][j * 4 + i] * inv);
          *reinterpret_cast<bf16x4 *>(dst) = v4;
        } else {
          f32x4 v4;
#pragma unroll
          for (int i = 0; i < 4; ++i) v4[i] = o[t][j * 4 + i] * inv;
          *reinterpret_cast<f32x4 *>(dst) = v4;
        }
      }
  }
}

template <typename T>
static hipError_t launch_attn_t(const AttnArgs &a, hipStream_t s) {
  dim3 grid((a.sq + ATT_BQ - 1) / ATT_BQ, a.heads);
  switch (a.head_dim) {
    case 32: attention_kernel<T, 32><<<grid, 256, 0, s>>>(a); break;
    case 64: attention_kernel<T, 64><<<grid, 256, 0, s>>>(a); break;
    case 128: attention_kernel<T, 128><<<grid, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attention(DType dt, const AttnArgs &a, hipStream_t s) {
  if (a.sq <= 0) return hipSuccess;
  return dt == DT_BF16 ? launch_attn_t<bf16>(a, s) : launch_attn_t<float>(a, s);
}

}  // namespace dit
