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
  // running max starts finite so the first tile always sets it
  float m_run = -1e30f, l_run = 0.0f;

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

  // Lazy rescaling: the running max m_run (log2 domain) only moves when a
  // tile's max exceeds it by more than RESCALE_T, so most tiles skip the O
  // rescale.  Exponents stay <= RESCALE_T (p <= 256): safe in fp32 and bf16.
  // The decision is made for the whole wave so the branch is uniform.
  constexpr float RESCALE_T = 8.0f;
  const float c = p.scale_log2;
  const T *kbase = ks + l32 * KROW + half * 8;
  const T *vbase = vs + l32 * VROW + half * 4;

  auto tile = [&](auto MASKED, int t0) {
    constexpr bool masked = decltype(MASKED)::value;
    // ---- S^T = K Q^T for two 32-key tiles (raw scores)
    f32x16 s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[mt][e] = 0.0f;
#pragma unroll
    for (int ch = 0; ch < QCH; ++ch) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        F kf = load8<T>(kbase + mt * 32 * KROW + ch * 16);
        mma32(kf, qf[ch], s[mt]);
      }
    }
    if constexpr (masked) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = t0 + mt * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
          if (key >= sk) s[mt][e] = -INFINITY;
        }
    }
    // ---- tile max of the raw scores (scale c > 0 preserves order)
    float mx = s[0][0];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[mt][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + RESCALE_T) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[t][e] *= alpha;
    }
    // ---- p = 2^(s c - m_run), row sums, bf16 fragments, O^T += V^T P^T
    const float nm = -m_run;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = fast_exp2(fmaf(s[mt][e], c, nm));
        s[mt][e] = pe;
        l_run += pe;
      }
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      const int mt = ch >> 1, j0 = (ch & 1) * 2;
      F pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = (T)s[mt][j0 * 4 + e];
      const int key_a = mt * 32 + j0 * 8;
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        F vf;
        load4_into<T>(vf, 0, vbase + t * 32 * VROW + key_a);
        load4_into<T>(vf, 4, vbase + t * 32 * VROW + key_a + 8);
        mma32(vf, pf, o[t]);
      }
    }
  };

  // Full tiles in the loop; the ragged last tile (if any) peeled after it, so
  // the loop carries a single version of the accumulators.
  const int n_tiles = (sk + ATT_BK - 1) / ATT_BK;
  const int n_full = sk / ATT_BK;
  gload(0);
  for (int it = 0; it < n_full; ++it) {
    const int t0 = it * ATT_BK;
    __syncthreads();  // previous tile fully consumed
    sstore();
    __syncthreads();
    if (it + 1 < n_tiles) gload(t0 + ATT_BK);
    tile(std::false_type{}, t0);
  }
  if (n_full < n_tiles) {
    __syncthreads();
    sstore();
    __syncthreads();
    tile(std::true_type{}, n_full * ATT_BK);
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

// ---------------------------------------------------------------------------
// bf16 kernel: K and V^T tiles move global -> LDS directly (buffer loads with
// the LDS destination, no staging registers), double-buffered in LDS, so the
// next tile streams in while the current one feeds the MFMAs.
//
// LDS layouts (per stage), chosen for conflict-free 16-byte fragment reads:
//   K    [64 rows][HD]: row m holds key sigma(m) of the tile, where sigma
//        swaps bits 2 and 3 of m; 16-byte chunk c of row m is stored at chunk
//        c ^ kswz(m).  The row permutation makes the P fragment of lane half
//        h in P.V chunk c cover the 8 consecutive keys c*16 + h*8 + 0..7.
//   V^T  [HD rows][64 keys]: chunk c of row r stored at c ^ ((r >> 1) & 7),
//        so a V^T fragment is one 16-byte read.
// Loads past the last key fall outside the buffer range and read zero; in
// the last, ragged tile the V^T entries past the last key are cleared
// explicitly (they lie inside the caller's rows and may hold anything).
// ---------------------------------------------------------------------------
__device__ __forceinline__ __amdgpu_buffer_rsrc_t att_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

// 16 bytes per lane from a buffer straight into LDS: lane i of the wave
// writes lds_block + 16 i (lds_block is wave-uniform).
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, void *lds_block, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds_block, 16,
                                           voff, 0, 0, 0);
}

template <int HD>
__device__ __forceinline__ int att_kswz(int row) {
  constexpr int KROWB = HD * 2, RP = 256 / KROWB, KCH = KROWB / 16;
  return (row / RP) % KCH;
}

template <int HD, int NW>
__global__ __launch_bounds__(64 * NW, 2) void attention_bf16_kernel(AttnArgs p) {
  typedef bf16x8 F;
  constexpr int KROWB = HD * 2;            // bytes per K row
  constexpr int KCHUNK = KROWB / 16;       // 16-byte chunks per K row
  constexpr int KBYTES = ATT_BK * KROWB;   // K tile
  constexpr int VBYTES = HD * ATT_BK * 2;  // V^T tile (rows of 128 bytes)
  constexpr int STAGE = KBYTES + VBYTES;
  constexpr int KPIECES = KBYTES / 16, VPIECES = VBYTES / 16;
  constexpr int KINSTR = KPIECES / (64 * NW), VINSTR = VPIECES / (64 * NW);
  static_assert(KINSTR >= 1 && VINSTR >= 1 && KPIECES % (64 * NW) == 0, "tile split");
  constexpr int QCH = HD / 16;
  constexpr int DT = HD / 32;
  constexpr int NT = 64 * NW;

  __shared__ __attribute__((aligned(1024))) char lds[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int head = blockIdx.y;
  const int q0 = blockIdx.x * (32 * NW) + wave * 32;
  const int sq = p.sq, sk = p.sk;
  const bf16 *Q = static_cast<const bf16 *>(p.q) + head * HD;

  const __amdgpu_buffer_rsrc_t krs = att_rsrc(p.k, (uint32_t)((int64_t)sk * p.ldk * 2));
  const __amdgpu_buffer_rsrc_t vrs =
      att_rsrc(p.vt, (uint32_t)((int64_t)p.heads * HD * p.ldv * 2));

  // Per-lane global byte offsets of the pieces this lane moves (tile 0);
  // piece P = (instr * NW + wave) * 64 + lane lands at LDS byte 16 P.
  uint32_t koff[KINSTR], voff[VINSTR];
#pragma unroll
  for (int j = 0; j < KINSTR; ++j) {
    const int P = (j * NW + wave) * 64 + lane;
    const int row = P / KCHUNK, phys = P % KCHUNK;
    const int logical = phys ^ att_kswz<HD>(row);
    const int key = (row & ~12) | ((row & 4) << 1) | ((row & 8) >> 1);
    koff[j] = (uint32_t)(((int64_t)key * p.ldk + head * HD + logical * 8) * 2);
  }
#pragma unroll
  for (int j = 0; j < VINSTR; ++j) {
    const int P = (j * NW + wave) * 64 + lane;
    const int row = P / 8, phys = P % 8;
    const int logical = phys ^ ((row >> 1) & 7);
    voff[j] = (uint32_t)((((int64_t)head * HD + row) * p.ldv + logical * 8) * 2);
  }
  const uint32_t kstep = (uint32_t)(ATT_BK * p.ldk * 2);
  auto issue = [&](int it, int stage) {
    char *sbase = lds + stage * STAGE;
#pragma unroll
    for (int j = 0; j < KINSTR; ++j)
      lds_load16(krs, sbase + (j * NW + wave) * 1024, koff[j] + it * kstep);
#pragma unroll
    for (int j = 0; j < VINSTR; ++j)
      lds_load16(vrs, sbase + KBYTES + (j * NW + wave) * 1024, voff[j] + it * (ATT_BK * 2));
  };

  // Q fragments stay in registers for the whole key loop.
  F qf[QCH];
  {
    const int qi = q0 + l32;
#pragma unroll
    for (int c = 0; c < QCH; ++c) {
      if (qi < sq) {
        qf[c] = *reinterpret_cast<const F *>(Q + (int64_t)qi * p.ldq + c * 16 + half * 8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[c][e] = (bf16)0.0f;
      }
    }
  }

  f32x16 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[t][e] = 0.0f;
  float m_run = -1e30f, l_run = 0.0f;
  constexpr float RESCALE_T = 8.0f;
  const float c = p.scale_log2;
  const int kswz = att_kswz<HD>(l32);
  const int vswz = (l32 >> 1) & 7;

  auto tile = [&](auto MASKED, int stage, int t0) {
    constexpr bool masked = decltype(MASKED)::value;
    const char *kb = lds + stage * STAGE + l32 * KROWB;
    const char *vb = lds + stage * STAGE + KBYTES + l32 * 128;
    f32x16 s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[mt][e] = 0.0f;
#pragma unroll
    for (int ch = 0; ch < QCH; ++ch) {
      const int off = ((ch * 2 + half) ^ kswz) * 16;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        F kf = *reinterpret_cast<const F *>(kb + mt * 32 * KROWB + off);
        mma32(kf, qf[ch], s[mt]);
      }
    }
    if constexpr (masked) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          // accumulator row m = (e>>2)*8 + half*4 + (e&3) holds key sigma(m)
          const int key = t0 + mt * 32 + (e >> 3) * 16 + half * 8 + ((e >> 2) & 1) * 4 + (e & 3);
          if (key >= sk) s[mt][e] = -INFINITY;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[mt][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c;
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(mx > m_run + RESCALE_T) != 0, 0)) {
      // rare: keep it a real branch (the empty asm stops the compiler from
      // speculating the 4*HD multiplies onto every tile)
      asm volatile("" ::: "memory");
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[t][e] *= alpha;
    }
    const float nm = -m_run;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = fast_exp2(fmaf(s[mt][e], c, nm));
        s[mt][e] = pe;
        l_run += pe;
      }
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      const int mt = ch >> 1, j0 = (ch & 1) * 2;
      F pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = (bf16)s[mt][j0 * 4 + e];
      const int off = ((ch * 2 + half) ^ vswz) * 16;
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        F vf = *reinterpret_cast<const F *>(vb + t * 32 * 128 + off);
        mma32(vf, pf, o[t]);
      }
    }
  };

  const int n_tiles = (sk + ATT_BK - 1) / ATT_BK;
  const int n_full = sk / ATT_BK;
  issue(0, 0);
  for (int it = 0; it < n_full; ++it) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this tile's loads landed
    __syncthreads();                      // ... for every wave; other stage free
    if (it + 1 < n_tiles) issue(it + 1, (it + 1) & 1);
    tile(std::false_type{}, it & 1, it * ATT_BK);
  }
  if (n_full < n_tiles) {
    const int stage = n_full & 1, t0 = n_full * ATT_BK;
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    // clear V^T entries of keys past the end (inside the caller's rows)
    bf16 *vt = reinterpret_cast<bf16 *>(lds + stage * STAGE + KBYTES);
    const int valid = sk - t0;
    for (int x = tid; x < HD * ATT_BK; x += NT) {
      const int row = x / ATT_BK, key = x % ATT_BK;
      if (key >= valid) {
        const int phys = (key >> 3) ^ ((row >> 1) & 7);
        vt[row * ATT_BK + phys * 8 + (key & 7)] = (bf16)0.0f;
      }
    }
    __syncthreads();
    tile(std::true_type{}, stage, t0);
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  const int qi = q0 + l32;
  if (qi < sq) {
    bf16 *O = static_cast<bf16 *>(p.o) + (int64_t)qi * p.ldo + head * HD;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 v4;
#pragma unroll
        for (int i = 0; i < 4; ++i) v4[i] = (bf16)(o[t][j * 4 + i] * inv);
        *reinterpret_cast<bf16x4 *>(O + t * 32 + j * 8 + half * 4) = v4;
      }
  }
}

template <int HD>
static hipError_t launch_attn_bf16(const AttnArgs &a, hipStream_t s) {
  // waves per workgroup: the largest of 4, 2, 1 that still gives >= 512 workgroups
  int nw = 4;
  while (nw > 1 && (int64_t)((a.sq + 32 * nw - 1) / (32 * nw)) * a.heads < 512) nw >>= 1;
  dim3 grid((a.sq + 32 * nw - 1) / (32 * nw), a.heads);
  if (nw == 4)
    attention_bf16_kernel<HD, 4><<<grid, 256, 0, s>>>(a);
  else if (nw == 2)
    attention_bf16_kernel<HD, 2><<<grid, 128, 0, s>>>(a);
  else
    attention_bf16_kernel<HD, 1><<<grid, 64, 0, s>>>(a);
  return hipGetLastError();
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
  if (dt == DT_BF16) {
    switch (a.head_dim) {
      case 32: return launch_attn_bf16<32>(a, s);
      case 64: return launch_attn_bf16<64>(a, s);
      case 128: return launch_attn_bf16<128>(a, s);
      default: return hipErrorInvalidValue;
    }
  }
  return launch_attn_t<float>(a, s);
}

}  // namespace dit
