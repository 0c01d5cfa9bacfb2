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

// Problem z of a batched launch: its operands start at the batch strides
// (elements of size es) from the first problem's.
__device__ __forceinline__ void att_select_batch(AttnArgs &p, int es, int64_t z) {
  if (p.batch > 1) {
    p.q = static_cast<const char *>(p.q) + z * p.bq * es;
    p.k = static_cast<const char *>(p.k) + z * p.bk * es;
    p.vt = static_cast<const char *>(p.vt) + z * p.bvt * es;
    p.o = static_cast<char *>(p.o) + z * p.bo * es;
  }
}
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
  att_select_batch(p, sizeof(T), blockIdx.z);
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
// the LDS destination, no staging registers), each in its own double-buffered
// ring, so the next tiles stream in while the current ones feed the MFMAs.
//
// Software pipeline, per wave and key tile i (64 keys):
//   phase A: S(i+1) = K(i+1) Q^T on the matrix cores, while the vector ALU
//            finishes P(i) = 2^x(i) (second half), packs it to bf16 and sums it;
//   phase B: O^T += V(i)^T P(i)^T on the matrix cores, while the vector ALU
//            forms x(i+1) = c S(i+1) - m and the first half of P(i+1);
// so the exponentials of one tile run under the products of its neighbours
// instead of between them.
//
// Running max: m is set from the first tile's exact row max and afterwards
// only moves when a lane's partial row sum of a tile exceeds 2^16 (some
// score rose ~16 log2 units above m), tested once per tile after phase A.
// That rare path finds the tile's row max, rescales O and the running sum,
// and recomputes P(i); otherwise p <= 2^16 keeps every value finite in fp32
// and bf16.  Row sums accumulate the bf16 P values (the very numbers the
// P.V product uses) with bf16 dot-2 instructions.
//
// LDS layouts, chosen for conflict-free 16-byte fragment reads:
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

// p = 2^x for the 16 scores of one 32-key half tile -> two bf16 P chunks;
// their sum (of the rounded values) is added to l.
__device__ __forceinline__ void att_exp_half(const f32x16 &x, bf16x8 &lo, bf16x8 &hi, float &l) {
#pragma unroll
  for (int e = 0; e < 8; ++e) lo[e] = (bf16)fast_exp2(x[e]);
#pragma unroll
  for (int e = 0; e < 8; ++e) hi[e] = (bf16)fast_exp2(x[8 + e]);
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bf16x2 pr = {lo[2 * k], lo[2 * k + 1]};
    l = __builtin_amdgcn_fdot2_f32_bf16(pr, one, l, false);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bf16x2 pr = {hi[2 * k], hi[2 * k + 1]};
    l = __builtin_amdgcn_fdot2_f32_bf16(pr, one, l, false);
  }
}

template <int HD, int NW, int KS = 1>
__global__ __launch_bounds__(64 * NW, NW == 8 ? 1 : 2) void attention_bf16_kernel(AttnArgs p) {
  // Workgroup order.  Without a key split (the long sequences) every XCD
  // takes one contiguous range of (query block, head, sequence) triples,
  // query blocks fastest, so its L2 fetches the K and V^T of the one or two
  // heads in its range instead of every head's (Wan-14B self-attention: 3.4
  // instead of 6.0 GB per launch, same time).  The key-split grids of short
  // sequences keep the hardware order: there the contiguous order cut the
  // image_s self-attention's bytes from 28.5 to 7.5 MB per launch, but the
  // step got 0.55 % slower, its output projection finding less of its input
  // in its own XCD's L2.
  int bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;
  if constexpr (KS == 1) {
    const int gx = gridDim.x, gy = gridDim.y;
    const int wg = xcd_contiguous(blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z),
                                  gx * gy * gridDim.z);
    bx = wg % gx;
    by = (wg / gx) % gy;
    bz = wg / (gx * gy);
  }
  att_select_batch(p, 2, bz);
  typedef bf16x8 F;
  constexpr int KROWB = HD * 2;            // bytes per K row
  constexpr int KCHUNK = KROWB / 16;       // 16-byte chunks per K row
  constexpr int KBYTES = ATT_BK * KROWB;   // K tile
  constexpr int VBYTES = HD * ATT_BK * 2;  // V^T tile (rows of 128 bytes)
  constexpr int KPIECES = KBYTES / 16, VPIECES = VBYTES / 16;
  // KS key ranges: the workgroup's waves form KS groups of NWG; the waves of
  // a group cover NWG different 32-query blocks over one key range with their
  // own K/V ring, and wave w of every group holds the same queries, so the
  // groups' partial results are merged through LDS at the end.
  static_assert(KS == 1 || KS == 2, "key split");
  constexpr int NWG = NW / KS;
  constexpr int KINSTR = KPIECES / (64 * NWG), VINSTR = VPIECES / (64 * NWG);
  static_assert(KINSTR >= 1 && VINSTR >= 1 && KPIECES % (64 * NWG) == 0, "tile split");
  constexpr int QCH = HD / 16;
  constexpr int DT = HD / 32;
  constexpr int NQK = 2 * QCH;             // S MFMAs per tile
  constexpr int NPV = 4 * DT;              // P.V MFMAs per tile
  // vector instructions per MFMA slot: phase A has 32 (16 exp, 8 pack, 8 dot),
  // phase B 64 (32 scale, 16 exp, 8 pack, 8 dot)
  constexpr int VA = (32 + NQK - 1) / NQK, VB = (64 + NPV - 1) / NPV;
  constexpr float PSUM_MAX = 65536.0f;

  // per key range: [K stage 0][K stage 1][V^T stage 0][V^T stage 1]
  constexpr int RING = 2 * KBYTES + 2 * VBYTES;
  __shared__ __attribute__((aligned(1024))) char lds[KS * RING];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave / NWG, wig = wave % NWG;  // key range, wave within it
  const int rbase = grp * RING;                  // LDS ring of this key range
  const int half = lane >> 5, l32 = lane & 31;
  const int head = by;
  const int q0 = bx * (32 * NWG) + wig * 32;
  const int sq = p.sq, sk = p.sk;
  const bf16 *Q = static_cast<const bf16 *>(p.q) + head * HD;

  const __amdgpu_buffer_rsrc_t krs = att_rsrc(p.k, (uint32_t)((int64_t)sk * p.ldk * 2));
  const __amdgpu_buffer_rsrc_t vrs =
      att_rsrc(p.vt, (uint32_t)((int64_t)p.heads * HD * p.ldv * 2));

  // Per-lane global byte offsets of the pieces this lane moves (tile 0);
  // piece P = (instr * NWG + wig) * 64 + lane lands at byte 16 P of the ring.
  uint32_t koff[KINSTR], voff[VINSTR];
#pragma unroll
  for (int j = 0; j < KINSTR; ++j) {
    const int P = (j * NWG + wig) * 64 + lane;
    const int row = P / KCHUNK, phys = P % KCHUNK;
    const int logical = phys ^ att_kswz<HD>(row);
    const int key = (row & ~12) | ((row & 4) << 1) | ((row & 8) >> 1);
    koff[j] = (uint32_t)(((int64_t)key * p.ldk + head * HD + logical * 8) * 2);
  }
#pragma unroll
  for (int j = 0; j < VINSTR; ++j) {
    const int P = (j * NWG + wig) * 64 + lane;
    const int row = P / 8, phys = P % 8;
    const int logical = phys ^ ((row >> 1) & 7);
    voff[j] = (uint32_t)((((int64_t)head * HD + row) * p.ldv + logical * 8) * 2);
  }
  const uint32_t kstep = (uint32_t)(ATT_BK * p.ldk * 2);
  // key tiles of this range: n_tiles of them from global tile t_base; with
  // two ranges every range gets the same count (barriers stay matched), the
  // second one ending in a partial or an empty tile (all keys masked)
  const int n_all = (sk + ATT_BK - 1) / ATT_BK;
  const int n_tiles = KS == 1 ? n_all : (n_all + 1) / 2;
  const int t_base = grp * n_tiles;
  const bool ragged = (int64_t)(t_base + n_tiles) * ATT_BK > sk;
  const bool ragged_wg = KS == 1 ? ragged : (int64_t)2 * n_tiles * ATT_BK > sk;  // the last range's
  auto issue_k = [&](int it, int slot) {
    char *b = lds + rbase + slot * KBYTES;
#pragma unroll
    for (int j = 0; j < KINSTR; ++j)
      lds_load16(krs, b + (j * NWG + wig) * 1024, koff[j] + (uint32_t)(t_base + it) * kstep);
  };
  auto issue_v = [&](int it, int slot) {
    char *b = lds + rbase + 2 * KBYTES + slot * VBYTES;
#pragma unroll
    for (int j = 0; j < VINSTR; ++j)
      lds_load16(vrs, b + (j * NWG + wig) * 1024,
                 voff[j] + (uint32_t)(t_base + it) * (ATT_BK * 2));
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

  // per-lane LDS byte offsets of the fragments (stage and tile row offsets
  // are added as immediates)
  int kaddr[QCH], vaddr[4];
  {
    const int kswz = att_kswz<HD>(l32), vswz = (l32 >> 1) & 7;
#pragma unroll
    for (int ch = 0; ch < QCH; ++ch) kaddr[ch] = rbase + l32 * KROWB + (((ch * 2 + half) ^ kswz) * 16);
#pragma unroll
    for (int ch = 0; ch < 4; ++ch)
      vaddr[ch] = rbase + 2 * KBYTES + l32 * 128 + (((ch * 2 + half) ^ vswz) * 16);
  }

  f32x16 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[t][e] = 0.0f;
  const float c = p.scale_log2;
  float m_run, l_run = 0.0f;

  // S^T of the tile in K stage `slot` into s (raw scores)
  auto qk = [&](f32x16 (&s)[2], int slot) {
    static_for<NQK>([&](auto U) {
      constexpr int u = decltype(U)::value, ch = u >> 1, mt = u & 1;
      const F kf = *reinterpret_cast<const F *>(lds + slot * KBYTES + kaddr[ch] + mt * 32 * KROWB);
      if constexpr (ch == 0) {
        f32x16 z;
#pragma unroll
        for (int e = 0; e < 16; ++e) z[e] = 0.0f;
        s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[0], z, 0, 0, 0);
      } else {
        s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ch], s[mt], 0, 0, 0);
      }
    });
  };
  // scores of keys at or past sk -> -inf (tile starting at key t0)
  auto mask = [&](f32x16 (&s)[2], int t0) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        // accumulator row m = (e>>2)*8 + half*4 + (e&3) holds key sigma(m)
        const int key = t0 + mt * 32 + (e >> 3) * 16 + half * 8 + ((e >> 2) & 1) * 4 + (e & 3);
        if (key >= sk) s[mt][e] = -INFINITY;
      }
  };
  // the rare path: move m to the tile's row max, rescale, recompute P
  auto rescale = [&](f32x16 (&x)[2], F (&pc)[4], float &lc) {
    float mx = x[0][0];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, x[mt][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float d = fmaxf(mx, 0.0f);
    m_run += d;
    const float alpha = fast_exp2(-d);
    l_run *= alpha;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[t][e] *= alpha;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) x[mt][e] -= d;
    lc = 0.0f;
    att_exp_half(x[0], pc[0], pc[1], lc);
    att_exp_half(x[1], pc[2], pc[3], lc);
  };

  // One pipeline step: finishes tile i (P(i), O += P(i) V(i)) and, with
  // HAS_NEXT, computes the scores and first half of P of tile i + 1.
  // par = i & 1 selects the stages: K(i+1) in K stage par^1, V(i) in V stage par.
  auto step = [&](auto HAS_NEXT, auto MASK_NEXT, f32x16 (&xc)[2], F (&pc)[4], float &lc,
                  f32x16 (&xn)[2], F (&pn)[4], float &ln, const int i, const int par) {
    constexpr bool has_next = decltype(HAS_NEXT)::value;
    constexpr bool mask_next = decltype(MASK_NEXT)::value;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): K(i+1), V(i) landed
    __syncthreads();                      // ... for every wave; K(i), V(i-1) free
    if (i + 2 < n_tiles) issue_k(i + 2, par);
    if (i + 1 < n_tiles) issue_v(i + 1, par ^ 1);
    if constexpr (!has_next) {
      // every wave of the workgroup takes this barrier when the last range
      // ends short, so the counts match across ranges
      if (ragged_wg) {
        if (ragged) {
          // clear V^T entries of keys past the end (inside the caller's rows)
          bf16 *vt = reinterpret_cast<bf16 *>(lds + rbase + 2 * KBYTES + par * VBYTES);
          const int valid = sk - (t_base + i) * ATT_BK;
          for (int x = wig * 64 + lane; x < HD * ATT_BK; x += NWG * 64) {
            const int row = x / ATT_BK, key = x % ATT_BK;
            if (key >= valid) {
              const int phys = (key >> 3) ^ ((row >> 1) & 7);
              vt[row * ATT_BK + phys * 8 + (key & 7)] = (bf16)0.0f;
            }
          }
        }
        __syncthreads();
      }
    }
    // ---- phase A: S(i+1) on the matrix cores | second half of P(i)
    if constexpr (has_next) qk(xn, par ^ 1);
    att_exp_half(xc[1], pc[2], pc[3], lc);
    if constexpr (has_next) {
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
      static_for<NQK>([&](auto) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x402, VA, 0);
      });
    }
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(!(lc <= PSUM_MAX)) != 0, 0)) {
      asm volatile("" ::: "memory");
      rescale(xc, pc, lc);
    }
    l_run += lc;
    // ---- phase B: O^T += V(i)^T P(i)^T | x(i+1) and first half of P(i+1)
    static_for<NPV>([&](auto U) {
      constexpr int u = decltype(U)::value, ch = u / DT, t = u % DT;
      const F vf = *reinterpret_cast<const F *>(lds + par * VBYTES + vaddr[ch] + t * 32 * 128);
      mma32(vf, pc[ch], o[t]);
    });
    if constexpr (has_next) {
      const float nm = -m_run;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) xn[mt][e] = fmaf(xn[mt][e], c, nm);
      if constexpr (mask_next) mask(xn, (t_base + i + 1) * ATT_BK);
      ln = 0.0f;
      att_exp_half(xn[0], pn[0], pn[1], ln);
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
      static_for<NPV>([&](auto) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x402, VB, 0);
      });
      // keep this work here, under the P.V products: without the pins the
      // compiler sinks it past the next step's barrier
      asm volatile("" : "+v"(xn[1]), "+v"(pn[0]), "+v"(pn[1]), "+v"(ln));
    }
  };

  f32x16 xa[2], xb[2];
  F pa[4], pb[4];
  float la = 0.0f, lb = 0.0f;

  // ---- prologue: tile 0 scores, exact row max, first half of P(0)
  issue_k(0, 0);
  issue_v(0, 0);
  if (n_tiles > 1) issue_k(1, 1);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  qk(xa, 0);
  if (n_tiles == 1 && ragged) mask(xa, t_base * ATT_BK);
  {
    float mx = xa[0][0];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, xa[mt][e]);
    m_run = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c;
    const float nm = -m_run;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) xa[mt][e] = fmaf(xa[mt][e], c, nm);
    att_exp_half(xa[0], pa[0], pa[1], la);
  }

  // ---- steps: pairs with full next tiles (stage parity known), then the
  // odd one, the step whose next tile is ragged, and the last tile
  const int n_plain = (ragged && n_tiles > 1) ? n_tiles - 2 : n_tiles - 1;
  int i = 0;
  for (; i + 1 < n_plain; i += 2) {
    step(std::true_type{}, std::false_type{}, xa, pa, la, xb, pb, lb, i, 0);
    step(std::true_type{}, std::false_type{}, xb, pb, lb, xa, pa, la, i + 1, 1);
  }
  auto take_b = [&]() {
    xa[0] = xb[0]; xa[1] = xb[1];
    pa[0] = pb[0]; pa[1] = pb[1];
    la = lb;
  };
  if (i < n_plain) {
    step(std::true_type{}, std::false_type{}, xa, pa, la, xb, pb, lb, i, 0);
    ++i;
    take_b();
  }
  if (ragged && n_tiles > 1) {
    step(std::true_type{}, std::true_type{}, xa, pa, la, xb, pb, lb, i, i & 1);
    ++i;
    take_b();
  }
  step(std::false_type{}, std::false_type{}, xa, pa, la, xb, pb, lb, i, i & 1);

  if constexpr (KS == 2) {
    // merge the second key range into the first: with m the larger running
    // max, O = O_0 2^(m_0 - m) + O_1 2^(m_1 - m) and the same for the sums
    // (every range holds at least one key, so both maxima are finite)
    float *mrg = reinterpret_cast<float *>(lds) + wig * (DT * 16 + 2) * 64;
    __syncthreads();  // both rings are free
    if (grp == 1) {
      mrg[lane] = m_run;
      mrg[64 + lane] = l_run;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) mrg[(2 + t * 16 + e) * 64 + lane] = o[t][e];
    }
    __syncthreads();
    if (grp == 1) return;
    const float m1 = mrg[lane], l1 = mrg[64 + lane];
    const float mn = fmaxf(m_run, m1);
    const float a0 = fast_exp2(m_run - mn), a1 = fast_exp2(m1 - mn);
    l_run = l_run * a0 + l1 * a1;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[t][e] = o[t][e] * a0 + mrg[(2 + t * 16 + e) * 64 + lane] * a1;
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
        for (int i2 = 0; i2 < 4; ++i2) v4[i2] = (bf16)(o[t][j * 4 + i2] * inv);
        *reinterpret_cast<bf16x4 *>(O + t * 32 + j * 8 + half * 4) = v4;
      }
  }
}

template <int HD>
static hipError_t launch_attn_bf16(const AttnArgs &a, hipStream_t s) {
  // Waves per workgroup: the largest of 8, 4, 2, 1 that still gives at least
  // half a workgroup per CU.  The wave count is fixed by the queries (one per
  // 32); more waves per workgroup share each K/V tile among more of them, so
  // fewer tile loads, against fewer workgroups in flight (measured at 1024
  // tokens, 12 heads: 2 waves and 192 workgroups 10 % faster than 1 and 384,
  // 4 and 96 no faster).  8 waves share each tile among 256 queries (half the
  // LDS fill traffic per MFMA); worth it on long key sequences only, where the
  // fill is the steady state (measured: +2 % at 32760 keys, -11 % at 512).
  // A K tile must give every thread of the workgroup at least one 16-byte piece.
  constexpr int MAXNW = HD >= 64 ? 8 : 4;
  int nw = MAXNW == 8 && a.sk >= 4096 ? 8 : 4;
  const int64_t problems = (int64_t)a.heads * (a.batch > 1 ? a.batch : 1);
  while (nw > 1 && (int64_t)((a.sq + 32 * nw - 1) / (32 * nw)) * problems < 128) nw >>= 1;
  dim3 grid((a.sq + 32 * nw - 1) / (32 * nw), a.heads, a.batch > 1 ? a.batch : 1);
  // Small grids (fewer waves in all than two per SIMD of the chip): split the
  // keys in two ranges, each covered by its own set of waves for the same
  // queries, so every workgroup runs twice the waves.  Needs at least two key
  // tiles.
  const int64_t waves = (int64_t)grid.x * grid.y * grid.z * nw;
  if (nw <= 4 && waves < 2048 && a.sk > ATT_BK) {
    if (nw == 4)
      dit_launch(attention_bf16_kernel<HD, 8, 2>, grid, 512, s, a);
    else if (nw == 2)
      dit_launch(attention_bf16_kernel<HD, 4, 2>, grid, 256, s, a);
    else
      dit_launch(attention_bf16_kernel<HD, 2, 2>, grid, 128, s, a);
    return hipGetLastError();
  }
  if constexpr (MAXNW == 8) {
    if (nw == 8) {
      dit_launch(attention_bf16_kernel<HD, 8>, grid, 512, s, a);
      return hipGetLastError();
    }
  }
  if (nw == 4)
    dit_launch(attention_bf16_kernel<HD, 4>, grid, 256, s, a);
  else if (nw == 2)
    dit_launch(attention_bf16_kernel<HD, 2>, grid, 128, s, a);
  else
    dit_launch(attention_bf16_kernel<HD, 1>, grid, 64, s, a);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_attn_t(const AttnArgs &a, hipStream_t s) {
  dim3 grid((a.sq + ATT_BQ - 1) / ATT_BQ, a.heads, a.batch > 1 ? a.batch : 1);
  switch (a.head_dim) {
    case 32: dit_launch(attention_kernel<T, 32>, grid, 256, s, a); break;
    case 64: dit_launch(attention_kernel<T, 64>, grid, 256, s, a); break;
    case 128: dit_launch(attention_kernel<T, 128>, grid, 256, s, a); break;
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
