// gemm.hip -- MFMA GEMM with fused epilogues for the DiT projections.
//
// C[M, N] = A[M, K] * W[N, K]^T + bias, both operands K-contiguous (the
// row-major [out, in] weight layout), fp32 accumulation on the matrix cores,
// then one epilogue (kernels.h): bias, GELU, gate * (.) added into the fp32
// residual stream, fp32 store, or a split store that routes column segments
// to separate buffers (transposed for the attention values, rotated by RoPE
// for q and k).
//
// A workgroup owns a BM x BN output tile, split over its waves as 32x32 MFMA
// tiles: 8 waves as 2 x 4 (each 128 x 64; two waves per SIMD) for the default
// 256x256 tile, 4 waves as 2 x 2 for the others.  Two main loops:
//   gemm_kernel (256x256 bf16, 64x64 fp32): 128-byte K slices staged through
//     registers into double-buffered, row-padded LDS; the instruction order
//     of a K step is pinned (sched_group_barrier) so fragment reads, staging
//     stores and global loads interleave with the MFMAs, with the barrier
//     before the last chunk.
//   gemm_dl_kernel (64x64, 128x128 bf16): K slices move global -> LDS
//     directly (buffer loads with the LDS destination) into a ring of NS
//     stages, so NS-1 slices are in flight; small problems have too few
//     workgroups per CU to hide memory latency any other way.
// Both share the LDS-staged epilogue (GemmEpilogue).
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

// Order this wave's LDS writes before its later LDS reads (other lanes' data).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// ---------------------------------------------------------------------------
// Epilogue, one 32-row strip of the wave's tile at a time, through the wave's
// own LDS region: phase 1 writes the accumulators (lane = column, 16 rows)
// with bias / GELU / gate applied; phase 2 reads them back as 8-column runs
// of one row, so every global access is a 16-byte (or 32-byte) vector and the
// fp32 residual read-modify-write is coalesced.  RoPE (split segments flagged
// for it) rotates the (2j, 2j+1) pairs of a run in fp32 before rounding.  A
// transposed segment goes through a transposed strip, so each output row
// (one column of C) gets 16-byte runs of consecutive tokens.
// The global operands of a lane (bias and gate of its columns; residual x or
// RoPE cos / sin of its runs) are read either strip by strip inside the
// epilogue or, with PRE, all at once by prefetch() before the main loop, so
// that their memory latency is spent under the products instead of after the
// last one (it is a visible part of a short-K problem; PRE costs registers,
// which the small tiles have to spare).  Every output element has one owner,
// and the residual stream is never an operand of its own product, so reading
// it early reads the same values.
// ---------------------------------------------------------------------------
template <typename T, int WN>
constexpr int gemm_strip_floats() {
  constexpr int SROW = WN + 4, TROW = 32 + 16 / (int)sizeof(T);
  return (32 * SROW * 4 > WN * TROW * (int)sizeof(T) ? 32 * SROW * 4 : WN * TROW * (int)sizeof(T)) / 4;
}

// NWN waves along N, NW waves in all (NW / NWN along M); each wave owns a
// WM x WN block, as TM x TN 32x32 accumulators (CW = 32: lane = column of a
// 32-column block, rows j*8 + (lane/32)*4 + i) or as (2 TM) x (2 TN) 16x16
// accumulators (CW = 16: lane % 16 = column of a 16-column block, rows
// (lane/16)*4 + i of a 16-row block).
template <typename T, int BM, int BN, int EPI, int NWN = 2, int NW = 4, bool PRE = false,
          int CW = 32>
struct GemmEpilogue {
  static constexpr int WM = BM * NWN / NW, WN = BN / NWN, TM = WM / 32, TN = WN / 32;
  static constexpr int NCB = WN / CW;                        // column blocks per wave
  static_assert(CW == 32 || CW == 16, "accumulator layouts");
  static constexpr int SROW = WN + 4;                        // fp32 strip row stride
  static constexpr int TROW = 32 + 16 / (int)sizeof(T);      // transposed strip row stride
  static constexpr int REG = gemm_strip_floats<T, WN>();
  static constexpr int UPR = WN / 8;                         // 8-column runs per strip row
  static constexpr int NIT = 32 * UPR / 64;                  // runs per lane per strip
  static_assert((32 * UPR) % 64 == 0, "whole runs per lane");
  static constexpr int VE = EPI == EPI_RESIDUAL || EPI == EPI_STORE_F32 || sizeof(T) == 4 ? 4 : 8;

  const GemmArgs &p;
  const T *bias;
  int lane, wave, wm, M, N, m0, colbase, segc, trans, rope;
  void *dst;
  int64_t ld;
  bool vec_ok;
  uint32_t bw[NCB];  // bias bits (bf16 in the low half, or fp32) until used
  float gv[NCB];
  f32x4 pre[PRE ? TM : 1][NIT][2];  // per strip with PRE, else the current strip's

  __device__ __forceinline__ GemmEpilogue(const GemmArgs &args, int m0_, int n0,
                                          const void *bias_g, int g)
      : p(args), bias(static_cast<const T *>(bias_g)) {
    lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar segment lookups
    wm = wave / NWN;
    M = p.M;
    N = p.N;
    m0 = m0_;
    colbase = n0 + (wave % NWN) * WN;
    segc = colbase;
    trans = 0;
    rope = 0;
    dst = p.out;
    ld = p.ldo;
    if constexpr (EPI == EPI_SPLIT) {
      const int seg = colbase / p.seg_width;  // a strip never straddles segments
      segc = colbase - seg * p.seg_width;
      trans = p.seg_trans[seg];
      rope = p.seg_rope[seg];
      dst = static_cast<T *>(p.seg_ptr[seg]) + (int64_t)g * p.seg_gstride[seg];
      ld = p.seg_ld[seg];
    }
    vec_ok = (ld % VE) == 0;
  }

  // bias and gate of the lane's column in each CW-column block, by raw buffer
  // loads: past column N, and for a missing operand (an empty range), they
  // return zero without a branch; the bias stays raw bits until it is used, so
  // nothing waits for these loads where they are issued
  __device__ __forceinline__ void load_cols() {
    const auto br = make_rsrc(bias ? static_cast<const void *>(bias) : p.A,
                              bias ? (uint32_t)(N * sizeof(T)) : 0u);
    const auto gr = make_rsrc(EPI == EPI_RESIDUAL && p.gate ? static_cast<const void *>(p.gate) : p.A,
                              EPI == EPI_RESIDUAL && p.gate ? (uint32_t)(N * 4) : 0u);
#pragma unroll
    for (int b = 0; b < NCB; ++b) {
      const uint32_t col = (uint32_t)(colbase + b * CW + (lane & (CW - 1)));
      if constexpr (sizeof(T) == 2)
        bw[b] = __builtin_amdgcn_raw_buffer_load_b16(br, col * 2, 0, 0);
      else
        bw[b] = __builtin_amdgcn_raw_buffer_load_b32(br, col * 4, 0, 0);
      gv[b] = 1.0f;
      if constexpr (EPI == EPI_RESIDUAL)
        gv[b] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(gr, col * 4, 0, 0));
    }
  }

  // residual x (or RoPE cos / sin) of the lane's runs in strip a; runs that
  // take the scalar path (ragged N, unaligned ld) read nothing here
  __device__ __forceinline__ void load_runs(int a, f32x4 (&r)[NIT][2]) {
    if constexpr (EPI == EPI_RESIDUAL || EPI == EPI_SPLIT) {
      if (EPI == EPI_SPLIT && (trans || !rope)) return;
      const int rowbase = m0 + wm * WM + a * 32;
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int u = lane + it * 64;
        const int rr = u / UPR, c8 = (u % UPR) * 8;
        const int row = rowbase + rr, col = colbase + c8;
        if (row >= M || col >= N) continue;
        if constexpr (EPI == EPI_RESIDUAL) {
          if (vec_ok && N - col >= 8) {
            const float *o = static_cast<const float *>(dst) + (int64_t)row * ld + col;
            r[it][0] = *reinterpret_cast<const f32x4 *>(o);
            r[it][1] = *reinterpret_cast<const f32x4 *>(o + 4);
          }
        } else {
          // pairs (2j, 2j+1) of the head; table column = channel / 2
          const int ch0 = (segc + c8) % (2 * p.rope_half_d);
          const int trow = p.seg_rows > 0 ? row % p.seg_rows : row;  // token position
          const int64_t t = (int64_t)trow * p.rope_half_d + ch0 / 2;
          r[it][0] = *reinterpret_cast<const f32x4 *>(p.rope_cos + t);
          r[it][1] = *reinterpret_cast<const f32x4 *>(p.rope_sin + t);
        }
      }
    }
  }

  __device__ __forceinline__ void prefetch() {
    static_assert(PRE, "prefetch() belongs to the PRE form");
    load_cols();
#pragma unroll
    for (int a = 0; a < TM; ++a) load_runs(a, pre[a]);
  }

  // Four consecutive rows r0 .. r0+3 of strip column sc, column block b:
  // bias, GELU or gate applied, into the strip (transposed for a transposed
  // segment).
  __device__ __forceinline__ void put4(float *strip, T *stripT, int sc, int r0, int b,
                                       const float (&a)[4]) {
    const float bv = __uint_as_float(sizeof(T) == 2 ? bw[b] << 16 : bw[b]);
    const float gb = EPI == EPI_RESIDUAL && p.gate ? gv[b] : 1.0f;
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i] + bv;
      if constexpr (EPI == EPI_GELU) v[i] = gelu_tanh(v[i]);
      if constexpr (EPI == EPI_RESIDUAL) v[i] *= gb;
    }
    if (EPI == EPI_SPLIT && trans) {
      if constexpr (sizeof(T) == 2) {
        bf16x4 t4;
#pragma unroll
        for (int i = 0; i < 4; ++i) t4[i] = (bf16)v[i];
        *reinterpret_cast<bf16x4 *>(stripT + sc * TROW + r0) = t4;
      } else {
        *reinterpret_cast<f32x4 *>(stripT + sc * TROW + r0) = f32x4{v[0], v[1], v[2], v[3]};
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) strip[(r0 + i) * SROW + sc] = v[i];
    }
  }

  // The caller has synchronised the workgroup: scratch is free LDS of at
  // least NW * REG floats.  acc is f32x16[TM][TN] (CW = 32) or
  // f32x4[2 TM][2 TN] (CW = 16).
  template <typename ACC>
  __device__ __forceinline__ void store(ACC &acc, float *scratch) {
    float *strip = scratch + wave * REG;
    T *stripT = reinterpret_cast<T *>(strip);
    if constexpr (!PRE) load_cols();
#pragma unroll
    for (int a = 0; a < TM; ++a) {
      const int rowbase = m0 + wm * WM + a * 32;
      // 1. accumulators -> strip
      if constexpr (CW == 32) {
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float v[4] = {acc[a][b][j * 4], acc[a][b][j * 4 + 1], acc[a][b][j * 4 + 2],
                                acc[a][b][j * 4 + 3]};
            put4(strip, stripT, b * 32 + (lane & 31), j * 8 + (lane >> 5) * 4, b, v);
          }
      } else {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int b = 0; b < NCB; ++b) {
            const f32x4 &c = acc[2 * a + t][b];
            const float v[4] = {c[0], c[1], c[2], c[3]};
            put4(strip, stripT, b * 16 + (lane & 15), t * 16 + (lane >> 4) * 4, b, v);
          }
      }
      wave_lds_sync();
      // 2. strip -> global, 8-element runs
      if (EPI == EPI_SPLIT && trans) {
        // row c of the transposed strip = column segc + c of C = output row
        for (int u = lane; u < WN * 4; u += 64) {
          const int c = u >> 2, rr = (u & 3) * 8;
          const int row = rowbase + rr;
          if (row >= M) continue;  // runs past M stay inside the padded rows
          // stacked sequences: token row % seg_rows of sequence row / seg_rows
          // (a run of 8 never straddles two: seg_rows is a multiple of 8)
          const int64_t tcol = p.seg_rows > 0
                                   ? (int64_t)(row / p.seg_rows) * p.seg_bstride + row % p.seg_rows
                                   : row;
          T *o = static_cast<T *>(dst) + (int64_t)(segc + c) * ld + tcol;
          const T *srcp = stripT + c * TROW + rr;
          if constexpr (sizeof(T) == 2) {
            *reinterpret_cast<U128 *>(o) = *reinterpret_cast<const U128 *>(srcp);
          } else {
            *reinterpret_cast<f32x4 *>(o) = *reinterpret_cast<const f32x4 *>(srcp);
            *reinterpret_cast<f32x4 *>(o + 4) = *reinterpret_cast<const f32x4 *>(srcp + 4);
          }
        }
      } else {
        // Without PRE, every global read of this lane's runs comes first, then
        // the stores: with a read and a store per run the compiler cannot move
        // the next run's read above the store (they may alias), and each run
        // would wait a full memory latency.
        const int pa = PRE ? a : 0;
        if constexpr (!PRE) load_runs(a, pre[0]);
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
          const int u = lane + it * 64;
          const int r = u / UPR, c8 = (u % UPR) * 8;
          const int row = rowbase + r, col = colbase + c8;
          if (row >= M || col >= N) continue;
          const int ocol = EPI == EPI_SPLIT ? segc + c8 : col;  // column in the destination
          const float *sp = strip + r * SROW + c8;
          const f32x4 lo = *reinterpret_cast<const f32x4 *>(sp);
          const f32x4 hi = *reinterpret_cast<const f32x4 *>(sp + 4);
          float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          if (EPI == EPI_SPLIT && rope) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float cs = pre[pa][it][0][q], sn = pre[pa][it][1][q];
              const float u0 = v[2 * q], u1 = v[2 * q + 1];
              v[2 * q] = u0 * cs - u1 * sn;
              v[2 * q + 1] = u0 * sn + u1 * cs;
            }
          }
          const int nvalid = N - col < 8 ? N - col : 8;
          if constexpr (EPI == EPI_RESIDUAL) {
            float *o = static_cast<float *>(dst) + (int64_t)row * ld + ocol;
            if (vec_ok && nvalid == 8) {
              f32x4 x0 = pre[pa][it][0], x1 = pre[pa][it][1];
#pragma unroll
              for (int e = 0; e < 4; ++e) { x0[e] += v[e]; x1[e] += v[4 + e]; }
              *reinterpret_cast<f32x4 *>(o) = x0;
              *reinterpret_cast<f32x4 *>(o + 4) = x1;
            } else {
              for (int e = 0; e < nvalid; ++e) o[e] = o[e] + v[e];
            }
          } else if constexpr (EPI == EPI_STORE_F32) {
            float *o = static_cast<float *>(dst) + (int64_t)row * ld + ocol;
            if (vec_ok && nvalid == 8) {
              *reinterpret_cast<f32x4 *>(o) = f32x4{v[0], v[1], v[2], v[3]};
              *reinterpret_cast<f32x4 *>(o + 4) = f32x4{v[4], v[5], v[6], v[7]};
            } else {
              for (int e = 0; e < nvalid; ++e) o[e] = v[e];
            }
          } else {
            T *o = static_cast<T *>(dst) + (int64_t)row * ld + ocol;
            if (vec_ok && nvalid == 8) {
              if constexpr (sizeof(T) == 2) {
                bf16x8 t8;
#pragma unroll
                for (int e = 0; e < 8; ++e) t8[e] = (bf16)v[e];
                *reinterpret_cast<bf16x8 *>(o) = t8;
              } else {
                *reinterpret_cast<f32x4 *>(o) = f32x4{v[0], v[1], v[2], v[3]};
                *reinterpret_cast<f32x4 *>(o + 4) = f32x4{v[4], v[5], v[6], v[7]};
              }
            } else {
              for (int e = 0; e < nvalid; ++e) o[e] = from_f32<T>(v[e]);
            }
          }
        }
      }
      wave_lds_sync();  // the strip is rewritten by the next pass
    }
  }
};

// Tile of this workgroup.  grid.x is 1-D over tiles; workgroups are dispatched to the
// 8 XCDs round-robin (id % 8), so id is first mapped to a contiguous range of
// tiles per XCD, and that range is walked in groups of GM tile rows (row
// fastest inside a group).  The ~32 workgroups an XCD runs at once then cover
// a compact block of the output and share their A and W slices in that XCD's
// L2 instead of spreading over all of them.
__device__ __forceinline__ void gemm_tile_of(int nx, int ny, int &tm, int &tn) {
  constexpr int GM = 4;
  const int T = nx * ny;
  const int t = xcd_contiguous(blockIdx.x, T);
  const int gsz = GM * nx;                       // tiles per group of GM rows
  const int g = t / gsz, r = t - g * gsz;
  const int rows = ny - g * GM < GM ? ny - g * GM : GM;  // rows in this (last) group
  tm = g * GM + r % rows;
  tn = r / rows;
}

// W and bias of this workgroup's problem (grid.y selects the group).
__device__ __forceinline__ void gemm_group(const GemmArgs &p, const void *&W, const void *&bias,
                                           int &g) {
  g = 0;
  W = p.W;
  bias = p.bias;
  if (p.gw) {  // a table is given: it holds the weights, one group per grid row
    g = blockIdx.y;
    W = p.gw[g];
    bias = p.gbias[g];
  }
}

// ---------------------------------------------------------------------------
// Register-staged main loop (256x256 bf16; 64x64 fp32).
// ---------------------------------------------------------------------------
template <typename T, int BM, int BN, int EPI, int NWN = 2, int NW = 4>
__global__ __launch_bounds__(64 * NW) void gemm_kernel(GemmArgs p) {
  constexpr int NT = 64 * NW;           // threads
  constexpr int BK = 128 / sizeof(T);   // elements in a 128-byte row slice
  constexpr int VEC = 16 / sizeof(T);   // elements per 16-byte move
  constexpr int ROW = BK + VEC;         // LDS row stride (elements), 16-byte pad
  constexpr int CHUNKS = BK / 16;       // MFMA k-chunks per slice
  constexpr int WM = BM * NWN / NW, WN = BN / NWN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int RPP = NT / 8;           // rows one pass of 16-byte moves covers
  constexpr int LA = BM / RPP;          // 16-byte loads per thread per slice (A)
  constexpr int LW = BN / RPP;          // (W)
  typedef typename Frag<T>::type F;

  __shared__ __attribute__((aligned(16))) T lds[2][(BM + BN) * ROW];
  static_assert(NW * gemm_strip_floats<T, WN>() * 4 <= (int)sizeof(lds), "epilogue strips");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / NWN, wn = wave % NWN;
  const int M = p.M, N = p.N, K = p.K;
  int tm, tn;
  gemm_tile_of((N + BN - 1) / BN, (M + BM - 1) / BM, tm, tn);
  const int m0 = tm * BM;
  const int n0 = tn * BN;

  // Each thread moves the 16-byte piece kk of rows (tid >> 3) + RPP i.
  const int kk = (tid & 7) * VEC;
  const int r0 = tid >> 3;
  const __amdgpu_buffer_rsrc_t ra_src = make_rsrc(p.A, (uint32_t)((int64_t)M * p.lda * sizeof(T)));
  const void *Wg, *bias_g;
  int g;
  gemm_group(p, Wg, bias_g, g);
  const __amdgpu_buffer_rsrc_t rw_src = make_rsrc(Wg, (uint32_t)((int64_t)N * p.ldw * sizeof(T)));
  const uint32_t a_off0 = (uint32_t)(((int64_t)(m0 + r0) * p.lda + kk) * sizeof(T));
  const uint32_t w_off0 = (uint32_t)(((int64_t)(n0 + r0) * p.ldw + kk) * sizeof(T));
  const uint32_t a_step = (uint32_t)(RPP * p.lda * sizeof(T));
  const uint32_t w_step = (uint32_t)(RPP * p.ldw * sizeof(T));

  // Staging registers for one slice: pieces 0..LA-1 are A rows, LA.. are W rows.
  constexpr int NP = LA + LW;
  U128 stage[NP];
  auto gload_piece = [&](int i, int kt) {
    const int k0 = kt * BK;
    const bool kin = (k0 + kk) < K;
    const uint32_t kb = (uint32_t)(k0 * sizeof(T));
    if (i < LA)
      stage[i] = buf_load16(ra_src, kin ? a_off0 + i * a_step + kb : OOB);
    else
      stage[i] = buf_load16(rw_src, kin ? w_off0 + (i - LA) * w_step + kb : OOB);
  };
  auto sstore_piece = [&](int i, T *base) {
    const int row = i < LA ? r0 + RPP * i : BM + r0 + RPP * (i - LA);
    *reinterpret_cast<U128 *>(base + row * ROW + kk) = stage[i];
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

  // fragment source rows of this lane within the LDS tile
  const int arow = (wm * WM + (lane & 31)) * ROW + (lane >> 5) * 8;
  const int wrow = (BM + wn * WN + (lane & 31)) * ROW + (lane >> 5) * 8;
  F af[2][TM], wf[2][TN];
  auto lload = [&](const T *base, int ch, int slot) {
#pragma unroll
    for (int a = 0; a < TM; ++a) af[slot][a] = lds_frag<T>(base + arow + a * 32 * ROW + ch * 16);
#pragma unroll
    for (int b = 0; b < TN; ++b) wf[slot][b] = lds_frag<T>(base + wrow + b * 32 * ROW + ch * 16);
  };

  // Schedule of one K step (slice kt in LDS buffer cur, slice kt+1 in the
  // staging registers):
  //   chunks 0 .. CHUNKS-2: read the next chunk's fragments, issue this
  //     chunk's MFMAs, and move a share of slice kt+1 from the staging
  //     registers into the other LDS buffer, refilling each register with
  //     slice kt+2 right after it is stored;
  //   barrier (all fragments of slice kt are in registers, slice kt+1 is in
  //     LDS), then the last chunk's MFMAs overlap with reading the first
  //     fragments of slice kt+1.
  // The buffer written during step kt was last read before the previous
  // step's barrier, so one barrier per step suffices.
  constexpr int PER = (NP + CHUNKS - 2) / (CHUNKS - 1);
  const int KT = (K + BK - 1) / BK;
#pragma unroll
  for (int i = 0; i < NP; ++i) gload_piece(i, 0);
#pragma unroll
  for (int i = 0; i < NP; ++i) sstore_piece(i, lds[0]);
#pragma unroll
  for (int i = 0; i < NP; ++i) gload_piece(i, 1);
  __syncthreads();
  lload(lds[0], 0, 0);
  // Instruction mix per chunk, for pinning the schedule: MFMAs, fragment
  // reads, and (chunks 0 .. CHUNKS-2) staging stores + global loads.
  constexpr int NM = TM * TN * (sizeof(T) == 2 ? 1 : 8);
  constexpr int NR = (TM + TN) * (sizeof(T) == 2 ? 1 : 2);
  constexpr bool PIN = NM >= NR;

  // The step body is branch-free: past the last slice the loads fall out of
  // range and return zero, and the stores go to a buffer nobody reads again.
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    const T *base = lds[cur];
    T *next = lds[cur ^ 1];
    static_for<CHUNKS>([&](auto CH) {
      constexpr int ch = CH;
      constexpr int slot = ch & 1;
      if constexpr (ch + 1 < CHUNKS) {
        lload(base, ch + 1, slot ^ 1);
      } else {
        __syncthreads();
        lload(next, 0, slot ^ 1);
      }
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b) mma32(af[slot][a], wf[slot][b], acc[a][b]);
      // staging pieces moved during this chunk
      constexpr int first = ch * PER;
      constexpr int nw = ch + 1 < CHUNKS ? (NP - first < PER ? (NP - first > 0 ? NP - first : 0) : PER) : 0;
#pragma unroll
      for (int i = first; i < first + nw; ++i) {
        sstore_piece(i, next);
        gload_piece(i, kt + 2);
      }
      if constexpr (PIN) {
        // fragment reads paired with MFMAs, then store + load (+ MFMA while
        // any are left), then the remaining MFMAs
        constexpr int PAIRS = NR < NM ? NR : NM;
        static_for<PAIRS>([&](auto) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        });
        constexpr int WM_ = nw < NM - PAIRS ? nw : NM - PAIRS;  // stores that get an MFMA
        static_for<nw>([&](auto W) {
          __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
          if constexpr (W < WM_) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        });
        constexpr int left = NM - PAIRS - WM_;
        if constexpr (left > 0) __builtin_amdgcn_sched_group_barrier(0x008, left, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    });
  }


  __syncthreads();  // every wave is done with the main-loop buffers
  GemmEpilogue<T, BM, BN, EPI, NWN, NW>(p, m0, n0, bias_g, g)
      .store(acc, reinterpret_cast<float *>(&lds[0][0]));
}

// ---------------------------------------------------------------------------
// Register-staged main loop on 16x16x32 MFMAs (bf16, 256x256, 8 waves).
// Same slice staging, LDS layout (128-byte rows + 16 bytes of padding) and
// one barrier per 64-k slice as gemm_kernel, but each slice is two 32-k
// chunks of v_mfma_f32_16x16x32_bf16, and a wave's WM x WN block is
// (WM/16) x (WN/16) 16x16 accumulators.  A fragment (16 bytes per lane) now
// covers 16 rows x 32 k, so a chunk needs twice the fragments of a 32x32x16
// chunk; to keep the register count, the W fragments are double-buffered
// across chunks while the A fragments stream through a ring of four: A
// fragment a + 4 (or, past the chunk's last, fragment a - 4 of the next
// chunk) is read as soon as the MFMAs of fragment a have been issued.
// Lane layout of the instruction: A and B lanes l hold row l % 16, k
// (l / 16) * 8 .. + 7; the accumulator lane l holds rows (l / 16) * 4 + i of
// column l % 16.
// ---------------------------------------------------------------------------
template <int EPI, int NWN = 4, int NW = 8>
__global__ __launch_bounds__(64 * NW) void gemm16_kernel(GemmArgs p) {
  typedef bf16 T;
  constexpr int BM = 256, BN = 256, NT = 64 * NW;
  // LDS rows of 128 bytes (64 k) without padding; the 16-byte chunk c of row
  // r is stored at chunk c ^ (r & 7).  A 16-row fragment read (lane l: row
  // l % 16, chunk 4 ch + l / 16) then meets no bank conflicts: with rows padded
  // to 144 bytes, as the 32x32x16 loop has them, the same reads took 1.7x as
  // long in an LDS probe, and the kernel counted 60x the conflict cycles.
  constexpr int BK = 64, VEC = 8, ROW = BK, CHUNKS = BK / 32;
  // 8 waves: 128 x 64 per wave as 8 x 4 accumulators.  (4 waves of 128 x 128,
  // one wave per SIMD with the accumulators in AGPRs, also fit this code; they
  // were 16-27 % slower on the step shapes.)
  constexpr int WM = BM * NWN / NW, WN = BN / NWN;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int RING = 4;
  static_assert(TM == 2 * RING, "the A ring covers half a chunk");
  constexpr int RPP = NT / 8, LA = BM / RPP, LW = BN / RPP, NP = LA + LW;
  // per A fragment: staging pieces moved in chunk 0, and (from fragment RING
  // on, i.e. after the last chunk's barrier) W fragments of the next chunk read
  constexpr int SPER = NP / TM, WPER = TN / (TM - RING);
  static_assert(SPER * TM == NP && WPER * (TM - RING) == TN, "schedule shares");
  __shared__ __attribute__((aligned(16))) T lds[2][(BM + BN) * ROW];
  static_assert(NW * gemm_strip_floats<T, WN>() * 4 <= (int)sizeof(lds), "epilogue strips");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / NWN, wn = wave % NWN;
  const int M = p.M, N = p.N, K = p.K;
  int tm, tn;
  gemm_tile_of((N + BN - 1) / BN, (M + BM - 1) / BM, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const int kk = (tid & 7) * VEC, r0 = tid >> 3;
  const __amdgpu_buffer_rsrc_t ra_src = make_rsrc(p.A, (uint32_t)((int64_t)M * p.lda * 2));
  const void *Wg, *bias_g;
  int g;
  gemm_group(p, Wg, bias_g, g);
  const __amdgpu_buffer_rsrc_t rw_src = make_rsrc(Wg, (uint32_t)((int64_t)N * p.ldw * 2));
  const uint32_t a_off0 = (uint32_t)(((int64_t)(m0 + r0) * p.lda + kk) * 2);
  const uint32_t w_off0 = (uint32_t)(((int64_t)(n0 + r0) * p.ldw + kk) * 2);
  const uint32_t a_step = (uint32_t)(RPP * p.lda * 2), w_step = (uint32_t)(RPP * p.ldw * 2);

  U128 stage[NP];
  auto gload_piece = [&](int i, int kt) {
    const int k0 = kt * BK;
    const bool kin = (k0 + kk) < K;
    const uint32_t kb = (uint32_t)(k0 * 2);
    if (i < LA)
      stage[i] = buf_load16(ra_src, kin ? a_off0 + i * a_step + kb : OOB);
    else
      stage[i] = buf_load16(rw_src, kin ? w_off0 + (i - LA) * w_step + kb : OOB);
  };
  // r0 + RPP i and BM + ... share r0's low three bits (RPP and BM are
  // multiples of 8), so the stored chunk is the same for every piece
  const int kk_sw = (((tid & 7) ^ (r0 & 7)) * VEC);
  auto sstore_piece = [&](int i, T *base) {
    const int row = i < LA ? r0 + RPP * i : BM + r0 + RPP * (i - LA);
    *reinterpret_cast<U128 *>(base + row * ROW + kk_sw) = stage[i];
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) acc[a][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // every fragment row of this lane has low bits (lane & 7): its chunk of
  // k-chunk ch is (4 ch + lane / 16) ^ (lane & 7)
  const int arow = (wm * WM + (lane & 15)) * ROW;
  const int wrow = (BM + wn * WN + (lane & 15)) * ROW;
  int chk[CHUNKS];
#pragma unroll
  for (int ch = 0; ch < CHUNKS; ++ch) chk[ch] = ((ch * 4 + (lane >> 4)) ^ (lane & 7)) * VEC;
  bf16x8 ar[RING], wf[2][TN];
  auto afrag = [&](const T *base, int ch, int a) {
    return *reinterpret_cast<const bf16x8 *>(base + arow + a * 16 * ROW + chk[ch]);
  };
  auto wfrag = [&](const T *base, int ch, int b) {
    return *reinterpret_cast<const bf16x8 *>(base + wrow + b * 16 * ROW + chk[ch]);
  };

  const int KT = (K + BK - 1) / BK;
#pragma unroll
  for (int i = 0; i < NP; ++i) gload_piece(i, 0);
#pragma unroll
  for (int i = 0; i < NP; ++i) sstore_piece(i, lds[0]);
#pragma unroll
  for (int i = 0; i < NP; ++i) gload_piece(i, 1);
  __syncthreads();
#pragma unroll
  for (int a = 0; a < RING; ++a) ar[a] = afrag(lds[0], 0, a);
#pragma unroll
  for (int b = 0; b < TN; ++b) wf[0][b] = wfrag(lds[0], 0, b);

  // Chunk 0 of a step moves every staging piece (slice kt+1 into the other
  // buffer, then slice kt+2 into the registers).  In the last chunk, the
  // ring reads of the current buffer come first (fragments 0 .. RING-1 of the
  // chunk are already in the ring), then the one barrier of the step, after
  // which slice kt+1 is in the other buffer for every wave and the current
  // buffer is no longer read by any wave (so the next step may overwrite it);
  // the next slice's first fragments are read after it.  The step body is
  // branch-free: past the last slice the loads fall out of range and return
  // zero.
  for (int kt = 0; kt < KT; ++kt) {
    const T *base = lds[kt & 1];
    T *next = lds[(kt & 1) ^ 1];
    static_for<CHUNKS>([&](auto CH) {
      constexpr int ch = CH;
      constexpr int slot = ch & 1;
      constexpr bool last = ch + 1 == CHUNKS;
      const T *nb = last ? next : base;   // buffer of the next chunk
      constexpr int nch = last ? 0 : ch + 1;
      static_for<TM>([&](auto A) {
        constexpr int a = A;
#pragma unroll
        for (int b = 0; b < TN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ar[a % RING], wf[slot][b], acc[a][b],
                                                              0, 0, 0);
        // refill the ring slot just used; the next chunk's W fragments
        if constexpr (a + RING < TM) ar[a % RING] = afrag(base, ch, a + RING);
        else ar[a % RING] = afrag(nb, nch, a + RING - TM);
        constexpr int NWR = a >= RING ? WPER : 0;
#pragma unroll
        for (int j = 0; j < NWR; ++j)
          wf[slot ^ 1][(a - RING) * WPER + j] = wfrag(nb, nch, (a - RING) * WPER + j);
        if constexpr (ch == 0) {
#pragma unroll
          for (int j = 0; j < SPER; ++j) {
            sstore_piece(a * SPER + j, next);
            gload_piece(a * SPER + j, kt + 2);
          }
        }
        // MFMAs with the ring read, the W reads and the staging stores +
        // loads between them, in that order
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        static_for<NWR>([&](auto) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        });
        constexpr int NST = ch == 0 ? SPER : 0;
        static_for<NST>([&](auto) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        });
        constexpr int REST = TN - 1 - NWR - NST;
        if constexpr (REST > 0) __builtin_amdgcn_sched_group_barrier(0x008, REST, 0);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (last && a == RING - 1) __syncthreads();
      });
    });
  }

  __syncthreads();
  GemmEpilogue<T, BM, BN, EPI, NWN, NW, false, 16>(p, m0, n0, bias_g, g)
      .store(acc, reinterpret_cast<float *>(&lds[0][0]));
}

// ---------------------------------------------------------------------------
// Direct-to-LDS main loop with an NS-stage ring (bf16, BM x BN up to 128).
// Stage layout: BM rows of A then BN rows of W, 128 bytes (64 k) each; the
// 16-byte chunk c of row r is stored at chunk c ^ ((r >> 1) & 7), which makes
// the fragment reads of 16 consecutive rows conflict-free while every wave
// load instruction still writes one contiguous 1 KB block (8 rows).
// ---------------------------------------------------------------------------
template <int BM, int BN, int NS, int EPI>
__global__ __launch_bounds__(256) void gemm_dl_kernel(GemmArgs p) {
  typedef bf16x8 F;
  constexpr int BK = 64, ROWB = 128;
  constexpr int STAGE = (BM + BN) * ROWB;        // bytes per stage
  constexpr int IPS = (BM + BN) / 32;            // load instructions per wave per stage
  constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
  static_assert((NS - 2) * IPS < 64, "vmcnt range");
  constexpr bool PRE = TM * TN == 1;  // epilogue operands before the main loop (64x64)
  __shared__ __attribute__((aligned(1024))) char lds[NS * STAGE];
  static_assert(4 * gemm_strip_floats<bf16, WN>() * 4 <= NS * STAGE, "epilogue strips");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, half = lane >> 5;
  const int M = p.M, N = p.N, K = p.K;
  // XCD-aware tile order: even when the whole grid is resident at once, each
  // XCD's L2 then holds only the A and W panels of its own block of tiles
  int tm, tn;
  gemm_tile_of((N + BN - 1) / BN, (M + BM - 1) / BM, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const i32x4 ars = buffer_words(p.A, (uint32_t)((int64_t)M * p.lda * 2));
  const void *Wg, *bias_g;
  int g;
  gemm_group(p, Wg, bias_g, g);
  const i32x4 wrs = buffer_words(Wg, (uint32_t)((int64_t)N * p.ldw * 2));

  // Load instruction j of this wave fills stage rows j*32 + wave*8 .. +7; lane
  // i moves physical chunk i & 7 of row j*32 + wave*8 + (i >> 3).
  const int prow = wave * 8 + (lane >> 3);           // row within each 32-row group
  const int logical = (lane & 7) ^ ((prow >> 1) & 7); // logical 16-byte chunk it carries
  uint32_t src[IPS];
#pragma unroll
  for (int j = 0; j < IPS; ++j) {
    const int row = j * 32 + prow;
    src[j] = row < BM ? (uint32_t)(((int64_t)(m0 + row) * p.lda + logical * 8) * 2)
                      : (uint32_t)(((int64_t)(n0 + row - BM) * p.ldw + logical * 8) * 2);
  }
  auto issue = [&](int kt, int stage) {
    const int k0 = kt * BK;
    const bool kin = k0 + logical * 8 < K;
    const uint32_t sb = (uint32_t)(uintptr_t)lds + stage * STAGE + wave * 1024;
#pragma unroll
    for (int j = 0; j < IPS; ++j)
      dma_to_lds16(j * 32 < BM ? ars : wrs, sb + j * 4096, kin ? src[j] + k0 * 2 : OOB);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

  const int swz = (l32 >> 1) & 7;
  const int arow = (wm * WM + l32) * ROWB, wrow = (BM + wn * WN + l32) * ROWB;
  // Fragments of a whole slice (4 k-chunks), double-buffered in registers:
  // the next slice's fragments are read while this slice's MFMAs run, so the
  // LDS latency is paid once per slice, under the products.
  F af[2][4][TM], wf[2][4][TN];
  auto lload = [&](int stage, int buf) {
    const char *sb = lds + stage * STAGE;
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      const int off = ((ch * 2 + half) ^ swz) * 16;
#pragma unroll
      for (int a = 0; a < TM; ++a)
        af[buf][ch][a] = *reinterpret_cast<const F *>(sb + arow + a * 32 * ROWB + off);
#pragma unroll
      for (int b = 0; b < TN; ++b)
        wf[buf][ch][b] = *reinterpret_cast<const F *>(sb + wrow + b * 32 * ROWB + off);
    }
  };
  // With a single 32x32 tile per wave (64x64), odd k-chunks accumulate into a
  // second set so consecutive MFMAs do not wait on each other's result.
  constexpr bool DUAL = TM * TN == 1;
  f32x16 acc2[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc2[a][b][e] = 0.0f;
  auto mfmas = [&](int buf) {
#pragma unroll
    for (int ch = 0; ch < 4; ++ch)
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b) {
          if (DUAL && (ch & 1))
            mma32(af[buf][ch][a], wf[buf][ch][b], acc2[a][b]);
          else
            mma32(af[buf][ch][a], wf[buf][ch][b], acc[a][b]);
        }
  };

  // Slices 0 .. NS-2 in flight; slice kt+1's fragments are read during step kt.
  const int KT = (K + BK - 1) / BK;
  // The epilogue's operands go out right after slice 0: vector memory
  // operations complete in issue order, so the count below covers both.
  issue(0, 0);
  GemmEpilogue<bf16, BM, BN, EPI, 2, 4, PRE> epi(p, m0, n0, bias_g, g);
  if constexpr (PRE) epi.prefetch();
#pragma unroll
  for (int s = 1; s < NS - 1; ++s) issue(s, s);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * IPS));  // slice 0 landed (this wave)
  __syncthreads();
  lload(0, 0);
  // One step: slice kt+1 landed for every wave, slice kt+NS-1 into the stage
  // of slice kt-1 (its fragments were read during step kt-2), fragments of
  // slice kt+1 into register buffer nb, MFMAs of slice kt from buffer cb.
  auto step = [&](int kt, int nstage, int fstage, int cb, int nb) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 3) * IPS));
    __syncthreads();
    issue(kt + NS - 1, fstage);
    lload(nstage, nb);
    mfmas(cb);
    constexpr int NRD = 4 * (TM + TN), NMF = 4 * TM * TN;
    constexpr int RPM = NRD / NMF > 0 ? NRD / NMF : 1;
    static_for<NMF>([&](auto) {
      __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);  // DS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
    });
  };
  // stage of slice s is s % NS; tracked incrementally
  int st1 = 1 % NS;            // stage of slice kt+1
  int stf = NS - 1;            // stage of slice kt+NS-1
  int kt = 0;
  for (; kt + 1 < KT; kt += 2) {
    step(kt, st1, stf, 0, 1);
    st1 = st1 + 1 == NS ? 0 : st1 + 1;
    stf = stf + 1 == NS ? 0 : stf + 1;
    step(kt + 1, st1, stf, 1, 0);
    st1 = st1 + 1 == NS ? 0 : st1 + 1;
    stf = stf + 1 == NS ? 0 : stf + 1;
  }
  if (kt < KT) mfmas(0);
  if constexpr (DUAL) {
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b) acc[a][b] += acc2[a][b];
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no load may still be landing in LDS
  __syncthreads();
  epi.store(acc, reinterpret_cast<float *>(lds));
}

template <typename T, int BM, int BN, int NWN = 2, int NW = 4>
static hipError_t launch_t(Epilogue epi, const GemmArgs &a, hipStream_t s) {
  dim3 grid(((a.N + BN - 1) / BN) * ((a.M + BM - 1) / BM), a.gw ? a.groups : 1);
  constexpr int NT = 64 * NW;
  switch (epi) {
    case EPI_STORE: dit_launch(gemm_kernel<T, BM, BN, EPI_STORE, NWN, NW>, grid, NT, s, a); break;
    case EPI_GELU: dit_launch(gemm_kernel<T, BM, BN, EPI_GELU, NWN, NW>, grid, NT, s, a); break;
    case EPI_RESIDUAL: dit_launch(gemm_kernel<T, BM, BN, EPI_RESIDUAL, NWN, NW>, grid, NT, s, a); break;
    case EPI_STORE_F32: dit_launch(gemm_kernel<T, BM, BN, EPI_STORE_F32, NWN, NW>, grid, NT, s, a); break;
    case EPI_SPLIT: dit_launch(gemm_kernel<T, BM, BN, EPI_SPLIT, NWN, NW>, grid, NT, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int NWN, int NW>
static hipError_t launch_16(Epilogue epi, const GemmArgs &a, hipStream_t s) {
  dim3 grid(((a.N + 255) / 256) * ((a.M + 255) / 256), a.gw ? a.groups : 1);
  constexpr int NT = 64 * NW;
  switch (epi) {
    case EPI_STORE: dit_launch(gemm16_kernel<EPI_STORE, NWN, NW>, grid, NT, s, a); break;
    case EPI_GELU: dit_launch(gemm16_kernel<EPI_GELU, NWN, NW>, grid, NT, s, a); break;
    case EPI_RESIDUAL: dit_launch(gemm16_kernel<EPI_RESIDUAL, NWN, NW>, grid, NT, s, a); break;
    case EPI_STORE_F32: dit_launch(gemm16_kernel<EPI_STORE_F32, NWN, NW>, grid, NT, s, a); break;
    case EPI_SPLIT: dit_launch(gemm16_kernel<EPI_SPLIT, NWN, NW>, grid, NT, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int BM, int BN, int NS>
static hipError_t launch_dl(Epilogue epi, const GemmArgs &a, hipStream_t s) {
  dim3 grid(((a.N + BN - 1) / BN) * ((a.M + BM - 1) / BM), a.gw ? a.groups : 1);
  switch (epi) {
    case EPI_STORE: dit_launch(gemm_dl_kernel<BM, BN, NS, EPI_STORE>, grid, 256, s, a); break;
    case EPI_GELU: dit_launch(gemm_dl_kernel<BM, BN, NS, EPI_GELU>, grid, 256, s, a); break;
    case EPI_RESIDUAL: dit_launch(gemm_dl_kernel<BM, BN, NS, EPI_RESIDUAL>, grid, 256, s, a); break;
    case EPI_STORE_F32: dit_launch(gemm_dl_kernel<BM, BN, NS, EPI_STORE_F32>, grid, 256, s, a); break;
    case EPI_SPLIT: dit_launch(gemm_dl_kernel<BM, BN, NS, EPI_SPLIT>, grid, 256, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool gemm_offsets_fit(DType dt, int64_t M, int64_t lda, int64_t N, int64_t ldw) {
  // 32-bit byte offsets, including the rows of the last (partial) tile
  const int64_t es = dt == DT_BF16 ? 2 : 4, lim = (int64_t)1 << 31;
  return (M + 256) * lda * es < lim && (N + 256) * ldw * es < lim;
}

// Tile choice (measured on MI355X): 256x256 with 8 waves (two per SIMD, 3-15%
// faster than 4 waves on every large step shape) on 16x16x32 MFMAs (0-3 %
// faster than the same tile on 32x32x16 on the large step shapes, never
// slower beyond noise) once the grid has at least half a tile per CU; else
// 64x64.  Below that size 64x64 beat 128x128
// everywhere it was timed: MLP-1 at 1024 tokens (768 tiles, 11.0 against
// 12.0 us), and, once the 64x64 epilogue read its operands ahead, the grouped
// cross K/V projection at 1024 tokens (1152 tiles) and the guided step's QKV
// and MLP-1 at 2048 rows (1152 and 1536 tiles): the guided 1024-token step
// went from 1.818 to 1.738 ms.  128x128 remains for explicit requests.
static int pick_tile(int M, int N, int groups) {
  const int64_t G = groups > 1 ? groups : 1;
  const int64_t t256 = G * ((M + 255) / 256) * ((N + 255) / 256);
  return t256 >= 128 ? 5 : 3;
}

hipError_t launch_gemm(DType dt, Epilogue epi, const GemmArgs &a, hipStream_t s, int tile) {
  if (a.M <= 0 || a.N <= 0 || a.K <= 0) return hipSuccess;
  // weights come from W, or (grouped) from the tables, which then need >= 1 group
  if (a.gw ? (!a.gbias || a.groups < 1) : (a.W == nullptr || a.groups > 1)) return hipErrorInvalidValue;
  if (!gemm_offsets_fit(dt, a.M, a.lda, a.N, a.ldw)) return hipErrorInvalidValue;
  if (dt == DT_BF16) {
    if (tile == 0) tile = pick_tile(a.M, a.N, a.groups);
    // a split store needs every wave's column strip inside one segment: 128
    // columns for tile 1, 64 for tiles 2 and 4, 32 for tile 3
    if (epi == EPI_SPLIT && tile == 1 && a.seg_width % 128 != 0) tile = 4;
    if (epi == EPI_SPLIT && tile != 3 && a.seg_width % 64 != 0) tile = 3;
    if (epi == EPI_SPLIT && tile == 5 && a.seg_width % 64 != 0) tile = 3;
    switch (tile) {
      case 1: return launch_t<bf16, 256, 256>(epi, a, s);
      case 4: return launch_t<bf16, 256, 256, 4, 8>(epi, a, s);
      case 5: return launch_16<4, 8>(epi, a, s);
      case 2: return launch_dl<128, 128, 4>(epi, a, s);
      default: {
        // 5 stages (80 KB of LDS, two workgroups per CU) unless the grid has
        // 513 .. 768 tiles: then 3 stages (48 KB, three per CU) run it in one
        // wave of workgroups instead of two (the QKV projection at 1024 tokens)
        const int64_t t64 = (int64_t)(a.gw ? a.groups : 1) * ((a.M + 63) / 64) * ((a.N + 63) / 64);
        if (t64 > 512 && t64 <= 768) return launch_dl<64, 64, 3>(epi, a, s);
        return launch_dl<64, 64, 5>(epi, a, s);
      }
    }
  }
  return launch_t<float, 64, 64>(epi, a, s);
}

}  // namespace dit
