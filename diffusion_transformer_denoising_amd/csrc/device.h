// device.h -- gfx950 device primitives shared by the DiT kernels: element
// types, bf16 conversion, and the 32x32 MFMA fragment contract.
//
// MFMA fragment contract (v_mfma_f32_32x32x16_bf16 and, eight at a time,
// v_mfma_f32_32x32x2_f32).  A "chunk" is 16 steps of the contracted index k.
// For C[32x32] += A[32x16] * B[16x32]:
//   A fragment: lane l holds row (l % 32), k = (l / 32) * 8 + e, e = 0..7;
//   B fragment: lane l holds column (l % 32), k = (l / 32) * 8 + e;
//   C:          lane l holds column (l % 32), rows j*8 + (l/32)*4 + i at
//               acc[j*4 + i], i, j = 0..3.
// With fp32 operands the chunk is eight 32x32x2 MFMAs; MFMA e takes element e
// of every lane, i.e. k = e from lanes 0..31 and k = 8 + e from lanes 32..63,
// so the fragment layout in registers is the same for both element types.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace dit {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

template <typename T> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 type; };
template <> struct Frag<float> { typedef f32x8 type; };

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

__device__ __forceinline__ void mma32(const bf16x8 &a, const bf16x8 &b, f32x16 &c) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma32(const f32x8 &a, const f32x8 &b, f32x16 &c) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], c, 0, 0, 0);
}

// 16-byte global/LDS vector moves.
struct alignas(16) U128 { uint32_t w[4]; };

// Raw buffer resource over `bytes` bytes: loads at offsets past the end
// return zero, so ragged edges and absent operands (an empty range) need no
// branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ U128 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(U128, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

constexpr uint32_t OOB = 0x80000000u;  // an offset past every operand (sizes < 2^31 bytes)

typedef int i32x4 __attribute__((ext_vector_type(4)));

// s_waitcnt immediate for "at most n vector-memory operations outstanding"
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt left open).
constexpr int vmcnt_imm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | 0x0F70; }

// Words of a raw buffer resource over `bytes` bytes at `base` (no stride;
// loads at offsets past the end return zero).
__device__ __forceinline__ i32x4 buffer_words(const void *base, uint32_t bytes) {
  // wave-uniform by construction; readfirstlane keeps the words in SGPRs
  const uint64_t b = (uint64_t)base;
  return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)b),
               __builtin_amdgcn_readfirstlane((int)((b >> 32) & 0xFFFF)),
               __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}

// 16 bytes per lane from a buffer straight into LDS: lane i of the wave
// writes lds_addr + 16 i (lds_addr is wave-uniform).  Issued as inline asm so
// that the compiler does not make every later LDS read wait for all such
// transfers in flight; callers order them with explicit vmcnt waits and
// barriers.
__device__ __forceinline__ void dma_to_lds16(i32x4 rsrc, uint32_t lds_addr, uint32_t voff) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voff), "s"(rsrc), "{m0}"(lds_addr) : "memory");
}

// Workgroups are handed to the chip's 8 XCDs round-robin by linear id (id % 8),
// and each XCD has its own L2.  This maps the linear id of a grid of n
// workgroups to a logical index so that every XCD gets one contiguous range
// of logical indices (the first n % 8 XCDs one more than the rest), walked in
// dispatch order.
__device__ __forceinline__ int xcd_contiguous(int id, int n) {
  const int xcd = id & 7, local = id >> 3, per = n >> 3, rem = n & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// GELU, tanh form: z/2 (1 + tanh(u)) with u = sqrt(2/pi) (z + 0.044715 z^3),
// evaluated as z / (1 + exp(-2u)) with the hardware reciprocal (1 ulp; the
// IEEE division sequence costs several times as much in the GEMM epilogue).
// Limits stay exact: exp(-2u) = inf gives -0, exp(-2u) = 0 gives z.
__device__ __forceinline__ float gelu_tanh(float z) {
  const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
  float u = k0 * (z + 0.044715f * z * z * z);
  float e = fast_exp2(-2.0f * 1.4426950408889634f * u);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + fast_exp2(-1.4426950408889634f * z)); }

// Sum over the 64 lanes of a wave, in every lane.  Butterflies inside each row
// of 16 lanes use DPP lane moves (no LDS round trip): xor 1, xor 2, then the
// half-row and row mirrors, which pair equal-valued groups of 4 and 8; the four
// row sums are then read out as scalars.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                              0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  v += dpp_mov<0x141>(v);  // row_half_mirror: quads 0 <-> 1 of each 8
  v += dpp_mov<0x140>(v);  // row_mirror: halves 0 <-> 1 of each 16
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Compile-time loop: f(std::integral_constant<int, 0>{}) ... f(<N-1>).
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  [&]<int... I>(std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
  }(std::make_integer_sequence<int, N>{});
}

}  // namespace dit
