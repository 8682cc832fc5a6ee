// Device helpers shared by the gfx950 kernels of libmoe.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr float kE4M3Max = 448.0f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even FP32 -> BF16 for finite values.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Two FP32 values to two E4M3 codes (low byte = a).  The hardware conversion
// rounds to nearest even and keeps subnormals; clamping first makes magnitudes
// above 448 saturate instead of becoming NaN.
__device__ __forceinline__ uint32_t f32x2_to_e4m3(float a, float b) {
  a = fminf(fmaxf(a, -kE4M3Max), kE4M3Max);
  b = fminf(fmaxf(b, -kE4M3Max), kE4M3Max);
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// Four FP32 values to four packed E4M3 codes (byte i = v_i).
__device__ __forceinline__ uint32_t f32x4_to_e4m3(float v0, float v1, float v2, float v3) {
  v0 = fminf(fmaxf(v0, -kE4M3Max), kE4M3Max);
  v1 = fminf(fmaxf(v1, -kE4M3Max), kE4M3Max);
  v2 = fminf(fmaxf(v2, -kE4M3Max), kE4M3Max);
  v3 = fminf(fmaxf(v3, -kE4M3Max), kE4M3Max);
  uint32_t r = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, r, true);
}

// Scale of a tile from its max-abs value: amax/448 (correctly rounded FP32
// division), 1.0 for an all-zero tile.
__device__ __forceinline__ float scale_from_amax(float amax) {
  return amax == 0.0f ? 1.0f : amax / kE4M3Max;
}

// Power-of-two scale: the smallest power of two not below fl32(amax/448), at
// least 2^-127 (the smallest E8M0 value, an FP32 subnormal); 1.0 for an
// all-zero tile.  Its FP32 exponent field is the E8M0 code of the scale.
__device__ __forceinline__ float scale_from_amax_pow2(float amax) {
  if (amax == 0.0f) return 1.0f;
  const uint32_t b = __float_as_uint(amax / kE4M3Max);
  if (b <= 0x00400000u) return __uint_as_float(0x00400000u);   // at most 2^-127
  if (b < 0x00800000u) return __uint_as_float(0x00800000u);    // other subnormals: 2^-126
  return (b & 0x007FFFFFu) ? __uint_as_float((b & 0x7F800000u) + 0x00800000u) : __uint_as_float(b);
}

// h = SiLU(g) * u with SiLU(g) = g / (1 + e^-g) in FP32: exp within an ulp,
// then correctly rounded addition, division and product, so h is within
// 2.5 ulp of the exactly rounded value (no hardware reciprocal estimate).
__device__ __forceinline__ float swiglu_f32(float g, float u) {
  return g / (1.0f + expf(-g)) * u;
}

// x / s for many x with one s, correctly rounded: r = 1/s is computed once by
// IEEE division (correctly rounded).  Per x, q0 = x r is within 1.5 ulp of x/s;
// one correction q1 = q0 + r (x - s q0) brings it within an ulp, so the next
// remainder x - s q1 is exact by FMA and q1 + r (x - s q1) rounds to the
// correctly rounded quotient (Markstein's theorem on division with a correctly
// rounded reciprocal; no overflow or underflow here).  An exact zero keeps its
// sign.
struct Divider {
  float s, r;
  __device__ __forceinline__ explicit Divider(float s_) : s(s_), r(1.0f / s_) {}
  __device__ __forceinline__ float operator()(float x) const {
    const float q0 = x * r;
    const float q1 = fmaf(fmaf(-s, q0, x), r, q0);
    return x == 0.0f ? q0 : fmaf(fmaf(-s, q1, x), r, q1);
  }
};

template <bool POW2>
__device__ __forceinline__ float tile_scale(float amax) {
  return POW2 ? scale_from_amax_pow2(amax) : scale_from_amax(amax);
}

// One 16x16x128 FP8 E4M3 MFMA: D = A * B^T + C.  Lane l supplies row l%16 of A
// (and row l%16 of B, i.e. column l%16 of the product) with the 32 K-values
// [(l/16)*32, (l/16)*32 + 32); D holds rows (l/16)*4 + i, column l%16.  The
// E8M0 block scales are fixed at 2^0 (code 127).
__device__ __forceinline__ v4f mfma_fp8_16x16x128(v8i a, v8i b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// The same MFMA with hardware block scales: D = (2^(ea-127) A) * (2^(eb-127) B)^T
// + C, where byte 0 of `ea` is the E8M0 code of the scale of the row (of A)
// that the lane supplies and byte 0 of `eb` that of the lane's B row (column
// of the product); each lane's code covers its own 32 K-values.
__device__ __forceinline__ v4f mfma_fp8_16x16x128_scaled(v8i a, v8i b, v4f c, int ea, int eb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, ea, 0, eb);
}

// 16x16x32 BF16 MFMA with the same row/column conventions; lane l holds the 8
// K-values [(l/16)*8, (l/16)*8 + 8).
__device__ __forceinline__ v4f mfma_bf16_16x16x32(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

// Direct global->LDS loads.  Lane l of the wave writes its 16 (or 4) bytes at
// LDS byte address lds + 16 l (4 l); the source address is per lane.  They are
// issued from inline assembly so that the compiler does not track them: it
// would otherwise make every later LDS read wait for all of them, which would
// drain the pipeline each K step.  The instructions have no register outputs
// (the data goes to LDS); every LDS read of their data follows an explicit
// vmcnt wait and a barrier, and every reuse of a ring slot follows a barrier.
// M0 carries the LDS address; the compiler does not allocate it.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}
// base: wave-uniform global address; off: per-lane byte offset (32 bits).
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(off), "s"(uniform_ptr(base)), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :: "v"(off), "s"(uniform_ptr(base)), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Wait for all of this wave's LDS reads and direct loads, then barrier.  The
// barrier is written in assembly with a memory clobber so that the compiler
// moves no LDS access across it.  (gfx9 s_waitcnt fields: vmcnt[3:0] bits 3:0,
// expcnt 6:4, lgkmcnt 11:8, vmcnt[5:4] bits 15:14.)
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0), expcnt unconstrained
  asm volatile("s_barrier" ::: "memory");
}

// LDS layout of 128-byte operand rows: 16-byte chunk c of row r sits at chunk
// position c ^ op_swz(r).  The pattern was chosen by measurement on gfx950: for
// the MFMA fragment reads (ds_read_b128, lanes 0..15 on rows r0..r0+15 at one
// chunk, lanes 16..63 on the next chunks) it runs at 92% of the rate of
// linear reads, where the XOR with (r >> 1) & 7 runs at 63%.
__device__ __forceinline__ int op_swz(int r) { return ((r & 3) << 1) ^ ((r >> 2) & 1); }

}  // namespace moe
