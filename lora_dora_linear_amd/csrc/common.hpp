// Shared device-side building blocks for the gfx950 (CDNA4) kernels.
//
// Everything here is plain HIP for a 64-lane wavefront.  The MFMA fragment
// conventions used by every kernel in the library:
//
//   v_mfma_f32_16x16x32_bf16 (and v_mfma_i32_16x16x64_i8):
//     operand P (lane l) holds row (l & 15) of a 16-row block and the 16-byte
//     reduction chunk (l >> 4) of a 32-element (bf16) / 64-element (int8) step;
//     operand Q likewise for the 16 columns.  The result lane l holds
//     D[4*(l >> 4) + i][l & 15], i = 0..3.
//   Both operands always use the same reduction-chunk assignment, so the
//   order of the reduction inside a chunk never matters.
//
//   Kernels pass the output-column operand first and the output-row operand
//   second, so that a lane's four results are four consecutive output columns
//   of one output row (one 8-byte bf16 store or one 16-byte fp32 store).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

namespace ldl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

// ------------------------------------------------------------------ bf16 helpers
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// fp32 -> bf16, round to nearest even, on the conversion unit (v_cvt_pk_bf16_f32: two
// values per instruction, where the integer form of the rounding took ~12); NaN stays NaN.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// The same rounding in integer arithmetic (finite inputs; NaN becomes the quiet NaN 0x7fc0),
// for kernels whose register allocation the conversion instruction upsets.
__device__ __forceinline__ uint32_t f32_to_bf16_bits_int(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2_int(float lo, float hi) {
  return f32_to_bf16_bits_int(lo) | (f32_to_bf16_bits_int(hi) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ i32x4 as_i32x4(u32x4 v) { return __builtin_bit_cast(i32x4, v); }

// ------------------------------------------------------------------ MFMA wrappers
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 p, u32x4 q, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(p), as_bf16x8(q), acc, 0, 0, 0);
}
__device__ __forceinline__ i32x4 mfma_i8(u32x4 p, u32x4 q, i32x4 acc) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(as_i32x4(p), as_i32x4(q), acc, 0, 0, 0);
}
// 32x32 blocks: operand lane l holds row (l & 31) and the 16-byte reduction
// chunk (l >> 5); result lane l holds D[8*(v >> 2) + 4*(l >> 5) + (v & 3)][l & 31]
// for v = 0..15.
__device__ __forceinline__ f32x16 mfma32_bf16(u32x4 p, u32x4 q, f32x16 acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(p), as_bf16x8(q), acc, 0, 0, 0);
}
__device__ __forceinline__ i32x16 mfma32_i8(u32x4 p, u32x4 q, i32x16 acc) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(as_i32x4(p), as_i32x4(q), acc, 0, 0, 0);
}

// ------------------------------------------------------------------ LDS swizzle
// Tiles in LDS are rows of 128 bytes (eight 16-byte chunks).  Chunk c of row
// `row` lives at chunk c ^ swz(row).  swz makes both access patterns the
// kernels use conflict free: eight consecutive rows at one chunk (MFMA
// fragment reads, row-major tile writes) and rows 8 apart at one chunk
// (transposed tile writes).
__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * 128 + ((chunk ^ swz(row)) << 4); }

// ------------------------------------------------------------------ 8x8 transpose of 16-bit values
// in[i] holds row i (8 values, 2 per dword); out[c] holds column c.
__device__ __forceinline__ void transpose8x8_b16(const u32x4 in[8], u32x4 out[8]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t a = in[2 * j][c];
      uint32_t b = in[2 * j + 1][c];
      out[2 * c][j] = (a & 0xffffu) | (b << 16);
      out[2 * c + 1][j] = (a >> 16) | (b & 0xffff0000u);
    }
  }
}

// int8 x8 (two dwords) -> bf16 x8 (four dwords), exact (|q| <= 128).
__device__ __forceinline__ u32x4 i8x8_to_bf16x8(u32x2 v) {
  u32x4 o;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t w = v[h];
    float f0 = float(int8_t(w & 0xff));
    float f1 = float(int8_t((w >> 8) & 0xff));
    float f2 = float(int8_t((w >> 16) & 0xff));
    float f3 = float(int8_t(w >> 24));
    o[2 * h] = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xffff0000u);
    o[2 * h + 1] = (__float_as_uint(f2) >> 16) | (__float_as_uint(f3) & 0xffff0000u);
  }
  return o;
}

// Scale 8 bf16 values by 8 per-element factors, round back to bf16.
__device__ __forceinline__ u32x4 scale_bf16x8(u32x4 v, f32x4 s0, f32x4 s1) {
  u32x4 o;
  o[0] = pack_bf16x2(bf16_lo(v[0]) * s0[0], bf16_hi(v[0]) * s0[1]);
  o[1] = pack_bf16x2(bf16_lo(v[1]) * s0[2], bf16_hi(v[1]) * s0[3]);
  o[2] = pack_bf16x2(bf16_lo(v[2]) * s1[0], bf16_hi(v[2]) * s1[1]);
  o[3] = pack_bf16x2(bf16_lo(v[3]) * s1[2], bf16_hi(v[3]) * s1[3]);
  return o;
}

// ------------------------------------------------------------------ LDS copies and reads
// Buffer resource over [base, base + bytes): reads past the end return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// Direct buffer -> LDS copy of 16 bytes per lane; lane l lands at lds_base + 16*l
// (lds_base wave-uniform, taken from M0).  Written as inline assembly so that
// the compiler does not treat the copy as an LDS store it must wait for before
// every later LDS read: the copies always target the stage that no wave is
// reading, and the kernel waits for them itself (vmcnt(0) + barrier) before
// that stage is read.
__device__ __forceinline__ void buf2lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint8_t* lds_base) {
  const uint32_t lds_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds_base;
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(r), "s"(soff), "{m0}"(lds_addr) : "memory");
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes the
// 16 eight-byte reads form a 16 x 4 matrix D (lane j's read is row j); lane
// 4a + b of the group receives D[a][b], D[a+4][b], D[a+8][b], D[a+12][b].
__device__ __forceinline__ u32x2 lds_tr16(const uint8_t* base, int off) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(base + off));
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// sigma(e) = 1 / (1 + exp(-e)) with the hardware reciprocal (1 ulp): the library is built
// with IEEE fp32 division for the int8 quantiser, which made every epilogue division a
// long instruction sequence; the activations only feed bf16 outputs.  exp(-e) = inf for
// very negative e gives rcp(inf) = 0.
__device__ __forceinline__ float sigmoid_f(float e) { return __builtin_amdgcn_rcpf(1.0f + __expf(-e)); }
__device__ __forceinline__ float silu_f(float e) { return e * sigmoid_f(e); }

// Gate activations of the gated MLPs (GemmParams::act): SiLU e.sigma(e) (SwiGLU); GELU
// e.Phi(e) with Phi the standard normal distribution function, 0.5 (1 + erf(e / sqrt 2))
// (GeGLU); and GELU in its tanh form 0.5 e (1 + tanh(sqrt(2/pi) (e + 0.044715 e^3))).
enum : int { ACT_SILU = 0, ACT_GELU = 1, ACT_GELU_TANH = 2 };
// erf by the rational approximation of Abramowitz and Stegun, Handbook of Mathematical
// Functions, formula 7.1.26 (absolute error below 1.5e-7, far below the bf16 outputs' rounding):
// erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2), t = 1 / (1 + p x) for x >= 0,
// odd in x.  One reciprocal and one exponential instead of the library erf's range reduction.
__device__ __forceinline__ float erf_as(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(1.f + 0.3275911f * ax);
  const float poly = t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
  return copysignf(1.f - poly * __expf(-ax * ax), x);
}
// tanh(y) = 1 - 2 / (exp(2 |y|) + 1), odd in y (absolute error ~1e-7; exp overflowing to inf
// gives 1)
__device__ __forceinline__ float tanh_e(float y) {
  return copysignf(1.f - 2.f * __builtin_amdgcn_rcpf(__expf(2.f * fabsf(y)) + 1.f), y);
}
__device__ __forceinline__ float glu_act(float e, int act) {
  if (act == ACT_GELU) return 0.5f * e * (1.f + erf_as(e * 0.70710678118654752f));
  if (act == ACT_GELU_TANH) return 0.5f * e * (1.f + tanh_e(0.79788456080286536f * (e + 0.044715f * e * e * e)));
  return silu_f(e);
}
// d act / d e:  SiLU sigma (1 + e (1 - sigma));  GELU Phi(e) + e phi(e), phi the normal density;
// tanh form 0.5 (1 + t) + 0.5 e (1 - t^2) sqrt(2/pi) (1 + 3 . 0.044715 e^2)
__device__ __forceinline__ float glu_act_grad(float e, int act) {
  if (act == ACT_GELU)
    return 0.5f * (1.f + erf_as(e * 0.70710678118654752f)) + e * 0.39894228040143268f * __expf(-0.5f * e * e);
  if (act == ACT_GELU_TANH) {
    const float t = tanh_e(0.79788456080286536f * (e + 0.044715f * e * e * e));
    return 0.5f * (1.f + t) + 0.5f * e * (1.f - t * t) * 0.79788456080286536f * (1.f + 0.134145f * e * e);
  }
  const float sg = sigmoid_f(e);
  return sg * (1.f + e * (1.f - sg));
}

}  // namespace ldl
