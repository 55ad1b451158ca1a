// nvfp4_device.hpp -- gfx950 device helpers: NVFP4 decode, bf16 packing, MFMA
// operand types.  Included by the HIP kernels only.
//
// NVFP4 (as used by the gllm PR "perf: gather tokens per MoE expert, run large
// NVFP4 GEMMs on bf16 tensor cores #91", section "bf16 NVFP4 GEMM (CUDA)"):
// 4-bit e2m1 codes, one e4m3 scale per 16 consecutive elements of a row, one
// fp32 global per tensor.  A code (2 significant bits) times a scale (4) is
// representable in bf16 (8), so the unpack is exact; the global is applied
// once, after the dot product.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;

// ---------------------------------------------------------------------------
// e4m3 (OCP E4M3FN) -> f32.  Exponent bias 7; e == 0 is subnormal (m * 2^-9);
// S.1111.111 is NaN; there is no infinity.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  uint32_t s = (b & 0x80u) << 24;
  uint32_t em = b & 0x7Fu;
  if (em == 0x7Fu) return __uint_as_float(0x7FC00000u | s);
  uint32_t e = em >> 3, m = em & 7u;
  float mag;
  if (e == 0)
    mag = (float)m * 0.001953125f;  // m * 2^-9, exact
  else
    mag = __uint_as_float(((e + 120u) << 23) | (m << 20));  // rebias 7 -> 127
  return __uint_as_float(__float_as_uint(mag) | s);
}

// The two e4m3 block scales of one 32-element group (low byte = first block),
// decoded with the OCP FP8 converter (unit scale: exact).
__device__ __forceinline__ void e4m3x2_to_f32(uint32_t two, float &s0, float &s1) {
  s0 = __builtin_amdgcn_cvt_scalef32_f32_fp8(two, 1.0f, 0);
  s1 = __builtin_amdgcn_cvt_scalef32_f32_fp8(two, 1.0f, 1);
}

// Decode 8 codes (one 32-bit word, element 0 in the low nibble of byte 0) into
// 8 bf16 values scale * e2m1, packed as 4 x (even element in the low half).
// The FP4 converter (unit scale) gives exact e2m1 values; every product with
// the e4m3 scale is exact in f32 and in bf16 (2 + 4 significant bits, inside
// the normal range), so the upper 16 bits of the f32 are the exact bf16.
__device__ __forceinline__ u32x4_t dq8_bf16(uint32_t w, float scale) {
  u32x4_t r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f32x2_t v;
    switch (j) {  // the byte selector must be an immediate
      case 0: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0); break;
      case 1: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1); break;
      case 2: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2); break;
      default: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3); break;
    }
    const uint32_t lo = __float_as_uint(v.x * scale);
    const uint32_t hi = __float_as_uint(v.y * scale);
    r[j] = __builtin_amdgcn_perm(hi, lo, 0x07060302u);  // {hi[31:16], lo[31:16]}
  }
  return r;
}

// Portable decode of one e2m1 code without the FP4 converter (used to check
// the converter's lane order in the unpack tests and as its fallback).  The
// three magnitude bits go into an fp16 bit pattern (exponent bits 11:10,
// mantissa bit 9), which encodes e2m1(c) * 2^-14 exactly (e == 0 lands on the
// fp16 subnormals, which the f16 -> f32 conversion keeps).
__device__ __forceinline__ float e2m1_to_f32_alu(uint32_t c) {
  uint32_t h = ((c & 7u) << 9) | ((c & 8u) << 12);
  _Float16 hv = __builtin_bit_cast(_Float16, (uint16_t)h);
  return (float)hv * 16384.0f;
}

__device__ __forceinline__ u32x4_t dq8_bf16_alu(uint32_t w, float scale) {
  u32x4_t r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t b = (w >> (8 * j)) & 0xFFu;
    uint32_t lo = __float_as_uint(e2m1_to_f32_alu(b & 15u) * scale);
    uint32_t hi = __float_as_uint(e2m1_to_f32_alu(b >> 4) * scale);
    r[j] = (lo >> 16) | (hi & 0xFFFF0000u);
  }
  return r;
}

// ---------------------------------------------------------------------------
// bf16 helpers
// ---------------------------------------------------------------------------

// f32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Split an f32 into three bf16 terms hi + mid + lo (each the RNE bf16 of the
// remaining residual).  hi + mid + lo carries 24 significant bits, i.e. the f32
// value to within one unit in its last place for normal values; each residual
// is exact in f32.
__device__ __forceinline__ void split3_bf16(float v, uint32_t &hi, uint32_t &mid, uint32_t &lo) {
  hi = f32_to_bf16_rne(v);
  float r1 = v - bf16_to_f32(hi);
  mid = f32_to_bf16_rne(r1);
  float r2 = r1 - bf16_to_f32(mid);
  lo = f32_to_bf16_rne(r2);
}

__device__ __forceinline__ uint32_t pack_bf16x2(uint32_t lo, uint32_t hi) { return lo | (hi << 16); }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// D(16x16, f32) += A(16x32, bf16) * B(32x16, bf16).  Lane l supplies row l%16 of
// A and column l%16 of B, each with the 8 k-values of slice l/16; it receives
// D[4*(l/16) + i][l%16], i = 0..3.
__device__ __forceinline__ f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

}  // namespace moe
