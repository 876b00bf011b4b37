// Device helpers shared by the layer kernels (gfx950 / CDNA4).
//
// MXFP4 decode follows "MXFP4 MoE decode kernels", The bottleneck (E2M1 values
// two per byte, one E8M0 scale per 32 values) and "GLM-5.2 and GLM-5.3 (744B)
// in MXFP4 on Gaudi 2", What was built, Byte-exact repack (low nibble first).
// One 16-byte chunk of a packed row is exactly one 32-value MX block, so a
// lane that loads 16 bytes needs one scale byte.  gfx950's scaled FP4
// converts (v_cvt_scalef32_pk_{bf16,f32}_fp4) decode two nibbles of a chosen
// byte and apply the block scale in one instruction: low nibble -> element 0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kWave = 64;

// E8M0 byte -> fp32 2^(s-127), built from the IEEE exponent field;
// s = 0 is the subnormal 2^-127, s = 255 is NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  uint32_t bits = s << 23;
  bits = (s == 0u) ? 0x00400000u : bits;
  bits = (s == 255u) ? 0x7FC00000u : bits;
  return __uint_as_float(bits);
}

// Decode one 32-value MX block (16 packed bytes) to 16 bf16 pairs, scaled.
// Pair i holds elements 2i (low half) and 2i+1 (high half).
__device__ __forceinline__ void decode_block_bf16(const uint4 q, float scale, bf16x2 (&out)[16]) {
  out[0]  = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q.x, scale, 0);
  out[1]  = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q.x, scale, 1);
  out[2]  = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q.x, scale, 2);
  out[3]  = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q.x, scale, 3);
  out[4]  = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q.y, scale, 0);
  out[5]  = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q.y, scale, 1);
  out[6]  = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q.y, scale, 2);
  out[7]  = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q.y, scale, 3);
  out[8]  = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q.z, scale, 0);
  out[9]  = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q.z, scale, 1);
  out[10] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q.z, scale, 2);
  out[11] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q.z, scale, 3);
  out[12] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q.w, scale, 0);
  out[13] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q.w, scale, 1);
  out[14] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q.w, scale, 2);
  out[15] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q.w, scale, 3);
}

// Decode one packed dword (8 values) to fp32 pairs, scaled.
__device__ __forceinline__ void decode_dword_f32(uint32_t q, float scale, f32x2 (&out)[4]) {
  out[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, scale, 0);
  out[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, scale, 1);
  out[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, scale, 2);
  out[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, scale, 3);
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

// 2-way bf16 dot product accumulated in fp32.
__device__ __forceinline__ float dot2(bf16x2 a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, as_bf16x2(b), c, false);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Sum over each row of 16 lanes with DPP; every lane of the row gets the sum.
__device__ __forceinline__ float row16_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false)); // row_ror:4
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false)); // row_ror:8
  return v;
}

__device__ __forceinline__ float sigmoidf(float v) { return 1.0f / (1.0f + expf(-v)); }

// Activation of one [gate; up] pair ("MXFP4 MoE decode kernels", Design,
// Fused epilogues; Beyond gpt-oss).  act: 0 = SiLU(gate)*up,
// 1 = SwiGLU-OAI with gate capped at +limit and up clamped to +-limit.
__device__ __forceinline__ float activate(float g, float u, int act, float alpha, float limit) {
  if (act == 0) return g * (1.0f / (1.0f + expf(-g))) * u;
  float gc = fminf(g, limit);
  float uc = fminf(fmaxf(u, -limit), limit);
  return gc * (1.0f / (1.0f + expf(-(alpha * gc)))) * (uc + 1.0f);
}

}  // namespace moe
