// Shared device helpers for the gfx950 MoE-LoRA kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

#define MOE_DEV __device__ __forceinline__

MOE_DEV float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 round-to-nearest-even (a NaN stays a NaN): gfx950's v_cvt_pk_bf16_f32,
// one instruction for two values where the software rounding took five per value.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
MOE_DEV uint32_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

MOE_DEV uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// SwiGLU of one (gate, up) pair: silu(g) * u with silu(g) = g / (1 + e^-g).  Uses the
// hardware exp2 and reciprocal (a few ulp in fp32, far below the bf16 rounding that
// follows); e^-g -> inf for very negative g gives g * 0 = -0, the limit of silu.
MOE_DEV float silu_mul(float g, float u) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u; }

// 16x16x32 bf16 MFMA: A lane l = row l%16, B lane l = column l%16, both holding the
// same 8 consecutive K values (group l/16); D lane l holds rows 4*(l/16)+i, column l%16.
MOE_DEV f32x4_t mfma_16x16x32(const u32x4_t &a, const u32x4_t &b, const f32x4_t &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

MOE_DEV int lane_id() { return __lane_id(); }

MOE_DEV u32x4_t zero_u32x4() {
  u32x4_t z = {0u, 0u, 0u, 0u};
  return z;
}

// Status codes mirrored from include/moe_lora.h for host code.
enum {
  ST_OK = 0,
  ST_INVALID = 1,
  ST_UNSUPPORTED = 2,
  ST_WS_SMALL = 3,
  ST_HIP = 4
};
