// dg_fp8_codec.h -- device arithmetic of the FP8 (e4m3) quantisers, shared
// by the stand-alone quantisers (dg_quant.hip) and the GEMM epilogue that
// applies SwiGLU and re-quantises (dg_kernels.hip), so that both produce the
// same codes and scales bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {
namespace codec {

constexpr float kE4m3Max = 448.0f;  // largest finite e4m3fn value

// s = amax / 448, 1 for an all-zero group
__device__ __forceinline__ float scale_of(float amax) { return amax == 0.0f ? 1.0f : amax / kE4m3Max; }

// Four values (already within +-448) -> four e4m3fn codes, round to nearest
// even (v_cvt_pk_fp8_f32; gfx950's FP8 conversion uses the OCP E4M3FN encoding).
__device__ __forceinline__ uint32_t encode4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// silu(g) = g / (1 + e^-g) for a bf16 gate g.  e^-g = 2^(-g log2 e) with
// log2 e split into a 15-bit head, whose product with g (8 significant bits)
// is exact in fp32, and a tail t = log2 e - head applied as the factor
// 2^(-g t) ~= 1 - g t ln 2 (|g t ln 2| < 4.4e-4 wherever e is finite, so the
// dropped second-order term is under 2 ulp).  The exp unit then sees an exact
// argument, and h stays within a few fp32 ulp of exact for every gate instead
// of losing |g| * 2^-24 to the rounding of g * log2 e.  Large negative g gives
// e = inf and silu = -0; large positive g gives e = 0 and silu = g.
__device__ __forceinline__ float silu(float g) {
  constexpr float kLog2eHead = 1.44268798828125f;     // 15 significant bits
  constexpr float kTailLn2 = -4.888495368504664e-06f;  // -(log2 e - head) * ln 2
  const float e = __builtin_amdgcn_exp2f(g * -kLog2eHead) * __builtin_fmaf(g, kTailLn2, 1.0f);
  return g * __builtin_amdgcn_rcpf(1.0f + e);
}

// The SwiGLU group quotient: h carries the exp unit's error (a few fp32 ulp),
// so h / s is taken as h * RN(1/s) rather than the exact division of the
// plain quantiser.  A scale below 2^-60 is raised by 2^64 (h alike, exactly)
// so that 1/s stays finite.  Returns the factor k and r = RN(1 / (s k)); the
// value fed to the encoder is clamp(h * k * r, -448, 448).
struct GroupRecip {
  float k, r;
};
__device__ __forceinline__ GroupRecip group_recip(float s) {
  const float k = s < 0x1p-60f ? 0x1p64f : 1.0f;
  return GroupRecip{k, 1.0f / (s * k)};
}
__device__ __forceinline__ float scaled(float h, const GroupRecip& g) {
  return fminf(fmaxf(h * g.k * g.r, -kE4m3Max), kE4m3Max);
}

}  // namespace codec
}  // namespace dg
