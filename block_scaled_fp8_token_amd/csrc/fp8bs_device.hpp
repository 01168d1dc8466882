// Device helpers shared by the gfx950 kernels of the block-scaled FP8 library.
//
// Number formats (readings of the vLLM DeepGEMM FP8 block GEMM benchmark post,
// section 4.1, and of vLLM PR #29546 "Deepgemm fused layout kernel for
// activations"):
//   * activations/weights: OCP e4m3 (E4M3FN, max 448), round to nearest even,
//     saturating at +-448, sign of zero kept;
//   * scales: UE8M0, i.e. a power of two 2^e stored as the byte e + 127, where
//     2^e is amax/448 rounded UP to a power of two and amax is floored at 1e-10;
//   * packed activation scales: the bytes of groups 4w..4w+3 of a row in one
//     32-bit word w, little-endian.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bs {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Exponent e of the UE8M0 scale of a group whose largest magnitude is amax (a
// non-negative fp32): the smallest integer with 448 * 2^e >= max(amax, 1e-10).
// With amax = f * 2^E, f in [1, 2), and 448 = 1.75 * 2^8 this is E - 8 when
// f <= 1.75 (mantissa field <= 0x600000) and E - 7 otherwise.  Every amax at or
// below 448 * 2^-42 (zero and fp32 subnormals included) gives -42, which is the
// exponent of the 1e-10 floor, so the floor is a clamp at -42.
__device__ __forceinline__ int ue8m0_exponent(float amax) {
  uint32_t bits = __float_as_uint(amax);
  int biased = (int)(bits >> 23);
  int e = biased - 127 - 8 + (((bits & 0x7FFFFFu) > 0x600000u) ? 1 : 0);
  if (biased == 0) e = -42;
  return e < -42 ? -42 : e;
}

// 2^k as fp32 for k in [-126, 127].
__device__ __forceinline__ float exp2i(int k) { return __uint_as_float((uint32_t)(k + 127) << 23); }

// Two fp32 values -> two e4m3 bytes (RNE) in the low 16 bits of the result.  The
// hardware conversion returns NaN above the e4m3 range instead of saturating, so
// the inputs are clamped to +-448 first (the clamp keeps the sign of zero).
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
  a = __builtin_fminf(__builtin_fmaxf(a, -448.0f), 448.0f);
  b = __builtin_fminf(__builtin_fmaxf(b, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// Eight fp32 values (already multiplied by 2^-e) -> eight e4m3 bytes.
__device__ __forceinline__ uint2 e4m3x8(const float* v) {
  uint2 r;
  r.x = e4m3x2(v[0], v[1]) | (e4m3x2(v[2], v[3]) << 16);
  r.y = e4m3x2(v[4], v[5]) | (e4m3x2(v[6], v[7]) << 16);
  return r;
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Max over the 16 lanes of each 16-lane row of the wavefront.
__device__ __forceinline__ float max16(float v) {
  v = __builtin_fmaxf(v, __shfl_xor(v, 1));
  v = __builtin_fmaxf(v, __shfl_xor(v, 2));
  v = __builtin_fmaxf(v, __shfl_xor(v, 4));
  v = __builtin_fmaxf(v, __shfl_xor(v, 8));
  return v;
}

}  // namespace fp8bs
