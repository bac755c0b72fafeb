// Small device helpers for the gfx950 kernels: bf16 bit handling, wave64
// lane reductions, base-2 exponent.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace duo {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// bf16 pair packed in a 32-bit word -> the two fp32 values (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32); NaN stays NaN.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Two bf16 products accumulated in fp32 (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP lane moves inside a 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of LANES (2, 4, 8 or 16) lanes; every lane of the
// group receives the group sum.
template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LANES == 2 || LANES == 4 || LANES == 8 || LANES == 16, "group size");
  x += dpp_mov<0xB1>(x);                              // quad_perm [1,0,3,2]: lane ^ 1
  if (LANES >= 4) x += dpp_mov<0x4E>(x);              // quad_perm [2,3,0,1]: lane ^ 2
  if (LANES >= 8) x += dpp_mov<0x141>(x);             // row_half_mirror: quads 0<->1
  if (LANES >= 16) x += dpp_mov<0x140>(x);            // row_mirror: halves of 16
  return x;
}

// Maximum over aligned groups of LANES (2, 4, 8 or 16) lanes; every lane of
// the group receives it.
template <int LANES>
__device__ __forceinline__ float group_max(float x) {
  static_assert(LANES == 2 || LANES == 4 || LANES == 8 || LANES == 16, "group size");
  x = fmaxf(x, dpp_mov<0xB1>(x));
  if (LANES >= 4) x = fmaxf(x, dpp_mov<0x4E>(x));
  if (LANES >= 8) x = fmaxf(x, dpp_mov<0x141>(x));
  if (LANES >= 16) x = fmaxf(x, dpp_mov<0x140>(x));
  return x;
}

// int8 row quantization of the retrieval cache (duo_kv_format DUO_KV_INT8):
// scale = amax / 127, code = clamp(rint(x / scale), -127, 127), both in fp32
// with round to nearest even; stored as the byte code + 128.  A zero row has
// scale 0; its codes come out 0 (x / 1 = 0).
__device__ __forceinline__ float int8_row_scale(float amax) { return __fdiv_rn(amax, 127.0f); }
__device__ __forceinline__ uint32_t int8_code(float x, float scale) {
  const float r = __builtin_rintf(__fdiv_rn(x, scale > 0.f ? scale : 1.0f));
  return (uint32_t)((int)fminf(fmaxf(r, -127.0f), 127.0f) + 128);
}

// Quantize the 8 bf16 values x (chunk c of a row whose CH lanes call this
// together) and store their 8 codes at codes + 8c; chunk 0 stores the scale.
template <int CH>
__device__ __forceinline__ void store_int8_row(uint8_t* codes, float* scale_out, const uint4& x, int c) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[e])), fabsf(bf16_hi(w[e]))));
  amax = group_max<CH>(amax);
  const float scale = int8_row_scale(amax);
  uint32_t q[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t lo = int8_code(bf16_lo(w[e]), scale), hi = int8_code(bf16_hi(w[e]), scale);
    q[e >> 1] |= (lo | (hi << 8)) << (16 * (e & 1));
  }
  reinterpret_cast<uint2*>(codes)[c] = make_uint2(q[0], q[1]);
  if (c == 0) *scale_out = scale;
}

}  // namespace duo
