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

// The eight values of codes w0, w1 (byte code + 128, as stored) of a row
// with scale sc, as bf16 pairs: (b - 128) sc rounded once to bf16, computed
// as one fma of b, sc and -128 sc (exact), so the same single rounding as
// the product.
__device__ __forceinline__ uint4 int8_dequant8(uint32_t w0, uint32_t w1, float sc) {
  const float off = -128.0f * sc;
  const uint32_t cw[2] = {w0, w1};
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t h = cw[e >> 1] >> (16 * (e & 1));
    w[e] = pack_bf16x2(fmaf((float)(h & 0xffu), sc, off), fmaf((float)((h >> 8) & 0xffu), sc, off));
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// fp8 retrieval cache (duo_kv_format DUO_KV_FP8): OCP E4M3 codes of
// x / scale, the scale a power of two (so x * (1/scale) is exact).  The
// conversion instruction rounds to nearest even but turns magnitudes from
// 465 up into NaN, so values are clamped to +-448 (the largest finite) first.
__device__ __forceinline__ float fp8_clamp(float x) { return fminf(fmaxf(x, -448.0f), 448.0f); }
// Codes of 4 values: bytes 0..3 of the result.
__device__ __forceinline__ uint32_t fp8_pack4(float a, float b, float c, float d) {
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_clamp(a), fp8_clamp(b), 0u, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(fp8_clamp(c), fp8_clamp(d), w, true);
}
// Store the codes of the 8 bf16 values x (chunk c of a row) at codes + 8c.
__device__ __forceinline__ void store_fp8_row8(uint8_t* codes, const uint4& x, int c, float inv_scale) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  const uint32_t lo = fp8_pack4(bf16_lo(w[0]) * inv_scale, bf16_hi(w[0]) * inv_scale, bf16_lo(w[1]) * inv_scale,
                                bf16_hi(w[1]) * inv_scale);
  const uint32_t hi = fp8_pack4(bf16_lo(w[2]) * inv_scale, bf16_hi(w[2]) * inv_scale, bf16_lo(w[3]) * inv_scale,
                                bf16_hi(w[3]) * inv_scale);
  reinterpret_cast<uint2*>(codes)[c] = make_uint2(lo, hi);
}
// The two fp32 values of the codes in bytes 2H, 2H+1 of w.
template <bool H>
__device__ __forceinline__ float2 fp8_unpack2(uint32_t w) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t f = __builtin_amdgcn_cvt_pk_f32_fp8(w, H);
  return make_float2(f.x, f.y);
}

// Eight e4m3 codes (bytes of w0, w1) times a power-of-two scale as bf16
// pairs: exact (an e4m3 value has 4 significant bits; decoded at unit scale,
// then scaled in fp32).
__device__ __forceinline__ uint4 fp8_to_bf16x8(uint32_t w0, uint32_t w1, float scale) {
  auto scaled = [scale](uint32_t x) { return pack_bf16x2(bf16_lo(x) * scale, bf16_hi(x) * scale); };
  return make_uint4(scaled(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false))),
                    scaled(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true))),
                    scaled(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false))),
                    scaled(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true))));
}

// The 8 bf16 values x as an fp8 cache stores them: code * scale, which
// bf16 holds exactly (e4m3 values have 4 significant bits).
__device__ __forceinline__ uint4 fp8_roundtrip8(const uint4& x, float inv_scale, float scale) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t c = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_clamp(bf16_lo(w[e]) * inv_scale),
                                                       fp8_clamp(bf16_hi(w[e]) * inv_scale), 0u, false);
    const float2 f = fp8_unpack2<false>(c);
    o[e] = pack_bf16x2(f.x * scale, f.y * scale);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Rotary position embedding (RoFormer): pair i of a head turns by p * theta_i
// at position p, theta_i = base^(-2i/D) = rho^i, (a, b) -> (a cos - b sin,
// a sin + b cos).  The angle is formed in fp64 revolutions (p * theta_i / 2 pi)
// and reduced to [-1/2, 1/2] before the fp32 sine and cosine: an fp32
// product p * theta_i would be off by whole radians at positions in the
// millions.  Revolutions per position of pair i, rho^i / (2 pi) by binary
// powering (a few fp64 roundings, ~1e-15 relative):
__device__ __forceinline__ double rope_rev(int i, double rho) {
  double r = 0.15915494309189535, b = rho;
#pragma unroll
  for (int k = 0; k < 6; ++k) {
    if (i & (1 << k)) r *= b;
    b *= b;
  }
  return r;
}

// sin and cos of 2 pi r (r in turns, fp64).  Whole and quarter turns come
// out in fp64 (exact); the rest, |x| <= pi/4, goes through the Taylor series
// of sin (to x^9) and cos (to x^10) in fp32, truncation below 3e-9.
__device__ __forceinline__ void sincos_turns(double r, float& s, float& c) {
  r -= rint(r);
  const double q = rint(4.0 * r);
  const float x = (float)((r - 0.25 * q) * 6.283185307179586);
  const float x2 = x * x;
  float sp = fmaf(x2, 1.0f / 362880.0f, -1.0f / 5040.0f);
  sp = fmaf(x2, sp, 1.0f / 120.0f);
  sp = fmaf(x2, sp, -1.0f / 6.0f);
  const float sx = fmaf(x * x2, sp, x);
  float cp = fmaf(x2, -1.0f / 3628800.0f, 1.0f / 40320.0f);
  cp = fmaf(x2, cp, -1.0f / 720.0f);
  cp = fmaf(x2, cp, 1.0f / 24.0f);
  cp = fmaf(x2, cp, -0.5f);
  const float cx = fmaf(x2, cp, 1.0f);
  const int k = (int)q & 3;  // quarter turns: the angle is x + k pi/2
  s = k == 0 ? sx : k == 1 ? cx : k == 2 ? -sx : -cx;
  c = k == 0 ? cx : k == 1 ? -sx : k == 2 ? -cx : sx;
}

__device__ __forceinline__ void rope_cos_sin(int p, double rev, float& c, float& s) {
  sincos_turns((double)p * rev, s, c);
}

// cos and sin of the angles of dims 8c .. 8c+7 at position p: interleaved
// pairs (2i, 2i+1) give 4 pairs (i = 4c ..), half-split pairs (i, i + D/2)
// 8 (i = 8c mod D/2 ..).
template <int D>
__device__ __forceinline__ void rope_angles8(int p, int c, bool half, double rho, float (&cs)[8], float (&sn)[8]) {
  double rev = rope_rev(half ? (8 * c) % (D / 2) : 4 * c, rho);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (half || (e & 1) == 0) {
      if (e > 0) rev *= rho;
      rope_cos_sin(p, rev, cs[e], sn[e]);
    } else {
      cs[e] = cs[e - 1];
      sn[e] = sn[e - 1];
    }
  }
}

// One step of a row group's angles: (cs, sn) turned by (cd, sd), the angles
// of the positions between two rows of the group (complex multiplication in
// fp32).
__device__ __forceinline__ void rope_step8(float (&cs)[8], float (&sn)[8], const float (&cd)[8], const float (&sd)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float c2 = fmaf(cs[e], cd[e], -sn[e] * sd[e]);
    sn[e] = fmaf(sn[e], cd[e], cs[e] * sd[e]);
    cs[e] = c2;
  }
}

// Positions between the rows that one lane loads in the prefill kernel's
// 64-row tiles (4 waves of 64 lanes, 16 bytes each: 512 / D rows per wave).
template <int D>
constexpr int rope_key_step() {
  return (512 / D) * 4;
}

// The angles of a K row at position p, formed the one way every K rotation
// forms them (the prefill's tile loads; the stores of append, decode and the
// int8 staging): the angles of the row group's base p - j R (R =
// rope_key_step, j = (p mod 64) / R) from fp64 turns, then j steps by the
// angles of R positions.  The tile loads turn R-spaced rows this way with
// one set of fp64 angles per lane; every other site reproduces it, so a key
// turns to the same bf16 value wherever it is turned.
template <int D>
__device__ __forceinline__ void rope_angles8_key(int p, int c, bool half, double rho, float (&cs)[8],
                                                 float (&sn)[8]) {
  constexpr int R = rope_key_step<D>();
  const int j = (p & 63) / R;
  rope_angles8<D>(p - j * R, c, half, rho, cs, sn);
  if (j > 0) {
    float cd[8], sd[8];
    rope_angles8<D>(R, c, half, rho, cd, sd);
    for (int t = 0; t < j; ++t) rope_step8(cs, sn, cd, sd);
  }
}

// Rotate the 8 bf16 values x (dims 8c .. 8c+7 of a row) by the angles of
// rope_angles8 and round them to bf16.  Half-split pairs join chunk c with
// chunk c ^ (CH/2), held by lane ^ (CH/2): the CH lanes of a row are
// consecutive and all call this together.
template <int CH>
__device__ __forceinline__ uint4 rope_apply8(const uint4& x, const float (&cs)[8], const float (&sn)[8], bool half,
                                             int c) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  float v[8], o[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = bf16_lo(w[e]);
    v[2 * e + 1] = bf16_hi(w[e]);
  }
  if (!half) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      o[e] = fmaf(v[e], cs[e], -v[e + 1] * sn[e]);
      o[e + 1] = fmaf(v[e], sn[e], v[e + 1] * cs[e]);
    }
  } else {
    const bool first = c < CH / 2;  // this lane holds the pairs' first dims
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t pw = (uint32_t)__shfl_xor((int)w[e], CH / 2);
      const float p0 = bf16_lo(pw), p1 = bf16_hi(pw);
      o[2 * e] = first ? fmaf(v[2 * e], cs[2 * e], -p0 * sn[2 * e]) : fmaf(p0, sn[2 * e], v[2 * e] * cs[2 * e]);
      o[2 * e + 1] = first ? fmaf(v[2 * e + 1], cs[2 * e + 1], -p1 * sn[2 * e + 1])
                           : fmaf(p1, sn[2 * e + 1], v[2 * e + 1] * cs[2 * e + 1]);
    }
  }
  return make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                    pack_bf16x2(o[6], o[7]));
}

}  // namespace duo
