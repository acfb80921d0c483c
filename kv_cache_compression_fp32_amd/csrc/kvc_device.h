// Device helpers of the compressor kernels (gfx950, wave64).
//
// Number formats: bf16 (round to nearest even), OCP e4m3fn scales and OCP
// e2m1 codes of the latent's fp4 round trip ("Module compress", Functions,
// fp4_quant_e4m3_inplace and to_e2m1_rne). Every rounding decision below is
// exact: scalings by powers of two, exact products and compares, and v_rndne.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
// amax floor of the latent's fp4 round trip: 6 * 2^-9
constexpr float kAmaxFloor = 0.01171875f;
// amax floor of the power-of-two-scaled fp4 round trip: 6 * 2^-126
constexpr float kAmaxFloorE8m0 = 7.052966e-38f;

__device__ __forceinline__ uint32_t as_u32(float f) { return __float_as_uint(f); }
__device__ __forceinline__ float as_f32(uint32_t u) { return __uint_as_float(u); }

// bf16 bits of f, round to nearest, ties to even; overflow goes to infinity,
// NaN to the quiet NaN (f >> 16) | 0x40. The hardware conversion
// (v_cvt_pk_bf16_f32 on gfx950) gives these bits: compared with the integer
// rounding (add 0x7fff plus the lowest kept bit, keep the high half) on every
// one of the 2^32 f32 patterns, with no difference.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ float bf16_val(uint32_t b) { return as_f32(b << 16); }

// e4m3fn code of q >= 0 (finite): nearest value, ties to even, saturating at
// 448. Below 2^-6 the values are multiples of 2^-9; above, 3 mantissa bits.
__device__ __forceinline__ uint32_t e4m3fn_rne(float q) {
  if (q >= 448.0f) return 0x7eu;
  if (q < 0.015625f) return (uint32_t)__builtin_rintf(q * 512.0f);  // 0..8; 8 is 2^-6
  const uint32_t u = as_u32(q);
  const int e = (int)(u >> 23) - 127;                             // -6 .. 8
  const float frac = as_f32((u & 0x007fffffu) | 0x3f800000u);     // [1, 2)
  const uint32_t m = (uint32_t)__builtin_rintf((frac - 1.0f) * 8.0f);  // 0..8
  const uint32_t code = ((uint32_t)(e + 7) << 3) + m;             // m == 8 carries
  return code > 0x7eu ? 0x7eu : code;
}

// value of an e4m3fn code (0x00..0x7e)
__device__ __forceinline__ float e4m3fn_val(uint32_t c) {
  const uint32_t e = c >> 3, m = c & 7u;
  if (e == 0) return (float)m * 0.001953125f;
  return as_f32(((e + 120u) << 23) | (m << 20));
}

// e2m1 code (sign in bit 3) of y / s by exact compares: |y| against the
// midpoints of the grid {0, .5, 1, 1.5, 2, 3, 4, 6} times s. The products are
// exact (s has at most 4 significant bits, the midpoints 3). A value on a
// midpoint goes to the even code: upward at 0.75, 1.75, 3.5, downward at
// 0.25, 1.25, 2.5, 5.
__device__ __forceinline__ uint32_t e2m1_rne(float y, float s) {
  const float a = __builtin_fabsf(y);
  uint32_t c = (a > 0.25f * s) + (a >= 0.75f * s) + (a > 1.25f * s) + (a >= 1.75f * s) +
               (a > 2.5f * s) + (a >= 3.5f * s) + (a > 5.0f * s);
  return c | ((as_u32(y) >> 31) << 3);
}

__device__ __forceinline__ float e2m1_val(uint32_t c) {
  // 0, .5, 1, 1.5, 2, 3, 4, 6 as (1 + m/2) * 2^(e-1), subnormal at e = 0
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  float v = (e == 0) ? 0.5f * (float)m : (1.0f + 0.5f * (float)m) * (float)(1u << (e - 1));
  return (c & 8u) ? -v : v;
}

// Softmax-weighted sum over NC candidates for each of VEC features, f32
// (the pooling formula of "DeepSeek V4.1 . Pool token pairs"). Shared by the
// pool kernels and the pooling GEMM epilogue, so both give the same bits.
// Candidates with logit -inf get weight exactly 0 (exp2(-inf) = 0).
template <int NC, int VEC>
__device__ __forceinline__ void softmax_pool(const float (&k)[NC][VEC], const float (&s)[NC][VEC],
                                             float (&out)[VEC]) {
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    float m = s[0][v];
#pragma unroll
    for (int i = 1; i < NC; ++i) m = __builtin_fmaxf(m, s[i][v]);
    float den = 0.0f, num = 0.0f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const float e = __builtin_amdgcn_exp2f((s[i][v] - m) * kLog2e);
      den += e;
      num = __builtin_fmaf(e, k[i][v], num);
    }
    out[v] = num * __builtin_amdgcn_rcpf(den);  // den in [1, NC]: v_rcp_f32 is within 1 ulp
  }
}

// Sum over all 64 lanes; every lane receives the same bits (each butterfly
// step adds the same two operands in both lanes of a pair).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// fp4 round trip of VEC consecutive bf16 values held by each lane, 16 / VEC
// neighbouring lanes forming one block of 16. `y` holds the bf16 values as
// f32. Returns through references: the packed codes of this lane (VEC / 2
// bytes, element 2k in the low nibble), the block's scale byte, and (DEQ)
// the bf16 bits of the dequantised values.
template <int VEC, bool DEQ = true>
__device__ __forceinline__ void fp4_block(const float (&y)[VEC], uint32_t &packed, uint32_t &scale_code,
                                          uint32_t (&deq)[VEC]) {
  static_assert(VEC >= 2 && VEC <= 8 && 16 % VEC == 0, "VEC must divide 16 and fit 32 code bits");
  float amax = 0.0f;
#pragma unroll
  for (int v = 0; v < VEC; ++v) amax = __builtin_fmaxf(amax, __builtin_fabsf(y[v]));
#pragma unroll
  for (int o = 1; o < 16 / VEC; o <<= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, o, kWave));
  const float a = __builtin_fmaxf(amax, kAmaxFloor);
  const float q = a / 6.0f;  // IEEE division (HIP's default for '/')
  scale_code = e4m3fn_rne(q);
  const float s = e4m3fn_val(scale_code);
  packed = 0;
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    const uint32_t c = e2m1_rne(y[v], s);
    packed |= c << (4 * v);
    if constexpr (DEQ) deq[v] = as_u32(e2m1_val(c) * s) >> 16;  // exact: at most 6 significant bits
  }
}

// e2m1 code (sign in bit 3) of t = |y| / scale already scaled exactly (the
// scale a power of two): compares against the grid midpoints, a value on a
// midpoint going to the even code.
__device__ __forceinline__ uint32_t e2m1_code_scaled(float t, uint32_t sign) {
  uint32_t c = (t > 0.25f) + (t >= 0.75f) + (t > 1.25f) + (t >= 1.75f) + (t > 2.5f) + (t >= 3.5f) + (t > 5.0f);
  return c | (sign << 3);
}

// fp4 round trip with power-of-two scales (the indexer's form, "Module
// compress", Functions, fp4_quant_e8m0_inplace) of VEC consecutive bf16
// values per lane, 32 / VEC neighbouring lanes forming one block of 32. The
// block's scale is 2^e, e the least integer with 2^e >= M / 6 (IEEE f32
// division), M its largest magnitude but at least 6 * 2^-126; the codes are
// those of y / 2^e and the dequantised values code * 2^e. Both scalings are
// ldexp by e, exact here.
// Returns the packed codes (element 2k in the low nibble), the e8m0 scale byte
// (e + 127) and the bf16 bits of the dequantised values.
template <int VEC, bool DEQ = true>
__device__ __forceinline__ void fp4_block_e8m0(const float (&y)[VEC], uint32_t &packed, uint32_t &scale_code,
                                               uint32_t (&deq)[VEC]) {
  static_assert(VEC >= 2 && VEC <= 8 && 32 % VEC == 0, "VEC must divide 32 and fit 32 code bits");
  float amax = 0.0f;
#pragma unroll
  for (int v = 0; v < VEC; ++v) amax = __builtin_fmaxf(amax, __builtin_fabsf(y[v]));
#pragma unroll
  for (int o = 1; o < 32 / VEC; o <<= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, o, kWave));
  const float q = __builtin_fmaxf(amax, kAmaxFloorE8m0) / 6.0f;  // normal, >= 2^-126
  const uint32_t qb = as_u32(q);
  const int e = (int)(qb >> 23) - 127 + ((qb & 0x007fffffu) != 0u);
  scale_code = (uint32_t)(e + 127);
  packed = 0;
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    const float t = __builtin_ldexpf(__builtin_fabsf(y[v]), -e);
    const uint32_t c = e2m1_code_scaled(t, as_u32(y[v]) >> 31);
    packed |= c << (4 * v);
    if constexpr (DEQ) deq[v] = as_u32(__builtin_ldexpf(e2m1_val(c), e)) >> 16;
  }
}

// bf16 bits of the exact sum p + q of two doubles, round to nearest even
// (single rounding). hi = p + q rounded to double with the exact error lo
// (TwoSum); lo can change the bf16 result only when hi lies exactly on a bf16
// midpoint, and then hi moves one double step towards lo. hi is then rounded
// to f32 with round-to-odd (toward zero, last bit set when inexact), and that
// f32 to bf16 with round to nearest even: f32 keeps 16 more bits than bf16, so
// the two steps round like one.
__device__ __forceinline__ uint32_t bf16_of_sum(double p, double q) {
  double hi = p + q;
  const double z = hi - p;
  const double lo = (p - (hi - z)) + (q - z);
  float f = (float)hi;
  const bool f_exact = (double)f == hi;
  if (f_exact && lo != 0.0 && (as_u32(f) & 0xffffu) == 0x8000u) {
    // move one double step towards lo (hi is nonzero here)
    const uint64_t hb = (uint64_t)__double_as_longlong(hi);
    const bool up = (lo > 0.0) == (hi > 0.0);  // away from zero?
    hi = __longlong_as_double((long long)(up ? hb + 1 : hb - 1));
    f = (float)hi;
  }
  if (__builtin_fabs((double)f) > __builtin_fabs(hi)) f = as_f32(as_u32(f) - 1u);  // toward zero
  uint32_t u = as_u32(f);
  if ((double)f != hi) u |= 1u;  // round to odd
  return bf16_rne(as_f32(u));
}

// One rotary pair (a, b) of bf16 values turned by (c, s): the exact
// a c - b s and a s + b c (products of a bf16 and an f32 value are exact in
// double), each rounded once to bf16.
__device__ __forceinline__ void rope_pair(float a, float b, float c, float s, uint32_t &r0, uint32_t &r1) {
  const double da = a, db = b, dc = c, ds = s;
  const double ac = da * dc, bs = db * ds, as = da * ds, bc = db * dc;
  r0 = bf16_of_sum(ac, -bs);
  r1 = bf16_of_sum(as, bc);
}

}  // namespace kvc
