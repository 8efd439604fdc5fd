// moe_device.hpp -- wave64 helpers and number-format conversions shared by
// the plan, dispatch and combine kernels (gfx950, CDNA4).
//
// Format rules implemented here (all round to nearest, ties to even):
//   bf16   from fp32: IEEE rounding of the low 16 bits (bias-add form).
//   E4M3   OCP 8-bit floating point, 4 exponent bits (bias 7), 3 mantissa
//          bits, largest finite 448, no infinities; values past 448 saturate.
//   E2M1   OCP MX v1.0 element: magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6;
//          saturating at 6.
//   E8M0   OCP MX v1.0 shared scale: X = floor(log2 amax) - 2 (2 is the
//          largest E2M1 exponent), stored as X + 127.
//   NVFP4  E2M1 codes, one E4M3 scale per 16 values, one fp32 global
//          encode scale.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

// -------------------------------------------------------------- buffers ---

// Raw (unstructured) buffer resource over `bytes` bytes at `base`.  Loads
// through it are bounds-checked by the hardware: a load at or past `bytes`
// returns zero and touches no memory (bytes = 0: no load touches memory).
// Kernels use them where a load is optional per lane or per wave: the
// load is then issued unconditionally, with no branch around it, so the
// compiler can wait for each load on its own instead of for all of them.
// Third-dword configuration of gfx9 raw buffers: 32-bit data format.
constexpr int kRawBufferConfig = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes),
                                           kRawBufferConfig);
}

// Cache-policy bits of a buffer load: streaming (non-temporal), or default.
constexpr int kLoadNT = 2;
constexpr int kLoadDefault = 0;

// ---------------------------------------------------------------- waves ---

__device__ __forceinline__ int lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// Number of set bits of `m` in lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) {
  return static_cast<uint64_t>(__ballot(p));
}

// Lanes of `active` holding the same key as this lane (keys < 2^bits).  One
// ballot per key bit: a lane survives bit b if its bit matches ours.
__device__ __forceinline__ uint64_t match_any(uint32_t key, int bits, uint64_t active) {
  uint64_t m = active;
  for (int b = 0; b < bits; ++b) {
    const bool set = (key >> b) & 1u;
    const uint64_t ones = ballot(set);
    m &= set ? ones : ~ones;
  }
  return m;
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}

// DPP controls (gfx9): quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror (lane i <- 7-i within 8), row_mirror (i <- 15-i within 16).
constexpr int kQuadSwap1 = 0xB1;
constexpr int kQuadSwap2 = 0x4E;
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// Maximum over the 4 lanes of a quad (unsigned compare).
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  v = max(v, dpp<kQuadSwap1>(v));
  v = max(v, dpp<kQuadSwap2>(v));
  return v;
}

// Maximum over the 16 lanes of a DPP row (unsigned compare).
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  v = quad_max(v);
  v = max(v, dpp<kRowHalfMirror>(v));
  v = max(v, dpp<kRowMirror>(v));
  return v;
}

// Inclusive prefix sum over the 64 lanes: four row shifts (1, 2, 4, 8) scan
// each 16-lane row, then row_bcast:15 / row_bcast:31 carry row totals into
// the rows above.  Lanes shifted in from outside a row read 0.
template <int CTRL, int ROWMASK, bool BOUND_ZERO>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWMASK, 0xF, BOUND_ZERO);
}

__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_i<0x111, 0xF, true>(v);   // row_shr:1
  v += dpp_i<0x112, 0xF, true>(v);   // row_shr:2
  v += dpp_i<0x114, 0xF, true>(v);   // row_shr:4
  v += dpp_i<0x118, 0xF, true>(v);   // row_shr:8
  v += dpp_i<0x142, 0xA, false>(v);  // row_bcast:15 -> rows 1 and 3
  v += dpp_i<0x143, 0xC, false>(v);  // row_bcast:31 -> rows 2 and 3
  return v;
}

// ---------------------------------------------------------------- bf16 ---

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;  // keep NaN a NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ void unpack8(const uint4 v, float (&f)[8]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// ---------------------------------------------------------------- E4M3 ---

// |v| is at most a hair above 448 here (v = x / (amax/448)).
__device__ __forceinline__ uint32_t e4m3_rne_sat(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x43E00000u) {            // |v| >= 448: largest finite code
    code = 0x7Eu;
  } else if (a < 0x3C800000u) {      // |v| < 2^-6: subnormal codes, step 2^-9
    code = static_cast<uint32_t>(__builtin_rintf(__uint_as_float(a) * 512.0f));
  } else {                           // normal: keep 3 mantissa bits
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    code = (r >> 20) - (120u << 3);  // exponent bias 127 -> 7
  }
  return sign | code;
}

// Blockwise FP8 quotient.  The code of x is E4M3(fl32(x / s)), s = amax/448.
// With r = fl32(1/s), q0 = fl32(x*r) and one fused correction
// q = fma(fma(-q0, s, x), r, q0), with the sign of x, gives the same E4M3
// code as the correctly rounded quotient for every bf16 pair |x| <= amax
// whose block maximum is at least 2^-103 (fp32 bits 0x0C000000); this was
// checked exhaustively over all such pairs on gfx950.  Blocks with smaller
// maxima take the IEEE division.
constexpr uint32_t kFp8FastMinBits = 0x0C000000u;

__device__ __forceinline__ float fp8_quotient_fast(float x, float s, float r) {
  const float q0 = x * r;
  return __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q0, s, x), r, q0), x);
}

// Two OCP E4M3 codes (round to nearest even) in the low 16 bits, code(a) in
// bits 0-7; gfx950's conversion matches the software rule above for every
// fp32 |v| < 464 (checked exhaustively), and |fl32(x/s)| <= 448 * (1 + 2^-22).
__device__ __forceinline__ uint32_t e4m3_pair_hw(float a, float b) {
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xFFFFu;
}

// Value of an E4M3 magnitude code (0 .. 0x7E): exact in fp32.
__device__ __forceinline__ float e4m3_magnitude(uint32_t code) {
  const uint32_t e = (code >> 3) & 15u, m = code & 7u;
  if (e == 0) return static_cast<float>(m) * 0x1p-9f;  // subnormals: m/8 * 2^-6
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// ---------------------------------------------------------------- E2M1 ---

// Midpoints between neighbouring E2M1 magnitudes; a tie goes to the even
// code, hence the alternation of > and >=.
__device__ __forceinline__ uint32_t e2m1_rne_sat(float v) {
  const float a = fabsf(v);
  const uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) +
                     (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return c | ((__float_as_uint(v) >> 28) & 8u);
}

// gfx950's conversion of two fp32 values to E2M1 codes, unscaled (scale
// operand 1.0), into byte SEL of `old`: a in the low nibble, b in the high
// one.  Equal to e2m1_rne_sat (nearest even, saturating) for every fp32
// input but NaN, which it saturates to 6 (checked exhaustively by the
// test-support kernels).
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pair_hw(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// Eight E2M1 codes of a lane, value i in bits 4i..4i+3.  With `hw`,
// gfx950's conversion (four independent byte conversions); otherwise the
// software rule.  The two agree on every input but NaN, which the hardware
// saturates to 6 and e2m1_rne_sat turns into a signed zero code, so callers
// pass hw only for a wave whose values hold no NaN (wave-uniform).
__device__ __forceinline__ uint32_t e2m1_lane8(const float (&q)[8], bool hw) {
  if (hw)
    return e2m1_pair_hw<0>(0u, q[0], q[1]) | e2m1_pair_hw<1>(0u, q[2], q[3]) |
           e2m1_pair_hw<2>(0u, q[4], q[5]) | e2m1_pair_hw<3>(0u, q[6], q[7]);
  uint32_t v = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) v |= e2m1_rne_sat(q[i]) << (4 * i);
  return v;
}

// Magnitude bits above those of infinity: a NaN.
__device__ __forceinline__ bool nan_bits(uint32_t abs_bits) { return abs_bits > 0x7F800000u; }

// E8M0 exponent X of a block with maximum magnitude bits `amax_bits` > 0:
// floor(log2 amax) - 2, clamped below at -127 (subnormal maxima land there).
__device__ __forceinline__ int mx_exponent(uint32_t amax_bits) {
  return max(static_cast<int>(amax_bits >> 23) - 129, -127);
}

}  // namespace moe
