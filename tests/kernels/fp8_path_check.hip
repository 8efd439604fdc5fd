// Exhaustive checks of libmoe's blockwise-FP8 device path (test support).
//
// fp8_quotient_check: for every bf16 block maximum a > 0 and every bf16 x
//   with |x| <= a, the code libmoe's dispatch produces (fast quotient with
//   reciprocal and one fused correction above kFp8FastMinBits, IEEE division
//   below, gfx950 hardware E4M3 conversion) equals the software E4M3
//   (nearest even, saturating) of the correctly rounded quotient fl32(x/s),
//   s = fl32(a/448).
// fp8_convert_check: for every fp32 bit pattern with |v| < 464, gfx950's
//   conversion equals the software E4M3 rule.
// fp4_convert_check: for every fp32 bit pattern v but NaN (infinities
//   included), gfx950's E2M1 pair conversion (e2m1_pair_hw) of (v, -v) into
//   each of the four bytes equals the software E2M1 rule (e2m1_rne_sat:
//   nearest even, saturating at 6), and leaves the other three bytes of the
//   destination as they were.  NaN, which the hardware saturates to 6 and
//   the software rule maps to a signed zero code, is left to e2m1_lane8's
//   software path; cnt[3] counts the NaN patterns whose hardware code is
//   not +-6.
// Outputs: cnt[0] pairs tested, cnt[1] mismatches, cnt[2] records written,
// rec[3*i..] (inputs, got, want) of the first 8 mismatches.
#include "moe_device.hpp"

using namespace moe;

__global__ void quotient_kernel(unsigned long long *cnt, unsigned int *rec) {
  const uint32_t a16 = blockIdx.x + 1;  // 0x0001 .. 0x7F7F
  if (a16 > 0x7F7Fu) return;
  const uint32_t am = a16 << 16;
  const float s = __uint_as_float(am) / 448.0f;
  const float r = 1.0f / s;
  unsigned long long bad = 0, tested = 0;
  for (uint32_t xb = threadIdx.x; xb < 65536u; xb += blockDim.x) {
    if ((xb & 0x7FFFu) > a16) continue;
    const float x = __uint_as_float(xb << 16);
    const uint32_t want = e4m3_rne_sat(x / s);
    const float q = am >= kFp8FastMinBits ? fp8_quotient_fast(x, s, r) : x / s;
    const uint32_t lo = e4m3_pair_hw(q, 0.0f) & 0xFFu;
    const uint32_t hi = (e4m3_pair_hw(0.0f, q) >> 8) & 0xFFu;
    ++tested;
    if (lo != want || hi != want) {
      ++bad;
      const unsigned long long slot = atomicAdd(&cnt[2], 1ull);
      if (slot < 8) {
        rec[3 * slot] = am | xb;
        rec[3 * slot + 1] = (lo << 8) | hi;
        rec[3 * slot + 2] = want;
      }
    }
  }
  atomicAdd(&cnt[0], tested);
  atomicAdd(&cnt[1], bad);
}

__global__ void convert_kernel(unsigned long long *cnt, unsigned int *rec) {
  unsigned long long bad = 0, tested = 0;
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
  for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < (1ull << 32);
       i += stride) {
    const uint32_t u = static_cast<uint32_t>(i);
    const float v = __uint_as_float(u);
    if (!(fabsf(v) < 464.0f)) continue;  // also skips NaN
    const uint32_t want = e4m3_rne_sat(v);
    const uint32_t got = e4m3_pair_hw(v, v);
    ++tested;
    if ((got & 0xFFu) != want || (got >> 8) != want) {
      ++bad;
      const unsigned long long slot = atomicAdd(&cnt[2], 1ull);
      if (slot < 8) {
        rec[3 * slot] = u;
        rec[3 * slot + 1] = got;
        rec[3 * slot + 2] = want;
      }
    }
  }
  atomicAdd(&cnt[0], tested);
  atomicAdd(&cnt[1], bad);
}

extern "C" __attribute__((visibility("default"))) int fp8_quotient_check(unsigned long long *cnt,
                                                                         unsigned int *rec,
                                                                         void *stream) {
  quotient_kernel<<<0x7F7F, 256, 0, static_cast<hipStream_t>(stream)>>>(cnt, rec);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" __attribute__((visibility("default"))) int fp8_convert_check(unsigned long long *cnt,
                                                                        unsigned int *rec,
                                                                        void *stream) {
  convert_kernel<<<8192, 256, 0, static_cast<hipStream_t>(stream)>>>(cnt, rec);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

__global__ void fp4_convert_kernel(unsigned long long *cnt, unsigned int *rec) {
  unsigned long long bad = 0, tested = 0;
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
  const uint32_t keep = 0xA5C3E1F0u;  // bytes that must survive
  for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < (1ull << 32);
       i += stride) {
    const uint32_t u = static_cast<uint32_t>(i);
    const float v = __uint_as_float(u), w = __uint_as_float(u ^ 0x80000000u);
    if (v != v) {  // NaN: the hardware saturates (sign kept)
      const uint32_t h = e2m1_pair_hw<0>(0u, v, w);
      const uint32_t sat = (u >> 31) ? 0x7Fu : 0xF7u;  // (v, -v) = (-6, +6) or (+6, -6)
      if (h != sat) atomicAdd(&cnt[3], 1ull);
      continue;
    }
    const uint32_t pair = e2m1_rne_sat(v) | (e2m1_rne_sat(w) << 4);
    const uint32_t g0 = e2m1_pair_hw<0>(keep, v, w), g1 = e2m1_pair_hw<1>(keep, v, w);
    const uint32_t g2 = e2m1_pair_hw<2>(keep, v, w), g3 = e2m1_pair_hw<3>(keep, v, w);
    ++tested;
    const bool ok = g0 == ((keep & ~0xFFu) | pair) && g1 == ((keep & ~0xFF00u) | (pair << 8)) &&
                    g2 == ((keep & ~0xFF0000u) | (pair << 16)) && g3 == ((keep & 0xFFFFFFu) | (pair << 24));
    if (!ok) {
      ++bad;
      const unsigned long long slot = atomicAdd(&cnt[2], 1ull);
      if (slot < 8) {
        rec[3 * slot] = u;
        rec[3 * slot + 1] = g0;
        rec[3 * slot + 2] = (keep & ~0xFFu) | pair;
      }
    }
  }
  atomicAdd(&cnt[0], tested);
  atomicAdd(&cnt[1], bad);
}

extern "C" __attribute__((visibility("default"))) int fp4_convert_check(unsigned long long *cnt,
                                                                        unsigned int *rec,
                                                                        void *stream) {
  fp4_convert_kernel<<<8192, 256, 0, static_cast<hipStream_t>(stream)>>>(cnt, rec);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
