// mx_device.h -- gfx950 device helpers shared by the MXFP4 kernels.
//
// MXFP4 as read from the MXAttention abstract (arXiv 2607.24377): 32-element
// blocks, E2M1 elements, one E8M0 power-of-two scale per block.  The block
// exponent rules are OCP MXFP4 (e = floor(log2 amax) - 2) and UOS with the
// boundary Qmax = 7.25 (e = smallest integer with amax <= 7.25 * 2^e).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxattn {

enum : int { kModeOCP = 0, kModeUOS = 1 };

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Block exponent from the bit pattern of a non-negative bf16 amax.  amax =
// 2^E * M, M in [1, 2): OCP e = E - 2; UOS e = E - 2 + [M > 1.8125], which is
// the least e with amax <= 7.25 * 2^e (7.25 = 1.8125 * 4; 1.8125 is mantissa
// field 0x68 of the 7 bf16 mantissa bits).  A zero or subnormal amax has
// exponent field 0 and lands below -127, where the clamp puts it.
template <int MODE>
__device__ __forceinline__ int block_exp_bf16bits(uint32_t bits) {
  int E = int((bits >> 7) & 0xFFu) - 127;
  int e = E - 2;
  if (MODE == kModeUOS) e += (bits & 0x7Fu) > 0x68u ? 1 : 0;
  e = e < -127 ? -127 : e;
  e = e > 127 ? 127 : e;
  return e;
}

// 2^e as an fp32 value for e in [-126, 127].
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float(uint32_t(e + 127) << 23); }

// Two fp32 values -> two E2M1 codes in byte `SEL` of `old`, each value divided
// by the power of two `scale` first.  The hardware rounds to nearest, ties to
// the even code, saturates at 6 and keeps the sign of values that round to 0.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4x2(uint32_t old, float a, float b, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, scale, SEL);
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Eight fp32 values, block exponent e -> eight E2M1 codes (element 2i in
// nibble 2i).  y = x / 2^e is exact; the convert divides through its scale
// operand and rounds.  For e <= -125 a subnormal input could round to a
// non-zero code, so those (rare) blocks are first multiplied by 2^-e in fp32,
// which makes every non-zero y normal, and converted with scale 1.
__device__ __forceinline__ uint32_t encode8(float f0, float f1, float f2, float f3, float f4,
                                            float f5, float f6, float f7, int e) {
  float scale;
  if (e >= -124) {
    scale = pow2f(e);
  } else {
    const float up = pow2f(-e);  // -e in [124, 127]
    f0 *= up; f1 *= up; f2 *= up; f3 *= up; f4 *= up; f5 *= up; f6 *= up; f7 *= up;
    scale = 1.0f;
  }
  uint32_t r = 0;
  r = cvt_fp4x2<0>(r, f0, f1, scale);
  r = cvt_fp4x2<1>(r, f2, f3, scale);
  r = cvt_fp4x2<2>(r, f4, f5, scale);
  r = cvt_fp4x2<3>(r, f6, f7, scale);
  return r;
}

__device__ __forceinline__ uint32_t encode8_bf16(const uint4& v, int e) {
  return encode8(bf16lo(v.x), bf16hi(v.x), bf16lo(v.y), bf16hi(v.y), bf16lo(v.z), bf16hi(v.z),
                 bf16lo(v.w), bf16hi(v.w), e);
}

// Largest |x| bit pattern of the 8 bf16 values in v (non-negative floats
// order like their bit patterns).
__device__ __forceinline__ uint32_t absmax8_bits(const uint4& v) {
  const uint32_t m = 0x7FFF7FFFu;
  uint32_t a = v.x & m, b = v.y & m, c = v.z & m, d = v.w & m;
  auto mx = [](uint32_t p, uint32_t q) {
    uint32_t lo = max(p & 0xFFFFu, q & 0xFFFFu);
    uint32_t hi = max(p >> 16, q >> 16);
    return lo | (hi << 16);
  };
  uint32_t t = mx(mx(a, b), mx(c, d));
  return max(t & 0xFFFFu, t >> 16);
}


// Largest s in [0, n) with pre[s] <= v, for a non-decreasing prefix array
// pre of a varlen table (callers check v < pre[n] first, so the segment
// found is never empty).
__device__ __forceinline__ int find_segment(const int* pre, int n, int v) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= v) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// One 16x16x128 MFMA on FP4 operands with E8M0 block scales.
// A (16 rows x 128 K): lane l holds row l%16, K = 32*(l/16) + [0, 32) as 32
// nibbles in a[0..3] (nibble n of the 128 bits = K offset n).  B (128 K x 16
// cols): lane l holds col l%16 with the same K slice.  C/D: lane l holds col
// l%16, rows 4*(l/16) + [0, 4).  sa/sb: registers holding the E8M0 scale of the
// lane's 32-element K slice in byte SA/SB.
template <int SA = 0, int SB = 0>
__device__ __forceinline__ v4f mfma_fp4_16x16x128(const uint4& a, const uint4& b, v4f c, int sa, int sb) {
  v8i A = {int(a.x), int(a.y), int(a.z), int(a.w), 0, 0, 0, 0};
  v8i B = {int(b.x), int(b.y), int(b.z), int(b.w), 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, 4, 4, SA, sa, SB, sb);
}

}  // namespace mxattn
