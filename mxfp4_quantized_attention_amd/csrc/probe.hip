// probe.hip -- issue costs of the attention kernel's per-score instructions
// on gfx950, and how much of them runs under the scaled FP4 MFMA.
//
// The fused attention kernel does, per score element, one fma (scale and max
// shift), one v_exp_f32, half a v_max3_f32 and half a
// v_cvt_scalef32_pk_fp4_f32, next to the two 16x16x128 FP4 MFMAs per 16 keys
// that its FLOP count is made of.  Its vector-unit ceiling is priced from what
// these instructions cost on the chip; this kernel measures those costs so the
// ceiling is reproducible (libmxprobe.so, driven by bench.py's probe
// workload; no part of the attention path).
//
// One launch runs `wg_per_cu` workgroups of 8 waves per CU (two waves per
// SIMD per workgroup).  Waves 0..3 of a workgroup (one per SIMD) run op A,
// waves 4..7 run op B, each for its own number of iterations; an iteration
// issues 8 instructions of the op (8 independent dependency chains, so only
// issue throughput is measured).  The kernel time with both roles busy,
// against each role alone, gives the overlap of the two instruction streams
// on one SIMD.  The interleaved ops put one scaled FP4 MFMA and R vector
// instructions of one kind into the same wave's stream.  Two other scaled
// MFMA forms are timed as well, for the choice of shape: the 32x32x64 FP4
// form (the same FLOP rate in half the instructions) and the 16x16x128 FP8
// form.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

enum : int {
  kNone = 0,
  kFma = 1,
  kExp = 2,
  kCvt = 3,
  kMax3 = 4,
  kMfma = 5,
  kMfma32 = 6,  // v_mfma_scale_f32_32x32x64_f8f6f4, FP4 operands
  kMfmaF8 = 7,  // v_mfma_scale_f32_16x16x128_f8f6f4, FP8 (E4M3) operands
  // one MFMA then R instructions of a vector op, 8 times per iteration
  kMixBase = 16,  // kMixBase + 4 * R + vector op (kFma, kExp, kCvt, kMax3), R in {1, 2, 4, 8}
};

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ void fma8(float (&a)[8], float b, float c) {
  asm volatile(
      "v_fma_f32 %0, %0, %8, %9\n\tv_fma_f32 %1, %1, %8, %9\n\tv_fma_f32 %2, %2, %8, %9\n\t"
      "v_fma_f32 %3, %3, %8, %9\n\tv_fma_f32 %4, %4, %8, %9\n\tv_fma_f32 %5, %5, %8, %9\n\t"
      "v_fma_f32 %6, %6, %8, %9\n\tv_fma_f32 %7, %7, %8, %9"
      : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]), "+v"(a[7])
      : "v"(b), "v"(c));
}

__device__ __forceinline__ void exp8(float (&a)[8]) {
  asm volatile(
      "v_exp_f32 %0, %0\n\tv_exp_f32 %1, %1\n\tv_exp_f32 %2, %2\n\tv_exp_f32 %3, %3\n\t"
      "v_exp_f32 %4, %4\n\tv_exp_f32 %5, %5\n\tv_exp_f32 %6, %6\n\tv_exp_f32 %7, %7"
      : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]), "+v"(a[7]));
}

__device__ __forceinline__ void cvt8(float (&a)[8], float b, float c, float sc) {
  asm volatile(
      "v_cvt_scalef32_pk_fp4_f32 %0, %8, %9, %10\n\tv_cvt_scalef32_pk_fp4_f32 %1, %8, %9, %10\n\t"
      "v_cvt_scalef32_pk_fp4_f32 %2, %8, %9, %10\n\tv_cvt_scalef32_pk_fp4_f32 %3, %8, %9, %10\n\t"
      "v_cvt_scalef32_pk_fp4_f32 %4, %8, %9, %10\n\tv_cvt_scalef32_pk_fp4_f32 %5, %8, %9, %10\n\t"
      "v_cvt_scalef32_pk_fp4_f32 %6, %8, %9, %10\n\tv_cvt_scalef32_pk_fp4_f32 %7, %8, %9, %10"
      : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]), "+v"(a[7])
      : "v"(b), "v"(c), "v"(sc));
}

__device__ __forceinline__ void max38(float (&a)[8], float b, float c) {
  asm volatile(
      "v_max3_f32 %0, %0, %8, %9\n\tv_max3_f32 %1, %1, %8, %9\n\tv_max3_f32 %2, %2, %8, %9\n\t"
      "v_max3_f32 %3, %3, %8, %9\n\tv_max3_f32 %4, %4, %8, %9\n\tv_max3_f32 %5, %5, %8, %9\n\t"
      "v_max3_f32 %6, %6, %8, %9\n\tv_max3_f32 %7, %7, %8, %9"
      : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]), "+v"(a[7])
      : "v"(b), "v"(c));
}

// One vector instruction of op VOP on chain register x.
template <int VOP>
__device__ __forceinline__ void vec1(float& x, float b, float c, float sc) {
  if constexpr (VOP == kFma) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x) : "v"(b), "v"(c));
  else if constexpr (VOP == kExp) asm volatile("v_exp_f32 %0, %0" : "+v"(x));
  else if constexpr (VOP == kCvt) asm volatile("v_cvt_scalef32_pk_fp4_f32 %0, %1, %2, %3" : "+v"(x) : "v"(b), "v"(c), "v"(sc));
  else asm volatile("v_max3_f32 %0, %0, %1, %2" : "+v"(x) : "v"(b), "v"(c));
}

__device__ __forceinline__ v4f mfma(const v8i& A, const v8i& B, v4f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, 4, 4, 0, sa, 0, sb);
}

struct State {
  float a[8];
  v4f acc[4];
  float b, c, sc;
  v8i A, B;
  int sa, sb;
};

// OP < kMixBase: 8 instructions of OP per iteration.  Otherwise one MFMA and
// R instructions of vector op VOP, 8 times per iteration.
template <int OP, int VOP = 0, int R = 0>
__device__ __forceinline__ void loop(State& st, int iters) {
  if constexpr (OP == kMfma32) {
    // one accumulator chain, local to this path, so its 16 registers are not
    // held by the kernel's other paths (the probe runs 8 waves per SIMD, at
    // most 64 VGPRs)
    v16f acc32 = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int m = 0; m < 8; ++m)
        acc32 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(st.A, st.B, acc32, 4, 4, 0, st.sa, 0, st.sb);
    }
    st.a[0] += acc32[0] + acc32[15];
    return;
  }
  for (int it = 0; it < iters; ++it) {
    if constexpr (OP == kFma) fma8(st.a, st.b, st.c);
    else if constexpr (OP == kExp) exp8(st.a);
    else if constexpr (OP == kCvt) cvt8(st.a, st.b, st.c, st.sc);
    else if constexpr (OP == kMax3) max38(st.a, st.b, st.c);
    else if constexpr (OP == kMfma) {
#pragma unroll
      for (int m = 0; m < 8; ++m) st.acc[m & 3] = mfma(st.A, st.B, st.acc[m & 3], st.sa, st.sb);
    } else if constexpr (OP == kMfmaF8) {
#pragma unroll
      for (int m = 0; m < 8; ++m)
        st.acc[m & 3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(st.A, st.B, st.acc[m & 3], 0, 0, 0, st.sa, 0,
                                                                          st.sb);
    } else {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        st.acc[m & 3] = mfma(st.A, st.B, st.acc[m & 3], st.sa, st.sb);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < R; ++i) vec1<VOP>(st.a[(m * R + i) & 7], st.b, st.c, st.sc);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

template <int VOP>
__device__ __forceinline__ void mix(State& st, int r, int iters) {
  if (r == 1) loop<kMixBase, VOP, 1>(st, iters);
  else if (r == 2) loop<kMixBase, VOP, 2>(st, iters);
  else if (r == 4) loop<kMixBase, VOP, 4>(st, iters);
  else loop<kMixBase, VOP, 8>(st, iters);
}

__device__ __forceinline__ void run_op(int op, int iters, float* out, int gid) {
  const int lane = threadIdx.x & 63;
  State st;
#pragma unroll
  for (int i = 0; i < 8; ++i) st.a[i] = 1.0f + 1e-3f * float(lane + i);
  st.b = 0.999f;
  st.c = 1e-4f * float(lane);
  st.sc = 1.0f;
  st.A = v8i{0x22222222 + lane, 0x13131313, 0x24242424, 0x31313131, 0x22222222, 0x13131313, 0x24242424, 0x31313131};
  st.B = v8i{0x21212121, 0x12121212 + lane, 0x23232323, 0x32323232, 0x21212121, 0x12121212, 0x23232323, 0x32323232};
#pragma unroll
  for (int i = 0; i < 4; ++i) st.acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
  st.sa = 127;
  st.sb = 127;
  switch (op) {
    case kNone: break;
    case kFma: loop<kFma>(st, iters); break;
    case kExp: loop<kExp>(st, iters); break;
    case kCvt: loop<kCvt>(st, iters); break;
    case kMax3: loop<kMax3>(st, iters); break;
    case kMfma: loop<kMfma>(st, iters); break;
    case kMfma32: loop<kMfma32>(st, iters); break;
    case kMfmaF8: loop<kMfmaF8>(st, iters); break;
    default: {
      const int vop = op - kMixBase;  // kMixBase + 4 * R + (VOP & 3)
      const int r = vop >> 2;
      switch (vop & 3) {
        case kFma: mix<kFma>(st, r, iters); break;
        case kExp: mix<kExp>(st, r, iters); break;
        case kCvt: mix<kCvt>(st, r, iters); break;
        default: mix<kMax3>(st, r, iters); break;
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += st.a[i];
#pragma unroll
  for (int i = 0; i < 4; ++i) s += st.acc[i][0] + st.acc[i][1] + st.acc[i][2] + st.acc[i][3];

  // the results only keep the work alive; one store per wave
  if (lane == 0) out[gid] = s;
}

__global__ __launch_bounds__(512) void probe_kernel(int op_a, int iters_a, int op_b, int iters_b, float* out,
                                                    unsigned long long* clocks) {
  // wave-uniform values in scalar registers, so every loop is a scalar loop
  // and the vector pipe sees only the measured instructions
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gid = blockIdx.x * 8 + wave;
  unsigned long long t0 = 0, r0 = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  if (wave < 4) run_op(__builtin_amdgcn_readfirstlane(op_a), __builtin_amdgcn_readfirstlane(iters_a), out, gid);
  else run_op(__builtin_amdgcn_readfirstlane(op_b), __builtin_amdgcn_readfirstlane(iters_b), out, gid);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    // shader-clock cycles and 100 MHz ticks over wave 0 of workgroup 0
    clocks[0] = __builtin_amdgcn_s_memtime() - t0;
    clocks[1] = __builtin_amdgcn_s_memrealtime() - r0;
  }
}

}  // namespace

extern "C" {

// One probe launch: grid = 256 * wg_per_cu workgroups of 512 threads; `out`
// holds 8 floats per workgroup, `clocks` 2 counters.  Returns 0 or a HIP
// error code.
int mxprobe_launch(int op_a, int iters_a, int op_b, int iters_b, int wg_per_cu, float* out,
                   unsigned long long* clocks, void* stream) {
  auto valid = [](int op) { return (op >= kNone && op <= kMfmaF8) || (op >= kMixBase + 4 && op < kMixBase + 36); };
  if (wg_per_cu < 1 || wg_per_cu > 8 || iters_a < 0 || iters_b < 0 || !out || !clocks || !valid(op_a) || !valid(op_b))
    return -1;
  probe_kernel<<<dim3(256 * wg_per_cu), dim3(512), 0, static_cast<hipStream_t>(stream)>>>(op_a, iters_a, op_b,
                                                                                          iters_b, out, clocks);
  return int(hipGetLastError());
}

}  // extern "C"
