// attention.hip -- fused non-causal MXFP4 attention forward for gfx950.
//
// MXAttention (arXiv 2607.24377), abstract: Q.K^T and P.V run on MXFP4
// operands; the softmax loop applies Pre-Normalization Quantization (PNQ),
// i.e. the unnormalized exponentials exp(s - m) are quantized to MXFP4 before
// they are summed, so the row sum and P.V see the same values.
//
// Kernel structure (one workgroup = 256 queries of one head, 8 waves of 32
// queries = two 16-query groups per wave):
//   for each key tile of kBC = 128 keys (ascending):
//     stage K codes/scales (keys x d) and V codes/scales (d x the tile's four
//       32-key blocks) in LDS;
//     S^T = K Q^T with one 16x16x128 FP4 MFMA per 16 keys (Q stays in
//       registers as the B operand; the E8M0 scales go in as MFMA scales);
//     running max per query, alpha = exp(m_old - m_new);
//     p = exp(s - m_new) in fp32, quantized per 32-key block in registers;
//     l = alpha l + sum(p_q)   (PNQ: one extra MFMA against a ones tile)
//       or alpha l + sum(p)    (PNQ off);
//     O^T = alpha O^T + V^T P_q^T, one 16x16x128 MFMA per 16 channels.
//   O = O / l rounded to bf16.
//
// The K rows fed to the S^T MFMA are permuted so that every lane's 32 output
// values are exactly one 32-key block of one query: lane l holds query l%16
// and keys 32*(l/16) + [0, 32) of the tile.  Block maxima and the FP4 encode
// then stay inside the lane, and the packed codes are already the lane's B
// operand slice (query l%16, keys 32*(l/16) + n) of the P.V MFMA.
#include "mx_device.h"

namespace mxattn {

struct AttnArgs {
  const uint8_t* qc;
  const uint8_t* qs;
  const uint8_t* kc;
  const uint8_t* ks;
  const uint8_t* vc;
  const uint8_t* vs;
  uint16_t* o;
  int BH;       // batch * heads
  int N;        // tokens per head (queries = keys)
  int nbn;      // 32-key blocks per V channel, ceil(N / 32)
  int ntq;      // query tiles per head
  int per_xcd;  // workgroups per XCD in the tile order below
  float c;      // softmax_scale * log2(e)
};

constexpr int kBC = 128;    // keys per tile: the running-max update granularity
constexpr int kWaves = 8;   // waves per workgroup
constexpr int kQG = 2;      // 16-query groups per wave
constexpr int kBR = kWaves * kQG * 16;  // queries per workgroup

namespace {

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

}  // namespace

template <int D, int MODE, bool PNQ>
__global__ __launch_bounds__(kWaves * 64, 1) void attn_fwd_kernel(AttnArgs a) {
  constexpr int DB = D / 32;      // 32-blocks along d in a Q/K row
  constexpr int CROW = D / 2;     // code bytes per Q/K row
  constexpr int KSTR = 80;        // LDS stride of a K row (64 code bytes + pad)
  constexpr int VSTR = 80;        // LDS stride of a V channel (4 blocks x 16 B + pad)
  constexpr int NCT = D / 16;     // 16-channel tiles of O^T
  constexpr int KCH = kBC * CROW / 16;  // 16-byte chunks of a K tile
  constexpr int VCH = D * 4;            // 16-byte chunks of a V tile
  static_assert(KCH <= kWaves * 64 && VCH <= kWaves * 64, "one chunk per thread");
  __shared__ __attribute__((aligned(16))) uint8_t k_lds[kBC * KSTR];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds[D * VSTR];
  __shared__ uint32_t ks_lds[kBC];  // byte b = scale of d-block b of the key
  __shared__ uint32_t vs_lds[D];    // byte b = scale of the tile's block b of the channel

  // Tile order: workgroup w is dispatched to XCD w % 8.  Each XCD gets a
  // contiguous range of (head, query tile) pairs, so the workgroups resident
  // on one XCD stream the same head's K/V through that XCD's L2.
  const int w = blockIdx.x;
  const int lin = (w & 7) * a.per_xcd + (w >> 3);
  if (lin >= a.BH * a.ntq) return;
  const int64_t bh = lin / a.ntq;
  const int qt = lin % a.ntq;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int N = a.N;
  const float c = a.c;

  // Q^T operand slices: query r16 of group g, d-block g4.
  uint4 qB[kQG];
  int qS[kQG];
#pragma unroll
  for (int g = 0; g < kQG; ++g) {
    const int qi = qt * kBR + wave * 32 + g * 16 + r16;
    qB[g] = make_uint4(0, 0, 0, 0);
    qS[g] = 127;
    if (qi < N && g4 < DB) {
      const int64_t row = bh * N + qi;
      qB[g] = *reinterpret_cast<const uint4*>(a.qc + row * CROW + 16 * g4);
      qS[g] = a.qs[row * DB + g4];
    }
  }

  v4f O[kQG][NCT];
  v4f L[kQG];
  float m[kQG];
#pragma unroll
  for (int g = 0; g < kQG; ++g) {
    m[g] = -INFINITY;
    L[g] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) O[g][ct] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  const uint4 ones = make_uint4(0x22222222u, 0x22222222u, 0x22222222u, 0x22222222u);  // E2M1 1.0

  // staging registers for the next tile
  uint4 kreg = make_uint4(0, 0, 0, 0), vreg = make_uint4(0, 0, 0, 0);
  uint32_t sreg = 0;
  const int ntk = (N + kBC - 1) / kBC;
  const uint8_t* kc_h = a.kc + bh * int64_t(N) * CROW;
  const uint8_t* ks_h = a.ks + bh * int64_t(N) * DB;
  const uint8_t* vc_h = a.vc + bh * int64_t(D) * a.nbn * 16;
  const uint8_t* vs_h = a.vs + bh * int64_t(D) * a.nbn;

  auto load_tile = [&](int j) {
    const int kb = j * kBC;
    const int vb0 = kb / 32;
    kreg = make_uint4(0, 0, 0, 0);
    vreg = make_uint4(0, 0, 0, 0);
    sreg = 0;
    if (tid < KCH) {
      const int row = tid / (CROW / 16), col = tid % (CROW / 16);
      if (kb + row < N) kreg = *reinterpret_cast<const uint4*>(kc_h + int64_t(kb + row) * CROW + 16 * col);
    }
    if (tid < VCH) {
      const int ch = tid >> 2, blk = tid & 3;
      if (vb0 + blk < a.nbn) vreg = *reinterpret_cast<const uint4*>(vc_h + (int64_t(ch) * a.nbn + vb0 + blk) * 16);
    }
    if (tid < kBC) {
      if (kb + tid < N) {
        const uint8_t* p = ks_h + int64_t(kb + tid) * DB;
#pragma unroll
        for (int b = 0; b < DB; ++b) sreg |= uint32_t(p[b]) << (8 * b);
      }
    } else if (tid < kBC + D) {
      const int ch = tid - kBC;
      const uint8_t* p = vs_h + int64_t(ch) * a.nbn + vb0;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (vb0 + b < a.nbn) sreg |= uint32_t(p[b]) << (8 * b);
    }
  };
  auto store_tile = [&]() {
    if (tid < KCH) {
      const int row = tid / (CROW / 16), col = tid % (CROW / 16);
      *reinterpret_cast<uint4*>(&k_lds[row * KSTR + 16 * col]) = kreg;
    }
    if (tid < VCH) {
      const int ch = tid >> 2, blk = tid & 3;
      *reinterpret_cast<uint4*>(&v_lds[ch * VSTR + 16 * blk]) = vreg;
    }
    if (tid < kBC)
      ks_lds[tid] = sreg;
    else if (tid < kBC + D)
      vs_lds[tid - kBC] = sreg;
  };

  load_tile(0);
  for (int j = 0; j < ntk; ++j) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (j + 1 < ntk) load_tile(j + 1);

    const int kb = j * kBC;
    // ---- S^T = K Q^T: 8 MFMAs of 16 keys per query group ----
    v4f S[kQG][8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int krow = 32 * (r16 >> 2) + 4 * t + (r16 & 3);
      uint4 kA = make_uint4(0, 0, 0, 0);
      int kS = 127;
      if (g4 < DB) {
        kA = *reinterpret_cast<const uint4*>(&k_lds[krow * KSTR + 16 * g4]);
        kS = int((ks_lds[krow] >> (8 * g4)) & 0xFFu);
      }
#pragma unroll
      for (int g = 0; g < kQG; ++g) S[g][t] = mfma_fp4_16x16x128(kA, qB[g], v4f{0.f, 0.f, 0.f, 0.f}, kS, qS[g]);
    }
    // keys past N (last tile only): s = -inf, so p = 0
    if (kb + kBC > N) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          if (kb + 32 * g4 + 4 * t + jj >= N) {
#pragma unroll
            for (int g = 0; g < kQG; ++g) S[g][t][jj] = -INFINITY;
          }
    }

    uint4 pk[kQG];
    int pS[kQG];
    float alpha[kQG];
#pragma unroll
    for (int g = 0; g < kQG; ++g) {
      // block max (this lane's 32 keys), then the row max over the 4 lanes of the query
      float bm = S[g][0][0];
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) bm = fmaxf(bm, S[g][t][jj]);
      float rm = fmaxf(bm, __shfl_xor(bm, 16));
      rm = fmaxf(rm, __shfl_xor(rm, 32));
      const float mnew = fmaxf(m[g], rm);
      alpha[g] = fast_exp2((m[g] - mnew) * c);
      m[g] = mnew;
      const float mc = mnew * c;
      // block scale from the block max; (bm - mnew) is exactly 0 for the block
      // holding the row max, so its amax is exactly 1
      const float amax = fast_exp2((bm - mnew) * c);
      int e = block_exp_f32bits<MODE>(__float_as_uint(amax));
      e = e < -126 ? -126 : e;
      pS[g] = e + 127;
      const float sc = pow2f(e);
      float p[8][4];
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) p[t][jj] = fast_exp2(fmaf(S[g][t][jj], c, -mc));
      // nibble n of the operand = key 32*g4 + n, n = 4t + jj
      uint32_t d0 = 0, d1 = 0, d2 = 0, d3 = 0;
      d0 = cvt_fp4x2<0>(d0, p[0][0], p[0][1], sc);
      d0 = cvt_fp4x2<1>(d0, p[0][2], p[0][3], sc);
      d0 = cvt_fp4x2<2>(d0, p[1][0], p[1][1], sc);
      d0 = cvt_fp4x2<3>(d0, p[1][2], p[1][3], sc);
      d1 = cvt_fp4x2<0>(d1, p[2][0], p[2][1], sc);
      d1 = cvt_fp4x2<1>(d1, p[2][2], p[2][3], sc);
      d1 = cvt_fp4x2<2>(d1, p[3][0], p[3][1], sc);
      d1 = cvt_fp4x2<3>(d1, p[3][2], p[3][3], sc);
      d2 = cvt_fp4x2<0>(d2, p[4][0], p[4][1], sc);
      d2 = cvt_fp4x2<1>(d2, p[4][2], p[4][3], sc);
      d2 = cvt_fp4x2<2>(d2, p[5][0], p[5][1], sc);
      d2 = cvt_fp4x2<3>(d2, p[5][2], p[5][3], sc);
      d3 = cvt_fp4x2<0>(d3, p[6][0], p[6][1], sc);
      d3 = cvt_fp4x2<1>(d3, p[6][2], p[6][3], sc);
      d3 = cvt_fp4x2<2>(d3, p[7][0], p[7][1], sc);
      d3 = cvt_fp4x2<3>(d3, p[7][2], p[7][3], sc);
      pk[g] = make_uint4(d0, d1, d2, d3);
      if (!PNQ) {
        float ps = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) ps += p[t][jj];
        L[g][0] = L[g][0] * alpha[g] + ps;
      }
    }
    // ---- rescale O (and l) only when some running max moved ----
    bool moved = false;
#pragma unroll
    for (int g = 0; g < kQG; ++g) moved |= alpha[g] != 1.0f;
    if (__any(moved)) {
#pragma unroll
      for (int g = 0; g < kQG; ++g) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) O[g][ct] *= alpha[g];
        if (PNQ) L[g] *= alpha[g];
      }
    }
    // ---- l += sum(p_q) (PNQ) and O^T += V^T P_q^T ----
    if (PNQ) {
#pragma unroll
      for (int g = 0; g < kQG; ++g) L[g] = mfma_fp4_16x16x128(ones, pk[g], L[g], 127, pS[g]);
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int vrow = 16 * ct + r16;
      const uint4 vA = *reinterpret_cast<const uint4*>(&v_lds[vrow * VSTR + 16 * g4]);
      const int vS = int((vs_lds[vrow] >> (8 * g4)) & 0xFFu);
#pragma unroll
      for (int g = 0; g < kQG; ++g) O[g][ct] = mfma_fp4_16x16x128(vA, pk[g], O[g][ct], vS, pS[g]);
    }
  }

  // ---- epilogue: O / l -> bf16 ----
#pragma unroll
  for (int g = 0; g < kQG; ++g) {
    float l = L[g][0];
    if (!PNQ) {
      l += __shfl_xor(l, 16);
      l += __shfl_xor(l, 32);
    }
    const int qi = qt * kBR + wave * 32 + g * 16 + r16;
    if (qi < N) {
      uint16_t* orow = a.o + (bh * N + qi) * int64_t(D);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const uint32_t b0 = f32_to_bf16_rne(O[g][ct][0] / l), b1 = f32_to_bf16_rne(O[g][ct][1] / l);
        const uint32_t b2 = f32_to_bf16_rne(O[g][ct][2] / l), b3 = f32_to_bf16_rne(O[g][ct][3] / l);
        *reinterpret_cast<uint2*>(orow + 16 * ct + 4 * g4) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
      }
    }
  }
}

hipError_t launch_attention(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                            const uint8_t* vc, const uint8_t* vs, int BH, int N, int d, int mode,
                            bool pnq, float softmax_scale, uint16_t* o, hipStream_t stream) {
  AttnArgs a;
  a.qc = qc; a.qs = qs; a.kc = kc; a.ks = ks; a.vc = vc; a.vs = vs; a.o = o;
  a.BH = BH;
  a.N = N;
  a.nbn = (N + 31) / 32;
  a.ntq = (N + kBR - 1) / kBR;
  const int total = BH * a.ntq;
  a.per_xcd = (total + 7) / 8;
  a.c = softmax_scale * 1.4426950408889634f;
  const dim3 grid(unsigned(a.per_xcd * 8)), block(kWaves * 64);
#define MXATTN_LAUNCH(D_, M_, P_) attn_fwd_kernel<D_, M_, P_><<<grid, block, 0, stream>>>(a)
  if (d == 128) {
    if (mode == kModeUOS) { if (pnq) MXATTN_LAUNCH(128, kModeUOS, true); else MXATTN_LAUNCH(128, kModeUOS, false); }
    else { if (pnq) MXATTN_LAUNCH(128, kModeOCP, true); else MXATTN_LAUNCH(128, kModeOCP, false); }
  } else {
    if (mode == kModeUOS) { if (pnq) MXATTN_LAUNCH(64, kModeUOS, true); else MXATTN_LAUNCH(64, kModeUOS, false); }
    else { if (pnq) MXATTN_LAUNCH(64, kModeOCP, true); else MXATTN_LAUNCH(64, kModeOCP, false); }
  }
#undef MXATTN_LAUNCH
  return hipGetLastError();
}

}  // namespace mxattn
