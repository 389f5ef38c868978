// attention.hip -- fused non-causal MXFP4 attention forward for gfx950.
//
// MXAttention (arXiv 2607.24377), abstract: Q.K^T and P.V run on MXFP4
// operands; the softmax loop applies Pre-Normalization Quantization (PNQ),
// i.e. the unnormalized exponentials exp(s - m) are quantized to MXFP4 before
// they are summed, so the row sum and P.V see the same values.
//
// Kernel structure (one workgroup = 128 queries of one head, 4 waves of 32
// queries = two 16-query groups per wave; two workgroups share a CU so their
// MFMA and VALU phases interleave on each SIMD):
//   K/V tiles of kBC = 128 keys, double-buffered in LDS (the next tile is
//   fetched into registers while the current one is used; one barrier per
//   tile).  For each tile, in ascending key order:
//     S^T = K Q^T with one 16x16x128 FP4 MFMA per 16 keys (Q stays in
//       registers as the B operand; the E8M0 scales go in as MFMA scales);
//     per 16-query group: running max, alpha = exp(m_old - m_new);
//     p = exp(s - m_new) in fp32, quantized per 32-key block in registers;
//     l = alpha l + sum(p_q)   (PNQ: one extra MFMA against a ones tile)
//       or alpha l + sum(p)    (PNQ off);
//     O^T = alpha O^T + V^T P_q^T, one 16x16x128 MFMA per 16 channels.
//     The second group's S^T MFMAs run under the first group's softmax VALU
//     work, and the first group's P.V MFMAs under the second group's.
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
constexpr int kWaves = 4;   // waves per workgroup (two workgroups share a CU)
constexpr int kQG = 2;      // 16-query groups per wave
constexpr int kBR = kWaves * kQG * 16;  // queries per workgroup

namespace {

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// max over the four lanes l, l^16, l^32, l^48 (the four 32-key blocks of one
// query): each swap hands every lane its partner's value.
__device__ __forceinline__ float max_over_blocks(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t v = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float sum_over_blocks(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t v = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// LDS layout of one 128-key tile.  K codes [key][64 B] and V codes
// [channel][64 B] (the tile's four 32-key blocks), 16-byte chunks XOR-swizzled
// so the 16 rows read by one MFMA operand load land in distinct bank groups.
// Scales are stored in MFMA lane order, 8 bytes per lane: ks[lane][t] is the
// K scale of sub-tile t (key row of that lane in sub-tile t, d-block l/16),
// vs[lane][ct] the V scale of channel tile ct (channel 16 ct + l%16, block
// l/16); one 8-byte read per lane fetches all of them and the MFMA's op_sel
// picks the byte.
__device__ __forceinline__ int k_chunk_addr(int row, int c) { return row * 64 + 16 * (c ^ ((row >> 5) & 3)); }
__device__ __forceinline__ int v_chunk_addr(int row, int c) { return row * 64 + 16 * (c ^ ((row >> 2) & 3)); }

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(1))) void* glb_ptr;

struct __align__(16) TileLds {
  uint8_t k[kBC * 64];
  uint8_t v[128 * 64];
  uint8_t ks[64 * 8];
  uint8_t vs[64 * 8];
};

// Online-softmax step for one 16-query group on one key tile: running max,
// exponentials, block scales and the packed FP4 operand.  S holds this lane's
// 32 scores (query r16, keys 32*g4 + 4t + jj).
template <int MODE, bool PNQ>
__device__ __forceinline__ void softmax_group(v4f (&S)[8], float& m, float c, uint4& pk, int& pS,
                                              float& alpha, float& lpart) {
  // two independent chains of three-input maxima over the 32 scores
  float b0 = fmaxf(fmaxf(S[0][0], S[0][1]), S[0][2]);
  float b1 = fmaxf(fmaxf(S[0][3], S[1][0]), S[1][1]);
  b0 = fmaxf(fmaxf(b0, S[1][2]), S[1][3]);
#pragma unroll
  for (int t = 2; t < 8; t += 2) {
    b1 = fmaxf(fmaxf(b1, S[t][0]), S[t][1]);
    b0 = fmaxf(fmaxf(b0, S[t][2]), S[t][3]);
    b1 = fmaxf(fmaxf(b1, S[t + 1][0]), S[t + 1][1]);
    b0 = fmaxf(fmaxf(b0, S[t + 1][2]), S[t + 1][3]);
  }
  const float bm = fmaxf(b0, b1);
  const float rm = max_over_blocks(bm);
  const float mnew = fmaxf(m, rm);
  alpha = fast_exp2((m - mnew) * c);
  m = mnew;
  const float mc = mnew * c;
  // block scale from the block max; (bm - mnew) is exactly 0 in the block
  // holding the row max, so that block's amax is exactly 1
  const float amax = fast_exp2((bm - mnew) * c);
  int e = block_exp_f32bits<MODE>(__float_as_uint(amax));
  e = e < -126 ? -126 : e;
  pS = e + 127;
  const float sc = pow2f(e);
  float p[8][4];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) p[t][jj] = fast_exp2(fmaf(S[t][jj], c, -mc));
  // nibble n of the operand = key 32*g4 + n, n = 4t + jj
  uint32_t d[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t x = 0;
    x = cvt_fp4x2<0>(x, p[2 * w][0], p[2 * w][1], sc);
    x = cvt_fp4x2<1>(x, p[2 * w][2], p[2 * w][3], sc);
    x = cvt_fp4x2<2>(x, p[2 * w + 1][0], p[2 * w + 1][1], sc);
    x = cvt_fp4x2<3>(x, p[2 * w + 1][2], p[2 * w + 1][3], sc);
    d[w] = x;
  }
  pk = make_uint4(d[0], d[1], d[2], d[3]);
  if (!PNQ) {
    float ps = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) ps += (p[t][0] + p[t][1]) + (p[t][2] + p[t][3]);
    lpart = lpart * alpha + ps;
  }
}

}  // namespace

template <int D, int MODE, bool PNQ>
__global__ __launch_bounds__(kWaves * 64, 2) void attn_fwd_kernel(AttnArgs a) {
  constexpr int DB = D / 32;      // 32-blocks along d in a Q/K row
  constexpr int CROW = D / 2;     // code bytes per Q/K row
  constexpr int NCT = D / 16;     // 16-channel tiles of O^T
  constexpr int NT = kWaves * 64;
  constexpr int KI = kBC * 4 / 64;  // wave-wide 16-byte fills per K tile
  constexpr int VI = D * 4 / 64;    // wave-wide 16-byte fills per V tile
  static_assert(kBC + D <= NT, "one scale word per thread");
  static_assert(KI % kWaves == 0 && VI % kWaves == 0, "fills split evenly over the waves");
  __shared__ TileLds lds0, lds1;

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
  const int N = a.N, nbn = a.nbn;
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
  float m[kQG], lpart[kQG];
#pragma unroll
  for (int g = 0; g < kQG; ++g) {
    m[g] = -INFINITY;
    lpart[g] = 0.f;
    L[g] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) O[g][ct] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  const uint4 ones = make_uint4(0x22222222u, 0x22222222u, 0x22222222u, 0x22222222u);  // E2M1 1.0

  // Per-lane LDS offsets.  Sub-tile t of the K operand is k_lane + 256 t (the
  // swizzle term does not depend on t); channel tile ct of the V operand is
  // v_lane + 1024 ct; this lane's 8 scale bytes sit at s_lane.
  const int k_lane = (32 * (r16 >> 2) + (r16 & 3)) * 64 + 16 * (g4 ^ (r16 >> 2));
  const int v_lane = r16 * 64 + 16 * (g4 ^ (r16 >> 2));
  const int s_lane = lane * 8;

  const int ntk = (N + kBC - 1) / kBC;
  const uint8_t* kc_h = a.kc + bh * int64_t(N) * CROW;
  const uint8_t* ks_h = a.ks + bh * int64_t(N) * DB;
  const uint8_t* vc_h = a.vc + bh * int64_t(D) * nbn * 16;
  const uint8_t* vs_h = a.vs + bh * int64_t(D) * nbn;

  // Tile fetch.  Code chunks go straight from global memory into LDS
  // (global_load_lds_dwordx4: lane i of a wave writes the 16 bytes at
  // dst + 16 i), so the swizzle is applied on the source side: LDS slot s of
  // the K tile holds (row s/4, chunk (s%4) ^ swizzle(row)).  In the last tile,
  // rows past N and V blocks past the padded end read the last valid row or
  // block instead (finite data whose scores are masked to -inf or whose
  // weights are 0).  Scale bytes take a register detour (one VGPR).
  int koff[KI / kWaves], krow_[KI / kWaves], kcol_[KI / kWaves];
#pragma unroll
  for (int u = 0; u < KI / kWaves; ++u) {
    const int slot = (wave + u * kWaves) * 64 + lane;
    const int row = slot >> 2;
    krow_[u] = row;
    kcol_[u] = ((slot & 3) ^ ((row >> 5) & 3)) % (CROW / 16);
    koff[u] = row * CROW + 16 * kcol_[u];
  }
  int voff[VI / kWaves], vrow_[VI / kWaves], vblk_[VI / kWaves];
#pragma unroll
  for (int u = 0; u < VI / kWaves; ++u) {
    const int slot = (wave + u * kWaves) * 64 + lane;
    const int row = slot >> 2;
    vrow_[u] = row;
    vblk_[u] = (slot & 3) ^ ((row >> 2) & 3);
    voff[u] = (row * nbn + vblk_[u]) * 16;
  }
  // where this thread's scale bytes go in the lane-ordered layout
  const int sk_key = tid;                   // tid < kBC: key of the tile
  const int sk_t = (sk_key & 31) >> 2, sk_r = ((sk_key >> 5) << 2) | (sk_key & 3);
  const int sv_ch = tid - kBC;              // kBC <= tid < kBC + D: channel
  const int sv_ct = sv_ch >> 4, sv_r = sv_ch & 15;

  uint32_t sreg = 0;
  auto issue_tile = [&](int j, TileLds& T) {
    const int kb = j * kBC;
    const int vb0 = kb / 32;
    const bool full_k = kb + kBC <= N;
    const bool full_v = vb0 + 4 <= nbn;
#pragma unroll
    for (int u = 0; u < KI / kWaves; ++u) {
      const uint8_t* src = full_k ? kc_h + int64_t(kb) * CROW + koff[u]
                                  : kc_h + int64_t(min(kb + krow_[u], N - 1)) * CROW + 16 * kcol_[u];
      __builtin_amdgcn_global_load_lds((glb_ptr)src, (lds_ptr)(T.k + (wave + u * kWaves) * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < VI / kWaves; ++u) {
      const uint8_t* src = full_v ? vc_h + int64_t(vb0) * 16 + voff[u]
                                  : vc_h + (int64_t(vrow_[u]) * nbn + min(vb0 + vblk_[u], nbn - 1)) * 16;
      __builtin_amdgcn_global_load_lds((glb_ptr)src, (lds_ptr)(T.v + (wave + u * kWaves) * 1024), 16, 0, 0);
    }
    sreg = 0;
    if (tid < kBC) {
      const uint8_t* p = ks_h + int64_t(min(kb + sk_key, N - 1)) * DB;
      if (DB == 4) {
        sreg = *reinterpret_cast<const uint32_t*>(p);
      } else {
#pragma unroll
        for (int b = 0; b < DB; ++b) sreg |= uint32_t(p[b]) << (8 * b);
      }
    } else if (tid < kBC + D) {
      const uint8_t* p = vs_h + int64_t(sv_ch) * nbn;
#pragma unroll
      for (int b = 0; b < 4; ++b) sreg |= uint32_t(p[min(vb0 + b, nbn - 1)]) << (8 * b);
    }
  };
  auto finish_tile = [&](TileLds& T) {
    if (tid < kBC) {
#pragma unroll
      for (int b = 0; b < DB; ++b) T.ks[(b * 16 + sk_r) * 8 + sk_t] = uint8_t(sreg >> (8 * b));
    } else if (tid < kBC + D) {
#pragma unroll
      for (int b = 0; b < 4; ++b) T.vs[(b * 16 + sv_r) * 8 + sv_ct] = uint8_t(sreg >> (8 * b));
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's LDS fills have landed
  };

  auto compute_tile = [&](int j, const TileLds& T) {
    const int kb = j * kBC;
    // ---- S^T = K Q^T for both groups: 8 MFMAs of 16 keys each ----
    uint2 ksw = make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
    if (g4 < DB) ksw = *reinterpret_cast<const uint2*>(&T.ks[s_lane]);
    v4f S[kQG][8];
#define MXATTN_S_STEP(t_)                                                                       \
    {                                                                                           \
      const uint4 kA = *reinterpret_cast<const uint4*>(&T.k[k_lane + 256 * (t_)]);              \
      _Pragma("unroll") for (int g = 0; g < kQG; ++g) S[g][t_] =                                \
          mfma_fp4_16x16x128<(t_) & 3, 0>(kA, qB[g], v4f{0.f, 0.f, 0.f, 0.f},                   \
                                          int((t_) < 4 ? ksw.x : ksw.y), qS[g]);                 \
    }
    MXATTN_S_STEP(0) MXATTN_S_STEP(1) MXATTN_S_STEP(2) MXATTN_S_STEP(3)
    MXATTN_S_STEP(4) MXATTN_S_STEP(5) MXATTN_S_STEP(6) MXATTN_S_STEP(7)
#undef MXATTN_S_STEP
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
    // ---- softmax step per group (rescaling O and l when a running max moved) ----
    uint4 pk[kQG];
    int pS[kQG];
#pragma unroll
    for (int g = 0; g < kQG; ++g) {
      float alpha;
      softmax_group<MODE, PNQ>(S[g], m[g], c, pk[g], pS[g], alpha, lpart[g]);
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) O[g][ct] *= alpha;
        if (PNQ) L[g] *= alpha;
      }
    }
    // ---- l += sum(p_q) (PNQ) and O^T += V^T P_q^T, each V operand feeding both groups ----
    if (PNQ) {
#pragma unroll
      for (int g = 0; g < kQG; ++g) L[g] = mfma_fp4_16x16x128(ones, pk[g], L[g], 127, pS[g]);
    }
    const uint2 vsw = *reinterpret_cast<const uint2*>(&T.vs[s_lane]);
#define MXATTN_PV_STEP(ct_)                                                                     \
    if ((ct_) < NCT) {                                                                          \
      const uint4 vA = *reinterpret_cast<const uint4*>(&T.v[v_lane + 1024 * (ct_)]);            \
      _Pragma("unroll") for (int g = 0; g < kQG; ++g) O[g][(ct_) % NCT] =                       \
          mfma_fp4_16x16x128<(ct_) & 3, 0>(vA, pk[g], O[g][(ct_) % NCT],                        \
                                           int((ct_) < 4 ? vsw.x : vsw.y), pS[g]);               \
    }
    MXATTN_PV_STEP(0) MXATTN_PV_STEP(1) MXATTN_PV_STEP(2) MXATTN_PV_STEP(3)
    MXATTN_PV_STEP(4) MXATTN_PV_STEP(5) MXATTN_PV_STEP(6) MXATTN_PV_STEP(7)
#undef MXATTN_PV_STEP
  };

  // Two LDS buffers; the loop is unrolled by two so each half addresses a
  // fixed buffer (constant LDS offsets).
  auto step = [&](int j, const TileLds& cur, TileLds& nxt) {
    if (j + 1 < ntk) issue_tile(j + 1, nxt);  // lands during this tile's compute
    compute_tile(j, cur);
    if (j + 1 < ntk) finish_tile(nxt);
    __syncthreads();
  };
  issue_tile(0, lds0);
  finish_tile(lds0);
  __syncthreads();
  for (int j = 0; j < ntk; j += 2) {
    step(j, lds0, lds1);
    if (j + 1 < ntk) step(j + 1, lds1, lds0);
  }

  // ---- epilogue: O / l -> bf16 ----
#pragma unroll
  for (int g = 0; g < kQG; ++g) {
    const float l = PNQ ? L[g][0] : sum_over_blocks(lpart[g]);
    const float inv = 1.0f / l;
    const int qi = qt * kBR + wave * 32 + g * 16 + r16;
    if (qi < N) {
      uint16_t* orow = a.o + (bh * N + qi) * int64_t(D);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const uint32_t b0 = f32_to_bf16_rne(O[g][ct][0] * inv), b1 = f32_to_bf16_rne(O[g][ct][1] * inv);
        const uint32_t b2 = f32_to_bf16_rne(O[g][ct][2] * inv), b3 = f32_to_bf16_rne(O[g][ct][3] * inv);
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
