// attention.hip -- fused non-causal MXFP4 attention forward for gfx950.
//
// MXAttention (arXiv 2607.24377), abstract: Q.K^T and P.V run on MXFP4
// operands; the online softmax applies Pre-Normalization Quantization (PNQ),
// i.e. the unnormalized exponentials exp(s - m) are quantized to MXFP4 before
// they are summed, so the row sum and P.V see the same values.
//
// Kernel structure: one workgroup = 128 queries of one head, 8 waves of one
// 16-query group each; two workgroups share a CU, so every SIMD holds four
// waves (at most 128 VGPRs each) and hides one wave's latency with the
// others' work.
//   K/V tiles of kBC = 128 keys, double-buffered in LDS: the next tile streams
//   from global memory straight into LDS while the current one is used, and
//   one barrier per tile publishes it.  For each tile, in ascending key order:
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
#include <type_traits>

#include "mx_device.h"

namespace mxattn {

struct AttnArgs {
  const uint16_t* q;   // bf16 Q (in-kernel quantization; strided, see below), or null
  const uint8_t* qc;   // else Q codes and scales, blocks along d
  const uint8_t* qs;
  const uint8_t* kc;
  const uint8_t* ks;
  const uint8_t* vc;
  const uint8_t* vs;
  uint16_t* o;
  // element strides of bf16 Q (when q is set) and of O: row (b, h, n) starts
  // at b * sb + h * sh + n * sn; d is contiguous
  int64_t q_sb, q_sh, q_sn, o_sb, o_sh, o_sn;
  int H;        // heads (splits the batch-head index of a workgroup)
  int BH;       // batch * heads
  int N;        // tokens per head (queries = keys); varlen: unused
  int vcs;      // V channel stride in 32-key blocks (dense: ceil(N / 32); varlen: from the table)
  int ntq;      // query tiles per head
  int per_xcd;  // workgroups per XCD in the tile order below
  float c;      // softmax_scale * log2(e)
  // varlen batches (packed [T][H][d] tokens): the table of sequence starts,
  // query-tile and V-block prefixes (4 (batch + 1) ints, built on the
  // device), the number of sequences, and T, the K code rows per head.
  // Workgroups then run over (head, query tile of any sequence).
  const int* vl;
  int batch;
  int kts;
};

constexpr int kBC = 128;    // keys per tile: the running-max update granularity
constexpr int kWaves = 8;   // waves per workgroup (two workgroups share a CU)
constexpr int kQG = 1;      // 16-query groups per wave
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
// by row.  The operand reads of both MFMAs touch rows whose offsets differ in
// bits the swizzle does not look at (K: key rows 4t apart; V: channel rows 16
// ct apart), so a lane's swizzle term is the same for every sub-tile.  The
// swizzle functions were chosen by measurement (SQ_LDS_BANK_CONFLICT for every
// XOR swizzle of this access shape on gfx950): a ds_read_b128 wave is served
// bank-conflict-free when the chunk flips with bit 2 of the lane's row index
// within its 16-row group (K: key-row bit 5; V: channel-row bit 2), and the
// previous swizzles, which also folded bit 3 into the low chunk bit, cost
// about 3.9 conflict cycles per read.
// Scales are stored in MFMA lane order, 8 bytes per lane: ks[lane][t] is the
// K scale of sub-tile t (key row of that lane in sub-tile t, d-block l/16),
// vs[lane][ct] the V scale of channel tile ct (channel 16 ct + l%16, block
// l/16); one 8-byte read per lane fetches all of them and the MFMA's op_sel
// picks the byte.
__device__ __forceinline__ int k_swz(int row) { return ((row >> 1) & 1) | ((row >> 4) & 2); }
__device__ __forceinline__ int v_swz(int row) { return (row >> 1) & 3; }

typedef __attribute__((address_space(3))) void* lds_ptr;

// Word 3 of a raw buffer descriptor on gfx9-class GPUs (32-bit data format,
// no swizzle): offsets at or past the record count read as zero.
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ const uint8_t* wave_uniform(const uint8_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<const uint8_t*>((uint64_t(hi) << 32) | lo);
}

struct __align__(16) TileLds {
  uint8_t k[kBC * 64];
  uint8_t v[128 * 64];
  uint8_t ks[64 * 8];
  uint8_t vs[64 * 8];
};

// Online-softmax step for one 16-query group on one key tile: running max,
// exponentials, block scales and the packed FP4 operand.  S holds this lane's
// 32 scores (query r16, keys 32*g4 + 4t + jj).  Returns whether any running
// max of the wave moved (alpha is then exp2((m_old - m_new) c), else 1).
template <int MODE, bool PNQ>
__device__ __forceinline__ bool softmax_group(v4f (&S)[8], float& m, float c, uint4& pk, int& pS,
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
  const float mold = m;
  const float mnew = fmaxf(mold, rm);
  const bool moved = __any(mnew != mold);
  alpha = 1.0f;
  if (moved) alpha = fast_exp2((mold - mnew) * c);
  m = mnew;
  const float mc = mnew * c;
  // Block exponent from xb = log2 of the block's largest exponential,
  // (bm - m) c, which is exactly 0 in the block holding the running max (its
  // amax is exactly 1).  OCP: e = floor(xb) - 2.  UOS: the least e with
  // 2^xb <= 7.25 2^e, e = ceil(xb - log2 7.25) = -floor(log2 7.25 - xb).
  // Both clamp at -126 (the convert takes its scale as a normal fp32); a block
  // with no valid key has xb = -inf and lands on the clamp.
  const float xb = (bm - mnew) * c;
  int eb;  // e + 127
  if (MODE == kModeUOS) {
    const int f = int(floorf(2.857981f - xb));  // log2(7.25)
    eb = 127 - min(f, 126);
  } else {
    const int f = int(floorf(xb));
    eb = max(f, -124) + 125;
  }
  pS = eb;
  const float sc = __uint_as_float(uint32_t(eb) << 23);
  // exponentials and their FP4 codes, one 8-code dword at a time (nibble n
  // of the operand = key 32*g4 + n, n = 4t + jj)
  uint32_t d[4];
  float ps = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = fast_exp2(fmaf(S[2 * w + i / 4][i % 4], c, -mc));
    // the four converts fill all four bytes, so the first one's merge input
    // can be any live register; reusing p[0] saves a v_mov per dword
    uint32_t x = __float_as_uint(p[0]);
    x = cvt_fp4x2<0>(x, p[0], p[1], sc);
    x = cvt_fp4x2<1>(x, p[2], p[3], sc);
    x = cvt_fp4x2<2>(x, p[4], p[5], sc);
    x = cvt_fp4x2<3>(x, p[6], p[7], sc);
    d[w] = x;
    if (!PNQ) {
      ps += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      // finish this dword's sum before the next dword's exponentials start:
      // left alone, the compiler runs all 32 exponentials first and spills
      asm volatile("" : "+v"(ps) : "v"(x));
    }
  }
  pk = make_uint4(d[0], d[1], d[2], d[3]);
  if (!PNQ) lpart = lpart * alpha + ps;
  return moved;
}

}  // namespace

template <int D, int MODE, bool PNQ, bool QBF16, bool VARLEN>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(4))) void attn_fwd_kernel(AttnArgs a) {
  constexpr int DB = D / 32;      // 32-blocks along d in a Q/K row
  constexpr int CROW = D / 2;     // code bytes per Q/K row
  constexpr int NCT = D / 16;     // 16-channel tiles of O^T
  constexpr int NT = kWaves * 64;
  constexpr int KI = kBC * 4 / 64;  // wave-wide 16-byte fills per K tile
  constexpr int VI = D * 4 / 64;    // wave-wide 16-byte fills per V tile
  static_assert(KI % kWaves == 0 || kWaves % KI == 0, "fills split evenly over the waves");
  static_assert(VI % kWaves == 0 || kWaves % VI == 0, "fills split evenly over the waves");
  constexpr int KU = (KI + kWaves - 1) / kWaves, VU = (VI + kWaves - 1) / kWaves;  // fills per wave
  static_assert(QBF16 || !VARLEN, "varlen batches take bf16 Q");
  __shared__ TileLds lds0, lds1;

  // Tile order: workgroup w is dispatched to XCD w % 8.  Each XCD gets a
  // contiguous range of (head, query tile) pairs, so the workgroups resident
  // on one XCD stream the same head's K/V through that XCD's L2.
  const int w = blockIdx.x;
  const int lin = (w & 7) * a.per_xcd + (w >> 3);
  if (lin >= int64_t(a.BH) * a.ntq) return;
  const int64_t bh = lin / a.ntq;  // dense: batch * H + head; varlen: head
  int qt = lin % a.ntq;
  int N = a.N;
  int64_t qrow, orow0;
  int64_t krow0 = bh * int64_t(N);         // K code rows before this sequence
  int vcs = a.vcs;                          // V channel stride in blocks
  int64_t vblk0 = bh * int64_t(D) * vcs;    // V blocks before this head
  int vskip = 0;                            // V blocks of this head before this sequence
  if constexpr (VARLEN) {
    // query tile qt of the varlen batch -> (sequence s, tile within s); the
    // query-tile count is an upper bound, so trailing workgroups exit
    const int n = a.batch + 1;
    const int* row = a.vl;
    const int* qtile = a.vl + n;
    if (qt >= qtile[a.batch]) return;
    const int s = find_segment(qtile, a.batch, qt);
    const int tok0 = row[s];
    N = row[s + 1] - tok0;
    qt -= qtile[s];
    qrow = tok0 * a.q_sn + bh * a.q_sh;
    orow0 = tok0 * a.o_sn + bh * a.o_sh;
    krow0 = bh * int64_t(a.kts) + tok0;
    // V rows hold exactly the blocks of all sequences, blk[batch] per
    // channel, so every block a tile reads past its sequence's last one is
    // data the quantizer wrote (the next sequence's, or the next channel's)
    vcs = a.vl[3 * n + a.batch];
    vskip = a.vl[3 * n + s];
    vblk0 = bh * int64_t(D) * vcs + vskip;
  } else {
    const int64_t hb = bh / a.H, hh = bh % a.H;
    qrow = hb * a.q_sb + hh * a.q_sh;
    orow0 = hb * a.o_sb + hh * a.o_sh;
  }

  // wave index through readfirstlane: the compiler then keeps everything
  // derived from it (LDS fill destinations) in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  const float c = a.c;

  // Q^T operand slices: query r16 of group g, d-block g4.  With bf16 Q the
  // lane quantizes its own 32-element block here (the same rule and encoder
  // as the stand-alone quantizer, so the codes are identical).
  uint4 qB[kQG];
  int qS[kQG];
#pragma unroll
  for (int g = 0; g < kQG; ++g) {
    const int qi = qt * kBR + wave * (kQG * 16) + g * 16 + r16;
    qB[g] = make_uint4(0, 0, 0, 0);
    qS[g] = 127;
    if (qi < N && g4 < DB) {
      const int64_t row = bh * N + qi;
      if constexpr (QBF16) {
        const uint4* src = reinterpret_cast<const uint4*>(a.q + qrow + qi * a.q_sn + 32 * g4);
        const uint4 x0 = src[0], x1 = src[1], x2 = src[2], x3 = src[3];
        const uint32_t amax = max(max(absmax8_bits(x0), absmax8_bits(x1)), max(absmax8_bits(x2), absmax8_bits(x3)));
        const int e = block_exp_bf16bits<MODE>(amax);
        qB[g] = make_uint4(encode8_bf16(x0, e), encode8_bf16(x1, e), encode8_bf16(x2, e), encode8_bf16(x3, e));
        qS[g] = e + 127;
      } else {
        qB[g] = *reinterpret_cast<const uint4*>(a.qc + row * CROW + 16 * g4);
        qS[g] = a.qs[row * DB + g4];
      }
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
  const int k_row0 = 32 * (r16 >> 2) + (r16 & 3);
  const int k_lane = k_row0 * 64 + 16 * (g4 ^ k_swz(k_row0));
  const int v_lane = r16 * 64 + 16 * (g4 ^ v_swz(r16));
  const int s_lane = lane * 8;

  const int ntk = (N + kBC - 1) / kBC;
  const uint8_t* kc_h = wave_uniform(a.kc + krow0 * CROW);
  const uint8_t* ks_h = wave_uniform(a.ks + krow0 * DB);
  const uint8_t* vc_h = wave_uniform(a.vc + vblk0 * 16);
  const uint8_t* vs_h = wave_uniform(a.vs + vblk0);

  // Tile fetch.  Code chunks go straight from global memory into LDS (lane i
  // of a wave writes the 16 bytes at dst + 16 i), so the swizzle is applied on
  // the source side: LDS slot s of the K tile holds (row s/4, chunk
  // (s%4) ^ swizzle(row)).  Scale bytes take a register detour.
  // Per-thread fill offsets (bytes from the tile's base in global memory).
  int koff[KU], voff[VU];
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    const int slot = (wave + u * kWaves) * 64 + lane;
    const int row = slot >> 2;
    koff[u] = row * CROW + 16 * (((slot & 3) ^ k_swz(row)) % (CROW / 16));
  }
#pragma unroll
  for (int u = 0; u < VU; ++u) {
    const int slot = (wave + u * kWaves) * 64 + lane;
    const int row = slot >> 2;
    voff[u] = (row * vcs + ((slot & 3) ^ v_swz(row))) * 16;
  }
  // Scale staging.  Thread tid < kBC carries the DB scale bytes of key kb + tid
  // (one load); the 4 D V scale bytes of the tile (item it: channel it % D,
  // block it / D) go VB per thread, items tid + NT v.  Both go to the
  // lane-ordered layout: byte b of key tid to ks[(16 b + r) * 8 + t], byte b
  // of channel 16 ct + r to vs[(16 b + r) * 8 + ct] (vs follows ks, so one
  // offset from ks serves both).
  static_assert(kBC <= NT, "one K scale word per thread");
  constexpr int VB = (4 * D + NT - 1) / NT;
  const int kdst = ((((tid >> 5) << 2) | (tid & 3)) * 8) + ((tid & 31) >> 2);
  // Threads with nothing to carry load from an offset past every record
  // count: the range check returns zero without touching memory, and every
  // thread runs the same instructions.
  const uint32_t kso = tid < kBC ? uint32_t(tid * DB) : 0x7FFFFFF0u;
  int vdst[VB];
  uint32_t vso[VB], vreg[VB];
#pragma unroll
  for (int v = 0; v < VB; ++v) {
    const int it = tid + NT * v, vch = it % D, vblk = it / D;
    vdst[v] = 64 * 8 + (vch & 15) * 8 + (vch >> 4) + 128 * vblk;
    vso[v] = it < 4 * D ? uint32_t(vch * vcs + vblk) : 0x7FFFFFF0u;
    vreg[v] = 0;
  }
  uint32_t kreg = 0;

  // Every fill is a raw buffer load whose descriptor starts at the tile's
  // first byte and whose record count is the bytes left in the head, so the
  // hardware range check returns zeros past the end.  K rows past N are zero
  // (and masked).  V code blocks and V scale bytes past the padded end of a
  // channel (or, in a varlen batch, of a sequence) read the next channel's
  // or sequence's finite data, which meets only zero weights.
  const int khead = __builtin_amdgcn_readfirstlane(N * CROW);
  const int vhead = __builtin_amdgcn_readfirstlane((D * vcs - vskip) * 16);
  const int kshead = __builtin_amdgcn_readfirstlane(N * DB);
  const int vshead = __builtin_amdgcn_readfirstlane(D * vcs - vskip);
  auto issue_tile = [&](int j, TileLds& T) {
    const int kb = j * kBC;
    const int vb0 = kb / 32;
    // scales first: the wait for them (at the end of the tile) then does not
    // cover the code fills issued after them
    const __amdgpu_buffer_rsrc_t ksrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(ks_h + int64_t(kb) * DB), 0, kshead - kb * DB, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vsrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vs_h + vb0), 0, vshead - vb0, kBufferFlags);
    if constexpr (DB == 4) kreg = __builtin_amdgcn_raw_buffer_load_b32(ksrs, kso, 0, 0);
    else kreg = __builtin_amdgcn_raw_buffer_load_b16(ksrs, kso, 0, 0);
#pragma unroll
    for (int v = 0; v < VB; ++v) vreg[v] = __builtin_amdgcn_raw_buffer_load_b8(vsrs, vso[v], 0, 0);
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kc_h + int64_t(kb) * CROW), 0, khead - kb * CROW, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vc_h + int64_t(vb0) * 16), 0, vhead - vb0 * 16, kBufferFlags);
#pragma unroll
    for (int u = 0; u < KU; ++u)
      if (KI % kWaves == 0 || wave + u * kWaves < KI)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_ptr)(T.k + (wave + u * kWaves) * 1024), 16,
                                                 uint32_t(koff[u]), 0, 0, 0);
#pragma unroll
    for (int u = 0; u < VU; ++u)
      if (VI % kWaves == 0 || wave + u * kWaves < VI)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_ptr)(T.v + (wave + u * kWaves) * 1024), 16,
                                                 uint32_t(voff[u]), 0, 0, 0);
  };
  auto finish_tile = [&](TileLds& T) {
    if (tid < kBC) {
#pragma unroll
      for (int b = 0; b < DB; ++b) T.ks[kdst + 128 * b] = uint8_t(kreg >> (8 * b));
    }
#pragma unroll
    for (int v = 0; v < VB; ++v)
      if (4 * D >= NT * (v + 1) || tid + NT * v < 4 * D) T.ks[vdst[v]] = uint8_t(vreg[v]);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's LDS fills have landed
  };


  // ---- one key tile: S^T, softmax step, l and O^T updates for every group ----
  auto compute_tile = [&](auto masked, int j, const TileLds& T) {
    constexpr bool MASKED = decltype(masked)::value;
    const int kb = j * kBC;
    uint2 ksw = make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
    if (g4 < DB) ksw = *reinterpret_cast<const uint2*>(&T.ks[s_lane]);
    v4f S[kQG][8];
#define MXATTN_S_STEP(t_)                                                                     \
    {                                                                                         \
      const uint4 kA = *reinterpret_cast<const uint4*>(&T.k[k_lane + 256 * (t_)]);            \
      _Pragma("unroll") for (int g = 0; g < kQG; ++g) S[g][t_] =                              \
          mfma_fp4_16x16x128<(t_) & 3, 0>(kA, qB[g], v4f{0.f, 0.f, 0.f, 0.f},                 \
                                          int((t_) < 4 ? ksw.x : ksw.y), qS[g]);               \
    }
    MXATTN_S_STEP(0) MXATTN_S_STEP(1) MXATTN_S_STEP(2) MXATTN_S_STEP(3)
    MXATTN_S_STEP(4) MXATTN_S_STEP(5) MXATTN_S_STEP(6) MXATTN_S_STEP(7)
#undef MXATTN_S_STEP
    if constexpr (MASKED) {
      // keys past N (the last tile only): s = -inf, so p = 0
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
    }
    uint4 pk[kQG];
    int pS[kQG];
#pragma unroll
    for (int g = 0; g < kQG; ++g) {
      float alpha;
      // the VALU-heavy part of the tile runs at raised wave priority, so a
      // SIMD prefers issuing it over waves that sit in their MFMA phases
      __builtin_amdgcn_s_setprio(1);
      const bool moved = softmax_group<MODE, PNQ>(S[g], m[g], c, pk[g], pS[g], alpha, lpart[g]);
      __builtin_amdgcn_s_setprio(0);
      if (moved) {  // rescale only when some running max moved
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) O[g][ct] *= alpha;
        if (PNQ) L[g][0] *= alpha;  // the four entries are equal; only [0] is read
      }
    }
    if (PNQ) {
#pragma unroll
      for (int g = 0; g < kQG; ++g) L[g] = mfma_fp4_16x16x128(ones, pk[g], L[g], 127, pS[g]);
    }
    const uint2 vsw = *reinterpret_cast<const uint2*>(&T.vs[s_lane]);
#define MXATTN_PV_STEP(ct_)                                                                   \
    if ((ct_) < NCT) {                                                                        \
      const uint4 vA = *reinterpret_cast<const uint4*>(&T.v[v_lane + 1024 * (ct_)]);          \
      _Pragma("unroll") for (int g = 0; g < kQG; ++g) O[g][(ct_) % NCT] =                     \
          mfma_fp4_16x16x128<(ct_) & 3, 0>(vA, pk[g], O[g][(ct_) % NCT],                      \
                                           int((ct_) < 4 ? vsw.x : vsw.y), pS[g]);             \
    }
    MXATTN_PV_STEP(0) MXATTN_PV_STEP(1) MXATTN_PV_STEP(2) MXATTN_PV_STEP(3)
    MXATTN_PV_STEP(4) MXATTN_PV_STEP(5) MXATTN_PV_STEP(6) MXATTN_PV_STEP(7)
#undef MXATTN_PV_STEP
    // An empty asm statement that reads the FP4 operands: without it the
    // compiler sinks the exponentials and converts below the end-of-tile
    // barrier, and the wait for the next tile's fills comes mid-tile.
#pragma unroll
    for (int g = 0; g < kQG; ++g) asm volatile("" ::"v"(pk[g].x), "v"(pk[g].y), "v"(pk[g].z), "v"(pk[g].w));
    // The same for the P.V MFMAs: kept above the barrier, their V operands
    // are read and consumed inside the tile instead of living across the
    // barrier next to the next tile's scores (100 VGPRs instead of 108).
#pragma unroll
    for (int g = 0; g < kQG; ++g)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) asm volatile("" : "+v"(O[g][ct]));
  };

  // ---- tile loop over two LDS buffers ----
  // Tile j+1 streams into the other buffer while tile j is used; one barrier
  // per tile publishes it (and frees the buffer just read).  Unrolled by two
  // so every buffer address is a constant; the last one or two tiles run the
  // variant that masks keys past N (a no-op unless the tile is ragged).
  const std::integral_constant<bool, false> full_tile;
  const std::integral_constant<bool, true> ragged_tile;
  auto step = [&](auto masked, int j, const TileLds& cur, TileLds& nxt) {
    if (j + 1 < ntk) issue_tile(j + 1, nxt);
    compute_tile(masked, j, cur);
    if (j + 1 < ntk) {
      // keep the wait for the fills at the end of the tile, so they have the
      // whole tile's compute to land
      __builtin_amdgcn_sched_barrier(0);
      finish_tile(nxt);
      __syncthreads();
    }
  };
  issue_tile(0, lds0);
  finish_tile(lds0);
  __syncthreads();
  int j = 0;
  for (; j + 2 < ntk; j += 2) {
    step(full_tile, j, lds0, lds1);
    step(full_tile, j + 1, lds1, lds0);
  }
  step(ragged_tile, j, lds0, lds1);
  if (j + 1 < ntk) step(ragged_tile, j + 1, lds1, lds0);

  // ---- epilogue: O / l -> bf16 ----
#pragma unroll
  for (int g = 0; g < kQG; ++g) {
    const float l = PNQ ? L[g][0] : sum_over_blocks(lpart[g]);
    const float inv = 1.0f / l;
    const int qi = qt * kBR + wave * (kQG * 16) + g * 16 + r16;
    if (qi < N) {
      uint16_t* orow = a.o + orow0 + qi * a.o_sn;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const uint32_t b0 = f32_to_bf16_rne(O[g][ct][0] * inv), b1 = f32_to_bf16_rne(O[g][ct][1] * inv);
        const uint32_t b2 = f32_to_bf16_rne(O[g][ct][2] * inv), b3 = f32_to_bf16_rne(O[g][ct][3] * inv);
        *reinterpret_cast<uint2*>(orow + 16 * ct + 4 * g4) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
      }
    }
  }
}

namespace {

template <int D, int MODE, bool PNQ>
void launch_variant(const AttnArgs& a, dim3 grid, bool qbf16, bool varlen, hipStream_t stream) {
  const dim3 block(kWaves * 64);
  if (varlen) attn_fwd_kernel<D, MODE, PNQ, true, true><<<grid, block, 0, stream>>>(a);
  else if (qbf16) attn_fwd_kernel<D, MODE, PNQ, true, false><<<grid, block, 0, stream>>>(a);
  else attn_fwd_kernel<D, MODE, PNQ, false, false><<<grid, block, 0, stream>>>(a);
}

hipError_t launch(AttnArgs& a, int d, int mode, bool pnq, bool varlen, float softmax_scale, hipStream_t stream) {
  const int64_t total = int64_t(a.BH) * a.ntq;  // fits an int: the ABI checks it
  a.per_xcd = int((total + 7) / 8);
  a.c = softmax_scale * 1.4426950408889634f;
  const dim3 grid(unsigned(a.per_xcd * 8));
  const bool qbf16 = a.q != nullptr;
  if (d == 128) {
    if (mode == kModeUOS) {
      if (pnq) launch_variant<128, kModeUOS, true>(a, grid, qbf16, varlen, stream);
      else launch_variant<128, kModeUOS, false>(a, grid, qbf16, varlen, stream);
    } else {
      if (pnq) launch_variant<128, kModeOCP, true>(a, grid, qbf16, varlen, stream);
      else launch_variant<128, kModeOCP, false>(a, grid, qbf16, varlen, stream);
    }
  } else {
    if (mode == kModeUOS) {
      if (pnq) launch_variant<64, kModeUOS, true>(a, grid, qbf16, varlen, stream);
      else launch_variant<64, kModeUOS, false>(a, grid, qbf16, varlen, stream);
    } else {
      if (pnq) launch_variant<64, kModeOCP, true>(a, grid, qbf16, varlen, stream);
      else launch_variant<64, kModeOCP, false>(a, grid, qbf16, varlen, stream);
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const uint16_t* q, const int64_t* q_strides, const uint8_t* qc, const uint8_t* qs,
                            const uint8_t* kc, const uint8_t* ks, const uint8_t* vc, const uint8_t* vs, int H,
                            int BH, int N, int d, int mode, bool pnq, float softmax_scale, uint16_t* o,
                            const int64_t* o_strides, hipStream_t stream) {
  AttnArgs a{};
  a.q = q; a.qc = qc; a.qs = qs; a.kc = kc; a.ks = ks; a.vc = vc; a.vs = vs; a.o = o;
  // null strides: dense [B][H][N][d]
  const int64_t dense[3] = {int64_t(H) * N * d, int64_t(N) * d, d};
  const int64_t* qst = q_strides ? q_strides : dense;
  const int64_t* ost = o_strides ? o_strides : dense;
  a.q_sb = qst[0]; a.q_sh = qst[1]; a.q_sn = qst[2];
  a.o_sb = ost[0]; a.o_sh = ost[1]; a.o_sn = ost[2];
  a.H = H;
  a.BH = BH;
  a.N = N;
  a.vcs = (N + 31) / 32;
  a.ntq = (N + kBR - 1) / kBR;
  return launch(a, d, mode, pnq, false, softmax_scale, stream);
}

// Varlen batch: bf16 Q and O with token stride q_sn / o_sn and head stride
// q_sh / o_sh (elements); K codes [H][T][d/2] (+ scales [H][T][d/32]); V codes
// [H][d][B * 16] (+ scales [H][d][B]) with B = tab.blk[batch], the blocks of
// all sequences, and sequence s in blocks tab.blk[s] ..; tab the varlen table
// of `batch` sequences over T tokens.
hipError_t launch_attention_varlen(const uint16_t* q, int64_t q_sn, int64_t q_sh, const uint8_t* kc,
                                   const uint8_t* ks, const uint8_t* vc, const uint8_t* vs, const int* tab,
                                   int batch, int T, int H, int d, int mode, bool pnq, float softmax_scale,
                                   uint16_t* o, int64_t o_sn, int64_t o_sh, hipStream_t stream) {
  AttnArgs a{};
  a.q = q; a.kc = kc; a.ks = ks; a.vc = vc; a.vs = vs; a.o = o;
  a.q_sn = q_sn; a.q_sh = q_sh; a.o_sn = o_sn; a.o_sh = o_sh;
  a.H = H;
  a.BH = H;
  a.ntq = (T + kBR - 1) / kBR + batch;  // at least the query tiles of all sequences
  a.vl = tab;
  a.batch = batch;
  a.kts = T;
  return launch(a, d, mode, pnq, true, softmax_scale, stream);
}

}  // namespace mxattn
