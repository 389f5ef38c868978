// gemm.hip -- MXFP4 GEMM for gfx950: Y = X W^T.
//
// MXAttention (arXiv 2607.24377), abstract: UOS picks MXFP4 block scales from
// a fixed, data-free boundary (Qmax = 7.25), so the same quantizer serves any
// MXFP4 contraction, not only attention.  Here X [M][K] (activations) and
// W [N][K] (weights) are both quantized along K in the canonical layout of
// mxq_quantize (codes [rows][K/2], scales [rows][K/32]); the products run on
// the scaled FP4 MFMA with fp32 accumulation and Y is rounded to bf16.
//
// Kernel structure: one workgroup computes a 256 x 256 tile of Y with 8 waves
// (4 along M x 2 along N, 64 x 128 each) at two waves per SIMD.  K advances
// 256 at a time: the W and X code tiles of the next step stream from global
// memory straight into the other half of a double-buffered LDS while the
// current step runs 64 MFMAs per wave, and one barrier per step publishes it.
// The MFMA computes Y^T tiles (A = 16 rows of W, B = 16 rows of X), so each
// lane ends up with four consecutive n of one m; the bf16 tile goes through
// LDS so that Y is written in whole 512-byte rows.
//
// QKV epilogue (the projection that feeds attention): Y's columns are
// [Q | K | V], each H * hd wide.  The tile goes through LDS as bf16, and the
// workgroup writes Q as bf16 [H][M][hd], K quantized along hd (codes
// [H][M][hd/2], scales [H][M][hd/32]) and V quantized along M (codes
// [H][hd][ceil(M/32) * 16], scales [H][hd][ceil(M/32)]): the operand layouts
// of the attention kernel, so K and V never exist in bf16 in memory.  K and V
// are rounded to bf16 first and quantized with the same rule and encoder as
// mxq_quantize, so the codes equal those of the unfused path.
#include <type_traits>

#include "mx_device.h"

namespace mxattn {

struct GemmArgs {
  const uint8_t* xc;  // X codes [M][K/2], scales [M][K/32]
  const uint8_t* xs;
  const uint8_t* wc;  // W codes [N][K/2], scales [N][K/32]
  const uint8_t* ws;
  uint16_t* y;        // bf16 [M][N]
  int M, N, K;
  int tn;             // tiles along N
  int ntiles;         // tiles in all
  int per_xcd;        // workgroups per XCD in the tile order below
  // QKV epilogue only (N = 3 H hd, M = tokens of one sequence)
  uint16_t* q;        // bf16 [H][M][hd]
  uint8_t* kc;        // [H][M][hd/2]
  uint8_t* ks;        // [H][M][hd/32]
  uint8_t* vc;        // [H][hd][nbm * 16]
  uint8_t* vs;        // [H][hd][nbm]
  int H, hd, nbm;     // heads, head dim, ceil(M / 32)
};

constexpr int kGM = 256, kGN = 256;  // workgroup tile
constexpr int kGK = 256;             // K per step: two 128-deep MFMA chunks
constexpr int kGWaves = 8;

namespace {

// LDS of one K step.  Codes: row-major, 128 bytes per row (two 64-byte
// chunks of 128 K, one per MFMA depth); the eight 16-byte pieces of a row
// are XOR-swizzled by the row (piece p at slot p ^ gswz(row % 16)).  The
// operand reads (lane l: row 16t + l % 16, piece 4h + l / 16) are served by
// ds_read_b128 in four groups of 16 lanes, which must hit 16 different
// 16-byte bank slots; a sweep of SQ_LDS_BANK_CONFLICT over XOR swizzles of
// this shape on gfx950 fits the groups (l2 ^ l3 ^ l4, l5) of the lane's bits,
// and this swizzle is conflict-free for every grouping the sweep allows.  On
// the FFN-shape GEMM it cut SQ_LDS_BANK_CONFLICT by 75% (the rest is the
// scale staging).  Scales: lane order,
// sl[h][(g * 16 + r) * 16 + t] = scale of row 16t + r, block g of chunk h.
struct __align__(16) GemmLds {
  uint8_t w[kGN * 128];
  uint8_t x[kGM * 128];
  uint8_t wsl[2][64 * 16];
  uint8_t xsl[2][64 * 16];
};

__device__ __forceinline__ int gswz(int row) { return (row & 1) | ((row >> 1) & 2) | ((row << 1) & 4); }

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef unsigned v4u __attribute__((ext_vector_type(4)));
constexpr int kBufferFlags = 0x00020000;  // raw buffer, 32-bit format, range checked

__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<const uint8_t*>((uint64_t(hi) << 32) | lo);
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

}  // namespace

namespace {

// Byte address of bf16 element (r, n) of the 256 x 256 epilogue tile, which
// reuses both operand buffers: rows 0-127 in t0, 128-255 in t1, 512 bytes per
// row, 16-byte chunk c of row r stored at chunk c ^ (r & 31) (the 32 lanes
// that read one chunk of 32 consecutive rows then spread over the banks).
__device__ __forceinline__ uint8_t* tile_elem(uint8_t* t0, uint8_t* t1, int r, int n) {
  return (r < 128 ? t0 : t1) + (r & 127) * 512 + (((n >> 3) ^ (r & 31)) << 4) + (n & 7) * 2;
}

template <int MODE>
__device__ __forceinline__ void qkv_epilogue(const GemmArgs& a, const v4f (&acc)[8][4], GemmLds& lds0,
                                             GemmLds& lds1, int m0, int n0, int wm, int wn, int wave,
                                             int lane) {
  const int r16 = lane & 15, g4 = lane >> 4;
  uint8_t* t0 = reinterpret_cast<uint8_t*>(&lds0);
  uint8_t* t1 = reinterpret_cast<uint8_t*>(&lds1);
  __syncthreads();  // every wave has finished reading the operand tiles
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 64 * wm + 16 * i + r16;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int n = 128 * wn + 16 * j + 4 * g4;
      const uint32_t b0 = f32_to_bf16_rne(acc[j][i][0]), b1 = f32_to_bf16_rne(acc[j][i][1]);
      const uint32_t b2 = f32_to_bf16_rne(acc[j][i][2]), b3 = f32_to_bf16_rne(acc[j][i][3]);
      *reinterpret_cast<uint2*>(tile_elem(t0, t1, r, n)) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
    }
  }
  __syncthreads();
  const int HD = a.H * a.hd, M = a.M;
  const int region0 = n0 / HD, region1 = (min(n0 + kGN, a.N) - 1) / HD;
  if (region0 == region1 && region0 == 0) {
    // A tile of Q only: whole tile rows, 32 lanes x 16 bytes each, two rows
    // per instruction (a 16-byte chunk never straddles a head: hd % 8 == 0)
    const int cc = lane & 31, n = n0 + 8 * cc;
    const int h = n / a.hd, c0 = n - h * a.hd;
#pragma unroll 4
    for (int k = 0; k < 16; ++k) {
      const int r = 32 * wave + 2 * k + (lane >> 5), m = m0 + r;
      if (m >= M || n >= a.N) continue;
      const v4u v = *reinterpret_cast<const v4u*>(tile_elem(t0, t1, r, 8 * cc));
      __builtin_nontemporal_store(v, reinterpret_cast<v4u*>(a.q + (int64_t(h) * M + m) * a.hd + c0));
    }
    return;
  }
  if (region0 == region1 && region0 == 1) {
    // A tile of K only: one 32-value block per lane, eight rows of eight
    // blocks per instruction, so the lanes of one head's row write its code
    // bytes contiguously
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int idx = (4 * wave + it) * 64 + lane, r = idx >> 3, b = idx & 7;
      const int m = m0 + r, n = n0 + 32 * b;
      uint4 v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = *reinterpret_cast<const uint4*>(tile_elem(t0, t1, r, 32 * b + 8 * q));
      const uint32_t amax = max(max(absmax8_bits(v[0]), absmax8_bits(v[1])), max(absmax8_bits(v[2]), absmax8_bits(v[3])));
      const int e = block_exp_bf16bits<MODE>(amax);
      if (m < M && n < a.N) {
        const int nn = n - HD, h = nn / a.hd, c0 = nn - h * a.hd;
        const int64_t row = int64_t(h) * M + m;
        *reinterpret_cast<uint4*>(a.kc + row * (a.hd / 2) + c0 / 2) =
            make_uint4(encode8_bf16(v[0], e), encode8_bf16(v[1], e), encode8_bf16(v[2], e), encode8_bf16(v[3], e));
        a.ks[row * (a.hd / 32) + c0 / 32] = uint8_t(e + 127);
      }
    }
    return;
  }
  // Otherwise (V, or a tile that straddles regions): 64 cells of 32 rows x
  // 32 columns; a cell lies inside one head of one of Q, K, V (H hd is a
  // multiple of 32).  Rows past M hold zeros (their X rows read as zero),
  // which is the padding of V's last block.
  for (int cell = wave; cell < 64; cell += kGWaves) {
    const int cg = cell & 7, rg = cell >> 3;
    const int n = n0 + 32 * cg;
    if (n >= a.N) continue;
    const int region = n / HD, nn = n - region * HD;
    const int h = nn / a.hd, c0 = nn - h * a.hd;
    const int rl = 32 * rg, m = m0 + rl;
    if (region == 0 || region == 1) {
      // Q rows, or one K block per row: two lanes per row, 16 columns each
      const int r = lane >> 1, half = lane & 1;
      const uint4 v0 = *reinterpret_cast<const uint4*>(tile_elem(t0, t1, rl + r, 32 * cg + 16 * half));
      const uint4 v1 = *reinterpret_cast<const uint4*>(tile_elem(t0, t1, rl + r, 32 * cg + 16 * half + 8));
      const int64_t row = int64_t(h) * M + m + r;
      if (region == 0) {
        if (m + r < M) {
          uint4* dst = reinterpret_cast<uint4*>(a.q + row * a.hd + c0 + 16 * half);
          dst[0] = v0;
          dst[1] = v1;
        }
      } else {
        uint32_t amax = max(absmax8_bits(v0), absmax8_bits(v1));
        amax = max(amax, uint32_t(__builtin_amdgcn_mov_dpp(int(amax), 0xB1, 0xF, 0xF, true)));  // partner lane
        const int e = block_exp_bf16bits<MODE>(amax);
        const uint2 c = make_uint2(encode8_bf16(v0, e), encode8_bf16(v1, e));
        if (m + r < M) {
          *reinterpret_cast<uint2*>(a.kc + row * (a.hd / 2) + c0 / 2 + 8 * half) = c;
          if (half == 0) a.ks[row * (a.hd / 32) + c0 / 32] = uint8_t(e + 127);
        }
      }
    } else {
      // one V block per column: lanes col and col + 32 take rows 0-15 and
      // 16-31 of the block
      const int col = lane & 31, half = lane >> 5;
      uint32_t w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t lo = *reinterpret_cast<const uint16_t*>(tile_elem(t0, t1, rl + 16 * half + 2 * i, 32 * cg + col));
        const uint32_t hi = *reinterpret_cast<const uint16_t*>(tile_elem(t0, t1, rl + 16 * half + 2 * i + 1, 32 * cg + col));
        w[i] = lo | (hi << 16);
      }
      const uint4 v0 = make_uint4(w[0], w[1], w[2], w[3]), v1 = make_uint4(w[4], w[5], w[6], w[7]);
      uint32_t amax = max(absmax8_bits(v0), absmax8_bits(v1));
      amax = max(amax, uint32_t(__shfl_xor(int(amax), 32)));
      const int e = block_exp_bf16bits<MODE>(amax);
      const uint2 c = make_uint2(encode8_bf16(v0, e), encode8_bf16(v1, e));
      const int mb = m / 32;
      if (mb < a.nbm) {
        const int64_t vrow = int64_t(h) * a.hd + c0 + col;
        *reinterpret_cast<uint2*>(a.vc + (vrow * a.nbm + mb) * 16 + 8 * half) = c;
        if (half == 0) a.vs[vrow * a.nbm + mb] = uint8_t(e + 127);
      }
    }
  }
}

}  // namespace

// EPI 0: Y in bf16; EPI 1: the QKV epilogue with block rule MODE.
template <int EPI, int MODE>
__global__ __launch_bounds__(kGWaves * 64) __attribute__((amdgpu_waves_per_eu(2))) void gemm_kernel(GemmArgs a) {
  constexpr int NT = kGWaves * 64;
  // two separate objects (not an array): the compiler then knows that the
  // fills into one buffer cannot alias the operand reads from the other
  __shared__ GemmLds lds0, lds1;

  // Tile order: workgroup w runs on XCD w % 8 and each XCD takes a
  // contiguous range of tiles.  Tiles come in groups of 8 M tiles:
  // consecutive tiles walk the 8 M tiles of a group for one N tile, so the
  // tiles in flight on an XCD share X rows and W rows through its L2.
  //
  // The plain GEMM runs a persistent grid (one workgroup per CU, see
  // persistent_grid): a workgroup walks the tiles lt, lt + slots, ... of its
  // XCD's range.  With an even number of K steps the last step computes from
  // lds1, so the next tile's first fills go into lds0 before this tile's last
  // MFMAs and its epilogue (which then stages Y through lds1 alone, in two
  // halves): they land while Y is written.  The QKV projection runs one tile
  // per workgroup.
  const int w = blockIdx.x;
  const int nslot = gridDim.x >> 3;  // workgroups per XCD (the grid is a multiple of 8)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  const int wm = wave & 3, wn = wave >> 2;  // wave tile: rows 64 wm of X, rows 128 wn of W
  const int K = a.K, KC = K / 2, KS = K / 32;
  const int nsteps = (K + kGK - 1) / kGK;
  const int tmc = a.ntiles / a.tn;
  const int gsz = 8 * a.tn;

  // operand sources of tile `lin`
  struct Src {
    const uint8_t *xc, *wc, *xs, *ws;
    int xcb, wcb, xsb, wsb;
    int m0, n0;
  };
  auto src_of = [&](int lin) {
    const int gid = lin / gsz, rr = lin % gsz;
    const int gm = min(8, tmc - 8 * gid);
    Src t;
    t.m0 = __builtin_amdgcn_readfirstlane((8 * gid + rr % gm) * kGM);
    t.n0 = __builtin_amdgcn_readfirstlane((rr / gm) * kGN);
    t.xc = uniform_ptr(a.xc + int64_t(t.m0) * KC);
    t.wc = uniform_ptr(a.wc + int64_t(t.n0) * KC);
    t.xs = uniform_ptr(a.xs + int64_t(t.m0) * KS);
    t.ws = uniform_ptr(a.ws + int64_t(t.n0) * KS);
    t.xcb = __builtin_amdgcn_readfirstlane((a.M - t.m0) * KC);
    t.wcb = __builtin_amdgcn_readfirstlane((a.N - t.n0) * KC);
    t.xsb = __builtin_amdgcn_readfirstlane((a.M - t.m0) * KS);
    t.wsb = __builtin_amdgcn_readfirstlane((a.N - t.n0) * KS);
    return t;
  };
  int lt = w >> 3;
  bool prefetched = false;  // the previous tile already issued this tile's first fills into lds0
  uint32_t sreg0 = 0, sreg1 = 0;
  do {
  const int lin = (w & 7) * a.per_xcd + lt;
  if (lin >= a.ntiles) break;
  const Src cur_src = src_of(lin);
  const int m0 = cur_src.m0, n0 = cur_src.n0;

  // Code fills: 256 rows x 128 bytes per operand = 2048 16-byte pieces, four
  // per thread per operand.  Slot s = (wave + 8u) * 64 + lane of the region
  // holds row s / 8, piece (s % 8) ^ gswz(row % 16) of that row (pieces
  // 0-3: the first 128 K of the step, 4-7: the second).  Rows past M or N
  // read as zero through the descriptor's range check.
  uint32_t foff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int s = (wave + kGWaves * u) * 64 + lane;
    const int row = s >> 3, piece = (s & 7) ^ gswz(row & 15);
    foff[u] = uint32_t(row * KC + piece * 16);
  }
  // Scale staging: thread tid < 256 carries the 8 scale bytes (blocks of the
  // step) of W row tid, the others those of X row tid - 256.
  const int srow = tid & 255;
  const uint32_t soff = uint32_t(srow * KS);
  const int sdst = ((srow & 15) * 16) + (srow >> 4);  // + (g * 16) * 16 per block g

  auto issue_from = [&](const Src& src, int step, GemmLds& T) {
    const int kb = step * kGK;
    const int sb = __builtin_amdgcn_readfirstlane(kb / 32);
    // waves 0-3 (threads 0-255) stage W scales, waves 4-7 X scales: the
    // choice is wave-uniform, so the descriptor stays scalar
    const __amdgpu_buffer_rsrc_t srs = wave < 4
        ? __builtin_amdgcn_make_buffer_rsrc((void*)(src.ws + sb), 0, src.wsb - sb, kBufferFlags)
        : __builtin_amdgcn_make_buffer_rsrc((void*)(src.xs + sb), 0, src.xsb - sb, kBufferFlags);
    sreg0 = __builtin_amdgcn_raw_buffer_load_b32(srs, soff, 0, 0);
    sreg1 = __builtin_amdgcn_raw_buffer_load_b32(srs, soff + 4, 0, 0);
    const int cb = __builtin_amdgcn_readfirstlane(kb / 2);
    const __amdgpu_buffer_rsrc_t wrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(src.wc + cb), 0, src.wcb - cb, kBufferFlags);
    const __amdgpu_buffer_rsrc_t xrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(src.xc + cb), 0, src.xcb - cb, kBufferFlags);
    // (wave & 7): a provably small offset lets the compiler see that these
    // fills stay inside T and cannot alias reads of the other buffer
#pragma unroll
    for (int u = 0; u < 4; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (lds_ptr)(T.w + ((wave & 7) + kGWaves * u) * 1024), 16, foff[u], 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (lds_ptr)(T.x + ((wave & 7) + kGWaves * u) * 1024), 16, foff[u], 0, 0, 0);
  };
  auto issue = [&](int step, GemmLds& T) { issue_from(cur_src, step, T); };
  auto finish = [&](GemmLds& T) {
    uint8_t* sl = wave < 4 ? &T.wsl[0][0] : &T.xsl[0][0];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint32_t v = b < 4 ? sreg0 : sreg1;
      sl[(b >> 2) * 1024 + (b & 3) * 256 + sdst] = uint8_t(v >> (8 * (b & 3)));
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's LDS fills have landed
  };

  v4f acc[8][4];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[j][i] = v4f{0.f, 0.f, 0.f, 0.f};

  // per-lane LDS offsets: operand row 16t + r16, piece 4h + g4
  const int lsw = gswz(r16);
  const int w_off0 = (128 * wn + r16) * 128 + 16 * (g4 ^ lsw), w_off1 = (128 * wn + r16) * 128 + 16 * ((4 + g4) ^ lsw);
  const int x_off0 = (64 * wm + r16) * 128 + 16 * (g4 ^ lsw), x_off1 = (64 * wm + r16) * 128 + 16 * ((4 + g4) ^ lsw);
  const int ws_lane = (g4 * 16 + r16) * 16 + 8 * wn;
  const int xs_lane = (g4 * 16 + r16) * 16 + 4 * wm;

  auto compute = [&](const GemmLds& T, auto nchunks) {
    constexpr int NCH = decltype(nchunks)::value;
#pragma unroll
    for (int h = 0; h < NCH; ++h) {
      const uint2 wsc = *reinterpret_cast<const uint2*>(&T.wsl[h][ws_lane]);
      const uint32_t xsc = *reinterpret_cast<const uint32_t*>(&T.xsl[h][xs_lane]);
      uint4 xb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xb[i] = *reinterpret_cast<const uint4*>(&T.x[(h ? x_off1 : x_off0) + i * 16 * 128]);
#define MXGEMM_ROW(j_)                                                                             \
      {                                                                                            \
        const uint4 wa = *reinterpret_cast<const uint4*>(&T.w[(h ? w_off1 : w_off0) + (j_) * 16 * 128]); \
        const int sa = int((j_) < 4 ? wsc.x : wsc.y);                                             \
        acc[j_][0] = mfma_fp4_16x16x128<(j_) & 3, 0>(wa, xb[0], acc[j_][0], sa, int(xsc));         \
        acc[j_][1] = mfma_fp4_16x16x128<(j_) & 3, 1>(wa, xb[1], acc[j_][1], sa, int(xsc));         \
        acc[j_][2] = mfma_fp4_16x16x128<(j_) & 3, 2>(wa, xb[2], acc[j_][2], sa, int(xsc));         \
        acc[j_][3] = mfma_fp4_16x16x128<(j_) & 3, 3>(wa, xb[3], acc[j_][3], sa, int(xsc));         \
      }
      // MFMA issue at raised wave priority: a SIMD prefers the wave that is
      // ready to feed the matrix core over one that is staging operands
      __builtin_amdgcn_s_setprio(1);
      MXGEMM_ROW(0) MXGEMM_ROW(1) MXGEMM_ROW(2) MXGEMM_ROW(3)
      MXGEMM_ROW(4) MXGEMM_ROW(5) MXGEMM_ROW(6) MXGEMM_ROW(7)
      // all 14 operand reads of the chunk first, then the 32 MFMAs: left to
      // itself the compiler cycles two W registers, so every second row of
      // MFMAs waits for a read issued only after the previous row
      __builtin_amdgcn_sched_group_barrier(0x100, 14, 0);  // DS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 32, 0);  // MFMAs
      __builtin_amdgcn_s_setprio(0);
#undef MXGEMM_ROW
    }
  };

  // K loop over two LDS buffers, unrolled by two so the buffers are constants.
  // Inside the loop every step has a successor, so its fills are issued with
  // no branch around them (a conditional fill makes the compiler wait for it
  // before the next operand reads); the last one or two steps follow.
  const bool half_last = (K % kGK) != 0;  // K % 256 == 128: the last step has one chunk
  const std::integral_constant<int, 1> one_chunk;
  const std::integral_constant<int, 2> two_chunks;
  auto step = [&](int s, const GemmLds& cur, GemmLds& nxt) {
    issue(s + 1, nxt);
    // keep the fills at the top of the step: they get the whole step to land
    __builtin_amdgcn_sched_barrier(0);
    compute(cur, two_chunks);
    __builtin_amdgcn_sched_barrier(0);
    finish(nxt);
    __syncthreads();
  };
  if (!prefetched) issue(0, lds0);
  finish(lds0);
  __syncthreads();
  int s = 0;
  for (; s + 2 < nsteps; s += 2) {
    step(s, lds0, lds1);
    step(s + 1, lds1, lds0);
  }
  const GemmLds* last = &lds0;
  if (s + 1 < nsteps) {
    step(s, lds0, lds1);
    last = &lds1;
  }
  // The next tile's first fills go out now, into lds0, when the last step
  // computes from lds1 (an even number of steps): lds0 is free, and the
  // fills land while this tile finishes and writes Y.
  const int lt_next = lt + nslot;
  const int lin_next = (w & 7) * a.per_xcd + lt_next;
  const bool pf = EPI == 0 && (nsteps & 1) == 0 && lt_next < a.per_xcd && lin_next < a.ntiles;
  if (pf) issue_from(src_of(lin_next), 0, lds0);
  if (half_last)
    compute(*last, one_chunk);
  else
    compute(*last, two_chunks);

  // epilogue: acc[j][i] is the Y^T tile of W rows 128 wn + 16 j and X rows
  // 64 wm + 16 i; lane: m = r16 of it, n = 4 g4 + [0, 4)
  if constexpr (EPI == 1) {
    qkv_epilogue<MODE>(a, acc, lds0, lds1, m0, n0, wm, wn, wave, lane);
    break;
  }
  // Y through LDS, in two halves through the last step's buffer (the other
  // one may hold the next tile's first fills): half h holds rows
  // 64 wm + 32 h + [0, 32) of every wave row, i.e. accumulators i = 2h, 2h+1,
  // as staged row 32 wm + 16 (i & 1) + r16.  Each wave then writes 16 whole
  // rows of the half, two per instruction (32 lanes x 16 bytes = one 512-byte
  // row), with nontemporal stores.
  uint8_t* tl = reinterpret_cast<uint8_t*>(const_cast<GemmLds*>(last));
  __syncthreads();  // every wave has finished reading the operand tiles
  const int cc = lane & 31, n = n0 + 8 * cc;
  const bool vec = (a.N & 7) == 0;  // 16-byte aligned rows
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (h) __syncthreads();  // the first half's rows have been read
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int i = 2 * h + ii;
      const int sr = 32 * wm + 16 * ii + r16;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int nn = 128 * wn + 16 * j + 4 * g4;
        const uint32_t b0 = f32_to_bf16_rne(acc[j][i][0]), b1 = f32_to_bf16_rne(acc[j][i][1]);
        const uint32_t b2 = f32_to_bf16_rne(acc[j][i][2]), b3 = f32_to_bf16_rne(acc[j][i][3]);
        *reinterpret_cast<uint2*>(tl + sr * 512 + (((nn >> 3) ^ (sr & 31)) << 4) + (nn & 7) * 2) =
            make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
      }
    }
    __syncthreads();
#pragma unroll 2
    for (int k = 0; k < 8; ++k) {
      const int sr = 16 * wave + 2 * k + (lane >> 5);
      const int m = m0 + 64 * (sr >> 5) + 32 * h + (sr & 31);
      if (m >= a.M || n >= a.N) continue;
      const v4u v = *reinterpret_cast<const v4u*>(tl + sr * 512 + ((cc ^ (sr & 31)) << 4));
      uint16_t* dst = a.y + int64_t(m) * a.N + n;
      if (vec) {
        __builtin_nontemporal_store(v, reinterpret_cast<v4u*>(dst));
      } else {
        for (int e = 0; e < 8 && n + e < a.N; ++e) dst[e] = uint16_t(v[e >> 1] >> (16 * (e & 1)));
      }
    }
  }
  // the next tile's barrier (after its first fills land) orders these reads
  // before the fills that reuse this buffer; without a prefetch its first
  // fills go to lds0 right away, so wait here
  if (!pf) __syncthreads();
  prefetched = pf;
  lt += nslot;
  } while (EPI == 0 && lt < a.per_xcd);
}

namespace {

// The plain GEMM's grid: one workgroup per CU (its LDS holds one), rounded
// down to a multiple of 8 so every XCD gets the same number of slots, and no
// more workgroups than tiles.  (On the DiT FFN shape, identical results:
// one workgroup per tile 1.34 ms, persistent 1.27 ms, persistent with the
// next tile's first fills issued before the epilogue 1.21-1.24 ms.)
int persistent_grid(const GemmArgs& a) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8) {
    (void)hipGetLastError();
    return a.per_xcd * 8;  // one workgroup per tile
  }
  const int g = (cus / 8) * 8;
  return g < a.per_xcd * 8 ? g : a.per_xcd * 8;
}

void set_tiles(GemmArgs& a) {
  const int tm = (a.M + kGM - 1) / kGM;
  a.tn = (a.N + kGN - 1) / kGN;
  a.ntiles = tm * a.tn;
  a.per_xcd = (a.ntiles + 7) / 8;
}

}  // namespace

hipError_t launch_gemm(const uint8_t* xc, const uint8_t* xs, const uint8_t* wc, const uint8_t* ws, int M,
                       int N, int K, uint16_t* y, hipStream_t stream) {
  GemmArgs a{};
  a.xc = xc; a.xs = xs; a.wc = wc; a.ws = ws; a.y = y;
  a.M = M; a.N = N; a.K = K;
  set_tiles(a);
  gemm_kernel<0, 0><<<dim3(unsigned(persistent_grid(a))), dim3(kGWaves * 64), 0, stream>>>(a);
  return hipGetLastError();
}

// The QKV projection of one sequence of M tokens with the QKV epilogue:
// W [3 H hd][K], outputs as in GemmArgs.
hipError_t launch_qkv_gemm(const uint8_t* xc, const uint8_t* xs, const uint8_t* wc, const uint8_t* ws, int M,
                           int K, int H, int hd, int mode, uint16_t* q, uint8_t* kc, uint8_t* ks, uint8_t* vc,
                           uint8_t* vs, hipStream_t stream) {
  GemmArgs a{};
  a.xc = xc; a.xs = xs; a.wc = wc; a.ws = ws;
  a.M = M; a.N = 3 * H * hd; a.K = K;
  a.q = q; a.kc = kc; a.ks = ks; a.vc = vc; a.vs = vs;
  a.H = H; a.hd = hd; a.nbm = (M + 31) / 32;
  set_tiles(a);
  const dim3 grid(unsigned(a.per_xcd * 8)), block(kGWaves * 64);
  if (mode == kModeUOS) gemm_kernel<1, kModeUOS><<<grid, block, 0, stream>>>(a);
  else gemm_kernel<1, kModeOCP><<<grid, block, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace mxattn
