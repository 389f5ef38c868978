// quantize.hip -- bf16 -> MXFP4 (E2M1 codes + E8M0 block scales) for gfx950.
//
// MXAttention (arXiv 2607.24377), abstract: MXFP4 with power-of-two block
// scales; OCP MXFP4 is the baseline rule, UOS the fixed boundary Qmax = 7.25.
// This pass is a streaming codec bound by HBM bandwidth: 2 bytes read and
// 0.5 + 1/32 bytes written per element.
//
// Encoding: for a block with exponent e, y = x / 2^e is rounded to the nearest
// E2M1 magnitude (ties to the even code, saturating at 6, sign kept); the
// block rule and the encoder (encode8) live in mx_device.h, shared with the
// attention kernel's in-kernel quantization of Q.
#include "mx_device.h"

namespace mxattn {

namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));

}  // namespace

// Where the batch entries and rows of a [batch][rows][cols] input sit when it
// is a strided view with contiguous columns: entry bi = (bi / H, bi % H)
// starts at sb * (bi / H) + sh * (bi % H) elements and its rows are sn apart.
// The dense layout is H = 1, sb = rows * cols, sn = cols.
struct Layout3 {
  int64_t H, sb, sh, sn;
  __device__ __forceinline__ int64_t base(int64_t bi) const { return (bi / H) * sb + (bi % H) * sh; }
};

// Flat stream of full 32-element blocks: block i = elements [32i, 32i + 32)
// of x, codes [16i, 16i + 16), scale [i].  Four lanes share a block (16 bytes
// of input each), so a wave reads 1 KiB and writes 256 code bytes per step,
// both contiguous.  nq = 4 * number of blocks.  Input and codes are touched
// once, so loads and stores carry the non-temporal hint (keeps them from
// displacing other data in the caches, and measurably faster here).
template <int MODE, int U>
__global__ __launch_bounds__(256) void quant_stream_kernel(const uint4* __restrict__ x,
                                                           uint32_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales,
                                                           int64_t nq) {
  const int64_t step = int64_t(gridDim.x) * 256 * U;
  for (int64_t base = int64_t(blockIdx.x) * 256 * U + threadIdx.x; base < nq; base += step) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t idx = base + int64_t(u) * 256;
      const v4u t = idx < nq ? __builtin_nontemporal_load(reinterpret_cast<const v4u*>(x) + idx) : v4u{0, 0, 0, 0};
      v[u] = make_uint4(t.x, t.y, t.z, t.w);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t idx = base + int64_t(u) * 256;
      uint32_t m = absmax8_bits(v[u]);
      // max over the 4 lanes of the quad: quad_perm [1,0,3,2] then [2,3,0,1]
      m = max(m, uint32_t(__builtin_amdgcn_mov_dpp(int(m), 0xB1, 0xF, 0xF, true)));
      m = max(m, uint32_t(__builtin_amdgcn_mov_dpp(int(m), 0x4E, 0xF, 0xF, true)));
      const int e = block_exp_bf16bits<MODE>(m);
      const uint32_t c = encode8_bf16(v[u], e);
      if (idx < nq) {
        __builtin_nontemporal_store(c, codes + idx);
        if ((idx & 3) == 0) scales[idx >> 2] = uint8_t(e + 127);
      }
    }
  }
}

// Blocks along the contiguous axis when cols is not a multiple of 32: one
// thread per block, element loads with bounds checks, zero padding.
template <int MODE>
__global__ __launch_bounds__(256) void quant_rows_general_kernel(const uint16_t* __restrict__ x,
                                                                 uint4* __restrict__ codes,
                                                                 uint8_t* __restrict__ scales,
                                                                 int64_t nvec, int64_t L, int64_t nb) {
  const int64_t b = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (b >= nvec * nb) return;
  const int64_t vec = b / nb, blk = b % nb;
  const uint16_t* src = x + vec * L + blk * 32;
  const int n = int(min(int64_t(32), L - blk * 32));
  float f[32];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t h = i < n ? uint32_t(src[i]) : 0u;
    m = max(m, h & 0x7FFFu);
    f[i] = __uint_as_float(h << 16);
  }
  const int e = block_exp_bf16bits<MODE>(m);
  uint4 c;
  c.x = encode8(f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[7], e);
  c.y = encode8(f[8], f[9], f[10], f[11], f[12], f[13], f[14], f[15], e);
  c.z = encode8(f[16], f[17], f[18], f[19], f[20], f[21], f[22], f[23], e);
  c.w = encode8(f[24], f[25], f[26], f[27], f[28], f[29], f[30], f[31], e);
  codes[b] = c;
  scales[b] = uint8_t(e + 127);
}

// Blocks along the contiguous axis of a strided view (cols % 32 == 0): batch
// entry blockIdx.y, 16-byte pieces of its rows walked with a grid stride
// along x, four lanes per block as in the stream kernel.
template <int MODE, int U>
__global__ __launch_bounds__(256) void quant_rows_strided_kernel(const uint16_t* __restrict__ x,
                                                                 uint32_t* __restrict__ codes,
                                                                 uint8_t* __restrict__ scales, int64_t rows,
                                                                 int64_t cols, Layout3 in) {
  const int64_t bi = blockIdx.y;
  const uint16_t* xb = x + in.base(bi);
  const uint32_t ppr = uint32_t(cols / 8);            // 16-byte pieces per row
  const uint32_t np = uint32_t(rows) * ppr;           // pieces in this entry
  const int64_t out0 = bi * int64_t(rows) * (cols / 8);  // code dwords before this entry
  const uint32_t step = gridDim.x * 256 * U;
  for (uint32_t base = blockIdx.x * 256 * U + threadIdx.x; base < np; base += step) {
    v4u v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t q = base + u * 256;
      const uint32_t r = q / ppr, pc = q - r * ppr;
      v[u] = q < np ? __builtin_nontemporal_load(reinterpret_cast<const v4u*>(xb + int64_t(r) * in.sn + pc * 8))
                    : v4u{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t q = base + u * 256;
      const uint4 w = make_uint4(v[u].x, v[u].y, v[u].z, v[u].w);
      uint32_t m = absmax8_bits(w);
      m = max(m, uint32_t(__builtin_amdgcn_mov_dpp(int(m), 0xB1, 0xF, 0xF, true)));
      m = max(m, uint32_t(__builtin_amdgcn_mov_dpp(int(m), 0x4E, 0xF, 0xF, true)));
      const int e = block_exp_bf16bits<MODE>(m);
      const uint32_t c = encode8_bf16(w, e);
      if (q < np) {
        __builtin_nontemporal_store(c, codes + out0 + q);
        if ((q & 3) == 0) scales[(out0 + q) >> 2] = uint8_t(e + 127);
      }
    }
  }
}

// Rows of a varlen input split into segments (sequences): segment s covers
// rows [row[s], row[s + 1]).  Its 256-row tiles are work tiles tile[s] ..
// tile[s + 1] - 1, and its 32-row blocks are output blocks blk[s] ..
// blk[s + 1] - 1 of every column, so blocks never straddle two segments and
// the last block of each segment is zero-padded.  All three arrays hold
// n + 1 prefix values (the varlen table, built on the device).
struct RowSegments {
  const int* row;
  const int* tile;
  const int* blk;
  int n;
};

// Blocks along rows (axis 0).  Work item = a 256-row x TC-column bf16 tile of
// one batch entry (TC = 128, or 64 for inputs at most 64 columns wide); each
// workgroup walks items with a grid stride and holds the next item's loads in
// registers while it encodes the current one from LDS.  Element (row r,
// column c) of a tile sits at tile[r * TC + (c ^ 8 (r / 32))], so the eight
// lanes that read one column of eight 32-row blocks hit eight different
// banks; eight consecutive lanes take the eight blocks of one column, so a
// wave writes whole 128-byte code lines.  Rows past the end are zero
// (padding).  Items run row tile first: consecutive items take consecutive
// 256-row tiles of the same columns, so the code lines the workgroups in
// flight write are adjacent lines of the same columns.  (Measured on the
// [2^18][1024] sweep input: 128-column tiles 55% -> 62% of HBM, row-first
// order 62% -> 63%; the Wan V shape, 128 columns, is unchanged at 63%.)
//
// SEG: the rows are the segments of `seg`; ntr is then the number of work
// tiles per entry (an upper bound on seg.tile[n]: items past it do nothing)
// and every column holds exactly the blocks of all segments, seg.blk[n]
// (vstride is ignored).  Otherwise ntr = ceil(rows / 256) and vstride = nb.
// Eight waves per workgroup (two workgroups, 16 waves, per CU): against four
// waves the encode of one tile is split over twice the waves, and Wan's V
// quantizes in 80 us instead of 84 (same codes).
constexpr int kColsThreads = 512;
template <int MODE, bool SEG, int TC>
__global__ __launch_bounds__(kColsThreads) void quant_cols_kernel(const uint16_t* __restrict__ x,
                                                         uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales, int64_t rows,
                                                         int64_t cols, int64_t ntr, int64_t ntc,
                                                         int64_t nitems, int64_t vstride, Layout3 in,
                                                         RowSegments seg) {
  constexpr int CPR = TC / 8;  // 16-byte chunks per tile row
  constexpr int LD = 256 * CPR / kColsThreads;  // chunks loaded per thread (256 rows x CPR chunks)
  __shared__ __attribute__((aligned(16))) uint16_t tile[256 * TC];
  const int tid = threadIdx.x;
  const bool vec8 = (cols & 7) == 0 && (in.sn & 7) == 0;
  if constexpr (SEG) vstride = seg.blk[seg.n];
  // One work item: entry bi, rows [r0, r0 + nrow) of the input (nrow <= 256),
  // columns [c0, c0 + TC), output blocks blk0 .. blk0 + nblk - 1.
  struct Item {
    int64_t bi, r0, c0, blk0;
    int nrow, nblk;
  };
  auto decode = [&](int64_t item) {
    Item w;
    w.bi = item / (ntr * ntc);
    const int64_t rest = item % (ntr * ntc), tr = rest % ntr;
    w.c0 = (rest / ntr) * TC;
    if constexpr (SEG) {
      w.nrow = 0;
      w.nblk = 0;
      w.r0 = w.blk0 = 0;
      if (tr < seg.tile[seg.n]) {
        const int s = find_segment(seg.tile, seg.n, int(tr));
        const int lt = int(tr) - seg.tile[s];
        const int len = seg.row[s + 1] - seg.row[s];
        w.r0 = seg.row[s] + int64_t(lt) * 256;
        w.nrow = min(256, len - lt * 256);
        w.blk0 = seg.blk[s] + int64_t(lt) * 8;
        w.nblk = (w.nrow + 31) / 32;
      }
    } else {
      w.r0 = tr * 256;
      w.nrow = int(min(int64_t(256), rows - w.r0));
      w.blk0 = tr * 8;
      w.nblk = (w.nrow + 31) / 32;
    }
    return w;
  };
  v4u buf[LD];
  auto load = [&](const Item& w) {
    const uint16_t* xb = x + in.base(w.bi);
#pragma unroll
    for (int i = 0; i < LD; ++i) {
      const int q = tid + kColsThreads * i;
      const int rr = q / CPR, cc = (q % CPR) * 8;
      buf[i] = v4u{0, 0, 0, 0};
      if (rr < w.nrow && w.c0 + cc < cols)
        buf[i] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(xb + (w.r0 + rr) * in.sn + w.c0 + cc));
    }
  };
  int64_t item = blockIdx.x;
  if (vec8 && item < nitems) load(decode(item));
  for (; item < nitems; item += gridDim.x) {
    const Item w = decode(item);
    if (vec8) {
#pragma unroll
      for (int i = 0; i < LD; ++i) {
        const int q = tid + kColsThreads * i;
        const int rr = q / CPR, cc = (q % CPR) * 8;
        *reinterpret_cast<v4u*>(&tile[rr * TC + (cc ^ (8 * (rr >> 5)))]) = buf[i];
      }
    } else {
      const uint16_t* xb = x + in.base(w.bi);
      for (int i = tid; i < 256 * TC; i += kColsThreads) {
        const int rr = i / TC, cc = i % TC;
        tile[rr * TC + (cc ^ (8 * (rr >> 5)))] =
            (rr < w.nrow && w.c0 + cc < cols) ? xb[(w.r0 + rr) * in.sn + w.c0 + cc] : uint16_t(0);
      }
    }
    __syncthreads();
    if (vec8 && item + gridDim.x < nitems) load(decode(item + gridDim.x));
#pragma unroll
    for (int k = 0; k < TC * 8 / kColsThreads; ++k) {
      const int it = tid + kColsThreads * k;
      const int jb = it & 7, c = it >> 3;
      if (w.c0 + c >= cols || jb >= w.nblk) continue;
      float f[32];
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const uint32_t h = tile[(32 * jb + i) * TC + (c ^ (8 * jb))];
        m = max(m, h & 0x7FFFu);
        f[i] = __uint_as_float(h << 16);
      }
      const int e = block_exp_bf16bits<MODE>(m);
      v4u cw;
      cw.x = encode8(f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[7], e);
      cw.y = encode8(f[8], f[9], f[10], f[11], f[12], f[13], f[14], f[15], e);
      cw.z = encode8(f[16], f[17], f[18], f[19], f[20], f[21], f[22], f[23], e);
      cw.w = encode8(f[24], f[25], f[26], f[27], f[28], f[29], f[30], f[31], e);
      const int64_t out = (w.bi * cols + w.c0 + c) * vstride + w.blk0 + jb;
      __builtin_nontemporal_store(cw, reinterpret_cast<v4u*>(codes + out * 16));
      scales[out] = uint8_t(e + 127);
    }
    __syncthreads();
  }
}

// Launch of the row-axis kernel: 128-column tiles unless the input is at
// most 64 columns wide.
template <int MODE, bool SEG>
void launch_cols(const uint16_t* x, uint8_t* codes, uint8_t* scales, int64_t rows, int64_t cols, int64_t batch,
                 int64_t ntr, int64_t vstride, const Layout3& in, const RowSegments& seg, int64_t grid_cap,
                 hipStream_t stream) {
  const int tc = cols > 64 ? 128 : 64;
  const int64_t ntc = (cols + tc - 1) / tc;
  const int64_t nitems = batch * ntr * ntc;
  const int64_t grid = nitems < grid_cap ? nitems : grid_cap;
  if (tc == 128)
    quant_cols_kernel<MODE, SEG, 128><<<dim3(unsigned(grid)), dim3(kColsThreads), 0, stream>>>(
        x, codes, scales, rows, cols, ntr, ntc, nitems, vstride, in, seg);
  else
    quant_cols_kernel<MODE, SEG, 64><<<dim3(unsigned(grid)), dim3(kColsThreads), 0, stream>>>(
        x, codes, scales, rows, cols, ntr, ntc, nitems, vstride, in, seg);
}

// The varlen table from cu_seqlens (batch + 1 entries, device memory): four
// arrays of batch + 1 ints, one after the other,
//   row[s]   = start token of sequence s: cu_seqlens clamped to [0, T] and
//              made non-decreasing (running maximum), so every sequence is a
//              token range inside [0, T) whatever the input holds;
//   qtile[s] = sum over earlier sequences of ceil(len / 128)  (attention
//              query tiles);
//   vtile[s] = sum of ceil(len / 256)  (row tiles of the V quantizer);
//   blk[s]   = sum of ceil(len / 32)   (32-token V blocks).
// One workgroup; each thread takes a contiguous chunk of entries, and the
// chunk totals are scanned in LDS.
__global__ __launch_bounds__(256) void varlen_table_kernel(const int* __restrict__ cu, int batch, int T,
                                                           int* __restrict__ tab) {
  __shared__ int part[4][256];
  const int n = batch + 1, tid = threadIdx.x;
  const int per = (n + 255) / 256;
  const int i0 = min(n, tid * per), i1 = min(n, i0 + per);
  int* row = tab;
  int* qtile = tab + n;
  int* vtile = tab + 2 * n;
  int* blk = tab + 3 * n;
  int m = 0;
  for (int i = i0; i < i1; ++i) m = max(m, min(max(cu[i], 0), T));
  part[0][tid] = m;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int t = 0; t < 256; ++t) {
      const int v = part[0][t];
      part[0][t] = run;
      run = max(run, v);
    }
  }
  __syncthreads();
  m = part[0][tid];
  for (int i = i0; i < i1; ++i) {
    m = max(m, min(max(cu[i], 0), T));
    row[i] = m;
  }
  __threadfence_block();
  __syncthreads();
  int sq = 0, sv = 0, sb = 0;
  for (int i = i0; i < i1 && i < batch; ++i) {
    const int len = row[i + 1] - row[i];
    sq += (len + 127) / 128;
    sv += (len + 255) / 256;
    sb += (len + 31) / 32;
  }
  part[1][tid] = sq;
  part[2][tid] = sv;
  part[3][tid] = sb;
  __syncthreads();
  if (tid == 0) {
    int rq = 0, rv = 0, rb = 0;
    for (int t = 0; t < 256; ++t) {
      const int a = part[1][t], b = part[2][t], c = part[3][t];
      part[1][t] = rq;
      part[2][t] = rv;
      part[3][t] = rb;
      rq += a;
      rv += b;
      rb += c;
    }
  }
  __syncthreads();
  sq = part[1][tid];
  sv = part[2][tid];
  sb = part[3][tid];
  for (int i = i0; i < i1; ++i) {
    qtile[i] = sq;
    vtile[i] = sv;
    blk[i] = sb;
    if (i < batch) {
      const int len = row[i + 1] - row[i];
      sq += (len + 127) / 128;
      sv += (len + 255) / 256;
      sb += (len + 31) / 32;
    }
  }
}

// Grid caps: the streaming kernel walks blocks with a grid stride (2^17
// workgroups cover 2^30 elements in one pass; a cap of 2^16, two passes per
// thread, ran 2^30 at 72% of HBM bandwidth against 75%); the row-axis
// kernel's workgroups each walk tiles (two 64 KiB tiles fit one CU's LDS, so
// 2560 workgroups are five rounds of 256 CUs x 2).
constexpr int64_t kStreamGrid = 131072;
constexpr int64_t kColsGrid = 2560;

// Host-side launchers (stream-ordered, no allocation).  Return the HIP error
// of the launch.
hipError_t launch_quantize(const void* x, int64_t batch, int64_t rows, int64_t cols, int axis,
                           int mode, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  if (batch == 0 || rows == 0 || cols == 0) return hipSuccess;
  if (axis == 1 && (cols & 31) == 0) {
    const int64_t nq = batch * rows * (cols / 32) * 4;
    constexpr int U = 4;
    int64_t grid = (nq + 256 * U - 1) / (256 * U);
    if (grid > kStreamGrid) grid = kStreamGrid;
    if (mode == kModeUOS)
      quant_stream_kernel<kModeUOS, U><<<dim3(unsigned(grid)), dim3(256), 0, stream>>>(
          static_cast<const uint4*>(x), reinterpret_cast<uint32_t*>(codes), scales, nq);
    else
      quant_stream_kernel<kModeOCP, U><<<dim3(unsigned(grid)), dim3(256), 0, stream>>>(
          static_cast<const uint4*>(x), reinterpret_cast<uint32_t*>(codes), scales, nq);
  } else if (axis == 1) {
    const int64_t nb = (cols + 31) / 32;
    const int64_t nblk = batch * rows * nb;
    const int64_t grid = (nblk + 255) / 256;
    if (mode == kModeUOS)
      quant_rows_general_kernel<kModeUOS><<<dim3(unsigned(grid)), dim3(256), 0, stream>>>(
          static_cast<const uint16_t*>(x), reinterpret_cast<uint4*>(codes), scales, batch * rows, cols, nb);
    else
      quant_rows_general_kernel<kModeOCP><<<dim3(unsigned(grid)), dim3(256), 0, stream>>>(
          static_cast<const uint16_t*>(x), reinterpret_cast<uint4*>(codes), scales, batch * rows, cols, nb);
  } else {
    const int64_t nb = (rows + 31) / 32;
    const int64_t ntr = (rows + 255) / 256;
    const Layout3 dense{1, rows * cols, 0, cols};
    const RowSegments none{nullptr, nullptr, nullptr, 0};
    const uint16_t* xp = static_cast<const uint16_t*>(x);
    if (mode == kModeUOS)
      launch_cols<kModeUOS, false>(xp, codes, scales, rows, cols, batch, ntr, nb, dense, none, kColsGrid, stream);
    else
      launch_cols<kModeOCP, false>(xp, codes, scales, rows, cols, batch, ntr, nb, dense, none, kColsGrid, stream);
  }
  return hipGetLastError();
}

// Quantization of a strided [B][H][rows][cols] view with contiguous columns
// (element (b, h, r, c) at x + b sb + h sh + r sn + c) into the canonical
// dense output of batch B * H.  Requires cols % 32 == 0 and, for loads of
// 16 bytes, sb, sh, sn multiples of 8 and x 16-byte aligned (the caller
// checks); B * H <= 65535.
hipError_t launch_quantize_strided(const void* x, int64_t B, int64_t H, int64_t rows, int64_t cols, int64_t sb,
                                   int64_t sh, int64_t sn, int axis, int mode, uint8_t* codes, uint8_t* scales,
                                   hipStream_t stream) {
  if (B == 0 || H == 0 || rows == 0 || cols == 0) return hipSuccess;
  const Layout3 in{H, sb, sh, sn};
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  if (axis == 1) {
    constexpr int U = 4;
    const int64_t np = rows * (cols / 8);
    int64_t gx = (np + 256 * U - 1) / (256 * U);
    if (gx > 1024) gx = 1024;
    const dim3 grid(unsigned(gx), unsigned(B * H));
    if (mode == kModeUOS)
      quant_rows_strided_kernel<kModeUOS, U><<<grid, dim3(256), 0, stream>>>(xp, reinterpret_cast<uint32_t*>(codes),
                                                                             scales, rows, cols, in);
    else
      quant_rows_strided_kernel<kModeOCP, U><<<grid, dim3(256), 0, stream>>>(xp, reinterpret_cast<uint32_t*>(codes),
                                                                             scales, rows, cols, in);
  } else {
    const int64_t nb = (rows + 31) / 32;
    const int64_t ntr = (rows + 255) / 256;
    const RowSegments none{nullptr, nullptr, nullptr, 0};
    if (mode == kModeUOS)
      launch_cols<kModeUOS, false>(xp, codes, scales, rows, cols, B * H, ntr, nb, in, none, kColsGrid, stream);
    else
      launch_cols<kModeOCP, false>(xp, codes, scales, rows, cols, B * H, ntr, nb, in, none, kColsGrid, stream);
  }
  return hipGetLastError();
}

// Varlen table (see varlen_table_kernel) into tab[4 (batch + 1)].
hipError_t launch_varlen_table(const int* cu_seqlens, int batch, int T, int* tab, hipStream_t stream) {
  varlen_table_kernel<<<dim3(1), dim3(256), 0, stream>>>(cu_seqlens, batch, T, tab);
  return hipGetLastError();
}

// V of a varlen batch, [T][H][d] with element (t, h, c) at x + t sn + h sh + c,
// quantized along tokens per sequence: codes [H][d][B * 16] and scales
// [H][d][B] with B = blk[batch] (at most ceil(T / 32) + batch), sequence s
// in blocks blk[s] .. blk[s + 1] - 1 of every channel.  tab is the varlen
// table.
hipError_t launch_quantize_varlen_cols(const void* x, int batch, int64_t T, int64_t H, int64_t d, int64_t sh,
                                       int64_t sn, const int* tab, int mode, uint8_t* codes, uint8_t* scales,
                                       hipStream_t stream) {
  if (T == 0 || H == 0) return hipSuccess;
  const int n = batch + 1;
  const RowSegments seg{tab, tab + 2 * n, tab + 3 * n, batch};
  const Layout3 in{H, 0, sh, sn};
  const int64_t ntr = (T + 255) / 256 + batch;
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  if (mode == kModeUOS)
    launch_cols<kModeUOS, true>(xp, codes, scales, T, d, H, ntr, 0, in, seg, kColsGrid, stream);
  else
    launch_cols<kModeOCP, true>(xp, codes, scales, T, d, H, ntr, 0, in, seg, kColsGrid, stream);
  return hipGetLastError();
}

}  // namespace mxattn
