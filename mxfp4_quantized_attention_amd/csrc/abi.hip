// abi.hip -- the C ABI of libmxattn.so (declared in include/mxattn.h).
//
// Every entry point validates its arguments on the host before touching the
// HIP runtime, so a rejected call enqueues nothing and needs no GPU.  Work is
// enqueued on the caller's stream; the library allocates no device memory.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <vector>

#include "mxattn.h"

namespace mxattn {
hipError_t launch_quantize(const void* x, int64_t batch, int64_t rows, int64_t cols, int axis,
                           int mode, uint8_t* codes, uint8_t* scales, hipStream_t stream);
hipError_t launch_attention(const uint16_t* q, const int64_t* q_strides, const uint8_t* qc, const uint8_t* qs,
                            const uint8_t* kc, const uint8_t* ks, const uint8_t* vc, const uint8_t* vs, int H,
                            int BH, int N, int d, int mode, bool pnq, float softmax_scale, uint16_t* o,
                            const int64_t* o_strides, hipStream_t stream);
hipError_t launch_quantize_strided(const void* x, int64_t B, int64_t H, int64_t rows, int64_t cols, int64_t sb,
                                   int64_t sh, int64_t sn, int axis, int mode, uint8_t* codes, uint8_t* scales,
                                   hipStream_t stream);
hipError_t launch_gemm(const uint8_t* xc, const uint8_t* xs, const uint8_t* wc, const uint8_t* ws, int M,
                       int N, int K, uint16_t* y, hipStream_t stream);
hipError_t launch_qkv_gemm(const uint8_t* xc, const uint8_t* xs, const uint8_t* wc, const uint8_t* ws, int M,
                           int K, int H, int hd, int mode, uint16_t* q, uint8_t* kc, uint8_t* ks, uint8_t* vc,
                           uint8_t* vs, hipStream_t stream);
hipError_t launch_varlen_table(const int* cu_seqlens, int batch, int T, int* tab, hipStream_t stream);
hipError_t launch_quantize_varlen_cols(const void* x, int batch, int64_t T, int64_t H, int64_t d, int64_t sh,
                                       int64_t sn, const int* tab, int mode, uint8_t* codes, uint8_t* scales,
                                       hipStream_t stream);
hipError_t launch_attention_varlen(const uint16_t* q, int64_t q_sn, int64_t q_sh, const uint8_t* kc,
                                   const uint8_t* ks, const uint8_t* vc, const uint8_t* vs, const int* tab,
                                   int batch, int T, int H, int d, int mode, bool pnq, float softmax_scale,
                                   uint16_t* o, int64_t o_sn, int64_t o_sh, hipStream_t stream);
}  // namespace mxattn

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 40;  // per quantize call
constexpr int64_t kMaxAttnElems = int64_t(1) << 34;  // B*H*N*d per attention call
constexpr int kKvTile = 128;
constexpr int64_t kQueryTile = 128;  // queries per attention workgroup (kBR in attention.hip)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool valid_mode(int mode) { return mode == MXQ_MODE_OCP || mode == MXQ_MODE_UOS; }
size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

struct WsLayout {
  size_t kc, ks, vc, vs, total;
};

// Workspace regions (each 256-byte aligned): K codes/scales (axis 1, rows = N,
// cols = d) and V codes/scales (axis 0).  Q is quantized inside the attention
// kernel and needs none.
WsLayout ws_layout(int64_t BH, int64_t N, int64_t d) {
  WsLayout w;
  const size_t qcb = size_t(BH * N * d / 2), qsb = size_t(BH * N * (d / 32));
  const int64_t nbn = (N + 31) / 32;
  const size_t vcb = size_t(BH * d * nbn * 16), vsb = size_t(BH * d * nbn);
  size_t off = 0;
  w.kc = off; off = round256(off + qcb);
  w.ks = off; off = round256(off + qsb);
  w.vc = off; off = round256(off + vcb);
  w.vs = off; off = round256(off + vsb);
  w.total = off;
  return w;
}

int check_attn_sizes(int64_t B, int64_t H, int64_t N, int64_t d) {
  if (B < 1 || H < 1 || N < 1) return MXQ_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return MXQ_ERR_UNSUPPORTED;
  if (B > (int64_t(1) << 20) || H > (int64_t(1) << 20) || N > (int64_t(1) << 24)) return MXQ_ERR_UNSUPPORTED;
  const int64_t BH = B * H;
  if (BH > (int64_t(1) << 24) || BH * N * d > kMaxAttnElems) return MXQ_ERR_UNSUPPORTED;
  // the workgroup count (BH * ceil(N / kQueryTile), rounded up to 8) must fit an int
  if (BH * ((N + kQueryTile - 1) / kQueryTile) + 8 > (int64_t(1) << 31) - 1) return MXQ_ERR_UNSUPPORTED;
  return MXQ_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MXQ_OK : MXQ_ERR_HIP; }

// Varlen workspace: K codes/scales [H][T], V codes/scales sized for
// [H][d][vstride] with vstride = ceil(T / 32) + batch blocks per channel (an
// upper bound on the blocks of all sequences, each padded to 32 tokens; the
// kernels use the exact count from the table), then the varlen table,
// 4 (batch + 1) ints.
struct VarlenLayout {
  size_t kc, ks, vc, vs, tab, total;
  int64_t vstride;
};

VarlenLayout varlen_layout(int64_t batch, int64_t T, int64_t H, int64_t d) {
  VarlenLayout w;
  w.vstride = (T + 31) / 32 + batch;
  size_t off = 0;
  w.kc = off; off = round256(off + size_t(H * T * d / 2));
  w.ks = off; off = round256(off + size_t(H * T * (d / 32)));
  w.vc = off; off = round256(off + size_t(H * d * w.vstride * 16));
  w.vs = off; off = round256(off + size_t(H * d * w.vstride));
  w.tab = off; off = round256(off + size_t(4 * (batch + 1)) * sizeof(int));
  w.total = off;
  return w;
}

int check_varlen_sizes(int64_t batch, int64_t T, int64_t H, int64_t d) {
  if (batch < 1 || T < 0 || H < 1) return MXQ_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return MXQ_ERR_UNSUPPORTED;
  if (batch > (int64_t(1) << 20) || T > (int64_t(1) << 24) || H > 65535) return MXQ_ERR_UNSUPPORTED;
  // V block offsets of one head (d channels of vstride blocks, 16 bytes each)
  // are 32-bit in the kernels, and so is the workgroup count
  const int64_t vstride = (T + 31) / 32 + batch;
  if (d * vstride * 16 > (int64_t(1) << 31) - 1) return MXQ_ERR_UNSUPPORTED;
  if (H * T * d > kMaxAttnElems) return MXQ_ERR_UNSUPPORTED;
  if (H * ((T + kQueryTile - 1) / kQueryTile + batch) + 8 > (int64_t(1) << 31) - 1) return MXQ_ERR_UNSUPPORTED;
  return MXQ_OK;
}

int check_gemm_sizes(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 1) return MXQ_ERR_INVALID_ARG;
  if (K % 128 != 0 || N % 4 != 0) return MXQ_ERR_UNSUPPORTED;
  // codes of X and W, and Y, addressed with 32-bit offsets per tile
  if (M * (K / 2) > (int64_t(1) << 31) - 1 || N * (K / 2) > (int64_t(1) << 31) - 1) return MXQ_ERR_UNSUPPORTED;
  if (M > (int64_t(1) << 30) || N > (int64_t(1) << 30) || M * N > (int64_t(1) << 40)) return MXQ_ERR_UNSUPPORTED;
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (tiles + 8 > (int64_t(1) << 31) - 1) return MXQ_ERR_UNSUPPORTED;
  return MXQ_OK;
}

}  // namespace

extern "C" {

const char* mxq_status_string(int status) {
  switch (status) {
    case MXQ_OK: return "MXQ_OK";
    case MXQ_ERR_INVALID_ARG: return "MXQ_ERR_INVALID_ARG";
    case MXQ_ERR_UNSUPPORTED: return "MXQ_ERR_UNSUPPORTED";
    case MXQ_ERR_WORKSPACE: return "MXQ_ERR_WORKSPACE";
    case MXQ_ERR_HIP: return "MXQ_ERR_HIP";
    case MXQ_ERR_IO: return "MXQ_ERR_IO";
    default: return "MXQ_ERR_UNKNOWN";
  }
}

int mxattn_version(void) { return 100; }

int mxq_quantize(const void* x_bf16, int64_t batch, int64_t rows, int64_t cols, int axis, int mode,
                 uint8_t* codes, uint8_t* scales, void* stream) {
  if (batch < 0 || rows < 0 || cols < 0 || (axis != 0 && axis != 1) || !valid_mode(mode))
    return MXQ_ERR_INVALID_ARG;
  if (batch == 0 || rows == 0 || cols == 0) return MXQ_OK;
  if (!x_bf16 || !codes || !scales) return MXQ_ERR_INVALID_ARG;
  if (!aligned16(x_bf16) || !aligned16(codes)) return MXQ_ERR_INVALID_ARG;
  if (rows > kMaxElems || cols > kMaxElems || batch > kMaxElems || rows * cols > kMaxElems ||
      batch * rows * cols > kMaxElems)
    return MXQ_ERR_UNSUPPORTED;
  if (axis == 0 && batch > 65535) return MXQ_ERR_UNSUPPORTED;
  if (axis == 0 && ((rows + 255) / 256) * ((cols + 63) / 64) > 0x7FFFFFFF) return MXQ_ERR_UNSUPPORTED;
  if (axis == 1 && (cols & 31) != 0 && (batch * rows * ((cols + 31) / 32) + 255) / 256 > 0x7FFFFFFF)
    return MXQ_ERR_UNSUPPORTED;
  return hip_status(mxattn::launch_quantize(x_bf16, batch, rows, cols, axis, mode, codes, scales,
                                            static_cast<hipStream_t>(stream)));
}

int mxq_quantize_strided(const void* x, int64_t B, int64_t H, int64_t rows, int64_t cols, const int64_t* strides,
                         int axis, int mode, uint8_t* codes, uint8_t* scales, void* stream) {
  if (B < 0 || H < 0 || rows < 0 || cols < 0 || (axis != 0 && axis != 1) || !valid_mode(mode) || !strides)
    return MXQ_ERR_INVALID_ARG;
  if (B == 0 || H == 0 || rows == 0 || cols == 0) return MXQ_OK;
  if (!x || !codes || !scales) return MXQ_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(codes)) return MXQ_ERR_INVALID_ARG;
  for (int i = 0; i < 3; ++i)
    if (strides[i] < 0 || strides[i] % 8 != 0 || strides[i] > (int64_t(1) << 40)) return MXQ_ERR_INVALID_ARG;
  if (cols % 32 != 0) return MXQ_ERR_UNSUPPORTED;
  if (B * H > 65535 || rows > (int64_t(1) << 24) || cols > (int64_t(1) << 16)) return MXQ_ERR_UNSUPPORTED;
  return hip_status(mxattn::launch_quantize_strided(x, B, H, rows, cols, strides[0], strides[1], strides[2], axis,
                                                    mode, codes, scales, static_cast<hipStream_t>(stream)));
}

int mxattn_kv_tile(int64_t d) { return (d == 64 || d == 128) ? kKvTile : 0; }

size_t mxattn_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d) {
  if (check_attn_sizes(B, H, N, d) != MXQ_OK) return 0;
  return ws_layout(B * H, N, d).total;
}

int mxattn_fwd_quantized(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                         const uint8_t* vc, const uint8_t* vs, int64_t B, int64_t H, int64_t N,
                         int64_t d, int mode, int pnq, float softmax_scale, void* o, void* stream) {
  int st = check_attn_sizes(B, H, N, d);
  if (st != MXQ_OK) return st;
  if (!valid_mode(mode) || (pnq != 0 && pnq != 1) || !std::isfinite(softmax_scale)) return MXQ_ERR_INVALID_ARG;
  if (!qc || !qs || !kc || !ks || !vc || !vs || !o) return MXQ_ERR_INVALID_ARG;
  if (!aligned16(qc) || !aligned16(kc) || !aligned16(vc) || !aligned16(o)) return MXQ_ERR_INVALID_ARG;
  const float scale = softmax_scale > 0.f ? softmax_scale : float(1.0 / std::sqrt(double(d)));
  return hip_status(mxattn::launch_attention(nullptr, nullptr, qc, qs, kc, ks, vc, vs, int(H), int(B * H), int(N),
                                             int(d), mode, pnq != 0, scale, static_cast<uint16_t*>(o), nullptr,
                                             static_cast<hipStream_t>(stream)));
}

int mxattn_fwd_kv_quantized(const void* q, const uint8_t* kc, const uint8_t* ks, const uint8_t* vc,
                            const uint8_t* vs, int64_t B, int64_t H, int64_t N, int64_t d, int mode, int pnq,
                            float softmax_scale, void* o, void* stream) {
  int st = check_attn_sizes(B, H, N, d);
  if (st != MXQ_OK) return st;
  if (!valid_mode(mode) || (pnq != 0 && pnq != 1) || !std::isfinite(softmax_scale)) return MXQ_ERR_INVALID_ARG;
  if (!q || !kc || !ks || !vc || !vs || !o) return MXQ_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(kc) || !aligned16(vc) || !aligned16(o)) return MXQ_ERR_INVALID_ARG;
  const float scale = softmax_scale > 0.f ? softmax_scale : float(1.0 / std::sqrt(double(d)));
  return hip_status(mxattn::launch_attention(static_cast<const uint16_t*>(q), nullptr, nullptr, nullptr, kc, ks, vc,
                                             vs, int(H), int(B * H), int(N), int(d), mode, pnq != 0, scale,
                                             static_cast<uint16_t*>(o), nullptr, static_cast<hipStream_t>(stream)));
}

int mxattn_fwd(const void* q, const void* k, const void* v, int64_t B, int64_t H, int64_t N, int64_t d,
               int mode, int pnq, float softmax_scale, void* o, void* workspace, size_t workspace_bytes,
               void* stream) {
  int st = check_attn_sizes(B, H, N, d);
  if (st != MXQ_OK) return st;
  if (!valid_mode(mode) || (pnq != 0 && pnq != 1) || !std::isfinite(softmax_scale)) return MXQ_ERR_INVALID_ARG;
  if (!q || !k || !v || !o) return MXQ_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return MXQ_ERR_INVALID_ARG;
  const int64_t BH = B * H;
  const WsLayout w = ws_layout(BH, N, d);
  if (!workspace || workspace_bytes < w.total) return MXQ_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MXQ_ERR_INVALID_ARG;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = mxattn::launch_quantize(k, BH, N, d, 1, mode, ws + w.kc, ws + w.ks, s);
  if (e == hipSuccess) e = mxattn::launch_quantize(v, BH, N, d, 0, mode, ws + w.vc, ws + w.vs, s);
  if (e != hipSuccess) return MXQ_ERR_HIP;
  const float scale = softmax_scale > 0.f ? softmax_scale : float(1.0 / std::sqrt(double(d)));
  return hip_status(mxattn::launch_attention(static_cast<const uint16_t*>(q), nullptr, nullptr, nullptr, ws + w.kc,
                                             ws + w.ks, ws + w.vc, ws + w.vs, int(H), int(BH), int(N), int(d),
                                             mode, pnq != 0, scale, static_cast<uint16_t*>(o), nullptr, s));
}

int mxattn_fwd_strided(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H, int64_t N,
                       int64_t d, const int64_t* q_strides, const int64_t* k_strides, const int64_t* v_strides,
                       const int64_t* o_strides, int mode, int pnq, float softmax_scale, void* workspace,
                       size_t workspace_bytes, void* stream) {
  int st = check_attn_sizes(B, H, N, d);
  if (st != MXQ_OK) return st;
  if (B * H > 65535) return MXQ_ERR_UNSUPPORTED;
  if (!valid_mode(mode) || (pnq != 0 && pnq != 1) || !std::isfinite(softmax_scale)) return MXQ_ERR_INVALID_ARG;
  if (!q || !k || !v || !o || !q_strides || !k_strides || !v_strides || !o_strides) return MXQ_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return MXQ_ERR_INVALID_ARG;
  const int64_t* all[4] = {q_strides, k_strides, v_strides, o_strides};
  for (const int64_t* sp : all)
    for (int i = 0; i < 3; ++i)  // every row must start 16-byte aligned; no stride may overflow an offset
      if (sp[i] < 0 || sp[i] % 8 != 0 || sp[i] > (int64_t(1) << 40)) return MXQ_ERR_INVALID_ARG;
  const int64_t BH = B * H;
  const WsLayout w = ws_layout(BH, N, d);
  if (!workspace || workspace_bytes < w.total) return MXQ_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MXQ_ERR_INVALID_ARG;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = mxattn::launch_quantize_strided(k, B, H, N, d, k_strides[0], k_strides[1], k_strides[2], 1, mode,
                                                 ws + w.kc, ws + w.ks, s);
  if (e == hipSuccess)
    e = mxattn::launch_quantize_strided(v, B, H, N, d, v_strides[0], v_strides[1], v_strides[2], 0, mode,
                                        ws + w.vc, ws + w.vs, s);
  if (e != hipSuccess) return MXQ_ERR_HIP;
  const float scale = softmax_scale > 0.f ? softmax_scale : float(1.0 / std::sqrt(double(d)));
  return hip_status(mxattn::launch_attention(static_cast<const uint16_t*>(q), q_strides, nullptr, nullptr,
                                             ws + w.kc, ws + w.ks, ws + w.vc, ws + w.vs, int(H), int(BH), int(N),
                                             int(d), mode, pnq != 0, scale, static_cast<uint16_t*>(o), o_strides,
                                             s));
}

size_t mxattn_varlen_workspace_bytes(int64_t batch, int64_t T, int64_t H, int64_t d) {
  if (check_varlen_sizes(batch, T, H, d) != MXQ_OK) return 0;
  return varlen_layout(batch, T, H, d).total;
}

int mxattn_fwd_varlen(const void* q, const void* k, const void* v, void* o, const int32_t* cu_seqlens,
                      int64_t batch, int64_t T, int64_t H, int64_t d, const int64_t* strides, int mode, int pnq,
                      float softmax_scale, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_varlen_sizes(batch, T, H, d);
  if (st != MXQ_OK) return st;
  if (!valid_mode(mode) || (pnq != 0 && pnq != 1) || !std::isfinite(softmax_scale)) return MXQ_ERR_INVALID_ARG;
  if (T == 0) return MXQ_OK;
  if (!q || !k || !v || !o || !cu_seqlens) return MXQ_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return MXQ_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) return MXQ_ERR_INVALID_ARG;
  // token and head strides of Q, K, V, O (elements); null: packed [T][H][d]
  const int64_t packed[8] = {H * d, d, H * d, d, H * d, d, H * d, d};
  const int64_t* sp = strides ? strides : packed;
  for (int i = 0; i < 8; ++i)
    if (sp[i] < 0 || sp[i] % 8 != 0 || sp[i] > (int64_t(1) << 40)) return MXQ_ERR_INVALID_ARG;
  const VarlenLayout w = varlen_layout(batch, T, H, d);
  if (!workspace || workspace_bytes < w.total) return MXQ_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MXQ_ERR_INVALID_ARG;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int* tab = reinterpret_cast<int*>(ws + w.tab);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = mxattn::launch_varlen_table(cu_seqlens, int(batch), int(T), tab, s);
  if (e == hipSuccess)
    e = mxattn::launch_quantize_strided(k, 1, H, T, d, 0, sp[3], sp[2], 1, mode, ws + w.kc, ws + w.ks, s);
  if (e == hipSuccess)
    e = mxattn::launch_quantize_varlen_cols(v, int(batch), T, H, d, sp[5], sp[4], tab, mode, ws + w.vc, ws + w.vs,
                                            s);
  if (e != hipSuccess) return MXQ_ERR_HIP;
  const float scale = softmax_scale > 0.f ? softmax_scale : float(1.0 / std::sqrt(double(d)));
  return hip_status(mxattn::launch_attention_varlen(static_cast<const uint16_t*>(q), sp[0], sp[1], ws + w.kc,
                                                    ws + w.ks, ws + w.vc, ws + w.vs, tab, int(batch), int(T), int(H),
                                                    int(d), mode, pnq != 0, scale, static_cast<uint16_t*>(o), sp[6],
                                                    sp[7], s));
}

size_t mxgemm_workspace_bytes(int64_t M, int64_t K) {
  if (M < 1 || K < 1 || K % 128 != 0 || M * (K / 2) > (int64_t(1) << 31) - 1) return 0;
  return round256(size_t(M * K / 2)) + round256(size_t(M * K / 32));
}

int mxgemm_quantized(const uint8_t* xc, const uint8_t* xs, const uint8_t* wc, const uint8_t* ws, int64_t M,
                     int64_t N, int64_t K, void* y, void* stream) {
  int st = check_gemm_sizes(M, N, K);
  if (st != MXQ_OK) return st;
  if (!xc || !xs || !wc || !ws || !y) return MXQ_ERR_INVALID_ARG;
  if (!aligned16(xc) || !aligned16(wc) || !aligned16(y)) return MXQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(xs) & 3u) || (reinterpret_cast<uintptr_t>(ws) & 3u)) return MXQ_ERR_INVALID_ARG;
  return hip_status(mxattn::launch_gemm(xc, xs, wc, ws, int(M), int(N), int(K), static_cast<uint16_t*>(y),
                                        static_cast<hipStream_t>(stream)));
}

int mxgemm(const void* x, const uint8_t* wc, const uint8_t* ws, int64_t M, int64_t N, int64_t K, int mode,
           void* y, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_gemm_sizes(M, N, K);
  if (st != MXQ_OK) return st;
  if (!valid_mode(mode)) return MXQ_ERR_INVALID_ARG;
  if (!x || !wc || !ws || !y) return MXQ_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(wc) || !aligned16(y)) return MXQ_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(ws) & 3u) return MXQ_ERR_INVALID_ARG;
  const size_t need = mxgemm_workspace_bytes(M, K);
  if (!workspace || workspace_bytes < need) return MXQ_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MXQ_ERR_INVALID_ARG;
  uint8_t* xc = static_cast<uint8_t*>(workspace);
  uint8_t* xs = xc + round256(size_t(M * K / 2));
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = mxattn::launch_quantize(x, 1, M, K, 1, mode, xc, xs, s);
  if (e != hipSuccess) return MXQ_ERR_HIP;
  return hip_status(mxattn::launch_gemm(xc, xs, wc, ws, int(M), int(N), int(K), static_cast<uint16_t*>(y), s));
}

int mxqkv_proj_quantized(const uint8_t* xc, const uint8_t* xs, const uint8_t* wc, const uint8_t* ws, int64_t T,
                         int64_t C, int64_t H, int64_t d, int mode, void* q, uint8_t* kc, uint8_t* ks, uint8_t* vc,
                         uint8_t* vs, void* stream) {
  if (T < 1 || C < 1 || H < 1) return MXQ_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return MXQ_ERR_UNSUPPORTED;
  if (H > (int64_t(1) << 20)) return MXQ_ERR_UNSUPPORTED;
  int st = check_gemm_sizes(T, 3 * H * d, C);
  if (st != MXQ_OK) return st;
  if (check_attn_sizes(1, H, T, d) != MXQ_OK) return MXQ_ERR_UNSUPPORTED;
  if (!valid_mode(mode)) return MXQ_ERR_INVALID_ARG;
  if (!xc || !xs || !wc || !ws || !q || !kc || !ks || !vc || !vs) return MXQ_ERR_INVALID_ARG;
  if (!aligned16(xc) || !aligned16(wc) || !aligned16(q) || !aligned16(kc) || !aligned16(vc))
    return MXQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(xs) & 3u) || (reinterpret_cast<uintptr_t>(ws) & 3u)) return MXQ_ERR_INVALID_ARG;
  return hip_status(mxattn::launch_qkv_gemm(xc, xs, wc, ws, int(T), int(C), int(H), int(d), mode,
                                            static_cast<uint16_t*>(q), kc, ks, vc, vs,
                                            static_cast<hipStream_t>(stream)));
}

int mxqkv_proj(const void* x, const uint8_t* wc, const uint8_t* ws, int64_t T, int64_t C, int64_t H, int64_t d,
               int mode, void* q, uint8_t* kc, uint8_t* ks, uint8_t* vc, uint8_t* vs, void* workspace,
               size_t workspace_bytes, void* stream) {
  if (T < 1 || C < 1 || H < 1) return MXQ_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return MXQ_ERR_UNSUPPORTED;
  if (H > (int64_t(1) << 20)) return MXQ_ERR_UNSUPPORTED;
  int st = check_gemm_sizes(T, 3 * H * d, C);
  if (st != MXQ_OK) return st;
  if (check_attn_sizes(1, H, T, d) != MXQ_OK) return MXQ_ERR_UNSUPPORTED;
  if (!valid_mode(mode)) return MXQ_ERR_INVALID_ARG;
  if (!x || !wc || !ws || !q || !kc || !ks || !vc || !vs) return MXQ_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(wc) || !aligned16(q) || !aligned16(kc) || !aligned16(vc))
    return MXQ_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(ws) & 3u) return MXQ_ERR_INVALID_ARG;
  const size_t need = mxgemm_workspace_bytes(T, C);
  if (!workspace || workspace_bytes < need) return MXQ_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MXQ_ERR_INVALID_ARG;
  uint8_t* xc = static_cast<uint8_t*>(workspace);
  uint8_t* xs = xc + round256(size_t(T * C / 2));
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = mxattn::launch_quantize(x, 1, T, C, 1, mode, xc, xs, s);
  if (e != hipSuccess) return MXQ_ERR_HIP;
  return hip_status(mxattn::launch_qkv_gemm(xc, xs, wc, ws, int(T), int(C), int(H), int(d), mode,
                                            static_cast<uint16_t*>(q), kc, ks, vc, vs, s));
}

int mxq_dump(const char* path, const uint8_t* codes, const uint8_t* scales, int64_t batch, int64_t nvec,
             int64_t L, int axis, int mode, void* stream) {
  if (!path || batch < 0 || nvec < 0 || L < 0 || (axis != 0 && axis != 1) || !valid_mode(mode))
    return MXQ_ERR_INVALID_ARG;
  if (batch > kMaxElems || nvec > kMaxElems || L > kMaxElems || batch * nvec > kMaxElems ||
      batch * nvec * ((L + 31) / 32) > kMaxElems / 16)
    return MXQ_ERR_INVALID_ARG;
  const int64_t nb = (L + 31) / 32;
  const size_t ncode = size_t(batch * nvec * nb * 16), nscale = size_t(batch * nvec * nb);
  if ((ncode > 0) && (!codes || !scales)) return MXQ_ERR_INVALID_ARG;
  char hdr[256];
  const int len = std::snprintf(hdr, sizeof hdr,
                                "{\"magic\":\"MXQ1\",\"version\":1,\"mode\":\"%s\",\"axis\":%d,\"batch\":%lld,"
                                "\"nvec\":%lld,\"L\":%lld,\"block\":32,\"elem\":\"e2m1\",\"scale\":\"e8m0\","
                                "\"nibble\":\"lo-first\"}",
                                mode == MXQ_MODE_OCP ? "ocp" : "uos", axis, (long long)batch,
                                (long long)nvec, (long long)L);
  if (len < 0 || len > 254) return MXQ_ERR_INVALID_ARG;
  std::memset(hdr + len, ' ', size_t(255 - len));
  hdr[255] = '\n';

  // Device pointers are copied on the caller's stream; host memory (or any
  // pointer the runtime does not know) is read directly.  codes and scales
  // must live in the same kind of memory: a device/host mix is rejected.
  std::vector<uint8_t> hc, hs;
  const uint8_t* pc = codes;
  const uint8_t* ps = scales;
  if (ncode > 0) {
    auto device_memory = [](const void* p) {
      hipPointerAttribute_t attr;
      if (hipPointerGetAttributes(&attr, p) == hipSuccess)
        return attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged;
      (void)hipGetLastError();  // unknown pointer: host memory
      return false;
    };
    const bool on_device = device_memory(codes);
    if (device_memory(scales) != on_device) return MXQ_ERR_INVALID_ARG;
    if (on_device) {
      hc.resize(ncode);
      hs.resize(nscale);
      hipStream_t s = static_cast<hipStream_t>(stream);
      if (hipMemcpyAsync(hc.data(), codes, ncode, hipMemcpyDeviceToHost, s) != hipSuccess ||
          hipMemcpyAsync(hs.data(), scales, nscale, hipMemcpyDeviceToHost, s) != hipSuccess ||
          hipStreamSynchronize(s) != hipSuccess)
        return MXQ_ERR_HIP;
      pc = hc.data();
      ps = hs.data();
    }
  }
  FILE* f = std::fopen(path, "wb");
  if (!f) return MXQ_ERR_IO;
  bool ok = std::fwrite(hdr, 1, 256, f) == 256;
  if (ok && ncode) ok = std::fwrite(pc, 1, ncode, f) == ncode;
  if (ok && nscale) ok = std::fwrite(ps, 1, nscale, f) == nscale;
  ok = (std::fclose(f) == 0) && ok;
  return ok ? MXQ_OK : MXQ_ERR_IO;
}

}  // extern "C"
