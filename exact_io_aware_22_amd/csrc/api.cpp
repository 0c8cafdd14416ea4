// C ABI of libfa.so (declared in include/fa.h): argument validation, then dispatch
// to the HIP kernel launchers. Validation makes no HIP call, so every error path
// below can be exercised on a machine without a GPU.
#include "fa.h"

#include <cmath>
#include <cstdint>

#include "launch.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Element count a*b*c*d must stay below 2^62 so every byte offset fits in int64.
bool count_ok(int64_t a, int64_t b, int64_t c, int64_t d) {
  const int64_t lim = int64_t(1) << 62;
  int64_t x = a;
  for (int64_t y : {b, c, d}) {
    if (y != 0 && x > lim / y) return false;
    x *= y;
  }
  return x < lim / 4;
}

bool head_dim_ok(int D) { return D == 64 || D == 128; }

int hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

}  // namespace

extern "C" {

int fa_abi_version(void) { return 2; }

const char* fa_strerror(int code) {
  switch (code) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid shape: negative size, D not 64 or 128, splits < 1, or too large";
    case FA_ERR_DTYPE: return "unsupported dtype (FA_F32 or FA_BF16; windows and packed sequences need FA_BF16)";
    case FA_ERR_ALIGN: return "misaligned pointer (tensors need 16-byte, m/d/lse/delta 4-byte alignment)";
    case FA_ERR_ARG: return "invalid argument: scale must be finite and > 0, causal 0 or 1, windows >= -1";
    case FA_ERR_HIP: return "the HIP runtime rejected the kernel launch";
    case FA_ERR_SCRATCH: return "scratch too small: fa_decode_noalloc's partial states exceed the library's static scratch (2*ceil64(B*H*splits) + B*H*splits*D > FA_DECODE_SCRATCH_FLOATS floats), or a scan's workspace is smaller than fa_scan_workspace_bytes";
    default: return "unknown fa error code";
  }
}

int fa_forward_ext(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                   int H, int N, int D, float scale, int causal, int window_left,
                   int window_right, const int* cu_seqlens, int max_seqlen, int dtype,
                   void* stream) {
  const bool packed = cu_seqlens != nullptr;
  // Packed tensors are [H][N][D]: size-check H x N x D (B counts sequences).
  if (B < 0 || H < 0 || N < 0 || !head_dim_ok(D) ||
      !count_ok(packed ? 1 : B, H, N, D) || (packed && max_seqlen < 0))
    return FA_ERR_SHAPE;
  if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (!std::isfinite(scale) || !(scale > 0.0f) || (causal != 0 && causal != 1) ||
      window_left < -1 || window_right < -1)
    return FA_ERR_ARG;
  const bool windowed = window_left >= 0 || window_right >= 0;
  if (dtype == FA_F32 && (windowed || packed)) return FA_ERR_DTYPE;  // bf16 kernels only
  if (B == 0 || H == 0 || N == 0 || (packed && max_seqlen == 0)) return FA_OK;  // empty
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4) || !aligned(cu_seqlens, 4))
    return FA_ERR_ALIGN;
  fa::FwdArgs a{q, k, v, o, lse, B, H, N, D, scale, causal == 1};
  a.window_left = window_left;
  a.window_right = window_right;
  a.cu_seqlens = cu_seqlens;
  a.max_seqlen = max_seqlen;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(dtype == FA_BF16 ? fa::launch_fwd_bf16(a, s) : fa::launch_fwd_f32(a, s));
}

int fa_forward(const void* q, const void* k, const void* v, float* o, float* lse, int B,
               int H, int N, int D, float scale, int causal, int dtype, void* stream) {
  return fa_forward_ext(q, k, v, o, lse, B, H, N, D, scale, causal, -1, -1, nullptr, 0, dtype,
                        stream);
}

int fa_decode_partials(const void* q, const void* k, const void* v, float* m, float* d,
                       float* o_part, int B, int H, int L, int D, float scale, int splits,
                       int dtype, void* stream) {
  if (B < 0 || H < 0 || L < 0 || splits < 1 || !head_dim_ok(D) || !count_ok(B, H, L, D) ||
      !count_ok(B, H, splits, D + 2))
    return FA_ERR_SHAPE;
  if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (!std::isfinite(scale) || !(scale > 0.0f)) return FA_ERR_ARG;
  if (B == 0 || H == 0) return FA_OK;  // empty: no pointer is touched
  // L == 0 is not empty: every chunk is written as the identity, so k and v may be
  // NULL then but q, m, d and o_part may not.
  if (!q || !m || !d || !o_part || (L > 0 && (!k || !v))) return FA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o_part, 16) ||
      !aligned(m, 4) || !aligned(d, 4))
    return FA_ERR_ALIGN;
  fa::DecodeArgs a{q, k, v, m, d, o_part, B, H, L, D, scale, splits};
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(dtype == FA_BF16 ? fa::launch_decode_partials_bf16(a, s)
                                     : fa::launch_decode_partials_f32(a, s));
}

int fa_decode_noalloc(const void* q, const void* k, const void* v, float* o, float* lse,
                      int B, int H, int L, int D, float scale, int splits, int dtype,
                      void* stream) {
  static_assert(fa::kDecodeScratchFloats == FA_DECODE_SCRATCH_FLOATS, "one capacity");
  if (B < 0 || H < 0 || L < 0 || splits < 1 || !head_dim_ok(D) || !count_ok(B, H, L, D) ||
      !count_ok(B, H, splits, D + 2))
    return FA_ERR_SHAPE;
  if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (!std::isfinite(scale) || !(scale > 0.0f)) return FA_ERR_ARG;
  if (fa::decode_noalloc_floats(int64_t(B) * H * splits, D) > fa::kDecodeScratchFloats)
    return FA_ERR_SCRATCH;
  if (B == 0 || H == 0) return FA_OK;  // empty: no pointer is touched
  if (!q || !o || !lse || (L > 0 && (!k || !v))) return FA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4))
    return FA_ERR_ALIGN;
  fa::DecodeArgs a{q, k, v, nullptr, nullptr, nullptr, B, H, L, D, scale, splits};
  return hip_status(fa::launch_decode_noalloc(a, dtype == FA_BF16, o, lse,
                                              static_cast<hipStream_t>(stream)));
}

int fa_backward(const void* q, const void* k, const void* v, const float* o, const float* lse,
                const void* dout, float* delta, float* dq, float* dk, float* dv, int B, int H,
                int N, int D, float scale, int causal, int dtype, void* stream) {
  if (B < 0 || H < 0 || N < 0 || !head_dim_ok(D) || !count_ok(B, H, N, D)) return FA_ERR_SHAPE;
  if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (!std::isfinite(scale) || !(scale > 0.0f) || (causal != 0 && causal != 1)) return FA_ERR_ARG;
  if (B == 0 || H == 0 || N == 0) return FA_OK;  // empty: no pointer is touched
  if (!q || !k || !v || !o || !lse || !dout || !delta || !dq || !dk || !dv) return FA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4) || !aligned(delta, 4))
    return FA_ERR_ALIGN;
  fa::BwdArgs a{q, k, v, o, lse, dout, delta, dq, dk, dv, B, H, N, D, scale, causal == 1};
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(dtype == FA_BF16 ? fa::launch_bwd_bf16(a, s) : fa::launch_bwd_f32(a, s));
}

int fa_combine_partials(const float* m, const float* d, const float* o_part, int splits,
                        int rows, int D, float* o, float* lse, void* stream) {
  if (rows < 0 || splits < 1 || !head_dim_ok(D) || !count_ok(rows, splits, D, 1))
    return FA_ERR_SHAPE;
  if (rows == 0) return FA_OK;  // empty: no pointer is touched
  if (!m || !d || !o_part || !o || !lse) return FA_ERR_NULL;
  if (!aligned(o_part, 16) || !aligned(o, 16) || !aligned(m, 4) || !aligned(d, 4) ||
      !aligned(lse, 4))
    return FA_ERR_ALIGN;
  fa::CombineArgs a{m, d, o_part, o, lse, rows, splits, D};
  return hip_status(fa::launch_combine_partials(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Shared validation of the two row reductions: x [rows][n] of dtype; out0, out1 [rows].
int row_reduce(const void* x, float* out0, float* out1, int rows, int n, int dtype, void* stream,
               hipError_t (*launch)(const fa::RowReduceArgs&, hipStream_t)) {
  if (rows < 0 || n < 0) return FA_ERR_SHAPE;
  if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (rows == 0) return FA_OK;  // empty: no pointer is touched
  if (!out0 || !out1 || (n > 0 && !x)) return FA_ERR_NULL;
  if (!aligned(x, dtype == FA_BF16 ? 2 : 4) || !aligned(out0, 4) || !aligned(out1, 4))
    return FA_ERR_ALIGN;
  fa::RowReduceArgs a{x, rows, n, dtype == FA_BF16, out0, out1};
  return hip_status(launch(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int fa_softmax_stats(const void* x, float* m, float* d, int rows, int n, int dtype,
                     void* stream) {
  return row_reduce(x, m, d, rows, n, dtype, stream, fa::launch_softmax_stats);
}

int fa_moments(const void* x, float* mean, float* m2, int rows, int n, int dtype, void* stream) {
  return row_reduce(x, mean, m2, rows, n, dtype, stream, fa::launch_moments);
}

}  // extern "C"

namespace {

// Shared validation of the two prefix scans: x [rows][n] of dtype; out0, out1 [rows][n].
int row_scan(const void* x, float* out0, float* out1, int rows, int n, int dtype, void* stream,
             hipError_t (*launch)(const fa::RowReduceArgs&, hipStream_t)) {
  if (rows < 0 || n < 0 || !count_ok(rows, n, 2, 1)) return FA_ERR_SHAPE;
  if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (rows == 0 || n == 0) return FA_OK;  // empty: no pointer is touched
  if (!x || !out0 || !out1) return FA_ERR_NULL;
  if (!aligned(x, dtype == FA_BF16 ? 2 : 4) || !aligned(out0, 4) || !aligned(out1, 4))
    return FA_ERR_ALIGN;
  fa::RowReduceArgs a{x, rows, n, dtype == FA_BF16, out0, out1};
  return hip_status(launch(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int fa_softmax_scan(const void* x, float* m, float* d, int rows, int n, int dtype,
                    void* stream) {
  return row_scan(x, m, d, rows, n, dtype, stream, fa::launch_softmax_scan);
}

int fa_moments_scan(const void* x, float* mean, float* m2, int rows, int n, int dtype,
                    void* stream) {
  return row_scan(x, mean, m2, rows, n, dtype, stream, fa::launch_moments_scan);
}

long long fa_scan_workspace_bytes(int rows, int n, int dtype) {
  if (rows < 0 || n < 0 || !count_ok(rows, n, 2, 1)) return -1;
  if (dtype != FA_F32 && dtype != FA_BF16) return -1;
  return fa::scan_workspace_bytes(rows, n, dtype == FA_BF16);
}

}  // extern "C"

namespace {

// The scans with a workspace: the same validation, then the workspace of the chained
// path (needed only when fa_scan_workspace_bytes is not 0).
int row_scan_ws(const void* x, float* out0, float* out1, int rows, int n, int dtype,
                void* workspace, long long workspace_bytes, int max_polls, void* stream,
                hipError_t (*launch)(const fa::RowReduceArgs&, hipStream_t)) {
  if (rows < 0 || n < 0 || !count_ok(rows, n, 2, 1)) return FA_ERR_SHAPE;
  if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (max_polls < 0) return FA_ERR_ARG;
  if (rows == 0 || n == 0) return FA_OK;  // empty: no pointer is touched
  if (!x || !out0 || !out1) return FA_ERR_NULL;
  if (!aligned(x, dtype == FA_BF16 ? 2 : 4) || !aligned(out0, 4) || !aligned(out1, 4))
    return FA_ERR_ALIGN;
  const int64_t need = fa::scan_workspace_bytes(rows, n, dtype == FA_BF16);
  fa::RowReduceArgs a{x, rows, n, dtype == FA_BF16, out0, out1};
  if (need > 0) {
    if (!workspace) return FA_ERR_NULL;
    if (!aligned(workspace, 8)) return FA_ERR_ALIGN;
    if (workspace_bytes < need) return FA_ERR_SCRATCH;
    a.slots = static_cast<uint64_t*>(workspace);
    a.max_polls = max_polls;
  }
  return hip_status(launch(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int fa_softmax_scan_ws(const void* x, float* m, float* d, int rows, int n, int dtype,
                       void* workspace, long long workspace_bytes, int max_polls,
                       void* stream) {
  return row_scan_ws(x, m, d, rows, n, dtype, workspace, workspace_bytes, max_polls, stream,
                     fa::launch_softmax_scan);
}

int fa_moments_scan_ws(const void* x, float* mean, float* m2, int rows, int n, int dtype,
                       void* workspace, long long workspace_bytes, int max_polls,
                       void* stream) {
  return row_scan_ws(x, mean, m2, rows, n, dtype, workspace, workspace_bytes, max_polls,
                     stream, fa::launch_moments_scan);
}

}  // extern "C"

extern "C" {

int fa_calibrate_mfma(float* out, int blocks, int iters, unsigned seed, void* stream) {
  if (blocks < 1 || blocks > (1 << 20) || iters < 0) return FA_ERR_SHAPE;
  if (!out) return FA_ERR_NULL;
  if (!aligned(out, 4)) return FA_ERR_ALIGN;
  return hip_status(
      fa::launch_calibrate_mfma(out, blocks, iters, seed, static_cast<hipStream_t>(stream)));
}

int fa_calibrate_overlap(float* out, int blocks, int iters, int mode, void* stream) {
  if (blocks < 1 || blocks > (1 << 20) || iters < 0) return FA_ERR_SHAPE;
  if (mode < 0 || mode > 13 || mode == 7) return FA_ERR_ARG;
  if (!out) return FA_ERR_NULL;
  if (!aligned(out, 4)) return FA_ERR_ALIGN;
  return hip_status(fa::launch_calibrate_overlap(out, blocks, iters, mode,
                                                 static_cast<hipStream_t>(stream)));
}

int fa_calibrate_read(const void* x, long long nbytes, unsigned* out, int blocks,
                      void* stream) {
  if (blocks < 1 || blocks > (1 << 22) || nbytes < 0 || nbytes % 16 != 0) return FA_ERR_SHAPE;
  if (!out || (nbytes > 0 && !x)) return FA_ERR_NULL;
  if (!aligned(out, 4) || !aligned(x, 16)) return FA_ERR_ALIGN;
  return hip_status(fa::launch_calibrate_read(x, nbytes, out, blocks,
                                              static_cast<hipStream_t>(stream)));
}

int fa_calibrate_write(void* y, long long nbytes, unsigned value, int blocks, void* stream) {
  if (blocks < 1 || blocks > (1 << 22) || nbytes < 0 || nbytes % 16 != 0) return FA_ERR_SHAPE;
  if (nbytes == 0) return FA_OK;  // empty: no pointer is touched, nothing is launched
  if (!y) return FA_ERR_NULL;
  if (!aligned(y, 16)) return FA_ERR_ALIGN;
  return hip_status(fa::launch_calibrate_write(y, nbytes, value, blocks,
                                               static_cast<hipStream_t>(stream)));
}

int fa_calibrate_mix(const void* x, long long nbytes, void* y, int ratio, int blocks,
                     void* stream) {
  if (blocks < 1 || blocks > (1 << 22) || nbytes < 0 || nbytes % 4096 != 0 ||
      (ratio != 1 && ratio != 2 && ratio != 4))
    return FA_ERR_SHAPE;
  if (nbytes == 0) return FA_OK;  // empty: no pointer is touched, nothing is launched
  if (!x || !y) return FA_ERR_NULL;
  if (!aligned(x, 16) || !aligned(y, 16)) return FA_ERR_ALIGN;
  return hip_status(fa::launch_calibrate_mix(x, nbytes, y, ratio, blocks,
                                             static_cast<hipStream_t>(stream)));
}

}  // extern "C"
