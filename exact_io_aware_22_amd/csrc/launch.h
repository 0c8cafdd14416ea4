// Internal launcher interface between the C ABI (api.cpp) and the HIP kernels.
// Arguments reaching these functions have already been validated; each returns
// hipSuccess or the error hipLaunchKernelGGL left behind.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  float* o;
  float* lse;
  int B, H, N, D;
  float scale;
  bool causal;
  int window_left = -1, window_right = -1;  // -1: unbounded on that side
  const int* cu_seqlens = nullptr;          // packed sequences (device), B + 1 entries
  int max_seqlen = 0;
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  float* m;
  float* d;
  float* o_part;
  int B, H, L, D;
  float scale;
  int splits;
};

struct CombineArgs {
  const float* m;
  const float* d;
  const float* o_part;
  float* o;
  float* lse;
  int rows, splits, D;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* o;
  const float* lse;
  const void* dout;
  float* delta;
  float* dq;
  float* dk;
  float* dv;
  int B, H, N, D;
  float scale;
  bool causal;
};

struct RowReduceArgs {
  const void* x;  // [rows][n], float32 or bfloat16
  int64_t rows;
  int n;
  bool bf16;
  float* out0;  // softmax: m; moments: mean ([rows], or [rows][n] for a scan)
  float* out1;  // softmax: d; moments: M2
  uint64_t* slots = nullptr;  // scans: workspace of the chained path (null: one row per workgroup)
  int max_polls = 0;          // scans: polls before a block is folded locally (0: default)
};

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s);
hipError_t launch_decode_partials_bf16(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_partials_f32(const DecodeArgs& a, hipStream_t s);
hipError_t launch_combine_partials(const CombineArgs& a, hipStream_t s);
// Partials into the library's static scratch, then their merge into o, lse.
hipError_t launch_decode_noalloc(const DecodeArgs& a, bool bf16, float* o, float* lse,
                                 hipStream_t s);
// Floats of static scratch the decode of B*H*splits units at head dim D needs (m and d
// padded to 64 floats each, then o_part), and the capacity.
int64_t decode_noalloc_floats(int64_t units, int D);
constexpr int64_t kDecodeScratchFloats = int64_t(1) << 23;
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_f32(const BwdArgs& a, hipStream_t s);
hipError_t launch_softmax_stats(const RowReduceArgs& a, hipStream_t s);
hipError_t launch_moments(const RowReduceArgs& a, hipStream_t s);
// Inclusive scans: out0, out1 are [rows][n].
hipError_t launch_softmax_scan(const RowReduceArgs& a, hipStream_t s);
hipError_t launch_moments_scan(const RowReduceArgs& a, hipStream_t s);
// Chained scans: rows of more than 32 KB of input whose length is a multiple of 2048
// elements with 2 to 64 such blocks are cut into blocks, one workgroup each (given a
// workspace and aligned tensors); the block count, or 0 when a row takes one workgroup.
int scan_chain_blocks(int n, bool bf16);
// Workspace bytes the chained scans need for rows x n (0 when they do not apply).
int64_t scan_workspace_bytes(int64_t rows, int n, bool bf16);

hipError_t launch_calibrate_mfma(float* out, int blocks, int iters, uint32_t seed, hipStream_t s);
hipError_t launch_calibrate_overlap(float* out, int blocks, int iters, int mode,
                                    hipStream_t s);
hipError_t launch_calibrate_read(const void* x, int64_t nbytes, uint32_t* out, int blocks,
                                 hipStream_t s);
hipError_t launch_calibrate_write(void* y, int64_t nbytes, uint32_t value, int blocks,
                                  hipStream_t s);
hipError_t launch_calibrate_mix(const void* x, int64_t nbytes, void* y, int ratio, int blocks,
                                hipStream_t s);

}  // namespace fa
