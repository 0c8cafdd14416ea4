// Measurement kernels: the chip's sustained rates on the two resources the attention
// kernels are bound by, used as measured roofline denominators beside the published
// peaks. They compute nothing of the method.
//
//   * mfma_loop_kernel: v_mfma_f32_32x32x16_bf16 only, on register operands, eight
//     wavefronts per workgroup (two per SIMD, as the prefill kernel runs). Operands are
//     random bf16 bit patterns: the matrix pipes draw more power on high-entropy data
//     and the clock follows, so constant operands would overstate the ceiling.
//   * read_stream_kernel: 16-byte non-temporal loads of a buffer, each workgroup over
//     one contiguous span, eight in flight per thread, XOR-folded so the loads cannot
//     be elided.
//   * write_stream_kernel: the same split with 16-byte non-temporal stores of a
//     checkable pattern.
#include "device.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int kMfmaThreads = 512;
constexpr int kReadThreads = 256;

// splitmix32-style mixer (a published integer hash), for operand bits only.
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x += 0x9e3779b9u;
  x = (x ^ (x >> 16)) * 0x85ebca6bu;
  x = (x ^ (x >> 13)) * 0xc2b2ae35u;
  return x ^ (x >> 16);
}

// Two random bf16 values in +-[0.5, 4): random sign and mantissa, exponent 126..128.
__device__ __forceinline__ uint32_t rand_bf16x2(uint32_t h) {
  auto one = [](uint32_t b) {
    const uint32_t e = 126u + (b >> 8) % 3u;
    return ((b >> 15) & 1u) << 15 | e << 7 | (b & 0x7fu);
  };
  return one(h & 0xffffu) | one(h >> 16) << 16;
}

__global__ __launch_bounds__(kMfmaThreads) void mfma_loop_kernel(float* __restrict__ out,
                                                                 int iters, uint32_t seed) {
  const uint32_t gid = blockIdx.x * kMfmaThreads + threadIdx.x;
  // The seed is hashed before it meets the index, so seeds that differ in a few bits do
  // not merely permute the same values among a thread's operands.
  const uint32_t sa = mix32(seed), sb = mix32(seed ^ 0x5bd1e995u);
  u32x4_t a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a[i][j] = rand_bf16x2(mix32(sa ^ (gid * 64u + 8u * i + j)));
      b[i][j] = rand_bf16x2(mix32(sb ^ (gid * 64u + 8u * i + j)));
    }
  f32x16_t acc[8] = {};
#pragma unroll 1
  for (int it = 0; it < iters; ++it) {
    // 16 products, eight independent accumulators, every operand pairing different.
#pragma unroll
    for (int i = 0; i < 16; ++i)
      acc[i & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[i & 7]),
                                                           as_bf16x8(b[(3 * i + 1) & 7]),
                                                           acc[i & 7], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[k][r];
  out[gid] = s;
}

// Workgroup b reads the 16-byte words [b span, min(n16, (b + 1) span)), thread t those at
// positions t mod 256 of the span, eight loads in flight.
__global__ __launch_bounds__(kReadThreads) void read_stream_kernel(const u32x4_t* __restrict__ x,
                                                                   int64_t n16, int64_t span,
                                                                   uint32_t* __restrict__ out) {
  const int64_t b0 = int64_t(blockIdx.x) * span;
  const int64_t end = min(n16, b0 + span);
  uint32_t acc = 0;
  int64_t i = b0 + threadIdx.x;
  for (; i + 7 * kReadThreads < end; i += 8 * kReadThreads) {
    u32x4_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = __builtin_nontemporal_load(x + i + j * kReadThreads);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
  }
  for (; i < end; i += kReadThreads) {
    const u32x4_t v = __builtin_nontemporal_load(x + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[int64_t(blockIdx.x) * kReadThreads + threadIdx.x] = acc;
}

// Workgroup b writes the 16-byte words of its span (the same split as the read stream),
// thread t those at positions t mod 256, eight stores in flight; every word gets
// {value, word index (low 32 bits), value, word index} so the result can be checked.
__global__ __launch_bounds__(kReadThreads) void write_stream_kernel(u32x4_t* __restrict__ y,
                                                                    int64_t n16, int64_t span,
                                                                    uint32_t value) {
  const int64_t b0 = int64_t(blockIdx.x) * span;
  const int64_t end = min(n16, b0 + span);
  int64_t i = b0 + threadIdx.x;
  for (; i + 7 * kReadThreads < end; i += 8 * kReadThreads) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t w = uint32_t(i + j * kReadThreads);
      __builtin_nontemporal_store(u32x4_t{value, w, value, w}, y + i + j * kReadThreads);
    }
  }
  for (; i < end; i += kReadThreads)
    __builtin_nontemporal_store(u32x4_t{value, uint32_t(i), value, uint32_t(i)}, y + i);
}

}  // namespace

hipError_t launch_calibrate_mfma(float* out, int blocks, int iters, uint32_t seed,
                                 hipStream_t s) {
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(unsigned(blocks)), dim3(kMfmaThreads), 0, s, out,
                     iters, seed);
  return hipGetLastError();
}

hipError_t launch_calibrate_read(const void* x, int64_t nbytes, uint32_t* out, int blocks,
                                 hipStream_t s) {
  // span: the words per workgroup, rounded up to whole rows of 256 threads
  const int64_t n16 = nbytes / 16;
  const int64_t span = ((n16 + blocks - 1) / blocks + kReadThreads - 1) / kReadThreads * kReadThreads;
  hipLaunchKernelGGL(read_stream_kernel, dim3(unsigned(blocks)), dim3(kReadThreads), 0, s,
                     static_cast<const u32x4_t*>(x), n16, span, out);
  return hipGetLastError();
}

hipError_t launch_calibrate_write(void* y, int64_t nbytes, uint32_t value, int blocks,
                                  hipStream_t s) {
  const int64_t n16 = nbytes / 16;
  const int64_t span = ((n16 + blocks - 1) / blocks + kReadThreads - 1) / kReadThreads * kReadThreads;
  hipLaunchKernelGGL(write_stream_kernel, dim3(unsigned(blocks)), dim3(kReadThreads), 0, s,
                     static_cast<u32x4_t*>(y), n16, span, value);
  return hipGetLastError();
}

}  // namespace fa
