// Exact attention backward for float32 inputs (vector ALU, float32 throughout).
//
// The same gradients as the bfloat16 kernels (derived by the chain rule from the
// forward definition of "Learning FlashAttention the Hard Way -- Part 1", section
// "FlashAttention: Not So Special"; P recomputed from the forward's log-sum-exp in
// base 2, section "Alternative Twist: Base 2"):
//   Delta_i = sum_d dO_id O_id,  P_ij = 2^{S_ij c - lse_i log2 e},
//   dS_ij = P_ij (dO_i . v_j - Delta_i),  dQ_i = scale sum_j dS_ij k_j,
//   dK_j = scale sum_i dS_ij q_i,  dV_j = sum_i P_ij dO_i.
// One thread owns one output row and loops over the other side's rows; the rows it
// walks are the same for every thread of a wavefront at a time, so they are read as
// broadcasts from L1. This path serves float32 inputs at small sizes; the bfloat16
// kernels are the fast path.
#include "device.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int kT = 128;  // threads per workgroup

template <int D>
__global__ __launch_bounds__(kT) void delta_f32_kernel(const float* __restrict__ dO,
                                                       const float* __restrict__ O,
                                                       float* __restrict__ delta, int64_t rows) {
  const int64_t r = int64_t(blockIdx.x) * kT + threadIdx.x;
  if (r >= rows) return;
  float acc = 0.f;
  for (int d = 0; d < D; ++d) acc = fmaf(dO[r * D + d], O[r * D + d], acc);
  delta[r] = acc;
}

// lse in natural-log units -> base-2 exponent offset; a row that sees no key gets
// +inf, so every P of it is 2^{-inf} = 0.
__device__ __forceinline__ float lse_base2(float l) { return l == kNegInf ? -kNegInf : l * kLog2e; }

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kT) void dq_f32_kernel(const float* __restrict__ Q,
                                                    const float* __restrict__ K,
                                                    const float* __restrict__ V,
                                                    const float* __restrict__ dO,
                                                    const float* __restrict__ LSE,
                                                    const float* __restrict__ DELTA,
                                                    float* __restrict__ dQ, int N, int nrt,
                                                    float c, float scale) {
  const int bh = blockIdx.x / nrt, i = (blockIdx.x % nrt) * kT + threadIdx.x;
  if (i >= N) return;
  const int64_t head = int64_t(bh) * N * D;
  const float* q = Q + head + int64_t(i) * D;
  const float* g = dO + head + int64_t(i) * D;
  const float l2 = lse_base2(LSE[int64_t(bh) * N + i]);
  const float dl = DELTA[int64_t(bh) * N + i];
  float acc[D];
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  const int jend = CAUSAL ? i + 1 : N;
  for (int j = 0; j < jend; ++j) {
    const float* k = K + head + int64_t(j) * D;
    const float* v = V + head + int64_t(j) * D;
    float s = 0.f, dp = 0.f;
    for (int d = 0; d < D; ++d) {
      s = fmaf(q[d], k[d], s);
      dp = fmaf(g[d], v[d], dp);
    }
    const float ds = exp2_hw(fmaf(s, c, -l2)) * (dp - dl);
    for (int d = 0; d < D; ++d) acc[d] = fmaf(ds, k[d], acc[d]);
  }
  float* out = dQ + head + int64_t(i) * D;
  for (int d = 0; d < D; ++d) out[d] = acc[d] * scale;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kT) void dkdv_f32_kernel(const float* __restrict__ Q,
                                                      const float* __restrict__ K,
                                                      const float* __restrict__ V,
                                                      const float* __restrict__ dO,
                                                      const float* __restrict__ LSE,
                                                      const float* __restrict__ DELTA,
                                                      float* __restrict__ dK,
                                                      float* __restrict__ dV, int N, int nrt,
                                                      float c, float scale) {
  const int bh = blockIdx.x / nrt, j = (blockIdx.x % nrt) * kT + threadIdx.x;
  if (j >= N) return;
  const int64_t head = int64_t(bh) * N * D;
  const float* k = K + head + int64_t(j) * D;
  const float* v = V + head + int64_t(j) * D;
  float ak[D], av[D];
  for (int d = 0; d < D; ++d) ak[d] = av[d] = 0.f;
  for (int i = CAUSAL ? j : 0; i < N; ++i) {
    const float* q = Q + head + int64_t(i) * D;
    const float* g = dO + head + int64_t(i) * D;
    float s = 0.f, dp = 0.f;
    for (int d = 0; d < D; ++d) {
      s = fmaf(q[d], k[d], s);
      dp = fmaf(g[d], v[d], dp);
    }
    const float p = exp2_hw(fmaf(s, c, -lse_base2(LSE[int64_t(bh) * N + i])));
    const float ds = p * (dp - DELTA[int64_t(bh) * N + i]);
    for (int d = 0; d < D; ++d) {
      av[d] = fmaf(p, g[d], av[d]);
      ak[d] = fmaf(ds, q[d], ak[d]);
    }
  }
  float* ok = dK + head + int64_t(j) * D;
  float* ov = dV + head + int64_t(j) * D;
  for (int d = 0; d < D; ++d) {
    ok[d] = ak[d] * scale;
    ov[d] = av[d];
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const BwdArgs& a, hipStream_t s) {
  const int64_t BH = int64_t(a.B) * a.H;
  const int64_t rows = BH * a.N;
  const int nrt = int((int64_t(a.N) + kT - 1) / kT);
  const int64_t blocks = BH * nrt, dblocks = (rows + kT - 1) / kT;
  if (blocks > 0x7fffffff || dblocks > 0x7fffffff) return hipErrorInvalidValue;
  const float c = a.scale * kLog2e;
  const auto* q = static_cast<const float*>(a.q);
  const auto* k = static_cast<const float*>(a.k);
  const auto* v = static_cast<const float*>(a.v);
  const auto* g = static_cast<const float*>(a.dout);
  hipLaunchKernelGGL((delta_f32_kernel<D>), dim3(unsigned(dblocks)), dim3(kT), 0, s, g, a.o,
                     a.delta, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((dq_f32_kernel<D, CAUSAL>), dim3(unsigned(blocks)), dim3(kT), 0, s, q, k, v,
                     g, a.lse, a.delta, a.dq, a.N, nrt, c, a.scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((dkdv_f32_kernel<D, CAUSAL>), dim3(unsigned(blocks)), dim3(kT), 0, s, q, k,
                     v, g, a.lse, a.delta, a.dk, a.dv, a.N, nrt, c, a.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_f32(const BwdArgs& a, hipStream_t s) {
  if (a.D == 128) return a.causal ? launch<128, true>(a, s) : launch<128, false>(a, s);
  return a.causal ? launch<64, true>(a, s) : launch<64, false>(a, s);
}

}  // namespace fa
