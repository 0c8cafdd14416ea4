// Exact attention forward for float32 inputs (vector ALU, float32 throughout).
//
// Same fold as the bfloat16 kernel ("Learning FlashAttention the Hard Way -- Part 1",
// sections "The State", "The Merge, and the Twist", "Alternative Twist: Base 2"):
// per query row a running (m, d, o), tiles of 32 keys merged with a 2^{(m_old -
// m_new) c} rescale, masked keys entering as the identity, one division at the end.
// There is no float32 contraction fast enough to be worth the MFMA fp32 path at
// the sizes this serves, so each query row is owned by a pair of lanes that split
// the head dimension (dims 4i + 2p and 4i + 2p + 1 for lane parity p) and finish
// each dot product with one cross-lane add. K and V tiles are staged in LDS and
// read as broadcasts.
#include "device.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int kQ = 64;        // query rows per workgroup
constexpr int kKT = 32;       // keys per tile
constexpr int kThreads = 128; // two lanes per query row

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(const float* __restrict__ Q,
                                                           const float* __restrict__ K,
                                                           const float* __restrict__ V,
                                                           float* __restrict__ O,
                                                           float* __restrict__ LSE, int N,
                                                           int nqt, float c) {
  constexpr int NP = D / 4;  // float2 pairs per lane
  __shared__ __attribute__((aligned(16))) float ks[kKT * D];
  __shared__ __attribute__((aligned(16))) float vs[kKT * D];

  const int tid = threadIdx.x, part = tid & 1;
  const int bh = blockIdx.x / nqt, qt = blockIdx.x % nqt;
  const int q0 = qt * kQ, qi = q0 + (tid >> 1);
  const int64_t head = int64_t(bh) * N * D;

  f32x2_t qv[NP], ov[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    qv[i] = qi < N ? *reinterpret_cast<const f32x2_t*>(Q + head + int64_t(qi) * D + 4 * i + 2 * part)
                   : f32x2_t{0.f, 0.f};
    ov[i] = f32x2_t{0.f, 0.f};
  }
  float m_run = kNegInf, d_run = 0.f;

  const int kv_end = CAUSAL ? min(N, q0 + kQ) : N;
  for (int k0 = 0; k0 < kv_end; k0 += kKT) {
    // Stage the tile; keys past the end are zero and masked below.
    for (int idx = tid; idx < kKT * D / 4; idx += kThreads) {
      const int key = idx / (D / 4), col = (idx % (D / 4)) * 4;
      const int gk = k0 + key;
      f32x4_t kk = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (gk < N) {
        kk = *reinterpret_cast<const f32x4_t*>(K + head + int64_t(gk) * D + col);
        vv = *reinterpret_cast<const f32x4_t*>(V + head + int64_t(gk) * D + col);
      }
      *reinterpret_cast<f32x4_t*>(ks + key * D + col) = kk;
      *reinterpret_cast<f32x4_t*>(vs + key * D + col) = vv;
    }
    __syncthreads();

    float s[kKT];
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < kKT; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const f32x2_t kk = *reinterpret_cast<const f32x2_t*>(ks + j * D + 4 * i + 2 * part);
        acc = fmaf(qv[i][0], kk[0], acc);
        acc = fmaf(qv[i][1], kk[1], acc);
      }
      acc += __shfl_xor(acc, 1);
      const int key = k0 + j;
      if (key >= N || (CAUSAL && key > qi)) acc = kNegInf;
      s[j] = acc;
      mx = fmaxf(mx, acc);
    }
    const float m_new = fmaxf(m_run, mx);
    const float mref = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2_hw((m_run - mref) * c);
    const float nmc = -mref * c;
    d_run *= alpha;
#pragma unroll
    for (int i = 0; i < NP; ++i) ov[i] *= alpha;
#pragma unroll
    for (int j = 0; j < kKT; ++j) {
      const float p = exp2_hw(fmaf(s[j], c, nmc));
      d_run += p;
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const f32x2_t vv = *reinterpret_cast<const f32x2_t*>(vs + j * D + 4 * i + 2 * part);
        ov[i][0] = fmaf(p, vv[0], ov[i][0]);
        ov[i][1] = fmaf(p, vv[1], ov[i][1]);
      }
    }
    m_run = m_new;
    __syncthreads();
  }

  if (qi < N) {
    const float inv = d_run > 0.f ? 1.f / d_run : 0.f;
#pragma unroll
    for (int i = 0; i < NP; ++i)
      *reinterpret_cast<f32x2_t*>(O + head + int64_t(qi) * D + 4 * i + 2 * part) = ov[i] * inv;
    if (part == 0)
      LSE[int64_t(bh) * N + qi] = d_run > 0.f ? (m_run * c + log2_hw(d_run)) * kLn2 : kNegInf;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t s) {
  const int nqt = int((int64_t(a.N) + kQ - 1) / kQ);
  const int64_t blocks = int64_t(a.B) * a.H * nqt;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3(unsigned(blocks)), dim3(kThreads), 0, s,
                     static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                     static_cast<const float*>(a.v), a.o, a.lse, a.N, nqt, a.scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s) {
  if (a.D == 128) return a.causal ? launch<128, true>(a, s) : launch<128, false>(a, s);
  return a.causal ? launch<64, true>(a, s) : launch<64, false>(a, s);
}

}  // namespace fa
