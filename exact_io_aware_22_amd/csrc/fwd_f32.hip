// Exact attention forward for float32 inputs (vector ALU, float32 throughout).
//
// Same fold as the bfloat16 kernel ("Learning FlashAttention the Hard Way -- Part 1",
// sections "The State", "The Merge, and the Twist", "Alternative Twist: Base 2"):
// per query row a running (m, d, o), tiles of 32 keys merged with a 2^{(m_old -
// m_new) c} rescale, masked keys entering as the identity, one division at the end.
// There is no float32 contraction fast enough to be worth the MFMA fp32 path at
// the sizes this serves. Two kernels, by problem size:
//   * small problems (few rows, short keys, such as one head of 256 rows): one to four
//     wavefronts per query row (more for longer rows, so that a row's loads are in
//     flight together), their lanes splitting the keys (16 key lanes) and the head
//     dimension (4 lanes per key, one 16-byte piece of every 64 bytes each). A lane
//     folds its own keys into a private (m, d, o) state; the key lanes' states merge at
//     the end by the same combine, a butterfly over the lanes, and the wavefronts'
//     states through LDS (section "Associativity is All You Need": any bracketing gives
//     the same result). Keys come straight from global memory; there is no reuse to
//     stage.
//   * larger problems: each query row is owned by a pair of lanes that split the head
//     dimension (dims 4i + 2p and 4i + 2p + 1 for lane parity p) and finish each dot
//     product with one cross-lane add. K and V tiles are staged in LDS and read as
//     broadcasts by the 64 rows of a workgroup.
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

// ---------------------------------------------------------------- small problems
constexpr int kSmallWaves = 4;  // wavefronts per workgroup

// A workgroup serves R query rows with 4 / R wavefronts each; wavefront w of a row takes
// the steps t = w, w + W, ... of 16 kG keys (W = 4 / R), so the loads of a short row
// are spread over several wavefronts instead of waiting one step after another.
// Lane l = 4 kk + dd: key lane kk takes keys 16 kG t + 16 g + kk (g < kG); dim lane dd
// takes head dims 16 i + 4 dd .. 16 i + 4 dd + 3 for i < D / 16.
template <int D, bool CAUSAL, int R>
__global__ __launch_bounds__(64 * kSmallWaves) void fwd_f32_rows_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int N, int64_t rows, float c) {
  constexpr int W = kSmallWaves / R;  // wavefronts per row
  constexpr int NV = D / 16;          // 16-byte pieces per lane and row
  // keys per lane and step: their key and value pieces (2 kG NV registers of 16 bytes)
  // stay within the registers of two wavefronts per SIMD
  constexpr int kG = D == 128 ? 2 : 4;
  // each wavefront's state for its row, merged by the row's first wavefront
  __shared__ __attribute__((aligned(16))) float part_o[kSmallWaves][D];
  __shared__ float part_m[kSmallWaves], part_d[kSmallWaves];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = wave / W, w = wave % W;
  const int64_t row = int64_t(blockIdx.x) * R + r;
  const bool live = row < rows;  // every wavefront reaches the barrier below
  const int64_t bh = live ? row / N : 0;
  const int qi = live ? int(row - bh * N) : 0;
  const int kk = lane >> 2, dd = lane & 3;
  const float* kh = K + bh * int64_t(N) * D + 4 * dd;
  const float* vh = V + bh * int64_t(N) * D + 4 * dd;

  f32x4_t qv[NV], ov[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    qv[i] = live ? *reinterpret_cast<const f32x4_t*>(Q + row * D + 16 * i + 4 * dd)
                 : f32x4_t{0.f, 0.f, 0.f, 0.f};
    ov[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  // (m, d) in base-2 units of the scaled scores: m = max s c, d = sum 2^{s c - m}
  float m = kNegInf, d = 0.f;
  const int kv_end = !live ? 0 : (CAUSAL ? qi + 1 : N);
  // Key and value loads of a step are all issued first.
  for (int jb = 16 * kG * w; jb < kv_end; jb += 16 * kG * W) {
    bool ok[kG];
    f32x4_t kr[kG][NV], vr[kG][NV];
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      const int j = jb + 16 * g + kk;
      ok[g] = j < kv_end;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        kr[g][i] = ok[g] ? *reinterpret_cast<const f32x4_t*>(kh + int64_t(j) * D + 16 * i)
                         : f32x4_t{0.f, 0.f, 0.f, 0.f};
        vr[g][i] = ok[g] ? *reinterpret_cast<const f32x4_t*>(vh + int64_t(j) * D + 16 * i)
                         : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
    float sc[kG];
    float mx = kNegInf;
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) a = fmaf(qv[i][e], kr[g][i][e], a);
      // the four dim lanes of a key are one quad
      a += __shfl_xor(a, 1);
      a += __shfl_xor(a, 2);
      sc[g] = ok[g] ? a * c : kNegInf;
      mx = fmaxf(mx, sc[g]);
    }
    const float m_new = fmaxf(m, mx);
    const float mref = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2_hw(m - mref);
    float p[kG];
    float ps = 0.f;
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      p[g] = exp2_hw(sc[g] - mref);
      ps += p[g];
    }
    d = fmaf(d, alpha, ps);
    m = m_new;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float acc = ov[i][e] * alpha;
#pragma unroll
        for (int g = 0; g < kG; ++g) acc = fmaf(p[g], vr[g][i][e], acc);
        ov[i][e] = acc;
      }
  }
  // Merge two states: both brought to the larger maximum (a side at -inf weighs 0; two
  // sides at -inf stay the identity).
  auto merge = [&](float m2, float d2, const f32x4_t (&o2)[NV]) __attribute__((always_inline)) {
    const float mx = fmaxf(m, m2);
    const float mref = mx == kNegInf ? 0.f : mx;
    const float f1 = exp2_hw(m - mref), f2 = exp2_hw(m2 - mref);
    d = fmaf(d, f1, d2 * f2);
    m = mx;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) ov[i][e] = fmaf(ov[i][e], f1, o2[i][e] * f2);
  };
  // the 16 key lanes of a wavefront (lanes 4 apart hold the same dims)
#pragma unroll
  for (int mask = 4; mask < 64; mask <<= 1) {
    f32x4_t o2[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) o2[i][e] = __shfl_xor(ov[i][e], mask);
    merge(__shfl_xor(m, mask), __shfl_xor(d, mask), o2);
  }
  if constexpr (W > 1) {
    // the row's wavefronts, through LDS: each writes its state, the first merges them
    if (kk == 0) {
#pragma unroll
      for (int i = 0; i < NV; ++i)
        *reinterpret_cast<f32x4_t*>(&part_o[wave][16 * i + 4 * dd]) = ov[i];
      if (dd == 0) {
        part_m[wave] = m;
        part_d[wave] = d;
      }
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int u = 1; u < W; ++u) {
        f32x4_t o2[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i)
          o2[i] = *reinterpret_cast<const f32x4_t*>(&part_o[wave + u][16 * i + 4 * dd]);
        merge(part_m[wave + u], part_d[wave + u], o2);
      }
    }
  }
  if (live && w == 0 && kk == 0) {
    const float inv = d > 0.f ? 1.f / d : 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      *reinterpret_cast<f32x4_t*>(O + row * D + 16 * i + 4 * dd) = ov[i] * inv;
    if (dd == 0) LSE[row] = d > 0.f ? (m + log2_hw(d)) * kLn2 : kNegInf;
  }
}

template <int D, bool CAUSAL, int R>
hipError_t launch_small(const FwdArgs& a, hipStream_t s) {
  const int64_t rows = int64_t(a.B) * a.H * a.N;
  const int64_t blocks = (rows + R - 1) / R;
  hipLaunchKernelGGL((fwd_f32_rows_kernel<D, CAUSAL, R>), dim3(unsigned(blocks)),
                     dim3(64 * kSmallWaves), 0, s, static_cast<const float*>(a.q),
                     static_cast<const float*>(a.k), static_cast<const float*>(a.v), a.o, a.lse,
                     a.N, rows, a.scale * kLog2e);
  return hipGetLastError();
}

// The small-problem kernel reads every key of its row from global memory, so it is
// used only while that traffic is small: B H N^2 D <= 2^25 (the single-head N = 256,
// D = 64 problem is 2^22).
bool small_problem(const FwdArgs& a) {
  return double(a.B) * a.H * a.N * a.N * a.D <= 33554432.0;
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t s) {
  if (small_problem(a)) {
    // wavefronts per row: one step of 16 kG keys each for up to four wavefronts
    const int step = D == 128 ? 32 : 64;
    if (a.N > 2 * step) return launch_small<D, CAUSAL, 1>(a, s);
    if (a.N > step) return launch_small<D, CAUSAL, 2>(a, s);
    return launch_small<D, CAUSAL, 4>(a, s);
  }
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
