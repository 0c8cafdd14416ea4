// Split-KV single-query attention ("Learning FlashAttention the Hard Way -- Part 1"):
// decode_partials writes one (m, d, o) state per chunk of keys (split-K, section
// "Associativity is All You Need"; the state of section "The State"); combine
// folds them with the merge of section "The Merge, and the Twist", skipping identity
// states (section "Why Attention's Combine Still Associates"), and reads each row
// out once as o / d with lse = M + ln D.
//
// decode_partials is a pure stream over K and V (about one flop per byte), so it is
// laid out for HBM: a workgroup folds kUnits consecutive (head, chunk) units, one
// after the other, four wavefronts each taking
// 16*R keys per step with non-temporal 16-byte loads that tile whole key rows (R rows
// per wave-wide load), K and V requests issued together, dot products finished with
// cross-lane adds inside a row, and the four wavefronts' states merged in LDS.
#include <mutex>

#include "device.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kLoads = 16;  // 16-byte loads per lane per step, per tensor
// (head, chunk) units per workgroup: consecutive units are consecutive chunks of one
// head, so a workgroup streams one longer contiguous span of K and V. Two measured
// best at the decode workload (1 to 8 tried: 8 and 4 lose more to the last
// workgroups' tail than they gain from longer spans).
constexpr int kUnits = 2;

template <bool BF16, int D>
__global__ __launch_bounds__(64 * kWaves) void decode_partials_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    float* __restrict__ Mo, float* __restrict__ Do, float* __restrict__ Op, int L, int splits,
    int64_t units, int chunk, float c, float scale) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int E = 16 / ESZ;       // elements per 16-byte load
  constexpr int LPR = D / E;        // lanes per key row
  constexpr int RPW = 64 / LPR;     // key rows per wave-wide load
  constexpr int KW = kLoads * RPW;  // keys per wavefront per step
  __shared__ float sm_m[kWaves], sm_d[kWaves];
  __shared__ __attribute__((aligned(16))) float sm_o[kWaves][D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int t = 0; t < kUnits; ++t) {
    const int64_t unit = int64_t(blockIdx.x) * kUnits + t;
    if (unit >= units) break;  // uniform: every thread of the workgroup sees the same unit
    const int split = int(unit % splits);
    const int64_t bh = unit / splits;
    const int64_t j0l = int64_t(split) * chunk;
    const int j0 = int(j0l < L ? j0l : L);
    const int j1 = int(j0l + chunk < L ? j0l + chunk : L);
    const int row = lane / LPR, col = (lane % LPR) * E;
    const int64_t rowbytes = int64_t(D) * ESZ;
    const uint8_t* Kh = K + bh * L * rowbytes + col * ESZ;
    const uint8_t* Vh = V + bh * L * rowbytes + col * ESZ;
    const u32x4_t qw = load16(Q + bh * rowbytes + col * ESZ);

    float m_run = kNegInf, d_run = 0.f;
    float o[E];
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = 0.f;

    for (int jb = j0 + wave * KW; jb < j1; jb += kWaves * KW) {
      u32x4_t kr[kLoads], vr[kLoads];
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int key = jb + i * RPW + row;
        const bool ok = key < j1;
        // Non-temporal: K and V are read once, so nothing is kept in the caches.
        kr[i] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(Kh + int64_t(key) * rowbytes))
                   : u32x4_t{0, 0, 0, 0};
        vr[i] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(Vh + int64_t(key) * rowbytes))
                   : u32x4_t{0, 0, 0, 0};
      }
      float s[kLoads];
      float mx = kNegInf;
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        float p = 0.f;
        if constexpr (BF16) {
#pragma unroll
          for (int w = 0; w < 4; ++w)
            p = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(kr[i][w]), as_bf16x2(qw[w]), p, false);
        } else {
#pragma unroll
          for (int w = 0; w < 4; ++w) p = fmaf(__uint_as_float(kr[i][w]), __uint_as_float(qw[w]), p);
        }
#pragma unroll
        for (int off = 1; off < LPR; off <<= 1) p += __shfl_xor(p, off);
        s[i] = (jb + i * RPW + row < j1) ? p : kNegInf;
        mx = fmaxf(mx, s[i]);
      }
#pragma unroll
      for (int off = LPR; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      const float m_new = fmaxf(m_run, mx);
      const float mref = m_new == kNegInf ? 0.f : m_new;
      const float alpha = exp2_hw((m_run - mref) * c);
      d_run *= alpha;
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] *= alpha;
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        // The maximum is subtracted before scaling, so the largest weight is exactly 1
        // at any magnitude of the scores (the stream is HBM-bound; the extra
        // instruction costs nothing here).
        const float p = exp2_hw((s[i] - mref) * c);
        d_run += p;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if constexpr (BF16) {
            o[2 * w] = fmaf(p, bf16_lo(vr[i][w]), o[2 * w]);
            o[2 * w + 1] = fmaf(p, bf16_hi(vr[i][w]), o[2 * w + 1]);
          } else {
            o[w] = fmaf(p, __uint_as_float(vr[i][w]), o[w]);
          }
        }
      }
      m_run = m_new;
    }

    // Sum the rows of this wavefront (same m everywhere in the wavefront).
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
      d_run += __shfl_xor(d_run, off);
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] += __shfl_xor(o[e], off);
    }
    if (lane < LPR) {
#pragma unroll
      for (int e = 0; e < E; ++e) sm_o[wave][col + e] = o[e];
    }
    if (lane == 0) {
      sm_m[wave] = m_run;
      sm_d[wave] = d_run;
    }
    __syncthreads();

    // Merge the wavefronts' states; write m in natural-log units of the scaled score.
    if (tid < D) {
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w]);
      const float mref = M == kNegInf ? 0.f : M;
      float den = 0.f, acc = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = exp2_hw((sm_m[w] - mref) * c);
        den = fmaf(f, sm_d[w], den);
        acc = fmaf(f, sm_o[w][tid], acc);
      }
      const int64_t out = bh * splits + split;
      Op[out * D + tid] = acc;
      if (tid == 0) {
        Mo[out] = M == kNegInf ? kNegInf : M * scale;
        Do[out] = den;
      }
    }
    __syncthreads();  // the next unit rewrites the merge buffers
  }
}

// Chunks of at most one wavefront step of keys (KW): every wavefront folds whole
// (head, chunk) units by itself, kWaveUnits in turn, and writes each unit's state
// straight from registers. With the four wavefronts of the kernel above sharing such a
// unit, three would have no keys; here none idles and no LDS merge is needed.
constexpr int kWaveUnits = 2;

template <bool BF16, int D>
__global__ __launch_bounds__(64 * kWaves) void decode_partials_wave_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    float* __restrict__ Mo, float* __restrict__ Do, float* __restrict__ Op, int L, int splits,
    int64_t units, int chunk, float c, float scale) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int E = 16 / ESZ;       // elements per 16-byte load
  constexpr int LPR = D / E;        // lanes per key row
  constexpr int RPW = 64 / LPR;     // key rows per wave-wide load
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane / LPR, col = (lane % LPR) * E;
  const int64_t rowbytes = int64_t(D) * ESZ;
  for (int t = 0; t < kWaveUnits; ++t) {
    const int64_t unit = (int64_t(blockIdx.x) * kWaves + wave) * kWaveUnits + t;
    if (unit >= units) break;  // uniform within the wavefront
    const int split = int(unit % splits);
    const int64_t bh = unit / splits;
    const int64_t j0l = int64_t(split) * chunk;
    const int j0 = int(j0l < L ? j0l : L);
    const int j1 = int(j0l + chunk < L ? j0l + chunk : L);  // j1 - j0 <= kLoads * RPW
    const uint8_t* Kh = K + bh * L * rowbytes + col * ESZ;
    const uint8_t* Vh = V + bh * L * rowbytes + col * ESZ;
    const u32x4_t qw = load16(Q + bh * rowbytes + col * ESZ);
    u32x4_t kr[kLoads], vr[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int key = j0 + i * RPW + row;
      const bool ok = key < j1;
      kr[i] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(Kh + int64_t(key) * rowbytes))
                 : u32x4_t{0, 0, 0, 0};
      vr[i] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(Vh + int64_t(key) * rowbytes))
                 : u32x4_t{0, 0, 0, 0};
    }
    float s[kLoads];
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      float p = 0.f;
      if constexpr (BF16) {
#pragma unroll
        for (int w = 0; w < 4; ++w)
          p = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(kr[i][w]), as_bf16x2(qw[w]), p, false);
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) p = fmaf(__uint_as_float(kr[i][w]), __uint_as_float(qw[w]), p);
      }
#pragma unroll
      for (int off = 1; off < LPR; off <<= 1) p += __shfl_xor(p, off);
      s[i] = (j0 + i * RPW + row < j1) ? p : kNegInf;
      mx = fmaxf(mx, s[i]);
    }
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    const float mref = mx == kNegInf ? 0.f : mx;
    float den = 0.f;
    float o[E];
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = 0.f;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const float p = exp2_hw((s[i] - mref) * c);  // maximum subtracted before scaling
      den += p;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if constexpr (BF16) {
          o[2 * w] = fmaf(p, bf16_lo(vr[i][w]), o[2 * w]);
          o[2 * w + 1] = fmaf(p, bf16_hi(vr[i][w]), o[2 * w + 1]);
        } else {
          o[w] = fmaf(p, __uint_as_float(vr[i][w]), o[w]);
        }
      }
    }
    // Sum the key rows of the wavefront (one reference maximum for all of them).
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
      den += __shfl_xor(den, off);
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] += __shfl_xor(o[e], off);
    }
    const int64_t out = bh * splits + split;
    if (lane < LPR) {
#pragma unroll
      for (int e = 0; e < E; ++e) Op[out * D + col + e] = o[e];
    }
    if (lane == 0) {
      Mo[out] = mx == kNegInf ? kNegInf : mx * scale;
      Do[out] = den;
    }
  }
}

template <bool BF16, int D>
hipError_t launch_partials(const DecodeArgs& a, hipStream_t s) {
  const int64_t BH = int64_t(a.B) * a.H;
  const int64_t units = BH * a.splits;
  const int chunk = int((int64_t(a.L) + a.splits - 1) / a.splits);
  constexpr int KW = kLoads * (64 / (D / (16 / (BF16 ? 2 : 4))));  // keys per wavefront step
  if (chunk <= KW) {
    const int64_t per_block = int64_t(kWaves) * kWaveUnits;
    const int64_t blocks = (units + per_block - 1) / per_block;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_partials_wave_kernel<BF16, D>), dim3(unsigned(blocks)),
                       dim3(64 * kWaves), 0, s, static_cast<const uint8_t*>(a.q),
                       static_cast<const uint8_t*>(a.k), static_cast<const uint8_t*>(a.v), a.m,
                       a.d, a.o_part, a.L, a.splits, units, chunk, a.scale * kLog2e, a.scale);
    return hipGetLastError();
  }
  const int64_t blocks = (units + kUnits - 1) / kUnits;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_partials_kernel<BF16, D>), dim3(unsigned(blocks)), dim3(64 * kWaves),
                     0, s, static_cast<const uint8_t*>(a.q), static_cast<const uint8_t*>(a.k),
                     static_cast<const uint8_t*>(a.v), a.m, a.d, a.o_part, a.L, a.splits, units,
                     chunk, a.scale * kLog2e, a.scale);
  return hipGetLastError();
}

// One workgroup of 256 threads per row: thread t owns the four head dims 4 (t mod D/4)
// .. + 3 of group t / (D/4); the groups split the partials between them. First the
// row's maximum (every thread strides over the partials' m, then a workgroup
// reduction), then each group folds its partials with weights e^{m_s - M}, four
// 16-byte partial pieces in flight per thread, and the groups' sums are added in LDS.
// Identity partials (m = -inf) contribute nothing.
constexpr int kCombineThreads = 256;

template <int D>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const float* __restrict__ M,
                                                                 const float* __restrict__ Dn,
                                                                 const float* __restrict__ Op,
                                                                 float* __restrict__ O,
                                                                 float* __restrict__ LSE,
                                                                 int splits) {
  constexpr int TPR = D / 4;                  // threads per partial (four floats each)
  constexpr int G = kCombineThreads / TPR;    // groups of partials
  __shared__ float red[kCombineThreads / 64];
  __shared__ f32x4_t acc_s[G][TPR];
  __shared__ float den_s[G];
  const int64_t r = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int q = t % TPR, g = t / TPR;
  const float* mr = M + r * splits;
  const float* dr = Dn + r * splits;
  const f32x4_t* orow = reinterpret_cast<const f32x4_t*>(Op + r * splits * D) + q;

  float mx = kNegInf;
  for (int s = t; s < splits; s += kCombineThreads) mx = fmaxf(mx, mr[s]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kCombineThreads / 64; ++w) mx = fmaxf(mx, red[w]);
  const float mref = mx == kNegInf ? 0.f : mx;

  float den = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  auto fold = [&](float ms, float ds, f32x4_t os) __attribute__((always_inline)) {
    if (ms == kNegInf) return;  // the identity contributes nothing
    const float f = exp2_hw((ms - mref) * kLog2e);
    den = fmaf(f, ds, den);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(f, os[i], acc[i]);
  };
  int s = g;
  for (; s + 3 * G < splits; s += 4 * G) {
    float ms[4], ds[4];
    f32x4_t os[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ms[u] = mr[s + u * G];
      ds[u] = dr[s + u * G];
      os[u] = orow[int64_t(s + u * G) * TPR];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) fold(ms[u], ds[u], os[u]);
  }
  for (; s < splits; s += G) fold(mr[s], dr[s], orow[int64_t(s) * TPR]);
  acc_s[g][q] = acc;
  if (q == 0) den_s[g] = den;
  __syncthreads();
  if (g == 0) {
    f32x4_t a = acc;
    float dn = den;
#pragma unroll
    for (int h = 1; h < G; ++h) {
      const f32x4_t o = acc_s[h][q];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] += o[i];
      dn += den_s[h];
    }
    f32x4_t out;
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = dn > 0.f ? a[i] / dn : 0.f;
    *reinterpret_cast<f32x4_t*>(O + r * D + 4 * q) = out;
    if (q == 0) LSE[r] = dn > 0.f ? mx + logf(dn) : kNegInf;
  }
}

// Static scratch of the allocation-free decode: the partial states (m, d, then o_part)
// of one call. Each GPU the library runs on holds its own copy at its own address. In
// host code `scratch` only names the symbol: kernels get the device address looked up
// below, never the array's name.
__device__ __align__(256) float scratch[kDecodeScratchFloats];

constexpr int kMaxDevices = 64;

// The current device's address of `scratch`, looked up on the first call on that
// device (with it current) and kept for later calls.
hipError_t scratch_address(float** out) {
  static std::mutex mu;
  static float* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = static_cast<float*>(p);
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace

int64_t decode_noalloc_floats(int64_t units, int D) {
  const int64_t padded = (units + 63) / 64 * 64;  // keeps o_part 256-byte aligned
  return 2 * padded + units * D;
}

hipError_t launch_decode_noalloc(const DecodeArgs& a, bool bf16, float* o, float* lse,
                                 hipStream_t s) {
  float* base = nullptr;
  hipError_t e = scratch_address(&base);
  if (e != hipSuccess) return e;
  const int64_t rows = int64_t(a.B) * a.H;
  const int64_t padded = (rows * a.splits + 63) / 64 * 64;
  DecodeArgs p = a;
  p.m = base;
  p.d = base + padded;
  p.o_part = base + 2 * padded;
  e = bf16 ? launch_decode_partials_bf16(p, s) : launch_decode_partials_f32(p, s);
  if (e != hipSuccess) return e;
  const CombineArgs c{p.m, p.d, p.o_part, o, lse, int(rows), a.splits, a.D};
  return launch_combine_partials(c, s);
}

hipError_t launch_decode_partials_bf16(const DecodeArgs& a, hipStream_t s) {
  return a.D == 128 ? launch_partials<true, 128>(a, s) : launch_partials<true, 64>(a, s);
}

hipError_t launch_decode_partials_f32(const DecodeArgs& a, hipStream_t s) {
  return a.D == 128 ? launch_partials<false, 128>(a, s) : launch_partials<false, 64>(a, s);
}

hipError_t launch_combine_partials(const CombineArgs& a, hipStream_t s) {
  if (a.D == 128)
    hipLaunchKernelGGL((combine_kernel<128>), dim3(unsigned(a.rows)), dim3(kCombineThreads), 0,
                       s, a.m, a.d, a.o_part, a.o, a.lse, a.splits);
  else
    hipLaunchKernelGGL((combine_kernel<64>), dim3(unsigned(a.rows)), dim3(kCombineThreads), 0, s,
                       a.m, a.d, a.o_part, a.o, a.lse, a.splits);
  return hipGetLastError();
}

}  // namespace fa
