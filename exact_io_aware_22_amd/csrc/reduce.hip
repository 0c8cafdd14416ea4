// Row reductions over a monoid on one schedule: the online-softmax normaliser (m, d)
// and Welford's moments (n, mu, M2), each over the rows of a [rows][n] matrix.
//
// Method ("Learning FlashAttention the Hard Way -- Part 1"): a reduction parallelises
// exactly when its combine is associative and has an identity (section "Associativity
// is All You Need"), and then only the combine changes from one reduction to another,
// never the schedule. The schedule here is the one attention uses for its keys: each
// lane folds a strided share of the row into a private state, then lanes merge
// pairwise across the wavefront, then wavefronts merge through LDS. The monoids:
//   * SoftmaxMonoid: the carrier (m, d), m the running maximum and d the denominator
//     relative to it; a score enters as (x, 1); two states merge by rescaling both
//     denominators to the larger maximum; identity (-inf, 0) (section "Online Softmax
//     Reparametrization"). Exponentials are base 2 with log2(e) folded in (section
//     "Alternative Twist: Base 2").
//   * WelfordMonoid: the carrier (n, mu, M2), count, mean and sum of squared
//     deviations; a sample enters as (1, x, 0); partials over disjoint chunks merge
//     by the Chan-Golub-LeVeque pairwise rule; identity (0, 0, 0) (section "The Same
//     Move: Welford's Variance").
//
// A lane's share arrives 8 elements at a time (one 16-byte load of bf16, two of
// float32, each part of a contiguous run across the lanes); the 8 are folded into a
// block state first (the fold of their 8
// injections, evaluated directly: maximum and shifted sum; mean and squared
// deviations), which then merges into the lane's running state. Row heads before the
// first 16-byte boundary and tails after the last whole block are injected one
// element at a time, so rows need only element alignment.
//
// HBM-bound by design: every element is read once, and the per-element work (about
// five vector instructions) stays well under the vector-ALU rate at full HBM
// bandwidth.
#include "device.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int kK = 8;  // elements per block

// ---------------------------------------------------------------- the two monoids
struct SoftmaxMonoid {
  struct S {
    float m, d;  // m: exact maximum of the elements seen (natural units); d relative to it
  };
  __device__ static S identity() { return {kNegInf, 0.f}; }
  __device__ static S inject(float x) { return x == kNegInf ? identity() : S{x, 1.f}; }
  // Both sides rescaled to the larger maximum: the side that holds it keeps its d, the
  // other is scaled by e^{(its m) - m}, one exponential per combine. A side at -inf
  // contributes 2^-inf = 0; when both are -inf the factor is 0 and no -inf - (-inf)
  // arises.
  __device__ static S combine(S a, S b) {
    const float m = fmaxf(a.m, b.m), lo = fminf(a.m, b.m);
    const float e = m == kNegInf ? 0.f : exp2_hw((lo - m) * kLog2e);
    return {m, a.m >= b.m ? fmaf(b.d, e, a.d) : fmaf(a.d, e, b.d)};
  }
  // Merge the fold of K injections into s: the running maximum takes the block's
  // maximum, d is rescaled once to it, then the block's shifted exponentials add.
  template <int K>
  __device__ static S absorb(S s, const float (&x)[K]) {
    float mx = fmaxf(x[0], x[1]);
#pragma unroll
    for (int i = 2; i < K; ++i) mx = fmaxf(mx, x[i]);
    const float m = fmaxf(s.m, mx);
    const float mr = m == kNegInf ? 0.f : m;
    float d = s.d * exp2_hw((s.m - mr) * kLog2e);
#pragma unroll
    for (int i = 0; i < K; ++i) d += exp2_hw((x[i] - mr) * kLog2e);
    return {m, d};
  }
  __device__ static S shfl_xor(S s, int mask) {
    return {__shfl_xor(s.m, mask), __shfl_xor(s.d, mask)};
  }
  __device__ static S shfl_up(S s, int delta) {
    return {__shfl_up(s.m, delta), __shfl_up(s.d, delta)};
  }
  __device__ static void store(S s, float* out0, float* out1, int64_t row) {
    out0[row] = s.m;
    out1[row] = s.d;
  }
  __device__ static float first(S s) { return s.m; }
  __device__ static float second(S s) { return s.d; }
};

struct WelfordMonoid {
  struct S {
    float n, mu, m2;  // count (exact: integers below 2^24 per lane), mean, M2
  };
  __device__ static S identity() { return {0.f, 0.f, 0.f}; }
  __device__ static S inject(float x) { return {1.f, x, 0.f}; }
  // Chan-Golub-LeVeque: n = na + nb, mu = mu_a + delta nb / n, M2 = M2a + M2b +
  // delta^2 na nb / n, delta = mu_b - mu_a. A side with n = 0 contributes nothing.
  __device__ static S combine(S a, S b) {
    const float n = a.n + b.n;
    if (n == 0.f) return identity();
    const float delta = b.mu - a.mu, r = b.n * __builtin_amdgcn_rcpf(n);
    return {n, a.mu + delta * r, a.m2 + b.m2 + delta * delta * a.n * r};
  }
  // The block's own triple (K, mean, squared deviations from it), merged into s.
  template <int K>
  __device__ static S absorb(S s, const float (&x)[K]) {
    float sum = x[0] + x[1];
#pragma unroll
    for (int i = 2; i < K; ++i) sum += x[i];
    const float mu = sum * (1.f / K);
    float m2 = 0.f;
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const float e = x[i] - mu;
      m2 = fmaf(e, e, m2);
    }
    return combine(s, S{float(K), mu, m2});
  }
  __device__ static S shfl_xor(S s, int mask) {
    return {__shfl_xor(s.n, mask), __shfl_xor(s.mu, mask), __shfl_xor(s.m2, mask)};
  }
  __device__ static S shfl_up(S s, int delta) {
    return {__shfl_up(s.n, delta), __shfl_up(s.mu, delta), __shfl_up(s.m2, delta)};
  }
  __device__ static void store(S s, float* out0, float* out1, int64_t row) {
    out0[row] = s.mu;
    out1[row] = s.m2;
  }
  __device__ static float first(S s) { return s.mu; }
  __device__ static float second(S s) { return s.m2; }
};

// ---------------------------------------------------------------- element access
// One 16-byte load (4 float32 or 8 bfloat16) as floats. Non-temporal: every element is
// read once, so there is nothing to keep in the caches.
template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kVec = 4;
  __device__ static float scalar(const float* p) { return *p; }
  __device__ static void vec(const float* p, float (&x)[kVec]) {
    const f32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = a[i];
  }
};
template <>
struct Elem<uint16_t> {  // bfloat16 bits
  static constexpr int kVec = 8;
  __device__ static float scalar(const uint16_t* p) { return __uint_as_float(uint32_t(*p) << 16); }
  __device__ static void vec(const uint16_t* p, float (&x)[kVec]) {
    const u32x4_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t wi = w[i];
      x[2 * i] = bf16_lo(wi);
      x[2 * i + 1] = bf16_hi(wi);
    }
  }
};

// ---------------------------------------------------------------- the schedule
// WPR wavefronts (G = 64 * WPR lanes) per row; a 256-thread workgroup holds 4 / WPR
// rows. The row (after its unaligned head) is read in rounds of G blocks of 8
// elements: in a round, load j of every lane reads G consecutive 16-byte vectors
// (lane t takes vector j * G + t), so each load instruction is one contiguous run;
// a lane's 8 elements (two float32 vectors or one bf16 vector) fold into one block
// state. Four rounds' loads are in flight before they are folded. Whole vectors left
// after the last round, then single elements, follow. The group then merges:
// pairwise across each wavefront (xor butterfly), then across wavefronts through LDS.
template <class M, typename T, int WPR>
__global__ __launch_bounds__(256) void row_reduce_kernel(const T* __restrict__ x, int64_t rows,
                                                       int n, float* __restrict__ out0,
                                                       float* __restrict__ out1) {
  using S = typename M::S;
  constexpr int G = 64 * WPR;
  constexpr int RPB = 4 / WPR;        // rows per workgroup
  constexpr int VEC = Elem<T>::kVec;  // elements per 16-byte load
  constexpr int VPB = kK / VEC;       // loads per block of 8
  constexpr int ROUND = G * kK;       // elements per round
  __shared__ S part[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = tid % G;  // lane within the row's group
  const int64_t row = int64_t(blockIdx.x) * RPB + tid / G;
  S s = M::identity();
  if (row < rows) {
    const T* p = x + row * int64_t(n);
    // head: elements before the first 16-byte boundary (fewer than VEC)
    const int mis = int((reinterpret_cast<uintptr_t>(p) & 15) / sizeof(T));
    const int head = min(n, mis == 0 ? 0 : VEC - mis);
    if (t < head) s = M::combine(s, M::inject(Elem<T>::scalar(p + t)));
    const T* body = p + head;
    const int nel = n - head;
    const int nrounds = nel / ROUND;
    // lane t's block in round r: vectors j * G + t, j < VPB
    auto load_block = [&](int r, float (&v)[kK]) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < VPB; ++j) {
        float w[VEC];
        Elem<T>::vec(body + int64_t(r) * ROUND + (j * G + t) * VEC, w);
#pragma unroll
        for (int i = 0; i < VEC; ++i) v[j * VEC + i] = w[i];
      }
    };
    int r = 0;
    for (; r + 3 < nrounds; r += 4) {
      float v0[kK], v1[kK], v2[kK], v3[kK];
      load_block(r, v0);
      load_block(r + 1, v1);
      load_block(r + 2, v2);
      load_block(r + 3, v3);
      s = M::absorb(s, v0);
      s = M::absorb(s, v1);
      s = M::absorb(s, v2);
      s = M::absorb(s, v3);
    }
    for (; r < nrounds; ++r) {
      float v[kK];
      load_block(r, v);
      s = M::absorb(s, v);
    }
    // whole vectors after the last round, then single elements (fewer than VEC)
    const T* rest = body + int64_t(nrounds) * ROUND;
    const int nleft = nel - nrounds * ROUND, nvec = nleft / VEC;
    for (int v = t; v < nvec; v += G) {
      float w[VEC];
      Elem<T>::vec(rest + v * VEC, w);
      s = M::absorb(s, w);
    }
    for (int e = nvec * VEC + t; e < nleft; e += G) s = M::combine(s, M::inject(Elem<T>::scalar(rest + e)));
  }
  // merge across the wavefront: every lane ends with the wavefront's state
#pragma unroll
  for (int mask = 32; mask >= 1; mask >>= 1) s = M::combine(s, M::shfl_xor(s, mask));
  if constexpr (WPR > 1) {
    if (lane == 0) part[wave] = s;
    __syncthreads();
    if (tid == 0) {
#pragma unroll
      for (int w = 1; w < WPR; ++w) s = M::combine(s, part[w]);
      if (row < rows) M::store(s, out0, out1, row);
    }
  } else {
    if (lane == 0 && row < rows) M::store(s, out0, out1, row);
  }
}

// ---------------------------------------------------------------- the prefix scan
// Inclusive scan of every row: output j is the state of elements 0..j. A prefix scan is
// one more re-bracketing any monoid allows (section "Wrap-Up", first point), here on
// the same pieces: one 256-thread workgroup per row, the row in blocks of 256 x 8
// elements. Thread t folds its 8 consecutive elements left to right (keeping each
// partial state), the 256 thread totals are scanned (an inclusive scan across each
// wavefront with shfl_up, then the four wavefront totals through LDS), and element i
// of thread t is written as carry + (totals of threads before t) + (its own partial i);
// the block's total joins the carry for the next block. ALIGNED: x and both outputs
// start on 16-byte boundaries and rows are whole 16-byte multiples, so a thread's 8
// elements are read and written with vector accesses.
template <class M, typename T, bool ALIGNED>
__global__ __launch_bounds__(256) void row_scan_kernel(const T* __restrict__ x, int n,
                                                     float* __restrict__ out0,
                                                     float* __restrict__ out1) {
  using S = typename M::S;
  __shared__ S wtot[4];
  // A whole block's outputs go out through LDS so that every store instruction writes
  // 1 KB of consecutive floats (a thread's own 8 results are 32 bytes apart per lane).
  __shared__ __attribute__((aligned(16))) float stage[2][256 * kK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const T* p = x + row * int64_t(n);
  float* o0 = out0 + row * int64_t(n);
  float* o1 = out1 + row * int64_t(n);
  S carry = M::identity();
  for (int base = 0; base < n; base += 256 * kK) {
    const int e0 = base + kK * tid;
    S st[kK];
    S run = M::identity();
    if (ALIGNED && e0 + kK <= n) {
      float v[kK];
#pragma unroll
      for (int j = 0; j < kK / Elem<T>::kVec; ++j) {
        float w[Elem<T>::kVec];
        Elem<T>::vec(p + e0 + j * Elem<T>::kVec, w);
#pragma unroll
        for (int i = 0; i < Elem<T>::kVec; ++i) v[j * Elem<T>::kVec + i] = w[i];
      }
#pragma unroll
      for (int i = 0; i < kK; ++i) {
        run = M::combine(run, M::inject(v[i]));
        st[i] = run;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kK; ++i) {
        if (e0 + i < n) run = M::combine(run, M::inject(Elem<T>::scalar(p + e0 + i)));
        st[i] = run;
      }
    }
    // inclusive scan of the thread totals across the wavefront
    S tot = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const S o = M::shfl_up(tot, off);
      if (lane >= off) tot = M::combine(o, tot);
    }
    S excl = M::shfl_up(tot, 1);  // totals of the lanes before this one
    if (lane == 0) excl = M::identity();
    if (lane == 63) wtot[wave] = tot;
    __syncthreads();
    S pre = carry, blk = carry;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (w < wave) pre = M::combine(pre, wtot[w]);
      blk = M::combine(blk, wtot[w]);
    }
    pre = M::combine(pre, excl);
    __syncthreads();  // wtot is rewritten by the next block
    float r0[kK], r1[kK];
#pragma unroll
    for (int i = 0; i < kK; ++i) {
      const S r = M::combine(pre, st[i]);
      r0[i] = M::first(r);
      r1[i] = M::second(r);
    }
    if (ALIGNED && base + 256 * kK <= n) {  // uniform: the whole block is in the row
#pragma unroll
      for (int j = 0; j < kK; j += 4) {
        *reinterpret_cast<f32x4_t*>(&stage[0][kK * tid + j]) = f32x4_t{r0[j], r0[j + 1], r0[j + 2], r0[j + 3]};
        *reinterpret_cast<f32x4_t*>(&stage[1][kK * tid + j]) = f32x4_t{r1[j], r1[j + 1], r1[j + 2], r1[j + 3]};
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kK / 4; ++q) {
        const int f = 4 * (tid + 256 * q);
        *reinterpret_cast<f32x4_t*>(o0 + base + f) = *reinterpret_cast<const f32x4_t*>(&stage[0][f]);
        *reinterpret_cast<f32x4_t*>(o1 + base + f) = *reinterpret_cast<const f32x4_t*>(&stage[1][f]);
      }
      // stage is rewritten by the next block only after that block's two barriers
    } else if (ALIGNED && e0 + kK <= n) {
#pragma unroll
      for (int j = 0; j < kK; j += 4) {
        *reinterpret_cast<f32x4_t*>(o0 + e0 + j) = f32x4_t{r0[j], r0[j + 1], r0[j + 2], r0[j + 3]};
        *reinterpret_cast<f32x4_t*>(o1 + e0 + j) = f32x4_t{r1[j], r1[j + 1], r1[j + 2], r1[j + 3]};
      }
    } else {
#pragma unroll
      for (int i = 0; i < kK; ++i)
        if (e0 + i < n) {
          o0[e0 + i] = r0[i];
          o1[e0 + i] = r1[i];
        }
    }
    carry = blk;
  }
}

template <class M, typename T>
hipError_t launch_scan(const RowReduceArgs& a, hipStream_t st) {
  if (a.rows > 0x7fffffff) return hipErrorInvalidValue;
  const T* x = static_cast<const T*>(a.x);
  const bool aligned = (reinterpret_cast<uintptr_t>(a.x) & 15) == 0 &&
                       (reinterpret_cast<uintptr_t>(a.out0) & 15) == 0 &&
                       (reinterpret_cast<uintptr_t>(a.out1) & 15) == 0 && (a.n % kK) == 0;
  if (aligned)
    hipLaunchKernelGGL((row_scan_kernel<M, T, true>), dim3(unsigned(a.rows)), dim3(256), 0, st, x,
                       a.n, a.out0, a.out1);
  else
    hipLaunchKernelGGL((row_scan_kernel<M, T, false>), dim3(unsigned(a.rows)), dim3(256), 0, st,
                       x, a.n, a.out0, a.out1);
  return hipGetLastError();
}

template <class M, typename T>
hipError_t launch_rows(const RowReduceArgs& a, hipStream_t st) {
  // Four wavefronts share a row: measured faster than one wavefront per row on the
  // 1 GiB workloads (65536 rows of 8192 bf16 and 8192 rows of 32768 float32): each
  // lane has fewer blocks to fold, so more of them are in flight at once. Rows
  // shorter than 8 * 256 elements leave lanes idle; one wavefront per row serves
  // those when rows are plentiful.
  const bool wave_per_row = a.n < 2048 && a.rows >= 8192;
  const int64_t blocks = wave_per_row ? (a.rows + 3) / 4 : a.rows;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const T* x = static_cast<const T*>(a.x);
  if (wave_per_row)
    hipLaunchKernelGGL((row_reduce_kernel<M, T, 1>), dim3(unsigned(blocks)), dim3(256), 0, st, x,
                       a.rows, a.n, a.out0, a.out1);
  else
    hipLaunchKernelGGL((row_reduce_kernel<M, T, 4>), dim3(unsigned(blocks)), dim3(256), 0, st, x,
                       a.rows, a.n, a.out0, a.out1);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_softmax_stats(const RowReduceArgs& a, hipStream_t s) {
  return a.bf16 ? launch_rows<SoftmaxMonoid, uint16_t>(a, s) : launch_rows<SoftmaxMonoid, float>(a, s);
}

hipError_t launch_moments(const RowReduceArgs& a, hipStream_t s) {
  return a.bf16 ? launch_rows<WelfordMonoid, uint16_t>(a, s) : launch_rows<WelfordMonoid, float>(a, s);
}

hipError_t launch_softmax_scan(const RowReduceArgs& a, hipStream_t s) {
  return a.bf16 ? launch_scan<SoftmaxMonoid, uint16_t>(a, s) : launch_scan<SoftmaxMonoid, float>(a, s);
}

hipError_t launch_moments_scan(const RowReduceArgs& a, hipStream_t s) {
  return a.bf16 ? launch_scan<WelfordMonoid, uint16_t>(a, s) : launch_scan<WelfordMonoid, float>(a, s);
}

}  // namespace fa
