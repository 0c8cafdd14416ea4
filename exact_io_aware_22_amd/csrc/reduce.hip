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

// v moved between lanes by the data-parallel primitive CTRL, written only in the rows of
// 16 lanes that ROWS selects; a lane that is not written, or whose source lies outside
// its row, gets `fill`.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp(float fill, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, fill),
                                                               __builtin_bit_cast(int, v), CTRL,
                                                               ROWS, 0xf, false));
}

// Lane l's value of v, for every lane (a scalar register read).
__device__ __forceinline__ float readlane(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// ---------------------------------------------------------------- the two monoids
struct SoftmaxMonoid {
  struct S {
    float m, d;  // m: exact maximum of the elements seen (natural units); d relative to it
  };
  __device__ static S identity() { return {kNegInf, 0.f}; }
  __device__ static S inject(float x) { return x == kNegInf ? identity() : S{x, 1.f}; }
  // Both sides rescaled to the larger maximum: the side that holds it keeps its d, the
  // other is scaled by e^{-|b.m - a.m|}, one exponential per combine. A side at -inf
  // contributes 2^-inf = 0; when both are -inf the difference is NaN, which the maximum
  // with -inf (it returns the number) turns into -inf, so d = 0 + 0 stays exact. The
  // maximum of the two m is IEEE 754-2019's, which takes its operands as they are (no
  // quieting step).
  __device__ static S combine(S a, S b) {
    const float t = fmaxf((b.m - a.m) * kLog2e, kNegInf);
    const float e = exp2_hw(-fabsf(t));
    return {__builtin_elementwise_maximum(a.m, b.m), t <= 0.f ? fmaf(b.d, e, a.d) : fmaf(a.d, e, b.d)};
  }
  // combine(s, inject(x)), with the injected d = 1 folded in.
  __device__ static S push(S s, float x) {
    const float t = fmaxf((x - s.m) * kLog2e, kNegInf);
    const float e = exp2_hw(-fabsf(t));
    return {__builtin_elementwise_maximum(s.m, x), t <= 0.f ? s.d + e : fmaf(s.d, e, 1.f)};
  }
  // Merge the fold of K injections into s: the running maximum takes the block's
  // maximum, d is rescaled once to it, then the block's shifted exponentials add.
  template <int K>
  __device__ static S absorb(S s, const float (&x)[K]) {
    float mx = __builtin_elementwise_maximum(x[0], x[1]);
#pragma unroll
    for (int i = 2; i < K; ++i) mx = __builtin_elementwise_maximum(mx, x[i]);
    const float m = __builtin_elementwise_maximum(s.m, mx);
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
  __device__ static S readlane(S s, int l) { return {fa::readlane(s.m, l), fa::readlane(s.d, l)}; }
  template <int CTRL, int ROWS>
  __device__ static S dpp(S s) {
    return {fa::dpp<CTRL, ROWS>(kNegInf, s.m), fa::dpp<CTRL, ROWS>(0.f, s.d)};
  }
  // The fold of K injections: their maximum, and the sum of each one's exponential
  // relative to it.
  template <int K>
  __device__ static S of_block(const float (&x)[K]) {
    float m = __builtin_elementwise_maximum(x[0], x[1]);
#pragma unroll
    for (int i = 2; i < K; ++i) m = __builtin_elementwise_maximum(m, x[i]);
    const float mr = m == kNegInf ? 0.f : m;
    float d = exp2_hw((x[0] - mr) * kLog2e);
#pragma unroll
    for (int i = 1; i < K; ++i) d += exp2_hw((x[i] - mr) * kLog2e);
    return {m, d};
  }
  __device__ static void store(S s, float* out0, float* out1, int64_t row) {
    out0[row] = s.m;
    out1[row] = s.d;
  }
  __device__ static float first(S s) { return s.m; }
  __device__ static float second(S s) { return s.d; }
  // A block aggregate as one 64-bit word for other workgroups: m in the low half, d in
  // the high half with its sign bit set (d >= 0, so the bit marks a published word; a
  // cleared word is 0). `count` (the block's element count) is not needed here.
  __device__ static uint64_t pack(S s) {
    return (uint64_t(__float_as_uint(s.d) | 0x80000000u) << 32) | __float_as_uint(s.m);
  }
  __device__ static S unpack(uint64_t w, float) {
    return {__uint_as_float(uint32_t(w)), __uint_as_float(uint32_t(w >> 32) & 0x7fffffffu)};
  }
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
  // combine(s, inject(x)): Welford's one-sample update.
  __device__ static S push(S s, float x) {
    const float n = s.n + 1.f, delta = x - s.mu;
    const float mu = fmaf(delta, __builtin_amdgcn_rcpf(n), s.mu);
    return {n, mu, fmaf(delta, x - mu, s.m2)};
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
  __device__ static S readlane(S s, int l) {
    return {fa::readlane(s.n, l), fa::readlane(s.mu, l), fa::readlane(s.m2, l)};
  }
  template <int CTRL, int ROWS>
  __device__ static S dpp(S s) {
    return {fa::dpp<CTRL, ROWS>(0.f, s.n), fa::dpp<CTRL, ROWS>(0.f, s.mu),
            fa::dpp<CTRL, ROWS>(0.f, s.m2)};
  }
  // The fold of K injections: (K, their mean, their squared deviations from it).
  template <int K>
  __device__ static S of_block(const float (&x)[K]) {
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
    return {float(K), mu, m2};
  }
  __device__ static void store(S s, float* out0, float* out1, int64_t row) {
    out0[row] = s.mu;
    out1[row] = s.m2;
  }
  __device__ static float first(S s) { return s.mu; }
  __device__ static float second(S s) { return s.m2; }
  // As SoftmaxMonoid::pack: mean low, M2 (>= 0) high with its sign bit set; the count of
  // a whole block is known to the reader.
  __device__ static uint64_t pack(S s) {
    return (uint64_t(__float_as_uint(s.m2) | 0x80000000u) << 32) | __float_as_uint(s.mu);
  }
  __device__ static S unpack(uint64_t w, float count) {
    return {count, __uint_as_float(uint32_t(w)), __uint_as_float(uint32_t(w >> 32) & 0x7fffffffu)};
  }
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
// the same pieces: one 256-thread workgroup per row, the row in blocks of 2048
// elements, wavefront w of a block over elements 512 w .. 512 w + 511 and its lane l
// over the 8 consecutive elements 8 l .. 8 l + 7. A lane folds its 8 elements into one
// state; the 64 states are scanned across the wavefront and the four wavefront totals
// combined through LDS; then the lane folds its elements again, one at a time, onto
// everything before them (the carry from earlier blocks, earlier wavefronts, earlier
// lanes) and writes each position's state. The block's total joins the carry.
//
// Global memory moves in whole contiguous runs: every load and store instruction of a
// wavefront covers 1 KB of consecutive bytes (lane l takes 16-byte vector l + 64 j of
// its wavefront's span), and a per-wavefront LDS area turns those runs into each lane's 8 consecutive elements and
// back (in for the input, out for each of the two outputs in turn). Vector v of an area
// sits in slot v ^ ((v >> 3) & 3): eight consecutive lanes that reach for their own
// vectors (vector P l + k, P = 1 or 2 vectors per lane) then hit eight distinct 16-byte
// bank groups, as do eight lanes that reach for consecutive vectors.
//
// ALIGNED: x and both outputs start on 16-byte boundaries and n is a multiple of the
// elements in one 16-byte input vector, so every vector is wholly inside the row or
// wholly past its end. Otherwise each lane reads and writes its elements one by one.
//
// Per element a lane spends about 25 vector instructions (the fold, the refold, its
// share of the scan and of the block's bookkeeping), which keeps the vector ALU well
// below the time the memory traffic takes.
constexpr int kOwn = 8;                     // consecutive elements per lane per block
constexpr int kWaveSpan = 64 * kOwn;        // elements per wavefront per block
constexpr int kScanBlock = 4 * kWaveSpan;   // elements per workgroup block
constexpr int kStageVecs = kWaveSpan / 4;   // 16-byte slots per wavefront: one output
constexpr int kDefaultPolls = 1 << 16;      // chained scans: polls before folding a block here

// Slot of vector v in a wavefront's LDS area.
__device__ __forceinline__ int slot(int v) { return v ^ ((v >> 3) & 3); }

// Orders one wavefront's LDS accesses on either side (its lanes exchange data through
// its own area; no other wavefront touches it).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Inclusive scan across the wavefront: lane l ends with the combine of lanes 0..l, in
// lane order. Data-parallel primitives move the states: shifts by 1, 2, 4 and 8 within
// each row of 16 lanes, then the last lane of row 0 (of row 2) into row 1 (row 3), then
// lane 31 into rows 2 and 3. A lane with no source takes the identity, which combines
// exactly (the identity is neutral in float32 arithmetic too).
template <class M>
__device__ __forceinline__ typename M::S wave_inclusive_scan(typename M::S t) {
  t = M::combine(M::template dpp<0x111, 0xf>(t), t);  // row_shr:1
  t = M::combine(M::template dpp<0x112, 0xf>(t), t);  // row_shr:2
  t = M::combine(M::template dpp<0x114, 0xf>(t), t);  // row_shr:4
  t = M::combine(M::template dpp<0x118, 0xf>(t), t);  // row_shr:8
  t = M::combine(M::template dpp<0x142, 0xa>(t), t);  // row_bcast:15 into rows 1 and 3
  t = M::combine(M::template dpp<0x143, 0xc>(t), t);  // row_bcast:31 into rows 2 and 3
  return t;
}

template <bool B>
struct Full {
  static constexpr bool value = B;
};

// Chained scans (CHAIN below) cut a row into its 2048-element blocks, one workgroup each,
// and hand the state before each block from workgroup to workgroup: block k publishes its
// own aggregate (the fold of its elements) as one flagged 64-bit word, and combines the
// aggregates of blocks 0 .. k-1 (at most 63) in order into the state before it. Lane t
// of wavefront 0 fetches block t's word; a block whose word has not appeared after
// max_polls polls is folded here from its elements instead (by the whole wavefront, so
// the rounding stays that of a tree of a few levels), so every wait ends. Words
// are written and read with device-scope atomics (the workgroups of a row run on
// different XCDs); a clearing kernel zeroes them before each launch.
template <class M, typename T>
__device__ typename M::S look_back(uint64_t* __restrict__ slots, int blk, typename M::S agg,
                                   int lane, int max_polls, const T* __restrict__ row_x) {
  using S = typename M::S;
  if (lane == 0)
    __hip_atomic_store(slots + blk, M::pack(agg), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const bool mine = lane < blk;
  uint64_t w = 0;
  bool wait = mine;
  for (int poll = 1;; ++poll) {
    if (wait) {
      w = __hip_atomic_load(slots + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      wait = (w >> 63) == 0;
    }
    if (__builtin_amdgcn_ballot_w64(wait) == 0 || poll >= max_polls) break;
    __builtin_amdgcn_s_sleep(2);
  }
  S st = (mine && !wait) ? M::unpack(w, float(kScanBlock)) : M::identity();
  // Blocks whose word did not appear: the wavefront folds each from its elements (lane l
  // takes elements 32 l .. 32 l + 31 in blocks of 8), merges the lanes by a butterfly,
  // and the block's lane keeps the result.
  uint64_t missing = __builtin_amdgcn_ballot_w64(mine && wait);
  while (missing != 0) {
    const int t = __builtin_ctzll(missing);
    missing &= missing - 1;
    const T* b = row_x + int64_t(t) * kScanBlock + 32 * lane;
    S part = M::identity();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = Elem<T>::scalar(b + 8 * c + i);
      part = M::combine(part, M::of_block(v));
    }
#pragma unroll
    for (int mask = 1; mask < 64; mask <<= 1) part = M::combine(part, M::shfl_xor(part, mask));
    if (lane == t) st = part;
  }
  st = wave_inclusive_scan<M>(st);
  return blk == 0 ? M::identity() : M::readlane(st, blk - 1);
}

template <class M, typename T, bool ALIGNED, bool CHAIN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8))) void row_scan_kernel(
    const T* __restrict__ x, int n, float* __restrict__ out0, float* __restrict__ out1,
    uint64_t* __restrict__ slots, int nblk, int max_polls) {
  using S = typename M::S;
  constexpr int VEC = 16 / int(sizeof(T));  // input elements per 16-byte vector
  constexpr int NIN = kWaveSpan / VEC / 64;  // input vectors per lane per block
  constexpr int NOUT = kWaveSpan / 4 / 64;   // vectors per lane per block of each output
  __shared__ S wtot[2][4];                   // wavefront totals, by block parity
  __shared__ u32x4_t stage[4][kStageVecs];
  __shared__ S chain_before;                 // CHAIN: the state before this block
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // CHAIN: workgroup b takes block b % nblk of row b / nblk (nblk = n / 2048)
  const int64_t row = CHAIN ? int64_t(blockIdx.x) / nblk : int64_t(blockIdx.x);
  const int my_blk = CHAIN ? int(int64_t(blockIdx.x) - row * nblk) : 0;
  const T* p = x + row * int64_t(n);
  float* o0 = out0 + row * int64_t(n);
  float* o1 = out1 + row * int64_t(n);
  u32x4_t* area = stage[wave];
  S carry = M::identity();

  auto block = [&](auto full, int base, int parity) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full)::value;
    const int w0 = base + kWaveSpan * wave;  // the wavefront's first element
    const int e0 = w0 + kOwn * lane;         // the lane's first element
    float v[kOwn];
    if (ALIGNED) {
      u32x4_t raw[NIN];
#pragma unroll
      for (int j = 0; j < NIN; ++j) {
        const int e = w0 + VEC * (lane + 64 * j);
        if (FULL || e < n)
          raw[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p + e));
      }
#pragma unroll
      for (int j = 0; j < NIN; ++j) area[slot(lane + 64 * j)] = raw[j];
      wave_sync();
#pragma unroll
      for (int k = 0; k < NIN; ++k) {
        const u32x4_t w = area[slot(NIN * lane + k)];
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          if constexpr (sizeof(T) == 4)
            v[VEC * k + i] = __uint_as_float(w[i]);
          else
            v[VEC * k + i] = (i & 1) ? bf16_hi(w[i / 2]) : bf16_lo(w[i / 2]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < kOwn; ++i) v[i] = e0 + i < n ? Elem<T>::scalar(p + e0 + i) : 0.f;
    }
    // the lane's total
    S tot;
    if (FULL) {
      tot = M::of_block(v);
    } else {
      tot = M::identity();
#pragma unroll
      for (int i = 0; i < kOwn; ++i)
        if (e0 + i < n) tot = M::push(tot, v[i]);
    }
    tot = wave_inclusive_scan<M>(tot);
    const S ex = M::template dpp<0x138, 0xf>(tot);  // wave_shr:1, the lanes before
    if (lane == 0) wtot[parity][wave] = M::readlane(tot, 63);
    __syncthreads();
    if constexpr (CHAIN) {
      S agg = wtot[parity][0];
#pragma unroll
      for (int w = 1; w < 4; ++w) agg = M::combine(agg, wtot[parity][w]);
      if (wave == 0) {
        const S before = look_back<M, T>(slots + row * nblk, my_blk, agg, lane, max_polls, p);
        if (lane == 0) chain_before = before;
      }
      __syncthreads();
      carry = chain_before;
    }
    // wtot[parity] is rewritten two blocks later, after every wavefront has passed the
    // next block's barrier, hence after these reads. The carry followed by the
    // wavefront totals in order: pre is the state before this wavefront's elements, blk
    // the state after the whole block.
    S pre = carry, blk = carry;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (w == wave) pre = blk;
      blk = M::combine(blk, wtot[parity][w]);
    }
    carry = blk;
    // fold again onto everything before the lane, keeping every position's state
    S r = M::combine(pre, ex);
    float r1[kOwn];
    if (ALIGNED) wave_sync();  // every lane has read its input from the area
#pragma unroll
    for (int k = 0; k < kOwn / 4; ++k) {
      float r0[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (FULL || e0 + 4 * k + i < n) r = M::push(r, v[4 * k + i]);
        r0[i] = M::first(r);
        r1[4 * k + i] = M::second(r);
      }
      if (ALIGNED)
        area[slot(NOUT * lane + k)] = __builtin_bit_cast(u32x4_t, f32x4_t{r0[0], r0[1], r0[2], r0[3]});
      else
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (e0 + 4 * k + i < n) o0[e0 + 4 * k + i] = r0[i];
    }
    if (ALIGNED) {
      // the two outputs leave through the area in turn, as 1 KB runs per instruction;
      // non-temporal: every output is written once and read by no one here
      auto drain = [&](float* o) __attribute__((always_inline)) {
        wave_sync();
        u32x4_t out[NOUT];
#pragma unroll
        for (int j = 0; j < NOUT; ++j) out[j] = area[slot(lane + 64 * j)];
#pragma unroll
        for (int j = 0; j < NOUT; ++j) {
          const int e = w0 + 4 * (lane + 64 * j);
          if (FULL || e < n)
            __builtin_nontemporal_store(__builtin_bit_cast(f32x4_t, out[j]),
                                        reinterpret_cast<f32x4_t*>(o + e));
        }
        wave_sync();
      };
      drain(o0);
#pragma unroll
      for (int k = 0; k < kOwn / 4; ++k)
        area[slot(NOUT * lane + k)] =
            __builtin_bit_cast(u32x4_t, f32x4_t{r1[4 * k], r1[4 * k + 1], r1[4 * k + 2], r1[4 * k + 3]});
      drain(o1);
    } else {
#pragma unroll
      for (int i = 0; i < kOwn; ++i)
        if (e0 + i < n) o1[e0 + i] = r1[i];
    }
  };

  if constexpr (CHAIN) {
    block(Full<true>(), my_blk * kScanBlock, 0);  // n is a multiple of the block
  } else {
    const int nfull = n / kScanBlock;  // blocks wholly inside the row
    int b = 0;
    for (; b < nfull; ++b) block(Full<true>(), b * kScanBlock, b & 1);
    if (b * kScanBlock < n) block(Full<false>(), b * kScanBlock, b & 1);
  }
}

// Zeroes the chained scans' published words before a launch.
__global__ __launch_bounds__(256) void clear_slots_kernel(uint64_t* __restrict__ slots,
                                                          int64_t count) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < count;
       i += int64_t(gridDim.x) * 256)
    slots[i] = 0;
}

template <class M, typename T>
hipError_t launch_scan(const RowReduceArgs& a, hipStream_t st) {
  if (a.rows > 0x7fffffff) return hipErrorInvalidValue;
  const T* x = static_cast<const T*>(a.x);
  const bool aligned = (reinterpret_cast<uintptr_t>(a.x) & 15) == 0 &&
                       (reinterpret_cast<uintptr_t>(a.out0) & 15) == 0 &&
                       (reinterpret_cast<uintptr_t>(a.out1) & 15) == 0 &&
                       (a.n % (16 / int(sizeof(T)))) == 0;
  const int64_t nblk = a.n / kScanBlock;
  if (aligned && a.slots != nullptr && scan_chain_blocks(a.n, a.bf16) > 0) {
    const int64_t words = a.rows * nblk;
    if (words > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(clear_slots_kernel, dim3(unsigned(min(words / 256 + 1, int64_t(4096)))),
                       dim3(256), 0, st, a.slots, words);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((row_scan_kernel<M, T, true, true>), dim3(unsigned(words)), dim3(256), 0,
                       st, x, a.n, a.out0, a.out1, a.slots, int(nblk),
                       a.max_polls > 0 ? a.max_polls : kDefaultPolls);
  } else if (aligned) {
    hipLaunchKernelGGL((row_scan_kernel<M, T, true, false>), dim3(unsigned(a.rows)), dim3(256), 0,
                       st, x, a.n, a.out0, a.out1, nullptr, 1, 0);
  } else {
    hipLaunchKernelGGL((row_scan_kernel<M, T, false, false>), dim3(unsigned(a.rows)), dim3(256),
                       0, st, x, a.n, a.out0, a.out1, nullptr, 1, 0);
  }
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

int scan_chain_blocks(int n, bool bf16) {
  if (n <= 0 || n % kScanBlock != 0) return 0;
  const int nb = n / kScanBlock;
  // Rows of up to 32 KB of input scan as fast with one workgroup each (measured on the
  // 8192-element bfloat16 rows: 0.98 ms, against 1.01 ms cut into 4 blocks), longer
  // ones faster cut (32768-element float32 rows: 0.63 -> 0.55 ms).
  const int64_t row_bytes = int64_t(n) * (bf16 ? 2 : 4);
  return nb >= 2 && nb <= 64 && row_bytes > 32768 ? nb : 0;
}

int64_t scan_workspace_bytes(int64_t rows, int n, bool bf16) {
  return rows * scan_chain_blocks(n, bf16) * int64_t(sizeof(uint64_t));
}

hipError_t launch_softmax_scan(const RowReduceArgs& a, hipStream_t s) {
  return a.bf16 ? launch_scan<SoftmaxMonoid, uint16_t>(a, s) : launch_scan<SoftmaxMonoid, float>(a, s);
}

hipError_t launch_moments_scan(const RowReduceArgs& a, hipStream_t s) {
  return a.bf16 ? launch_scan<WelfordMonoid, uint16_t>(a, s) : launch_scan<WelfordMonoid, float>(a, s);
}

}  // namespace fa
