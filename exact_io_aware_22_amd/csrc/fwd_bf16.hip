// Exact attention forward, bfloat16 inputs, float32 accumulation, on gfx950 MFMA.
//
// Method ("Learning FlashAttention the Hard Way -- Part 1"): every query row folds
// its keys, 32 at a time, into u = (m, d, o) (section "The State"); merging a block
// rescales the running state by 2^{(m_old - m_new) c} (section "The Merge, and the
// Twist") with all exponentials in base 2 and log2(e) folded into the scale,
// c = scale * log2(e) (section "Alternative Twist: Base 2"); masked and ragged keys
// get score -inf, i.e. they enter as the identity (section "Why Attention's Combine
// Still Associates"); o / d is formed once at the end.
//
// Reference maximum. Any reference value r may stand in for the running maximum m:
// (m, d, o) and (r, d e^{m-r}, o e^{m-r}) are the same state in other coordinates
// (section "Twisted Monoid": the combine is transported by any bijection). The kernel
// keeps r fixed until a new block's maximum exceeds it by more than 2^kTau in
// weight, so weights stay in [0, 2^kTau] (no overflow, same relative precision) and
// the accumulator is rescaled only on those rare steps instead of every block. O is
// normalised by the sum of the weights as rounded to bf16 for the PV product, so it
// is divided by exactly the weights it was built from; the log-sum-exp uses the
// float32 sum.
//
// Work decomposition (one workgroup = 8 wavefronts = 256 query rows of one head):
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     the 32x32 accumulator gives each lane one query column and 16 key rows, so a
//     query's block maximum needs one cross-half exchange (v_permlane32_swap) and
//     its denominator none until the end.
//   * The output is accumulated transposed too, O^T += V^T P^T. The probabilities a
//     lane holds for its query are, after bf16 packing, exactly the B operand of the
//     PV MFMA, provided keys are assigned to the rows of the K operand in the order
//     given by swap23() below. P never leaves registers.
//   * Each 32-key step g issues, in one basic block, the QK MFMAs of block g+1, the
//     PV MFMAs of block g-1 and the softmax of block g, which are independent, so the
//     hardware overlaps vector-ALU work with the matrix pipe.
//   * K and V arrive 64 keys per tile through three-slot LDS rings (K two tiles
//     ahead, V one tile ahead), copied global -> registers -> LDS by all threads
//     (loads issued at the start of a tile, stores at its end), one barrier per
//     tile. Both are row-major in LDS with padded rows (K: +16 bytes, V: +64 bytes),
//     which keeps the fragment reads free of bank conflicts on 64 LDS banks and
//     makes every fragment address one per-lane base plus a constant.
//   * The V^T operand of the PV MFMA is read with the transposing LDS read
//     ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
//     (i mod 4) of what lane 4e + i/4 addressed, for e = 0..3, so lanes that address
//     four consecutive head dims of four consecutive keys hand each lane four keys
//     of one head dim.
//   * Causal: a wavefront stops at its diagonal block, which is the only block it
//     masks (plus the ragged tail); heaviest query tiles launch first and all tiles
//     of a head go to one XCD so its K/V stream is shared in that XCD's L2.
#include "device.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup
constexpr int kBN = 64;           // keys per LDS tile (two 32-key blocks)
constexpr int kSlots = 3;         // LDS ring depth for K and for V
constexpr float kTau = 8.0f;      // rescale when the maximum grows by more than 2^8

// Row r of a 32-row K operand block holds key swap23(r): bits 2 and 3 exchanged.
// With this order the accumulator registers 8c..8c+7 of a lane hold 8 consecutive
// keys (16c + 8*half + i), which is the k order the PV MFMA's B operand expects.
__device__ __forceinline__ int swap23(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));
#define FA_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

template <int D>
struct Geo {
  static constexpr int NCH = D / 16;             // 16-wide k chunks of the head dim
  static constexpr int NDB = D / 32;             // 32-row blocks of O^T
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int KSTRIDE = D * 2 + 16;     // bytes per K row in LDS
  static constexpr int VSTRIDE = D * 2 + 64;     // bytes per V row in LDS
  static constexpr int KTILE = kBN * KSTRIDE;
  static constexpr int VTILE = kBN * VSTRIDE;
  static constexpr int LDS = kSlots * (KTILE + VTILE);
  static constexpr int SPT = kBN * CPR / kThreads;  // chunks of a tile per thread
};

// Workgroup -> (head, query tile). Workgroups are dispatched round-robin over the
// 8 XCDs; all query tiles of a head go to the same XCD, heaviest (causal) first.
__device__ __forceinline__ void map_tile(int bid, int BH, int nqt, bool causal, int& bh,
                                         int& qt) {
  if ((BH & 7) == 0) {
    const int xcd = bid & 7, slot = bid >> 3, hpx = BH >> 3;
    bh = (slot % hpx) * 8 + xcd;
    qt = slot / hpx;
  } else {
    bh = bid % BH;
    qt = bid / BH;
  }
  if (causal) qt = nqt - 1 - qt;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE, int N,
    int BH, int nqt, float c) {
  using G = Geo<D>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[G::LDS];
  uint8_t* const kring = smem;
  uint8_t* const vring = smem + kSlots * G::KTILE;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int half = lane >> 5, l32 = lane & 31;
  int bh, qt;
  map_tile(blockIdx.x, BH, nqt, CAUSAL, bh, qt);
  const int q0 = qt * kBM;
  const int64_t head = int64_t(bh) * N * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;

  // Blocks of 32 keys: this wavefront folds blocks [0, nblk); the workgroup stages
  // tiles [0, ntiles) covering the most any of its wavefronts needs.
  const int qw0 = q0 + 32 * wave;  // first query row of this wavefront
  const int nblk_all = (N + 31) >> 5;
  const int nblk = qw0 >= N ? 0 : (CAUSAL ? min(nblk_all, (qw0 >> 5) + 1) : nblk_all);
  const int nblk_wg = CAUSAL ? min(nblk_all, ((min(N, q0 + kBM) - 1) >> 5) + 1) : nblk_all;
  const int ntiles = (nblk_wg + 1) >> 1;

  // ---- staging: each thread copies SPT 16-byte chunks of a K tile and SPT of a V
  // tile, global -> registers at the start of a tile, registers -> LDS at its end.
  // Rows past the end of the sequence are stored as zeros, so masked keys meet
  // finite values (zero weight times zero); the load itself reads the last row.
  u32x4_t stg[2 * G::SPT];
  auto gload = [&](int tk, int tv) {
#pragma unroll
    for (int i = 0; i < 2 * G::SPT; ++i) {
      const bool is_v = i >= G::SPT;
      const int idx = tid + kThreads * (i % G::SPT);
      const int t = max(is_v ? tv : tk, 0);
      const int gk = min(t * kBN + idx / G::CPR, N - 1);
      stg[i] = load16((is_v ? Vh : Kh) + int64_t(gk) * D + (idx % G::CPR) * 8);
    }
  };
  auto lstore = [&](int tk, int tv) {
#pragma unroll
    for (int i = 0; i < 2 * G::SPT; ++i) {
      const bool is_v = i >= G::SPT;
      const int t = is_v ? tv : tk;
      if (t < 0) continue;
      const int idx = tid + kThreads * (i % G::SPT);
      const int row = idx / G::CPR;
      uint8_t* dst = (is_v ? vring + (t % kSlots) * G::VTILE + row * G::VSTRIDE
                           : kring + (t % kSlots) * G::KTILE + row * G::KSTRIDE) +
                     (idx % G::CPR) * 16;
      *reinterpret_cast<u32x4_t*>(dst) = t * kBN + row < N ? stg[i] : u32x4_t{0, 0, 0, 0};
    }
  };

  // ---- per-lane state: Q^T fragments, O^T accumulator, reference max r, d
  const int qrow = qw0 + l32;
  u32x4_t qf[G::NCH];
#pragma unroll
  for (int c2 = 0; c2 < G::NCH; ++c2)
    qf[c2] = qrow < N ? load16(Qh + int64_t(qrow) * D + 16 * c2 + 8 * half) : u32x4_t{0, 0, 0, 0};
  f32x16_t oacc[G::NDB];
#pragma unroll
  for (int db = 0; db < G::NDB; ++db) oacc[db] = f32x16_t{};
  // d_lse sums the weights in float32 (for the log-sum-exp); d_out sums the same
  // weights as rounded to bf16 for the PV MFMA, so O is normalised by exactly the
  // weights it was built from.
  float m_ref = kNegInf, d_lse = 0.f, d_out = 0.f;

  // Per-lane fragment offsets (loop invariant). K operand: row swap23(l32) of the
  // block, chunk 2c + half. V^T operand (transposing read): key 8*half + j/4 and
  // head dims 16*((lane>>4)&1) + 4*(j%4) for lane j = lane % 16 of its group.
  const int koff = swap23(l32) * G::KSTRIDE + half * 16;
  const int voff = (8 * half + ((lane & 15) >> 2)) * G::VSTRIDE +
                   (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;

  // S^T block g (32 keys x this wavefront's 32 queries) from the K ring.
  auto qk = [&](int g) {
    const uint8_t* kb = kring + ((g >> 1) % kSlots) * G::KTILE + (g & 1) * 32 * G::KSTRIDE + koff;
    f32x16_t s = f32x16_t{};
#pragma unroll
    for (int c2 = 0; c2 < G::NCH; ++c2) {
      const u32x4_t a = load16(kb + 32 * c2);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(qf[c2]), s, 0, 0, 0);
    }
    return s;
  };
  // O^T += V^T (block g) P^T (block g). A operand rows: head dims 32db + l32; k:
  // keys 16cc + 8*half + 0..7 of the block, from two transposing reads (r = 0, 1).
  auto pv = [&](int g, const uint32_t (&pk)[8]) {
    const uint8_t* vb = vring + ((g >> 1) % kSlots) * G::VTILE + (g & 1) * 32 * G::VSTRIDE + voff;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const u32x4_t b = {pk[4 * cc], pk[4 * cc + 1], pk[4 * cc + 2], pk[4 * cc + 3]};
#pragma unroll
      for (int db = 0; db < G::NDB; ++db) {
        const uint8_t* a0 = vb + 16 * cc * G::VSTRIDE + 64 * db;
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(FA_LDS(v4i16_t, a0));
        const v4i16_t hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16(FA_LDS(v4i16_t, a0 + 4 * G::VSTRIDE));
        const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
        const u32x4_t a = {l2[0], l2[1], h2[0], h2[1]};
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b),
                                                           oacc[db], 0, 0, 0);
      }
    }
  };
  auto apply_mask = [&](int g, f32x16_t& s) {
    const int qi = qw0 + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 32 * g + swap23(8 * (r >> 2) + 4 * half + (r & 3));
      if (key >= N || (CAUSAL && key > qi)) s[r] = kNegInf;
    }
  };
  // Softmax of block g against the reference maximum; returns the factor the
  // accumulator must be multiplied by before block g is added (1 if unchanged).
  auto softmax = [&](const f32x16_t& s, uint32_t (&pk)[8]) {
    float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) mx = fmaxf(fmaxf(mx, s[r]), s[r + 1]);
    mx = fmaxf(mx, s[15]);
    mx = halves_max(mx);
    const bool grow = (mx - m_ref) * c > kTau;  // false when both are -inf
    const float m_new = grow ? mx : m_ref;
    const float alpha = grow ? exp2_hw((m_ref - m_new) * c) : 1.f;
    const float nmc = m_new == kNegInf ? 0.f : -m_new * c;
    float ps = 0.f, pq = 0.f;
    const bf16x2_t ones = as_bf16x2(0x3f803f80u);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p0 = exp2_hw(fmaf(s[2 * i], c, nmc));
      const float p1 = exp2_hw(fmaf(s[2 * i + 1], c, nmc));
      ps += p0 + p1;
      pk[i] = pack_bf16x2(p0, p1);
      pq = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pk[i]), ones, pq, false);
    }
    d_lse = fmaf(d_lse, alpha, ps);
    d_out = fmaf(d_out, alpha, pq);
    m_ref = m_new;
    return alpha;
  };
  auto rescale = [&](float alpha) {
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < G::NDB; ++db) oacc[db] *= alpha;
    }
  };
  auto needs_mask = [&](int g) { return (32 * g + 32 > N) || (CAUSAL && 32 * g + 31 > qw0); };

  // ---- prologue: K tiles 0 and 1, V tile 0
  gload(0, 0);
  lstore(0, 0);
  if (ntiles > 1) {
    gload(1, -1);
    lstore(1, -1);
  }
  __syncthreads();

  f32x16_t s_cur = f32x16_t{};
  uint32_t p_prev[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float alpha_prev = 1.f;  // factor O owes the reference of the latest softmax
  if (nblk > 0) s_cur = qk(0);

  // One iteration per 32-key block; tiles (two blocks) are staged on even blocks
  // and published after odd ones. Slots (t+2)%3 of K and (t+1)%3 of V, refilled at
  // the start of tile t, were last read during tile t-1.
  // A step is one basic block: QK of block g+1 (issued even past a wavefront's last
  // block, reading a resident slot, result unused), PV of block g-1 (at g = 0 with
  // zero weights against tile 0) and the softmax of block g. The only branches come
  // first: the mask of the diagonal / ragged block and the rare rescale of O.
#pragma unroll 1
  for (int g = 0; g < 2 * ntiles; ++g) {
    const int t = g >> 1;
    const int tk = t + 2 < ntiles ? t + 2 : -1, tv = t + 1 < ntiles ? t + 1 : -1;
    if ((g & 1) == 0 && (tk >= 0 || tv >= 0)) gload(tk, tv);
    if (g < nblk) {
      if (needs_mask(g)) apply_mask(g, s_cur);
      // Bring O to the reference block g-1 was weighted against, then add PV(g-1).
      rescale(alpha_prev);
      uint32_t p_cur[8];
      const f32x16_t s_next = qk(g + 1);
      pv(g > 0 ? g - 1 : 0, p_prev);
      alpha_prev = softmax(s_cur, p_cur);
      s_cur = s_next;
#pragma unroll
      for (int i = 0; i < 8; ++i) p_prev[i] = p_cur[i];
      if (g + 1 == nblk) {  // last block: fold it in while its V tile is resident
        rescale(alpha_prev);
        pv(g, p_prev);
      }
    }
    if (g & 1) {
      if (tk >= 0 || tv >= 0) lstore(tk, tv);
      __syncthreads();
    }
  }

  // ---- read out: o / d once, lse = ln(sum) = (r c + log2 d) ln 2
  const float dl = halves_sum(d_lse), dq = halves_sum(d_out);
  const int qi = qw0 + l32;
  if (qi < N) {
    const float inv = dq > 0.f ? 1.f / dq : 0.f;
    float* orow = O + head + int64_t(qi) * D;
#pragma unroll
    for (int db = 0; db < G::NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4_t val = {oacc[db][4 * g4] * inv, oacc[db][4 * g4 + 1] * inv,
                             oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv};
        *reinterpret_cast<f32x4_t*>(orow + 32 * db + 8 * g4 + 4 * half) = val;
      }
    if (half == 0)
      LSE[int64_t(bh) * N + qi] = dl > 0.f ? (m_ref * c + log2_hw(dl)) * kLn2 : kNegInf;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t s) {
  const int BH = a.B * a.H;
  const int nqt = (a.N + kBM - 1) / kBM;
  const int64_t blocks = int64_t(BH) * nqt;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3(unsigned(blocks)), dim3(kThreads), 0,
                     s, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), a.o, a.lse, a.N, BH, nqt,
                     a.scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s) {
  if (a.D == 128) return a.causal ? launch<128, true>(a, s) : launch<128, false>(a, s);
  return a.causal ? launch<64, true>(a, s) : launch<64, false>(a, s);
}

}  // namespace fa
