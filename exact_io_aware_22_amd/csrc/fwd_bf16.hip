// Exact attention forward, bfloat16 inputs, float32 accumulation, on gfx950 MFMA.
//
// Method ("Learning FlashAttention the Hard Way -- Part 1"): every query row folds
// its key/value tiles into u = (m, d, o) (section "The State"); a new tile is merged
// by rescaling the running state by 2^{(m_old - m_new) c} (section "The Merge, and
// the Twist") with all exponentials in base 2 and log2(e) folded into the scale,
// c = scale * log2(e) (section "Alternative Twist: Base 2"); masked and ragged keys
// get score -inf, i.e. they enter as the identity (section "Why Attention's Combine
// Still Associates"); o / d is formed once at the end.
//
// Work decomposition (one workgroup = 4 wavefronts = 128 query rows of one head):
//   * The scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     the 32x32 accumulator gives each lane one query column and 16 key rows, so a
//     query's running max needs one cross-half exchange (v_permlane32_swap) per tile
//     and its denominator none until the end.
//   * The output is accumulated transposed too, O^T += V^T P^T. The probabilities a
//     lane holds for its query are, after bf16 packing, exactly the B operand of the
//     PV MFMA, provided keys are assigned to the rows of the K operand in the order
//     given by swap23() below. P never leaves registers.
//   * Q fragments live in VGPRs for the whole loop; K and V tiles of 64 keys are
//     staged global -> registers -> LDS, double-buffered so the next tile's global
//     loads are in flight while the current tile is computed. K is kept row-major
//     in LDS, V transposed (V^T), both with a 16-byte-chunk XOR swizzle so that the
//     fragment reads are free of bank conflicts.
//   * Causal: tiles above a wavefront's diagonal are skipped, only tiles that cross
//     the diagonal or the ragged end of the sequence are masked, the heaviest query
//     tiles are launched first and all tiles of one head are mapped to one XCD so
//     its K/V stream is shared in that XCD's L2.
#include "device.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int kBM = 128;  // query rows per workgroup (32 per wavefront)
constexpr int kBN = 64;   // keys per LDS tile
constexpr int kThreads = 256;

// Row r of a 32-row K operand block holds key swap23(r): bits 2 and 3 exchanged.
// With this order the accumulator registers 8c..8c+7 of a lane hold 8 consecutive
// keys (16c + 8*half + i), which is the k order the PV MFMA's B operand expects.
__device__ __forceinline__ int swap23(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// XOR applied to the 16-byte chunk index of K row `key` in LDS. The 8 lanes that
// read together touch keys {0,1,2,3,8,9,10,11} + const (or +4), which this maps
// to 8 distinct chunk slots.
__device__ __forceinline__ int kswz(int key) { return (key & 3) | ((key >> 1) & 4); }

template <int D>
struct Tile {
  static constexpr int NCH = D / 16;          // 16-wide k chunks of the head dim
  static constexpr int NDB = D / 32;          // 32-row blocks of O^T
  static constexpr int KROW = D * 2;          // bytes per K row in LDS
  static constexpr int VTROW = kBN * 2;       // bytes per V^T row in LDS
  static constexpr int KBYTES = kBN * KROW;
  static constexpr int STAGE = KBYTES + D * VTROW;
  static constexpr int KLOADS = kBN * D / 8 / kThreads;  // 16-byte K loads per thread
  static constexpr int VGROUPS = (D / 8) * (kBN / 4);    // 4-key x 8-dim V blocks
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
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE, int N,
    int BH, int nqt, float c) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * T::STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  int bh, qt;
  map_tile(blockIdx.x, BH, nqt, CAUSAL, bh, qt);
  const int q0 = qt * kBM;
  const int64_t head = int64_t(bh) * N * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;

  // Q^T fragments (B operand): lane holds Q[qrow][16c + 8*half .. +7].
  const int qrow = q0 + wave * 32 + l32;
  u32x4_t qf[T::NCH];
#pragma unroll
  for (int c2 = 0; c2 < T::NCH; ++c2)
    qf[c2] = qrow < N ? load16(Qh + int64_t(qrow) * D + 16 * c2 + 8 * half) : u32x4_t{0, 0, 0, 0};

  const int kv_end = CAUSAL ? min(N, q0 + kBM) : N;
  const int ntiles = (kv_end + kBN - 1) / kBN;

  // ---- staging of one K/V tile: global -> registers -> LDS
  u32x4_t kst[T::KLOADS];
  u32x4_t vst[4];
  const bool v_loader = T::VGROUPS >= kThreads || tid < T::VGROUPS;
  const int vdg = tid % (D / 8), vkg = tid / (D / 8);

  auto gload = [&](int t) {
    const int k0 = t * kBN;
#pragma unroll
    for (int i = 0; i < T::KLOADS; ++i) {
      const int idx = tid + kThreads * i;
      const int key = idx / (D / 8), cc = idx % (D / 8);
      const int gk = k0 + key;
      kst[i] = gk < N ? load16(Kh + int64_t(gk) * D + cc * 8) : u32x4_t{0, 0, 0, 0};
    }
    if (v_loader) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int gk = k0 + 4 * vkg + r;
        vst[r] = gk < N ? load16(Vh + int64_t(gk) * D + vdg * 8) : u32x4_t{0, 0, 0, 0};
      }
    }
  };
  auto lstore = [&](int buf) {
    uint8_t* ks = smem + buf * T::STAGE;
    uint8_t* vs = ks + T::KBYTES;
#pragma unroll
    for (int i = 0; i < T::KLOADS; ++i) {
      const int idx = tid + kThreads * i;
      const int key = idx / (D / 8), cc = idx % (D / 8);
      *reinterpret_cast<u32x4_t*>(ks + key * T::KROW + ((cc ^ kswz(key)) << 4)) = kst[i];
    }
    if (v_loader) {
      // Transpose a 4-key x 8-dim block: row d of V^T receives keys 4*vkg .. +3.
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = vdg * 8 + e;
        const uint32_t a0 = vst[0][e >> 1], a1 = vst[1][e >> 1];
        const uint32_t a2 = vst[2][e >> 1], a3 = vst[3][e >> 1];
        const uint32_t w0 = (e & 1) ? ((a0 >> 16) | (a1 & 0xffff0000u)) : ((a0 & 0xffffu) | (a1 << 16));
        const uint32_t w1 = (e & 1) ? ((a2 >> 16) | (a3 & 0xffff0000u)) : ((a2 & 0xffffu) | (a3 << 16));
        const int off = d * T::VTROW + ((((vkg >> 1) ^ (d & 7))) << 4) + ((vkg & 1) << 3);
        *reinterpret_cast<u32x2_t*>(vs + off) = u32x2_t{w0, w1};
      }
    }
  };

  // ---- running state of this lane's query: m (raw score units), d (this half's keys)
  f32x16_t oacc[T::NDB];
#pragma unroll
  for (int db = 0; db < T::NDB; ++db) oacc[db] = f32x16_t{};
  float m_run = kNegInf, d_run = 0.f;

  gload(0);
  lstore(0);
  __syncthreads();

  const int qw_first = q0 + wave * 32;  // first query row of this wavefront
  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) gload(t + 1);
    const int k0 = t * kBN;
    const bool active = !CAUSAL || k0 <= qw_first + 31;
    if (active) {
      const uint8_t* ks = smem + (t & 1) * T::STAGE;
      const uint8_t* vs = ks + T::KBYTES;

      // S^T block kb: rows = keys k0 + 32kb + swap23(row), columns = this wave's queries.
      f32x16_t s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16_t{};
        const int key = kb * 32 + swap23(l32);
        const uint8_t* krow = ks + key * T::KROW;
        const int sw = kswz(key);
#pragma unroll
        for (int c2 = 0; c2 < T::NCH; ++c2) {
          const u32x4_t a = load16(krow + (((2 * c2 + half) ^ sw) << 4));
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(qf[c2]),
                                                          s[kb], 0, 0, 0);
        }
      }

      // Neutral-element masking, only on tiles that reach past the end or the diagonal.
      const bool need_mask = (k0 + kBN > N) || (CAUSAL && k0 + kBN - 1 > qw_first);
      if (need_mask) {
        const int qi = qw_first + l32;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + swap23(8 * (r >> 2) + 4 * half + (r & 3));
            if (key >= N || (CAUSAL && key > qi)) s[kb][r] = kNegInf;
          }
      }

      // Tile maximum of this query (16 keys per lane per block, then the other half).
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = halves_max(mx);
      const float m_new = fmaxf(m_run, mx);
      // Reference point for the exponentials; a still-empty state stays the identity.
      const float mref = m_new == kNegInf ? 0.f : m_new;
      const float alpha = exp2_hw((m_run - mref) * c);
      const float nmc = -mref * c;

      uint32_t pk[2][8];
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p0 = exp2_hw(fmaf(s[kb][2 * i], c, nmc));
          const float p1 = exp2_hw(fmaf(s[kb][2 * i + 1], c, nmc));
          ps += p0 + p1;
          pk[kb][i] = pack_bf16x2(p0, p1);
        }
      d_run = d_run * alpha + ps;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < T::NDB; ++db) oacc[db] *= alpha;

      // O^T[d][query] += sum_key V^T[d][key] P^T[key][query]
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const u32x4_t b = {pk[kb][4 * cc], pk[kb][4 * cc + 1], pk[kb][4 * cc + 2],
                             pk[kb][4 * cc + 3]};
          const int ch = 4 * kb + 2 * cc + half;  // 16-byte chunk of keys in a V^T row
#pragma unroll
          for (int db = 0; db < T::NDB; ++db) {
            const int d = 32 * db + l32;
            const u32x4_t a = load16(vs + d * T::VTROW + ((ch ^ (d & 7)) << 4));
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b),
                                                               oacc[db], 0, 0, 0);
          }
        }
    }
    if (t + 1 < ntiles) lstore((t + 1) & 1);
    __syncthreads();
  }

  // ---- read out: o / d once, lse = ln(sum) = (m c + log2 d) ln 2
  const float dt = halves_sum(d_run);
  const int qi = qw_first + l32;
  if (qi < N) {
    const float inv = dt > 0.f ? 1.f / dt : 0.f;
    float* orow = O + head + int64_t(qi) * D;
#pragma unroll
    for (int db = 0; db < T::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4_t val = {oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv,
                             oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv};
        *reinterpret_cast<f32x4_t*>(orow + 32 * db + 8 * g + 4 * half) = val;
      }
    if (half == 0)
      LSE[int64_t(bh) * N + qi] = dt > 0.f ? (m_run * c + log2_hw(dt)) * kLn2 : kNegInf;
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
