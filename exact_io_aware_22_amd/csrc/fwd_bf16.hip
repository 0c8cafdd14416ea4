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
// weights each block against the current r straight away and keeps r until some
// weight would exceed 2^kTau (checked on each lane's block sum, after the fact); only
// then is the block's maximum taken as the new r and the block weighted again. So
// weights stay in [0, 2^kTau], no maximum is computed on ordinary steps, and the
// accumulator is rescaled only on those rare steps instead of every block. Floating
// point keeps the same relative precision at any magnitude, and with kTau = 32 the
// sums stay far inside float32 range (d <= N 2^32; |o| <= N 2^32 max|v|) for any
// sequence length an int holds. O is normalised by the sum of the weights as rounded
// to bf16 for the PV product, so it is divided by exactly the weights it was built
// from; the log-sum-exp uses the float32 sum.
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
//     hardware overlaps vector-ALU work with the matrix pipe. Scores and weights of
//     consecutive steps live in alternating register sets (the loop body is one
//     64-key tile, two steps), so nothing forces the softmax of block g ahead of the
//     QK MFMAs that produce block g+1.
//   * K and V arrive 64 keys per tile through three-slot LDS rings by direct global ->
//     LDS loads (global_load_lds_dwordx4, no register staging), issued two steps
//     before the one barrier per tile that publishes them. Both are row-major in LDS with
//     rows padded to one stride (304 bytes at D = 128, 144 at D = 64), so the two
//     tensors share their staging offsets; slot offsets are uniform scalars rotated
//     once per tile, so every fragment address is one per-lane base plus a constant.
//   * Tiles where nothing is masked, ragged or final run in a loop of their own with
//     no branches but the rare rescale; the remaining tiles take the general body,
//     which the steady loop is nested in (one copy of each).
//   * The V^T operand of the PV MFMA is read with the transposing LDS read
//     ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
//     (i mod 4) of what lane 4e + i/4 addressed, for e = 0..3, so lanes that address
//     four consecutive head dims of four consecutive keys hand each lane four keys
//     of one head dim.
//   * Causal: a wavefront stops at its diagonal block, which is the only block it
//     masks (plus the ragged tail); heaviest query tiles launch first and all tiles
//     of a head go to one XCD so its K/V stream is shared in that XCD's L2.
//   * Sliding windows and packed sequences use the same loop: a wavefront folds only
//     the blocks its rows' windows reach, the workgroup stages only the tiles they
//     cover, and blocks that straddle a window edge are masked. A packed unit is one
//     (sequence, head) pair with its own row count and first row.
//   * O is normalised in registers and leaves through LDS (each wavefront's 32 rows
//     staged and read back row-contiguous), so every store writes whole row pieces.
#include "device.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup
constexpr int kBN = 64;           // keys per LDS tile (two 32-key blocks)
constexpr int kSlots = 3;         // LDS ring depth for K and for V
constexpr int kTau = 32;          // rescale when the maximum grows by more than 2^32
constexpr float kSumLimit = float(1ull << kTau);  // 2^kTau
constexpr float kInf = __builtin_inff();

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
  // Bytes per K and V row in LDS, one stride for both so they share their staging
  // offsets. On 64 banks of 4 bytes, the K fragments' 16-byte row reads (16 lanes at a
  // time: one chunk of 16 consecutive rows) are free of conflicts at this stride; the V
  // fragments' transposing reads (32 lanes at a time: 64 bytes of 4 consecutive rows)
  // meet a 2-way conflict on a quarter of their accesses, which they would avoid at
  // 320 bytes. Measured against 272-byte K rows and 320-byte V rows (no conflicts, but
  // separate offsets, three of them spilled): the same speed, no scratch.
  static constexpr int KSTRIDE = D == 128 ? 304 : 144;
  static constexpr int VSTRIDE = KSTRIDE;
  static constexpr int KTILE = kBN * KSTRIDE;
  static constexpr int VTILE = kBN * VSTRIDE;
  static constexpr int LDS = kSlots * (KTILE + VTILE);
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

// Dense: units are the B*H heads of [B][H][Ntot][D] tensors. Packed (cu != nullptr):
// units are (sequence, head) pairs of [H][Ntot][D] tensors, sequence s owning rows
// [cu[s], cu[s+1]) (values clamped into [0, Ntot], length capped at max_len).
// Window: key j visible to query i iff i - wl <= j <= i + wr (negative = unbounded);
// causal is the wr = 0 case.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE, int Ntot,
    int U, int nqt, float c, int wl, int wr_in, const int* __restrict__ cu, int nseq,
    int max_len) {
  using G = Geo<D>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[G::LDS];
  uint8_t* const kring = smem;
  uint8_t* const vring = smem + kSlots * G::KTILE;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int half = lane >> 5, l32 = lane & 31;
  int unit, qt;
  map_tile(blockIdx.x, U, nqt, CAUSAL, unit, qt);
  int N;            // rows of this unit
  int64_t row0;     // its first row within the [.][Ntot] row space
  if (cu != nullptr) {
    // Sequence-major units: the heads of one sequence are consecutive units, so the
    // round-robin over XCDs spreads every sequence's heads evenly over the XCDs and
    // each XCD gets the same share of long and short sequences.
    const int nh = U / nseq, sq = unit / nh, h = unit % nh;
    const int a = min(max(cu[sq], 0), Ntot), b = min(max(cu[sq + 1], a), Ntot);
    N = min(b - a, max_len);
    row0 = int64_t(h) * Ntot + a;
  } else {
    N = Ntot;
    row0 = int64_t(unit) * Ntot;
  }
  // Uniform by construction; readfirstlane lets the compiler keep them in SGPRs.
  N = __builtin_amdgcn_readfirstlane(N);
  row0 = int64_t(uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(row0))))) |
         (int64_t(__builtin_amdgcn_readfirstlane(int(row0 >> 32))) << 32);
  const int q0 = qt * kBM;
  if (q0 >= N) return;  // the whole workgroup leaves before any barrier
  const int64_t head = row0 * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;
  const int wr = CAUSAL ? 0 : wr_in;  // causal bounds the window on the right at 0

  // Blocks of 32 keys: this wavefront folds blocks [g_lo, nblk) (the window's edges,
  // causal diagonal and N); the workgroup stages tiles [t_lo, ntiles) covering them.
  const int qw0 = q0 + 32 * wave;  // first query row of this wavefront
  const int nblk_all = (N + 31) >> 5;
  // One past the last block a query qlast <= N - 1 may see (wr is capped at the distance
  // to the last key before it is added, so no sum overflows).
  auto end_blk = [&](int qlast) {
    return wr < 0 ? nblk_all : min(nblk_all, ((qlast + min(wr, N - 1 - qlast)) >> 5) + 1);
  };
  // g_lo is rounded down to an even block, so a wavefront's first block always opens
  // a tile and its scores always land in the same register set; the block added that
  // way lies wholly left of the window and is folded in fully masked, i.e. as the
  // identity.
  const int g_lo = (qw0 >= N || wl < 0) ? 0 : ((max(0, qw0 - wl) >> 5) & ~1);
  const int nblk = qw0 >= N ? 0 : end_blk(qw0 + 31);
  const int nblk_wg = end_blk(min(N, q0 + kBM) - 1);
  const int t_lo = wl < 0 ? 0 : (max(0, q0 - wl) >> 6);
  const int ntiles = (nblk_wg + 1) >> 1;

  // ---- staging by direct global -> LDS loads (global_load_lds_dwordx4): one such
  // load moves 64 lanes x 16 bytes to 1 KB of consecutive LDS at M0 + 16 * lane. A
  // padded ring tile is exactly CK (K) or CV (V) such kilobytes, so each kilobyte j
  // is one load in which lane i fills LDS chunk 64 j + i, i.e. row (64 j + i) / C and
  // column (64 j + i) % C of the padded tile; pad columns take a copy of column
  // CPR - 1 and are never read. Wavefront w issues kilobytes w, w + 8, w + 16. In the
  // ragged last tile, rows past the end of the sequence take a copy of the last row
  // (finite, so masked keys still meet zero weight times a finite value).
  // The loads are issued from inline assembly so that the compiler, which does not
  // see them write LDS, inserts no waits before the fragment reads; the code waits
  // for them itself (vmcnt) before the barrier that publishes a tile. The compiler
  // makes no use of M0 in this kernel, which the assembly sets for each load.
  constexpr int CK = G::KSTRIDE / 16, CV = G::VSTRIDE / 16;  // chunks per padded row
  constexpr int MAXI = (CV + kWaves - 1) / kWaves;            // loads per wave per tile
  static_assert(CK <= CV && G::KTILE == CK * 1024 && G::VTILE == CV * 1024, "tile = C KB");
  // Source offset (bytes from the tile base) of lane's chunk of kilobyte j in a full tile.
  auto chunk_off = [&](int j, int C) __attribute__((always_inline)) -> uint32_t {
    const int p = 64 * j + lane, r = p / C, col = min(p % C, G::CPR - 1);
    return uint32_t(r * D * 2 + col * 16);
  };
  static_assert(CK == CV, "K and V tiles share one layout, hence one set of offsets");
  uint32_t dk[MAXI];
#pragma unroll
  for (int i = 0; i < MAXI; ++i) dk[i] = chunk_off(wave + kWaves * i, CK);
  const uint32_t (&dv)[MAXI] = dk;
  // The same chunk in tile t when rows past N - 1 are redirected to row N - 1 (its row
  // is off / (2D), a power-of-two division).
  auto clamp_off = [&](uint32_t off, int t) __attribute__((always_inline)) -> uint32_t {
    constexpr int kRowShift = __builtin_ctz(2 * D);
    const int r = int(off >> kRowShift);
    return off - uint32_t((r - (min(t * kBN + r, N - 1) - t * kBN)) << kRowShift);
  };
  auto dma = [&](const uint16_t* src, uint8_t* slot, int C, const uint32_t (&d)[MAXI], int t,
                 bool full) __attribute__((always_inline)) {
    // The tile base is uniform; readfirstlane keeps it in the SGPR pair the load takes.
    const uint64_t b64 = reinterpret_cast<uint64_t>(src) + uint64_t(t) * kBN * D * 2;
    const uint8_t* base = reinterpret_cast<const uint8_t*>(
        uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(b64))))) |
        (uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(b64 >> 32))))) << 32));
    const bool ragged = !full && t * kBN + kBN > N;
    const uint32_t lds0 =
        uint32_t(reinterpret_cast<uintptr_t>(FA_LDS(uint8_t, slot)));
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int j = wave + kWaves * i;
      if (j < C) {
        const uint32_t off = ragged ? clamp_off(d[i], t) : d[i];
        const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds0 + 1024u * uint32_t(j));
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                     :
                     : "s"(m0), "v"(off), "s"(base)
                     : "memory");
      }
    }
  };
  // s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima). Issued through the
  // builtin, not assembly, so the compiler's own wait bookkeeping also learns that
  // every vector-memory load (the Q fragments included) has completed.
  auto dma_wait = []() { __builtin_amdgcn_s_waitcnt(0x0F70); };

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
  float nmc_ref = kInf;  // -m_ref * c; +inf while there is no reference yet

  // Per-lane fragment offsets (loop invariant). K operand: row swap23(l32) of the
  // block, chunk 2c + half. V^T operand (transposing read): key 8*half + j/4 and
  // head dims 16*((lane>>4)&1) + 4*(j%4) for lane j = lane % 16 of its group.
  const int koff = swap23(l32) * G::KSTRIDE + half * 16;
  // voffr: the same offset from the start of LDS, i.e. with the V ring's base included,
  // kept opaque to the compiler so the base is added once here rather than folded into
  // the reads' immediates (which it would overflow, costing a second add per step).
  int voffr = kSlots * G::KTILE + (8 * half + ((lane & 15) >> 2)) * G::VSTRIDE +
              (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
  asm volatile("" : "+v"(voffr));

  // Fragments of S^T block g (32 keys x this wavefront's 32 queries): the K operand
  // rows from the K ring, one 16-byte read per 16-wide chunk of the head dim.
  // koff_blk / voff_blk: byte offset of a 32-key block in its ring (uniform).
  auto kload = [&](int koff_blk, u32x4_t (&kf)[G::NCH]) __attribute__((always_inline)) {
    const uint8_t* kb = kring + koff_blk + koff;
#pragma unroll
    for (int c2 = 0; c2 < G::NCH; ++c2) kf[c2] = load16(kb + 32 * c2);
  };
  auto qk = [&](const u32x4_t (&kf)[G::NCH]) __attribute__((always_inline)) {
    f32x16_t s = f32x16_t{};
#pragma unroll
    for (int c2 = 0; c2 < G::NCH; ++c2)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[c2]), as_bf16x8(qf[c2]), s, 0, 0, 0);
    return s;
  };
  // O^T += V^T (block g) P^T (block g). A operand rows: head dims 32db + l32; k:
  // keys 16cc + 8*half + 0..7 of the block, from two transposing reads.
  auto vload = [&](int voff_blk, u32x4_t (&vf)[2 * G::NDB]) __attribute__((always_inline)) {
    const uint8_t* vb = smem + voff_blk + voffr;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int db = 0; db < G::NDB; ++db) {
        const uint8_t* a0 = vb + 16 * cc * G::VSTRIDE + 64 * db;
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(FA_LDS(v4i16_t, a0));
        const v4i16_t hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16(FA_LDS(v4i16_t, a0 + 4 * G::VSTRIDE));
        const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
        vf[cc * G::NDB + db] = u32x4_t{l2[0], l2[1], h2[0], h2[1]};
      }
  };
  auto pv = [&](const u32x4_t (&vf)[2 * G::NDB], const uint32_t (&pk)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const u32x4_t b = {pk[4 * cc], pk[4 * cc + 1], pk[4 * cc + 2], pk[4 * cc + 3]};
#pragma unroll
      for (int db = 0; db < G::NDB; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf[cc * G::NDB + db]),
                                                           as_bf16x8(b), oacc[db], 0, 0, 0);
    }
  };
  // Masks block g: key 32g + k is visible to query qw0 + l32 iff the key is below N
  // and rel = key - query lies in [rlo, rhi] (an unbounded side: the int range).
  const int rlo = wl < 0 ? INT_MIN : -wl, rhi = wr < 0 ? INT_MAX : wr;
  auto apply_mask = [&](int g, f32x16_t& s) __attribute__((always_inline)) {
    const int rel0 = 32 * g - (qw0 + l32);
    const int lim = N - 32 * g;  // key 32g + k exists iff k < lim
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int k = swap23(8 * (r >> 2) + 4 * half + (r & 3));
      const int rel = rel0 + k;
      if (k >= lim || rel > rhi || rel < rlo) s[r] = kNegInf;
    }
  };
  // Softmax of block g against the reference maximum; returns the factor the
  // accumulator must be multiplied by before block g is added (1 if unchanged).
  // Weights of one block against the reference, packed to bf16 for the PV MFMA, with
  // their float32 sum (ps) and the sum of the packed values (pq).
  // ps: the block's float32 sum (from its first pair, no add of a zero); pq: pq0 plus the
  // sum of the packed values, so the running normaliser is carried through the chain.
  auto weights = [&](const f32x16_t& s, float nmc, uint32_t (&pk)[8], float& ps, float& pq,
                     float pq0) __attribute__((always_inline)) {
    const bf16x2_t ones = as_bf16x2(0x3f803f80u);
    pq = pq0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p0 = exp2_hw(fmaf(s[2 * i], c, nmc));
      const float p1 = exp2_hw(fmaf(s[2 * i + 1], c, nmc));
      ps = i == 0 ? p0 + p1 : ps + (p0 + p1);
      pk[i] = pack_bf16x2(p0, p1);
      pq = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pk[i]), ones, pq, false);
    }
  };
  // The block is weighted against the current reference straight away; only if some
  // lane's 16 weights sum past 2^kTau (which also catches +inf, NaN and the first
  // block, whose reference is -inf) does the wavefront take the rare path: the
  // block's maximum becomes the reference, O owes the factor alpha, and the block is
  // weighted again. No weight above 2^kTau is ever kept.
  // `resc` (wavefront-uniform) is set only on the rare path, so ordinary steps test a
  // scalar flag instead of comparing a per-lane factor with 1.
  auto softmax = [&](const f32x16_t& s, uint32_t (&pk)[8], bool& resc) __attribute__((always_inline)) {
    float ps, pq, alpha = 1.f;
    resc = false;
    weights(s, nmc_ref, pk, ps, pq, d_out);
    if (__builtin_amdgcn_ballot_w64(!(ps <= kSumLimit))) {
      resc = true;
      float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
      for (int r = 3; r < 15; r += 2) mx = fmaxf(fmaxf(mx, s[r]), s[r + 1]);
      mx = halves_max(fmaxf(mx, s[15]));
      const float m_new = fmaxf(m_ref, mx);
      alpha = m_ref == kNegInf ? 1.f : exp2_hw((m_ref - m_new) * c);
      m_ref = m_new;
      // A row with no visible key yet keeps +inf, so its first finite score comes
      // back here; its masked scores get weight exp2(-inf) = 0 below.
      nmc_ref = m_new == kNegInf ? kInf : -m_new * c;
      weights(s, m_new == kNegInf ? 0.f : nmc_ref, pk, ps, pq, d_out * alpha);
    }
    d_lse = fmaf(d_lse, alpha, ps);
    d_out = pq;
    return alpha;
  };
  auto rescale = [&](float alpha, bool resc) __attribute__((always_inline)) {
    if (resc) {
#pragma unroll
      for (int db = 0; db < G::NDB; ++db) oacc[db] *= alpha;
    }
  };
  // Blocks from first_masked on need masking: the ragged tail (32g + 32 > N) and keys
  // past the window's right edge for this wavefront's first query (qw0 + wr, qw0 a
  // multiple of 32; the causal diagonal when wr = 0). Blocks up to mask_lo_end need it
  // for the window's left edge of its last query.
  const int first_masked = wr < 0 ? (N >> 5) : min(N >> 5, (qw0 + min(wr, N) + 1) >> 5);
  const int mask_lo_end = wl < 0 ? -1 : ((qw0 + 31 - wl) >> 5);

  // ---- prologue: K tiles t_lo and t_lo + 1 and V tile t_lo in slots 0, 1, 0.
  dma(Kh, kring, CK, dk, t_lo, false);
  dma(Vh, vring, CV, dv, t_lo, false);
  if (t_lo + 1 < ntiles) dma(Kh, kring + G::KTILE, CK, dk, t_lo + 1, false);
  dma_wait();
  __syncthreads();

  // Scores and weights alternate between two register sets from one step to the
  // next (a, b), so the QK MFMAs of block g+1 never wait for the softmax of block g
  // to release its scores, and no copies are made.
  f32x16_t sa = f32x16_t{}, sb = f32x16_t{};
  uint32_t pa[8] = {0, 0, 0, 0, 0, 0, 0, 0}, pb[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float alpha_prev = 1.f;  // factor O owes the reference of the latest softmax
  bool resc_prev = false;  // whether it differs from 1 in some lane (uniform)
  u32x4_t kf[G::NCH], vf[2 * G::NDB];

  // Step g: scores of block g in s_in, weights of block g-1 in p_in; K block g+1 at
  // kblk, V block g-1 at vblk. One basic block issues QK of block g+1 (issued even
  // past a wavefront's last block, reading a resident slot, result unused), PV of
  // block g-1 (at a wavefront's first block g_lo with zero weights against block g_lo
  // itself) and the softmax of block g. The only branches come first: the mask of the
  // window-edge, diagonal or ragged blocks and the rare rescale of O.
  auto step = [&](int g, int kblk, int vblk, f32x16_t& s_in, f32x16_t& s_out,
                  const uint32_t (&p_in)[8], uint32_t (&p_out)[8], bool unmasked) __attribute__((always_inline)) {
    if (!unmasked && (g >= first_masked || g <= mask_lo_end)) apply_mask(g, s_in);
    // Bring O to the reference block g-1 was weighted against, then add PV(g-1).
    rescale(alpha_prev, resc_prev);
    kload(kblk, kf);
    s_out = qk(kf);
    vload(vblk, vf);
    pv(vf, p_in);
    alpha_prev = softmax(s_in, p_out, resc_prev);
  };

  // The steady loop's step: the K fragments of the block its QK computes arrive in kf
  // from the previous step, and the step loads those of the next step's block (knext)
  // once its own products have taken them, so the LDS latency of a step's K reads
  // overlaps the rest of the previous step (and, across a tile, its barrier).
  auto step_pf = [&](int knext, int vblk, f32x16_t& s_in, f32x16_t& s_out,
                     const uint32_t (&p_in)[8], uint32_t (&p_out)[8]) __attribute__((always_inline)) {
    rescale(alpha_prev, resc_prev);
    s_out = qk(kf);
    kload(knext, kf);
    vload(vblk, vf);
    pv(vf, p_in);
    alpha_prev = softmax(s_in, p_out, resc_prev);
  };

  // One iteration per tile t (blocks 2t and 2t+1). Slot offsets of K tiles t, t+1,
  // t+2 and of V tiles t-1, t, t+1 rotate through the three slots of each ring.
  // Tile t opens by issuing the direct loads of K tile t+2 and V tile t+1 and closes
  // by waiting for them before its barrier, so they have two steps to land. During
  // tile t the steps read K tiles t, t+1 and V tiles t-1, t, so the slots written
  // (those of K tile t-1 and V tile t-2) were last read before the barrier that ended
  // tile t-1, and what is written is first read after the barrier that ends tile t.
  int ks0 = 0, ks1 = G::KTILE, ks2 = 2 * G::KTILE;
  int vsp = 2 * G::VTILE, vs0 = 0, vs1 = G::VTILE;
  constexpr int KH = 32 * G::KSTRIDE, VH = 32 * G::VSTRIDE;  // second block of a tile
  auto rotate = [&]() __attribute__((always_inline)) {
    const int k0 = ks0, v0 = vsp;
    ks0 = ks1; ks1 = ks2; ks2 = k0;
    vsp = vs0; vs0 = vs1; vs1 = v0;
  };
  // Steady tiles [t_s0, t_s1): both steps run unmasked and past the wavefront's first
  // block, its last block lies beyond the tile, and the tiles staged during it (t+1,
  // t+2) are full, so the body needs no branch but the rescale. Other tiles take the
  // general body. Every wavefront passes one barrier per tile of [t_lo, ntiles) in
  // whichever loop, so the counts match across the workgroup.
  const int last_free = min(first_masked, nblk - 1);  // blocks below it are plain
  const int t_s0 = max(t_lo, (max(g_lo, mask_lo_end) + 2) >> 1);
  const int t_s1 = max(t_s0, min(min(last_free >> 1, ntiles - 2), (N >> 6) - 2));
  // Scores of a wavefront's first block g_lo (even, so it opens tile g_lo / 2), computed
  // at the start of that tile, whose K is resident from its barrier on.
  auto first_scores = [&]() __attribute__((always_inline)) {
    kload(ks0, kf);
    sa = qk(kf);
  };
  auto general_tile = [&](int t) __attribute__((always_inline)) {
    if (t + 2 < ntiles) dma(Kh, kring + ks2, CK, dk, t + 2, false);
    if (t + 1 < ntiles) dma(Vh, vring + vs1, CV, dv, t + 1, false);
    if (2 * t == g_lo && g_lo < nblk) first_scores();
    // At g = g_lo the PV reads a resident V block with the zero weights of pb.
    if (2 * t >= g_lo && 2 * t < nblk)
      step(2 * t, ks0 + KH, 2 * t > g_lo ? vsp + VH : vs0, sa, sb, pa, pb, false);
    if (2 * t >= g_lo && 2 * t + 1 < nblk) step(2 * t + 1, ks1, vs0, sb, sa, pb, pa, false);
    if (nblk - 1 >= g_lo && (nblk - 1 == 2 * t || nblk - 1 == 2 * t + 1)) {
      // This wavefront's last block is in tile t: fold it in while its V is resident.
      rescale(alpha_prev, resc_prev);
      vload(vs0 + ((nblk & 1) ? 0 : VH), vf);
      pv(vf, (nblk & 1) ? pb : pa);
    }
    dma_wait();
    __syncthreads();
    rotate();
  };
  // One copy of each body: the general tile loop drops into the steady loop at t_s0.
  // When the steady run is not empty it ends at t_s1 <= ntiles - 2, so a general tile
  // follows it.
#pragma unroll 1
  for (int t = t_lo; t < ntiles; ++t) {
    if (t == t_s0) {
      // Block 2t + 1 (second half of K tile t) is the first the steady loop's QK takes;
      // each step then loads the next: block 2t + 2 (first half of tile t + 1, resident
      // during tile t) and block 2t + 3 (its second half, which is the slot ks0 + KH
      // after the rotation). The last prefetch of the run is overwritten by the general
      // tile that follows.
      if (t < t_s1) kload(ks0 + KH, kf);
#pragma unroll 1
      for (; t < t_s1; ++t) {
        dma(Kh, kring + ks2, CK, dk, t + 2, true);
        dma(Vh, vring + vs1, CV, dv, t + 1, true);
        step_pf(ks1, vsp + VH, sa, sb, pa, pb);       // blocks 2t (softmax), 2t+1 (QK)
        step_pf(ks1 + KH, vs0, sb, sa, pb, pa);       // blocks 2t+1, 2t+2
        dma_wait();
        __syncthreads();
        rotate();
      }
    }
    general_tile(t);
  }

  // ---- read out: o / d once, lse = ln(sum) = (r c + log2 d) ln 2
  const float dl = halves_sum(d_lse), dq = halves_sum(d_out);
  const int qi = qw0 + l32;
  // O leaves through LDS so that every global store writes whole row pieces: each
  // wavefront stages its 32 rows x W head dims (normalised) in its own LDS region (the
  // rings are idle after the last barrier, and every direct load has been waited for),
  // then reads them back row-contiguous; W = 64 (D = 128) or 32 (D = 64), D / W passes.
  {
    const float inv = dq > 0.f ? 1.f / dq : 0.f;
    constexpr int W = D == 128 ? 64 : 32, CH = W / 4, RPI = 64 / CH;
    constexpr int OS = W * 4 + 16;  // bytes per staged row (+16: 16 rows on distinct banks)
    static_assert(kWaves * 32 * OS <= G::LDS, "output staging fits the rings");
    uint8_t* const ost = smem + wave * (32 * OS);
#pragma unroll
    for (int pass = 0; pass < D / W; ++pass) {
#pragma unroll
      for (int dbp = 0; dbp < W / 32; ++dbp) {
        const int db = pass * (W / 32) + dbp;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4_t val = {oacc[db][4 * g4] * inv, oacc[db][4 * g4 + 1] * inv,
                               oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv};
          *reinterpret_cast<f32x4_t*>(ost + l32 * OS + (32 * dbp + 8 * g4 + 4 * half) * 4) = val;
        }
      }
#pragma unroll
      for (int i = 0; i < 32 / RPI; ++i) {
        const int r = RPI * i + lane / CH, ch = lane % CH;
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(ost + r * OS + ch * 16);
        if (qw0 + r < N)
          *reinterpret_cast<f32x4_t*>(O + head + int64_t(qw0 + r) * D + pass * W + ch * 4) = v;
      }
    }
    if (qi < N && half == 0)
      LSE[row0 + qi] = dl > 0.f ? (m_ref * c + log2_hw(dl)) * kLn2 : kNegInf;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t s) {
  // Dense: one unit per (b, h). Packed: one per (sequence, h), B = sequence count.
  const int64_t U = int64_t(a.B) * a.H;
  const int64_t rows = a.cu_seqlens ? a.max_seqlen : a.N;
  const int nqt = int((rows + kBM - 1) / kBM);
  if (U > 0x7fffffff) return hipErrorInvalidValue;
  const int64_t blocks = U * nqt;  // < 2^31 * 2^24
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3(unsigned(blocks)), dim3(kThreads), 0,
                     s, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), a.o, a.lse, a.N, int(U), nqt,
                     a.scale * kLog2e, a.window_left, a.window_right, a.cu_seqlens,
                     a.cu_seqlens ? a.B : 1, a.max_seqlen);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s) {
  if (a.D == 128) return a.causal ? launch<128, true>(a, s) : launch<128, false>(a, s);
  return a.causal ? launch<64, true>(a, s) : launch<64, false>(a, s);
}

}  // namespace fa
