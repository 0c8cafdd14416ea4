// Exact attention backward, bfloat16 inputs, float32 accumulation, on gfx950 MFMA.
//
// The pages name the backward pass that recomputes attention instead of storing it,
// keeping only the per-row log-sum-exp of the forward ("Learning FlashAttention the
// Hard Way -- Part 1", its topic list), but print no formula. The gradients follow
// by the chain rule from the forward definition (section "FlashAttention: Not So
// Special": S = scale Q K^T, P = row softmax(S), O = P V). With lse from the forward,
// P_ij = e^{S_ij - lse_i} = 2^{S_ij c - lse_i log2 e}, c = scale log2 e (section
// "Alternative Twist: Base 2"), and for an upstream gradient dO:
//   dV = P^T dO,  dP = dO V^T,  Delta_i = sum_d dO_id O_id (= sum_j P_ij dP_ij),
//   dS = P (dP - Delta),  dQ = scale dS K,  dK = scale dS^T Q.
// Masked keys have P = 0 and contribute nothing.
//
// Two kernels, dQ first:
//   * dq_kernel: a wavefront owns 32 query rows (Q^T and dO^T fragments in registers)
//     and first forms its rows' Delta from those dO values and the forward's O (fp32),
//     writing it for the dK/dV kernel; then it walks the key tiles: S^T = K Q^T and
//     dP^T = V dO^T (A operands: K and V rows from LDS), P^T and dS^T element-wise (one
//     lse and one Delta per lane), then dQ^T += K^T dS^T with K^T read by the
//     transposing LDS read.
//   * dkdv_kernel: a wavefront owns 32 key rows (K^T and V^T fragments in registers)
//     and walks the query tiles, each 32-query block as one chain: S = Q K^T (A
//     operand: Q rows from LDS), P element-wise (16 queries per lane, their lse read
//     from LDS), dV^T += dO^T P (dO^T by the transposing LDS read); then dP = dO V^T,
//     dS = P (dP - Delta) from the bf16 P the dV product used (the dP products start
//     from -Delta, so they yield dP - Delta), dK^T += Q^T dS.
// Every product is v_mfma_f32_32x32x16_bf16; the element-wise results a lane holds
// are, after bf16 packing, exactly the B operand of the next product (the swap23 row
// order used by the forward kernel). A tile is read both row-wise (16-byte reads) and
// column-wise (transposing reads) from one padded LDS copy (BGeo below).
// Staging: both kernels load their 64-row tiles by direct global -> LDS loads, so no
// registers hold staged data (dq_kernel: K and V, 8 wavefronts, 256 query rows;
// dkdv_kernel: Q and dO, 8 wavefronts, 256 key rows). Two LDS slots, one barrier per
// tile.
#include <type_traits>

#include "device.h"
#include "launch.h"

namespace fa {
namespace {

// dK/dV: eight wavefronts per workgroup, two per SIMD, so one's element-wise work
// overlaps the other's products. At D = 128 that leaves 256 registers per wavefront for
// the two 32 x 128 accumulators (128), the own K^T and V^T fragments (64) and one 32 x 32
// product at a time: S and dP are formed one after the other, never both live.
template <int D>
struct KV {
  static constexpr int kWaves = 8;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kRows = 32 * kWaves;  // key rows a workgroup owns
};
constexpr int kTile = 64;                  // rows per LDS tile (two 32-row blocks)
// dQ: 8 wavefronts (two per SIMD, so one's element-wise work overlaps the other's
// products) and 256 query rows per workgroup; it fits 256 VGPRs per wavefront.
constexpr int kWavesQ = 8, kThreadsQ = 64 * kWavesQ, kRowsQ = 32 * kWavesQ;

typedef short v4i16_t __attribute__((ext_vector_type(4)));
#define FA_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

// Row r of a 32-row A operand holds row swap23(r) (bits 2 and 3 exchanged), so a
// lane's accumulator registers 8c..8c+7 hold 8 consecutive rows 16c + 8 half + i.
__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// LDS has 64 banks of 4 bytes. A 16-byte row read serves 16 lanes at a time, which read
// one chunk of 16 consecutive rows (16-byte windows); a transposing read serves 32 lanes
// at a time, which read 64 bytes of 4 consecutive rows. A read is free of bank
// conflicts iff its windows, spaced by the row stride, are disjoint modulo 256 bytes:
// for the row reads a stride of 16 times an odd number of bytes (mod 256), for the
// transposing reads 64 times an odd number. No plain padding does both.
constexpr bool windows_disjoint(int stride, int rows, int bytes) {
  for (int a = 1; a < rows; ++a) {
    const int d = (a * stride) % 256;  // distance between rows r and r + a
    if (d < bytes || 256 - d < bytes) return false;
  }
  return true;
}

template <int D>
struct BGeo {
  static constexpr int NCH = D / 16;       // 16-wide k chunks of the head dim
  static constexpr int NDB = D / 32;       // 32-row blocks of a transposed accumulator
  static constexpr int CPR = D / 8;        // 16-byte chunks per row
  // Row stride of a staged tile, read both ways from one copy: the row reads are free
  // of conflicts, and a quarter of the transposing reads' accesses meet a 2-way
  // conflict. Measured against the alternatives at D = 128: two copies (272-byte rows
  // for the row reads, 320 for the transposing reads, no conflicts) were 4% slower
  // (twice the staging); one 320-byte copy with the 16-byte chunks of each 64-byte
  // quarter permuted by row (no conflicts either) ran at the same speed, and 3-4%
  // slower at D = 64.
  static constexpr int SS = D == 128 ? 304 : 144;
  static constexpr int ST = kTile * SS;    // bytes of one staged tile
  static_assert(windows_disjoint(SS, 16, 16), "row reads must be free of bank conflicts");
};

// Per-lane offsets of the two fragment read patterns (see the forward kernel):
// row reads: row swap23(l32) of a 32-row block, chunk 2c + half at +32 c bytes;
// transposing reads: rows 8 half + (lane & 15) / 4, head dims 16 ((lane >> 4) & 1) +
// 4 (lane & 3); block (cc, db) at +16 cc SS + 64 db, high half at +4 SS (SS: the row stride).
__device__ __forceinline__ int row_off(int lane, int SS) {
  return swap23(lane & 31) * SS + (lane >> 5) * 16;
}
__device__ __forceinline__ int tr_off(int lane, int SS) {
  return (8 * (lane >> 5) + ((lane & 15) >> 2)) * SS + (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
}

// A operand of rows [32 block] (row reads), k chunk c2.
__device__ __forceinline__ bf16x8_t frag_row(const uint8_t* base, int c2) {
  return as_bf16x8(load16(base + 32 * c2));
}
// A operand of the transposed block (head dims 32 db.., rows 16 cc + 8 half + 0..7).
__device__ __forceinline__ bf16x8_t frag_tr(const uint8_t* base, int cc, int db, int SS) {
  const uint8_t* a0 = base + 16 * cc * SS + 64 * db;
  const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(FA_LDS(v4i16_t, a0));
  const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(FA_LDS(v4i16_t, a0 + 4 * SS));
  const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
  return as_bf16x8(u32x4_t{l2[0], l2[1], h2[0], h2[1]});
}
__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Direct global -> LDS staging of 64-row tiles (global_load_lds_dwordx4, as in the
// forward kernel) into a padded layout of C kilobytes (row stride 16 C bytes): one load
// moves 64 lanes x 16 bytes to 1 KB of consecutive LDS at M0 + 16 lane, so lane i of
// kilobyte j fills chunk 64 j + i of the padded tile, i.e. row (64 j + i) / C and column
// (64 j + i) % C; pad columns take a copy of column CPR - 1 and are never read. Rows
// past N - 1 take row N - 1 (finite; masked by the caller). Wavefront w issues
// kilobytes w, w + WAVES, ... The loads are issued from inline assembly so that the
// compiler, which does not see them write LDS, adds no waits before later LDS reads;
// callers wait for them (vmcnt) before the barrier that publishes the tile. The
// compiler makes no use of M0 in these kernels, which the assembly sets per load.
// The source offsets depend only on the lane, the wavefront and (for the ragged last
// tile) on N, so one set serves every tensor staged into the same layout; the compiler
// keeps each load's row and chunk in registers across the tile loop and forms the
// offsets with two instructions per load. (With two layouts, twice the offsets kept
// that way pushed the dK/dV kernel past 256 registers, and a spilled offset reloaded
// between two staging loads waited for every load in flight; they were recomputed at
// every tile instead.)
template <int D, int C, int WAVES>
struct Staging {
  static constexpr int MAXI = (C + WAVES - 1) / WAVES;  // loads per wavefront and tile
  uint32_t off[MAXI];  // byte offset of each load's source chunk within the tile

  __device__ __forceinline__ Staging(int t, int N, int wave, int lane) {
    constexpr int CPR = D / 8;
    constexpr int kRowShift = __builtin_ctz(2 * D);
    __builtin_assume(wave >= 0 && wave < WAVES);
    // Last row of tile t that exists (>= kTile - 1 unless t is the ragged last tile).
    const uint32_t last = uint32_t(N - 1 - t * kTile);
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const uint32_t p = 64u * uint32_t(wave + WAVES * i) + uint32_t(lane);
      const uint32_t r = p / C, col = min(p - r * C, uint32_t(CPR - 1));
      off[i] = (min(r, last) << kRowShift) + col * 16u;
    }
  }

  __device__ __forceinline__ void issue(const uint16_t* src, const uint8_t* region, int t,
                                        int wave) const {
    __builtin_assume(wave >= 0 && wave < WAVES);
    const uint64_t b64 = reinterpret_cast<uint64_t>(src) + uint64_t(t) * kTile * D * 2;
    const uint8_t* base = reinterpret_cast<const uint8_t*>(
        uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(b64))))) |
        (uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(b64 >> 32))))) << 32));
    const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>(FA_LDS(const uint8_t, region)));
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int j = wave + WAVES * i;
      if (j < C) {
        const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds0 + 1024u * uint32_t(j));
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                     :
                     : "s"(m0), "v"(off[i]), "s"(base)
                     : "memory");
      }
    }
  }
};
// s_waitcnt vmcnt(0), through the builtin so the compiler's own bookkeeping sees it.
__device__ __forceinline__ void dma_wait() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup -> (head, tile): all tiles of a head on one XCD, heaviest first.
// heavy_last_tile: causal dq (the last query tiles see the most keys); otherwise causal
// dk/dv (the first key tiles see the most queries).
__device__ __forceinline__ void map_bwd(int bid, int BH, int ntile, bool causal, bool heavy_last,
                                        int& bh, int& t) {
  if ((BH & 7) == 0) {
    const int xcd = bid & 7, slot = bid >> 3, hpx = BH >> 3;
    bh = (slot % hpx) * 8 + xcd;
    t = slot / hpx;
  } else {
    bh = bid % BH;
    t = bid / BH;
  }
  if (causal && heavy_last) t = ntile - 1 - t;
}

// ------------------------------------------------------------------ dQ
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreadsQ, 1) void dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ O, const float* __restrict__ LSE, float* __restrict__ DELTA,
    float* __restrict__ dQ, int N, int BH, int nqt, float c, float scale) {
  using G = BGeo<D>;
  constexpr int SLOT = 2 * G::ST;  // K, then V
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * SLOT];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  int bh, qt;
  map_bwd(blockIdx.x, BH, nqt, CAUSAL, true, bh, qt);
  const int64_t head = int64_t(bh) * N * D;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;
  const int q0 = qt * kRowsQ, qw0 = q0 + 32 * wave, qrow = qw0 + l32;

  const int nblk_all = (N + 31) >> 5;
  const int nblk = qw0 >= N ? 0 : (CAUSAL ? min(nblk_all, (qw0 >> 5) + 1) : nblk_all);
  const int nblk_wg = CAUSAL ? min(nblk_all, ((min(N, q0 + kRowsQ) - 1) >> 5) + 1) : nblk_all;
  const int ntiles = (nblk_wg + 1) >> 1;

  // Own rows: Q^T and dO^T as B operands (k = head dims 16 c2 + 8 half + 0..7). Delta of
  // the row, dO . O, is formed here from the same dO values and the matching O values
  // (the two halves of the row's head dims sit in lanes l and l ^ 32) and written for
  // the dK/dV kernel.
  u32x4_t qf[G::NCH], df[G::NCH];
  float lse2 = kInfB, dl = 0.f;
  {
    const bool ok = qrow < N;
    const int64_t rowoff = head + int64_t(qrow) * D + 8 * half;
#pragma unroll
    for (int c2 = 0; c2 < G::NCH; ++c2) {
      qf[c2] = ok ? load16(Q + rowoff + 16 * c2) : u32x4_t{0, 0, 0, 0};
      df[c2] = ok ? load16(dO + rowoff + 16 * c2) : u32x4_t{0, 0, 0, 0};
    }
    float part = 0.f;
    if (ok) {
#pragma unroll
      for (int c2 = 0; c2 < G::NCH; ++c2) {
        const f32x4_t o0 = *reinterpret_cast<const f32x4_t*>(O + rowoff + 16 * c2);
        const f32x4_t o1 = *reinterpret_cast<const f32x4_t*>(O + rowoff + 16 * c2 + 4);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          part = fmaf(bf16_lo(df[c2][i]), o0[2 * i], part);
          part = fmaf(bf16_hi(df[c2][i]), o0[2 * i + 1], part);
          part = fmaf(bf16_lo(df[c2][2 + i]), o1[2 * i], part);
          part = fmaf(bf16_hi(df[c2][2 + i]), o1[2 * i + 1], part);
        }
      }
    }
    const float delta_row = part + __shfl_xor(part, 32);
    if (ok) {
      const float l = LSE[int64_t(bh) * N + qrow];
      lse2 = l == kNegInf ? kInfB : l * kLog2e;  // a row that sees no key gets P = 0
      dl = delta_row;
      if (half == 0) DELTA[int64_t(bh) * N + qrow] = dl;
    }
  }
  f32x16_t acc[G::NDB];
#pragma unroll
  for (int db = 0; db < G::NDB; ++db) acc[db] = f32x16_t{};
  // At D = 128 the dP^T products accumulate onto -Delta (one value per lane: its query),
  // so they yield dP - Delta directly and dS needs one multiply per element. (At D = 64
  // the 16 registers would cost the second workgroup per CU.)
  constexpr bool kFoldDelta = D == 128;
  f32x16_t ndl;
#pragma unroll
  for (int r = 0; r < 16; ++r) ndl[r] = kFoldDelta ? -dl : 0.f;

  // Staging: K and V tiles of 64 keys by direct loads; rows past the end read the last
  // row (finite; masked below).
  constexpr int CS = G::SS / 16;
  static_assert(G::ST == CS * 1024, "a padded tile is CS kilobytes");
  auto gload = [&](int t, int slot) __attribute__((always_inline)) {
    const uint8_t* s = smem + slot * SLOT;
    const Staging<D, CS, kWavesQ> st(t, N, wave, lane);
    st.issue(Kh, s, t, wave);
    st.issue(Vh, s + G::ST, t, wave);
  };
  const int roff = row_off(lane, G::SS), toff = tr_off(lane, G::SS);
  const int first_masked = CAUSAL ? min(N >> 5, qw0 >> 5) : (N >> 5);

  auto step = [&](int g, const uint8_t* s) {
    const int b = (g & 1) * 32;
    const uint8_t* kr = s + b * G::SS + roff;
    const uint8_t* kt = s + b * G::SS + toff;
    const uint8_t* vr = s + G::ST + b * G::SS + roff;
    f32x16_t st = f32x16_t{}, dp = ndl;
#pragma unroll
    for (int c2 = 0; c2 < G::NCH; ++c2) {
      st = mfma(frag_row(kr, c2), as_bf16x8(qf[c2]), st);
      dp = mfma(frag_row(vr, c2), as_bf16x8(df[c2]), dp);
    }
    if (g >= first_masked) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * g + swap23(8 * (r >> 2) + 4 * half + (r & 3));
        if (key >= N || (CAUSAL && key > qrow)) st[r] = kNegInf;
      }
    }
    uint32_t ds[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p0 = exp2_hw(fmaf(st[2 * i], c, -lse2));
      const float p1 = exp2_hw(fmaf(st[2 * i + 1], c, -lse2));
      if constexpr (kFoldDelta)
        ds[i] = pack_bf16x2(p0 * dp[2 * i], p1 * dp[2 * i + 1]);
      else
        ds[i] = pack_bf16x2(p0 * (dp[2 * i] - dl), p1 * (dp[2 * i + 1] - dl));
    }
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const u32x4_t bop = {ds[4 * cc], ds[4 * cc + 1], ds[4 * cc + 2], ds[4 * cc + 3]};
#pragma unroll
      for (int db = 0; db < G::NDB; ++db)
        acc[db] = mfma(frag_tr(kt, cc, db, G::SS), as_bf16x8(bop), acc[db]);
    }
  };

  if (ntiles > 0) gload(0, 0);
  dma_wait();
  __syncthreads();
  // Tile t is read from slot t & 1; the loads of tile t + 1 go to the other slot, last
  // read before the barrier that ended tile t - 1, and are waited for before the
  // barrier that ends tile t.
#pragma unroll 1
  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) gload(t + 1, (t + 1) & 1);
    const uint8_t* s = smem + (t & 1) * SLOT;
    if (2 * t < nblk) step(2 * t, s);
    if (2 * t + 1 < nblk) step(2 * t + 1, s);
    dma_wait();
    __syncthreads();
  }

  if (qrow < N) {
    float* orow = dQ + head + int64_t(qrow) * D;
#pragma unroll
    for (int db = 0; db < G::NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4_t val = {acc[db][4 * g4] * scale, acc[db][4 * g4 + 1] * scale,
                             acc[db][4 * g4 + 2] * scale, acc[db][4 * g4 + 3] * scale};
        *reinterpret_cast<f32x4_t*>(orow + 32 * db + 8 * g4 + 4 * half) = val;
      }
  }
}

// ------------------------------------------------------------------ dK, dV
template <int D, bool CAUSAL>
__global__ __launch_bounds__(KV<D>::kThreads, 1) void dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ DELTA, float* __restrict__ dK,
    float* __restrict__ dV, int N, int BH, int nkt, float c, float scale) {
  using G = BGeo<D>;
  // Q, dO, then lse2 and Delta of the tile's 64 queries.
  constexpr int SLOT = 2 * G::ST + 2 * kTile * 4;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * SLOT];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  int bh, kt;
  map_bwd(blockIdx.x, BH, nkt, CAUSAL, false, bh, kt);
  const int64_t head = int64_t(bh) * N * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* dOh = dO + head;
  const float* lseh = LSE + int64_t(bh) * N;
  const float* delh = DELTA + int64_t(bh) * N;
  constexpr int kWavesB = KV<D>::kWaves;
  const int k0 = kt * KV<D>::kRows, kw0 = k0 + 32 * wave, krow = kw0 + l32;

  // Query blocks this wavefront folds: [gs, nblk_all) (causal: from its diagonal).
  const int nblk_all = (N + 31) >> 5;
  const int gs = kw0 >= N ? nblk_all : (CAUSAL ? (kw0 >> 5) : 0);
  const int t_first = CAUSAL ? (k0 >> 6) : 0;          // first tile the workgroup stages
  const int ntiles_all = (nblk_all + 1) >> 1;

  // Own rows: K^T and V^T as B operands (k = head dims 16 c2 + 8 half + 0..7).
  u32x4_t kf[G::NCH], vf[G::NCH];
  {
    const bool ok = krow < N;
#pragma unroll
    for (int c2 = 0; c2 < G::NCH; ++c2) {
      kf[c2] = ok ? load16(K + head + int64_t(krow) * D + 16 * c2 + 8 * half) : u32x4_t{0, 0, 0, 0};
      vf[c2] = ok ? load16(V + head + int64_t(krow) * D + 16 * c2 + 8 * half) : u32x4_t{0, 0, 0, 0};
    }
  }
  f32x16_t dva[G::NDB], dka[G::NDB];
#pragma unroll
  for (int db = 0; db < G::NDB; ++db) {
    dva[db] = f32x16_t{};
    dka[db] = f32x16_t{};
  }

  // Q and dO by direct loads, each into its row and transposing layouts; the 64 lse
  // and Delta values of a tile go through registers (threads 0..63).
  constexpr int CS = G::SS / 16;
  static_assert(G::ST == CS * 1024, "a padded tile is CS kilobytes");
  float sl = 0.f, sdl = 0.f;
  auto gload = [&](int t, int slot) __attribute__((always_inline)) {
    const uint8_t* s = smem + slot * SLOT;
    const Staging<D, CS, kWavesB> st(t, N, wave, lane);
    st.issue(Qh, s, t, wave);
    st.issue(dOh, s + G::ST, t, wave);
    if (tid < kTile) {
      const int q = t * kTile + tid;
      const float l = q < N ? lseh[q] : kNegInf;
      sl = l == kNegInf ? kInfB : l * kLog2e;  // padding or key-less rows: P = 0
      sdl = q < N ? delh[q] : 0.f;
    }
  };
  auto lstore = [&](int slot) __attribute__((always_inline)) {
    uint8_t* s = smem + slot * SLOT;
    if (tid < kTile) {
      float* f = reinterpret_cast<float*>(s + 2 * G::ST);
      f[tid] = sl;
      f[kTile + tid] = -sdl;  // -Delta: the dP products accumulate onto it
    }
  };
  const int roff = row_off(lane, G::SS), toff = tr_off(lane, G::SS);

  // Registers 8 cc + 4 h4 + k hold query 32 g + 16 cc + 8 half + 4 h4 + k: each group
  // of four reads its four lse (P) or Delta (dS) values just before use.
  // P of block g, packed to bf16; `masked` is a std::integral_constant: unmasked blocks
  // carry no mask arithmetic.
  auto ew_p = [&](int g, const uint8_t* s, const f32x16_t& st, auto masked, uint32_t (&pk)[8])
      __attribute__((always_inline)) {
    const float* fl = reinterpret_cast<const float*>(s + 2 * G::ST) + (g & 1) * 32;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int h4 = 0; h4 < 2; ++h4) {
        const f32x4_t l4 = *reinterpret_cast<const f32x4_t*>(fl + 16 * cc + 8 * half + 4 * h4);
#pragma unroll
        for (int k2 = 0; k2 < 4; k2 += 2) {
          float pv[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int k = k2 + e, r = 8 * cc + 4 * h4 + k;
            const int q = 32 * g + 16 * cc + 8 * half + 4 * h4 + k;
            float sv = st[r];
            if (decltype(masked)::value && (q >= N || (CAUSAL && krow > q))) sv = kNegInf;
            pv[e] = exp2_hw(fmaf(sv, c, -l4[k]));
          }
          pk[(8 * cc + 4 * h4 + k2) >> 1] = pack_bf16x2(pv[0], pv[1]);
        }
      }
  };
  // -Delta of block g's queries in accumulator order: the initial value of its dP
  // products, which thereby yield dP - Delta.
  auto neg_delta = [&](int g, const uint8_t* s) __attribute__((always_inline)) {
    const float* fd = reinterpret_cast<const float*>(s + 2 * G::ST) + kTile + (g & 1) * 32;
    f32x16_t init;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int h4 = 0; h4 < 2; ++h4) {
        const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(fd + 16 * cc + 8 * half + 4 * h4);
#pragma unroll
        for (int k = 0; k < 4; ++k) init[8 * cc + 4 * h4 + k] = d4[k];
      }
    return init;
  };
  // dS = P (dP - Delta) of block g from the packed P (the values the dV product used);
  // masked entries have P = 0, so dS needs no mask.
  auto ew_ds = [&](const f32x16_t& dpd, const uint32_t (&pk)[8], uint32_t (&dsk)[8])
      __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      dsk[i] = pack_bf16x2(bf16_lo(pk[i]) * dpd[2 * i], bf16_hi(pk[i]) * dpd[2 * i + 1]);
  };
  // dV^T += dO^T P or dK^T += Q^T dS for block g (transposing reads of the tile).
  auto tr_product = [&](int g, const uint8_t* tb0, const uint32_t (&b)[8], f32x16_t (&acc)[G::NDB])
      __attribute__((always_inline)) {
    const uint8_t* tb = tb0 + (g & 1) * 32 * G::SS + toff;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const u32x4_t bop = {b[4 * cc], b[4 * cc + 1], b[4 * cc + 2], b[4 * cc + 3]};
#pragma unroll
      for (int db = 0; db < G::NDB; ++db)
        acc[db] = mfma(frag_tr(tb, cc, db, G::SS), as_bf16x8(bop), acc[db]);
    }
  };
  // S = Q K^T or dP = dO V^T of block g (row reads of the tile, own fragments), added
  // to the initial value of `out`.
  auto rows_product = [&](int g, const uint8_t* rb0, const u32x4_t (&own)[G::NCH], f32x16_t& out)
      __attribute__((always_inline)) {
    const uint8_t* r = rb0 + (g & 1) * 32 * G::SS + roff;
#pragma unroll
    for (int c2 = 0; c2 < G::NCH; ++c2) out = mfma(frag_row(r, c2), as_bf16x8(own[c2]), out);
  };
  // One block, one chain: S, P, dV^T, then dP, dS, dK^T, so S and dP are never live at
  // once (with both 32 x D accumulators and the own K^T, V^T fragments this fits the 256
  // registers of two wavefronts per SIMD). The diagonal and ragged blocks (queries past
  // N, or below a key of this wavefront under the causal mask) take the masked P.
  auto step = [&](int g, const uint8_t* s) __attribute__((always_inline)) {
    uint32_t pk[8], dsk[8];
    {
      f32x16_t st = f32x16_t{};
      rows_product(g, s, kf, st);
      if ((32 * g + 32 > N) || (CAUSAL && 32 * g < kw0 + 32))
        ew_p(g, s, st, std::true_type{}, pk);
      else
        ew_p(g, s, st, std::false_type{}, pk);
    }
    tr_product(g, s + G::ST, pk, dva);
    {
      f32x16_t dp = neg_delta(g, s);
      rows_product(g, s + G::ST, vf, dp);
      ew_ds(dp, pk, dsk);
    }
    tr_product(g, s, dsk, dka);
  };

  const int ntiles = k0 >= N ? 0 : ntiles_all - t_first;
  if (ntiles > 0) {
    gload(t_first, 0);
    lstore(0);
  }
  dma_wait();
  __syncthreads();
  // Tile i is read from slot i & 1; the loads of tile i + 1 go to the other slot, which
  // was last read before the barrier that ended tile i - 1, and are waited for before
  // the barrier that ends tile i.
#pragma unroll 1
  for (int i = 0; i < ntiles; ++i) {
    const int t = t_first + i;
    if (i + 1 < ntiles) gload(t + 1, (i + 1) & 1);
    const uint8_t* s = smem + (i & 1) * SLOT;
    if (2 * t >= gs && 2 * t < nblk_all) step(2 * t, s);
    if (2 * t + 1 >= gs && 2 * t + 1 < nblk_all) step(2 * t + 1, s);
    if (i + 1 < ntiles) lstore((i + 1) & 1);
    dma_wait();
    __syncthreads();
  }

  if (krow < N) {
    float* vrow = dV + head + int64_t(krow) * D;
    float* krw = dK + head + int64_t(krow) * D;
#pragma unroll
    for (int db = 0; db < G::NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int col = 32 * db + 8 * g4 + 4 * half;
        *reinterpret_cast<f32x4_t*>(vrow + col) =
            f32x4_t{dva[db][4 * g4], dva[db][4 * g4 + 1], dva[db][4 * g4 + 2], dva[db][4 * g4 + 3]};
        *reinterpret_cast<f32x4_t*>(krw + col) =
            f32x4_t{dka[db][4 * g4] * scale, dka[db][4 * g4 + 1] * scale,
                    dka[db][4 * g4 + 2] * scale, dka[db][4 * g4 + 3] * scale};
      }
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const BwdArgs& a, hipStream_t s) {
  const int64_t BH = int64_t(a.B) * a.H;
  const float c = a.scale * kLog2e;
  const auto* q = static_cast<const uint16_t*>(a.q);
  const auto* k = static_cast<const uint16_t*>(a.k);
  const auto* v = static_cast<const uint16_t*>(a.v);
  const auto* dout = static_cast<const uint16_t*>(a.dout);
  const int nt = int((int64_t(a.N) + KV<D>::kRows - 1) / KV<D>::kRows);
  const int ntq = int((int64_t(a.N) + kRowsQ - 1) / kRowsQ);
  const int64_t blocks = BH * nt, qblocks = BH * ntq;
  if (qblocks > 0x7fffffff || blocks > 0x7fffffff) return hipErrorInvalidValue;
  // dQ first: it also writes Delta, which the dK/dV kernel reads
  hipLaunchKernelGGL((dq_kernel<D, CAUSAL>), dim3(unsigned(qblocks)), dim3(kThreadsQ), 0, s, q,
                     k, v, dout, a.o, a.lse, a.delta, a.dq, a.N, int(BH), ntq, c, a.scale);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((dkdv_kernel<D, CAUSAL>), dim3(unsigned(blocks)), dim3(KV<D>::kThreads), 0, s, q,
                     k, v, dout, a.lse, a.delta, a.dk, a.dv, a.N, int(BH), nt, c, a.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s) {
  if (a.D == 128) return a.causal ? launch<128, true>(a, s) : launch<128, false>(a, s);
  return a.causal ? launch<64, true>(a, s) : launch<64, false>(a, s);
}

}  // namespace fa
