/*
 * fa.h -- C ABI of libfa.so: exact tiled attention forward, its backward, split-KV
 * decode, and row reductions on the same schedule, for AMD Instinct MI355X (gfx950).
 *
 * What is computed (definitions from "Learning FlashAttention the Hard Way --
 * Part 1", cloudrift.ai):
 *   S = scale * Q K^T, P = row-wise softmax(S), O = P V  (section "FlashAttention:
 *   Not So Special"), without ever writing S or P to memory: each query row folds
 *   its key/value tiles into the state u = (m, d, o) -- running maximum, running
 *   denominator relative to it, unnormalised output row -- where one key enters as
 *   (s_j, 1, v_j), two states merge by rescaling each side by e^{(its max) - (new
 *   max)} and adding (sections "The State" and "The Merge, and the Twist"), the
 *   identity (-inf, 0, 0) pads ragged and masked keys (sections "Associativity is
 *   All You Need" and "Why Attention's Combine Still Associates"), and the row is
 *   read out once as o / d.  The log-sum-exp written beside O is
 *   lse = ln sum_j e^{s_j} = m + ln d, the absolute-coordinate denominator of
 *   section "Why Attention's Combine Still Associates", in natural-log units.
 *
 * Conventions shared by every call:
 *   - Every tensor pointer is a DEVICE pointer allocated and owned by the caller.
 *     The library allocates nothing, keeps no pointer after a call returns and
 *     holds no mutable global state; calls on different streams are independent.
 *   - Tensors are dense and row-major: q, k, v are [B][H][rows][D] with D fastest.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Every
 *     call only enqueues work on it and returns; nothing synchronises the host.
 *     Faults inside a kernel surface at the caller's next synchronisation.
 *   - Return value: FA_OK (0) or a negative FA_ERR_* code. Arguments are fully
 *     validated before any HIP call is made, so a rejected call enqueues nothing.
 *     Checks run in this order: sizes (FA_ERR_SHAPE), dtype, scalar arguments;
 *     then an empty problem (B, H or N zero; B or H zero for decode; rows zero for
 *     combine) returns FA_OK without touching any pointer, which may then be NULL;
 *     then NULL pointers and alignment.
 *   - NaN or Inf in the inputs is not checked; it propagates into the outputs.
 */
#ifndef FA_H
#define FA_H

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k and v. Accumulation and all outputs are float32. */
typedef enum { FA_F32 = 0, FA_BF16 = 1 } fa_dtype;

enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,  /* a required pointer is NULL                                  */
  FA_ERR_SHAPE = -2, /* negative size, D not in {64, 128}, splits < 1, or a size
                        whose element count does not fit in 63 bits                 */
  FA_ERR_DTYPE = -3, /* dtype is neither FA_F32 nor FA_BF16 (or FA_F32 with a
                        window or packed sequences)                                 */
  FA_ERR_ALIGN = -4, /* a tensor pointer is not 16-byte aligned; m, d, lse or delta
                        not 4-byte aligned; a row-reduction input not aligned to its
                        element                                                     */
  FA_ERR_HIP = -5,   /* the HIP runtime rejected the kernel launch                   */
  FA_ERR_ARG = -6,   /* scale not finite or not > 0, causal not 0 or 1, or a window
                        bound below -1 (numbered after FA_ERR_HIP so the first five
                        codes keep the values of the original five-code interface) */
  FA_ERR_SCRATCH = -7 /* fa_decode_noalloc: the partial states need more than the
                         library's static scratch (FA_DECODE_SCRATCH_FLOATS); a _ws
                         scan: the workspace is smaller than fa_scan_workspace_bytes */
};

/* Capacity, in floats, of the static device array fa_decode_noalloc keeps its
   partial states in (32 MiB per GPU). */
#define FA_DECODE_SCRATCH_FLOATS 8388608

/*
 * fa_forward -- exact attention forward with log-sum-exp.
 *
 *   q, k, v : [B][H][N][D] elements of `dtype` (bfloat16 or float32), read only.
 *   o       : [B][H][N][D] float32, written: o[b][h][i] = sum_j P_ij v_j.
 *   lse     : [B][H][N] float32, written: lse[b][h][i] = ln sum_j e^{S_ij} over the
 *             keys row i may see (-inf and an all-zero o row if it sees none).
 *   scale   : the softmax scale multiplying Q K^T (e.g. 1/sqrt(D)); finite, > 0.
 *   causal  : 0 = every key visible; 1 = key j visible to query i iff j <= i.
 *   D       : head dimension, 64 or 128.
 * Scores are formed from the inputs exactly as given, accumulated in float32; the
 * probabilities fed to the P V product are rounded to the input type.
 * Range: each weight's exponent is formed as s c - m c in one float32 fused
 * multiply-add (c = scale log2 e, m the running maximum), so the rounding of m c,
 * |m c| 2^-24, enters it. Results hold to bf16 precision while the scaled scores stay
 * below about 2e4 in magnitude (attention's are tens to hundreds); far larger ones
 * (a scale of 1e20 on unit-size inputs) lose the weights and can come back as NaN.
 * The same holds for fa_forward_ext and fa_backward; fa_decode_partials subtracts
 * the maximum before scaling and holds at any magnitude.
 */
int fa_forward(const void* q, const void* k, const void* v, float* o, float* lse,
               int B, int H, int N, int D, float scale, int causal, int dtype,
               void* stream);

/*
 * fa_forward_ext -- fa_forward with mask variants: a sliding window and packed
 * variable-length sequences. Masked keys enter as the identity of the fold (score
 * -inf, weight 0; sections "Associativity is All You Need" and "Why Attention's
 * Combine Still Associates"), and key tiles wholly outside a row block's window are
 * not visited at all.
 *
 *   window_left, window_right : key j is visible to query i iff
 *             i - window_left <= j <= i + window_right; -1 leaves that side
 *             unbounded (other negative values: FA_ERR_ARG). causal = 1 also bounds
 *             the right side at 0 (j <= i).
 *   cu_seqlens : NULL for the dense layout of fa_forward. Otherwise a DEVICE array of
 *             B + 1 int32 offsets (nondecreasing, cu_seqlens[0] = 0,
 *             cu_seqlens[B] <= N): B packed sequences, sequence s owning rows
 *             [cu_seqlens[s], cu_seqlens[s+1]) of every head; q, k, v and o are then
 *             [H][N][D] and lse is [H][N], and each sequence attends only to itself
 *             (positions counted from its first row). Offsets are clamped into
 *             [0, N] on the device, so inconsistent contents cannot make the library
 *             touch memory outside the tensors.
 *   max_seqlen : packed only: an upper bound on every sequence length. A longer
 *             sequence is taken as its first max_seqlen rows (they attend to those rows
 *             only) and its later rows are left unwritten; rows past cu_seqlens[B] are
 *             never written.
 * Windows and packed sequences need dtype FA_BF16 (FA_F32 returns FA_ERR_DTYPE).
 * fa_forward(...) is fa_forward_ext(..., -1, -1, NULL, 0, ...).
 */
int fa_forward_ext(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                   int H, int N, int D, float scale, int causal, int window_left,
                   int window_right, const int* cu_seqlens, int max_seqlen, int dtype,
                   void* stream);

/*
 * fa_decode_partials -- split-KV single-query attention, first step.
 * Split-K as in section "Associativity is All You Need": the L keys of every head
 * are cut into `splits` chunks of c = ceil(L / splits) keys (chunk s covers keys
 * [s*c, min(L, (s+1)*c)); chunks past the end are empty), and each chunk's state
 * is written to caller-owned scratch for fa_combine_partials to fold.
 *
 *   q       : [B][H][D] (one query row per head) of `dtype`.
 *   k, v    : [B][H][L][D] of `dtype`.
 *   m, d    : [B*H][splits] float32, written. m = max_j s_j over the chunk in
 *             natural-log units of the scaled score s_j = scale * q.k_j;
 *             d = sum_j e^{s_j - m}, so 1 <= d <= chunk length.
 *   o_part  : [B*H][splits][D] float32, written: sum_j e^{s_j - m} v_j (NOT
 *             divided by d).
 *   An empty chunk is written as the identity: m = -inf, d = 0, o_part = 0.
 *   L may be 0 (every chunk is empty); k and v may then be NULL.
 * Scratch size: B*H*splits*(D + 2) floats, owned and freed by the caller.
 */
int fa_decode_partials(const void* q, const void* k, const void* v, float* m, float* d,
                       float* o_part, int B, int H, int L, int D, float scale, int splits,
                       int dtype, void* stream);

/*
 * fa_decode_noalloc -- fa_decode_partials followed by fa_combine_partials in one call
 * that allocates nothing: the partial states live in a static device array of the
 * library instead of caller scratch. For callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Same kernels, so the same results as the two calls with caller scratch.
 *
 *   q, k, v, B, H, L, D, scale, splits, dtype : as for fa_decode_partials.
 *   o       : [B*H][D] float32, written: the merged o / d of every head.
 *   lse     : [B*H] float32, written: the merged log-sum-exp (-inf for L = 0).
 *   Limit: with R = B*H*splits and R64 = R rounded up to a multiple of 64,
 *   2*R64 + R*D <= FA_DECODE_SCRATCH_FLOATS (m and d, then o_part, 256-byte aligned);
 *   a larger problem returns FA_ERR_SCRATCH before anything is launched. The
 *   split-KV decode of 16 x 32 heads at D = 128 in 64 chunks uses 4.26 M of the 8.39 M.
 *   Sharing: each GPU holds one such array (32 MiB, kept until the process ends), and
 *   every call on that GPU uses it. Calls that overlap on one GPU (other streams, other
 *   host threads) race on it and must be ordered by the caller; calls on one stream
 *   are ordered by the stream. Nothing in it needs clearing: every call writes all the
 *   states it reads.
 *   The first call on a device looks up that device's address of the array (a host
 *   query, no allocation); later calls reuse it.
 */
int fa_decode_noalloc(const void* q, const void* k, const void* v, float* o, float* lse,
                      int B, int H, int L, int D, float scale, int splits, int dtype,
                      void* stream);

/*
 * fa_combine_partials -- fold partial states with the combine of section "The
 * Merge, and the Twist" (identity states are skipped) and read each row out once.
 *
 *   m, d    : [rows][splits] float32 partial maxima (natural-log units) and
 *             denominators relative to them.
 *   o_part  : [rows][splits][D] float32 unnormalised partial outputs.
 *   o       : [rows][D] float32, written: the merged o / d.
 *   lse     : [rows] float32, written: M + ln(sum_s d_s e^{m_s - M}), M = max_s m_s.
 *   A row whose partials are all the identity is written as o = 0, lse = -inf.
 *   rows >= 0 (0 is an empty call), splits >= 1, D in {64, 128}.
 */
int fa_combine_partials(const float* m, const float* d, const float* o_part, int splits,
                        int rows, int D, float* o, float* lse, void* stream);

/*
 * fa_backward -- gradients of the attention forward with respect to q, k and v.
 * The pages name the backward pass that recomputes the attention matrix from the
 * per-row log-sum-exp instead of storing it, without printing formulas; the
 * gradients follow from the forward definition by the chain rule (dV = P^T dO,
 * dP = dO V^T, dS = P (dP - Delta) with Delta_i = sum_d dO_id O_id, dQ = scale dS K,
 * dK = scale dS^T Q), with P recomputed from lse.
 *
 *   q, k, v : [B][H][N][D] of `dtype`, the forward's inputs.
 *   o       : [B][H][N][D] float32 and
 *   lse     : [B][H][N] float32, the outputs fa_forward wrote for the same inputs,
 *             scale and causal (read only).
 *   dout    : [B][H][N][D] of `dtype`, the gradient of the loss with respect to o.
 *   delta   : [B][H][N] float32 caller-owned scratch, written (Delta_i); its
 *             contents on return are defined (Delta) but not part of the result.
 *   dq, dk, dv : [B][H][N][D] float32, written (overwritten, not accumulated).
 *   scale, causal, D : as for fa_forward.
 * For bfloat16 the products take bfloat16 operands (P and dS are rounded to
 * bfloat16 before the products that consume them) and accumulate in float32.
 * Alignment: q, k, v, o, dout, dq, dk, dv 16 bytes; lse, delta 4 bytes.
 */
int fa_backward(const void* q, const void* k, const void* v, const float* o, const float* lse,
                const void* dout, float* delta, float* dq, float* dk, float* dv, int B, int H,
                int N, int D, float scale, int causal, int dtype, void* stream);

/*
 * Row reductions on the same schedule as the attention fold, with another combine
 * (section "Associativity is All You Need": only the combine changes, never the
 * schedule). Both read x as [rows][n] elements of `dtype` (float32 or bfloat16),
 * dense and row-major, each element once; x needs only element alignment (2 or 4
 * bytes), the outputs 4 bytes. rows = 0 is an empty call (no pointer touched); n = 0
 * writes the identity state for every row (x may then be NULL). Accumulation is
 * float32.
 */

/*
 * fa_softmax_stats -- the online-softmax normaliser of every row (section "Online
 * Softmax Reparametrization"): the state (m, d) of the row, m = max_j x_j (exactly one
 * of the inputs) and d = sum_j e^{x_j - m}, so ln sum_j e^{x_j} = m + ln d and the
 * softmax of the row is e^{x_j - m} / d. -inf entries are the identity and add
 * nothing; a row of only -inf (or n = 0) is written as (-inf, 0).
 *   m, d : [rows] float32, written.
 */
int fa_softmax_stats(const void* x, float* m, float* d, int rows, int n, int dtype,
                     void* stream);

/*
 * fa_moments -- Welford's moments of every row in the pairwise form of Chan, Golub and
 * LeVeque (section "The Same Move: Welford's Variance"): the state (n, mu, M2) with
 * mu = (1/n) sum_j x_j and M2 = sum_j (x_j - mu)^2; the population variance is M2 / n,
 * the sample variance M2 / (n - 1). n is the row length and is not written; n = 0
 * writes mean = M2 = 0 (the identity).
 *   mean, m2 : [rows] float32, written.
 */
int fa_moments(const void* x, float* mean, float* m2, int rows, int n, int dtype, void* stream);

/*
 * fa_softmax_scan, fa_moments_scan -- inclusive prefix scans of the same two monoids:
 * a prefix sum is one more re-bracketing that any monoid allows (section "Wrap-Up",
 * first point). For every row r and position j the state of x[r][0..j] is written:
 *   fa_softmax_scan: m[r][j] = max_{i<=j} x[r][i], d[r][j] = sum_{i<=j} e^{x[r][i] - m[r][j]}
 *                    (-inf, 0 while the prefix holds only -inf);
 *   fa_moments_scan: mean[r][j] and m2[r][j] of the j + 1 elements x[r][0..j].
 *   outputs : two [rows][n] float32 arrays, written.
 * rows = 0 or n = 0 is an empty call (no pointer touched). Alignment: x to its element,
 * outputs 4 bytes (16-byte aligned x and outputs with n a multiple of 8 take vector
 * accesses). Element counts must fit int64 byte offsets (FA_ERR_SHAPE otherwise).
 */
int fa_softmax_scan(const void* x, float* m, float* d, int rows, int n, int dtype,
                    void* stream);
int fa_moments_scan(const void* x, float* mean, float* m2, int rows, int n, int dtype,
                    void* stream);

/*
 * fa_softmax_scan_ws, fa_moments_scan_ws -- the same scans, with a caller workspace that
 * lets one row be shared by several workgroups. A row of more than 32 KB of input whose
 * length n is a multiple of 2048 with 2 to 64 such blocks is cut into its 2048-element
 * blocks, one workgroup each: block k publishes the fold of its own elements and starts
 * from the fold of blocks 0 .. k-1 (the prefix of a monoid can be bracketed at any block
 * boundary, section "Associativity is All You Need"). Other rows, or tensors not
 * 16-byte aligned, take the one-workgroup-per-row path of fa_softmax_scan /
 * fa_moments_scan and leave the workspace untouched.
 *   workspace       : device memory of at least fa_scan_workspace_bytes(rows, n) bytes,
 *                     8-byte aligned, owned by the caller; may be NULL when that size is
 *                     0. The call clears and rewrites it (its contents on return mean
 *                     nothing); calls that overlap in time need separate workspaces.
 *   workspace_bytes : its size; smaller than needed returns FA_ERR_SCRATCH.
 *   max_polls       : how many times a block polls for an earlier block's published
 *                     fold before folding that block's elements itself (0: 65536; a
 *                     negative value returns FA_ERR_ARG). Every wait is bounded by it.
 * Results agree with fa_softmax_scan / fa_moments_scan to rounding (the folds are
 * bracketed differently), not bit for bit. Two calls on the same input give the same
 * bits unless a block ran out of polls in one of them (it then folds the late block
 * itself, bracketed differently again); at the default bound that takes a wait of tens
 * of milliseconds.
 */
int fa_softmax_scan_ws(const void* x, float* m, float* d, int rows, int n, int dtype,
                       void* workspace, long long workspace_bytes, int max_polls,
                       void* stream);
int fa_moments_scan_ws(const void* x, float* mean, float* m2, int rows, int n, int dtype,
                       void* workspace, long long workspace_bytes, int max_polls,
                       void* stream);
/* Workspace bytes the _ws scans need for rows x n elements of dtype: 8 per 2048-element
 * block when a row of more than 32 KB has 2 to 64 whole blocks, else 0; -1 for negative
 * or oversized sizes or an unknown dtype. */
long long fa_scan_workspace_bytes(int rows, int n, int dtype);

/*
 * Measurement calls. They compute nothing of the method: they measure the chip's
 * sustained rates on the two resources the kernels above are bound by, the measured
 * roofline denominators reported beside the published peaks.
 *
 * fa_calibrate_mfma -- `blocks` workgroups of 8 wavefronts; each wavefront runs `iters`
 * rounds of 16 bf16 matrix products 32x32x16 (8 independent float32 accumulators) on
 * register operands of random bf16 values in +-[0.5, 4) drawn from `seed`. One launch
 * is 2^19 * 8 * blocks * iters flops.
 *   out : [blocks * 512] float32, written (each thread's accumulator sum, which keeps
 *         the products from being elided; deterministic for a given seed).
 *   1 <= blocks <= 2^20 and iters >= 0 (FA_ERR_SHAPE otherwise); out 4-byte aligned.
 *
 * fa_calibrate_read -- a read-only stream over x[0 .. nbytes) in 16-byte non-temporal
 * loads by `blocks` workgroups of 256 threads. With n16 = nbytes / 16 words of 16 bytes
 * and S = ceil(n16 / blocks) rounded up to a multiple of 256, workgroup b reads words
 * [b S, min(n16, (b + 1) S)), its thread t those at offsets t, t + 256, t + 512, ...
 *   out : [blocks * 256] uint32, written: out[256 b + t] is the XOR of the four 32-bit
 *         words of every 16-byte word that thread read (0 if none).
 *   nbytes >= 0 and a multiple of 16, 1 <= blocks <= 2^22 (FA_ERR_SHAPE otherwise);
 *   x 16-byte aligned (may be NULL only when nbytes = 0), out 4-byte aligned.
 */
int fa_calibrate_mfma(float* out, int blocks, int iters, unsigned seed, void* stream);
/*
 * fa_calibrate_overlap -- whether one SIMD overlaps a matrix-product wavefront with a
 * vector-ALU wavefront. `blocks` workgroups of 8 wavefronts, one per CU (each reserves
 * 96 KB of LDS), so wavefronts w and w + 4 share a SIMD. Per round the matrix role
 * issues 16 bf16 products 32x32x16 in the pattern of one 32-key prefill step (a chain
 * of 8 and four chains of 2); the vector role issues that step's softmax instructions
 * (16 FMA, 16 exp2, 15 adds, 8 bf16 packs, 8 bf16 dot products).
 *   mode 0: wavefronts 0-3 matrix role only; 1: wavefronts 4-7 vector role only;
 *   2: both at once (one of each per SIMD); 3: every wavefront both roles in one
 *   instruction stream; 4: every wavefront the matrix role; 5: every wavefront the
 *   vector role; 6: each thread writes its wavefront's SIMD index (placement check);
 *   8 + m (m = 0..5): mode m, writing instead of checksums each wavefront's elapsed
 *   shader-clock cycles (lanes 0-31) and 100 MHz real-time ticks (lanes 32-63).
 *   Each role runs exactly `iters` rounds.
 *   out : [blocks * 512] float32, written: each thread's checksum (mode 6: SIMD index;
 *         modes 8-13: elapsed cycles or ticks; 0 for a wavefront with no role).
 *   1 <= blocks <= 2^20, iters >= 0 (FA_ERR_SHAPE); mode in 0..6 or 8..13 (FA_ERR_ARG).
 */
int fa_calibrate_overlap(float* out, int blocks, int iters, int mode, void* stream);
int fa_calibrate_read(const void* x, long long nbytes, unsigned* out, int blocks, void* stream);
/*
 * fa_calibrate_write -- a write-only stream over y[0 .. nbytes) in 16-byte non-temporal
 * stores, split over `blocks` workgroups of 256 threads as fa_calibrate_read splits its
 * reads. The 16-byte word w (w = 0, 1, ...) is written as the four 32-bit words
 * {value, w mod 2^32, value, w mod 2^32}.
 *   nbytes >= 0 and a multiple of 16, 1 <= blocks <= 2^22 (FA_ERR_SHAPE otherwise);
 *   y 16-byte aligned. nbytes = 0 returns FA_OK at once (y may then be NULL).
 */
int fa_calibrate_write(void* y, long long nbytes, unsigned value, int blocks, void* stream);
/*
 * fa_calibrate_mix -- one read stream and two write streams, with no arithmetic: the
 * traffic of a kernel that reads a buffer and writes two outputs `ratio` times its size
 * (the prefix scans: ratio 1 for float32 input, 2 for bfloat16), so its rate is the
 * measured ceiling for that mix of reads and writes. `blocks` workgroups of 256 threads
 * split x[0 .. nbytes) as fa_calibrate_read does and read their 16-byte words with
 * non-temporal loads; the run of 256 words starting at word j (j a multiple of 256) is
 * written, with non-temporal stores, to words ratio j + 256 r + t (r < ratio, t < 256:
 * word j + t) of both output streams. Stream 0 is y[0 .. ratio nbytes), stream 1
 * y[ratio nbytes .. 2 ratio nbytes).
 *   nbytes >= 0 and a multiple of 4096, ratio 1, 2 or 4, 1 <= blocks <= 2^22
 *   (FA_ERR_SHAPE otherwise); x and y 16-byte aligned, y holding 2 ratio nbytes bytes.
 *   nbytes = 0 returns FA_OK at once (x and y may then be NULL).
 */
int fa_calibrate_mix(const void* x, long long nbytes, void* y, int ratio, int blocks,
                     void* stream);

/* Static, human-readable name of an FA_* code (never NULL). */
const char* fa_strerror(int code);

/* ABI version of this header: 2 (version 1 had no workspace scans). */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
