/*
 * fa.h - C ABI of the exact IO-aware attention library (libfa.so), gfx950.
 *
 * What it computes. Exact scaled-dot-product attention forward,
 *     O = softmax(scale * Q K^T) V,  LSE_i = ln sum_{visible j} e^(scale <q_i, k_j>),
 * evaluated as tiled online softmax: score tiles live only in registers and
 * the N x N score matrix never reaches device memory
 * (FlashAttention: Part 2, section 2.1 for the function; section 6.2
 * "FlashAttention Summary" for the tile -> score -> online softmax -> V
 * accumulation -> discard pipeline; section 1.3 for the one log-sum-exp per
 * query row kept next to the output; section 1.2 for one workgroup per
 * query-row tile).
 *
 * Conventions shared by every entry point.
 *  - Pointers: every tensor pointer is a DEVICE pointer (HIP device memory)
 *    owned by the caller. The library never allocates, frees or
 *    synchronises; it only enqueues kernels on `stream`.
 *  - stream: a hipStream_t passed as void*; NULL means the null stream.
 *    Calls return as soon as the kernels are enqueued; results are ready
 *    once the stream reaches them. Device faults surface at the caller's
 *    next synchronisation.
 *  - Layout: dense, contiguous, row-major (batch, sequence, heads, head_dim)
 *    for q, k, v, o and the caches; lse is (batch, heads, queries) float32.
 *  - Grouped heads (pyshine.com FlashAttention code tour, "Why You Need
 *    This": K and V may carry fewer heads than Q when the counts divide):
 *    Hq must be a positive multiple of Hkv, and query head h reads key/value
 *    head h / (Hq / Hkv) (contiguous groups).
 *  - Errors: arguments are checked on the host before anything is
 *    enqueued; on any error nothing is written and a non-zero fa_status_t
 *    is returned. FA_ERR_LAUNCH reports a failed kernel launch.
 *  - Sizes are ints. Sequence lengths, capacities and packed row totals
 *    above 2^31 - 1024, grids beyond 32-bit indexing and row counts B * N
 *    above 2^31 - 1 return FA_ERR_UNSUPPORTED; the tensors themselves may
 *    hold more than 2^31 elements.
 *  - Thread safety: the library keeps no mutable state; concurrent calls
 *    on different streams are safe.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1, /* null pointer, negative size, Hq % Hkv != 0, bad scale */
  FA_ERR_UNSUPPORTED = 2, /* head_dim, dtype or sizes the library has no kernel for */
  FA_ERR_WORKSPACE = 3,   /* decode workspace missing or smaller than required */
  FA_ERR_LAUNCH = 4       /* the HIP runtime rejected a kernel launch */
} fa_status_t;

typedef enum {
  FA_DTYPE_BF16 = 0, /* bfloat16 in/out; bf16 MFMA products, fp32 accumulation */
  FA_DTYPE_F32 = 1   /* float32 in/out; fp32 products and accumulation */
} fa_dtype_t;

/* Version of this ABI (bumped on any incompatible change). */
int fa_abi_version(void);

/* Human-readable name of a status code; never NULL. */
const char* fa_status_string(int status);

/*
 * fa_fwd - prefill / training forward.
 *
 * q   : (B, Nq, Hq, d) of `dtype`.
 * k, v: (B, Nk, Hkv, d) of `dtype`.
 * o   : (B, Nq, Hq, d) of `dtype`, written.
 * lse : (B, Hq, Nq) float32, written (natural-log units of the scaled
 *       scores); may be NULL when the caller does not need it.
 * causal: 0 = every key visible; 1 = top-left causal, key j is visible to
 *       query i iff j <= i (pyshine.com FlashAttention code tour, "From
 *       Install to Causal Attention"; for Nq == Nk top-left and bottom-right
 *       alignment coincide).
 * scale: multiplies q.k before the softmax; must be finite and > 0
 *       (1/sqrt(d) reproduces the usual definition).
 * d   : 64, 128 or 256 for FA_DTYPE_BF16; 64 for FA_DTYPE_F32.
 *
 * B == 0 or Nq == 0 is a no-op. Nk == 0 leaves every row without a visible
 * key: o = 0 and lse = -inf. Rows never produce NaN from masking.
 * Returns FA_ERR_INVALID_ARG for a negative size, Hq % Hkv != 0, a null
 * q/k/v/o pointer with non-zero extent, or a bad scale; FA_ERR_UNSUPPORTED
 * for an unsupported (dtype, d), B or Hq above 65535, or B * Nq or B * Nk
 * above 2^31 - 1 rows (32-bit row indices; tensors themselves may exceed
 * 2^31 elements).
 */
fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int Nq, int Nk, int d,
                   int causal, float scale, int dtype, void* stream);

/*
 * fa_fwd_kvcache - split-KV decode: one new query per sequence against a
 * contiguous key/value cache (pyshine.com FlashAttention code tour, "Why You
 * Need This": with query length one the cache loading is split across
 * workgroups and the partial results are combined; FlashAttention: Part 2,
 * section 4.1: decode reads the cache and is memory-bound).
 *
 * q            : (B, 1, Hq, d) bf16.
 * kcache,vcache: (B, capacity, Hkv, d) bf16; rows at or beyond
 *                cache_seqlens[b] are never read.
 * cache_seqlens: (B,) int32 device array; key j of sequence b is visible iff
 *                j < cache_seqlens[b]. Values are clamped to [0, capacity].
 * o            : (B, 1, Hq, d) bf16, written.
 * lse          : (B, Hq) float32, written; may be NULL.
 * num_splits   : S >= 1. S == 1: one workgroup per (sequence, key/value
 *                head) streams all its keys and writes o directly; no
 *                workspace. S >= 2: the tiles of 64 keys (32 at d = 256) of
 *                every (sequence, key/value head) pair, laid end to end in
 *                (b, h) order, are cut into U = (S - 1) B Hkv equal runs,
 *                one per workgroup, whatever the lengths; a run writes a
 *                partial (O, LSE) for each pair it touches into the
 *                workspace and a second kernel merges a pair's parts with
 *                log-sum-exp weights, in run order.
 * workspace    : device scratch of at least
 *                fa_fwd_kvcache_workspace_size(B, Hq, d, num_splits) bytes
 *                (may be NULL when that size is 0). Contents on entry are
 *                ignored; calls sharing one workspace must be ordered on
 *                one stream.
 * d            : 64, 128 or 256; Hq / Hkv must be at most 16.
 * L_b == 0 gives o = 0 and lse = -inf for that sequence.
 */
fa_status_t fa_fwd_kvcache(const void* q, const void* kcache, const void* vcache,
                           const int32_t* cache_seqlens, void* o, float* lse,
                           int num_splits, int B, int Hq, int Hkv, int capacity, int d,
                           float scale, void* workspace, size_t workspace_bytes, void* stream);

/* fa_fwd_kvcache for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments, results and errors as fa_fwd_kvcache (the
 * same kernels run), except that there is no workspace argument: the split
 * partials go to a scratch array that the library holds in static device
 * memory, FA_NOALLOC_SCRATCH_BYTES per GPU, for as long as the process
 * lives. Nothing is allocated or freed by the call.
 *  - Sizes whose workspace (fa_fwd_kvcache_workspace_size(B, Hq, d,
 *    num_splits)) exceeds FA_NOALLOC_SCRATCH_BYTES return FA_ERR_WORKSPACE
 *    before anything is enqueued (fewer splits, or fa_fwd_kvcache with a
 *    caller workspace, serve larger batches).
 *  - Every call on one GPU uses that GPU's single scratch array, whose
 *    contents carry over from the previous call (the kernels write every
 *    partial before reading it, so nothing has to start cleared). Calls
 *    that can overlap on one GPU (different streams, or several host
 *    threads) race on it: order them on one stream.
 *  - The scratch array of a device is looked up (hipGetSymbolAddress) on the
 *    first call that needs it with that device current; a failed lookup
 *    returns FA_ERR_LAUNCH. */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
fa_status_t fa_fwd_kvcache_noalloc(const void* q, const void* kcache, const void* vcache,
                                   const int32_t* cache_seqlens, void* o, float* lse,
                                   int num_splits, int B, int Hq, int Hkv, int capacity, int d,
                                   float scale, void* stream);

/* Bytes of workspace fa_fwd_kvcache needs for these sizes (0 when
 * num_splits <= 1); 0 also for invalid sizes. */
size_t fa_fwd_kvcache_workspace_size(int B, int Hq, int d, int num_splits);

/* A num_splits for fa_fwd_kvcache (and fa_fwd_kvcache_paged / _noalloc) on
 * B sequences of at most `capacity` keys, Hkv key/value heads and head
 * dimension d, on a device with `num_cus` compute units each holding
 * `wgs_per_cu` resident decode workgroups. Pass 0 for num_cus to use the
 * current device's count, and 0 for wgs_per_cu to take it from
 * hipOccupancyMaxActiveBlocksPerMultiprocessor for the decode kernel that d
 * selects (2 if no device can be queried); counts above 65536 CUs and 1024
 * workgroups per CU are taken as those. With num_splits = S >= 2 the
 * single-query decode cuts the cache work of all sequences into
 * (S - 1) B Hkv equal runs, which the resident workgroups take in waves;
 * the default takes the fewest runs per pair (1 .. max(8, resident
 * workgroups / pairs)) whose waves leave at most 1/8 of the workgroup time
 * idle (else the least idle), each run at least ~8 tiles of 64 keys, and 1
 * (no split) when
 * there are four or more (sequence, key/value head) pairs per resident
 * workgroup. Always >= 1. */
int fa_kvcache_default_splits(int B, int Hkv, int capacity, int d, int num_cus, int wgs_per_cu);

/* A num_splits for the decode calls with appended rows or several queries
 * per sequence (fa_fwd_kvcache_append, fa_fwd_kvcache_paged_append). With
 * Nq * (Hq / Hkv) <= 16 those calls take the balanced decode and this is
 * fa_kvcache_default_splits(B, Hkv, capacity, d, num_cus, wgs_per_cu).
 * Wider calls split every sequence's keys by position, split s covering
 * keys [s c, (s+1) c): splits of about 1024 keys, at least enough to fill
 * every resident workgroup (wgs_per_cu, or 0: from the occupancy API for
 * that kernel), at most 4 workgroups per resident slot. Always >= 1 (1
 * also for invalid sizes). */
int fa_kvcache_append_default_splits(int B, int Nq, int Hkv, int Hq, int capacity, int d, int num_cus,
                                     int wgs_per_cu);

/* fa_fwd with a local window, aligned to the bottom-right corner
 * (pyshine.com FlashAttention code tour: bottom-right causal alignment
 * since 2.1, sliding windows since 2.3). Key j is visible to query i iff
 *     i + off - window_left <= j <= i + off + window_right,  off = Nk - Nq;
 * a negative bound is unlimited. (-1, 0) is bottom-right causal (for
 * Nq == Nk the same as fa_fwd's causal), (-1, -1) no mask, (w, 0) a
 * causal sliding window of w + 1 keys. Rows that see no key get O = 0 and
 * LSE = -inf. bfloat16 only, d in {64, 128, 256}; other arguments and
 * errors as fa_fwd. */
fa_status_t fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int Hq, int Hkv, int Nq, int Nk, int d,
                          int window_left, int window_right, float scale, void* stream);

/* fa_fwd_window over a packed variable-length batch (pyshine.com code
 * tour: variable-length batches since 2.0; padded batches are flattened
 * into packed token arrays). Sequence b is rows cu_seqlens_q[b] ..
 * cu_seqlens_q[b+1]-1 of q and o, (total_q, Hq, d) bfloat16, against rows
 * cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 of k and v, (total_k, Hkv, d);
 * the window is aligned to each sequence's own bottom-right corner.
 *   cu_seqlens_q, cu_seqlens_k : (B + 1,) int32 on the device, nondecreasing,
 *                                starting at 0 and ending at total_q / total_k
 *   max_seqlen_q               : the longest query sequence (the grid covers
 *                                that many rows per sequence; longer ones are
 *                                cut there)
 *   lse                        : (Hq, total_q) float32, or NULL
 * Offsets outside [0, total] are clamped, so no access leaves the arrays.
 * bfloat16 only, d in {64, 128, 256}. */
fa_status_t fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                          int B, int Hq, int Hkv, int max_seqlen_q, int total_q, int total_k, int d,
                          int window_left, int window_right, float scale, void* stream);

/* fa_fwd_kvcache over a paged cache (pyshine.com FlashAttention code tour:
 * the paged KV cache of flash_attn_with_kvcache, after the PagedAttention
 * layout). Keys [i * page_size, (i + 1) * page_size) of sequence b live in
 * page block_table[b * pages_per_seq + i] of the page pools:
 *   kpages, vpages : (num_pages, page_size, Hkv, d) bfloat16
 *   block_table    : (B, pages_per_seq) int32 on the device; only the
 *                    entries covering [0, cache_seqlens[b]) are read, and an
 *                    entry outside [0, num_pages) is clamped into it (no
 *                    out-of-range read; the result is then unspecified)
 * Everything else (q, o, lse, cache_seqlens, num_splits, workspace,
 * results) is as fa_fwd_kvcache with capacity = page_size * pages_per_seq;
 * on the same keys the two return bitwise-identical results.
 * page_size must be a positive multiple of 64 (FA_ERR_INVALID_ARG). */
fa_status_t fa_fwd_kvcache_paged(const void* q, const void* kpages, const void* vpages,
                                 const int32_t* block_table, const int32_t* cache_seqlens, void* o, float* lse,
                                 int num_splits, int B, int Hq, int Hkv, int page_size, int pages_per_seq,
                                 int num_pages, int d, float scale, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* Decode step that appends to the cache in the same launch (pyshine.com
 * FlashAttention code tour, "Why You Need This" and its usage example: the
 * with-kvcache entry point updates the preallocated cache in place with the
 * new tokens, then attends; causal masking is bottom-right aligned since
 * version 2.1). Nq >= 1 queries per sequence:
 *   q, o           : (B, Nq, Hq, d) bfloat16    lse : (B, Hq, Nq) float32 or NULL
 *   k_new, v_new   : (B, Nq, Hkv, d) bfloat16, both NULL (attend to the
 *                    cache as it is) or both set (append first)
 *   kcache, vcache : (B, capacity, Hkv, d) bfloat16; with k_new set, rows
 *                    base_b .. base_b + Nq - 1 are overwritten, where base_b
 *                    is cache_seqlens[b] clamped to [0, capacity]; rows at or
 *                    past capacity are dropped. No other row is written.
 *   cache_seqlens  : (B,) int32 on the device, read only (the caller
 *                    advances it after the step)
 * With n_b = base_b + (Nq if appending else 0), query i of sequence b sees
 * keys j < min(n_b, capacity) and, when causal, only j <= n_b - Nq + i; a
 * query that sees no key gets o = 0 and lse = -inf.
 * Splits, workspace and stream rules are those of fa_fwd_kvcache with B * Nq
 * in place of B in fa_fwd_kvcache_workspace_size. The new rows must not
 * alias q, o or one another. Calls that write one cache must be ordered on
 * one stream. With Nq = 1 and nothing appended the results are bitwise
 * those of fa_fwd_kvcache. Nq * (Hq / Hkv) (query, head) pairs per key/value
 * head are served 16 per workgroup; each such group streams the cache once.
 * With at most 16 of them and num_splits = S >= 2 the cache work is cut
 * into (S - 1) B Hkv equal runs as in fa_fwd_kvcache, and a tile's appended
 * rows are written by the workgroup that then reads that tile; with more,
 * each sequence's keys are cut into S ranges by position.
 * FA_ERR_INVALID_ARG for Nq < 1 or only one of k_new / v_new. */
fa_status_t fa_fwd_kvcache_append(const void* q, const void* k_new, const void* v_new, void* kcache, void* vcache,
                                  const int32_t* cache_seqlens, void* o, float* lse, int causal, int num_splits,
                                  int B, int Nq, int Hq, int Hkv, int capacity, int d, float scale,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* fa_fwd_kvcache_append over a paged cache: the pages and block_table are
 * those of fa_fwd_kvcache_paged (capacity = page_size * pages_per_seq), the
 * new rows land in the pages that block_table names for positions base_b ..
 * base_b + Nq - 1. */
fa_status_t fa_fwd_kvcache_paged_append(const void* q, const void* k_new, const void* v_new, void* kpages,
                                        void* vpages, const int32_t* block_table, const int32_t* cache_seqlens,
                                        void* o, float* lse, int causal, int num_splits, int B, int Nq, int Hq,
                                        int Hkv, int page_size, int pages_per_seq, int num_pages, int d, float scale,
                                        void* workspace, size_t workspace_bytes, void* stream);

/* ---- FP8 (e4m3) forward (FlashAttention: Part 2, section 1.6 "FA3 FP8":
 * block quantisation plus incoherent processing; the computation is still
 * exact attention, its arithmetic FP8). Quantise Q, K and V with
 * fa_quantize_fp8, then run fa_fwd_fp8 on the codes. */

/* Rows of a quantised head: n rounded up to a multiple of 64 (0 for n <= 0
 * or n > 2^31 - 1024). */
int fa_fp8_padded_rows(int n);

/* Block quantisation of a bf16 tensor x (B, N, H, d) to e4m3 codes, one
 * scale per 64-row block of each (batch, head). Rows of a block are
 * optionally rotated first by R = H_d diag(signs) / sqrt(d) (H_d the
 * Sylvester Hadamard matrix; signs: d device floats, each +1 or -1, or NULL
 * for no rotation). Rotate Q and K with the same signs and leave V
 * unrotated: Q K^T, and so the attention, is unchanged.
 * A block's scale is 2^e with e the smallest integer such that the block's
 * largest |value| <= 448 * 2^e (e = 0 for an all-zero block, clamped to
 * [-127, 127]); codes are round-to-nearest-even e4m3 (OCP E4M3: bias 7,
 * largest finite 448) of value * 2^-e. Outputs, with Np =
 * fa_fp8_padded_rows(N) and padding rows written as code 0:
 *   codes  : (B, H, Np, d) bytes, or (B, H, d, Np) when transpose = 1 (the
 *            layout fa_fwd_fp8 takes for V)
 *   scales : (B, H, Np / 64) bytes, E8M0: 127 + e
 * Inputs must be finite. d in {64, 128, 256}; B, H <= 65535.
 * FA_ERR_INVALID_ARG for negative sizes, transpose not 0/1 or a NULL
 * buffer; B == 0 or N == 0 is a no-op. */
fa_status_t fa_quantize_fp8(const void* x, const float* signs, void* codes, uint8_t* scales, int transpose,
                            int B, int N, int H, int d, void* stream);

/* Attention on FP8 operands: O = softmax(scale * Qh Kh^T) Vh with Qh, Kh, Vh
 * the dequantised codes (per-block scales applied exactly by the MFMA's
 * E8M0 scale operands). Both products run on the FP8 MFMA: the
 * probabilities are quantised as e4m3 of 2^(t - m + 6), t = scale log2(e)
 * (Qh Kh^T) and m an integer reference >= max t - 2, so every probability
 * code is that of the row's own maximum up to a power of two; the
 * denominator sums the unquantised probabilities.
 *   q8 (B, Hq, Nqp, d), k8 (B, Hkv, Nkp, d), vt8 (B, Hkv, d, Nkp) codes and
 *   their scales, as fa_quantize_fp8 writes them (Nqp, Nkp = padded Nq, Nk)
 *   o   : (B, Nq, Hq, d) bfloat16     lse : (B, Hq, Nq) float32 or NULL
 * causal is top-left (key j visible to query i iff j <= i). A row that sees
 * no key gets o = 0, lse = -inf. d in {64, 128, 256}; Nk <= 65536; B, Hq <= 65535;
 * Hq % Hkv == 0.
 * Error codes as fa_fwd. */
fa_status_t fa_fwd_fp8(const void* q8, const uint8_t* q_scales, const void* k8, const uint8_t* k_scales,
                       const void* vt8, const uint8_t* v_scales, void* o, float* lse,
                       int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale, void* stream);

/* Bytes of device workspace fa_bwd needs: two float32 values (D_i and
 * -LSE_i / scale) per (batch, query head, query), the query count rounded
 * up to a multiple of 32. 0 when B, Hq or Nq is not positive. */
size_t fa_bwd_workspace_size(int B, int Hq, int Nq);

/* Attention backward: dQ, dK, dV of O = softmax(scale * Q K^T) V for an
 * upstream gradient dO, from the forward's O and LSE (the score tiles are
 * recomputed from the saved row log-sum-exp, never stored: FlashAttention:
 * Part 2, section 1.3; the pyshine.com code tour's "recompute then
 * accumulate" backward). With P = exp(scale S - LSE):
 *     dV = P^T dO, dP = dO V^T, dS = P o (dP - D), D_i = sum_d dO_id O_id,
 *     dQ = scale dS K, dK = scale dS^T Q;
 * a key/value head's gradients are summed over its group of query heads.
 *
 *   q, o, dout, dq : (B, Nq, Hq, d) bfloat16      lse : (B, Hq, Nq) float32,
 *   k, v, dk, dv   : (B, Nk, Hkv, d) bfloat16     as fa_fwd writes it
 *   causal, scale  : as fa_fwd (top-left mask, finite positive scale)
 *   workspace      : device memory of at least fa_bwd_workspace_size(B, Hq, Nq)
 *                    bytes (may be NULL when that is 0); contents need no
 *                    initialisation and are overwritten.
 *
 * dq, dk, dv are fully overwritten (rows with no visible key get zeros);
 * nothing is accumulated into them, and no atomics are used, so results
 * are bitwise reproducible.
 * Returns FA_ERR_INVALID_ARG (as fa_fwd), FA_ERR_UNSUPPORTED for d other
 * than 64 or 128 or for grids, workspaces or row counts (B * Nq, B * Nk)
 * beyond 32-bit indexing,
 * FA_ERR_WORKSPACE when the workspace is missing or too small. */
fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv,
                   int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                   void* workspace, size_t workspace_bytes, void* stream);

/* fa_bwd under the visibility rule of fa_fwd_window (bottom-right aligned:
 * key j is visible to query i iff i + off - window_left <= j <= i + off +
 * window_right, off = Nk - Nq, a negative bound unlimited; causal is
 * (-1, 0)). o and lse are those fa_fwd_window returned for the same window.
 * Everything else (layouts, workspace, errors) is as fa_bwd. A query that
 * sees no key gets dq = 0; a key no query sees gets dk = dv = 0. */
fa_status_t fa_bwd_window(const void* q, const void* k, const void* v, const void* o, const float* lse,
                          const void* dout, void* dq, void* dk, void* dv,
                          int B, int Hq, int Hkv, int Nq, int Nk, int d, int window_left, int window_right,
                          float scale, void* workspace, size_t workspace_bytes, void* stream);

/* fa_bwd_window over a packed variable-length batch, the layouts of
 * fa_fwd_varlen: q, o, dout, dq (total_q, Hq, d); k, v, dk, dv (total_k,
 * Hkv, d); lse (Hq, total_q); cu_seqlens_q / cu_seqlens_k (B + 1,) int32 on
 * the device. max_seqlen_q / max_seqlen_k bound the sequence lengths (longer
 * sequences are cut there); the workspace is fa_bwd_workspace_size(B, Hq,
 * max_seqlen_q) bytes. Offsets are clamped into the arrays. */
fa_status_t fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                          const void* dout, void* dq, void* dk, void* dv,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                          int B, int Hq, int Hkv, int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
                          int d, int window_left, int window_right, float scale,
                          void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
