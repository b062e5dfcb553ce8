/*
 * msa.h -- C ABI of libmsa.so: the MiniMax Sparse Attention (MSA) forward pass
 * on AMD Instinct MI355X (gfx950).
 *
 * Pages defining the operations (cited by title and section):
 *   [M3-20x] "MiniMax M3 算力省 20 倍" (mizuki-eaf.pages.dev): §二 MSA -- Index
 *            Branch (one index-query head per GQA group, one index-key head shared
 *            by all groups, dot-product scores over the causal window, max-pooled
 *            into blocks, top-k blocks chosen per group, the query's own block always
 *            chosen) and Main Branch (standard softmax attention over the tokens of
 *            the chosen blocks only; B = 128, k = 16, a 2048-token budget);
 *            §三 item 4 (the local block keeps one of the slots);
 *            §四 Kernel (exp-free top-k; KV-outer iteration that gathers the queries
 *            of each KV block; pre-scheduled chunking of hot tiles; two-phase combine
 *            without atomics).
 *   [SERVE]  "MiniMax M3 的采用瓶颈，会卡在 serving 生态" (the-context.pages.dev):
 *            §发生了什么 / §对建设者的影响 -- a block-selection step plus a dedicated
 *            sparse kernel, a KV-block-major layout, index scoring, paged decode.
 *
 * Conventions shared by every entry point
 *   - Tensors are DEVICE pointers owned by the caller, row-major, token-major.
 *     bf16 values are passed as their uint16_t bit patterns.
 *   - Shapes: L tokens, H query heads, G KV heads (= index groups; H % G == 0,
 *     query head h belongs to group h / (H/G)), d head dim, dI index dim, B block
 *     size, k slots per (query, group) INCLUDING the query's own block.
 *   - Token i sees keys t <= i.  Block of token i: b(i) = i / B.
 *   - scale: softmax scale applied to q.k; pass a value <= 0 for 1/sqrt(d).
 *   - ws / ws_bytes: caller-owned device workspace, 256-byte aligned.  The size
 *     returned by the matching *_workspace_size() call is the preferred one (largest
 *     query chunk).  msa_select_blocks, msa_sparse_attn and msa_prefill also accept
 *     less: they then process the queries in smaller chunks (multiples of 128
 *     queries) and fail with MSA_ERR_WORKSPACE_TOO_SMALL only when not even one
 *     128-query chunk fits.  msa_decode needs its full workspace size.
 *     The library never allocates device memory and never synchronises; all work is
 *     enqueued on `stream` (a hipStream_t passed as void*, NULL = default stream)
 *     as kernel launches only (no memset or copy), so a call may be captured into a
 *     HIP graph and replayed; a replay reads the buffers as they are at replay time
 *     (for msa_prefill_varlen the host offsets are read at capture).
 *   - Return value: an msa_status.  Every argument is validated BEFORE anything is
 *     launched; on an error nothing is launched and no output is written.  Faults
 *     inside kernels surface at the caller's next synchronisation of `stream`.
 *   - The compute entry points are stateless and thread-safe; calls on one stream
 *     are ordered.  (The optional timing facility at the end is process-wide.)
 *   - Supported on the GPU: B = 128; d in {64, 128}; dI in {32, 64, 128};
 *     H/G in {1, 2, 4, 8, 16, 32}; G * dI <= 512; 1 <= k <= 32;
 *     0 <= L <= 1048576 for msa_prefill / msa_sparse_attn (any L for
 *     msa_select_blocks; any Lmax for msa_decode).
 *     Anything else returns MSA_ERR_UNSUPPORTED.
 *   - Rows are independent: results do not depend on how the library splits the
 *     queries into chunks, and repeated calls give bitwise-identical outputs.
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define MSA_API __attribute__((visibility("default")))
#else
#define MSA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum msa_status {
    MSA_OK = 0,
    MSA_ERR_INVALID_ARG = 1,          /* null pointer, negative size, H % G != 0, k < 1 */
    MSA_ERR_UNSUPPORTED = 2,          /* shape outside the supported set above */
    MSA_ERR_WORKSPACE_TOO_SMALL = 3,  /* ws_bytes below the required size, or ws misaligned */
    MSA_ERR_HIP = 4                   /* a HIP launch reported an error */
} msa_status;

/* Human-readable name of a status code (static string, never NULL). */
MSA_API const char *msa_status_string(int status);

/* ---------------------------------------------------------------------------
 * Index branch [M3-20x §二 Index Branch; §三 item 4; §四 exp-free TopK].
 * For every token i and group g: score every key t <= i as
 * s = sum_c idx_q[i,g,c] * idx_k[t,c], max-pool the scores of each B-token block,
 * and select the query's own block b(i) plus the k-1 blocks b < b(i) with the
 * largest block scores (raw scores, no exp; equal scores -> smaller id first).
 *   idx_q     [L, G, dI] bf16      index-query head of each group
 *   idx_k     [L, dI]    bf16      index-key head shared by all groups
 *   block_ids [L, G, k]  int32 OUT selected block ids, ascending, padded with -1
 *                                  when b(i) + 1 < k (fewer blocks exist)
 * ------------------------------------------------------------------------- */
MSA_API size_t msa_select_blocks_workspace_size(int64_t L, int G, int dI, int B, int k);
MSA_API int msa_select_blocks(const uint16_t *idx_q, const uint16_t *idx_k, int64_t L, int G, int dI,
                      int B, int k, int32_t *block_ids, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Main branch [M3-20x §二 Main Branch; §四 KV-outer attention, hot-tile chunking,
 * two-phase combine].  Exact softmax attention of each query head over the tokens
 * t <= i of the blocks listed for its group (entries < 0 are ignored):
 *   out[i,h] = sum_t softmax_t(scale * q[i,h].k[t,g]) v[t,g],  g = h / (H/G).
 *   q         [L, H, d]  bf16
 *   k, v      [L, G, d]  bf16
 *   block_ids [L, G, kslots] int32  each valid id must lie in [0, b(i)] and be
 *                                   unique within its row; the own block b(i) must
 *                                   be present (it is what msa_select_blocks emits).
 *                                   Rows violating this give unspecified values in
 *                                   their own output rows only.
 *   out       [L, H, d]  bf16 OUT
 * Inputs must be finite.  The queries of one block attend that block's keys as one
 * tile with the keys past each query masked to weight 0, so a non-finite V value at
 * token t would also reach the outputs of the queries of t's block that precede t.
 * ------------------------------------------------------------------------- */
MSA_API size_t msa_sparse_attn_workspace_size(int64_t L, int H, int G, int d, int B, int kslots);
MSA_API int msa_sparse_attn(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                    const int32_t *block_ids, int64_t L, int H, int G, int d, int B, int kslots,
                    float scale, uint16_t *out, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Whole prefill: msa_select_blocks followed by msa_sparse_attn on the same rows.
 * block_ids_out [L, G, k] may be NULL (the ids then live only in the workspace).
 * A sequence of at most kslots blocks (L <= kslots * B) keeps every causal block of
 * every row whatever the scores [M3-20x §二 Index Branch, §三 item 4], so its
 * selection is blocks 0 .. b(i) (ascending, then -1) and its main branch is dense
 * causal GQA attention: such a call runs one kernel ("kd_dense") that attends each
 * query over its causal blocks with an online softmax and writes those ids; the
 * index inputs are not read.  The outputs equal the general path's up to fp32
 * rounding order (the ids are the same).
 * ------------------------------------------------------------------------- */
MSA_API size_t msa_prefill_workspace_size(int64_t L, int H, int G, int d, int dI, int B, int k);
MSA_API int msa_prefill(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *idx_q,
                const uint16_t *idx_k, int64_t L, int H, int G, int d, int dI, int B, int kslots,
                float scale, uint16_t *out, int32_t *block_ids_out, void *ws, size_t ws_bytes,
                void *stream);

/* ---------------------------------------------------------------------------
 * Varlen / prefix prefill [M3-20x §二 (causal window per sequence); SERVE
 * 对建设者的影响: cache management around the sparse kernel].  A batch of nseq
 * independent causal sequences, packed token-major.  Sequence s holds
 * Ls = cu_kv[s+1] - cu_kv[s] tokens, of which the last Cs = cu_q[s+1] - cu_q[s]
 * are new: its first Ps = Ls - Cs tokens are an existing prefix whose K, V and
 * index keys are in the cache.  The new tokens are prefilled exactly as rows
 * Ps .. Ls-1 of msa_prefill over the whole sequence (bitwise the same results).
 *   q     [sum Cs, H, d]   idx_q [sum Cs, G, dI]   (new tokens only)
 *   k, v  [sum Ls, G, d]   idx_k [sum Ls, dI]      (prefix + new tokens)
 *   out   [sum Cs, H, d] OUT;  block_ids_out [sum Cs, G, k] OUT or NULL
 *   cu_q, cu_kv: HOST int64 arrays of nseq + 1 offsets (non-decreasing).
 * Requires Ps % 128 == 0 (whole prefix blocks) and Ls <= 1048576 for every
 * sequence with new tokens, else MSA_ERR_UNSUPPORTED; Cs > Ls or a negative
 * offset is MSA_ERR_INVALID_ARG.
 * Consecutive sequences of at most 8192 new tokens are prefilled together in
 * batches (up to 128 sequences, 131072 new tokens and 8192 KV blocks per batch,
 * as far as the workspace holds them), every kernel of the path launched once per
 * batch.  Longer sequences,
 * and any that no batch can take, run alone in query chunks like msa_prefill.
 * Sequences of at most kslots blocks run apart, all in one "kd_dense" launch (see
 * msa_prefill), and end the open batch.
 * The results do not depend on the batching.
 * Workspace: msa_prefill_varlen_workspace_size gives the size at which every
 * batch is formed; the minimum is one 128-query chunk of
 * msa_prefill_workspace_size(max Ls, ...) (then every sequence runs alone).
 * ------------------------------------------------------------------------- */
MSA_API size_t msa_prefill_varlen_workspace_size(const int64_t *cu_q, const int64_t *cu_kv,
                                                 int nseq, int H, int G, int d, int dI, int B,
                                                 int k);
MSA_API int msa_prefill_varlen(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               const uint16_t *idx_q, const uint16_t *idx_k, const int64_t *cu_q,
                               const int64_t *cu_kv, int nseq, int H, int G, int d, int dI, int B,
                               int kslots, float scale, uint16_t *out, int32_t *block_ids_out,
                               void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Decode [M3-20x §二, §四 decode result; SERVE: paged MSA decode].  N independent
 * sequences; sequence n holds seq_len[n] cached tokens and its query is the LAST
 * cached token, position p = seq_len[n] - 1 (the new token is already inserted).
 * The query scores every block of its own cache, selects as in the index branch,
 * and attends over the selected blocks (exact softmax over their tokens, the slots
 * merged by the log-sum-exp rule).
 *   q           [N, H, d]         bf16   query of each sequence
 *   idx_q       [N, G, dI]        bf16
 *   k_cache     [N, Lmax, G, d]   bf16   contiguous per-sequence caches
 *   v_cache     [N, Lmax, G, d]   bf16
 *   idx_k_cache [N, Lmax, dI]     bf16
 *   seq_len     [N] int32 DEVICE  1 <= seq_len[n] <= Lmax.  A sequence outside that
 *                                 range gets ids all -1 and a zero output row;
 *                                 nothing outside its cache is read.  Rows at and
 *                                 past seq_len[n] of its caches are never read (they
 *                                 may hold anything, non-finite values included).
 *   out         [N, H, d]         bf16 OUT
 *   block_ids_out [N, G, k] int32 OUT, may be NULL
 * ------------------------------------------------------------------------- */
MSA_API size_t msa_decode_workspace_size(int N, int64_t Lmax, int H, int G, int d, int dI, int B, int k);
MSA_API int msa_decode(const uint16_t *q, const uint16_t *idx_q, const uint16_t *k_cache,
               const uint16_t *v_cache, const uint16_t *idx_k_cache, const int32_t *seq_len,
               int N, int64_t Lmax, int H, int G, int d, int dI, int B, int kslots, float scale,
               uint16_t *out, int32_t *block_ids_out, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Decode without a caller workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  The arguments, kernels and results (bitwise) of msa_decode, minus
 * ws / ws_bytes: the workspace is a device array of the library,
 * MSA_STATIC_SCRATCH_BYTES on each GPU the library runs on, held until the process
 * ends.  A shape whose msa_decode_workspace_size() exceeds MSA_STATIC_SCRATCH_BYTES
 * returns MSA_ERR_WORKSPACE_TOO_SMALL (checked before any HIP call); `stream` must
 * belong to the current device (else MSA_ERR_INVALID_ARG).  Calls no allocating
 * routine.  Every call on one GPU shares that GPU's array and leaves its contents
 * there: calls that may overlap on one GPU (other streams, other host threads) race
 * and must be ordered by the caller.
 * ------------------------------------------------------------------------- */
#define MSA_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
MSA_API int msa_decode_static(const uint16_t *q, const uint16_t *idx_q, const uint16_t *k_cache,
                              const uint16_t *v_cache, const uint16_t *idx_k_cache,
                              const int32_t *seq_len, int N, int64_t Lmax, int H, int G, int d,
                              int dI, int B, int kslots, float scale, uint16_t *out,
                              int32_t *block_ids_out, void *stream);

/* ---------------------------------------------------------------------------
 * Paged decode [SERVE: paged MSA decode; M3-20x §二 (B = 128-token blocks)].
 * The same computation as msa_decode, with the caches held in fixed 128-token
 * pages so that every MSA block is exactly one page: logical token t of sequence
 * n is row t % 128 of page block_table[n * max_blocks + t / 128].  Pages may be
 * shared between sequences (a common prefix); they are only read.
 *   q            [N, H, d]                bf16
 *   idx_q        [N, G, dI]               bf16
 *   k_pages      [num_pages, 128, G, d]   bf16
 *   v_pages      [num_pages, 128, G, d]   bf16
 *   idx_k_pages  [num_pages, 128, dI]     bf16
 *   block_table  [N, max_blocks] int32 DEVICE  page of each logical block; only
 *                                 the entries of blocks 0 .. (seq_len[n]-1)/128 are
 *                                 read, the rest may hold anything
 *   seq_len      [N] int32 DEVICE  1 <= seq_len[n] <= max_blocks * 128
 *   out          [N, H, d] bf16 OUT;  block_ids_out [N, G, k] int32 OUT or NULL
 * A sequence whose length is out of range, or one of whose needed table entries
 * lies outside [0, num_pages), gets ids all -1 and a zero output row, and none of
 * its pages is read (the table is checked on the device before any page read).
 * The rows of a sequence's last page at and past its length are never read.
 * Requires B == 128 and max_blocks * 128 <= INT32_MAX; other limits as msa_decode.
 * ------------------------------------------------------------------------- */
MSA_API size_t msa_decode_paged_workspace_size(int N, int max_blocks, int H, int G, int d, int dI,
                                               int B, int k);
MSA_API int msa_decode_paged(const uint16_t *q, const uint16_t *idx_q, const uint16_t *k_pages,
                             const uint16_t *v_pages, const uint16_t *idx_k_pages,
                             int64_t num_pages, const int32_t *block_table, int max_blocks,
                             const int32_t *seq_len, int N, int H, int G, int d, int dI, int B,
                             int kslots, float scale, uint16_t *out, int32_t *block_ids_out,
                             void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Decode with an FP8 index-key cache [M3.1 kernel list: the index QK of decode
 * runs on FP8 keys; SERVE: index scoring].  Identical to msa_decode except that
 * the index keys are stored in the OCP 8-bit floating point E4M3 encoding with one
 * fp32 scale per token, halving the bytes of the decode index stream:
 *   idx_k_e4m3  [N, Lmax, dI] uint8 DEVICE  E4M3 bytes
 *   idx_k_scale [N, Lmax]     fp32 DEVICE   > 0
 * The index key of token t is idx_k_scale[t] * e4m3(idx_k_e4m3[t, :]) and its
 * score is idx_k_scale[t] * (idx_q . e4m3(...)), the dot product accumulated in
 * fp32 from exact bf16 x E4M3 products.  Selection and attention then proceed as
 * in msa_decode (K/V caches stay bf16).  Workspace: msa_decode_workspace_size.
 * ------------------------------------------------------------------------- */
MSA_API int msa_decode_fp8idx(const uint16_t *q, const uint16_t *idx_q, const uint16_t *k_cache,
                              const uint16_t *v_cache, const uint8_t *idx_k_e4m3,
                              const float *idx_k_scale, const int32_t *seq_len, int N,
                              int64_t Lmax, int H, int G, int d, int dI, int B, int kslots,
                              float scale, uint16_t *out, int32_t *block_ids_out, void *ws,
                              size_t ws_bytes, void *stream);

/* Paged decode with an E4M3 index-key cache: the caches of msa_decode_paged, with
 * the index keys in pages of E4M3 bytes and their per-token scales,
 *   idx_k_pages_e4m3   [num_pages, 128, dI] uint8
 *   idx_k_scale_pages  [num_pages, 128]     fp32 > 0
 * addressed through the same block table (the index key of logical token t of
 * sequence n is scale * e4m3(bytes) of row t % 128 of page block_table[n][t/128]).
 * Scores, selection, attention, the page check and the error behaviour are those
 * of msa_decode_fp8idx and msa_decode_paged.  Workspace:
 * msa_decode_paged_workspace_size. */
MSA_API int msa_decode_paged_fp8idx(const uint16_t *q, const uint16_t *idx_q,
                                    const uint16_t *k_pages, const uint16_t *v_pages,
                                    const uint8_t *idx_k_pages_e4m3, const float *idx_k_scale_pages,
                                    int64_t num_pages, const int32_t *block_table, int max_blocks,
                                    const int32_t *seq_len, int N, int H, int G, int d, int dI,
                                    int B, int kslots, float scale, uint16_t *out,
                                    int32_t *block_ids_out, void *ws, size_t ws_bytes,
                                    void *stream);

/* Index-key cache writer for msa_decode_fp8idx: rows [rows, dI] bf16 (dI in
 * {32, 64, 128}) -> E4M3 bytes [rows, dI] and scales [rows].  Per row: scale = 2^e
 * with e the smallest integer such that max|x| <= 448 * 2^e (1 for an all-zero
 * row); byte = the E4M3 value nearest to x / scale, ties to the even code, sign of
 * x kept.  Power-of-two scales make every dequantised key exact in bf16.  Input
 * values must be finite.  Stream-ordered, no workspace. */
MSA_API int msa_quantize_idx_k_e4m3(const uint16_t *idx_k, int64_t rows, int dI,
                                    uint8_t *idx_k_e4m3, float *idx_k_scale, void *stream);

/* ---------------------------------------------------------------------------
 * Optional per-kernel timing (measurement support, process-wide, not
 * thread-safe).  While enabled, every kernel stage the entry points above enqueue
 * is bracketed by a pair of hipEvents recorded on the caller's stream; stages are
 * named "k1_index_pool", "k2_select", "k3_schedule" (its four small kernels as
 * one), "k4_kv_outer", "k5_combine", "k1d_index_pool", "k4d_split", "page_check",
 * "k1d_index_pool_fp8", "quantize_e4m3", "kd_dense" (the main branch of sequences
 * of at most kslots blocks, as dense causal attention), "k4d_online" (decode's attention for up to
 * 16 heads per group: one launch, each slot folded into a running log-sum-exp merge,
 * used from 256 (sequence, group) pairs on), "k4d_parts" (the same for fewer pairs:
 * each pair's slots in parts, then "k5_combine" merges the parts), "k4d_merge"
 * (32 heads per group: the slots' combine in the same launch where their partials
 * fit in LDS: k <= 16 and k * (H/G) * d * 2 bytes <= 96 KiB; else "k4d_split" and
 * "k5_combine"), "k12_index_select" (index
 * scores, max-pool and selection in one launch, with no block scores in memory:
 * msa_select_blocks and msa_prefill use it for the query chunks whose shortest row
 * has at least as many competitor blocks as the chunk has query blocks, k <= 17;
 * the other chunks run k1_index_pool + k2_select; the ids are the same).
 *   msa_timing_enable(max_launches): start recording (events for up to
 *       max_launches stages are created up front; further stages are not timed).
 *   msa_timing_collect(out, max_entries, n_out): waits for the recorded events
 *       (this call synchronises), sums the elapsed times per stage name into `out`
 *       and clears the record; recording stays enabled.
 *   msa_timing_disable(): stop recording and release the events.
 * ------------------------------------------------------------------------- */
typedef struct msa_kernel_time {
    char name[32];
    int launches;
    double total_ms;
} msa_kernel_time;

MSA_API int msa_timing_enable(int max_launches);
MSA_API int msa_timing_collect(msa_kernel_time *out, int max_entries, int *n_out);
MSA_API void msa_timing_disable(void);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H_ */
