// msa_launch.h -- internal launchers of the MSA kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

constexpr int kBlock = 128;   // tokens per MSA block (B)

// Key blocks scored by one K1 work-group item, and blocks buffered before a flush.
constexpr int kK1KeyChunk = 32;
// A single-range K1 launch with fewer than kK1MinWorkGroups work-groups halves its
// key chunk, down to kK1MinKeyChunk blocks.
constexpr int kK1MinKeyChunk = 8;
constexpr int kK1MinWorkGroups = 512;
// Queries per K4 work item (one staged K/V block serves up to this many queries).
constexpr int kK4Queries = 128;
// Consecutive K4 work items that one XCD takes before the next XCD's turn.
constexpr int kK4Run = 16;
// Queries whose entries one K3 work-group sorts (count and scatter passes); small
// chunks use fewer, halving from kK3Queries while the passes would have fewer than
// kK3TargetGroups work-groups, down to kK3MinQueries.
constexpr int kK3Queries = 2048;
constexpr int kK3MinQueries = 64;
constexpr int kK3TargetGroups = 256;
// Chunks of at most this many queries skip K4's run-order sort (their q rows are
// few; three launches saved): K4 then runs the items in list order.
constexpr int64_t kK3NoOrderQueries = 4096;
// K4 work items that one work-group of K3's tile-ordering passes handles, and the
// most (group, query window) buckets those passes sort the items into.
constexpr int kK3Tiles = 4096;
constexpr int kK3Buckets = 2048;

// Round n up to a multiple of m.
inline int64_t round_up(int64_t n, int64_t m) { return (n + m - 1) / m * m; }

// Number of K1 work items for the query blocks [qb0, qb1), key chunks of kc blocks.
int64_t k1_num_items(int qb0, int qb1, int kc = kK1KeyChunk);

// K1: block scores S[(i-q0)*G + g][b] for queries i in [q0, qend), blocks b < b(i).
hipError_t launch_k1_index_pool(const uint16_t *iq, const uint16_t *ik, float *S, int64_t L,
                                int64_t q0, int64_t qend, int G, int dI, int nbp,
                                hipStream_t s);

// K12: K1 and K2 in one kernel -- ids [(i-q0)*G + g][k] of queries [q0, qend) (q0 a
// multiple of 128) without block scores in memory; cand holds k12_cand_entries(C, G)
// 8-byte candidate entries for a chunk of C queries.  Only where k12_supported.
bool k12_supported(int G, int dI, int k);
int64_t k12_cand_entries(int64_t C, int G);
// K12 work-groups of a chunk of C queries (one per 64 queries at G = 4, each over
// all key blocks of its rows), and the fewest worth a K12 launch: four per CU, so
// that the long-lived work-groups fill the part.
int64_t k12_num_workgroups(int64_t C, int G);
constexpr int64_t kK12MinWorkgroups = 1024;
hipError_t launch_k12_index_select(const uint16_t *iq, const uint16_t *ik, int32_t *ids,
                                   void *cand, int64_t q0, int64_t qend, int G, int dI, int k,
                                   hipStream_t s);

// K1d: decode block scores S[n*G + g][b] for blocks b < b(seq_len[n]-1).
// table == nullptr: contiguous cache ikc [N, Lmax, dI]; otherwise a paged cache
// [pages, 128, dI] with block b of sequence n in page table[n * maxb + b].
hipError_t launch_k1d_index_pool(const uint16_t *iq, const uint16_t *ikc, const int32_t *seq_len,
                                 const int32_t *table, int maxb, float *S, int N, int64_t Lmax,
                                 int G, int dI, int nbp, hipStream_t s);

// K1d over an FP8 (E4M3) index-key cache ik8 [N, Lmax, dI] with per-token fp32
// scales ksc [N, Lmax]: score = ksc[t] * (iq . e4m3(ik8[t])).
// table != nullptr: paged caches ik8 [pages, 128, dI], ksc [pages, 128] (as K1d).
hipError_t launch_k1d_index_pool_fp8(const uint16_t *iq, const uint8_t *ik8, const float *ksc,
                                     const int32_t *seq_len, const int32_t *table, int maxb,
                                     float *S, int N, int64_t Lmax, int G, int dI, int nbp,
                                     hipStream_t s);

// Index-key cache writer: rows [rows, dI] bf16 -> E4M3 bytes + power-of-two scales.
hipError_t launch_quant_e4m3(const uint16_t *x, int64_t rows, int dI, uint8_t *out, float *scale,
                             hipStream_t s);

// K2: exp-free selection.  Row r of S belongs to query position
// q0 + r / G (prefill, seq_len == nullptr) or seq_len[r / G] - 1 (decode).
hipError_t launch_k2_select(const float *S, int nbp, int64_t nrows, int G, int k, int64_t q0,
                            const int32_t *seq_len, int64_t Lmax, int32_t *ids, hipStream_t s);

// A packed batch of sequences run as one set of launches (varlen prefill).  Row r
// of the batch is a new token of one sequence; the batch's KV blocks are numbered
// sequence after sequence ("global" blocks).  Built on the device by
// launch_batch_setup; a BatchMap of null pointers means a single sequence.
struct BatchMap {
    const int32_t *row_len = nullptr;    // [rows] position of the row's token + 1
    const int32_t *row_kvpos = nullptr;  // [rows] absolute index of that token in k / v
    const int32_t *row_blk0 = nullptr;   // [rows] global number of its sequence's block 0
    const int32_t *blk_tok0 = nullptr;   // [blocks] absolute first token of a global block
    const int32_t *blk_rows = nullptr;   // [blocks] tokens in the block (<= 128)
};
constexpr int kBatchMaxSeq = 128;        // sequences per batched launch set
constexpr int kBatchMaxBlocks = 8192;    // global blocks per batched launch set
// Host description of a batch, passed by value to the setup kernel (2.6 KB), which
// also copies it to device memory for K1.
struct BatchTable {
    int n = 0, rows = 0, blocks = 0;
    int q_off[kBatchMaxSeq + 1];     // first row of each sequence; q_off[n] = rows
    int blk_off[kBatchMaxSeq + 1];   // first global block; blk_off[n] = blocks
    int k1_off[kBatchMaxSeq + 1];    // first K1 work-group of each sequence
    int kv_off[kBatchMaxSeq];        // absolute first K/V token of each sequence
    int kv_len[kBatchMaxSeq];        // its tokens, cached prefix + new
};
// Dense main branch of sequences of at most k blocks (their selection is every
// causal block): up to kBatchMaxSeq sequences per launch.  Member m's new queries are
// positions prefix[m] .. len[m]-1 of its sequence (prefix a multiple of 128), at rows
// q_row0[m] .. of q / out / ids; its keys are rows kv_row0[m] .. + len[m]-1 of k / v.
// tile_off: prefix sum of the work-groups' query tiles (dense_tile_queries queries
// each) over the members.
struct DenseTable {
    int n = 0;
    int tile_off[kBatchMaxSeq + 1];
    int q_row0[kBatchMaxSeq];
    int kv_row0[kBatchMaxSeq];
    int len[kBatchMaxSeq];
    int prefix[kBatchMaxSeq];
};
int dense_tile_queries(int H, int G);
// out [rows, H, d] and, when ids is not null, ids [rows, G, k] (0 .. b(i), then -1).
hipError_t launch_kd_dense(const uint16_t *q, const uint16_t *kx, const uint16_t *vx,
                           uint16_t *out, int32_t *ids, const DenseTable &t, int H, int G, int d,
                           int k, float scale, hipStream_t s);
hipError_t launch_batch_setup(const BatchTable &t, BatchTable *dtab, int32_t *row_len,
                              int32_t *row_kvpos, int32_t *row_blk0, int32_t *blk_tok0,
                              int32_t *blk_rows, hipStream_t s);
// K1 over a batch: the work-groups of every sequence in one launch.  iq holds the
// batch's rows, ik all tokens; S rows follow the batch rows.
hipError_t launch_k1_index_pool_batch(const uint16_t *iq, const uint16_t *ik, float *S,
                                      const BatchTable &t, const BatchTable *dtab, int G, int dI,
                                      int nbp, hipStream_t s);
// K1 work-groups of the queries [q0, qend) of one sequence.
int64_t k1_num_workgroups(int64_t q0, int64_t qend, int G);

// K3: invert query-major ids of queries [q0, q0 + C) into per-(g, block) lists.
// With a batch map, ids are local to each row's sequence and lists are per global
// block; an id is scheduled when 0 <= id <= b(row) (batch) or 0 <= id < nb.
struct SchedBuffers {
    int *counts;     // [nlists]
    int *offs;       // [nlists + 1]
    int *toff;       // [nlists + 1] prefix sum of ceil(count / kK4Queries)
    int *wcnt;       // [G * k3_num_groups(C, G) * nb] per-work-group counts / prefixes
    int *total;      // [1] number of K4 work items
    int *items;      // [k4_max_items] list index of every K4 work item
    int *order;      // [k4_max_items] K4's run order: work items by (group, first query)
    int *tcnt;       // [k3_tile_groups(k4_max_items) * kK3Buckets] bucket counts / bases
    uint32_t *list;  // [C * G * k] entries (i - q0) << 5 | slot
};
hipError_t launch_k3_schedule(const int32_t *ids, int64_t C, int G, int k, int nb,
                              const SchedBuffers &sb, const BatchMap &bm, hipStream_t s);
int64_t k4_max_items(int64_t C, int G, int k, int nb);
int k3_queries_per_group(int64_t C, int G);
int k3_num_groups(int64_t C, int G);
int64_t k3_tile_groups(int64_t max_items);

// K4: KV-outer attention over the scheduled lists -> partials per (query, head,
// slot): po holds one block of R*d bf16 per (query i, group g, slot), at
// ((i*G + g)*k + slot)*R*d, chunk-major: the 8 values of chunk c (d = 8c .. 8c+7)
// of head h % R at (c*R + h % R)*8 (o NOT normalised); at pml = plse viewed as
// float pairs, [((i*G + g)*k + slot)*R + h % R] = (row maximum of the scaled scores
// in log2 units, row sum of 2^(score - maximum)); plse holds 2*C*H*k floats.
// With a batch map, q holds the batch's rows (q0 = 0) and the lists are per global
// block.
hipError_t launch_k4_kv_outer(const uint16_t *q, const uint16_t *kx, const uint16_t *vx,
                              const SchedBuffers &sb, int nb, int64_t L, int64_t q0, int64_t C,
                              int H, int G, int d, int k, float scale, uint16_t *po, float *plse,
                              const BatchMap &bm, hipStream_t s);

// K4d for R = H/G = 32: decode split over slots -> partials per (sequence, head, slot): rows
// po [(n*H + h)*k + slot][d] (o normalised) and plse [((n*G + g)*k + slot)*R + h % R]
// (log2-sum-exp).  Cache
// addressing as in K1d (kc, vc [N, Lmax, G, d] or pages [pages, 128, G, d]).
hipError_t launch_k4d_split(const uint16_t *q, const uint16_t *kc, const uint16_t *vc,
                            const int32_t *ids, const int32_t *seq_len, const int32_t *table,
                            int maxb, int N, int64_t Lmax, int H, int G, int d, int k, float scale,
                            uint16_t *po, float *plse, hipStream_t s);

// K4d and K5 in one launch for R = 32: one work-group per (sequence, group) attends
// its valid slots in order and merges them in LDS; out [N, H, d] bitwise as K4d + K5.
// Only where k4d_merge_supported(d, H/G, k) (the partials of k slots fit in LDS).
bool k4d_merge_supported(int d, int R, int k);
hipError_t launch_k4d_merge(const uint16_t *q, const uint16_t *kc, const uint16_t *vc,
                            const int32_t *ids, const int32_t *seq_len, const int32_t *table,
                            int maxb, int N, int64_t Lmax, int H, int G, int d, int k, float scale,
                            uint16_t *out, hipStream_t s);

// K4d with an online merge, one launch: one work-group per (sequence, group) attends
// its valid slots in order (two K/V buffers in LDS) and folds each slot into a running
// log-sum-exp merge held in registers; out [N, H, d].  Any k; R = H/G <= 16
// (k4d_online_supported).
bool k4d_online_supported(int d, int R);
hipError_t launch_k4d_online(const uint16_t *q, const uint16_t *kc, const uint16_t *vc,
                             const int32_t *ids, const int32_t *seq_len, const int32_t *table,
                             int maxb, int N, int64_t Lmax, int H, int G, int d, int k, float scale,
                             uint16_t *out, hipStream_t s);

// K4d in P parts of consecutive slots, one work-group each (two per CU): part
// outputs normalised in po [((n*H + h)*P + part)*d], log2-sum-exp in
// plse [((n*G + g)*P + part)*R + h % R], mark [(n*G + g)*P + part] = 0 (valid) or -1
// (no valid slot).  K5 with k = P, nb_lim = 1 and ids = mark merges them.  R <= 16.
hipError_t launch_k4d_parts(const uint16_t *q, const uint16_t *kc, const uint16_t *vc,
                            const int32_t *ids, const int32_t *seq_len, const int32_t *table,
                            int maxb, int N, int64_t Lmax, int H, int G, int d, int k, int P,
                            float scale, uint16_t *po, float *plse, int32_t *mark,
                            hipStream_t s);

// Paged decode: eff_len[n] = seq_len[n] when 1 <= seq_len[n] <= maxb * 128 and
// every page id the sequence needs is in [0, num_pages), else 0.
hipError_t launch_page_check(const int32_t *table, int maxb, int64_t num_pages,
                             const int32_t *seq_len, int N, int32_t *eff_len, hipStream_t s);

// K5: two-phase combine of the partials of `nq` queries into out[nq, H, d].
// ids [nq, G, k]: a slot is merged when 0 <= id < nb_lim, or with a batch map when
// 0 <= id <= b(row) -- the rule K3 scheduled by.  unnorm: the partials are K4's
// (unnormalised o with (maximum, sum) pairs); else K4d's (normalised o with their
// log2-sum-exp, plse [((i*G + g)*k + slot)*R + h % R]).
// sparse_rows: most rows hold few valid slots (a batch of short sequences); then a
// grid-stride form that requests the next item's ids with the current partials runs.
hipError_t launch_k5_combine(const uint16_t *po, const float *plse, const int32_t *ids, int64_t nq,
                             int H, int G, int d, int k, int nb_lim, uint16_t *out,
                             const BatchMap &bm, bool unnorm, bool sparse_rows, hipStream_t s);

// Fill n ints with a value (used instead of hipMemsetAsync so calls stay capturable).
hipError_t launch_fill_i32(int *p, int64_t n, int value, hipStream_t s);

}  // namespace msa
