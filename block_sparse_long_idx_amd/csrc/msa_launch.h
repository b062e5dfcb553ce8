// msa_launch.h -- internal launchers of the MSA kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

constexpr int kBlock = 128;   // tokens per MSA block (B)

// Key blocks scored by one K1 work-group item, and blocks buffered before a flush.
constexpr int kK1KeyChunk = 32;
// Queries per K4 work item (one staged K/V block serves up to this many queries).
constexpr int kK4Queries = 128;
// Queries whose entries one K3 work-group sorts.
constexpr int kK3Queries = 2048;

// Round n up to a multiple of m.
inline int64_t round_up(int64_t n, int64_t m) { return (n + m - 1) / m * m; }

// Number of K1 work items for the query blocks [qb0, qb1).
int64_t k1_num_items(int qb0, int qb1);

// K1: block scores S[(i-q0)*G + g][b] for queries i in [q0, qend), blocks b < b(i).
hipError_t launch_k1_index_pool(const uint16_t *iq, const uint16_t *ik, float *S, int64_t L,
                                int64_t q0, int64_t qend, int G, int dI, int nbp,
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

// K3: invert query-major ids of queries [q0, q0 + C) into per-(g, block) lists.
struct SchedBuffers {
    int *counts;     // [nlists]
    int *offs;       // [nlists + 1]
    int *toff;       // [nlists + 1] prefix sum of ceil(count / kK4Queries)
    int *wcnt;       // [G * k3_num_groups(C) * nb] per-work-group counts / prefixes
    int *total;      // [1] number of K4 work items
    int *items;      // [k4_max_items] list index of every K4 work item
    uint32_t *list;  // [C * G * k] entries (i - q0) << 5 | slot
};
hipError_t launch_k3_schedule(const int32_t *ids, int64_t C, int G, int k, int nb,
                              const SchedBuffers &sb, hipStream_t s);
int64_t k4_max_items(int64_t C, int G, int k, int nb);
int k3_num_groups(int64_t C);

// K4: KV-outer attention over the scheduled lists -> partials per (query, head,
// slot): po [(i*H + h)*k + slot][d] bf16 (normalised o), plse [((i*G + g)*k + slot)*R
// + h % R] fp32 (log2-sum-exp of the scaled scores).
hipError_t launch_k4_kv_outer(const uint16_t *q, const uint16_t *kx, const uint16_t *vx,
                              const SchedBuffers &sb, int nb, int64_t L, int64_t q0, int64_t C,
                              int H, int G, int d, int k, float scale, uint16_t *po, float *plse,
                              hipStream_t s);

// K4d: decode split over slots -> partials per (sequence, head, slot).  Cache
// addressing as in K1d (kc, vc [N, Lmax, G, d] or pages [pages, 128, G, d]).
hipError_t launch_k4d_split(const uint16_t *q, const uint16_t *kc, const uint16_t *vc,
                            const int32_t *ids, const int32_t *seq_len, const int32_t *table,
                            int maxb, int N, int64_t Lmax, int H, int G, int d, int k, float scale,
                            uint16_t *po, float *plse, hipStream_t s);

// Paged decode: eff_len[n] = seq_len[n] when 1 <= seq_len[n] <= maxb * 128 and
// every page id the sequence needs is in [0, num_pages), else 0.
hipError_t launch_page_check(const int32_t *table, int maxb, int64_t num_pages,
                             const int32_t *seq_len, int N, int32_t *eff_len, hipStream_t s);

// K5: two-phase combine of the partials of `nq` queries into out[nq, H, d].
// ids [nq, G, k]: a slot is merged when 0 <= id < nb_lim.
hipError_t launch_k5_combine(const uint16_t *po, const float *plse, const int32_t *ids, int64_t nq,
                             int H, int G, int d, int k, int nb_lim, uint16_t *out,
                             hipStream_t s);

// Fill n ints with a value (used instead of hipMemsetAsync so calls stay capturable).
hipError_t launch_fill_i32(int *p, int64_t n, int value, hipStream_t s);

}  // namespace msa
