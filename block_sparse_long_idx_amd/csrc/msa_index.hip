// msa_index.hip -- index branch, scoring part: token index scores max-pooled
// into block scores ("MiniMax M3 算力省 20 倍", §二 Index Branch: one index-query
// head per GQA group, one index-key head shared by all groups, dot products
// over the causal window, max-pooling into B = 128-token blocks).
//
// K1 (prefill) is a short-K GEMM with a max-pool epilogue, run on bf16 MFMA with
// fp32 accumulation.  One work-group (4 waves) owns part of one query block (64
// or 128 queries x G groups of stacked index rows, contiguous in idx_q[L,G,dI]) and
// a range of up to 32 key blocks strictly before the query block; the query's
// own block is never scored because it is always selected.  Index rows stay in
// registers for the whole range; each 128-key block of idx_k is staged once in
// LDS (double-buffered) and multiplied as S^T = K * IQ^T so that a lane's
// accumulators hold 16 keys of one index row: the 128-key max is an in-lane max
// plus one exchange between the two half-waves.  Block maxima are buffered in
// LDS and flushed as contiguous 32-byte row segments.  The L x L token score
// matrix never exists in memory.
//
// K1d (decode) streams each sequence's idx_k cache once (the HBM-bound part of
// decode): one wave per 128-key block, 16x16x32 MFMA with the G index heads as
// the N dimension, operands loaded straight from global memory.  The cache is
// either contiguous per sequence or paged: with a block table, logical block b of
// sequence n is the 128-token page table[n][b].
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

constexpr int kK1Flush = 8;   // key blocks buffered in LDS between flushes

// Work items are ordered key-chunk-major: for key chunk c of kc blocks, query
// blocks qb in [max(qb0, kc*c+1), qb1) -- each split into P parts of 128/P queries
// -- score key blocks [kc*c, min(kc*c+kc, qb)).  Every (query, key block) score is
// written by exactly one item whatever kc: kc = kK1KeyChunk, or fewer for a small
// query range so that the launch has enough work-groups (k1_key_chunk).
__device__ __forceinline__ bool k1_item(int64_t item, int qb0, int qb1, int P, int kc, int &qb,
                                        int &part, int &c) {
    for (c = 0;; ++c) {
        const int lo = max(qb0, c * kc + 1);
        if (lo >= qb1) return false;
        const int64_t n = (int64_t)(qb1 - lo) * P;
        if (item < n) {
            qb = lo + (int)(item / P);
            part = (int)(item % P);
            return true;
        }
        item -= n;
    }
}

int64_t k1_num_items(int qb0, int qb1, int kc) {
    int64_t total = 0;
    for (int c = 0;; ++c) {
        const int lo = qb0 > c * kc + 1 ? qb0 : c * kc + 1;
        if (lo >= qb1) break;
        total += qb1 - lo;
    }
    return total;
}

// Four waves per work-group, 32*NT index rows per wave; a work-group covers
// QT = 128*NT/G queries (all G groups) of one query block, P = 128/QT parts.
//   G = 1: NT 1, 128 queries;  G = 2: NT 1, 64;  G = 4: NT 2, 64;  G = 8: NT 2, 32.
// Two work-groups fit on a CU (LDS 64 KB key tiles + row maxima each), so one
// work-group's barrier is covered by the other's MFMAs.
template <int G> struct K1Tiling {
    static constexpr int NT = G >= 4 ? 2 : 1;
    static constexpr int ROWS = 4 * 32 * NT;
    static constexpr int QT = ROWS / G;
    static constexpr int P = kBlock / QT;
    static constexpr int THREADS = 256;
};

// BATCH: the work-groups of several sequences in one launch; tab (device copy of
// the batch table) gives each sequence's first work-group, rows and tokens, and
// the work-group rebases iq, ik, S and its query range on its own sequence.
template <int G, int DI, bool BATCH>
__global__ __launch_bounds__(256, 2) void k1_index_pool(
    const uint16_t *__restrict__ iq, const uint16_t *__restrict__ ik, float *__restrict__ S,
    int64_t q0, int64_t qend, int nbp, int qb0, int qb1, int64_t n_items, int kc,
    const BatchTable *__restrict__ tab) {
    constexpr int NT = K1Tiling<G>::NT;
    constexpr int NTHR = K1Tiling<G>::THREADS;
    constexpr int P = K1Tiling<G>::P;
    constexpr int CPR = DI / 8;            // 16-byte chunks per index row
    constexpr int KS = DI / 16;            // MFMA K-steps
    constexpr int NCOL = K1Tiling<G>::ROWS;   // stacked index rows of the work-group
    constexpr int TILE = kBlock * DI * 2;  // bytes of one staged key block
    __shared__ __attribute__((aligned(16))) char lds_k[2][TILE];
    __shared__ float lds_s[kK1Flush][NCOL];

    // XCD-aware order: consecutive logical items (same key chunk) on one XCD.
    const int64_t per = gridDim.x / 8;
    int64_t item = (blockIdx.x % 8) * per + blockIdx.x / 8;
    if constexpr (BATCH) {
        if (item >= tab->k1_off[tab->n]) return;
        int lo = 0, hi = tab->n;   // the sequence: largest sq with k1_off[sq] <= item
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (tab->k1_off[mid] <= item) lo = mid;
            else hi = mid;
        }
        const int sq = lo;
        const int64_t L = tab->kv_len[sq];
        const int64_t P0 = L - (tab->q_off[sq + 1] - tab->q_off[sq]);   // cached prefix
        q0 = P0;
        qend = L;
        qb0 = (int)(P0 / kBlock);
        qb1 = (int)((L + kBlock - 1) / kBlock);
        // the row of query position p is batch row q_off + p - P0
        iq += ((int64_t)tab->q_off[sq] - P0) * G * DI;
        ik += (int64_t)tab->kv_off[sq] * DI;
        S += (int64_t)tab->q_off[sq] * G * nbp;
        item -= tab->k1_off[sq];
    } else {
        if (item >= n_items * P) return;
    }
    int qb, part, c;
    if (!k1_item(item, qb0, qb1, P, kc, qb, part, c)) return;
    const int j0 = c * kc;
    const int j1 = min(j0 + kc, qb);

    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const int hf = lane >> 5, l32 = lane & 31;

    // B operand: index rows of this wave, kept in registers.
    bf16x8 bq[NT][KS];
    const int64_t row0 = ((int64_t)qb * kBlock + part * K1Tiling<G>::QT) * G;   // [L*G] row of column 0
    const int64_t row_end = qend * G;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int64_t row = row0 + wave * 32 * NT + nt * 32 + l32;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            bq[nt][ks] = as_bf16x8(row < row_end ? load16(iq + row * DI + (2 * ks + hf) * 8)
                                                 : u32x4{0, 0, 0, 0});
    }

    const char *ikb = reinterpret_cast<const char *>(ik);
    const int64_t blk_bytes = (int64_t)kBlock * DI * 2;
    // key blocks j < qb are always full, so the tiles need no zero fill
    stage_rows_direct<CPR, NTHR>(lds_k[0], ikb + j0 * blk_bytes, DI * 2, tid);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int j = j0; j < j1; ++j) {
        const int buf = (j - j0) & 1;
        const bool more = j + 1 < j1;
        float mx[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) mx[nt] = -INFINITY;
        // A operands (key rows) of M-tile mt+1 are read from LDS while the MFMAs of
        // M-tile mt run, so LDS latency is not exposed between MFMAs
        const char *kt = lds_k[buf];
        bf16x8 a_cur[KS], a_nxt[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) a_cur[ks] = as_bf16x8(load16(kt + swz<CPR>(l32, 2 * ks + hf)));
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            if (mt < 3) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    a_nxt[ks] = as_bf16x8(load16(kt + swz<CPR>((mt + 1) * 32 + l32, 2 * ks + hf)));
            }
            // The next key block goes straight into the other LDS buffer (last read in
            // the previous iteration, before its closing barrier).  It is issued after
            // this block's last operand reads: the compiler cannot tell the two buffers
            // apart and waits for these loads before any later LDS read.
            if (mt == 2 && more)
                stage_rows_direct<CPR, NTHR>(lds_k[buf ^ 1], ikb + (j + 1) * blk_bytes, DI * 2, tid);
            // one M-tile of operand reads in flight: nothing crosses this point
            __builtin_amdgcn_sched_barrier(0);
            f32x16 acc[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma32(a_cur[ks], bq[nt][ks], acc[nt]);
            }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                float m = acc[nt][0];
#pragma unroll
                for (int r = 1; r < 16; ++r) m = __builtin_fmaxf(m, acc[nt][r]);
                mx[nt] = __builtin_fmaxf(mx[nt], m);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) a_cur[ks] = a_nxt[ks];
        }
        const int slot = (j - j0) % kK1Flush;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const float m = fmaxf(mx[nt], xor_shfl(mx[nt], 32));
            if (hf == 0) lds_s[slot][wave * 32 * NT + nt * 32 + l32] = m;
        }
        __builtin_amdgcn_s_waitcnt(0);   // the next tile has landed in LDS
        __syncthreads();
        if (slot == kK1Flush - 1 || j == j1 - 1) {
            const int nj = slot + 1;
            const int jb = j - slot;
            for (int col = tid; col < NCOL; col += NTHR) {
                const int64_t row = row0 + col;
                if (row >= row_end) continue;
                float *dst = S + (row - q0 * G) * nbp + jb;
                if (nj == kK1Flush) {
                    store16(dst, u32x4{__float_as_uint(lds_s[0][col]), __float_as_uint(lds_s[1][col]),
                                       __float_as_uint(lds_s[2][col]), __float_as_uint(lds_s[3][col])});
                    store16(dst + 4, u32x4{__float_as_uint(lds_s[4][col]), __float_as_uint(lds_s[5][col]),
                                           __float_as_uint(lds_s[6][col]), __float_as_uint(lds_s[7][col])});
                } else {
                    for (int jj = 0; jj < nj; ++jj) dst[jj] = lds_s[jj][col];
                }
            }
            __syncthreads();
        }
    }
}

template <int G, int DI>
static hipError_t k1_dispatch(const uint16_t *iq, const uint16_t *ik, float *S, int64_t q0,
                              int64_t qend, int nbp, hipStream_t s) {
    const int qb0 = (int)(q0 / kBlock);
    const int qb1 = (int)((qend + kBlock - 1) / kBlock);
    // key chunk: halved from kK1KeyChunk while the launch would have fewer than two
    // work-groups per CU (a short query range otherwise leaves most CUs idle and
    // serialises each work-group's key blocks), down to kK1MinKeyChunk
    int kc = kK1KeyChunk;
    while (kc > kK1MinKeyChunk && k1_num_items(qb0, qb1, kc) * K1Tiling<G>::P < kK1MinWorkGroups)
        kc /= 2;
    const int64_t n = k1_num_items(qb0, qb1, kc);
    if (n == 0) return hipSuccess;
    const int64_t grid = round_up(n * K1Tiling<G>::P, 8);
    hipLaunchKernelGGL((k1_index_pool<G, DI, false>), dim3((unsigned)grid), dim3(K1Tiling<G>::THREADS),
                       0, s, iq, ik, S, q0, qend, nbp, qb0, qb1, n, kc, nullptr);
    return hipGetLastError();
}

template <int G, int DI>
static hipError_t k1_dispatch_batch(const uint16_t *iq, const uint16_t *ik, float *S,
                                    const BatchTable &t, const BatchTable *dtab, int nbp,
                                    hipStream_t s) {
    const int64_t grid = round_up(t.k1_off[t.n], 8);
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((k1_index_pool<G, DI, true>), dim3((unsigned)grid), dim3(K1Tiling<G>::THREADS),
                       0, s, iq, ik, S, 0, 0, nbp, 0, 0, 0, kK1KeyChunk, dtab);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// K12: index scores, block max-pool and the exp-free selection in one kernel
// ("MiniMax M3 算力省 20 倍", §二 Index Branch: max-pooled block scores, top-k per
// group, the own block always kept; §四 Kernel: selection on raw scores, no exp).
// The block scores never leave the chip: a work-group owns 256 stacked index rows
// (64 queries x G groups of one query block) and sweeps ALL their competitor key
// blocks 0 .. b(i)-1 (K1 splits that range into 32-block items), scoring each
// staged 128-key tile with K1's MFMA tiling.  Every row keeps, in registers, the
// score tau of its current (k-1)-th best block and the length of a short candidate
// list in memory (CAP entries of (score, block) per row, in the workspace): a block
// enters the list only when its score is above tau -- so a block scoring the same
// as the current (k-1)-th best, which has a smaller id, never displaces it -- and
// whenever some row's list is full the wave cuts every row's list to its k-1 best
// (rank = number of entries with a larger score, or an equal score and a smaller
// block id) and raises tau.  Blocks arrive in increasing id order, so the final
// cut is exactly the selection of K2.  After the sweep each row emits its own block
// plus the kept competitors, ascending, padded with -1.
// Work-groups run longest first (query block descending) and go to the XCDs in
// turn, so the work-groups that share an XCD sweep nearby key ranges together and
// reuse the staged key tiles from its L2.
// ---------------------------------------------------------------------------
constexpr int kK12Cap = 32;   // candidate list entries per row
constexpr int kK12Keep = 16;  // most competitors kept per row (k - 1), half the list

// Cuts one row's list (cnt entries at c) to its `keep` best entries, stored in rank
// order; tau becomes the keep-th best score once cnt >= keep.
__device__ __forceinline__ void k12_cut(uint2 *c, int &cnt, float &tau, int keep) {
    float sc[kK12Cap];
    int id[kK12Cap];
#pragma unroll
    for (int e = 0; e < kK12Cap; ++e) {
        const uint2 v = e < cnt ? c[e] : uint2{__float_as_uint(-INFINITY), 0x7FFFFFFFu};
        sc[e] = __uint_as_float(v.x);
        id[e] = (int)v.y;
    }
    float t = -INFINITY;
#pragma unroll
    for (int a = 0; a < kK12Cap; ++a) {
        int rank = 0;
#pragma unroll
        for (int b = 0; b < kK12Cap; ++b)
            rank += (sc[b] > sc[a]) || (sc[b] == sc[a] && id[b] < id[a]);
        if (rank < keep && a < cnt) c[rank] = uint2{__float_as_uint(sc[a]), (uint32_t)id[a]};
        if (rank == keep - 1 && a < cnt) t = sc[a];
    }
    if (cnt >= keep) tau = t;
    cnt = min(cnt, keep);
}

template <int G, int DI>
__global__ __launch_bounds__(256, 2) void k12_index_select(
    const uint16_t *__restrict__ iq, const uint16_t *__restrict__ ik, int32_t *__restrict__ ids,
    uint2 *__restrict__ cand, int64_t q0, int64_t qend, int qb0, int qb1, int k) {
    constexpr int NT = K1Tiling<G>::NT;
    constexpr int NTHR = K1Tiling<G>::THREADS;
    constexpr int P = K1Tiling<G>::P;
    constexpr int CPR = DI / 8;
    constexpr int KS = DI / 16;
    constexpr int TILE = kBlock * DI * 2;
    __shared__ __attribute__((aligned(16))) char lds_k[2][TILE];

    const int qb = qb1 - 1 - (int)(blockIdx.x / P);     // longest first
    const int part = (int)(blockIdx.x % P);
    if (qb < qb0) return;
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const int hf = lane >> 5, l32 = lane & 31;

    bf16x8 bq[NT][KS];
    const int64_t row0 = ((int64_t)qb * kBlock + part * K1Tiling<G>::QT) * G;
    const int64_t row_end = qend * G;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int64_t row = row0 + wave * 32 * NT + nt * 32 + l32;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            bq[nt][ks] = as_bf16x8(row < row_end ? load16(iq + row * DI + (2 * ks + hf) * 8)
                                                 : u32x4{0, 0, 0, 0});
    }
    // The row this lane keeps the selection of: with two N-tiles lane half hf owns
    // row nt = hf; with one both halves hold the same row and half 0 owns it.
    const int my_nt = NT == 2 ? hf : 0;
    const int64_t my_row = row0 + wave * 32 * NT + my_nt * 32 + l32;
    const bool owner = (NT == 2 || hf == 0) && my_row < row_end;
    uint2 *my_cand = cand + (owner ? (my_row - q0 * G) * kK12Cap : 0);
    const int keep = k - 1;
    float tau = -INFINITY;
    int cnt = 0;

    if (qb > 0 && keep > 0) {
        const char *ikb = reinterpret_cast<const char *>(ik);
        const int64_t blk_bytes = (int64_t)kBlock * DI * 2;
        stage_rows_direct<CPR, NTHR>(lds_k[0], ikb, DI * 2, tid);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        // A row's candidate from block j is written to its list at the start of block
        // j + 1, ahead of that block's tile copy: the wait for the copy at the end of
        // an iteration then does not also wait on a store just issued.  pend holds its
        // score (-inf: none; scores are finite).
        float pend = -INFINITY;
        for (int j = 0; j < qb; ++j) {
            const int buf = j & 1;
            const bool more = j + 1 < qb;
            if (owner && pend > -INFINITY)
                my_cand[cnt - 1] = uint2{__float_as_uint(pend), (uint32_t)(j - 1)};
            pend = -INFINITY;
            // the per-block scoring of K1 (same operands, same MFMA order)
            float mx[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) mx[nt] = -INFINITY;
            const char *kt = lds_k[buf];
            bf16x8 a_cur[KS], a_nxt[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                a_cur[ks] = as_bf16x8(load16(kt + swz<CPR>(l32, 2 * ks + hf)));
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                if (mt < 3) {
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
                        a_nxt[ks] = as_bf16x8(load16(kt + swz<CPR>((mt + 1) * 32 + l32, 2 * ks + hf)));
                }
                if (mt == 2 && more)
                    stage_rows_direct<CPR, NTHR>(lds_k[buf ^ 1], ikb + (j + 1) * blk_bytes, DI * 2, tid);
                __builtin_amdgcn_sched_barrier(0);
                f32x16 acc[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x16{};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma32(a_cur[ks], bq[nt][ks], acc[nt]);
                }
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    float m = acc[nt][0];
#pragma unroll
                    for (int r = 1; r < 16; ++r) m = __builtin_fmaxf(m, acc[nt][r]);
                    mx[nt] = __builtin_fmaxf(mx[nt], m);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) a_cur[ks] = a_nxt[ks];
            }
            float mine = -INFINITY;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const float m = fmaxf(mx[nt], xor_shfl(mx[nt], 32));
                if (nt == my_nt) mine = m;
            }
            if (owner && mine > tau) {
                pend = mine;
                ++cnt;
            }
            // a full list, or the last block: cut (the last cut leaves the selection)
            if (__ballot(cnt == kK12Cap) || j == qb - 1) {
                if (owner && pend > -INFINITY)
                    my_cand[cnt - 1] = uint2{__float_as_uint(pend), (uint32_t)j};
                pend = -INFINITY;
                if (owner) k12_cut(my_cand, cnt, tau, keep);
            }
            __builtin_amdgcn_s_waitcnt(0);   // the next tile has landed in LDS
            __syncthreads();
        }
    }
    if (!owner) return;
    // the own block and the kept competitors (at most kK12Keep), ascending
    int sel[kK12Keep];
#pragma unroll
    for (int e = 0; e < kK12Keep; ++e) sel[e] = e < cnt ? (int)my_cand[e].y : 0x7FFFFFFF;
    int32_t *out = ids + (my_row - q0 * G) * k;
#pragma unroll
    for (int a = 0; a < kK12Keep; ++a) {
        int rank = 0;
#pragma unroll
        for (int b = 0; b < kK12Keep; ++b) rank += sel[b] < sel[a];
        if (a < cnt) out[rank] = sel[a];
    }
    out[cnt] = qb;                               // every competitor id is below qb
    for (int sl = cnt + 1; sl < k; ++sl) out[sl] = -1;
}

template <int G, int DI>
static hipError_t k12_dispatch(const uint16_t *iq, const uint16_t *ik, int32_t *ids, uint2 *cand,
                               int64_t q0, int64_t qend, int k, hipStream_t s) {
    const int qb0 = (int)(q0 / kBlock);
    const int qb1 = (int)((qend + kBlock - 1) / kBlock);
    const int64_t grid = (int64_t)(qb1 - qb0) * K1Tiling<G>::P;
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL((k12_index_select<G, DI>), dim3((unsigned)grid), dim3(K1Tiling<G>::THREADS),
                       0, s, iq, ik, ids, cand, q0, qend, qb0, qb1, k);
    return hipGetLastError();
}

bool k12_supported(int G, int dI, int k) {
    return k >= 1 && k - 1 <= kK12Keep && (G == 1 || G == 2 || G == 4 || G == 8) &&
           (dI == 32 || dI == 64 || dI == 128) && G * dI <= 512;
}

int64_t k12_cand_entries(int64_t C, int G) { return C * G * kK12Cap; }

int64_t k12_num_workgroups(int64_t C, int G) {
    const int64_t nqb = (C + kBlock - 1) / kBlock;
    switch (G) {
    case 1: return nqb * K1Tiling<1>::P;
    case 2: return nqb * K1Tiling<2>::P;
    case 4: return nqb * K1Tiling<4>::P;
    default: return nqb * K1Tiling<8>::P;
    }
}

hipError_t launch_k12_index_select(const uint16_t *iq, const uint16_t *ik, int32_t *ids,
                                   void *cand, int64_t q0, int64_t qend, int G, int dI, int k,
                                   hipStream_t s) {
    uint2 *c = static_cast<uint2 *>(cand);
#define K12_CASE(g, di) \
    if (G == g && dI == di) return k12_dispatch<g, di>(iq, ik, ids, c, q0, qend, k, s);
    K12_CASE(1, 32) K12_CASE(1, 64) K12_CASE(1, 128)
    K12_CASE(2, 32) K12_CASE(2, 64) K12_CASE(2, 128)
    K12_CASE(4, 32) K12_CASE(4, 64) K12_CASE(4, 128)
    K12_CASE(8, 32) K12_CASE(8, 64)
#undef K12_CASE
    return hipErrorInvalidValue;
}

int64_t k1_num_workgroups(int64_t q0, int64_t qend, int G) {
    const int qb0 = (int)(q0 / kBlock), qb1 = (int)((qend + kBlock - 1) / kBlock);
    const int64_t n = k1_num_items(qb0, qb1);
    switch (G) {
    case 1: return n * K1Tiling<1>::P;
    case 2: return n * K1Tiling<2>::P;
    case 4: return n * K1Tiling<4>::P;
    default: return n * K1Tiling<8>::P;
    }
}

hipError_t launch_k1_index_pool_batch(const uint16_t *iq, const uint16_t *ik, float *S,
                                      const BatchTable &t, const BatchTable *dtab, int G, int dI,
                                      int nbp, hipStream_t s) {
#define K1B_CASE(g, di) \
    if (G == g && dI == di) return k1_dispatch_batch<g, di>(iq, ik, S, t, dtab, nbp, s);
    K1B_CASE(1, 32) K1B_CASE(1, 64) K1B_CASE(1, 128)
    K1B_CASE(2, 32) K1B_CASE(2, 64) K1B_CASE(2, 128)
    K1B_CASE(4, 32) K1B_CASE(4, 64) K1B_CASE(4, 128)
    K1B_CASE(8, 32) K1B_CASE(8, 64)
#undef K1B_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_k1_index_pool(const uint16_t *iq, const uint16_t *ik, float *S, int64_t L,
                                int64_t q0, int64_t qend, int G, int dI, int nbp,
                                hipStream_t s) {
    (void)L;
#define K1_CASE(g, di) \
    if (G == g && dI == di) return k1_dispatch<g, di>(iq, ik, S, q0, qend, nbp, s);
    K1_CASE(1, 32) K1_CASE(1, 64) K1_CASE(1, 128)
    K1_CASE(2, 32) K1_CASE(2, 64) K1_CASE(2, 128)
    K1_CASE(4, 32) K1_CASE(4, 64) K1_CASE(4, 128)
    K1_CASE(8, 32) K1_CASE(8, 64)
#undef K1_CASE
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// K1d: one wave per (sequence, 128-key block).  grid = (ceil(nbmax/4), N).
// table == nullptr: ikc is [N, Lmax, DI]; otherwise ikc is [pages, 128, DI] and
// table[n * maxb + b] names the page of block b (checked by the caller).
// ---------------------------------------------------------------------------
template <int G, int DI, bool PAGED>
__global__ __launch_bounds__(256) void k1d_index_pool(const uint16_t *__restrict__ iq,
                                                      const uint16_t *__restrict__ ikc,
                                                      const int32_t *__restrict__ seq_len,
                                                      const int32_t *__restrict__ table, int maxb,
                                                      float *__restrict__ S, int64_t Lmax,
                                                      int nbp) {
    constexpr int KS = DI / 32;
    const int n = blockIdx.y;
    // the wave index as a wave-uniform value, so that the block and its page-table
    // entry are read with scalar loads
    const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int b = blockIdx.x * 4 + wave;
    const int sl = seq_len[n];
    if (sl < 1 || sl > Lmax) return;
    const int ncomp = (sl - 1) / kBlock;       // blocks before the query's own block
    if (b >= ncomp) return;
    const int l16 = lane & 15, qt = lane >> 4;

    bf16x8 bq[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        bq[ks] = as_bf16x8(l16 < G ? load16(iq + ((int64_t)n * G + l16) * DI + 32 * ks + 8 * qt)
                                   : u32x4{0, 0, 0, 0});
    const int64_t tok0 = table ? (int64_t)table[(int64_t)n * maxb + b] * kBlock
                               : (int64_t)n * Lmax + (int64_t)b * kBlock;
    const uint16_t *base = ikc + tok0 * DI;
    u32x4 a[8][KS];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            a[mt][ks] = load16(base + (mt * 16 + l16) * DI + 32 * ks + 8 * qt);
    // paged: every key load of the page issued before the first MFMA (the page id's
    // read comes first, so the whole page's bytes are requested at once); contiguous
    // blocks keep the compiler's interleaving, which measures the same or better
    if constexpr (PAGED) __builtin_amdgcn_sched_barrier(0);
    float m = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
        f32x4 acc = f32x4{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = mfma16(as_bf16x8(a[mt][ks]), bq[ks], acc);
        m = fmaxf(m, fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3])));
    }
    m = fmaxf(m, xor_shfl(m, 16));
    m = fmaxf(m, xor_shfl(m, 32));
    if (lane < G) S[((int64_t)n * G + lane) * nbp + b] = m;
}

template <int G, int DI>
static hipError_t k1d_dispatch(const uint16_t *iq, const uint16_t *ikc, const int32_t *seq_len,
                               const int32_t *table, int maxb, float *S, int N, int64_t Lmax,
                               int nbp, hipStream_t s) {
    const int64_t nbmax = (Lmax - 1) / kBlock;   // competitors of the longest sequence
    if (nbmax <= 0 || N <= 0) return hipSuccess;
    dim3 grid((unsigned)((nbmax + 3) / 4), (unsigned)N);
    if (table)
        hipLaunchKernelGGL((k1d_index_pool<G, DI, true>), grid, dim3(256), 0, s, iq, ikc, seq_len,
                           table, maxb, S, Lmax, nbp);
    else
        hipLaunchKernelGGL((k1d_index_pool<G, DI, false>), grid, dim3(256), 0, s, iq, ikc, seq_len,
                           table, maxb, S, Lmax, nbp);
    return hipGetLastError();
}

hipError_t launch_k1d_index_pool(const uint16_t *iq, const uint16_t *ikc, const int32_t *seq_len,
                                 const int32_t *table, int maxb, float *S, int N, int64_t Lmax,
                                 int G, int dI, int nbp, hipStream_t s) {
#define K1D_CASE(g, di) \
    if (G == g && dI == di) return k1d_dispatch<g, di>(iq, ikc, seq_len, table, maxb, S, N, Lmax, nbp, s);
    K1D_CASE(1, 32) K1D_CASE(1, 64) K1D_CASE(1, 128)
    K1D_CASE(2, 32) K1D_CASE(2, 64) K1D_CASE(2, 128)
    K1D_CASE(4, 32) K1D_CASE(4, 64) K1D_CASE(4, 128)
    K1D_CASE(8, 32) K1D_CASE(8, 64)
#undef K1D_CASE
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// K1d over an FP8 index-key cache: bytes ik8[N, Lmax, DI] in the OCP E4M3 encoding
// and one fp32 scale per token, ksc[N, Lmax]; the score of token t is
// ksc[t] * (iq . e4m3(ik8[t])).  Half the bytes of the bf16 cache per key.  One
// wave scores BPW consecutive blocks, requesting all their bytes up front.  Each
// E4M3 value is exact in bf16, so bytes are widened in registers
// (v_cvt_scalef32_pk_bf16_fp8, scale 1) and the bf16 MFMA of K1d runs unchanged;
// the token scale multiplies the fp32 dot product before the block max.  The
// contraction index is relabelled so that a lane's key bytes are contiguous: in
// MFMA step ks, quarter qt of the wave holds elements 8*KS*qt + 8*ks .. +7 of
// both operands.
// ---------------------------------------------------------------------------
template <int G, int DI, int BPW>
__global__ __launch_bounds__(256) void k1d_index_pool_fp8(const uint16_t *__restrict__ iq,
                                                          const uint8_t *__restrict__ ik8,
                                                          const float *__restrict__ ksc,
                                                          const int32_t *__restrict__ seq_len,
                                                          const int32_t *__restrict__ table,
                                                          int maxb, float *__restrict__ S,
                                                          int64_t Lmax, int nbp, int sc_aligned) {
    constexpr int KS = DI / 32;
    constexpr int SPAN = 8 * KS;          // contiguous key bytes per lane and token
    // first token row of block b: contiguous caches [N, Lmax, ...], or the block's
    // page of paged caches [pages, 128, ...]
    auto tok0 = [&](int64_t n, int b) {
        return table ? (int64_t)table[n * maxb + b] * kBlock : n * Lmax + (int64_t)b * kBlock;
    };
    const int n = blockIdx.y;
    // wave-uniform, so that the blocks' page-table entries are read with scalar loads
    const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int b0 = (blockIdx.x * 4 + wave) * BPW;   // this wave's first block
    const int sl = seq_len[n];
    if (sl < 1 || sl > Lmax) return;
    const int ncomp = (sl - 1) / kBlock;
    if (b0 >= ncomp) return;
    const int l16 = lane & 15, qt = lane >> 4;

    bf16x8 bq[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        bq[ks] = as_bf16x8(l16 < G ? load16(iq + ((int64_t)n * G + l16) * DI + SPAN * qt + 8 * ks)
                                   : u32x4{0, 0, 0, 0});
    // raw[bb][mt][w]: dword w of this lane's SPAN bytes of token mt*16 + l16 of block
    // b0 + bb; every block's bytes are requested before any is converted
    uint32_t raw[BPW][8][SPAN / 4];
#pragma unroll
    for (int bb = 0; bb < BPW; ++bb) {
        // a block past the sequence's competitors re-reads the first block (discarded)
        const int b = b0 + bb < ncomp ? b0 + bb : b0;
        const uint8_t *base = ik8 + tok0(n, b) * DI + SPAN * qt;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const uint8_t *p = base + (mt * 16 + l16) * DI;
            if constexpr (SPAN >= 16) {
#pragma unroll
                for (int c = 0; c < SPAN / 16; ++c) {
                    const u32x4 v = load16(p + 16 * c);
#pragma unroll
                    for (int e = 0; e < 4; ++e) raw[bb][mt][4 * c + e] = v[e];
                }
            } else {
                const u32x2 v = *reinterpret_cast<const u32x2 *>(p);
                raw[bb][mt][0] = v[0];
                raw[bb][mt][1] = v[1];
            }
        }
    }
#pragma unroll
    for (int bb = 0; bb < BPW; ++bb) {
        const int b = b0 + bb;
        if (b >= ncomp) break;
        // token scales of this lane's accumulator rows: tokens mt*16 + 4*qt + r
        const float *sp = ksc + tok0(n, b) + 4 * qt;
        float m = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            f32x4 acc = f32x4{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                bf16x8 a;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t w = raw[bb][mt][2 * ks + h];
                    const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
                    const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
                    a[4 * h + 0] = lo[0];
                    a[4 * h + 1] = lo[1];
                    a[4 * h + 2] = hi[0];
                    a[4 * h + 3] = hi[1];
                }
                acc = mfma16(a, bq[ks], acc);
            }
            const float *p = sp + mt * 16;
            const f32x4 sc = sc_aligned ? *reinterpret_cast<const f32x4 *>(p)
                                        : f32x4{p[0], p[1], p[2], p[3]};
            m = fmaxf(m, fmaxf(fmaxf(acc[0] * sc[0], acc[1] * sc[1]),
                               fmaxf(acc[2] * sc[2], acc[3] * sc[3])));
        }
        m = fmaxf(m, xor_shfl(m, 16));
        m = fmaxf(m, xor_shfl(m, 32));
        if (lane < G) S[((int64_t)n * G + lane) * nbp + b] = m;
    }
}

template <int G, int DI>
static hipError_t k1d8_dispatch(const uint16_t *iq, const uint8_t *ik8, const float *ksc,
                                const int32_t *seq_len, const int32_t *table, int maxb, float *S,
                                int N, int64_t Lmax, int nbp, hipStream_t s) {
    const int64_t nbmax = (Lmax - 1) / kBlock;
    if (nbmax <= 0 || N <= 0) return hipSuccess;
    // 16-byte scale loads need every block's scales 16-byte aligned (pages of 128
    // scales always are)
    const int aligned = (table || Lmax % 4 == 0) && (reinterpret_cast<uintptr_t>(ksc) % 16 == 0);
    // two blocks per wave: 32 KB in flight per wave at 2 waves per SIMD (measured
    // faster than one block at 3 waves per SIMD, and than four at one wave)
    constexpr int BPW = 2;
    dim3 grid((unsigned)((nbmax + 4 * BPW - 1) / (4 * BPW)), (unsigned)N);
    hipLaunchKernelGGL((k1d_index_pool_fp8<G, DI, BPW>), grid, dim3(256), 0, s, iq, ik8, ksc,
                       seq_len, table, maxb, S, Lmax, nbp, aligned);
    return hipGetLastError();
}

hipError_t launch_k1d_index_pool_fp8(const uint16_t *iq, const uint8_t *ik8, const float *ksc,
                                     const int32_t *seq_len, const int32_t *table, int maxb,
                                     float *S, int N, int64_t Lmax, int G, int dI, int nbp,
                                     hipStream_t s) {
#define K1D8_CASE(g, di) \
    if (G == g && dI == di) return k1d8_dispatch<g, di>(iq, ik8, ksc, seq_len, table, maxb, S, N, Lmax, nbp, s);
    K1D8_CASE(1, 32) K1D8_CASE(1, 64) K1D8_CASE(1, 128)
    K1D8_CASE(2, 32) K1D8_CASE(2, 64) K1D8_CASE(2, 128)
    K1D8_CASE(4, 32) K1D8_CASE(4, 64) K1D8_CASE(4, 128)
    K1D8_CASE(8, 32) K1D8_CASE(8, 64)
#undef K1D8_CASE
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Index-key cache writer: per-row power-of-two scale and E4M3 rounding.  For a
// row x of DI bf16 values: scale = 2^e with e the smallest integer such that
// max|x| <= 448 * 2^e (e = 0 for a zero row); each byte is the E4M3 value nearest
// to x / scale (ties to the even code), which the hardware conversion
// v_cvt_pk_fp8_f32 produces in round-to-nearest-even mode.  DI/8 threads per row,
// 8 values (16 bytes in, 8 bytes out) per thread.
// ---------------------------------------------------------------------------
template <int DI>
__global__ __launch_bounds__(256) void k_quant_e4m3(const uint16_t *__restrict__ x, int64_t rows,
                                                    uint8_t *__restrict__ out,
                                                    float *__restrict__ scale) {
    constexpr int TPR = DI / 8;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = t / TPR;
    const int sub = (int)(t % TPR);
    const bool active = row < rows;
    float v[8];
    float amax = 0.0f;
    if (active) {
        const u32x4 w = load16(x + row * DI + 8 * sub);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = bf16_to_f32(w[e] & 0xFFFFu);
            v[2 * e + 1] = bf16_to_f32(w[e] >> 16);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
    }
    // row maximum over the TPR threads of the row (aligned groups of lanes)
#pragma unroll
    for (int m = 1; m < TPR; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, kWave));
    if (!active) return;
    int e = 0;
    if (amax > 0.0f) {
        int ex;
        const float fr = frexpf(amax / 448.0f, &ex);   // amax/448 = fr * 2^ex, fr in [0.5, 1)
        e = fr == 0.5f ? ex - 1 : ex;
    }
    uint32_t lo = 0, hi = 0;
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[0], -e), ldexpf(v[1], -e), lo, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[2], -e), ldexpf(v[3], -e), lo, true);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4], -e), ldexpf(v[5], -e), hi, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[6], -e), ldexpf(v[7], -e), hi, true);
    store8(out + row * DI + 8 * sub, u32x2{lo, hi});
    if (sub == 0) scale[row] = ldexpf(1.0f, e);
}

hipError_t launch_quant_e4m3(const uint16_t *x, int64_t rows, int dI, uint8_t *out, float *scale,
                             hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    const int64_t threads = rows * (dI / 8);
    const dim3 grid((unsigned)((threads + 255) / 256));
    if (dI == 32) hipLaunchKernelGGL(k_quant_e4m3<32>, grid, dim3(256), 0, s, x, rows, out, scale);
    else if (dI == 64) hipLaunchKernelGGL(k_quant_e4m3<64>, grid, dim3(256), 0, s, x, rows, out, scale);
    else if (dI == 128) hipLaunchKernelGGL(k_quant_e4m3<128>, grid, dim3(256), 0, s, x, rows, out, scale);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace msa
