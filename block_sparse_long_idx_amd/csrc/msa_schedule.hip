// msa_schedule.hip -- K3: turn query-major selections into KV-block-major work
// ("MiniMax M3 算力省 20 倍", §四 Kernel: KV-outer iteration gathers the queries that
// picked each KV block; a scheduling kernel splits hot tiles ahead of time along the
// query dimension so no single work-group owns a block picked by almost every query;
// "MiniMax M3 的采用瓶颈…" §对建设者的影响: KV-block-major layout).
//
// A counting sort with no global atomics.  Work-group (w, g) owns the entries of
// group g for qpw consecutive queries of the chunk (kK3Queries, halved for small
// chunks until the count and scatter passes have about kK3TargetGroups work-groups,
// down to kK3MinQueries):
//   count    per-work-group histogram over the group's blocks, in LDS
//   colscan  per list: exclusive prefix of the work-group counts, list total
//   scan     offs = exclusive prefix of the list totals; toff = exclusive prefix of
//            the number of pre-sized tiles ceil(count / kK4Queries) per list
//   scatter  list[offs[l] + prefix(w) + rank] = (query - q0) << 5 | slot
// Hot blocks (picked by nearly every query) only cost LDS atomics.  The order of
// entries inside one work-group's share of a list depends on LDS atomic timing, but
// no result does: every entry's partial goes to its own (query, head, slot).
//
// Then K4's run order: the work items (tiles of 128 entries of one list) sorted by
// group and by the window of 2^sh queries that holds their middle entry, by the same
// counting sort over work-groups of kK3Tiles items:
//   tile_count    per-work-group bucket histogram
//   tile_scan     bucket-major, work-group-minor exclusive prefix (the bases)
//   tile_scatter  order[base + rank] = item
// Run in that order, the items in flight at any time gather the q rows of a narrow
// range of queries, which the last-level cache holds across much of their 16
// re-reads (one per selected block) -- K4 writes its partial rows with streaming
// stores, so they do not displace them -- where the list order spreads those reads
// over the whole chunk.
//
// Also here: the page-table check of paged decode ("MiniMax M3 的采用瓶颈…"
// §对建设者的影响: paged MSA decode), run before any page is read.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

__global__ void k_fill_i32(int *p, int64_t n, int v) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < n) p[t] = v;
}

hipError_t launch_fill_i32(int *p, int64_t n, int value, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, value);
    return hipGetLastError();
}

// Paged decode: one work-group per sequence checks the page ids of the blocks it
// needs (0 .. b(seq_len - 1)) and writes the length the later kernels may use: the
// sequence's own length, or 0 (no block selected, zero output) when the length is
// out of range or a needed page id is outside [0, num_pages).
__global__ __launch_bounds__(256) void k_page_check(const int32_t *__restrict__ table, int maxb,
                                                    int64_t num_pages,
                                                    const int32_t *__restrict__ seq_len,
                                                    int32_t *__restrict__ eff_len) {
    const int n = blockIdx.x;
    const int sl = seq_len[n];
    const bool len_ok = sl >= 1 && (int64_t)sl <= (int64_t)maxb * kBlock;
    int bad = 0;
    if (len_ok) {
        const int nblk = (sl - 1) / kBlock + 1;
        const int32_t *row = table + (int64_t)n * maxb;
#pragma unroll 8
        for (int b = threadIdx.x; b < nblk; b += 256) {
            const int32_t pg = row[b];
            bad |= pg < 0 || (int64_t)pg >= num_pages;
        }
    }
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) eff_len[n] = (len_ok && !bad) ? sl : 0;
}

hipError_t launch_page_check(const int32_t *table, int maxb, int64_t num_pages,
                             const int32_t *seq_len, int N, int32_t *eff_len, hipStream_t s) {
    if (N <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_page_check, dim3((unsigned)N), dim3(256), 0, s, table, maxb, num_pages,
                       seq_len, eff_len);
    return hipGetLastError();
}

// Batched varlen prefill: per-row and per-global-block tables from the batch's
// host description (one thread per row and per block; the sequence is found by
// binary search over the offsets, which live in the kernel-argument segment).
__global__ __launch_bounds__(256) void k_batch_setup(const BatchTable t, BatchTable *__restrict__ dtab,
                                                     int32_t *__restrict__ row_len,
                                                     int32_t *__restrict__ row_kvpos,
                                                     int32_t *__restrict__ row_blk0,
                                                     int32_t *__restrict__ blk_tok0,
                                                     int32_t *__restrict__ blk_rows) {
    const BatchTable *tp = &t;
    const int x = blockIdx.x * 256 + threadIdx.x;
    if (blockIdx.x == 0) {   // device copy of the table, one int per thread and step
        const int *src = reinterpret_cast<const int *>(tp);
        int *dst = reinterpret_cast<int *>(dtab);
        for (int w = threadIdx.x; w < (int)(sizeof(BatchTable) / sizeof(int)); w += 256)
            dst[w] = src[w];
    }
    auto seq_of = [&](const int *off, int v) {   // largest s with off[s] <= v
        int lo = 0, hi = tp->n;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (off[mid] <= v) lo = mid;
            else hi = mid;
        }
        return lo;
    };
    if (x < tp->rows) {
        const int sq = seq_of(tp->q_off, x);
        const int newc = tp->q_off[sq + 1] - tp->q_off[sq];
        const int pos = tp->kv_len[sq] - newc + (x - tp->q_off[sq]);
        row_len[x] = pos + 1;
        row_kvpos[x] = tp->kv_off[sq] + pos;
        row_blk0[x] = tp->blk_off[sq];
    }
    if (x < tp->blocks) {
        const int sq = seq_of(tp->blk_off, x);
        const int j = x - tp->blk_off[sq];
        blk_tok0[x] = tp->kv_off[sq] + j * kBlock;
        blk_rows[x] = min(kBlock, tp->kv_len[sq] - j * kBlock);
    }
}

hipError_t launch_batch_setup(const BatchTable &t, BatchTable *dtab, int32_t *row_len,
                              int32_t *row_kvpos, int32_t *row_blk0, int32_t *blk_tok0,
                              int32_t *blk_rows, hipStream_t s) {
    const int n = t.rows > t.blocks ? t.rows : t.blocks;
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_batch_setup, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, t, dtab,
                       row_len, row_kvpos, row_blk0, blk_tok0, blk_rows);
    return hipGetLastError();
}

// Entries of one work-group: queries [w*qpw, (w+1)*qpw) of the chunk, group g, all
// k slots; entry e -> query w*qpw + e / k, slot e % k.  Returns
// the entry's list block, or -1 for an id that is not scheduled: outside [0, nb),
// or in a batch outside [0, b(row)] (then the list block is the global one).
__device__ __forceinline__ int entry_block(const int32_t *ids, int64_t C, int G, int k, int nb,
                                           const BatchMap &bm, int g, int64_t i, int s) {
    if (i >= C) return -1;
    const int id = ids[(i * G + g) * k + s];
    if (bm.row_len) {
        const int own = (bm.row_len[i] - 1) / kBlock;
        return (id >= 0 && id <= own) ? bm.row_blk0[i] + id : -1;
    }
    return (id >= 0 && id < nb) ? id : -1;
}

// Count pass: per-work-group histogram in LDS, written (zeros included) to
// wcnt[(g * nW + w) * nb + b].  No global atomics.
__global__ __launch_bounds__(256) void k3_count(const int32_t *__restrict__ ids, int64_t C, int G,
                                                int k, int nb, int qpw, const BatchMap bm,
                                                int *__restrict__ wcnt) {
    extern __shared__ int lds_cnt[];
    const int w = blockIdx.x, g = blockIdx.y, nW = gridDim.x;
    for (int b = threadIdx.x; b < nb; b += 256) lds_cnt[b] = 0;
    __syncthreads();
    const int64_t i0 = (int64_t)w * qpw;
    for (int e = threadIdx.x; e < qpw * k; e += 256) {
        const int id = entry_block(ids, C, G, k, nb, bm, g, i0 + e / k, e % k);
        if (id >= 0) atomicAdd(&lds_cnt[id], 1);
    }
    __syncthreads();
    int *dst = wcnt + ((int64_t)g * nW + w) * nb;
    for (int b = threadIdx.x; b < nb; b += 256) dst[b] = lds_cnt[b];
}

// Column pass: for every list (g, b), turn the work-group counts into exclusive
// prefixes over w (in place) and store the list's total in counts[g * nb + b].
__global__ __launch_bounds__(256) void k3_colscan(int *__restrict__ wcnt, int G, int nb, int nW,
                                                  int *__restrict__ counts) {
    const int64_t l = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (l >= (int64_t)G * nb) return;
    const int g = (int)(l / nb), b = (int)(l % nb);
    int *col = wcnt + (int64_t)g * nW * nb + b;   // work-group w's count at col[w * nb]
    // the counts are read 16 at a time before any prefix is written, so that a
    // batch's loads are in flight together rather than one round trip per count
    constexpr int kBatch = 16;
    int run = 0;
    for (int w0 = 0; w0 < nW; w0 += kBatch) {
        int c[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) c[j] = w0 + j < nW ? col[(int64_t)(w0 + j) * nb] : 0;
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            if (w0 + j < nW) col[(int64_t)(w0 + j) * nb] = run;
            run += c[j];
        }
    }
    counts[l] = run;
}

// Scatter pass: each work-group places its entries at
// offs[list] + (entries of earlier work-groups) + (rank inside this work-group).
__global__ __launch_bounds__(256) void k3_scatter(const int32_t *__restrict__ ids, int64_t C, int G,
                                                  int k, int nb, int qpw, const BatchMap bm,
                                                  const int *__restrict__ offs,
                                                  const int *__restrict__ wcnt,
                                                  uint32_t *__restrict__ list) {
    extern __shared__ int lds[];
    int *base = lds;          // [nb] first position of this work-group's entries per list
    int *rank = lds + nb;     // [nb] entries placed so far per list
    const int w = blockIdx.x, g = blockIdx.y, nW = gridDim.x;
    const int *pre = wcnt + ((int64_t)g * nW + w) * nb;
    for (int b = threadIdx.x; b < nb; b += 256) {
        base[b] = offs[g * nb + b] + pre[b];
        rank[b] = 0;
    }
    __syncthreads();
    const int64_t i0 = (int64_t)w * qpw;
    for (int e = threadIdx.x; e < qpw * k; e += 256) {
        const int64_t i = i0 + e / k;
        const int s = e % k;
        const int id = entry_block(ids, C, G, k, nb, bm, g, i, s);
        if (id < 0) continue;
        const int r = atomicAdd(&rank[id], 1);
        list[base[id] + r] = ((uint32_t)i << 5) | (uint32_t)s;
    }
}

// One work-group of 1024 threads scans all lists.
__global__ __launch_bounds__(1024) void k3_scan(const int *__restrict__ counts, int nlists,
                                                int *__restrict__ offs, int *__restrict__ toff,
                                                int *__restrict__ total, int *__restrict__ items) {
    __shared__ int sc[1024], st[1024];
    const int tid = threadIdx.x;
    const int per = (nlists + 1023) / 1024;
    const int beg = min(tid * per, nlists), end = min(beg + per, nlists);
    int c_sum = 0, t_sum = 0;
    for (int l = beg; l < end; ++l) {
        const int c = counts[l];
        c_sum += c;
        t_sum += (c + kK4Queries - 1) / kK4Queries;
    }
    sc[tid] = c_sum;
    st[tid] = t_sum;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int a = tid >= off ? sc[tid - off] : 0;
        const int b = tid >= off ? st[tid - off] : 0;
        __syncthreads();
        sc[tid] += a;
        st[tid] += b;
        __syncthreads();
    }
    int ec = sc[tid] - c_sum, et = st[tid] - t_sum;
    for (int l = beg; l < end; ++l) {
        const int c = counts[l];
        const int nt = (c + kK4Queries - 1) / kK4Queries;
        offs[l] = ec;
        toff[l] = et;
        for (int t = 0; t < nt; ++t) items[et + t] = l;   // tile -> list table for K4
        ec += c;
        et += nt;
    }
    if (tid == 1023) {
        offs[nlists] = sc[1023];
        toff[nlists] = st[1023];
        *total = st[1023];
    }
}

// Bucket of K4 work item u: its group and the query window of its middle entry.
__device__ __forceinline__ int tile_bucket(int u, const int *offs, const int *toff,
                                           const int *items, const uint32_t *list, int nb,
                                           int sh, int nw) {
    const int li = items[u];
    const int first = offs[li] + (u - toff[li]) * kK4Queries;
    const int mid = first + min(kK4Queries, offs[li + 1] - first) / 2;
    return (li / nb) * nw + (int)((list[mid] >> 5) >> sh);
}

// Histogram of the buckets of items [w*kK3Tiles, (w+1)*kK3Tiles), zeros included.
__global__ __launch_bounds__(256) void k3_tile_count(const int *__restrict__ offs,
                                                     const int *__restrict__ toff,
                                                     const int *__restrict__ total,
                                                     const int *__restrict__ items,
                                                     const uint32_t *__restrict__ list, int nb,
                                                     int sh, int nw, int nbk,
                                                     int *__restrict__ tcnt) {
    __shared__ int lds_h[kK3Buckets];
    for (int b = threadIdx.x; b < nbk; b += 256) lds_h[b] = 0;
    __syncthreads();
    const int u0 = blockIdx.x * kK3Tiles, u1 = min(u0 + kK3Tiles, *total);
    for (int u = u0 + (int)threadIdx.x; u < u1; u += 256)
        atomicAdd(&lds_h[tile_bucket(u, offs, toff, items, list, nb, sh, nw)], 1);
    __syncthreads();
    int *dst = tcnt + (int64_t)blockIdx.x * nbk;
    for (int b = threadIdx.x; b < nbk; b += 256) dst[b] = lds_h[b];
}

// One work-group of 1024 threads: tcnt[w][b] <- (items in buckets < b) + (items of
// bucket b in work-groups < w).  Thread t owns a contiguous range of buckets.
__global__ __launch_bounds__(1024) void k3_tile_scan(int *__restrict__ tcnt, int nW, int nbk) {
    __shared__ int sc[1024];
    const int tid = threadIdx.x;
    const int per = (nbk + 1023) / 1024;
    const int beg = min(tid * per, nbk), end = min(beg + per, nbk);
    int sum = 0;
    for (int b = beg; b < end; ++b)
        for (int w = 0; w < nW; ++w) sum += tcnt[(int64_t)w * nbk + b];
    sc[tid] = sum;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int a = tid >= off ? sc[tid - off] : 0;
        __syncthreads();
        sc[tid] += a;
        __syncthreads();
    }
    int run = sc[tid] - sum;
    for (int b = beg; b < end; ++b)
        for (int w = 0; w < nW; ++w) {
            int *p = tcnt + (int64_t)w * nbk + b;
            const int c = *p;
            *p = run;
            run += c;
        }
}

// Each work-group places its items at their bucket's base plus a rank in LDS (the
// order inside one bucket and work-group follows LDS atomic timing; no result
// depends on the run order).
__global__ __launch_bounds__(256) void k3_tile_scatter(const int *__restrict__ offs,
                                                       const int *__restrict__ toff,
                                                       const int *__restrict__ total,
                                                       const int *__restrict__ items,
                                                       const uint32_t *__restrict__ list, int nb,
                                                       int sh, int nw, int nbk,
                                                       const int *__restrict__ tcnt,
                                                       int *__restrict__ order) {
    __shared__ int lds_base[kK3Buckets];
    const int *src = tcnt + (int64_t)blockIdx.x * nbk;
    for (int b = threadIdx.x; b < nbk; b += 256) lds_base[b] = src[b];
    __syncthreads();
    const int u0 = blockIdx.x * kK3Tiles, u1 = min(u0 + kK3Tiles, *total);
    for (int u = u0 + (int)threadIdx.x; u < u1; u += 256)
        order[atomicAdd(&lds_base[tile_bucket(u, offs, toff, items, list, nb, sh, nw)], 1)] = u;
}

int64_t k3_tile_groups(int64_t max_items) { return (max_items + kK3Tiles - 1) / kK3Tiles; }

int64_t k4_max_items(int64_t C, int G, int k, int nb) {
    const int64_t entries = C * G * k;
    const int64_t lists = (int64_t)G * nb;
    return (entries + kK4Queries - 1) / kK4Queries + (lists < entries ? lists : entries);
}

int k3_queries_per_group(int64_t C, int G) {
    int qpw = kK3Queries;
    while (qpw > kK3MinQueries && ((C + qpw - 1) / qpw) * G < kK3TargetGroups) qpw >>= 1;
    return qpw;
}

int k3_num_groups(int64_t C, int G) {
    const int qpw = k3_queries_per_group(C, G);
    return (int)((C + qpw - 1) / qpw);
}

hipError_t launch_k3_schedule(const int32_t *ids, int64_t C, int G, int k, int nb,
                              const SchedBuffers &sb, const BatchMap &bm, hipStream_t s) {
    const int nlists = G * nb;
    const int qpw = k3_queries_per_group(C, G);
    const int nW = k3_num_groups(C, G);
    hipError_t e;
    const dim3 grid((unsigned)nW, (unsigned)G);
    hipLaunchKernelGGL(k3_count, grid, dim3(256), nb * sizeof(int), s, ids, C, G, k, nb, qpw, bm,
                       sb.wcnt);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k3_colscan, dim3((unsigned)((nlists + 255) / 256)), dim3(256), 0, s,
                       sb.wcnt, G, nb, nW, sb.counts);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k3_scan, dim3(1), dim3(1024), 0, s, sb.counts, nlists, sb.offs, sb.toff,
                       sb.total, sb.items);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k3_scatter, grid, dim3(256), 2 * nb * sizeof(int), s, ids, C, G, k, nb, qpw,
                       bm, sb.offs, sb.wcnt, sb.list);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    // K4's run order: query windows of 2^sh rows, the smallest (at least 512) for
    // which the G * (windows) buckets fit in kK3Buckets.
    int sh = 9;
    while ((int64_t)G * ((C + (1ll << sh) - 1) >> sh) > kK3Buckets) ++sh;
    const int nw = (int)((C + (1ll << sh) - 1) >> sh);
    const int nbk = G * nw;
    const int64_t nTW = k3_tile_groups(k4_max_items(C, G, k, nb));
    if (nTW == 0 || C <= kK3NoOrderQueries) return hipSuccess;
    hipLaunchKernelGGL(k3_tile_count, dim3((unsigned)nTW), dim3(256), 0, s, sb.offs, sb.toff,
                       sb.total, sb.items, sb.list, nb, sh, nw, nbk, sb.tcnt);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k3_tile_scan, dim3(1), dim3(1024), 0, s, sb.tcnt, (int)nTW, nbk);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k3_tile_scatter, dim3((unsigned)nTW), dim3(256), 0, s, sb.offs, sb.toff,
                       sb.total, sb.items, sb.list, nb, sh, nw, nbk, sb.tcnt, sb.order);
    return hipGetLastError();
}

}  // namespace msa
