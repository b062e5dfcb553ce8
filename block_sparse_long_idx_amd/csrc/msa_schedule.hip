// msa_schedule.hip -- K3: turn query-major selections into KV-block-major work
// ("MiniMax M3 算力省 20 倍", §四 Kernel: KV-outer iteration gathers the queries that
// picked each KV block; a scheduling kernel splits hot tiles ahead of time along the
// query dimension so no single work-group owns a block picked by almost every query;
// "MiniMax M3 的采用瓶颈…" §对建设者的影响: KV-block-major layout).
//
//   hist    count[g*nb + b]  += 1 for every valid (query, group, slot) entry
//   scan    offs = exclusive prefix of counts; toff = exclusive prefix of the number
//           of pre-sized tiles ceil(count / kK4Queries) per list; total tiles
//   scatter list[offs[l] + rank] = (query - q0) << 5 | slot
//
// Threads walk the entries slot-major and query-fastest, so a wave holds 64
// consecutive queries at one (group, slot).  Hot blocks (selected by nearly every
// query) then sit in the same slot of all 64 lanes and are counted with one
// atomic per wave (wave-aggregated leader atomics).  The order of entries inside a
// list depends on atomic timing, but no result does: every entry's partial is
// written to its own (query, head, slot) location.
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

// Adds 1 to ctr[key] for every lane with key >= 0 and returns each such lane's
// previous-count rank.  Lanes sharing the first active lane's key use one atomic.
__device__ __forceinline__ int aggregated_increment(int *ctr, int key) {
    const int lane = lane_id();
    const bool valid = key >= 0;
    const uint64_t act = __ballot(valid);
    if (act == 0) return 0;
    const int first = __ffsll((unsigned long long)act) - 1;
    const int lead = __shfl(key, first, kWave);
    const bool same = valid && key == lead;
    const uint64_t m = __ballot(same);
    int base = 0;
    if (lane == first) base = atomicAdd(&ctr[lead], (int)__popcll(m));
    base = __shfl(base, first, kWave);
    const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
    if (same) return base + rank;
    if (valid) return atomicAdd(&ctr[key], 1);
    return 0;
}

__device__ __forceinline__ int entry_key(const int32_t *ids, int64_t t, int64_t C, int G, int k,
                                         int nb, int64_t &i, int &s) {
    i = t % C;
    const int64_t gs = t / C;
    const int g = (int)(gs / k);
    s = (int)(gs % k);
    const int id = ids[(i * G + g) * k + s];
    return (id >= 0 && id < nb) ? g * nb + id : -1;   // ids outside [0, nb) are ignored
}

__global__ __launch_bounds__(256) void k3_hist(const int32_t *__restrict__ ids, int64_t C, int G,
                                               int k, int nb, int *__restrict__ counts) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    int key = -1;
    if (t < C * G * k) {
        int64_t i;
        int s;
        key = entry_key(ids, t, C, G, k, nb, i, s);
    }
    aggregated_increment(counts, key);
}

__global__ __launch_bounds__(256) void k3_scatter(const int32_t *__restrict__ ids, int64_t C, int G,
                                                  int k, int nb, const int *__restrict__ offs,
                                                  int *__restrict__ cursor,
                                                  uint32_t *__restrict__ list) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    int key = -1;
    int64_t i = 0;
    int s = 0;
    if (t < C * G * k) key = entry_key(ids, t, C, G, k, nb, i, s);
    const int rank = aggregated_increment(cursor, key);
    if (key >= 0) list[offs[key] + rank] = ((uint32_t)i << 5) | (uint32_t)s;
}

// One work-group of 1024 threads scans all lists.
__global__ __launch_bounds__(1024) void k3_scan(const int *__restrict__ counts, int nlists,
                                                int *__restrict__ offs, int *__restrict__ toff,
                                                int *__restrict__ cursor, int *__restrict__ total) {
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
        offs[l] = ec;
        toff[l] = et;
        cursor[l] = 0;
        ec += c;
        et += (c + kK4Queries - 1) / kK4Queries;
    }
    if (tid == 1023) {
        offs[nlists] = sc[1023];
        toff[nlists] = st[1023];
        *total = st[1023];
    }
}

int64_t k4_max_items(int64_t C, int G, int k, int nb) {
    const int64_t entries = C * G * k;
    const int64_t lists = (int64_t)G * nb;
    return (entries + kK4Queries - 1) / kK4Queries + (lists < entries ? lists : entries);
}

hipError_t launch_k3_schedule(const int32_t *ids, int64_t C, int G, int k, int nb,
                              const SchedBuffers &sb, hipStream_t s) {
    const int nlists = G * nb;
    hipError_t e = launch_fill_i32(sb.counts, nlists, 0, s);
    if (e != hipSuccess) return e;
    const int64_t entries = C * G * k;
    const unsigned grid = (unsigned)((entries + 255) / 256);
    if (entries > 0) {
        hipLaunchKernelGGL(k3_hist, dim3(grid), dim3(256), 0, s, ids, C, G, k, nb, sb.counts);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k3_scan, dim3(1), dim3(1024), 0, s, sb.counts, nlists, sb.offs, sb.toff,
                       sb.cursor, sb.total);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (entries > 0) {
        hipLaunchKernelGGL(k3_scatter, dim3(grid), dim3(256), 0, s, ids, C, G, k, nb, sb.offs,
                           sb.cursor, sb.list);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace msa
