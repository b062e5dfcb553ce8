// msa_attn.hip -- main branch: exact softmax attention over the selected blocks
// ("MiniMax M3 算力省 20 倍", §二 Main Branch: standard softmax attention over the
// tokens of the selected blocks only; §四 Kernel: KV-outer iteration that gathers
// the queries of each KV block into matrix-core tiles, pre-sized hot tiles, and a
// two-phase combine of partial results without atomics;
// "MiniMax-M3上架DEVUP…": no approximation inside a selected block).
//
// K4  (prefill, KV-outer): one work item = one (group g, KV block j) list slice of
//     up to 64 (query, slot) entries.  K_j and V_j of KV head g are staged once in
//     LDS (V transposed); every wave then takes 32 MFMA columns = 32/R queries x R
//     heads of the group, gathers their q rows straight into MFMA registers,
//     computes S^T = K Q^T, the block-local softmax (causal mask only in the query's
//     own block), O^T = V^T P^T, and writes the normalised partial o (bf16) and its
//     log2-sum-exp (fp32) to the entry's own (query, head, slot) location.
// K4d (decode, split over slots): one work item per (sequence, group, slot).
// K5  (combine, both paths): per (query, head) the partials of its valid slots are
//     merged with the log-sum-exp rule  out = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M),
//     M = max_s lse_s -- the merge that keeps the softmax exact.
//
// Contraction-index relabelling: the K rows fed as the A operand of S^T are
// permuted (pi below) so that the S^T accumulators of a lane, read 8 at a time,
// are exactly the P^T B operand of the next MFMA for 8 CONSECUTIVE keys; V^T then
// serves its A operand with one 16-byte LDS read.  No register shuffles are needed
// between the two products.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

// Key offset (within a 32-key M-tile) of A-operand row m.
__device__ __forceinline__ int k_row_perm(int m) {
    return 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}

// One pass of 32 columns of a wave over a staged block.  Lane column = l % 32.
//   qrow   : the column's q row (d values), read only when `active`
//   qpos   : the column's token position (its causal limit in its own block)
//   j      : the staged KV block
//   orow / lse_dst : destination of the column's partial (written when active)
template <int D>
__device__ __forceinline__ void attend_pass(const char *lds_k, const char *lds_vt, int j,
                                            const uint16_t *qrow, bool active, int64_t qpos,
                                            uint16_t *orow, float *lse_dst, float scale_log2,
                                            int lane) {
    constexpr int KS = D / 16;   // K-steps of S^T over d
    constexpr int CPR = D / 8;
    constexpr int MD = D / 32;   // M-tiles of O^T over d
    const int hf = lane >> 5, l32 = lane & 31;

    bf16x8 qb[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qb[ks] = as_bf16x8(active ? load16(qrow + (2 * ks + hf) * 8) : u32x4{0, 0, 0, 0});

    const int prow = k_row_perm(l32);
    f32x16 sc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        sc[mt] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 a = as_bf16x8(load16(lds_k + swz<CPR>(mt * 32 + prow, 2 * ks + hf)));
            sc[mt] = mfma32(a, qb[ks], sc[mt]);
        }
    }
    // scale to the log2 domain; causal mask inside the query's own block
    const bool local = active && (qpos / kBlock == j);
    const int lim = (int)(qpos - (int64_t)j * kBlock);
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int ip = r >> 2, jj = r & 3;
            const int key = 32 * mt + 16 * (ip >> 1) + 8 * hf + 4 * (ip & 1) + jj;
            float v = sc[mt][r] * scale_log2;
            if (local && key > lim) v = -INFINITY;
            sc[mt][r] = v;
            mx = fmaxf(mx, v);
        }
    }
    mx = fmaxf(mx, xor_shfl(mx, 32));
    float sum = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = __builtin_amdgcn_exp2f(sc[mt][r] - mx);
            sc[mt][r] = p;
            sum += p;
        }
    }
    sum += xor_shfl(sum, 32);
    // P^T as B operand: K-step kt holds keys 16kt + 8hf + e = registers 8(kt%2)+e of M-tile kt/2
    bf16x8 pb[8];
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
        const int mt = kt >> 1, r0 = 8 * (kt & 1);
        u32x4 w;
        w[0] = pack_bf16x2(sc[mt][r0 + 0], sc[mt][r0 + 1]);
        w[1] = pack_bf16x2(sc[mt][r0 + 2], sc[mt][r0 + 3]);
        w[2] = pack_bf16x2(sc[mt][r0 + 4], sc[mt][r0 + 5]);
        w[3] = pack_bf16x2(sc[mt][r0 + 6], sc[mt][r0 + 7]);
        pb[kt] = as_bf16x8(w);
    }
    f32x16 o[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md) {
        o[md] = f32x16{};
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) {
            const bf16x8 a = as_bf16x8(load16(lds_vt + swz<16>(md * 32 + l32, 2 * kt + hf)));
            o[md] = mfma32(a, pb[kt], o[md]);
        }
    }
    if (!active) return;
    const float inv = 1.0f / sum;
#pragma unroll
    for (int md = 0; md < MD; ++md) {
#pragma unroll
        for (int ip = 0; ip < 4; ++ip) {
            const int d0 = 32 * md + 8 * ip + 4 * hf;
            store8(orow + d0, u32x2{pack_bf16x2(o[md][4 * ip + 0] * inv, o[md][4 * ip + 1] * inv),
                                    pack_bf16x2(o[md][4 * ip + 2] * inv, o[md][4 * ip + 3] * inv)});
        }
    }
    if (hf == 0) *lse_dst = mx + __log2f(sum);
}

// ---------------------------------------------------------------------------
// K4: KV-outer sparse attention over the scheduled lists.
// ---------------------------------------------------------------------------
template <int D, int R>
__global__ __launch_bounds__(256) void k4_kv_outer(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kx,
    const uint16_t *__restrict__ vx, const int *__restrict__ offs, const int *__restrict__ toff,
    const int *__restrict__ total, const uint32_t *__restrict__ list, int nlists, int nb,
    int64_t L, int64_t q0, int H, int G, int kslots, float scale_log2, uint16_t *__restrict__ po,
    float *__restrict__ plse) {
    __shared__ __attribute__((aligned(16))) char lds_k[kBlock * D * 2];
    __shared__ __attribute__((aligned(16))) char lds_vt[D * kBlock * 2];
    const int per = gridDim.x / 8;
    const int x = (blockIdx.x % 8) * per + blockIdx.x / 8;   // XCD-contiguous items
    if (x >= *total) return;
    int lo = 0, hi = nlists;                                 // toff[lo] <= x < toff[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (toff[mid] <= x) lo = mid;
        else hi = mid;
    }
    const int li = lo;
    const int g = li / nb, j = li % nb;
    const int t = x - toff[li];
    const int begin = offs[li] + t * kK4Queries;
    const int cnt = min(kK4Queries, offs[li + 1] - begin);

    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const int64_t kv_row_bytes = (int64_t)G * D * 2;
    const char *ksrc = reinterpret_cast<const char *>(kx + ((int64_t)j * kBlock * G + g) * D);
    const char *vsrc = reinterpret_cast<const char *>(vx + ((int64_t)j * kBlock * G + g) * D);
    const int nrows = (int)min<int64_t>(kBlock, L - (int64_t)j * kBlock);
    stage_rows<D / 8>(lds_k, ksrc, kv_row_bytes, nrows, tid);
    stage_v_transposed<D>(lds_vt, vsrc, kv_row_bytes, nrows, tid);
    __syncthreads();

    constexpr int QPW = 32 / R;   // queries per wave pass
    const int l32 = lane & 31;
    const int a = l32 / R, h = l32 % R;
    for (int base = wave * QPW; base < cnt; base += 4 * QPW) {
        const int e = base + a;
        const bool active = e < cnt;
        const uint32_t entry = active ? list[begin + e] : 0u;
        const int64_t il = entry >> 5;
        const int s = entry & 31;
        const int64_t i = q0 + il;
        const int64_t hh = (int64_t)g * R + h;
        const uint16_t *qrow = q + (i * H + hh) * D;
        const int64_t prow = (il * H + hh) * kslots + s;
        attend_pass<D>(lds_k, lds_vt, j, qrow, active, i, po + prow * D, plse + prow, scale_log2,
                       lane);
    }
}

template <int D, int R>
static hipError_t k4_dispatch(const uint16_t *q, const uint16_t *kx, const uint16_t *vx,
                              const SchedBuffers &sb, int nb, int64_t L, int64_t q0, int64_t C,
                              int H, int G, int k, float scale_log2, uint16_t *po, float *plse,
                              hipStream_t s) {
    const int64_t grid = round_up(k4_max_items(C, G, k, nb), 8);
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((k4_kv_outer<D, R>), dim3((unsigned)grid), dim3(256), 0, s, q, kx, vx,
                       sb.offs, sb.toff, sb.total, sb.list, G * nb, nb, L, q0, H, G, k,
                       scale_log2, po, plse);
    return hipGetLastError();
}

hipError_t launch_k4_kv_outer(const uint16_t *q, const uint16_t *kx, const uint16_t *vx,
                              const SchedBuffers &sb, int nb, int64_t L, int64_t q0, int64_t C,
                              int H, int G, int d, int k, float scale, uint16_t *po, float *plse,
                              hipStream_t s) {
    const float sl2 = scale * kLog2e;
    const int R = H / G;
#define K4_CASE(dd, rr) \
    if (d == dd && R == rr) return k4_dispatch<dd, rr>(q, kx, vx, sb, nb, L, q0, C, H, G, k, sl2, po, plse, s);
    K4_CASE(64, 1) K4_CASE(64, 2) K4_CASE(64, 4) K4_CASE(64, 8) K4_CASE(64, 16) K4_CASE(64, 32)
    K4_CASE(128, 1) K4_CASE(128, 2) K4_CASE(128, 4) K4_CASE(128, 8) K4_CASE(128, 16) K4_CASE(128, 32)
#undef K4_CASE
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// K4d: decode, one work-group per (sequence, group, slot).
// ---------------------------------------------------------------------------
template <int D, int R>
__global__ __launch_bounds__(256) void k4d_split(const uint16_t *__restrict__ q,
                                                 const uint16_t *__restrict__ kc,
                                                 const uint16_t *__restrict__ vc,
                                                 const int32_t *__restrict__ ids,
                                                 const int32_t *__restrict__ seq_len,
                                                 int64_t Lmax, int H, int G, int kslots,
                                                 float scale_log2, uint16_t *__restrict__ po,
                                                 float *__restrict__ plse) {
    __shared__ __attribute__((aligned(16))) char lds_k[kBlock * D * 2];
    __shared__ __attribute__((aligned(16))) char lds_vt[D * kBlock * 2];
    const int64_t item = blockIdx.x;
    const int64_t n = item / ((int64_t)G * kslots);
    const int g = (int)((item / kslots) % G);
    const int s = (int)(item % kslots);
    const int j = ids[(n * G + g) * kslots + s];
    if (j < 0) return;
    const int64_t p = (int64_t)seq_len[n] - 1;
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const int64_t kv_row_bytes = (int64_t)G * D * 2;
    const int64_t row0 = (n * Lmax + (int64_t)j * kBlock) * G + g;
    const int nrows = (int)min<int64_t>(kBlock, Lmax - (int64_t)j * kBlock);
    stage_rows<D / 8>(lds_k, reinterpret_cast<const char *>(kc + row0 * D), kv_row_bytes, nrows, tid);
    stage_v_transposed<D>(lds_vt, reinterpret_cast<const char *>(vc + row0 * D), kv_row_bytes,
                          nrows, tid);
    __syncthreads();
    if (wave != 0) return;
    const int l32 = lane & 31;
    const bool active = l32 < R;
    const int64_t hh = (int64_t)g * R + (active ? l32 : 0);
    const int64_t prow = (n * H + hh) * kslots + s;
    attend_pass<D>(lds_k, lds_vt, j, q + (n * H + hh) * D, active, p, po + prow * D, plse + prow,
                   scale_log2, lane);
}

template <int D, int R>
static hipError_t k4d_dispatch(const uint16_t *q, const uint16_t *kc, const uint16_t *vc,
                               const int32_t *ids, const int32_t *seq_len, int N, int64_t Lmax,
                               int H, int G, int k, float sl2, uint16_t *po, float *plse,
                               hipStream_t s) {
    const int64_t grid = (int64_t)N * G * k;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((k4d_split<D, R>), dim3((unsigned)grid), dim3(256), 0, s, q, kc, vc, ids,
                       seq_len, Lmax, H, G, k, sl2, po, plse);
    return hipGetLastError();
}

hipError_t launch_k4d_split(const uint16_t *q, const uint16_t *kc, const uint16_t *vc,
                            const int32_t *ids, const int32_t *seq_len, int N, int64_t Lmax, int H,
                            int G, int d, int k, float scale, uint16_t *po, float *plse,
                            hipStream_t s) {
    const float sl2 = scale * kLog2e;
    const int R = H / G;
#define K4D_CASE(dd, rr) \
    if (d == dd && R == rr) return k4d_dispatch<dd, rr>(q, kc, vc, ids, seq_len, N, Lmax, H, G, k, sl2, po, plse, s);
    K4D_CASE(64, 1) K4D_CASE(64, 2) K4D_CASE(64, 4) K4D_CASE(64, 8) K4D_CASE(64, 16) K4D_CASE(64, 32)
    K4D_CASE(128, 1) K4D_CASE(128, 2) K4D_CASE(128, 4) K4D_CASE(128, 8) K4D_CASE(128, 16) K4D_CASE(128, 32)
#undef K4D_CASE
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// K5: combine.  D/8 threads per (query, head), 8 d values per thread.
// Slots are valid when 0 <= id < nb_lim (the same rule K3 used to build lists).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k5_combine(const uint16_t *__restrict__ po,
                                                  const float *__restrict__ plse,
                                                  const int32_t *__restrict__ ids, int64_t nq,
                                                  int H, int G, int kslots, int nb_lim,
                                                  uint16_t *__restrict__ out) {
    constexpr int TPH = D / 8;
    constexpr int PPW = 256 / TPH;
    const int64_t ih = (int64_t)blockIdx.x * PPW + threadIdx.x / TPH;
    if (ih >= nq * H) return;
    const int sub = threadIdx.x % TPH;
    const int64_t i = ih / H;
    const int h = (int)(ih % H);
    const int g = h / (H / G);
    const int32_t *idr = ids + (i * G + g) * kslots;
    const float *lr = plse + ih * kslots;
    float M = -INFINITY;
    for (int s = 0; s < kslots; ++s) {
        const int id = idr[s];
        if (id >= 0 && id < nb_lim) M = fmaxf(M, lr[s]);
    }
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float wsum = 0.0f;
    for (int s = 0; s < kslots; ++s) {
        const int id = idr[s];
        if (id < 0 || id >= nb_lim) continue;
        const float w = __builtin_amdgcn_exp2f(lr[s] - M);
        wsum += w;
        const u32x4 v = load16(po + (ih * kslots + s) * D + sub * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += w * bf16_to_f32(v[e] & 0xFFFFu);
            acc[2 * e + 1] += w * bf16_to_f32(v[e] >> 16);
        }
    }
    const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
    store16(out + ih * D + sub * 8, r);
}

hipError_t launch_k5_combine(const uint16_t *po, const float *plse, const int32_t *ids, int64_t nq,
                             int H, int G, int d, int k, int nb_lim, uint16_t *out,
                             hipStream_t s) {
    if (nq <= 0) return hipSuccess;
    const int64_t pairs = nq * H;
    if (d == 64) {
        hipLaunchKernelGGL((k5_combine<64>), dim3((unsigned)((pairs + 31) / 32)), dim3(256), 0, s,
                           po, plse, ids, nq, H, G, k, nb_lim, out);
    } else if (d == 128) {
        hipLaunchKernelGGL((k5_combine<128>), dim3((unsigned)((pairs + 15) / 16)), dim3(256), 0, s,
                           po, plse, ids, nq, H, G, k, nb_lim, out);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace msa
