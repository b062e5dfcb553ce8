// msa_dense.hip -- the main branch of sequences of at most k blocks.
//
// A query keeps its own block and the k-1 best of the blocks before it
// ("MiniMax M3 算力省 20 倍", §二 Index Branch and §三 item 4: the local block keeps
// its slot).  When a sequence has at most k blocks, every query's causal blocks are
// all kept whatever the index scores, so its selection is blocks 0 .. b(i) and
// its attention over them is dense causal GQA attention -- the case in which MSA
// is GQA ("MiniMax-M3上架DEVUP…": MSA extends GQA; §二 Main Branch: exact softmax
// over the selected tokens).  Such sequences need neither the index branch nor the
// KV-outer attention's partials: one kernel attends each query tile over its
// blocks with an online softmax and writes the outputs, and the ids 0 .. b(i)
// directly.
//
// Work-group = (sequence, group g, tile of 128/R consecutive queries, all in one
// 128-token block b).  Each wave holds 32 MFMA columns (32/R queries x R heads) of
// the tile; for key blocks 0 .. b in order, K and V^T of the block are staged in
// LDS once for the work-group (as in K4), and each wave computes S^T = K Q^T, folds
// the block into its running maximum M and sum l (o <- 2^(M - M') o, scores
// exponentiated against M'), and accumulates O^T += V^T P^T in fp32.  out = o / l.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

// Staging of one key block for the whole work-group (256 threads), K straight into
// LDS and V transposed through registers.  Keys past `last` (the partial last block
// of a sequence) re-read key `last`: they lie past every query of the sequence, so
// their scores are masked and their probabilities are exactly 0, and the rows read
// are the sequence's own (finite) rows.
//
// K: LDS row p holds key k_lds_row<false>(p) (bits 2 and 3 swapped, an involution)
// in the swz<D/8> layout, as K4 reads it; one wave instruction fills 1 KB, lane l
// the bytes [16 l, 16 l + 16), fetching the global chunk that the swizzle puts there.
template <int D>
__device__ __forceinline__ void stage_k_direct(char *lds_k, const char *src, int stride_bytes,
                                               int last, int tid) {
    constexpr int CPR = D / 8;
    constexpr int kSegs = kBlock * CPR * 16 / 1024;
    constexpr int kMask = (CPR < 16 ? CPR : 16) - 1;
    const int lane = tid % kWave, wave = tid / kWave;
#pragma unroll
    for (int it = 0; it < kSegs / 4; ++it) {
        const int seg = it * 4 + wave;
        const int pos = seg * 1024 + lane * 16;
        const int prow = pos / (CPR * 16);
        const int chunk = ((pos / 16) % CPR) ^ (prow & kMask);
        const int key = min(k_lds_row<false>(prow), last);
        __builtin_amdgcn_global_load_lds(src + (uint32_t)(key * stride_bytes + chunk * 16),
                                         (lds_ptr_t)(lds_k + seg * 1024), 16, 0, 0);
    }
}

// V^T in the swz_vt layout: thread (c, kq) loads chunk c (d = 8c .. 8c + 7) of keys
// 4kq .. 4kq + 3 and writes, for each of its 8 d, those 4 keys as one 8-byte word
// (halves picked with byte permutes).
template <int D>
struct VStageT {
    static constexpr int CPR = D / 8;
    static constexpr int kQuadsPerIter = 256 / CPR;
    static constexpr int kIters = (kBlock / 4) / kQuadsPerIter;
    u32x4 vr[kIters][4];

    __device__ __forceinline__ void load(const char *src, int stride_bytes, int last, int tid) {
        const int c = tid % CPR;
#pragma unroll
        for (int it = 0; it < kIters; ++it) {
            const int kq = tid / CPR + it * kQuadsPerIter;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                vr[it][kk] = load16(src + (uint32_t)(min(4 * kq + kk, last) * stride_bytes + c * 16));
        }
    }

    __device__ __forceinline__ void store(char *lds_vt, int tid) const {
        const int c = tid % CPR;
#pragma unroll
        for (int it = 0; it < kIters; ++it) {
            const int key0 = 4 * (tid / CPR + it * kQuadsPerIter);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int w = e >> 1;
                // low halves (even e) or high halves (odd e) of two words, as one word
                const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                const uint32_t lo = __builtin_amdgcn_perm(vr[it][1][w], vr[it][0][w], sel);
                const uint32_t hi = __builtin_amdgcn_perm(vr[it][3][w], vr[it][2][w], sel);
                store8(lds_vt + swz_vt(8 * c + e, key0 >> 3) + ((key0 >> 2) & 1) * 8,
                       u32x2{lo, hi});
            }
        }
    }
};

// Running-maximum slack (log2 units): a block moves the maximum only when some
// column of the wave exceeds it by more than this, so most blocks skip the rescale
// of o; probabilities then stay below 2^8, far inside fp32 and bf16 range, and
// out = o / l is unchanged (o and l share the same reference maximum).
constexpr float kMaxSlack = 8.0f;

// One key block for a wave's 32 columns: the core of K4's attention pass (same
// operand layouts and relabelled contraction index), with the block's softmax taken
// against the running maximum instead of the block's own.
//   nmt  : M-tiles (32 keys each) computed, 1..4, wave-uniform; the others lie past
//          every query of the wave and get probability 0 with no MFMA work
//   mask : the queries' own block: keys past the column's query are masked
//   rel  : the column's query position minus the block's first token
//   rmin : the smallest rel of the wave (wave-uniform)
//   first: the sequence's first block (o, l still zero; no rescale)
//   o, M, l : the running fp32 output (unnormalised), maximum (scaled, log2 units)
//             and sum of the column
template <int D>
__device__ __forceinline__ void dense_block(const char *lds_k, const char *lds_vt,
                                            const bf16x8 (&qb)[D / 16], int rel, int rmin, int nmt,
                                            bool mask, bool first, float scale_log2, int lane,
                                            f32x16 (&o)[D / 32], float &M, float &l) {
    constexpr int KS = D / 16;
    constexpr int CPR = D / 8;
    constexpr int MD = D / 32;
    const int hf = lane >> 5, l32 = lane & 31;
    f32x16 sc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        sc[mt] = f32x16{};
        if (mt < nmt) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 a = as_bf16x8(load16(lds_k + swz<CPR>(mt * 32 + l32, 2 * ks + hf)));
                sc[mt] = mfma32(a, qb[ks], sc[mt]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if (mask) {
        // register r of M-tile mt holds key 32mt + 16(ip/2) + 8hf + 4(ip%2) + jj
        const int lim = rel - 8 * hf;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            if (mt >= nmt || 32 * mt + 31 <= rmin) continue;   // skipped, or all visible
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ip = r >> 2, jj = r & 3;
                const int key = 32 * mt + 16 * (ip >> 1) + 4 * (ip & 1) + jj;   // minus 8hf
                if (key > lim) sc[mt][r] = -INFINITY;
            }
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
        if (mt < nmt)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[mt][r]);
    mx = fmaxf(mx, xor_shfl(mx, 32));
    // key 0 of every block up to the query's own is visible, so mx is finite
    const float ms = mx * scale_log2;
    const bool grow = first || __ballot(ms > M + kMaxSlack) != 0;
    const float Mn = grow ? fmaxf(M, ms) : M;
    const float alpha = __builtin_amdgcn_exp2f(M - Mn);   // 1 when M stays; 0 on the first block
    // skipped M-tiles keep their zero scores as probabilities 0
    float sum = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
        if (mt < nmt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(fmaf(sc[mt][r], scale_log2, -Mn));
                sc[mt][r] = p;
                sum += p;
            }
    sum += xor_shfl(sum, 32);
    l = fmaf(l, alpha, sum);
    M = Mn;
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
#pragma unroll
    for (int md = 0; md < MD; ++md) {
        if (grow && !first) {
#pragma unroll
            for (int e = 0; e < 16; ++e) o[md][e] *= alpha;
        }
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) {
            if (kt < 2 * nmt) {
                const bf16x8 a = as_bf16x8(load16(lds_vt + swz_vt(md * 32 + l32, 2 * kt + hf)));
                o[md] = mfma32(a, pb[kt], o[md]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int D, int R>
__global__ __launch_bounds__(256, 2) void kd_dense(const uint16_t *__restrict__ q,
                                                   const uint16_t *__restrict__ kx,
                                                   const uint16_t *__restrict__ vx,
                                                   uint16_t *__restrict__ out,
                                                   int32_t *__restrict__ ids, const DenseTable t,
                                                   int H, int G, int kslots, float scale_log2) {
    __shared__ __attribute__((aligned(16))) char lds_k[kBlock * D * 2];
    __shared__ __attribute__((aligned(16))) char lds_vt[D * kBlock * 2];
    constexpr int QPW = 32 / R;          // queries per wave
    constexpr int TILE = 4 * QPW;        // queries per work-group (divides 128)
    const int g = (int)(blockIdx.x % G);
    const int tile = (int)(blockIdx.x / G);
    // the sequence of this tile: the last member whose first tile is <= tile
    int m = 0, hi = t.n - 1;
    while (m < hi) {
        const int mid = (m + hi + 1) / 2;
        if (t.tile_off[mid] <= tile) m = mid;
        else hi = mid - 1;
    }
    const int P = t.prefix[m], L = t.len[m];
    const int i0 = P + (tile - t.tile_off[m]) * TILE;   // first query of the tile
    const int b = i0 / kBlock;                          // the tile's own block
    const int tid = threadIdx.x, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int hf = lane >> 5, l32 = lane & 31;
    const int a = l32 / R, h = l32 % R;
    const int qw = i0 + wave * QPW;                      // the wave's first query
    const int i = qw + a;                                // this column's query
    const bool act = i < L;
    // rows of the column's query in q / out / ids; an inactive column reads the
    // tile's first query row and its result is discarded
    const int64_t row = (int64_t)t.q_row0[m] + ((act ? i : i0) - P);
    const int64_t hh = (int64_t)g * R + h;
    bf16x8 qb[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
        qb[ks] = as_bf16x8(load16(q + (row * H + hh) * D + (2 * ks + hf) * 8));
    f32x16 o[D / 32];
#pragma unroll
    for (int md = 0; md < D / 32; ++md) o[md] = f32x16{};
    float M = -INFINITY, l = 0.0f;
    const int kv_row_bytes = G * D * 2;
    const int64_t kv0 = (int64_t)t.kv_row0[m];
    for (int kb = 0;; ++kb) {
        if (kb > 0) __syncthreads();                     // the previous block is read
        {
            const int last = min(kBlock, L - kb * kBlock) - 1;
            const int64_t off = ((kv0 + (int64_t)kb * kBlock) * G + g) * D;
            // the staging addresses are recomputed per block (an opaque copy of the
            // thread index), not held across the loop beside the running output
            int stid = tid;
            asm volatile("" : "+v"(stid));
            stage_k_direct<D>(lds_k, reinterpret_cast<const char *>(kx + off), kv_row_bytes, last,
                              stid);
            VStageT<D> vs;
            vs.load(reinterpret_cast<const char *>(vx + off), kv_row_bytes, last, stid);
            vs.store(lds_vt, stid);
            __builtin_amdgcn_s_waitcnt(0);               // the direct K loads have landed
        }
        __syncthreads();
        const bool own = kb == b;
        const int rmin = qw - kb * kBlock;
        const int nmt = own ? (rmin + QPW - 1) / 32 + 1 : 4;
        dense_block<D>(lds_k, lds_vt, qb, i - kb * kBlock, rmin, nmt, own, kb == 0, scale_log2, lane,
                       o, M, l);
        if (own) break;
    }
    // ids of the column's query: every block 0 .. b, ascending, then -1
    if (ids && act && hf == 0)
        for (int s = h; s < kslots; s += R) ids[(row * G + g) * kslots + s] = s <= b ? s : -1;
    // out = o / l, packed as in K4: lane halves swapped so that each lane holds 8
    // consecutive d values (chunk 4(u/2) + 2(u%2) + hf of the row in w[u])
    const float inv = 1.0f / l;
#pragma unroll
    for (int md = 0; md < D / 32; ++md) {
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
            const int r0 = 8 * q2;
            const uint32_t a0 = pack_bf16x2(o[md][r0 + 0] * inv, o[md][r0 + 1] * inv);
            const uint32_t a1 = pack_bf16x2(o[md][r0 + 2] * inv, o[md][r0 + 3] * inv);
            const uint32_t b0 = pack_bf16x2(o[md][r0 + 4] * inv, o[md][r0 + 5] * inv);
            const uint32_t b1 = pack_bf16x2(o[md][r0 + 6] * inv, o[md][r0 + 7] * inv);
            const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
            if (act)
                store16(out + (row * H + hh) * D + 8 * (4 * md + 2 * q2 + hf),
                        u32x4{s0[0], s1[0], s0[1], s1[1]});
        }
    }
}

template <int D, int R>
static hipError_t kd_dispatch(const uint16_t *q, const uint16_t *kx, const uint16_t *vx,
                              uint16_t *out, int32_t *ids, const DenseTable &t, int H, int G,
                              int k, float sl2, hipStream_t s) {
    const int64_t grid = (int64_t)t.tile_off[t.n] * G;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((kd_dense<D, R>), dim3((unsigned)grid), dim3(256), 0, s, q, kx, vx, out, ids,
                       t, H, G, k, sl2);
    return hipGetLastError();
}

int dense_tile_queries(int H, int G) { return 4 * (32 / (H / G)); }

hipError_t launch_kd_dense(const uint16_t *q, const uint16_t *kx, const uint16_t *vx,
                           uint16_t *out, int32_t *ids, const DenseTable &t, int H, int G, int d,
                           int k, float scale, hipStream_t s) {
    const float sl2 = scale * kLog2e;
    const int R = H / G;
#define KD_CASE(dd, rr) \
    if (d == dd && R == rr) return kd_dispatch<dd, rr>(q, kx, vx, out, ids, t, H, G, k, sl2, s);
    KD_CASE(64, 1) KD_CASE(64, 2) KD_CASE(64, 4) KD_CASE(64, 8) KD_CASE(64, 16) KD_CASE(64, 32)
    KD_CASE(128, 1) KD_CASE(128, 2) KD_CASE(128, 4) KD_CASE(128, 8) KD_CASE(128, 16) KD_CASE(128, 32)
#undef KD_CASE
    return hipErrorInvalidValue;
}

}  // namespace msa
