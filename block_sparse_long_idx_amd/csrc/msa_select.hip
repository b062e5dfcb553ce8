// msa_select.hip -- K2: exp-free top-k block selection with the forced local block
// ("MiniMax M3 算力省 20 倍", §二 Index Branch: each GQA group picks its own top-k
// blocks and the query's own block is always picked; §三 item 4: that block keeps
// one of the k slots; §四 exp-free TopK: softmax keeps order, so raw scores are
// ranked directly and no exp is evaluated).
//
// One 64-lane wave per (query, group) row; kk = k - 1 competitors are kept next to
// the local block.  Ranking: larger score first, smaller block id on equal scores
// (float compares: -0 and +0 are equal).  Scores are compared as order-preserving
// 32-bit keys, so a selection threshold is found by counting, one key bit at a
// time, how many keys of the wave reach a candidate value (one ballot and one
// popcount per bit and register slot, no cross-lane shuffles).
//   1. the first 1024 scores of the row are loaded into registers (16 per lane);
//   2. tau = the kk-th largest lane maximum, truncated to its upper 16 bits: at
//      least kk of these scores reach tau, so every true top-kk score does too;
//   3. the scores >= tau go to a per-wave candidate list in LDS (about 17 on
//      random rows), in ascending block order;
//   4. the rest of the row is streamed once, 256 scores per lane-wide load, and a
//      score enters the list only if it beats the running threshold strictly (a
//      later block loses every tie against the list).  When the list would
//      outgrow 64 entries it is cut to its exact top kk, which raises the
//      threshold to the kk-th best score seen so far;
//   5. the exact top kk of the list, still in ascending block order, is written,
//      followed by the local block (the largest id).
// If step 3 would overflow the list (heavy ties), the exact top kk of the 1024
// register-held scores is taken instead (step 5's cut, applied to the registers).
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {
namespace {

constexpr int kRowsPerBlock = 4;   // one row per wave, 256 threads
constexpr int kHead = 1024;        // scores held in registers (16 per lane)
constexpr int kCap = 320;          // list entries per wave: >= 31 kept + 256 appended
constexpr int kSoft = 64;          // cut the list before it outgrows one entry per lane
constexpr int kStream = 4;         // 256-score groups loaded together when streaming

// Order-preserving key of a float (-0 counts as +0); never 0 for a non-NaN value,
// so 0 marks an absent score.
__device__ __forceinline__ uint32_t okey(float v) {
    const uint32_t u = __float_as_uint(v + 0.0f);
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ int mbcnt64(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

__device__ __forceinline__ int wave_count(bool p) { return __popcll(__ballot(p)); }

// Largest key value V (low `lo` bits zero) such that at least kk keys of the wave
// reach it: with lo = 0 this is the kk-th largest key exactly.
template <int NP>
__device__ __forceinline__ uint32_t kth_key(const uint32_t (&key)[NP], int kk, int lo) {
    uint32_t prefix = 0;
#pragma unroll
    for (int bit = 31; bit >= 0; --bit) {
        if (bit < lo) break;
        const uint32_t cand = prefix | (1u << bit);
        int c = 0;
#pragma unroll
        for (int j = 0; j < NP; ++j) c += wave_count(key[j] >= cand);
        if (c >= kk) prefix = cand;
    }
    return prefix;
}

// The per-wave candidate list: keys and block ids in ascending block order.
struct List {
    uint32_t *key;
    int32_t *id;
};

// Exact top kk of the list's cnt (>= kk) entries, kept in list order: every key
// above the kk-th largest V, then the first entries equal to V (smallest ids)
// until kk are taken.  Calls emit(position, id, key) once per kept entry,
// positions 0 .. kk-1 in ascending block order; returns V.
template <int NP, typename Emit>
__device__ __forceinline__ uint32_t top_of_list(List ls, int cnt, int kk, int lane, Emit emit) {
    uint32_t key[NP];
    int32_t id[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) {
        const int p = lane + kWave * j;
        key[j] = p < cnt ? ls.key[p] : 0u;
        id[j] = p < cnt ? ls.id[p] : 0;
    }
    const uint32_t V = kth_key<NP>(key, kk, 0);
    int gt = 0;
#pragma unroll
    for (int j = 0; j < NP; ++j) gt += wave_count(key[j] > V);
    const int need = kk - gt;          // entries equal to V still to take (>= 1)
    int eq_before = 0, kept_before = 0;
    bool keep[NP];
    int pos[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) {
        const uint64_t meq = __ballot(key[j] == V);
        keep[j] = key[j] > V || (key[j] == V && eq_before + mbcnt64(meq) < need);
        eq_before += __popcll(meq);
        const uint64_t mk = __ballot(keep[j]);
        pos[j] = kept_before + mbcnt64(mk);
        kept_before += __popcll(mk);
    }
    // every lane has read its entries before any is overwritten
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < NP; ++j)
        if (keep[j]) emit(pos[j], id[j], key[j]);
    return V;
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

}  // namespace

__global__ __launch_bounds__(256) void k2_select(const float *__restrict__ S, int nbp,
                                                 int64_t nrows, int G, int k, int64_t q0,
                                                 const int32_t *__restrict__ seq_len,
                                                 int64_t Lmax, int32_t *__restrict__ ids) {
    __shared__ uint32_t lkey[kRowsPerBlock][kCap];
    __shared__ int32_t lid[kRowsPerBlock][kCap];
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + wave;
    if (row >= nrows) return;
    int32_t *out = ids + row * k;
    int64_t pos;
    if (seq_len) {
        const int sl = seq_len[row / G];
        if (sl < 1 || sl > Lmax) {
            if (lane < k) out[lane] = -1;
            return;
        }
        pos = sl - 1;
    } else {
        pos = q0 + row / G;
    }
    const int bi = (int)(pos / kBlock);
    const int n = bi;                 // competitors: blocks 0 .. b(i)-1
    const int kk = k - 1;             // slots left after the local block
    if (kk == 0) {                    // k = 1: the local block alone
        if (lane == 0) out[0] = bi;
        return;
    }
    if (n <= kk) {
        if (lane < k) out[lane] = lane <= bi ? lane : -1;
        return;
    }
    const float *srow = S + row * nbp;
    const List ls{lkey[wave], lid[wave]};
    // 1. the head of the row: lane l holds scores 4(l + 64t) + e (16-byte loads;
    //    rows are 32-byte aligned and padded, so a load that starts below n stays
    //    inside the row)
    uint32_t hk[4][4];
    uint32_t lane_max = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int i0 = 4 * (lane + kWave * t);
        const f32x4 x = i0 < n ? __builtin_bit_cast(f32x4, load16_stream(srow + i0))
                               : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            hk[t][e] = i0 + e < n ? okey(x[e]) : 0u;
            lane_max = max(lane_max, hk[t][e]);
        }
    }
    // 2. tau from the lane maxima
    uint32_t lm[1] = {lane_max};
    const uint32_t tau = max(kth_key<1>(lm, kk, 16), 1u);
    // 3. head scores >= tau into the list, in block order (block 4(l + 64t) + e
    //    precedes everything of lanes above l and of later t)
    int cnt = 0;
    auto append4 = [&](const bool (&f)[4], const uint32_t (&key)[4], int i0) {
        uint64_t m[4];
        int below = 0, tot = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            m[e] = __ballot(f[e]);
            below += mbcnt64(m[e]);
            tot += __popcll(m[e]);
        }
        int own = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (f[e]) {
                const int p = cnt + below + own;
                ls.key[p] = key[e];
                ls.id[p] = i0 + e;
            }
            own += f[e] ? 1 : 0;
        }
        cnt += tot;
    };
    int head_cands = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) head_cands += wave_count(hk[t][e] >= tau);
    uint32_t thr;   // later scores enter the list only with a key > thr
    if (head_cands <= kCap) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            bool f[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) f[e] = hk[t][e] >= tau;
            append4(f, hk[t], 4 * (lane + kWave * t));
        }
        thr = tau;
    } else {
        // heavy ties: exact top kk of the head, ties to the smallest block
        uint32_t flat[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) flat[j] = hk[j / 4][j % 4];
        const uint32_t V = kth_key<16>(flat, kk, 0);
        int gt = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) gt += wave_count(flat[j] > V);
        const int need = kk - gt;
        int eq_before = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            bool eq[4], f[4];
            uint64_t m[4];
            int below = 0, tot = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                eq[e] = hk[t][e] == V;
                m[e] = __ballot(eq[e]);
                below += mbcnt64(m[e]);
                tot += __popcll(m[e]);
            }
            int own = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[e] = hk[t][e] > V || (eq[e] && eq_before + below + own < need);
                own += eq[e] ? 1 : 0;
            }
            eq_before += tot;
            append4(f, hk[t], 4 * (lane + kWave * t));
        }
        thr = V;
    }
    // 4. stream the rest of the row
    auto cut = [&]() {
        auto to_list = [&](int p, int32_t id, uint32_t key) {
            ls.key[p] = key;
            ls.id[p] = id;
        };
        wave_lds_sync();
        thr = cnt <= kWave ? top_of_list<1>(ls, cnt, kk, lane, to_list)
                           : top_of_list<kCap / kWave>(ls, cnt, kk, lane, to_list);
        cnt = kk;
    };
    for (int base = kHead; base < n; base += kStream * 4 * kWave) {
        f32x4 x[kStream];
#pragma unroll
        for (int u = 0; u < kStream; ++u) {
            const int i0 = base + 4 * (lane + kWave * u);
            x[u] = i0 < n ? __builtin_bit_cast(f32x4, load16_stream(srow + i0))
                          : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < kStream; ++u) {
            if (base + 4 * kWave * u >= n) break;
            const int i0 = base + 4 * (lane + kWave * u);
            uint32_t key[4];
            bool f[4];
            int tot = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                key[e] = i0 + e < n ? okey(x[u][e]) : 0u;
                f[e] = key[e] > thr;
                tot += wave_count(f[e]);
            }
            if (tot == 0) continue;
            if (cnt + tot > kSoft && cnt > kk) {
                cut();
#pragma unroll
                for (int e = 0; e < 4; ++e) f[e] = key[e] > thr;
            }
            append4(f, key, i0);
        }
    }
    // 5. exact top kk of the list, ascending ids, then the local block
    wave_lds_sync();
    auto to_out = [&](int p, int32_t id, uint32_t) { out[p] = id; };
    if (cnt <= kWave) top_of_list<1>(ls, cnt, kk, lane, to_out);
    else top_of_list<kCap / kWave>(ls, cnt, kk, lane, to_out);
    if (lane == 0) out[kk] = bi;
}

hipError_t launch_k2_select(const float *S, int nbp, int64_t nrows, int G, int k, int64_t q0,
                            const int32_t *seq_len, int64_t Lmax, int32_t *ids, hipStream_t s) {
    if (nrows <= 0) return hipSuccess;
    const int64_t grid = (nrows + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL(k2_select, dim3((unsigned)grid), dim3(256), 0, s, S, nbp, nrows, G, k, q0,
                       seq_len, Lmax, ids);
    return hipGetLastError();
}

}  // namespace msa
