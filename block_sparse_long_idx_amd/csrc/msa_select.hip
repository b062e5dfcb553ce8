// msa_select.hip -- K2: exp-free top-k block selection with the forced local block
// ("MiniMax M3 算力省 20 倍", §二 Index Branch: each GQA group picks its own top-k
// blocks and the query's own block is always picked; §三 item 4: that block keeps
// one of the k slots; §四 exp-free TopK: softmax keeps order, so raw scores are
// ranked directly and no exp is evaluated).
//
// One 64-lane wave per (query, group) row.  Scores and block ids are fused into
// one 64-bit key (order-preserving float bits in the high word, inverted id in
// the low word), so "larger score first, smaller id on ties" is plain unsigned
// order and every key is distinct.
//   1. each lane streams its share of the row (16-byte loads) and keeps its best
//      (score, index) with float compares (the first 1024 scores of a row stay in
//      registers for step 3);
//   2. a bitonic sort of the 64 lane-best keys across the wave gives tau, the
//      (k-1)-th largest lane best; every one of the true top k-1 keys is >= tau;
//   3. a second pass compacts the keys >= tau into a per-wave LDS list (in the
//      common case only a little more than k-1 of them);
//   4. a bitonic sort of that list yields the top k-1; a final ascending sort of
//      their ids, followed by the local block (the largest id), is written out.
// If more than 64 keys pass tau (heavy ties), a k-1 round exact fallback runs.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
    const uint32_t lo = __shfl_xor((uint32_t)v, m, kWave);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, kWave);
    return ((uint64_t)hi << 32) | lo;
}

// Bitonic sort of one value per lane across the 64-lane wave.
template <bool Desc, typename T>
__device__ __forceinline__ T wave_bitonic(T x, int lane) {
#pragma unroll
    for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            T y;
            if constexpr (sizeof(T) == 8) y = shfl_xor_u64(x, stride);
            else y = (T)__shfl_xor((uint32_t)x, stride, kWave);
            const bool lower = (lane & stride) == 0;
            const bool seg_desc = ((lane & size) == 0) == Desc;
            const bool keep_max = lower == seg_desc;
            x = keep_max ? (x > y ? x : y) : (x < y ? x : y);
        }
    }
    return x;
}

__device__ __forceinline__ uint64_t make_key(float v, int idx) {
    return ((uint64_t)float_order_key(v) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)idx);
}
__device__ __forceinline__ int key_id(uint64_t key) {
    return (int)(0xFFFFFFFFu - (uint32_t)key);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const uint64_t o = shfl_xor_u64(v, m);
        v = v > o ? v : o;
    }
    return v;
}

__global__ __launch_bounds__(256) void k2_select(const float *__restrict__ S, int nbp,
                                                 int64_t nrows, int G, int k, int64_t q0,
                                                 const int32_t *__restrict__ seq_len,
                                                 int64_t Lmax, int32_t *__restrict__ ids) {
    __shared__ uint64_t cand[4][64];
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int64_t row = (int64_t)blockIdx.x * 4 + wave;
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
    // Scores are read 4 per lane per step (16 bytes; rows are 32-byte aligned):
    // lane l owns elements 4(l + 64 v) + e, visited in increasing index order.
    // The first 1024 scores of a row stay in registers for step 3.
    constexpr int kVec = 4;                       // float4 loads per lane kept in registers
    f32x4 cache[kVec];
    // 1. lane-best (score, smallest index on equal scores) with float compares
    float bv = -INFINITY;
    int bi_idx = 0x7FFFFFFF;
    auto scan4 = [&](const f32x4 &x, int i0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int idx = i0 + e;
            if (idx < n && (x[e] > bv || bi_idx == 0x7FFFFFFF)) {
                bv = x[e];
                bi_idx = idx;
            }
        }
    };
#pragma unroll
    for (int t = 0; t < kVec; ++t) {
        const int i0 = 4 * (lane + kWave * t);
        cache[t] = i0 < n ? *reinterpret_cast<const f32x4 *>(srow + i0) : f32x4{0, 0, 0, 0};
        scan4(cache[t], i0);
    }
    for (int i0 = 4 * (lane + kWave * kVec); i0 < n; i0 += 4 * kWave)
        scan4(*reinterpret_cast<const f32x4 *>(srow + i0), i0);
    const uint64_t best = bi_idx == 0x7FFFFFFF ? 0 : make_key(bv, bi_idx);
    // 2. tau = (k-1)-th largest lane best
    const uint64_t sorted = wave_bitonic<true>(best, lane);
    const uint32_t tlo = __shfl((uint32_t)sorted, kk - 1, kWave);
    const uint32_t thi = __shfl((uint32_t)(sorted >> 32), kk - 1, kWave);
    const uint64_t tau = ((uint64_t)thi << 32) | tlo;
    const int tau_idx = key_id(tau);
    // score of tau: invert the order-preserving map of float_order_key
    const uint32_t tau_key = (uint32_t)(tau >> 32);
    const float tau_v = __uint_as_float((tau_key & 0x80000000u) ? (tau_key & 0x7FFFFFFFu) : ~tau_key);
    // With 4 consecutive scores per lane, a short row can have fewer than k-1 lanes
    // holding scores: tau is then the empty key and every score is a candidate.
    const bool take_all = tau == 0;

    // 3. compact the elements ranked at or above tau (score > tau, or equal score
    //    and index <= tau's) into the per-wave candidate list
    int cnt = 0;
    auto consider4 = [&](const f32x4 &x, int i0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int idx = i0 + e;
            const bool f = idx < n && (take_all || x[e] > tau_v || (x[e] == tau_v && idx <= tau_idx));
            const uint64_t m = __ballot(f);
            if (f) {
                const int p = cnt + (int)__builtin_amdgcn_mbcnt_hi(
                                        (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
                if (p < 64) cand[wave][p] = make_key(x[e], idx);
            }
            cnt += __popcll(m);
        }
    };
#pragma unroll
    for (int t = 0; t < kVec; ++t) {
        if (4 * kWave * t >= n) break;
        consider4(cache[t], 4 * (lane + kWave * t));
    }
    for (int base = 4 * kWave * kVec; base < n; base += 4 * kWave) {
        const int i0 = base + 4 * lane;
        consider4(i0 < n ? *reinterpret_cast<const f32x4 *>(srow + i0) : f32x4{0, 0, 0, 0}, i0);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

    int sel;   // valid on lanes < kk: a selected id
    if (cnt <= 64) {
        const uint64_t mine = lane < cnt ? cand[wave][lane] : 0;
        const uint64_t top = wave_bitonic<true>(mine, lane);
        sel = key_id(top);
    } else {
        // exact fallback: kk rounds of "largest key below the previous one"
        uint64_t prev = ~0ull;
        sel = 0;
        for (int r = 0; r < kk; ++r) {
            uint64_t b2 = 0;
            for (int idx = lane; idx < n; idx += kWave) {
                const uint64_t key = make_key(srow[idx], idx);
                if (key < prev && key > b2) b2 = key;
            }
            b2 = wave_max_u64(b2);
            if (lane == r) sel = key_id(b2);
            prev = b2;
        }
    }
    // 4. ascending ids, then the local block
    const uint32_t v = lane < kk ? (uint32_t)sel : 0xFFFFFFFFu;
    const uint32_t asc = wave_bitonic<false>(v, lane);
    if (lane < kk) out[lane] = (int32_t)asc;
    else if (lane == kk) out[lane] = bi;
}

hipError_t launch_k2_select(const float *S, int nbp, int64_t nrows, int G, int k, int64_t q0,
                            const int32_t *seq_len, int64_t Lmax, int32_t *ids, hipStream_t s) {
    if (nrows <= 0) return hipSuccess;
    const int64_t grid = (nrows + 3) / 4;
    hipLaunchKernelGGL(k2_select, dim3((unsigned)grid), dim3(256), 0, s, S, nbp, nrows, G, k, q0,
                       seq_len, Lmax, ids);
    return hipGetLastError();
}

}  // namespace msa
