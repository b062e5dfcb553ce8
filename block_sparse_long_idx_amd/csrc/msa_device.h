// msa_device.h -- device helpers shared by the MSA kernels (gfx950, wave64).
//
// MFMA lane layouts used throughout (v_mfma_f32_32x32x16_bf16 and
// v_mfma_f32_16x16x32_bf16; lane l, half hf = l / 32, quarter qt = l / 16):
//   32x32x16:  A[m][k]: lane m + 32*hf holds k = 8*hf .. 8*hf+7 of row m
//              B[k][n]: lane n + 32*hf holds k = 8*hf .. 8*hf+7 of column n
//              D[m][n]: lane n + 32*((m/4)%2), register (m%4) + 4*(m/8)
//   16x16x32:  A[m][k]: lane m + 16*qt holds k = 8*qt .. 8*qt+7
//              B[k][n]: lane n + 16*qt holds k = 8*qt .. 8*qt+7
//              D[m][n]: lane n + 16*(m/4), register m%4
// Because A and B pair the same (lane half, element) to the same k, any
// consistent relabelling of the contraction index is free; the kernels use that
// to keep every operand load a single 16-byte contiguous read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msa_launch.h"

namespace msa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 (round-to-nearest-even) in one v_cvt_pk_bf16_f32; `lo`
// lands in the low half-word.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 load16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}
__device__ __forceinline__ void store16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }
// Streaming forms (the `nt` cache policy) for data that one pass writes and a later
// kernel reads once: partial rows, their combine, the output, the block scores the
// selector reads.  They keep such streams from displacing data that is re-read
// meanwhile (K4's q rows and K/V blocks) in the caches.
__device__ __forceinline__ u32x4 load16_stream(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ void store16_stream(void *p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}
__device__ __forceinline__ void store8(void *p, u32x2 v) { *reinterpret_cast<u32x2 *>(p) = v; }

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float xor_shfl(float v, int m) { return __shfl_xor(v, m, kWave); }

// Monotone map of a float to uint32 (larger float -> larger key).  -0 and +0
// map to the same key after canonicalisation.
__device__ __forceinline__ uint32_t float_order_key(float v) {
    if (v == 0.0f) v = 0.0f;
    uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// LDS tile of 128 rows x W bf16 (W = 8*CPR), 16-byte chunks XOR-swizzled by row so
// that 16 consecutive rows read at one chunk position hit distinct banks.
template <int CPR>
__device__ __forceinline__ int swz(int row, int chunk) {
    constexpr int kMask = (CPR < 16 ? CPR : 16) - 1;
    return row * (CPR * 16) + ((chunk ^ (row & kMask)) << 4);
}

typedef void __attribute__((address_space(3))) *lds_ptr_t;

// Direct global -> LDS copy (global_load_lds_dwordx4, no registers) of a full
// 128-row tile with CPR 16-byte chunks per row into the swz<CPR> layout.  One
// instruction of a wave fills 1 KB of LDS, lane l the bytes [16 l, 16 l + 16), so
// each lane fetches the global chunk that the swizzle places there.  NTHR threads
// call it; the data is visible after an s_waitcnt on vmcnt and a barrier.
template <int CPR, int NTHR>
__device__ __forceinline__ void stage_rows_direct(char *lds, const char *src, int64_t stride_bytes,
                                                  int tid) {
    constexpr int kSegs = kBlock * CPR * 16 / 1024;
    constexpr int kWaves = NTHR / kWave;
    static_assert(kSegs % kWaves == 0, "tile must split evenly over the waves");
    constexpr int kMask = (CPR < 16 ? CPR : 16) - 1;
    const int lane = tid % kWave, wave = tid / kWave;
#pragma unroll
    for (int it = 0; it < kSegs / kWaves; ++it) {
        const int seg = it * kWaves + wave;
        const int pos = seg * 1024 + lane * 16;
        const int row = pos / (CPR * 16);
        const int chunk = ((pos / 16) % CPR) ^ (row & kMask);
        __builtin_amdgcn_global_load_lds(src + row * stride_bytes + chunk * 16,
                                         (lds_ptr_t)(lds + seg * 1024), 16, 0, 0);
    }
}

// V^T tile: D rows (one per d) of 128 keys = 16 chunks of 8 keys.  The chunk is
// XOR-swizzled with bits 0-3 and 4-6 of d: operand reads (32 consecutive d, one
// chunk) and the transposing stores (d = 8*dc + e over 16 dc, one e) both spread
// over distinct banks.
__device__ __forceinline__ int swz_vt(int d, int chunk) {
    return d * 256 + ((chunk ^ (d & 15) ^ ((d >> 4) & 7)) << 4);
}

// One KV block staged through registers: K (rows permuted by swapping bits 2 and 3,
// swz<D/8> layout) and V transposed (swz_vt layout), from rows at
// `ksrc/vsrc + key*stride_bytes`; keys >= nrows (1 <= nrows <= 128) are zero.
// load() issues every global load of both tiles with no branch around any load
// (out-of-range keys re-read row nrows-1 and are replaced by zero at store time),
// so a block costs one memory round trip; store() writes LDS.  Between the two the
// caller may do other work (the loads stay in flight).  NTHR threads (tid in
// [0, NTHR)) take part.
// LDS row of key `row` in a staged K tile.  32x32 attention (P16 false): bits 2
// and 3 swapped, so that a lane's S^T accumulators, read 8 at a time, are the P^T
// operand for 8 consecutive keys.  16x16 attention (P16 true): with
// key = 32a + 8b + 4c + r (r < 4, c < 2, b < 4) the row is 32a + 16c + 4b + r, so
// that M-tile 2t + c, register r of lane quarter b holds key 32t + 8b + 4c + r and
// a lane's two M-tiles of step t give it the keys 32t + 8b .. 32t + 8b + 7.
template <bool P16>
__device__ __forceinline__ int k_lds_row(int row) {
    if constexpr (P16) return (row & 0x63) | (((row >> 3) & 3) << 2) | (((row >> 2) & 1) << 4);
    else return (row & ~12) | ((row & 4) << 1) | ((row & 8) >> 1);
}

template <int D, int NTHR = 256, bool P16 = false>
struct KVStage {
    static constexpr int CPR = D / 8;
    static constexpr int kRowsPerIter = NTHR / CPR;
    static_assert(kBlock % (4 * kRowsPerIter) == 0, "block must split evenly");
    static constexpr int kKIters = kBlock / kRowsPerIter;          // K chunks per thread
    static constexpr int kVIters = (kBlock / 4) / kRowsPerIter;    // V key quads per thread
    u32x4 kr[kKIters], vr[kVIters][4];
    int last;

    // ksrc / vsrc are the same for every thread; offsets within the block are 32-bit
    // (at most 127 rows of stride_bytes <= 2 KiB), one address register per load.
    __device__ __forceinline__ void load(const char *ksrc, const char *vsrc, int stride_bytes,
                                         int nrows, int tid) {
        const int c = tid % CPR;
        last = nrows - 1;
#pragma unroll
        for (int it = 0; it < kKIters; ++it) {
            const int row = tid / CPR + it * kRowsPerIter;
            kr[it] = load16(ksrc + (uint32_t)(min(row, last) * stride_bytes + c * 16));
        }
#pragma unroll
        for (int it = 0; it < kVIters; ++it) {
            const int kq = tid / CPR + it * kRowsPerIter;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                vr[it][kk] = load16(vsrc + (uint32_t)(min(4 * kq + kk, last) * stride_bytes + c * 16));
        }
    }

    __device__ __forceinline__ void store(char *lds_k, char *lds_vt, int tid) const {
        const int c = tid % CPR;
        const u32x4 zero = {0, 0, 0, 0};
#pragma unroll
        for (int it = 0; it < kKIters; ++it) {
            const int row = tid / CPR + it * kRowsPerIter;
            store16(lds_k + swz<CPR>(k_lds_row<P16>(row), c), row <= last ? kr[it] : zero);
        }
#pragma unroll
        for (int it = 0; it < kVIters; ++it) {
            const int kq = tid / CPR + it * kRowsPerIter;
            u32x4 r[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) r[kk] = 4 * kq + kk <= last ? vr[it][kk] : zero;
            // element e of chunk c is d = 8c + e; gather the 4 keys for each d
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int w = e >> 1, sh = (e & 1) * 16;
                const uint32_t v0 = (r[0][w] >> sh) & 0xFFFFu, v1 = (r[1][w] >> sh) & 0xFFFFu;
                const uint32_t v2 = (r[2][w] >> sh) & 0xFFFFu, v3 = (r[3][w] >> sh) & 0xFFFFu;
                const int d = 8 * c + e;
                const int key0 = 4 * kq;
                char *p = lds_vt + swz_vt(d, key0 >> 3) + ((key0 >> 2) & 1) * 8;
                store8(p, u32x2{v0 | (v1 << 16), v2 | (v3 << 16)});
            }
        }
    }
};

}  // namespace msa
