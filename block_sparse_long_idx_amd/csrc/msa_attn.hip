// msa_attn.hip -- main branch: exact softmax attention over the selected blocks
// ("MiniMax M3 算力省 20 倍", §二 Main Branch: standard softmax attention over the
// tokens of the selected blocks only; §四 Kernel: KV-outer iteration that gathers
// the queries of each KV block into matrix-core tiles, pre-sized hot tiles, and a
// two-phase combine of partial results without atomics;
// "MiniMax-M3上架DEVUP…": no approximation inside a selected block).
//
// K4  (prefill, KV-outer): one work item = one (group g, KV block j) list slice of
//     up to 128 (query, slot) entries.  K_j and V_j of KV head g are staged once in
//     LDS (V transposed); every wave then takes 32 MFMA columns = 32/R queries x R
//     heads of the group, gathers their q rows straight into MFMA registers,
//     computes S^T = K Q^T, the block-local softmax (causal mask only in the query's
//     own block), O^T = V^T P^T, and writes the partial o unnormalised (bf16, one
//     chunk-major block per (query, group, slot)) with its row maximum m and row sum
//     l (fp32) to the entry's own location.
// K4d (decode), up to 16 heads per group: one work-group per (sequence, group)
//     attends its slots in order (two K/V buffers, the next slots' K/V in flight) and
//     folds each into a running log-sum-exp merge in registers (k4d_online); small
//     batches split each (sequence, group)'s slots into parts, one work-group each,
//     whose normalised outputs K5 merges (k4d_parts).  32 heads per group: the
//     slots' partials merged in LDS (k4d_merge), or where they do not fit the split
//     form (one work item per (sequence, group, slot)) feeding K5.
// K5  (combine): per (query, head) the partials of its valid slots are merged with
//     the log-sum-exp rule  out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,
//     M = max_s m_s (for normalised partials l_s = 1 and m_s = lse_s) -- the merge
//     that keeps the softmax exact.
//
// Contraction-index relabelling: the K rows fed as the A operand of S^T are
// permuted (pi below) so that the S^T accumulators of a lane, read 8 at a time,
// are exactly the P^T B operand of the next MFMA for 8 CONSECUTIVE keys; V^T then
// serves its A operand with one 16-byte LDS read.  No register shuffles are needed
// between the two products.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

// A-operand row m of an S^T M-tile holds key pi(m) = m with bits 2 and 3 swapped:
//   pi(m) = 16*(m>>4) + 8*((m>>2)&1) + 4*((m>>3)&1) + (m&3).
// K tiles are staged with that permutation applied (KVStage), so the
// MFMA operand reads are plain row reads.

// Q operand of one lane's column: D/16 chunks of 8 values (K-step ks takes chunk 2ks+hf).
// The loaded registers are left untouched until the MFMAs read them (no select on
// the value): the first use of a load is where the wait for it lands.
template <int D>
__device__ __forceinline__ void load_q(bf16x8 (&qb)[D / 16], const uint16_t *qrow, int hf) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qb[ks] = as_bf16x8(load16(qrow + (2 * ks + hf) * 8));
}

// One pass of 32 columns of a wave over a staged block.  Lane column = l % 32.
//   qb     : the column's q row as the B operand (see load_q)
//   rel    : the column's token position minus the staged block's first position;
//            0 <= rel < 128 marks the query's own block, whose keys past it are masked
//   emit   : receives the column's partial as bf16 16-byte chunks -- w[u] holds
//            chunk 4(u/2) + 2(u%2) + hf of the row (elements 8c .. 8c+7) -- and writes
//            it.  NORM: o normalised by its row sum, plus the log2-sum-exp of the
//            scaled scores (emit(w, lse, sum)); !NORM: o NOT normalised, plus the row
//            maximum m (scaled, log2 units) and the row sum l of 2^(s - m)
//            (emit(w, m, l)) -- the combine divides, which saves the multiplies here
template <int D, bool NORM, typename Emit>
__device__ __forceinline__ void attend_pass(const char *lds_k, const char *lds_vt,
                                            const bf16x8 (&qb)[D / 16], bool active, int64_t rel,
                                            float scale_log2, int lane, Emit emit) {
    constexpr int KS = D / 16;   // K-steps of S^T over d
    constexpr int CPR = D / 8;
    constexpr int MD = D / 32;   // M-tiles of O^T over d
    const int hf = lane >> 5, l32 = lane & 31;

    f32x16 sc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        sc[mt] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 a = as_bf16x8(load16(lds_k + swz<CPR>(mt * 32 + l32, 2 * ks + hf)));
            sc[mt] = mfma32(a, qb[ks], sc[mt]);
        }
        // keep each M-tile's operand reads next to its MFMAs (bounds live registers)
        __builtin_amdgcn_sched_barrier(0);
    }
    // causal mask inside the query's own block (skipped by waves holding no such
    // query); register r of M-tile mt holds key 32mt + 16(ip/2) + 8hf + 4(ip%2) + jj
    const bool local = active && rel < kBlock;
    if (__ballot(local)) {
        const int lim = local ? (int)rel - 8 * hf : kBlock;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
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
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[mt][r]);
    mx = fmaxf(mx, xor_shfl(mx, 32));
    // p = 2^((s - max) * scale * log2 e), one FMA + one exp per score
    const float nmx = -mx * scale_log2;
    float sum = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = __builtin_amdgcn_exp2f(fmaf(sc[mt][r], scale_log2, nmx));
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
            const bf16x8 a = as_bf16x8(load16(lds_vt + swz_vt(md * 32 + l32, 2 * kt + hf)));
            o[md] = mfma32(a, pb[kt], o[md]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    // normalise (NORM), pack to bf16, and swap half-rows between the lane halves
    // (v_permlane32_swap) so each lane holds 8 consecutive d values (16 bytes):
    // before, lane half hf holds d = 16q + 4hf + {0..3} and 16q + 8 + 4hf + {0..3}
    const float inv = NORM ? 1.0f / sum : 1.0f;
    u32x4 w[D / 16];
#pragma unroll
    for (int md = 0; md < MD; ++md) {
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
            const f32x16 &acc = o[md];
            const int r0 = 8 * q2;          // registers of ip = 2q2 (r0..r0+3) and 2q2+1
            uint32_t a0, a1, b0, b1;
            if constexpr (NORM) {
                a0 = pack_bf16x2(acc[r0 + 0] * inv, acc[r0 + 1] * inv);
                a1 = pack_bf16x2(acc[r0 + 2] * inv, acc[r0 + 3] * inv);
                b0 = pack_bf16x2(acc[r0 + 4] * inv, acc[r0 + 5] * inv);
                b1 = pack_bf16x2(acc[r0 + 6] * inv, acc[r0 + 7] * inv);
            } else {
                a0 = pack_bf16x2(acc[r0 + 0], acc[r0 + 1]);
                a1 = pack_bf16x2(acc[r0 + 2], acc[r0 + 3]);
                b0 = pack_bf16x2(acc[r0 + 4], acc[r0 + 5]);
                b1 = pack_bf16x2(acc[r0 + 6], acc[r0 + 7]);
            }
            const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
            // lower half now holds d = 32md + 16q2 + 0..7, upper half 32md + 16q2 + 8..15
            w[2 * md + q2] = u32x4{s0[0], s1[0], s0[1], s1[1]};
        }
    }
    if constexpr (NORM) emit(w, mx * scale_log2 + __log2f(sum), sum);
    else emit(w, mx * scale_log2, sum);
}

// Decode's attention core on v_mfma_f32_16x16x32_bf16: one query's R <= 16 heads are
// the 16 columns, so half the arithmetic of the 32-column core above is not spent on
// empty columns.  Lane l: head n = l % 16, quarter qt = l / 16.  K is staged with
// k_lds_row<true> (KVStage<..., true>): M-tile mt, register r of quarter qt holds key
// 32 (mt / 2) + 8 qt + 4 (mt % 2) + r, so M-tiles 2t and 2t + 1 give a lane exactly the
// P^T operand of keys 32t + 8qt .. 32t + 8qt + 7; V^T is read in key order.
//   qb    : the head's q row as the B operand: step ks holds d = 32ks + 8qt .. + 7
//   rel   : the query's position minus the block's first; keys past it are masked
// attend16_core leaves o unnormalised in fp32: o[md] holds d = 16md + 4qt .. + 3 of
// head n, with the row maximum ms of the scaled scores (log2 units) and the row sum
// of 2^(score - ms).
template <int D>
__device__ __forceinline__ void load_q16(bf16x8 (&qb)[D / 32], const uint16_t *qrow, int qt) {
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) qb[ks] = as_bf16x8(load16(qrow + (4 * ks + qt) * 8));
}

template <int D>
__device__ __forceinline__ void attend16_core(const char *lds_k, const char *lds_vt,
                                              const bf16x8 (&qb)[D / 32], bool active, int64_t rel,
                                              float scale_log2, int lane, f32x4 (&o)[D / 16],
                                              float &ms, float &sum) {
    constexpr int CPR = D / 8;
    const int m = lane & 15, qt = lane >> 4;
    f32x4 sc[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
        sc[mt] = f32x4{};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            const bf16x8 a = as_bf16x8(load16(lds_k + swz<CPR>(16 * mt + m, 4 * ks + qt)));
            sc[mt] = mfma16(a, qb[ks], sc[mt]);
        }
    }
    // causal mask inside the query's own block
    const bool local = active && rel < kBlock;
    if (__ballot(local)) {
        const int lim = local ? (int)rel : kBlock;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (32 * (mt >> 1) + 8 * qt + 4 * (mt & 1) + r > lim) sc[mt][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[mt][r]);
    mx = fmaxf(mx, xor_shfl(mx, 16));
    mx = fmaxf(mx, xor_shfl(mx, 32));
    const float nmx = -mx * scale_log2;
    sum = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float p = __builtin_amdgcn_exp2f(fmaf(sc[mt][r], scale_log2, nmx));
            sc[mt][r] = p;
            sum += p;
        }
    }
    sum += xor_shfl(sum, 16);
    sum += xor_shfl(sum, 32);
    bf16x8 pb[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
        u32x4 w;
        w[0] = pack_bf16x2(sc[2 * kt][0], sc[2 * kt][1]);
        w[1] = pack_bf16x2(sc[2 * kt][2], sc[2 * kt][3]);
        w[2] = pack_bf16x2(sc[2 * kt + 1][0], sc[2 * kt + 1][1]);
        w[3] = pack_bf16x2(sc[2 * kt + 1][2], sc[2 * kt + 1][3]);
        pb[kt] = as_bf16x8(w);
    }
#pragma unroll
    for (int md = 0; md < D / 16; ++md) {
        o[md] = f32x4{};
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const bf16x8 a = as_bf16x8(load16(lds_vt + swz_vt(16 * md + m, 4 * kt + qt)));
            o[md] = mfma16(a, pb[kt], o[md]);
        }
    }
    ms = mx * scale_log2;
}

// ---------------------------------------------------------------------------
// K4: KV-outer sparse attention over the scheduled lists.
// ---------------------------------------------------------------------------
template <int D, int R, bool BATCH>
__global__ __launch_bounds__(256, 2) void k4_kv_outer(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kx,
    const uint16_t *__restrict__ vx, const int *__restrict__ offs, const int *__restrict__ toff,
    const int *__restrict__ total, const int *__restrict__ items, const int *__restrict__ order,
    const uint32_t *__restrict__ list, int nb, int64_t L, int64_t q0, int H, int G, int kslots,
    float scale_log2, uint16_t *__restrict__ po, f32x2 *__restrict__ pml, const BatchMap bm) {
    __shared__ __attribute__((aligned(16))) char lds_k[kBlock * D * 2];
    __shared__ __attribute__((aligned(16))) char lds_vt[D * kBlock * 2];
    static_assert(kK4Queries <= 256, "one entry per thread is staged");
    __shared__ uint32_t lds_e[kK4Queries];                   // the item's (query, slot) entries
    // XCD-aware order: work-group b runs on XCD b % 8.  Runs of kK4Run consecutive
    // items of the run order (one group, middle entries in one query window) go to
    // the XCDs in turn, so at any time all XCDs gather the q rows of one narrow range
    // of queries, which the last-level cache holds across their re-reads, where
    // contiguous eighths per XCD would span the whole chunk.  Work-groups past the
    // items actually scheduled (the grid is an upper bound) exit.
    const int tot = *total;
    const int run = blockIdx.x / 8;
    const int x = ((run / kK4Run) * 8 + (int)(blockIdx.x % 8)) * kK4Run + run % kK4Run;
    if (x >= tot) return;
    const int u = order ? order[x] : x;                      // the work item (tile)
    if ((unsigned)u >= (unsigned)tot) return;                // (order is a permutation)
    const int li = items[u];                                 // list of this tile
    const int g = li / nb, j = li % nb;
    // the block's first token (single sequence: block j; batch: global block j)
    const int64_t blk0 = BATCH ? (int64_t)bm.blk_tok0[j] : (int64_t)j * kBlock;
    // batch: position of an entry's query relative to the block's first token,
    // fetched with the entry one pass ahead (a single sequence computes it)
    auto rel_of = [&](bool on, uint32_t e) -> int {
        if constexpr (BATCH) return on ? bm.row_kvpos[e >> 5] - (int)blk0 : 0;
        else return 0;
    };
    const int t = u - toff[li];
    const int begin = offs[li] + t * kK4Queries;
    const int cnt = min(kK4Queries, offs[li + 1] - begin);

    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const int hf = lane >> 5, l32 = lane & 31;
    constexpr int QPW = 32 / R;   // queries per wave pass
    const int a = l32 / R, h = l32 % R;
    const int64_t hh = (int64_t)g * R + h;

    // Pass p of a wave covers entries wave*QPW + p*STEP + (column / R).  Its q rows
    // (and entry, and in a batch its position) are requested at the start of pass
    // p - 1 and consumed -- an empty asm statement that reads the registers --
    // after that pass's arithmetic and before its partial rows are stored.  Loads
    // and stores share one counter, and the stores sit in branches that may be
    // skipped, so any later first use of the loaded registers (the copy at the
    // loop's end) would wait for every partial row just stored.  The loaded rows
    // are used unmasked: an inactive column reads a valid row (that of entry 0)
    // and its result is discarded.  The first pass's rows are requested before the
    // K/V staging.
    constexpr int STEP = 4 * QPW;
    const int first_e = wave * QPW;
    const int npass = first_e < cnt ? (cnt - first_e + STEP - 1) / STEP : 0;
    struct PassIn {
        bool act;
        uint32_t entry;
        int rel;
    };
    auto request = [&](int pass, bool from_lds, PassIn &in, bf16x8 (&qr)[D / 16]) {
        const int e = first_e + pass * STEP + a;
        in.act = e < cnt;
        in.entry = in.act ? (from_lds ? lds_e[e] : list[begin + e]) : 0u;
        load_q<D>(qr, q + ((q0 + (in.entry >> 5)) * H + hh) * D, hf);
        in.rel = rel_of(in.act, in.entry);
    };
    // the item's entries (one per thread, for LDS) are requested with the first
    // pass's, so that one wait covers both before the q rows and K/V are requested
    const uint32_t my_e = tid < cnt ? list[begin + tid] : 0u;
    PassIn in0;
    bf16x8 qr0[D / 16];
    request(0, false, in0, qr0);

    if (tid < cnt) lds_e[tid] = my_e;
    const int kv_row_bytes = G * D * 2;
    const char *ksrc = reinterpret_cast<const char *>(kx + (blk0 * G + g) * D);
    const char *vsrc = reinterpret_cast<const char *>(vx + (blk0 * G + g) * D);
    const int nrows = BATCH ? bm.blk_rows[j] : (int)min<int64_t>(kBlock, L - blk0);
    {
        KVStage<D> st;
        st.load(ksrc, vsrc, kv_row_bytes, nrows, tid);
        st.store(lds_k, lds_vt, tid);
    }
    __syncthreads();

    auto attend = [&](int pass, const PassIn &in, const bf16x8 (&qr)[D / 16],
                      const PassIn &nin, const bf16x8 (&nqr)[D / 16]) {
        const int64_t il = in.entry >> 5;
        const int s = in.entry & 31;
        const int64_t lrow = ((il * G + g) * kslots + s) * R + h;
        const bool act = in.act;
        attend_pass<D, false>(lds_k, lds_vt, qr, act, BATCH ? (int64_t)in.rel : q0 + il - blk0,
                       scale_log2, lane, [&](const u32x4 (&w)[D / 16], float m, float l) {
#pragma unroll
                           for (int ks = 0; ks < D / 16; ++ks) asm volatile("" ::"v"(nqr[ks]));
                           asm volatile("" ::"v"(nin.entry), "v"(nin.rel));
                           if (act && hf == 0) pml[lrow] = f32x2{m, l};
                           // The partials of one (query, group, slot) are a block of R
                           // heads x D/8 chunks of 16 bytes, chunk-major: chunk c of
                           // head h at (c * R + h) * 16 bytes.  The lane holds chunks
                           // 2u + hf of its column's head, so the columns of one query
                           // write 2 * R * 16 contiguous bytes per store instruction --
                           // whole lines, with no staging through LDS.
                           if (act) {
                               uint16_t *dst = po + (size_t)(lrow - h) * D + h * 8;
#pragma unroll
                               for (int u = 0; u < D / 16; ++u)
                                   store16_stream(dst + (2 * u + hf) * (R * 8), w[u]);
                           }
                       });
    };
    for (int p = 0; p < npass; ++p) {
        PassIn in1;
        bf16x8 qr1[D / 16];
        request(p + 1, true, in1, qr1);
        attend(p, in0, qr0, in1, qr1);
        in0 = in1;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) qr0[ks] = qr1[ks];
    }
}

template <int D, int R>
static hipError_t k4_dispatch(const uint16_t *q, const uint16_t *kx, const uint16_t *vx,
                              const SchedBuffers &sb, int nb, int64_t L, int64_t q0, int64_t C,
                              int H, int G, int k, float scale_log2, uint16_t *po, float *plse,
                              const BatchMap &bm, hipStream_t s) {
    const int64_t grid = round_up(k4_max_items(C, G, k, nb), 8 * kK4Run);
    if (grid == 0) return hipSuccess;
    f32x2 *pml = reinterpret_cast<f32x2 *>(plse);
    // small chunks have no run order (K3 skips the sort): items in list order
    const int *order = C <= kK3NoOrderQueries ? nullptr : sb.order;
    if (bm.row_kvpos)
        hipLaunchKernelGGL((k4_kv_outer<D, R, true>), dim3((unsigned)grid), dim3(256), 0, s, q, kx,
                           vx, sb.offs, sb.toff, sb.total, sb.items, order, sb.list, nb, L, q0, H, G, k,
                           scale_log2, po, pml, bm);
    else
        hipLaunchKernelGGL((k4_kv_outer<D, R, false>), dim3((unsigned)grid), dim3(256), 0, s, q, kx,
                           vx, sb.offs, sb.toff, sb.total, sb.items, order, sb.list, nb, L, q0, H, G, k,
                           scale_log2, po, pml, bm);
    return hipGetLastError();
}

hipError_t launch_k4_kv_outer(const uint16_t *q, const uint16_t *kx, const uint16_t *vx,
                              const SchedBuffers &sb, int nb, int64_t L, int64_t q0, int64_t C,
                              int H, int G, int d, int k, float scale, uint16_t *po, float *plse,
                              const BatchMap &bm, hipStream_t s) {
    const float sl2 = scale * kLog2e;
    const int R = H / G;
#define K4_CASE(dd, rr) \
    if (d == dd && R == rr) return k4_dispatch<dd, rr>(q, kx, vx, sb, nb, L, q0, C, H, G, k, sl2, po, plse, bm, s);
    K4_CASE(64, 1) K4_CASE(64, 2) K4_CASE(64, 4) K4_CASE(64, 8) K4_CASE(64, 16) K4_CASE(64, 32)
    K4_CASE(128, 1) K4_CASE(128, 2) K4_CASE(128, 4) K4_CASE(128, 8) K4_CASE(128, 16) K4_CASE(128, 32)
#undef K4_CASE
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// K4d: decode, one work-group per (sequence, group, slot).
// ---------------------------------------------------------------------------
template <int D, int R>
__global__ __launch_bounds__(256, 2) void k4d_split(const uint16_t *__restrict__ q,
                                                 const uint16_t *__restrict__ kc,
                                                 const uint16_t *__restrict__ vc,
                                                 const int32_t *__restrict__ ids,
                                                 const int32_t *__restrict__ seq_len,
                                                 const int32_t *__restrict__ table, int maxb,
                                                 int64_t Lmax, int H, int G, int kslots,
                                                 float scale_log2, uint16_t *__restrict__ po,
                                                 float *__restrict__ plse, int64_t n_items) {
    __shared__ __attribute__((aligned(16))) char lds_k[kBlock * D * 2];
    __shared__ __attribute__((aligned(16))) char lds_vt[D * kBlock * 2];
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const int kv_row_bytes = G * D * 2;
    // Items (sequence, group, slot) with a valid id, visited with stride gridDim.x.
    // The next item's K/V loads are issued before the current item is attended, so
    // the memory latency of one overlaps the attention of the other.
    auto next_valid = [&](int64_t it) {
        for (; it < n_items; it += gridDim.x)
            if (ids[it] >= 0) return it;
        return n_items;
    };
    // item -> first K/V element of its block: contiguous cache [N, Lmax, G, D], or the
    // block's page of a paged cache [pages, 128, G, D].  Only the sequence's cached
    // rows are read: in the query's own block the rows at and past seq_len (not yet
    // written, possibly non-finite) are staged as zeros, so that a masked key
    // contributes exactly 0 to the P V product.
    auto kv_src = [&](int64_t it, int &nrows) {
        const int64_t n = it / ((int64_t)G * kslots);
        const int g = (int)((it / kslots) % G);
        const int j = ids[it];
        const int64_t tok0 =
            table ? (int64_t)table[n * maxb + j] * kBlock : n * Lmax + (int64_t)j * kBlock;
        nrows = (int)max<int64_t>(1, min<int64_t>(kBlock, (int64_t)seq_len[n] - (int64_t)j * kBlock));
        return (tok0 * G + g) * D;
    };
    // Roles by wave: waves 2-3 stage K/V (store the current item, then load the next
    // into registers), wave 0 attends, wave 1 only keeps the barrier count.  Every
    // role walks the same item sequence and meets the same two barriers per item;
    // the roles' code paths are disjoint, so the staging registers are never live
    // during the attention.
    const int64_t first = next_valid(blockIdx.x);
    if (first >= n_items) return;
    if (wave >= 2) {
        const int stid = tid - 2 * kWave;
        KVStage<D, 2 * kWave> st;
        int64_t item = first;
        int nrows;
        int64_t off = kv_src(item, nrows);
        st.load(reinterpret_cast<const char *>(kc + off), reinterpret_cast<const char *>(vc + off),
                kv_row_bytes, nrows, stid);
        while (item < n_items) {
            st.store(lds_k, lds_vt, stid);
            __syncthreads();                       // (A) the item is in LDS
            const int64_t nxt = next_valid(item + gridDim.x);
            if (nxt < n_items) {
                off = kv_src(nxt, nrows);
                st.load(reinterpret_cast<const char *>(kc + off),
                        reinterpret_cast<const char *>(vc + off), kv_row_bytes, nrows, stid);
            }
            __syncthreads();                       // (B) the item's attention is done
            item = nxt;
        }
    } else if (wave == 0) {
        // The q rows of an item are requested before barrier (B) of the previous one,
        // so their latency overlaps the stagers' LDS stores.  An inactive lane reads
        // the group's first head row and its result is discarded.
        const int l32 = lane & 31, hf = lane >> 5;
        const bool active = l32 < R;
        auto q_row = [&](int64_t it) {
            const int64_t n = it / ((int64_t)G * kslots);
            const int g = (int)((it / kslots) % G);
            return q + (n * H + (int64_t)g * R + (active ? l32 : 0)) * D;
        };
        bf16x8 qb[D / 16];
        load_q<D>(qb, q_row(first), hf);
        for (int64_t item = first; item < n_items;) {
            __syncthreads();                       // (A)
            const int64_t n = item / ((int64_t)G * kslots);
            const int g = (int)((item / kslots) % G);
            const int s = (int)(item % kslots);
            const int j = ids[item];
            const int64_t p = (int64_t)seq_len[n] - 1;
            const int64_t hh = (int64_t)g * R + (active ? l32 : 0);
            const int64_t prow = (n * H + hh) * kslots + s;
            const int64_t lrow = ((n * G + g) * kslots + s) * R + (active ? l32 : 0);
            attend_pass<D, true>(lds_k, lds_vt, qb, active, p - (int64_t)j * kBlock, scale_log2, lane,
                           [&](const u32x4 (&w)[D / 16], float lse, float) {
                               if (!active) return;
#pragma unroll
                               for (int u = 0; u < D / 16; ++u)
                                   store16_stream(po + prow * D + 8 * (4 * (u >> 1) + 2 * (u & 1) + hf), w[u]);
                               if (hf == 0) plse[lrow] = lse;
                           });
            const int64_t nxt = next_valid(item + gridDim.x);
            if (nxt < n_items) load_q<D>(qb, q_row(nxt), hf);
            __syncthreads();                       // (B)
            item = nxt;
        }
    } else {
        for (int64_t item = first; item < n_items; item = next_valid(item + gridDim.x)) {
            __syncthreads();                       // (A)
            __syncthreads();                       // (B)
        }
    }
}

template <int D, int R>
static hipError_t k4d_dispatch(const uint16_t *q, const uint16_t *kc, const uint16_t *vc,
                               const int32_t *ids, const int32_t *seq_len, const int32_t *table,
                               int maxb, int N, int64_t Lmax, int H, int G, int k, float sl2,
                               uint16_t *po, float *plse, hipStream_t s) {
    const int64_t n_items = (int64_t)N * G * k;
    if (n_items == 0) return hipSuccess;
    // two work-groups per CU (64 KB of LDS each), a few items per work-group
    const int64_t grid = n_items < 512 ? n_items : 512;
    hipLaunchKernelGGL((k4d_split<D, R>), dim3((unsigned)grid), dim3(256), 0, s, q, kc, vc, ids,
                       seq_len, table, maxb, Lmax, H, G, k, sl2, po, plse, n_items);
    return hipGetLastError();
}

hipError_t launch_k4d_split(const uint16_t *q, const uint16_t *kc, const uint16_t *vc,
                            const int32_t *ids, const int32_t *seq_len, const int32_t *table,
                            int maxb, int N, int64_t Lmax, int H, int G, int d, int k, float scale,
                            uint16_t *po, float *plse, hipStream_t s) {
    const float sl2 = scale * kLog2e;
    const int R = H / G;
#define K4D_CASE(dd, rr) \
    if (d == dd && R == rr) return k4d_dispatch<dd, rr>(q, kc, vc, ids, seq_len, table, maxb, N, Lmax, H, G, k, sl2, po, plse, s);
    K4D_CASE(64, 32) K4D_CASE(128, 32)
#undef K4D_CASE
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// K4d with the combine inside: one work-group per (sequence, group) walks that
// group's valid slots in slot order (K/V of the next slot staged while the current
// one is attended, as in K4d; the q rows loaded once), keeps every slot's
// normalised o (bf16) and log2-sum-exp in LDS, and finally merges them per
// (head, 8 d values) with K5's arithmetic, in slot order: the output is bitwise
// the one K4d + K5 give, without the partials' trip through memory and the second
// launch.  Used when the slots' partials fit in LDS beside the staged block.
// ---------------------------------------------------------------------------
// The combine's arithmetic for one (query, head) and 8 consecutive d values: slots
// with ok[s] carry a normalised partial v[s] (8 bf16) and its log2-sum-exp l[s];
//   out = sum_s 2^(l[s] - M) v[s] / sum_s 2^(l[s] - M),  M = max_s l[s],
// summed in slot order, rounded once to bf16 (all zeros when no slot is valid).
// Shared by K5 and K4d's merged form, so both give the same bits.
template <int KMAX>
__device__ __forceinline__ u32x4 lse_merge(const u32x4 (&v)[KMAX], const float (&l)[KMAX],
                                           const bool (&ok)[KMAX]) {
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < KMAX; ++s)
        if (ok[s]) M = fmaxf(M, l[s]);
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float wsum = 0.0f;
#pragma unroll
    for (int s = 0; s < KMAX; ++s) {
        if (!ok[s]) continue;
        const float w = __builtin_amdgcn_exp2f(l[s] - M);
        wsum += w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += w * bf16_to_f32(v[s][e] & 0xFFFFu);
            acc[2 * e + 1] += w * bf16_to_f32(v[s][e] >> 16);
        }
    }
    const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
    return r;
}

// The same merge for partials that carry their o unnormalised, with the row maximum
// m[s] (log2 units) and row sum l[s] of 2^(score - m[s]):
//   out = sum_s 2^(m[s] - M) v[s] / sum_s 2^(m[s] - M) l[s],  M = max_s m[s],
// summed in slot order, rounded once to bf16 (all zeros when no slot is valid).
template <int KMAX>
__device__ __forceinline__ u32x4 ml_merge(const u32x4 (&v)[KMAX], const f32x2 (&ml)[KMAX],
                                          const bool (&ok)[KMAX]) {
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < KMAX; ++s)
        if (ok[s]) M = fmaxf(M, ml[s][0]);
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float wsum = 0.0f;
#pragma unroll
    for (int s = 0; s < KMAX; ++s) {
        if (!ok[s]) continue;
        const float w = __builtin_amdgcn_exp2f(ml[s][0] - M);
        wsum += w * ml[s][1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += w * bf16_to_f32(v[s][e] & 0xFFFFu);
            acc[2 * e + 1] += w * bf16_to_f32(v[s][e] >> 16);
        }
    }
    const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
    return r;
}

// LDS: the staged block (4 * kBlock * D bytes, 64 KB at d = 128) plus the partials,
// at most 96 KB, so the whole stays within the CU's 160 KB.
constexpr size_t kK4dmPartialBytes = 96 * 1024;
template <int D, int R, int KMAX>
constexpr bool k4dm_fits() {
    return (size_t)KMAX * R * D * 2 + (size_t)KMAX * R * 4 <= kK4dmPartialBytes;
}

template <int D, int R, int KMAX>
__global__ __launch_bounds__(256, 1) void k4d_merge(const uint16_t *__restrict__ q,
                                                 const uint16_t *__restrict__ kc,
                                                 const uint16_t *__restrict__ vc,
                                                 const int32_t *__restrict__ ids,
                                                 const int32_t *__restrict__ seq_len,
                                                 const int32_t *__restrict__ table, int maxb,
                                                 int64_t Lmax, int H, int G, int kslots,
                                                 float scale_log2, uint16_t *__restrict__ out) {
    static_assert(k4dm_fits<D, R, KMAX>(), "partials must fit in LDS");
    __shared__ __attribute__((aligned(16))) char lds_k[kBlock * D * 2];
    __shared__ __attribute__((aligned(16))) char lds_vt[D * kBlock * 2];
    __shared__ __attribute__((aligned(16))) uint16_t lds_po[KMAX][R][D];
    __shared__ float lds_l[KMAX][R];
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const int kv_row_bytes = G * D * 2;
    const int64_t ng = blockIdx.x;
    const int64_t n = ng / G;
    const int g = (int)(ng % G);
    const int32_t *idr = ids + ng * kslots;
    auto next_valid = [&](int sl) {
        for (; sl < kslots; ++sl)
            if (idr[sl] >= 0) return sl;
        return kslots;
    };
    // first K/V element of slot sl's block (contiguous cache or its page); rows at and
    // past seq_len in the own block are staged as zeros (as in K4d)
    auto kv_src = [&](int sl, int &nrows) {
        const int j = idr[sl];
        const int64_t tok0 =
            table ? (int64_t)table[n * maxb + j] * kBlock : n * Lmax + (int64_t)j * kBlock;
        nrows = (int)max<int64_t>(1, min<int64_t>(kBlock, (int64_t)seq_len[n] - (int64_t)j * kBlock));
        return (tok0 * G + g) * D;
    };
    // Roles by wave as in K4d: waves 2-3 stage, wave 0 attends, wave 1 keeps the
    // barrier count; every role walks the same valid slots and meets two barriers
    // per slot.
    const int first = next_valid(0);
    if (wave >= 2) {
        const int stid = tid - 2 * kWave;
        KVStage<D, 2 * kWave> st;
        int sl = first, nrows;
        if (sl < kslots) {
            int64_t off = kv_src(sl, nrows);
            st.load(reinterpret_cast<const char *>(kc + off),
                    reinterpret_cast<const char *>(vc + off), kv_row_bytes, nrows, stid);
        }
        while (sl < kslots) {
            st.store(lds_k, lds_vt, stid);
            __syncthreads();                       // (A) the slot's block is in LDS
            const int nxt = next_valid(sl + 1);
            if (nxt < kslots) {
                const int64_t off = kv_src(nxt, nrows);
                st.load(reinterpret_cast<const char *>(kc + off),
                        reinterpret_cast<const char *>(vc + off), kv_row_bytes, nrows, stid);
            }
            __syncthreads();                       // (B) the slot's attention is done
            sl = nxt;
        }
    } else if (wave == 0) {
        // an inactive lane reads the group's first head row; its result is discarded
        const int l32 = lane & 31, hf = lane >> 5;
        const bool active = l32 < R;
        bf16x8 qb[D / 16];
        load_q<D>(qb, q + (n * H + (int64_t)g * R + (active ? l32 : 0)) * D, hf);
        const int64_t p = (int64_t)seq_len[n] - 1;
        for (int sl = first; sl < kslots; sl = next_valid(sl + 1)) {
            __syncthreads();                       // (A)
            const int j = idr[sl];
            attend_pass<D, true>(lds_k, lds_vt, qb, active, p - (int64_t)j * kBlock, scale_log2, lane,
                           [&](const u32x4 (&w)[D / 16], float lse, float) {
                               if (!active) return;
#pragma unroll
                               for (int u = 0; u < D / 16; ++u)
                                   *reinterpret_cast<u32x4 *>(
                                       &lds_po[sl][l32][8 * (4 * (u >> 1) + 2 * (u & 1) + hf)]) = w[u];
                               if (hf == 0) lds_l[sl][l32] = lse;
                           });
            __syncthreads();                       // (B)
        }
    } else {
        for (int sl = first; sl < kslots; sl = next_valid(sl + 1)) {
            __syncthreads();                       // (A)
            __syncthreads();                       // (B)
        }
    }
    __syncthreads();                               // every slot's partial is in LDS
    // the combine, per (head, 8 d values), slots in order
    constexpr int TPH = D / 8;
    for (int t = tid; t < R * TPH; t += 256) {
        const int h = t / TPH, sub = t % TPH;
        u32x4 v[KMAX];
        float l[KMAX];
        bool ok[KMAX];
#pragma unroll
        for (int sl = 0; sl < KMAX; ++sl) {
            ok[sl] = sl < kslots && idr[sl] >= 0;
            l[sl] = ok[sl] ? lds_l[sl][h] : 0.0f;
            v[sl] = ok[sl] ? *reinterpret_cast<const u32x4 *>(&lds_po[sl][h][sub * 8])
                           : u32x4{0, 0, 0, 0};
        }
        store16_stream(out + ((n * H) + (int64_t)g * R + h) * D + sub * 8,
                       lse_merge<KMAX>(v, l, ok));
    }
}

template <int D, int R, int KMAX>
static hipError_t k4dm_launch(const uint16_t *q, const uint16_t *kc, const uint16_t *vc,
                              const int32_t *ids, const int32_t *seq_len, const int32_t *table,
                              int maxb, int N, int64_t Lmax, int H, int G, int k, float sl2,
                              uint16_t *out, hipStream_t s) {
    if constexpr (k4dm_fits<D, R, KMAX>()) {
        hipLaunchKernelGGL((k4d_merge<D, R, KMAX>), dim3((unsigned)((int64_t)N * G)), dim3(256),
                           0, s, q, kc, vc, ids, seq_len, table, maxb, Lmax, H, G, k, sl2, out);
        return hipGetLastError();
    } else {
        return hipErrorNotSupported;
    }
}

template <int D, int R>
static hipError_t k4dm_dispatch(const uint16_t *q, const uint16_t *kc, const uint16_t *vc,
                                const int32_t *ids, const int32_t *seq_len, const int32_t *table,
                                int maxb, int N, int64_t Lmax, int H, int G, int k, float sl2,
                                uint16_t *out, hipStream_t s) {
    if (k <= 4) return k4dm_launch<D, R, 4>(q, kc, vc, ids, seq_len, table, maxb, N, Lmax, H, G, k, sl2, out, s);
    if (k <= 8) return k4dm_launch<D, R, 8>(q, kc, vc, ids, seq_len, table, maxb, N, Lmax, H, G, k, sl2, out, s);
    if (k <= 16) return k4dm_launch<D, R, 16>(q, kc, vc, ids, seq_len, table, maxb, N, Lmax, H, G, k, sl2, out, s);
    return hipErrorNotSupported;
}

hipError_t launch_k4d_merge(const uint16_t *q, const uint16_t *kc, const uint16_t *vc,
                            const int32_t *ids, const int32_t *seq_len, const int32_t *table,
                            int maxb, int N, int64_t Lmax, int H, int G, int d, int k, float scale,
                            uint16_t *out, hipStream_t s) {
    if (N <= 0) return hipSuccess;
    const float sl2 = scale * kLog2e;
    const int R = H / G;
#define K4DM_CASE(dd, rr) \
    if (d == dd && R == rr) return k4dm_dispatch<dd, rr>(q, kc, vc, ids, seq_len, table, maxb, N, Lmax, H, G, k, sl2, out, s);
    K4DM_CASE(64, 32) K4DM_CASE(128, 32)
#undef K4DM_CASE
    return hipErrorNotSupported;
}

bool k4d_merge_supported(int d, int R, int k) {
    if (k < 1 || k > 16 || (d != 64 && d != 128)) return false;
    const int km = k <= 4 ? 4 : (k <= 8 ? 8 : 16);
    return (size_t)km * R * d * 2 + (size_t)km * R * 4 <= kK4dmPartialBytes;
}

// ---------------------------------------------------------------------------
// K4d with an online merge, one launch (R <= 16): one work-group per (sequence,
// group) walks the group's valid slots in slot order with two K/V buffers in LDS.
// Waves 2-3 stage: each holds two slots' K/V in registers, so that while slot t + 1
// is stored into the free buffer, slot t + 2 is already in flight, and slot t + 3 is
// requested as soon as slot t + 1's registers are free.  Wave 0 attends slot t with
// the 16-column core and keeps a running merge in registers: per head the largest
// scaled score M seen so far, the sum l of 2^(score - M), and o (fp32,
// unnormalised).  Each slot's (o_s, m_s, l_s) is folded in with a = 2^(M - M'),
// b = 2^(m_s - M'), M' = max(M, m_s):  o <- a o + b o_s,  l <- a l + b l_s -- the
// log-sum-exp merge of the combine, one slot at a time and without rounding a slot's
// o to bf16.  out = o / l (zeros when no slot is valid).  No partials leave the
// work-group, so any k fits.  Wave 1 only keeps the barrier count.
//
// Barrier t closes step t: before it the stagers have stored the t-th valid slot
// into buffer t & 1 and wave 0 has finished slot t - 1 (held in the other buffer,
// which the stagers overwrite only after barrier t).  Every wave meets one barrier
// per valid slot.
// ---------------------------------------------------------------------------
template <int D, int R>
__global__ __launch_bounds__(256, 1) void k4d_online(const uint16_t *__restrict__ q,
                                                  const uint16_t *__restrict__ kc,
                                                  const uint16_t *__restrict__ vc,
                                                  const int32_t *__restrict__ ids,
                                                  const int32_t *__restrict__ seq_len,
                                                  const int32_t *__restrict__ table, int maxb,
                                                  int64_t Lmax, int H, int G, int kslots,
                                                  float scale_log2, uint16_t *__restrict__ out) {
    static_assert(R <= 16, "the 16-column core holds one query's heads");
    __shared__ __attribute__((aligned(16))) char lds_k[2][kBlock * D * 2];
    __shared__ __attribute__((aligned(16))) char lds_vt[2][D * kBlock * 2];
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const int kv_row_bytes = G * D * 2;
    const int64_t ng = blockIdx.x;
    const int64_t n = ng / G;
    const int g = (int)(ng % G);
    const int32_t *idr = ids + ng * kslots;
    auto next_valid = [&](int sl) {
        for (; sl < kslots; ++sl)
            if (idr[sl] >= 0) return sl;
        return kslots;
    };
    const int first = next_valid(0);
    if (wave >= 2) {
        const int stid = tid - 2 * kWave;
        using Stage = KVStage<D, 2 * kWave, true>;   // K rows as the 16-column core reads them
        // request slot sl's block (contiguous cache or its page); rows at and past
        // seq_len in the own block are staged as zeros (as in K4d)
        auto request = [&](Stage &x, int sl) {
            const int j = idr[sl];
            const int64_t tok0 =
                table ? (int64_t)table[n * maxb + j] * kBlock : n * Lmax + (int64_t)j * kBlock;
            const int nrows = (int)max<int64_t>(
                1, min<int64_t>(kBlock, (int64_t)seq_len[n] - (int64_t)j * kBlock));
            const int64_t off = (tok0 * G + g) * D;
            x.load(reinterpret_cast<const char *>(kc + off), reinterpret_cast<const char *>(vc + off),
                   kv_row_bytes, nrows, stid);
        };
        Stage sa_regs, sb_regs;
        int sa = first;
        int sb = sa < kslots ? next_valid(sa + 1) : kslots;
        if (sa < kslots) request(sa_regs, sa);
        if (sb < kslots) request(sb_regs, sb);
        int t = 0;
        while (sa < kslots) {
            sa_regs.store(lds_k[t & 1], lds_vt[t & 1], stid);
            const int na = sb < kslots ? next_valid(sb + 1) : kslots;
            if (na < kslots) request(sa_regs, na);
            __syncthreads();                       // barrier t
            ++t;
            if (sb >= kslots) break;
            sb_regs.store(lds_k[t & 1], lds_vt[t & 1], stid);
            const int nb = na < kslots ? next_valid(na + 1) : kslots;
            if (nb < kslots) request(sb_regs, nb);
            __syncthreads();                       // barrier t
            ++t;
            sa = na;
            sb = nb;
        }
    } else if (wave == 0) {
        // head n16 = lane % 16 in every lane quarter; an inactive lane reads the
        // group's first head row and its result is discarded
        const int n16 = lane & 15, qt = lane >> 4;
        const bool active = n16 < R;
        bf16x8 qb[D / 32];
        load_q16<D>(qb, q + (n * H + (int64_t)g * R + (active ? n16 : 0)) * D, qt);
        const int64_t p = (int64_t)seq_len[n] - 1;
        f32x4 acc[D / 16];
#pragma unroll
        for (int md = 0; md < D / 16; ++md) acc[md] = f32x4{};
        float M = -INFINITY, l = 0.0f;
        for (int sl = first, t = 0; sl < kslots; sl = next_valid(sl + 1), ++t) {
            __syncthreads();                       // barrier t
            f32x4 o[D / 16];
            float ms, ls;
            attend16_core<D>(lds_k[t & 1], lds_vt[t & 1], qb, active,
                             p - (int64_t)idr[sl] * kBlock, scale_log2, lane, o, ms, ls);
            const float Mn = fmaxf(M, ms);
            const float a = __builtin_amdgcn_exp2f(M - Mn), b = __builtin_amdgcn_exp2f(ms - Mn);
            l = fmaf(l, a, ls * b);
#pragma unroll
            for (int md = 0; md < D / 16; ++md)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[md][e] = fmaf(acc[md][e], a, o[md][e] * b);
            M = Mn;
        }
        if (active) {
            const float inv = l > 0.0f ? 1.0f / l : 0.0f;
            uint16_t *dst = out + (n * H + (int64_t)g * R + n16) * D + 4 * qt;
#pragma unroll
            for (int md = 0; md < D / 16; ++md)
                store8(dst + 16 * md, u32x2{pack_bf16x2(acc[md][0] * inv, acc[md][1] * inv),
                                            pack_bf16x2(acc[md][2] * inv, acc[md][3] * inv)});
        }
    } else {
        for (int sl = first; sl < kslots; sl = next_valid(sl + 1)) __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// K4d in parts: the valid slots of a (sequence, group) are split into P parts of
// consecutive slots, one work-group each (64 KB of LDS: two work-groups per CU), so
// that twice as many slots are in flight per CU as with one work-group per (sequence,
// group).  Within a part: waves 2-3 stage the next slot's K/V in registers while
// wave 0 attends the current one with the 16-column core and folds it into a running
// merge (as in k4d_online); the part then writes its o normalised (bf16) with its
// log2-sum-exp, po [((n*H + h)*P + part)*D] and plse [((n*G + g)*P + part)*R + h%R],
// and marks the part valid (mark = 0) or empty (-1).  K5 merges the parts.
// ---------------------------------------------------------------------------
template <int D, int R>
__global__ __launch_bounds__(256, 2) void k4d_parts(const uint16_t *__restrict__ q,
                                                 const uint16_t *__restrict__ kc,
                                                 const uint16_t *__restrict__ vc,
                                                 const int32_t *__restrict__ ids,
                                                 const int32_t *__restrict__ seq_len,
                                                 const int32_t *__restrict__ table, int maxb,
                                                 int64_t Lmax, int H, int G, int kslots, int P,
                                                 float scale_log2, uint16_t *__restrict__ po,
                                                 float *__restrict__ plse, int32_t *__restrict__ mark) {
    static_assert(R <= 16, "the 16-column core holds one query's heads");
    __shared__ __attribute__((aligned(16))) char lds_k[kBlock * D * 2];
    __shared__ __attribute__((aligned(16))) char lds_vt[D * kBlock * 2];
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const int kv_row_bytes = G * D * 2;
    const int64_t ngp = blockIdx.x;
    const int part = (int)(ngp % P);
    const int64_t ng = ngp / P;
    const int64_t n = ng / G;
    const int g = (int)(ng % G);
    const int32_t *idr = ids + ng * kslots;
    const int per = (kslots + P - 1) / P;
    const int s_end = min(kslots, (part + 1) * per);
    auto next_valid = [&](int sl) {
        for (; sl < s_end; ++sl)
            if (idr[sl] >= 0) return sl;
        return s_end;
    };
    const int first = next_valid(part * per);
    if (wave >= 2) {
        const int stid = tid - 2 * kWave;
        using Stage = KVStage<D, 2 * kWave, true>;   // K rows as the 16-column core reads them
        // request slot sl's block (contiguous cache or its page); rows at and past
        // seq_len in the own block are staged as zeros (as in K4d)
        auto request = [&](Stage &x, int sl) {
            const int j = idr[sl];
            const int64_t tok0 =
                table ? (int64_t)table[n * maxb + j] * kBlock : n * Lmax + (int64_t)j * kBlock;
            const int nrows = (int)max<int64_t>(
                1, min<int64_t>(kBlock, (int64_t)seq_len[n] - (int64_t)j * kBlock));
            const int64_t off = (tok0 * G + g) * D;
            x.load(reinterpret_cast<const char *>(kc + off), reinterpret_cast<const char *>(vc + off),
                   kv_row_bytes, nrows, stid);
        };
        Stage st;
        int sl = first;
        if (sl < s_end) request(st, sl);
        while (sl < s_end) {
            st.store(lds_k, lds_vt, stid);
            __syncthreads();                       // (A) the slot is in LDS
            const int nxt = next_valid(sl + 1);
            if (nxt < s_end) request(st, nxt);
            __syncthreads();                       // (B) the slot's attention is done
            sl = nxt;
        }
    } else if (wave == 0) {
        // head n16 = lane % 16 in every lane quarter; an inactive lane reads the
        // group's first head row and its result is discarded
        const int n16 = lane & 15, qt = lane >> 4;
        const bool active = n16 < R;
        bf16x8 qb[D / 32];
        load_q16<D>(qb, q + (n * H + (int64_t)g * R + (active ? n16 : 0)) * D, qt);
        const int64_t p = (int64_t)seq_len[n] - 1;
        f32x4 acc[D / 16];
#pragma unroll
        for (int md = 0; md < D / 16; ++md) acc[md] = f32x4{};
        float M = -INFINITY, l = 0.0f;
        for (int sl = first; sl < s_end; sl = next_valid(sl + 1)) {
            __syncthreads();                       // (A)
            f32x4 o[D / 16];
            float ms, ls;
            attend16_core<D>(lds_k, lds_vt, qb, active, p - (int64_t)idr[sl] * kBlock,
                             scale_log2, lane, o, ms, ls);
            const float Mn = fmaxf(M, ms);
            const float a = __builtin_amdgcn_exp2f(M - Mn), b = __builtin_amdgcn_exp2f(ms - Mn);
            l = fmaf(l, a, ls * b);
#pragma unroll
            for (int md = 0; md < D / 16; ++md)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[md][e] = fmaf(acc[md][e], a, o[md][e] * b);
            M = Mn;
            __syncthreads();                       // (B)
        }
        if (lane == 0) mark[ngp] = first < s_end ? 0 : -1;
        if (first < s_end && active) {
            const int64_t h = (int64_t)g * R + n16;
            const float inv = 1.0f / l;
            uint16_t *dst = po + ((n * H + h) * P + part) * D + 4 * qt;
#pragma unroll
            for (int md = 0; md < D / 16; ++md)
                store8(dst + 16 * md, u32x2{pack_bf16x2(acc[md][0] * inv, acc[md][1] * inv),
                                            pack_bf16x2(acc[md][2] * inv, acc[md][3] * inv)});
            if (qt == 0) plse[(ng * P + part) * R + n16] = M + __log2f(l);
        }
    } else {
        for (int sl = first; sl < s_end; sl = next_valid(sl + 1)) {
            __syncthreads();                       // (A)
            __syncthreads();                       // (B)
        }
    }
}

hipError_t launch_k4d_parts(const uint16_t *q, const uint16_t *kc, const uint16_t *vc,
                            const int32_t *ids, const int32_t *seq_len, const int32_t *table,
                            int maxb, int N, int64_t Lmax, int H, int G, int d, int k, int P,
                            float scale, uint16_t *po, float *plse, int32_t *mark,
                            hipStream_t s) {
    if (N <= 0) return hipSuccess;
    const float sl2 = scale * kLog2e;
    const int R = H / G;
    const dim3 grid((unsigned)((int64_t)N * G * P));
#define K4DP_CASE(dd, rr)                                                                         \
    if (d == dd && R == rr) {                                                                    \
        hipLaunchKernelGGL((k4d_parts<dd, rr>), grid, dim3(256), 0, s, q, kc, vc, ids, seq_len,   \
                           table, maxb, Lmax, H, G, k, P, sl2, po, plse, mark);                  \
        return hipGetLastError();                                                                \
    }
    K4DP_CASE(64, 1) K4DP_CASE(64, 2) K4DP_CASE(64, 4) K4DP_CASE(64, 8) K4DP_CASE(64, 16)
    K4DP_CASE(128, 1) K4DP_CASE(128, 2) K4DP_CASE(128, 4) K4DP_CASE(128, 8) K4DP_CASE(128, 16)
#undef K4DP_CASE
    return hipErrorNotSupported;
}

hipError_t launch_k4d_online(const uint16_t *q, const uint16_t *kc, const uint16_t *vc,
                             const int32_t *ids, const int32_t *seq_len, const int32_t *table,
                             int maxb, int N, int64_t Lmax, int H, int G, int d, int k, float scale,
                             uint16_t *out, hipStream_t s) {
    if (N <= 0) return hipSuccess;
    const float sl2 = scale * kLog2e;
    const int R = H / G;
    const dim3 grid((unsigned)((int64_t)N * G));
#define K4DO_CASE(dd, rr)                                                                         \
    if (d == dd && R == rr) {                                                                    \
        hipLaunchKernelGGL((k4d_online<dd, rr>), grid, dim3(256), 0, s, q, kc, vc, ids, seq_len,  \
                           table, maxb, Lmax, H, G, k, sl2, out);                                \
        return hipGetLastError();                                                                \
    }
    K4DO_CASE(64, 1) K4DO_CASE(64, 2) K4DO_CASE(64, 4) K4DO_CASE(64, 8) K4DO_CASE(64, 16)
    K4DO_CASE(128, 1) K4DO_CASE(128, 2) K4DO_CASE(128, 4) K4DO_CASE(128, 8) K4DO_CASE(128, 16)
#undef K4DO_CASE
    return hipErrorNotSupported;
}

bool k4d_online_supported(int d, int R) { return (d == 64 || d == 128) && R >= 1 && R <= 16; }

// ---------------------------------------------------------------------------
// K5: combine.  One thread per (query, head, 8 d values).  The partials of all
// valid slots of a thread are requested at once; a slot is valid when
// 0 <= id < nb_lim -- the rule K3 used to build the lists -- so stale workspace
// contents never enter the result, and padding slots (rows with fewer than k
// selectable blocks) cost no memory traffic.
//
// Two partial layouts:
//   UNNORM (prefill, K4): o unnormalised with (maximum, sum) pairs; the partials of a
//     (query, group, slot) are one block of R heads x D/8 chunks, chunk-major
//     (chunk c of head h at (c * R + h) * 16 bytes).  Thread T takes block row
//     bq = T / (R * D/8) (= query * G + group), chunk c = (T % (R * D/8)) / R and head
//     h = T % R, so a wave reads whole runs of a block.
//   !UNNORM (decode's split form): o normalised with its log2-sum-exp; one row of D
//     per (query, head, slot).  Thread T takes item T / (D/8) = query * H + head,
//     chunk T % (D/8).
// ---------------------------------------------------------------------------
struct K5Map {
    int64_t bq;        // query * G + group
    int hl;            // head within the group
    int c;             // 16-byte chunk of the d values
};

template <int D, bool UNNORM>
__device__ __forceinline__ K5Map k5_map(int64_t T, int R) {
    constexpr int TPH = D / 8;
    K5Map m;
    if constexpr (UNNORM) {
        const int64_t n = (int64_t)R * TPH;
        m.bq = T / n;
        const int w = (int)(T - m.bq * n);
        m.c = w / R;
        m.hl = w - m.c * R;
    } else {
        const int64_t ih = T / TPH;
        m.c = (int)(T - ih * TPH);
        m.bq = ih / R;
        m.hl = (int)(ih - m.bq * R);
    }
    return m;
}

// Where thread m's chunk of slot 0 lives, and the distance between slots.
template <int D, bool UNNORM>
__device__ __forceinline__ const uint16_t *k5_partial(const uint16_t *po, const K5Map &m, int R,
                                                      int kslots, int64_t &slot_stride) {
    if constexpr (UNNORM) {
        slot_stride = (int64_t)R * D;
        return po + m.bq * kslots * R * D + m.c * (R * 8) + m.hl * 8;
    } else {
        slot_stride = D;
        return po + (m.bq * R + m.hl) * kslots * D + m.c * 8;
    }
}

// The merge of thread T's share (valid and in range), from its partials.
template <int D, int KMAX, bool UNNORM>
__device__ __forceinline__ u32x4 k5_share(const uint16_t *__restrict__ po,
                                          const float *__restrict__ plse,
                                          const int32_t *__restrict__ ids, const K5Map &mp, int R,
                                          int G, int kslots, int nb_lim, const BatchMap &bm) {
    const int64_t i = mp.bq / G;
    const int32_t *idr = ids + mp.bq * kslots;
    // batch: ids are local to the row's sequence and valid up to its own block
    if (bm.row_len) nb_lim = (bm.row_len[i] - 1) / kBlock + 1;
    // slot s at lr[s * R] (normalised partials: log2-sum-exp) or mlr[s * R]
    // (unnormalised: row maximum and row sum)
    const float *lr = plse + mp.bq * kslots * R + mp.hl;
    const f32x2 *mlr = reinterpret_cast<const f32x2 *>(plse) + mp.bq * kslots * R + mp.hl;
    int64_t ss;
    const uint16_t *pr = k5_partial<D, UNNORM>(po, mp, R, kslots, ss);
    u32x4 v[KMAX];
    float l[KMAX];
    f32x2 ml[KMAX];
    bool ok[KMAX];
    if (kslots == KMAX) {
        // full rows: ids as 16-byte vectors (rows are 16-byte aligned)
#pragma unroll
        for (int s4 = 0; s4 < KMAX / 4; ++s4) {
            const u32x4 iv = load16(idr + 4 * s4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int id = (int)iv[e];
                ok[4 * s4 + e] = id >= 0 && id < nb_lim;
            }
        }
#pragma unroll
        for (int s = 0; s < KMAX; ++s) {
            if constexpr (UNNORM) ml[s] = ok[s] ? mlr[s * R] : f32x2{0.0f, 0.0f};
            else l[s] = ok[s] ? lr[s * R] : 0.0f;
            v[s] = ok[s] ? load16_stream(pr + s * ss) : u32x4{0, 0, 0, 0};
        }
    } else {
#pragma unroll
        for (int s = 0; s < KMAX; ++s) {
            if (s < kslots) {
                const int id = idr[s];
                ok[s] = id >= 0 && id < nb_lim;
                if constexpr (UNNORM) ml[s] = ok[s] ? mlr[s * R] : f32x2{0.0f, 0.0f};
                else l[s] = ok[s] ? lr[s * R] : 0.0f;
                v[s] = ok[s] ? load16_stream(pr + s * ss) : u32x4{0, 0, 0, 0};
            } else {
                ok[s] = false;
            }
        }
    }
    if constexpr (UNNORM) return ml_merge<KMAX>(v, ml, ok);
    else return lse_merge<KMAX>(v, l, ok);
}

template <int D, int KMAX, bool UNNORM>
__global__ __launch_bounds__(256) void k5_combine(const uint16_t *__restrict__ po,
                                                  const float *__restrict__ plse,
                                                  const int32_t *__restrict__ ids, int64_t nq,
                                                  int H, int G, int kslots, int nb_lim,
                                                  uint16_t *__restrict__ out, const BatchMap bm) {
    const int R = H / G;
    const int64_t T = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t n_thr = nq * H * (D / 8);
    const bool live = T < n_thr;
    K5Map mp{0, 0, 0};
    u32x4 r = {0, 0, 0, 0};
    if (live) {
        mp = k5_map<D, UNNORM>(T, R);
        r = k5_share<D, KMAX, UNNORM>(po, plse, ids, mp, R, G, kslots, nb_lim, bm);
    }
    const int64_t o_idx = (mp.bq * R + mp.hl) * (D / 8) + mp.c;   // output chunk
    // Chunk-major blocks that fit a work-group whole (R * D/8 <= 256, a divisor of
    // 256) give it the output chunks [256 b, 256 b + 256) -- the same set as its
    // threads' T, since whole blocks are live or not -- in another order: the
    // results are exchanged through LDS so that the stores write them contiguously.
    if (UNNORM && R * (D / 8) <= 256) {
        // one 16-byte pad per 16 entries: the writes (16 heads of one chunk, 256 B
        // apart) then fall in distinct banks
        __shared__ u32x4 lds_out[256 + 16];
        const int e = (int)(o_idx - (int64_t)blockIdx.x * 256);
        if (live) lds_out[e + (e >> 4)] = r;
        __syncthreads();
        if (live) store16_stream(out + T * 8, lds_out[threadIdx.x + (threadIdx.x >> 4)]);
    } else if (live) {
        store16_stream(out + o_idx * 8, r);
    }
}

template <int D, int KMAX, bool UNNORM>
__global__ __launch_bounds__(256) void k5_combine_strided(const uint16_t *__restrict__ po,
                                                  const float *__restrict__ plse,
                                                  const int32_t *__restrict__ ids, int64_t nq,
                                                  int H, int G, int kslots, int nb_lim,
                                                  uint16_t *__restrict__ out, const BatchMap bm) {
    const int64_t n_thr = nq * H * (D / 8);
    const int64_t stride = (int64_t)gridDim.x * 256;
    const int R = H / G;
    // Rows with few valid slots (a batch of short sequences) leave k5_combine bound by
    // two memory round trips per thread: ids, then the partials they select.  Here
    // each thread walks its shares with a grid stride, one ahead: the next share's ids
    // row (and in a batch its length) are requested with the current share's
    // partials.  Same merge, bitwise the same output; for full rows the extra
    // registers (three waves per SIMD instead of four) cost more than it saves.
    struct Sel {
        int id[KMAX];
        int lim;
    };
    auto fetch = [&](int64_t T, Sel &x) {
        const K5Map mp = k5_map<D, UNNORM>(T < n_thr ? T : 0, R);
        const int32_t *idr = ids + mp.bq * kslots;
        if (kslots == KMAX) {
            // full rows: ids as 16-byte vectors (rows are 16-byte aligned)
#pragma unroll
            for (int s4 = 0; s4 < KMAX / 4; ++s4) {
                const u32x4 iv = load16(idr + 4 * s4);
#pragma unroll
                for (int e = 0; e < 4; ++e) x.id[4 * s4 + e] = (int)iv[e];
            }
        } else {
#pragma unroll
            for (int s = 0; s < KMAX; ++s) x.id[s] = s < kslots ? idr[s] : -1;
        }
        // batch: ids are local to the row's sequence and valid up to its own block
        x.lim = bm.row_len ? (bm.row_len[mp.bq / G] - 1) / kBlock + 1 : nb_lim;
    };
    auto step = [&](int64_t T, const Sel &cur, Sel &nxt) {
        const K5Map mp = k5_map<D, UNNORM>(T, R);
        // slot s at lr[s * R] (normalised partials: log2-sum-exp) or mlr[s * R]
        // (unnormalised: row maximum and row sum)
        const float *lr = plse + mp.bq * kslots * R + mp.hl;
        const f32x2 *mlr = reinterpret_cast<const f32x2 *>(plse) + mp.bq * kslots * R + mp.hl;
        int64_t ss;
        const uint16_t *pr = k5_partial<D, UNNORM>(po, mp, R, kslots, ss);
        u32x4 v[KMAX];
        float l[KMAX];
        f32x2 ml[KMAX];
        bool ok[KMAX];
#pragma unroll
        for (int s = 0; s < KMAX; ++s) {
            ok[s] = cur.id[s] >= 0 && cur.id[s] < cur.lim;
            if constexpr (UNNORM) ml[s] = ok[s] ? mlr[s * R] : f32x2{0.0f, 0.0f};
            else l[s] = ok[s] ? lr[s * R] : 0.0f;
            v[s] = ok[s] ? load16_stream(pr + s * ss) : u32x4{0, 0, 0, 0};
        }
        fetch(T + stride, nxt);
        uint16_t *dst = out + (mp.bq * R + mp.hl) * D + mp.c * 8;
        if constexpr (UNNORM) store16_stream(dst, ml_merge<KMAX>(v, ml, ok));
        else store16_stream(dst, lse_merge<KMAX>(v, l, ok));
    };
    int64_t T = (int64_t)blockIdx.x * 256 + threadIdx.x;
    Sel sa, sb;
    fetch(T, sa);
    for (; T < n_thr; T += 2 * stride) {
        step(T, sa, sb);
        if (T + stride < n_thr) step(T + stride, sb, sa);
    }
}

template <int D, int KMAX, bool UNNORM>
static void k5_launch(const uint16_t *po, const float *plse, const int32_t *ids, int64_t nq,
                      int H, int G, int k, int nb_lim, uint16_t *out, const BatchMap &bm,
                      bool sparse_rows, hipStream_t s) {
    const int64_t need = (nq * H * (D / 8) + 255) / 256;
    if (sparse_rows) {
        // enough work-groups to fill the part several times over; each thread then
        // walks its items with a stride
        constexpr int64_t kMaxGrid = 4096;
        hipLaunchKernelGGL((k5_combine_strided<D, KMAX, UNNORM>),
                           dim3((unsigned)(need < kMaxGrid ? need : kMaxGrid)), dim3(256), 0, s,
                           po, plse, ids, nq, H, G, k, nb_lim, out, bm);
    } else {
        hipLaunchKernelGGL((k5_combine<D, KMAX, UNNORM>), dim3((unsigned)need), dim3(256), 0, s,
                           po, plse, ids, nq, H, G, k, nb_lim, out, bm);
    }
}

template <int D, bool UNNORM>
static hipError_t k5_dispatch(const uint16_t *po, const float *plse, const int32_t *ids,
                              int64_t nq, int H, int G, int k, int nb_lim, uint16_t *out,
                              const BatchMap &bm, bool sparse_rows, hipStream_t s) {
    if (k <= 4) k5_launch<D, 4, UNNORM>(po, plse, ids, nq, H, G, k, nb_lim, out, bm, sparse_rows, s);
    else if (k <= 8) k5_launch<D, 8, UNNORM>(po, plse, ids, nq, H, G, k, nb_lim, out, bm, sparse_rows, s);
    else if (k <= 16) k5_launch<D, 16, UNNORM>(po, plse, ids, nq, H, G, k, nb_lim, out, bm, sparse_rows, s);
    else k5_launch<D, 32, UNNORM>(po, plse, ids, nq, H, G, k, nb_lim, out, bm, sparse_rows, s);
    return hipGetLastError();
}

hipError_t launch_k5_combine(const uint16_t *po, const float *plse, const int32_t *ids, int64_t nq,
                             int H, int G, int d, int k, int nb_lim, uint16_t *out,
                             const BatchMap &bm, bool unnorm, bool sparse_rows, hipStream_t s) {
    if (nq <= 0) return hipSuccess;
    if (d == 64)
        return unnorm ? k5_dispatch<64, true>(po, plse, ids, nq, H, G, k, nb_lim, out, bm, sparse_rows, s)
                      : k5_dispatch<64, false>(po, plse, ids, nq, H, G, k, nb_lim, out, bm, sparse_rows, s);
    if (d == 128)
        return unnorm ? k5_dispatch<128, true>(po, plse, ids, nq, H, G, k, nb_lim, out, bm, sparse_rows, s)
                      : k5_dispatch<128, false>(po, plse, ids, nq, H, G, k, nb_lim, out, bm, sparse_rows, s);
    return hipErrorInvalidValue;
}

}  // namespace msa
