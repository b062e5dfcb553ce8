// msa_api.hip -- the C ABI of libmsa.so (declared in include/msa.h): argument
// validation, workspace carving and the launch sequence of each entry point.
//
// Prefill runs over query chunks so that the workspace stays bounded at any L
// (block scores and partials are per chunk): the preferred chunk is kChunkQ
// queries; a caller that passes a smaller workspace gets the largest chunk
// (a multiple of 128 queries) that fits.  Every query's result is independent of
// the chunking.  Per chunk:
//   K1 index score + block max-pool -> K2 exp-free top-k -> K3 schedule ->
//   K4 KV-outer attention -> K5 combine.
// Decode: K1d -> K2 -> K4d -> K5 (paged decode: page-table check first; FP8
// index-key cache: the E4M3 variant of K1d).
// The compute entry points never allocate device memory, free or synchronise;
// only the optional timing calls at the end create events and synchronise.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <mutex>
#include <new>

#include "msa.h"
#include "msa_launch.h"

namespace {

using namespace msa;

constexpr int64_t kChunkQ = 131072;    // preferred queries per prefill chunk
constexpr size_t kAlign = 256;
// decode attention: one work-group per (sequence, group) once a launch has that many
// (one per CU of the 256-CU part); fewer pairs split their slots into parts, two
// work-groups per CU
constexpr int64_t kDecodeOneLaunchPairs = 256;
constexpr int64_t kDecodePartWorkGroups = 512;

// Workspace carving: with base == nullptr only the size is accumulated.  With a
// buffer, `cap` is its size: every entry point checks fits() after carving and
// before its first launch, so a planner that carved more than the buffer holds is
// an error, never an out-of-bounds write.
struct Carver {
    char *base;
    size_t cap;
    size_t used = 0;
    explicit Carver(void *b, size_t capacity = SIZE_MAX)
        : base(static_cast<char *>(b)), cap(capacity) {}
    template <typename T>
    T *take(int64_t count) {
        used = (used + kAlign - 1) / kAlign * kAlign;
        T *p = base ? reinterpret_cast<T *>(base + used) : nullptr;
        used += (size_t)std::max<int64_t>(count, 0) * sizeof(T);
        return p;
    }
    bool fits() const { return used <= cap; }
};
#define MSA_CHECK_CARVE(c)                                             \
    do {                                                               \
        if (!(c).fits()) return MSA_ERR_WORKSPACE_TOO_SMALL;           \
    } while (0)

struct AttnWs {
    SchedBuffers sb;
    uint16_t *po;
    float *plse;
};

AttnWs carve_attn(Carver &c, int64_t C, int H, int G, int d, int k, int nb) {
    AttnWs w;
    const int64_t lists = (int64_t)G * nb;
    w.sb.counts = c.take<int>(lists);
    w.sb.offs = c.take<int>(lists + 1);
    w.sb.toff = c.take<int>(lists + 1);
    w.sb.wcnt = c.take<int>((int64_t)k3_num_groups(C, G) * lists);
    w.sb.total = c.take<int>(1);
    const int64_t max_items = k4_max_items(C, G, k, nb);
    w.sb.items = c.take<int>(max_items);
    w.sb.order = c.take<int>(max_items);
    w.sb.tcnt = c.take<int>(k3_tile_groups(max_items) * kK3Buckets);
    w.sb.list = c.take<uint32_t>(C * G * k);
    w.po = c.take<uint16_t>(C * H * k * d);
    w.plse = c.take<float>(2 * C * H * k);   // (maximum, sum) per partial row
    return w;
}

int64_t chunk_of(int64_t L) { return std::min<int64_t>(round_up(std::max<int64_t>(L, 1), kBlock), kChunkQ); }
int64_t nblocks(int64_t L) { return (L + kBlock - 1) / kBlock; }

// Valid selection slots over queries at positions [p0, p1): a query in block j has
// min(k, j + 1) candidate blocks (its own and the earlier ones), the rest are -1.
int64_t valid_slots(int64_t p0, int64_t p1, int k) {
    int64_t n = 0;
    for (int64_t j = p0 / kBlock; j * kBlock < p1; ++j) {
        const int64_t a = std::max(p0, j * kBlock), b = std::min(p1, (j + 1) * kBlock);
        n += (b - a) * std::min<int64_t>(k, j + 1);
    }
    return n;
}

// Rows that hold fewer valid slots than empty ones on the whole take K5's grid-stride
// form (its one round trip per row beats the extra registers it needs).
bool sparse_rows(int64_t valid, int64_t rows, int k) { return 2 * valid < rows * k; }
int nb_padded(int64_t L) { return (int)round_up(std::max<int64_t>(nblocks(L), 1), 8); }

// Index branch of a query chunk [q0, qend): the fused kernel K12 (no block scores in
// memory) when it serves the shape, the chunk's rows are long and alike -- its
// shortest row has at least as many competitor blocks as the chunk has query
// blocks, so that its work-groups (one per 64 queries, over all their key blocks)
// run for similar times and sweep the key tiles together, reusing them from L2 --
// and the chunk has enough queries for K12's work-groups to fill the part.
// Otherwise K1 (32-block key chunks, L2-friendly for the triangle of short rows,
// and many short items) and K2.
// MSA_FUSED_INDEX=1 in the environment (read at every chunk) uses K12 for every
// chunk whose rows are long, however few work-groups it gets (tests use it to run
// K12 on small shapes).  The ids are the same either way.
bool use_k12(int64_t q0, int64_t qend, int G, int dI, int k) {
    if (!k12_supported(G, dI, k)) return false;
    if (q0 / kBlock < (qend - q0 + kBlock - 1) / kBlock) return false;
    const char *e = getenv("MSA_FUSED_INDEX");
    return (e && e[0] == '1') || k12_num_workgroups(qend - q0, G) >= kK12MinWorkgroups;
}
// Workspace: K12's candidate lists and the block scores of the chunks K1 + K2
// serve.  Where K12 takes the chunks whose rows are long (chunks of C queries give
// it enough work-groups), K1 serves only chunks that end before 2C, which bounds
// their rows; otherwise the rows must hold every key block of the sequence.
struct IndexWs {
    float *S = nullptr;        // K1 + K2
    int64_t s_floats = 0;      // its capacity
    uint64_t *cand = nullptr;  // K12
};
IndexWs carve_index(Carver &c, int64_t C, int64_t L, int G, int dI, int k) {
    IndexWs w;
    int64_t nb = nb_padded(L);
    if (k12_supported(G, dI, k)) {
        w.cand = c.take<uint64_t>(k12_cand_entries(C, G));
        if (k12_num_workgroups(C, G) >= kK12MinWorkgroups) nb = nb_padded(std::min(L, 2 * C));
    }
    w.s_floats = C * G * nb;
    w.S = c.take<float>(w.s_floats);
    return w;
}
size_t select_bytes(int64_t C, int64_t L, int G, int dI, int k) {
    Carver c(nullptr);
    carve_index(c, C, L, G, dI, k);
    return c.used;
}
size_t attn_bytes(int64_t C, int64_t L, int H, int G, int d, int k) {
    Carver c(nullptr);
    carve_attn(c, C, H, G, d, k, (int)nblocks(L));
    return c.used;
}
size_t prefill_bytes(int64_t C, int64_t L, int H, int G, int d, int dI, int k) {
    Carver c(nullptr);
    carve_index(c, C, L, G, dI, k);
    c.take<int32_t>(C * G * k);
    carve_attn(c, C, H, G, d, k, (int)nblocks(L));
    return c.used;
}

// Largest chunk (preferred size, then halving in multiples of 128 queries) whose
// workspace fits in ws_bytes; 0 when not even one 128-query chunk fits.
template <typename SizeFn>
int64_t fit_chunk(int64_t L, size_t ws_bytes, SizeFn size_of) {
    int64_t C = chunk_of(L);
    while (C > kBlock && size_of(C) > ws_bytes) C = round_up(C / 2, kBlock);
    return size_of(C) <= ws_bytes ? C : 0;
}

int check_ptr(void *ws) {
    return (!ws || (reinterpret_cast<uintptr_t>(ws) % kAlign)) ? MSA_ERR_WORKSPACE_TOO_SMALL : MSA_OK;
}

bool r_ok(int H, int G) {
    if (G <= 0 || H % G) return false;
    const int r = H / G;
    return r == 1 || r == 2 || r == 4 || r == 8 || r == 16 || r == 32;
}
bool d_ok(int d) { return d == 64 || d == 128; }
// The scheduler keeps two LDS counters per block of a group: at most 8192 blocks.
constexpr int64_t kMaxPrefillLen = 8192 * (int64_t)kBlock;
bool index_ok(int G, int dI) {
    return (G == 1 || G == 2 || G == 4 || G == 8) && (dI == 32 || dI == 64 || dI == 128) &&
           G * dI <= 512;
}

int check_ws(void *ws, size_t ws_bytes, size_t need) {
    if (need == 0) return MSA_OK;
    if (!ws || (reinterpret_cast<uintptr_t>(ws) % kAlign)) return MSA_ERR_WORKSPACE_TOO_SMALL;
    return ws_bytes >= need ? MSA_OK : MSA_ERR_WORKSPACE_TOO_SMALL;
}

float default_scale(float scale, int d) { return scale > 0.0f ? scale : 1.0f / sqrtf((float)d); }

// ---- optional per-kernel timing (see msa_timing_enable in msa.h) ----------
struct TimedLaunch {
    int name;
    hipEvent_t start, stop;
};
enum StageName { kK1, kK2, kK3, kK4, kK5, kK1d, kK4d, kKpc, kK1d8, kQuant, kK4dm, kK12, kK4do,
                 kK4dp, kKd, kNumStages };
const char *const kStageNames[kNumStages] = {"k1_index_pool", "k2_select", "k3_schedule",
                                             "k4_kv_outer", "k5_combine", "k1d_index_pool",
                                             "k4d_split", "page_check", "k1d_index_pool_fp8",
                                             "quantize_e4m3", "k4d_merge", "k12_index_select",
                                             "k4d_online", "k4d_parts", "kd_dense"};
struct Timing {
    bool on = false;
    int cap = 0, used = 0;
    TimedLaunch *rec = nullptr;
};
Timing g_timing;

// Debug aid: with MSA_DEBUG_SYNC=1 in the environment every stage is followed by a
// synchronisation of its stream, so an asynchronous fault is reported (on stderr,
// as MSA_ERR_HIP) by the call and stage that caused it.  Not for use under graph
// capture, where synchronising is not allowed.  Read at every stage, so a process
// may switch it on and off.
bool debug_sync() {
    const char *e = getenv("MSA_DEBUG_SYNC");
    return e && e[0] == '1';
}

hipError_t after_stage(int stage, hipStream_t s, hipError_t e) {
    if (e != hipSuccess || !debug_sync()) return e;
    const hipError_t w = hipStreamSynchronize(s);
    const hipError_t l = hipGetLastError();
    const hipError_t r = w != hipSuccess ? w : l;
    if (r != hipSuccess)
        fprintf(stderr, "[msa] stage %s failed: %s\n", kStageNames[stage], hipGetErrorString(r));
    return r;
}

// Runs `launch` (returning hipError_t), bracketed by events when timing is on.
template <typename F>
hipError_t timed(int stage, hipStream_t s, F &&launch) {
    if (!g_timing.on || g_timing.used >= g_timing.cap) return after_stage(stage, s, launch());
    TimedLaunch &t = g_timing.rec[g_timing.used];
    if (hipEventRecord(t.start, s) != hipSuccess) return hipErrorUnknown;
    const hipError_t e = launch();
    if (e != hipSuccess) return e;
    if (hipEventRecord(t.stop, s) != hipSuccess) return hipErrorUnknown;
    t.name = stage;
    ++g_timing.used;
    return after_stage(stage, s, hipSuccess);
}

#define MSA_TRY(expr)                                   \
    do {                                                \
        if ((expr) != hipSuccess) return MSA_ERR_HIP;   \
    } while (0)
#define MSA_TIMED(stage, expr) MSA_TRY(timed(stage, s, [&]() { return (expr); }))

// Index branch of queries [q0, qend): ids [(i-q0)*G + g][k] at ids_c.
int index_chunk(const IndexWs &w, const uint16_t *idx_q, const uint16_t *idx_k, int64_t L,
                int64_t q0, int64_t qend, int G, int dI, int k, int32_t *ids_c, hipStream_t s) {
    // block-score rows of the chunk's own length; K1 + K2 only where the carve holds
    // them (otherwise K12, which needs no block scores and gives the same ids)
    const int nbp = k12_supported(G, dI, k) ? nb_padded(qend) : nb_padded(L);
    const bool k1_fits = (qend - q0) * G * (int64_t)nbp <= w.s_floats;
    if (use_k12(q0, qend, G, dI, k) || (!k1_fits && k12_supported(G, dI, k))) {
        MSA_TIMED(kK12, launch_k12_index_select(idx_q, idx_k, ids_c, w.cand, q0, qend, G, dI, k, s));
        return MSA_OK;
    }
    if (!k1_fits) return MSA_ERR_WORKSPACE_TOO_SMALL;   // unreachable: the carve holds nb_padded(L)
    MSA_TIMED(kK1, launch_k1_index_pool(idx_q, idx_k, w.S, L, q0, qend, G, dI, nbp, s));
    MSA_TIMED(kK2, launch_k2_select(w.S, nbp, (qend - q0) * G, G, k, q0, nullptr, 0, ids_c, s));
    return MSA_OK;
}

// Shared by prefill and sparse_attn: K3 + K4 + K5 for queries [q0, qend).
int attn_chunk(const uint16_t *q, const uint16_t *kx, const uint16_t *vx, const int32_t *ids_c,
               int64_t L, int64_t q0, int64_t qend, int H, int G, int d, int k, float scale,
               uint16_t *out, const AttnWs &w, hipStream_t s) {
    const int64_t C = qend - q0;
    const int nbc = (int)((qend - 1) / kBlock + 1);
    const BatchMap single;
    MSA_TIMED(kK3, launch_k3_schedule(ids_c, C, G, k, nbc, w.sb, single, s));
    MSA_TIMED(kK4, launch_k4_kv_outer(q, kx, vx, w.sb, nbc, L, q0, C, H, G, d, k, scale, w.po, w.plse,
                                      single, s));
    MSA_TIMED(kK5, launch_k5_combine(w.po, w.plse, ids_c, C, H, G, d, k, nbc, out + q0 * H * d,
                                     single, true, sparse_rows(valid_slots(q0, qend, k), C, k), s));
    return MSA_OK;
}

// Decode main branch over the selected slots.  Up to 16 heads per group: one launch
// with a running merge per (sequence, group) once there are 256 such pairs, else the
// slots in parts (two work-groups per CU) merged by K5.  32 heads per group: the
// launch that merges each (sequence, group)'s slots in LDS where their partials fit,
// else K4d + K5 (same output bits).  po / plse hold the parts' or the slots' partials,
// mark the parts' validity.
int decode_attend(const uint16_t *q, const uint16_t *kc, const uint16_t *vc, const int32_t *ids,
                  const int32_t *len, const int32_t *table, int maxb, int N, int64_t Lmax, int H,
                  int G, int d, int kslots, float scale, uint16_t *po, float *plse, int32_t *mark,
                  uint16_t *out, hipStream_t s) {
    if (k4d_online_supported(d, H / G)) {
        // parts per (sequence, group) for small batches: enough work-groups for two per CU
        const int64_t ng = (int64_t)N * G;
        const int P = ng >= kDecodeOneLaunchPairs
                          ? 1
                          : (int)std::min<int64_t>(kslots, (kDecodePartWorkGroups + ng - 1) / ng);
        if (P > 1) {
            MSA_TIMED(kK4dp, launch_k4d_parts(q, kc, vc, ids, len, table, maxb, N, Lmax, H, G, d,
                                              kslots, P, scale, po, plse, mark, s));
            MSA_TIMED(kK5, launch_k5_combine(po, plse, mark, N, H, G, d, P, 1, out, BatchMap{},
                                             false, false, s));
            return MSA_OK;
        }
        MSA_TIMED(kK4do, launch_k4d_online(q, kc, vc, ids, len, table, maxb, N, Lmax, H, G, d,
                                           kslots, scale, out, s));
        return MSA_OK;
    }
    if (k4d_merge_supported(d, H / G, kslots)) {
        MSA_TIMED(kK4dm, launch_k4d_merge(q, kc, vc, ids, len, table, maxb, N, Lmax, H, G, d,
                                          kslots, scale, out, s));
        return MSA_OK;
    }
    MSA_TIMED(kK4d, launch_k4d_split(q, kc, vc, ids, len, table, maxb, N, Lmax, H, G, d, kslots,
                                     scale, po, plse, s));
    MSA_TIMED(kK5, launch_k5_combine(po, plse, ids, N, H, G, d, kslots, 0x7FFFFFFF, out,
                                     BatchMap{}, false, false, s));
    return MSA_OK;
}

}  // namespace

extern "C" {

const char *msa_status_string(int status) {
    switch (status) {
    case MSA_OK: return "MSA_OK";
    case MSA_ERR_INVALID_ARG: return "MSA_ERR_INVALID_ARG";
    case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED";
    case MSA_ERR_WORKSPACE_TOO_SMALL: return "MSA_ERR_WORKSPACE_TOO_SMALL";
    case MSA_ERR_HIP: return "MSA_ERR_HIP";
    default: return "MSA_ERR_UNKNOWN";
    }
}

// ------------------------------- select -----------------------------------
size_t msa_select_blocks_workspace_size(int64_t L, int G, int dI, int B, int k) {
    (void)B;
    if (L <= 0 || G <= 0) return 0;
    return select_bytes(chunk_of(L), L, G, dI, k);
}

int msa_select_blocks(const uint16_t *idx_q, const uint16_t *idx_k, int64_t L, int G, int dI,
                      int B, int k, int32_t *block_ids, void *ws, size_t ws_bytes, void *stream) {
    if (L < 0 || G <= 0 || dI <= 0 || B <= 0 || k < 1) return MSA_ERR_INVALID_ARG;
    if (L == 0) return MSA_OK;
    if (!idx_q || !idx_k || !block_ids) return MSA_ERR_INVALID_ARG;
    if (B != kBlock || !index_ok(G, dI) || k > 32) return MSA_ERR_UNSUPPORTED;
    if (check_ptr(ws) != MSA_OK) return MSA_ERR_WORKSPACE_TOO_SMALL;
    const int64_t C =
        fit_chunk(L, ws_bytes, [&](int64_t c) { return select_bytes(c, L, G, dI, k); });
    if (C == 0) return MSA_ERR_WORKSPACE_TOO_SMALL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Carver c(ws, ws_bytes);
    const IndexWs iw = carve_index(c, C, L, G, dI, k);
    MSA_CHECK_CARVE(c);
    for (int64_t q0 = 0; q0 < L; q0 += C) {
        const int64_t qend = std::min(L, q0 + C);
        const int rc = index_chunk(iw, idx_q, idx_k, L, q0, qend, G, dI, k, block_ids + q0 * G * k, s);
        if (rc != MSA_OK) return rc;
    }
    return MSA_OK;
}

// ----------------------------- sparse attn --------------------------------
size_t msa_sparse_attn_workspace_size(int64_t L, int H, int G, int d, int B, int kslots) {
    (void)B;
    if (L <= 0 || G <= 0 || H <= 0 || d <= 0 || kslots <= 0) return 0;
    return attn_bytes(chunk_of(L), L, H, G, d, kslots);
}

int msa_sparse_attn(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                    const int32_t *block_ids, int64_t L, int H, int G, int d, int B, int kslots,
                    float scale, uint16_t *out, void *ws, size_t ws_bytes, void *stream) {
    if (L < 0 || H <= 0 || G <= 0 || d <= 0 || B <= 0 || kslots < 1 || H % G)
        return MSA_ERR_INVALID_ARG;
    if (L == 0) return MSA_OK;
    if (!q || !k || !v || !block_ids || !out) return MSA_ERR_INVALID_ARG;
    if (B != kBlock || !d_ok(d) || !r_ok(H, G) || kslots > 32 || L > kMaxPrefillLen)
        return MSA_ERR_UNSUPPORTED;
    if (check_ptr(ws) != MSA_OK) return MSA_ERR_WORKSPACE_TOO_SMALL;
    const int64_t C = fit_chunk(L, ws_bytes,
                                [&](int64_t c) { return attn_bytes(c, L, H, G, d, kslots); });
    if (C == 0) return MSA_ERR_WORKSPACE_TOO_SMALL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    scale = default_scale(scale, d);
    Carver c(ws, ws_bytes);
    const AttnWs w = carve_attn(c, C, H, G, d, kslots, (int)nblocks(L));
    MSA_CHECK_CARVE(c);
    for (int64_t q0 = 0; q0 < L; q0 += C) {
        const int64_t qend = std::min(L, q0 + C);
        const int rc = attn_chunk(q, k, v, block_ids + q0 * G * kslots, L, q0, qend, H, G, d, kslots,
                                  scale, out, w, s);
        if (rc != MSA_OK) return rc;
    }
    return MSA_OK;
}

// -------------------------------- prefill ---------------------------------
size_t msa_prefill_workspace_size(int64_t L, int H, int G, int d, int dI, int B, int k) {
    (void)dI; (void)B;
    if (L <= 0 || G <= 0 || H <= 0 || d <= 0 || k <= 0) return 0;
    return prefill_bytes(chunk_of(L), L, H, G, d, dI, k);
}

}  // extern "C"

namespace {

// A sequence of at most k blocks keeps every causal block for every query (its own
// block and all earlier ones are at most k): its main branch is dense causal
// attention, run by kd_dense with no index branch, lists or partials.
bool dense_sequence(int64_t L, int kslots) { return L <= (int64_t)kslots * kBlock; }

// Packs dense sequences into launches of kd_dense: add() one sequence at a time (its
// new queries at row q_row0 of q / out / ids, its tokens at row kv_row0 of k / v,
// L tokens of which the first P are a cached prefix), then finish().  Row offsets
// inside one launch are relative to its first member's rows and fit 32 bits.
struct DenseLauncher {
    const uint16_t *q, *k, *v;
    uint16_t *out;
    int32_t *ids;
    int H, G, d, kslots;
    float scale;
    hipStream_t s;
    DenseTable t;
    int64_t q_base = 0, kv_base = 0;
    int tiles = 0;
    int status = MSA_OK;

    void flush() {
        if (t.n == 0) return;
        t.tile_off[t.n] = tiles;
        const hipError_t e = timed(kKd, s, [&]() {
            return launch_kd_dense(q + q_base * H * d, k + kv_base * G * d, v + kv_base * G * d,
                                   out + q_base * H * d, ids ? ids + q_base * G * kslots : nullptr,
                                   t, H, G, d, kslots, scale, s);
        });
        if (e != hipSuccess && status == MSA_OK) status = MSA_ERR_HIP;
        t.n = 0;
        tiles = 0;
    }
    void add(int64_t q_row0, int64_t kv_row0, int64_t L, int64_t P) {
        const int tq = dense_tile_queries(H, G);
        const int64_t nt = (L - P + tq - 1) / tq;
        for (int pass = 0; pass < 2; ++pass) {
            if (t.n == 0) {
                q_base = q_row0;
                kv_base = kv_row0;
            }
            const int64_t dq = q_row0 - q_base, dk = kv_row0 - kv_base;
            const bool fits = t.n < kBatchMaxSeq && dq >= 0 && dk >= 0 &&
                              dq + (L - P) <= INT32_MAX && dk + L <= INT32_MAX &&
                              ((int64_t)tiles + nt) * G <= INT32_MAX;
            if (fits) {
                t.tile_off[t.n] = tiles;
                t.q_row0[t.n] = (int)dq;
                t.kv_row0[t.n] = (int)dk;
                t.len[t.n] = (int)L;
                t.prefix[t.n] = (int)P;
                ++t.n;
                tiles += (int)nt;
                return;
            }
            flush();   // a full launch: the sequence opens the next one
        }
    }
    int finish() {
        flush();
        return status;
    }
};

// Queries [P, L) of one causal sequence of L tokens (P a multiple of the chunk
// granularity): K1..K5 per query chunk.  q, idx_q, out and ids are addressed by
// absolute position (row i of the sequence at q + i*H*d); only rows >= P are
// ever dereferenced, so a caller that holds the new rows only passes pointers
// shifted back by P rows.  ids == nullptr: ids live in the workspace.
int prefill_range(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *idx_q,
                  const uint16_t *idx_k, int64_t L, int64_t P, int H, int G, int d, int dI,
                  int kslots, float scale, uint16_t *out, int32_t *ids, void *ws, size_t ws_bytes,
                  hipStream_t s) {
    const int64_t C = fit_chunk(
        L, ws_bytes, [&](int64_t c) { return prefill_bytes(c, L, H, G, d, dI, kslots); });
    if (C == 0) return MSA_ERR_WORKSPACE_TOO_SMALL;
    Carver c(ws, ws_bytes);
    const IndexWs iw = carve_index(c, C, L, G, dI, kslots);
    int32_t *ids_ws = c.take<int32_t>(C * G * kslots);
    const AttnWs w = carve_attn(c, C, H, G, d, kslots, (int)nblocks(L));
    MSA_CHECK_CARVE(c);
    for (int64_t q0 = P; q0 < L; q0 += C) {
        const int64_t qend = std::min(L, q0 + C);
        int32_t *ids_c = ids ? ids + q0 * G * kslots : ids_ws;
        int rc = index_chunk(iw, idx_q, idx_k, L, q0, qend, G, dI, kslots, ids_c, s);
        if (rc != MSA_OK) return rc;
        rc = attn_chunk(q, k, v, ids_c, L, q0, qend, H, G, d, kslots, scale, out, w, s);
        if (rc != MSA_OK) return rc;
    }
    return MSA_OK;
}

// Address of row -rows (rows may be negative) of a row-major array starting at p;
// prefill_range never dereferences it below p.
template <typename T>
T *rows_back(T *p, int64_t rows, int64_t row_elems) {
    const intptr_t bytes = (intptr_t)(rows * row_elems) * (intptr_t)sizeof(T);
    return reinterpret_cast<T *>(reinterpret_cast<intptr_t>(p) - bytes);
}

// ------------------- varlen prefill: batches of sequences -------------------
// Short sequences are prefilled together: K1 ... K5 run once over the rows of a
// batch of up to kBatchMaxSeq sequences, so that a batch of short prompts costs a
// few launches instead of a few per sequence.  Results are identical to
// prefilling every sequence on its own.

// Workspace of one batch: `rows` new tokens over `blocks` KV blocks, block-score
// rows of nbp entries.
size_t batch_bytes(int64_t rows, int64_t blocks, int nbp, int H, int G, int d, int k) {
    Carver c(nullptr);
    c.take<float>(rows * G * nbp);
    c.take<int32_t>(rows * G * k);
    for (int m = 0; m < 3; ++m) c.take<int32_t>(rows);
    for (int m = 0; m < 2; ++m) c.take<int32_t>(blocks);
    c.take<BatchTable>(1);
    carve_attn(c, rows, H, G, d, k, (int)blocks);
    return c.used;
}

// Greedy batching, in sequence order: a sequence with at most kBatchMaxNew new
// tokens joins the open batch while the batch stays within kBatchMaxSeq sequences
// and follows the batch's last rows (a sequence of at most k blocks, which runs the
// dense main branch instead, ends the open batch),
// kChunkQ rows, kBatchMaxBlocks blocks and `ws_limit` bytes; a longer sequence
// runs alone (measured: alone, the q rows of one long sequence stay in the
// last-level cache across the attention's 16 re-reads of each row, which beats
// the saved launches from about 16384 new tokens on).  Sequences without new
// tokens are skipped.  Calls run(batch) for every batch in order (the caller
// prefills a single-member batch as an ordinary sequence, chunked if need be).
constexpr int64_t kBatchMaxNew = 8192;
struct BatchPlan {
    int members[kBatchMaxSeq];
    int n = 0;
    bool solo = false;       // the first member runs alone
    int64_t rows = 0, blocks = 0;
    int nbp = 8;
};
template <typename Run>
int plan_batches(const int64_t *cu_q, const int64_t *cu_kv, int nseq, int H, int G, int d, int k,
                 size_t ws_limit, bool allow_batch, Run run) {
    BatchPlan b;
    for (int sq = 0; sq < nseq; ++sq) {
        const int64_t C = cu_q[sq + 1] - cu_q[sq], L = cu_kv[sq + 1] - cu_kv[sq];
        if (C == 0) continue;
        if (dense_sequence(L, k)) {
            // dense sequences run apart (kd_dense); a batch's rows are contiguous, so
            // the open batch ends before this sequence's rows
            if (b.n > 0) {
                const int rc = run(b);
                if (rc != MSA_OK) return rc;
                b = BatchPlan{};
            }
            continue;
        }
        const bool batchable = allow_batch && C <= kBatchMaxNew;
        if (b.n > 0) {
            const int64_t rows = b.rows + C, blocks = b.blocks + nblocks(L);
            const int nbp = std::max(b.nbp, nb_padded(L));
            const bool join = batchable && !b.solo && b.n < kBatchMaxSeq && rows <= kChunkQ &&
                              blocks <= kBatchMaxBlocks &&
                              batch_bytes(rows, blocks, nbp, H, G, d, k) <= ws_limit;
            if (!join) {
                const int rc = run(b);
                if (rc != MSA_OK) return rc;
                b = BatchPlan{};
            }
        }
        if (b.n == 0) b.solo = !batchable;
        b.members[b.n++] = sq;
        b.rows += C;
        b.blocks += nblocks(L);
        b.nbp = std::max(b.nbp, nb_padded(L));
    }
    return b.n > 0 ? run(b) : MSA_OK;
}

int run_batch(const BatchPlan &b, const uint16_t *q, const uint16_t *k, const uint16_t *v,
              const uint16_t *idx_q, const uint16_t *idx_k, const int64_t *cu_q,
              const int64_t *cu_kv, int H, int G, int d, int dI, int kslots, float scale,
              uint16_t *out, int32_t *block_ids_out, void *ws, size_t ws_bytes,
              hipStream_t s) {
    BatchTable t;
    t.n = b.n;
    t.rows = (int)b.rows;
    t.blocks = (int)b.blocks;
    const int64_t q_base = cu_q[b.members[0]];
    int64_t maxL = 0, blk = 0, k1wg = 0, valid = 0;
    for (int m = 0; m < b.n; ++m) {
        const int sq = b.members[m];
        const int64_t L = cu_kv[sq + 1] - cu_kv[sq], C = cu_q[sq + 1] - cu_q[sq];
        t.q_off[m] = (int)(cu_q[sq] - q_base);
        t.blk_off[m] = (int)blk;
        t.k1_off[m] = (int)k1wg;
        t.kv_off[m] = (int)cu_kv[sq];
        t.kv_len[m] = (int)L;
        blk += nblocks(L);
        k1wg += k1_num_workgroups(L - C, L, G);
        valid += valid_slots(L - C, L, kslots);
        maxL = std::max(maxL, L);
    }
    t.q_off[b.n] = t.rows;
    t.blk_off[b.n] = t.blocks;
    t.k1_off[b.n] = (int)k1wg;
    const int64_t rows = b.rows;
    const int nbp = b.nbp;
    Carver c(ws, ws_bytes);
    float *S = c.take<float>(rows * G * nbp);
    int32_t *ids_ws = c.take<int32_t>(rows * G * kslots);
    int32_t *row_len = c.take<int32_t>(rows);
    int32_t *row_kvpos = c.take<int32_t>(rows);
    int32_t *row_blk0 = c.take<int32_t>(rows);
    int32_t *blk_tok0 = c.take<int32_t>(b.blocks);
    int32_t *blk_rows = c.take<int32_t>(b.blocks);
    BatchTable *dtab = c.take<BatchTable>(1);
    const AttnWs w = carve_attn(c, rows, H, G, d, kslots, (int)b.blocks);
    MSA_CHECK_CARVE(c);
    int32_t *ids = block_ids_out ? block_ids_out + q_base * G * kslots : ids_ws;
    BatchMap bm;
    bm.row_len = row_len;
    bm.row_kvpos = row_kvpos;
    bm.row_blk0 = row_blk0;
    bm.blk_tok0 = blk_tok0;
    bm.blk_rows = blk_rows;
    MSA_TIMED(kK3, launch_batch_setup(t, dtab, row_len, row_kvpos, row_blk0, blk_tok0, blk_rows, s));
    MSA_TIMED(kK1, launch_k1_index_pool_batch(idx_q + q_base * G * dI, idx_k, S, t, dtab, G, dI,
                                              nbp, s));
    MSA_TIMED(kK2, launch_k2_select(S, nbp, rows * G, G, kslots, 0, row_len, maxL, ids, s));
    MSA_TIMED(kK3, launch_k3_schedule(ids, rows, G, kslots, (int)b.blocks, w.sb, bm, s));
    MSA_TIMED(kK4, launch_k4_kv_outer(q + q_base * H * d, k, v, w.sb, (int)b.blocks, 0, 0, rows, H,
                                      G, d, kslots, scale, w.po, w.plse, bm, s));
    MSA_TIMED(kK5, launch_k5_combine(w.po, w.plse, ids, rows, H, G, d, kslots, 0,
                                     out + q_base * H * d, bm, true,
                                     sparse_rows(valid, rows, kslots), s));
    return MSA_OK;
}

}  // namespace

extern "C" {

int msa_prefill(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *idx_q,
                const uint16_t *idx_k, int64_t L, int H, int G, int d, int dI, int B, int kslots,
                float scale, uint16_t *out, int32_t *block_ids_out, void *ws, size_t ws_bytes,
                void *stream) {
    if (L < 0 || H <= 0 || G <= 0 || d <= 0 || dI <= 0 || B <= 0 || kslots < 1 || H % G)
        return MSA_ERR_INVALID_ARG;
    if (L == 0) return MSA_OK;
    if (!q || !k || !v || !idx_q || !idx_k || !out) return MSA_ERR_INVALID_ARG;
    if (B != kBlock || !d_ok(d) || !r_ok(H, G) || !index_ok(G, dI) || kslots > 32 ||
        L > kMaxPrefillLen)
        return MSA_ERR_UNSUPPORTED;
    if (check_ptr(ws) != MSA_OK) return MSA_ERR_WORKSPACE_TOO_SMALL;
    if (fit_chunk(L, ws_bytes, [&](int64_t c) { return prefill_bytes(c, L, H, G, d, dI, kslots); }) == 0)
        return MSA_ERR_WORKSPACE_TOO_SMALL;
    if (dense_sequence(L, kslots)) {
        DenseLauncher dl{q, k, v, out, block_ids_out, H, G, d, kslots, default_scale(scale, d),
                         static_cast<hipStream_t>(stream)};
        dl.add(0, 0, L, 0);
        return dl.finish();
    }
    return prefill_range(q, k, v, idx_q, idx_k, L, 0, H, G, d, dI, kslots, default_scale(scale, d),
                         out, block_ids_out, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

// ------------------------ varlen / prefix prefill -------------------------
int msa_prefill_varlen(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                       const uint16_t *idx_q, const uint16_t *idx_k, const int64_t *cu_q,
                       const int64_t *cu_kv, int nseq, int H, int G, int d, int dI, int B,
                       int kslots, float scale, uint16_t *out, int32_t *block_ids_out, void *ws,
                       size_t ws_bytes, void *stream) {
    if (nseq < 0 || H <= 0 || G <= 0 || d <= 0 || dI <= 0 || B <= 0 || kslots < 1 || H % G)
        return MSA_ERR_INVALID_ARG;
    if (nseq == 0) return MSA_OK;
    if (!cu_q || !cu_kv) return MSA_ERR_INVALID_ARG;
    if (B != kBlock || !d_ok(d) || !r_ok(H, G) || !index_ok(G, dI) || kslots > 32)
        return MSA_ERR_UNSUPPORTED;
    int64_t total_q = 0, max_L = 0;
    for (int sq = 0; sq < nseq; ++sq) {
        const int64_t C = cu_q[sq + 1] - cu_q[sq], L = cu_kv[sq + 1] - cu_kv[sq];
        if (cu_q[sq] < 0 || cu_kv[sq] < 0 || C < 0 || L < C) return MSA_ERR_INVALID_ARG;
        if (C > 0 && (L > kMaxPrefillLen || (L - C) % kBlock)) return MSA_ERR_UNSUPPORTED;
        total_q += C;
        if (C > 0) max_L = std::max(max_L, L);
    }
    if (total_q == 0) return MSA_OK;
    if (!q || !k || !v || !idx_q || !idx_k || !out) return MSA_ERR_INVALID_ARG;
    if (check_ptr(ws) != MSA_OK) return MSA_ERR_WORKSPACE_TOO_SMALL;
    // every sequence must fit at least one 128-query chunk (the longest needs most)
    if (fit_chunk(max_L, ws_bytes,
                  [&](int64_t c) { return prefill_bytes(c, max_L, H, G, d, dI, kslots); }) == 0)
        return MSA_ERR_WORKSPACE_TOO_SMALL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    scale = default_scale(scale, d);
    // batches address K/V tokens with 32-bit offsets
    const bool allow_batch = cu_kv[nseq] < (int64_t)INT32_MAX - kBlock;
    auto one_sequence = [&](int sq) {
        const int64_t C = cu_q[sq + 1] - cu_q[sq], L = cu_kv[sq + 1] - cu_kv[sq], P = L - C;
        // queries are the last C tokens of the sequence: shift the new-token arrays back
        // by P rows so that row i of the sequence is addressed at its absolute position
        const int64_t back = P - cu_q[sq];
        int32_t *ids = block_ids_out ? rows_back(block_ids_out, back, (int64_t)G * kslots) : nullptr;
        return prefill_range(rows_back(q, back, (int64_t)H * d), k + cu_kv[sq] * G * d,
                             v + cu_kv[sq] * G * d, rows_back(idx_q, back, (int64_t)G * dI),
                             idx_k + cu_kv[sq] * dI, L, P, H, G, d, dI, kslots, scale,
                             rows_back(out, back, (int64_t)H * d), ids, ws, ws_bytes, s);
    };
    {
        DenseLauncher dl{q, k, v, out, block_ids_out, H, G, d, kslots, scale, s};
        for (int sq = 0; sq < nseq; ++sq) {
            const int64_t C = cu_q[sq + 1] - cu_q[sq], L = cu_kv[sq + 1] - cu_kv[sq];
            if (C > 0 && dense_sequence(L, kslots)) dl.add(cu_q[sq], cu_kv[sq], L, L - C);
        }
        const int rc = dl.finish();
        if (rc != MSA_OK) return rc;
    }
    return plan_batches(cu_q, cu_kv, nseq, H, G, d, kslots, ws_bytes, allow_batch,
                        [&](const BatchPlan &b) {
                            if (b.n == 1) return one_sequence(b.members[0]);
                            return run_batch(b, q, k, v, idx_q, idx_k, cu_q, cu_kv, H, G, d, dI,
                                             kslots, scale, out, block_ids_out, ws, ws_bytes, s);
                        });
}

size_t msa_prefill_varlen_workspace_size(const int64_t *cu_q, const int64_t *cu_kv, int nseq,
                                         int H, int G, int d, int dI, int B, int k) {
    (void)dI; (void)B;
    if (nseq <= 0 || !cu_q || !cu_kv || G <= 0 || H <= 0 || d <= 0 || k <= 0) return 0;
    size_t need = 0;
    for (int sq = 0; sq < nseq; ++sq) {
        const int64_t C = cu_q[sq + 1] - cu_q[sq], L = cu_kv[sq + 1] - cu_kv[sq];
        if (C <= 0 || L < C) continue;
        need = std::max(need, prefill_bytes(chunk_of(L), L, H, G, d, dI, k));
    }
    // the batches formed when the workspace is not the limit
    plan_batches(cu_q, cu_kv, nseq, H, G, d, k, SIZE_MAX, cu_kv[nseq] < (int64_t)INT32_MAX - kBlock,
                 [&](const BatchPlan &b) {
                     if (b.n > 1) need = std::max(need, batch_bytes(b.rows, b.blocks, b.nbp, H, G, d, k));
                     return MSA_OK;
                 });
    return need;
}

// -------------------------------- decode ----------------------------------
size_t msa_decode_workspace_size(int N, int64_t Lmax, int H, int G, int d, int dI, int B, int k) {
    (void)dI; (void)B;
    if (N <= 0 || Lmax <= 0 || G <= 0 || H <= 0 || d <= 0 || k <= 0) return 0;
    Carver c(nullptr);
    c.take<float>((int64_t)N * G * nb_padded(Lmax));
    c.take<int32_t>((int64_t)N * G * k);
    c.take<uint16_t>((int64_t)N * H * k * d);
    c.take<float>((int64_t)N * H * k);
    c.take<int32_t>((int64_t)N * G * k);
    return c.used;
}

namespace {
// Argument checks of msa_decode (everything but the workspace); MSA_OK with N == 0
// means there is nothing to do.
int decode_args_status(const uint16_t *q, const uint16_t *idx_q, const uint16_t *k_cache,
                       const uint16_t *v_cache, const uint16_t *idx_k_cache,
                       const int32_t *seq_len, int N, int64_t Lmax, int H, int G, int d, int dI,
                       int B, int kslots, const uint16_t *out) {
    if (N < 0 || Lmax < 0 || H <= 0 || G <= 0 || d <= 0 || dI <= 0 || B <= 0 || kslots < 1 ||
        H % G)
        return MSA_ERR_INVALID_ARG;
    if (N == 0) return MSA_OK;
    if (Lmax == 0 || !q || !idx_q || !k_cache || !v_cache || !idx_k_cache || !seq_len || !out)
        return MSA_ERR_INVALID_ARG;
    if (B != kBlock || !d_ok(d) || !r_ok(H, G) || !index_ok(G, dI) || kslots > 32)
        return MSA_ERR_UNSUPPORTED;
    return MSA_OK;
}
}  // namespace

int msa_decode(const uint16_t *q, const uint16_t *idx_q, const uint16_t *k_cache,
               const uint16_t *v_cache, const uint16_t *idx_k_cache, const int32_t *seq_len,
               int N, int64_t Lmax, int H, int G, int d, int dI, int B, int kslots, float scale,
               uint16_t *out, int32_t *block_ids_out, void *ws, size_t ws_bytes, void *stream) {
    const int as = decode_args_status(q, idx_q, k_cache, v_cache, idx_k_cache, seq_len, N, Lmax,
                                      H, G, d, dI, B, kslots, out);
    if (as != MSA_OK || N == 0) return as;
    const int st = check_ws(ws, ws_bytes, msa_decode_workspace_size(N, Lmax, H, G, d, dI, B, kslots));
    if (st != MSA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    scale = default_scale(scale, d);
    const int nbp = nb_padded(Lmax);
    Carver c(ws, ws_bytes);
    float *S = c.take<float>((int64_t)N * G * nbp);
    int32_t *ids_ws = c.take<int32_t>((int64_t)N * G * kslots);
    uint16_t *po = c.take<uint16_t>((int64_t)N * H * kslots * d);
    float *plse = c.take<float>((int64_t)N * H * kslots);
    int32_t *mark = c.take<int32_t>((int64_t)N * G * kslots);
    MSA_CHECK_CARVE(c);
    int32_t *ids = block_ids_out ? block_ids_out : ids_ws;
    MSA_TIMED(kK1d, launch_k1d_index_pool(idx_q, idx_k_cache, seq_len, nullptr, 0, S, N, Lmax, G,
                                          dI, nbp, s));
    MSA_TIMED(kK2, launch_k2_select(S, nbp, (int64_t)N * G, G, kslots, 0, seq_len, Lmax, ids, s));
    return decode_attend(q, k_cache, v_cache, ids, seq_len, nullptr, 0, N, Lmax, H, G, d,
                         kslots, scale, po, plse, mark, out, s);
}

// ------------------- decode without a caller workspace ---------------------
// The workspace of msa_decode_static: a device array of the library, one copy per
// GPU (each GPU the library runs on holds its MSA_STATIC_SCRATCH_BYTES until the
// process ends).  Host code never passes `scratch` itself to a kernel (in host code
// the name is only a stand-in for the symbol): it takes each device's address of
// the array once, with hipGetSymbolAddress, and uses that address.
static __device__ __align__(256) char scratch[MSA_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// This device's address of `scratch`, looked up on the first call on the device.
// The stream must belong to the current device.
int scratch_address(hipStream_t s, void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MSA_ERR_HIP;
    if (s) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(s, &sdev) != hipSuccess) return MSA_ERR_HIP;
        if ((int)sdev != dev) return MSA_ERR_INVALID_ARG;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MSA_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MSA_OK;
}
}  // namespace

int msa_decode_static(const uint16_t *q, const uint16_t *idx_q, const uint16_t *k_cache,
                      const uint16_t *v_cache, const uint16_t *idx_k_cache,
                      const int32_t *seq_len, int N, int64_t Lmax, int H, int G, int d, int dI,
                      int B, int kslots, float scale, uint16_t *out, int32_t *block_ids_out,
                      void *stream) {
    const int as = decode_args_status(q, idx_q, k_cache, v_cache, idx_k_cache, seq_len, N, Lmax,
                                      H, G, d, dI, B, kslots, out);
    if (as != MSA_OK || N == 0) return as;
    // the shape's workspace must fit in the array (checked before any HIP call)
    if (msa_decode_workspace_size(N, Lmax, H, G, d, dI, B, kslots) > MSA_STATIC_SCRATCH_BYTES)
        return MSA_ERR_WORKSPACE_TOO_SMALL;
    void *ws = nullptr;
    const int st = scratch_address(static_cast<hipStream_t>(stream), &ws);
    if (st != MSA_OK) return st;
    // same kernels and launches as msa_decode; no part of the workspace needs to
    // start at zero (every value read was written earlier in the same call)
    return msa_decode(q, idx_q, k_cache, v_cache, idx_k_cache, seq_len, N, Lmax, H, G, d, dI, B,
                      kslots, scale, out, block_ids_out, ws, MSA_STATIC_SCRATCH_BYTES, stream);
}

// ----------------------------- paged decode -------------------------------
size_t msa_decode_paged_workspace_size(int N, int max_blocks, int H, int G, int d, int dI, int B,
                                       int k) {
    if (N <= 0 || max_blocks <= 0 || B <= 0) return 0;
    const size_t base = msa_decode_workspace_size(N, (int64_t)max_blocks * B, H, G, d, dI, B, k);
    if (base == 0) return 0;
    Carver c(nullptr);
    c.used = base;
    c.take<int32_t>(N);
    return c.used;
}

int msa_decode_paged(const uint16_t *q, const uint16_t *idx_q, const uint16_t *k_pages,
                     const uint16_t *v_pages, const uint16_t *idx_k_pages, int64_t num_pages,
                     const int32_t *block_table, int max_blocks, const int32_t *seq_len, int N,
                     int H, int G, int d, int dI, int B, int kslots, float scale, uint16_t *out,
                     int32_t *block_ids_out, void *ws, size_t ws_bytes, void *stream) {
    if (N < 0 || num_pages < 0 || max_blocks < 0 || H <= 0 || G <= 0 || d <= 0 || dI <= 0 ||
        B <= 0 || kslots < 1 || H % G)
        return MSA_ERR_INVALID_ARG;
    if (N == 0) return MSA_OK;
    if (max_blocks == 0 || num_pages == 0 || !q || !idx_q || !k_pages || !v_pages ||
        !idx_k_pages || !block_table || !seq_len || !out)
        return MSA_ERR_INVALID_ARG;
    if (B != kBlock || !d_ok(d) || !r_ok(H, G) || !index_ok(G, dI) || kslots > 32 ||
        (int64_t)max_blocks * B > INT32_MAX)
        return MSA_ERR_UNSUPPORTED;
    const int st = check_ws(ws, ws_bytes,
                            msa_decode_paged_workspace_size(N, max_blocks, H, G, d, dI, B, kslots));
    if (st != MSA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    scale = default_scale(scale, d);
    const int64_t Lmax = (int64_t)max_blocks * B;
    const int nbp = nb_padded(Lmax);
    Carver c(ws, ws_bytes);
    float *S = c.take<float>((int64_t)N * G * nbp);
    int32_t *ids_ws = c.take<int32_t>((int64_t)N * G * kslots);
    uint16_t *po = c.take<uint16_t>((int64_t)N * H * kslots * d);
    float *plse = c.take<float>((int64_t)N * H * kslots);
    int32_t *mark = c.take<int32_t>((int64_t)N * G * kslots);
    int32_t *eff_len = c.take<int32_t>(N);
    MSA_CHECK_CARVE(c);
    int32_t *ids = block_ids_out ? block_ids_out : ids_ws;
    // every later stage sees only lengths whose pages were checked
    MSA_TIMED(kKpc, launch_page_check(block_table, max_blocks, num_pages, seq_len, N, eff_len, s));
    MSA_TIMED(kK1d, launch_k1d_index_pool(idx_q, idx_k_pages, eff_len, block_table, max_blocks, S,
                                          N, Lmax, G, dI, nbp, s));
    MSA_TIMED(kK2, launch_k2_select(S, nbp, (int64_t)N * G, G, kslots, 0, eff_len, Lmax, ids, s));
    return decode_attend(q, k_pages, v_pages, ids, eff_len, block_table, max_blocks, N, Lmax, H,
                         G, d, kslots, scale, po, plse, mark, out, s);
}

// ----------------------- FP8 (E4M3) index-key cache ------------------------
int msa_quantize_idx_k_e4m3(const uint16_t *idx_k, int64_t rows, int dI, uint8_t *idx_k_e4m3,
                            float *idx_k_scale, void *stream) {
    if (rows < 0 || dI <= 0) return MSA_ERR_INVALID_ARG;
    if (rows == 0) return MSA_OK;
    if (!idx_k || !idx_k_e4m3 || !idx_k_scale) return MSA_ERR_INVALID_ARG;
    if (dI != 32 && dI != 64 && dI != 128) return MSA_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    MSA_TIMED(kQuant, launch_quant_e4m3(idx_k, rows, dI, idx_k_e4m3, idx_k_scale, s));
    return MSA_OK;
}

int msa_decode_fp8idx(const uint16_t *q, const uint16_t *idx_q, const uint16_t *k_cache,
                      const uint16_t *v_cache, const uint8_t *idx_k_e4m3, const float *idx_k_scale,
                      const int32_t *seq_len, int N, int64_t Lmax, int H, int G, int d, int dI,
                      int B, int kslots, float scale, uint16_t *out, int32_t *block_ids_out,
                      void *ws, size_t ws_bytes, void *stream) {
    if (N < 0 || Lmax < 0 || H <= 0 || G <= 0 || d <= 0 || dI <= 0 || B <= 0 || kslots < 1 ||
        H % G)
        return MSA_ERR_INVALID_ARG;
    if (N == 0) return MSA_OK;
    if (Lmax == 0 || !q || !idx_q || !k_cache || !v_cache || !idx_k_e4m3 || !idx_k_scale ||
        !seq_len || !out)
        return MSA_ERR_INVALID_ARG;
    if (B != kBlock || !d_ok(d) || !r_ok(H, G) || !index_ok(G, dI) || kslots > 32)
        return MSA_ERR_UNSUPPORTED;
    const int st = check_ws(ws, ws_bytes, msa_decode_workspace_size(N, Lmax, H, G, d, dI, B, kslots));
    if (st != MSA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    scale = default_scale(scale, d);
    const int nbp = nb_padded(Lmax);
    Carver c(ws, ws_bytes);
    float *S = c.take<float>((int64_t)N * G * nbp);
    int32_t *ids_ws = c.take<int32_t>((int64_t)N * G * kslots);
    uint16_t *po = c.take<uint16_t>((int64_t)N * H * kslots * d);
    float *plse = c.take<float>((int64_t)N * H * kslots);
    int32_t *mark = c.take<int32_t>((int64_t)N * G * kslots);
    MSA_CHECK_CARVE(c);
    int32_t *ids = block_ids_out ? block_ids_out : ids_ws;
    MSA_TIMED(kK1d8, launch_k1d_index_pool_fp8(idx_q, idx_k_e4m3, idx_k_scale, seq_len, nullptr, 0,
                                               S, N, Lmax, G, dI, nbp, s));
    MSA_TIMED(kK2, launch_k2_select(S, nbp, (int64_t)N * G, G, kslots, 0, seq_len, Lmax, ids, s));
    return decode_attend(q, k_cache, v_cache, ids, seq_len, nullptr, 0, N, Lmax, H, G, d,
                         kslots, scale, po, plse, mark, out, s);
}

int msa_decode_paged_fp8idx(const uint16_t *q, const uint16_t *idx_q, const uint16_t *k_pages,
                            const uint16_t *v_pages, const uint8_t *idx_k_pages_e4m3,
                            const float *idx_k_scale_pages, int64_t num_pages,
                            const int32_t *block_table, int max_blocks, const int32_t *seq_len,
                            int N, int H, int G, int d, int dI, int B, int kslots, float scale,
                            uint16_t *out, int32_t *block_ids_out, void *ws, size_t ws_bytes,
                            void *stream) {
    if (N < 0 || num_pages < 0 || max_blocks < 0 || H <= 0 || G <= 0 || d <= 0 || dI <= 0 ||
        B <= 0 || kslots < 1 || H % G)
        return MSA_ERR_INVALID_ARG;
    if (N == 0) return MSA_OK;
    if (max_blocks == 0 || num_pages == 0 || !q || !idx_q || !k_pages || !v_pages ||
        !idx_k_pages_e4m3 || !idx_k_scale_pages || !block_table || !seq_len || !out)
        return MSA_ERR_INVALID_ARG;
    if (B != kBlock || !d_ok(d) || !r_ok(H, G) || !index_ok(G, dI) || kslots > 32 ||
        (int64_t)max_blocks * B > INT32_MAX)
        return MSA_ERR_UNSUPPORTED;
    const int st = check_ws(ws, ws_bytes,
                            msa_decode_paged_workspace_size(N, max_blocks, H, G, d, dI, B, kslots));
    if (st != MSA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    scale = default_scale(scale, d);
    const int64_t Lmax = (int64_t)max_blocks * B;
    const int nbp = nb_padded(Lmax);
    Carver c(ws, ws_bytes);
    float *S = c.take<float>((int64_t)N * G * nbp);
    int32_t *ids_ws = c.take<int32_t>((int64_t)N * G * kslots);
    uint16_t *po = c.take<uint16_t>((int64_t)N * H * kslots * d);
    float *plse = c.take<float>((int64_t)N * H * kslots);
    int32_t *mark = c.take<int32_t>((int64_t)N * G * kslots);
    int32_t *eff_len = c.take<int32_t>(N);
    MSA_CHECK_CARVE(c);
    int32_t *ids = block_ids_out ? block_ids_out : ids_ws;
    // every later stage sees only lengths whose pages were checked
    MSA_TIMED(kKpc, launch_page_check(block_table, max_blocks, num_pages, seq_len, N, eff_len, s));
    MSA_TIMED(kK1d8, launch_k1d_index_pool_fp8(idx_q, idx_k_pages_e4m3, idx_k_scale_pages, eff_len,
                                               block_table, max_blocks, S, N, Lmax, G, dI, nbp, s));
    MSA_TIMED(kK2, launch_k2_select(S, nbp, (int64_t)N * G, G, kslots, 0, eff_len, Lmax, ids, s));
    return decode_attend(q, k_pages, v_pages, ids, eff_len, block_table, max_blocks, N, Lmax, H,
                         G, d, kslots, scale, po, plse, mark, out, s);
}

// ------------------------------ timing ------------------------------------
int msa_timing_enable(int max_launches) {
    if (max_launches <= 0) return MSA_ERR_INVALID_ARG;
    msa_timing_disable();
    g_timing.rec = new (std::nothrow) TimedLaunch[max_launches];
    if (!g_timing.rec) return MSA_ERR_INVALID_ARG;
    for (int i = 0; i < max_launches; ++i) {
        if (hipEventCreate(&g_timing.rec[i].start) != hipSuccess ||
            hipEventCreate(&g_timing.rec[i].stop) != hipSuccess) {
            g_timing.cap = i;
            msa_timing_disable();
            return MSA_ERR_HIP;
        }
    }
    g_timing.cap = max_launches;
    g_timing.used = 0;
    g_timing.on = true;
    return MSA_OK;
}

int msa_timing_collect(msa_kernel_time *out, int max_entries, int *n_out) {
    if (!out || !n_out || max_entries < kNumStages) return MSA_ERR_INVALID_ARG;
    double total[kNumStages] = {};
    int count[kNumStages] = {};
    for (int i = 0; i < g_timing.used; ++i) {
        const TimedLaunch &t = g_timing.rec[i];
        float ms = 0.0f;
        if (hipEventSynchronize(t.stop) != hipSuccess ||
            hipEventElapsedTime(&ms, t.start, t.stop) != hipSuccess)
            return MSA_ERR_HIP;
        total[t.name] += ms;
        ++count[t.name];
    }
    int n = 0;
    for (int k = 0; k < kNumStages; ++k) {
        if (!count[k]) continue;
        snprintf(out[n].name, sizeof out[n].name, "%s", kStageNames[k]);
        out[n].launches = count[k];
        out[n].total_ms = total[k];
        ++n;
    }
    *n_out = n;
    g_timing.used = 0;
    return MSA_OK;
}

void msa_timing_disable(void) {
    for (int i = 0; i < g_timing.cap; ++i) {
        (void)hipEventDestroy(g_timing.rec[i].start);
        (void)hipEventDestroy(g_timing.rec[i].stop);
    }
    delete[] g_timing.rec;
    g_timing = Timing{};
}

}  // extern "C"
