/*
 * msa_oracle.c -- plain, slow CPU oracle for the MiniMax Sparse Attention (MSA)
 * forward pass.  TEST INFRASTRUCTURE ONLY: it is built and called by the test
 * suite, by the smoke check and by the benchmark's CPU-baseline leg, never by
 * the product path.  It shares no code, header or constant with the HIP library.
 *
 * Pages followed (cited by title and section, no line numbers):
 *   [M3-20x]  mizuki-eaf.pages.dev, "MiniMax M3 算力省 20 倍" post,
 *             section 二 (MSA: Index Branch / Main Branch),
 *             section 三 item 4 (Local Block), section 四 (exp-free TopK).
 *   [DEVUP]   163.com, "MiniMax-M3上架DEVUP：被忽略的arXiv论文揭示稀疏注意力如何
 *             将百万上下文压进生产环境", body paragraphs on the index branch and
 *             main branch (per-group selection; no approximation inside a block).
 *   [M3.1]    feinterview.poetries.top, "MiniMax M3.1 Flash 开放权重与部署要点",
 *             section "稀疏注意力为什么还会撞上显存墙" (score keys, 128-token max-pool,
 *             top 16 blocks, at most 2,048 keys per query).
 *
 * What is computed (the plain definition, written out):
 *   1. token index score  s[i,g,t] = sum_c iq[i,g,c] * ik[t,c]   for keys t <= i
 *      (one index-query head per GQA group, one index-key head shared by all
 *      groups; dot product over the causal window)            [M3-20x §二 Index Branch]
 *   2. block score        S[i,g,b] = max_{t in block b, t <= i} s[i,g,t]
 *      (max-pooling of token scores into B-token blocks)      [M3-20x §二; M3.1]
 *   3. selection: the query's own block b(i) = floor(i/B) is always selected and
 *      occupies one of the k slots [M3-20x §三 item 4: the slot of the query's
 *      block is kept]; the other k-1 slots go to the blocks b < b(i) with the
 *      largest raw scores [M3-20x §四 exp-free TopK: softmax keeps order, so the
 *      raw score is ranked directly].  Each GQA group selects on its own
 *      [M3-20x §二; DEVUP].
 *   4. main branch: exact softmax attention of every query head h (group
 *      g = h / (H/G)) over the tokens t <= i of the selected blocks only
 *      [M3-20x §二 Main Branch; DEVUP: no approximation inside a block].
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - token scores are accumulated exactly (fp64; products and sums of bf16
 *     values are exact there) and rounded once to fp32, the precision in which
 *     the GPU path takes the selection decision;
 *   - ties in block score go to the smaller block id;
 *   - ids are emitted ascending and padded with -1 when fewer than k blocks
 *     exist (b(i)+1 < k);
 *   - the causal window includes the query token itself (t <= i);
 *   - attention is computed in fp64 with the softmax maximum subtracted.
 *
 * Inputs are bf16 bit patterns (uint16), token-major:
 *   prefill: q[L,H,d]  k[L,G,d]  v[L,G,d]  iq[L,G,dI]  ik[L,dI]
 *   decode : q[N,H,d]  iq[N,G,dI]  kc[N,Lmax,G,d]  vc[N,Lmax,G,d]
 *            ikc[N,Lmax,dI]  seq_len[N]; the query is the last cached token.
 *   decode with an FP8 index-key cache: ik8[N,Lmax,dI] E4M3 bytes plus
 *            kscale[N,Lmax] fp32 (key = scale * value), in place of ikc.
 * Rows are processed in parallel with OpenMP; each row is independent.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_to_double(uint16_t x)
{
    uint32_t u = ((uint32_t)x) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ---- step 1 + 2: block scores of one query row --------------------------- */
/* iq_row: [G,dI] of query i.  ik: key rows, row t at ik + t*dI.
 * S_out: [G,nb]; entries b > b(i) are set to -INFINITY (not in the window). */
static void row_block_scores(const uint16_t *iq_row, const uint16_t *ik,
                             int64_t i, int64_t L, int G, int dI, int B,
                             float *S_out)
{
    int64_t nb = (L + B - 1) / B;
    int64_t bi = i / B;
    for (int g = 0; g < G; ++g) {
        const uint16_t *qv = iq_row + (int64_t)g * dI;
        for (int64_t b = 0; b < nb; ++b) {
            if (b > bi) {
                S_out[(int64_t)g * nb + b] = -INFINITY;
                continue;
            }
            double best = -INFINITY;
            int64_t t_end = (b + 1) * B;
            if (t_end > i + 1) t_end = i + 1;            /* causal window t <= i */
            for (int64_t t = b * B; t < t_end; ++t) {
                const uint16_t *kv = ik + t * dI;
                double s = 0.0;
                for (int c = 0; c < dI; ++c)
                    s += bf16_to_double(qv[c]) * bf16_to_double(kv[c]);
                if (s > best) best = s;
            }
            S_out[(int64_t)g * nb + b] = (float)best;   /* one rounding to fp32 */
        }
    }
}

/* ---- step 1 + 2 over an FP8 index-key cache (decode variant) -------------
 * Index keys held as OCP 8-bit floating point E4M3 bytes with one positive fp32
 * scale per token: key t is scale[t] * e4m3(ik8[t*dI + c]).  E4M3 (OCP 8-bit
 * floating point specification, "OFP8"): 1 sign bit, 4 exponent bits with bias 7,
 * 3 mantissa bits; exponent field 0 holds subnormals (m/8) * 2^-6; the patterns
 * S.1111.111 are NaN; there are no infinities; the largest finite value is 448. */
static double e4m3_to_double(uint8_t x)
{
    int sgn = x >> 7, e = (x >> 3) & 15, m = x & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, -6);
    else v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sgn ? -v : v;
}

static void row_block_scores_fp8(const uint16_t *iq_row, const uint8_t *ik8,
                                 const float *kscale, int64_t i, int64_t L, int G, int dI,
                                 int B, float *S_out)
{
    int64_t nb = (L + B - 1) / B;
    int64_t bi = i / B;
    for (int g = 0; g < G; ++g) {
        const uint16_t *qv = iq_row + (int64_t)g * dI;
        for (int64_t b = 0; b < nb; ++b) {
            if (b > bi) {
                S_out[(int64_t)g * nb + b] = -INFINITY;
                continue;
            }
            double best = -INFINITY;
            int64_t t_end = (b + 1) * B;
            if (t_end > i + 1) t_end = i + 1;            /* causal window t <= i */
            for (int64_t t = b * B; t < t_end; ++t) {
                const uint8_t *kv = ik8 + t * dI;
                double s = 0.0;
                for (int c = 0; c < dI; ++c)
                    s += bf16_to_double(qv[c]) * e4m3_to_double(kv[c]);
                s *= (double)kscale[t];                  /* the token's scale */
                if (s > best) best = s;
            }
            S_out[(int64_t)g * nb + b] = (float)best;   /* one rounding to fp32 */
        }
    }
}

/* ---- step 3: selection for one (query, group) ----------------------------- */
/* S: [nb] block scores of this (i,g).  Writes k ids (ascending, -1 padded) and
 * the relative gap between the last selected and the first unselected
 * competitor (+INFINITY when every competitor is selected). */
static int cmp_int32(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

static void select_one(const float *S, int64_t bi, int k, int32_t *ids, float *gap)
{
    int64_t ncand = bi;                      /* competitors: blocks 0 .. b(i)-1 */
    int32_t *chosen = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
    int nchosen = 0;
    chosen[nchosen++] = (int32_t)bi;         /* local block takes one slot */
    *gap = INFINITY;
    if (ncand <= k - 1) {
        for (int64_t b = 0; b < ncand; ++b) chosen[nchosen++] = (int32_t)b;
    } else {
        /* pick k-1 times the best remaining competitor: larger score first,
         * smaller id on equal scores */
        char *taken = (char *)calloc((size_t)ncand, 1);
        float last = 0.0f;
        for (int r = 0; r < k - 1; ++r) {
            int64_t best = -1;
            for (int64_t b = 0; b < ncand; ++b) {
                if (taken[b]) continue;
                if (best < 0 || S[b] > S[best]) best = b;
            }
            taken[best] = 1;
            chosen[nchosen++] = (int32_t)best;
            last = S[best];
        }
        /* first unselected competitor */
        int64_t nxt = -1;
        for (int64_t b = 0; b < ncand; ++b) {
            if (taken[b]) continue;
            if (nxt < 0 || S[b] > S[nxt]) nxt = b;
        }
        if (k - 1 >= 1) {
            double a = last, c = S[nxt];
            double den = fmax(fabs(a), fabs(c));
            *gap = (den == 0.0) ? 0.0f : (float)(fabs(a - c) / den);
        }
        free(taken);
    }
    qsort(chosen, (size_t)nchosen, sizeof(int32_t), cmp_int32);
    for (int s = 0; s < k; ++s) ids[s] = (s < nchosen) ? chosen[s] : -1;
    free(chosen);
}

/* ---- step 4: main branch for one query row -------------------------------- */
/* q_row [H,d]; key/value token t, group g at kv + (t*G + g)*d. */
static void row_attend(const uint16_t *q_row, const uint16_t *kk, const uint16_t *vv,
                       const int32_t *ids /*[G,k]*/, int64_t i, int64_t L,
                       int H, int G, int d, int B, int k, double scale, double *out /*[H,d]*/)
{
    int r = H / G;
    int64_t cap = (int64_t)k * B;
    double *z = (double *)malloc(sizeof(double) * (size_t)cap);
    int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (size_t)cap);
    for (int h = 0; h < H; ++h) {
        int g = h / r;
        const int32_t *sel = ids + (int64_t)g * k;
        /* token set T: tokens of the selected blocks inside the causal window */
        int64_t n = 0;
        for (int s = 0; s < k; ++s) {
            if (sel[s] < 0) continue;
            int64_t t0 = (int64_t)sel[s] * B, t1 = t0 + B;
            if (t1 > L) t1 = L;
            for (int64_t t = t0; t < t1; ++t)
                if (t <= i) tok[n++] = t;
        }
        const uint16_t *qh = q_row + (int64_t)h * d;
        double m = -INFINITY;
        for (int64_t u = 0; u < n; ++u) {
            const uint16_t *kt = kk + (tok[u] * G + g) * d;
            double s = 0.0;
            for (int c = 0; c < d; ++c) s += bf16_to_double(qh[c]) * bf16_to_double(kt[c]);
            z[u] = scale * s;
            if (z[u] > m) m = z[u];
        }
        double denom = 0.0;
        for (int64_t u = 0; u < n; ++u) { z[u] = exp(z[u] - m); denom += z[u]; }
        double *o = out + (int64_t)h * d;
        for (int c = 0; c < d; ++c) o[c] = 0.0;
        for (int64_t u = 0; u < n; ++u) {
            const uint16_t *vt = vv + (tok[u] * G + g) * d;
            double p = z[u] / denom;
            for (int c = 0; c < d; ++c) o[c] += p * bf16_to_double(vt[c]);
        }
    }
    free(z);
    free(tok);
}

/* ======================= exported entry points =========================== */

/* Block scores S[nrows,G,nb] (fp32) for the listed query rows of a prefill. */
void oracle_block_scores(const uint16_t *iq, const uint16_t *ik, int64_t L, int G, int dI,
                         int B, const int64_t *rows, int64_t nrows, float *S)
{
    int64_t nb = (L + B - 1) / B;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t i = rows[r];
        row_block_scores(iq + i * G * dI, ik, i, L, G, dI, B, S + r * G * nb);
    }
}

/* Selection from block scores: ids[nrows,G,k], gap[nrows,G]. */
void oracle_select(const float *S, const int64_t *rows, int64_t nrows, int G, int64_t nb,
                   int B, int k, int32_t *ids, float *gap)
{
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t bi = rows[r] / B;
        for (int g = 0; g < G; ++g)
            select_one(S + (r * G + g) * nb, bi, k, ids + (r * G + g) * k, gap + r * G + g);
    }
}

/* Main branch for the listed rows with the given ids[nrows,G,k]: out[nrows,H,d]. */
void oracle_attend(const uint16_t *q, const uint16_t *kk, const uint16_t *vv, const int32_t *ids,
                   const int64_t *rows, int64_t nrows, int64_t L, int H, int G, int d, int B,
                   int k, double scale, double *out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t i = rows[r];
        row_attend(q + i * H * d, kk, vv, ids + r * G * k, i, L, H, G, d, B, k, scale,
                   out + r * H * d);
    }
}

/* Whole prefill for the listed rows: ids, gap and out of each row. */
void oracle_prefill_rows(const uint16_t *q, const uint16_t *kk, const uint16_t *vv,
                         const uint16_t *iq, const uint16_t *ik, int64_t L, int H, int G,
                         int d, int dI, int B, int k, double scale, const int64_t *rows,
                         int64_t nrows, int32_t *ids, float *gap, double *out)
{
    int64_t nb = (L + B - 1) / B;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t i = rows[r];
        float *S = (float *)malloc(sizeof(float) * (size_t)(G * nb));
        row_block_scores(iq + i * G * dI, ik, i, L, G, dI, B, S);
        for (int g = 0; g < G; ++g)
            select_one(S + g * nb, i / B, k, ids + (r * G + g) * k, gap + r * G + g);
        row_attend(q + i * H * d, kk, vv, ids + r * G * k, i, L, H, G, d, B, k, scale,
                   out + r * H * d);
        free(S);
    }
}

/* Decode: for each listed sequence n the query is the token at seq_len[n]-1,
 * scored and attended against that sequence's own caches. */
void oracle_decode(const uint16_t *q, const uint16_t *iq, const uint16_t *kc,
                   const uint16_t *vc, const uint16_t *ikc, const int64_t *seq_len,
                   int64_t Lmax, int H, int G, int d, int dI, int B, int k, double scale,
                   const int64_t *seqs, int64_t nseqs, int32_t *ids, float *gap, double *out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nseqs; ++r) {
        int64_t n = seqs[r];
        int64_t Ln = seq_len[n];
        int64_t i = Ln - 1;
        int64_t nb = (Ln + B - 1) / B;
        float *S = (float *)malloc(sizeof(float) * (size_t)(G * nb));
        const uint16_t *ik_n = ikc + n * Lmax * dI;
        const uint16_t *k_n = kc + n * Lmax * G * d;
        const uint16_t *v_n = vc + n * Lmax * G * d;
        row_block_scores(iq + n * G * dI, ik_n, i, Ln, G, dI, B, S);
        for (int g = 0; g < G; ++g)
            select_one(S + g * nb, i / B, k, ids + (r * G + g) * k, gap + r * G + g);
        row_attend(q + n * H * d, k_n, v_n, ids + r * G * k, i, Ln, H, G, d, B, k, scale,
                   out + r * H * d);
        free(S);
    }
}

/* Decode main branch only, for the listed sequences with the given ids[nseqs,G,k]:
 * the query of sequence n is its last cached token (position seq_len[n]-1), attended
 * over the listed blocks of that sequence's own K/V caches (step 4). */
void oracle_decode_attend(const uint16_t *q, const uint16_t *kc, const uint16_t *vc,
                          const int64_t *seq_len, int64_t Lmax, int H, int G, int d, int B, int k,
                          double scale, const int64_t *seqs, int64_t nseqs, const int32_t *ids,
                          double *out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nseqs; ++r) {
        int64_t n = seqs[r];
        int64_t Ln = seq_len[n];
        int64_t qpos = Ln - 1;                           /* the last cached token */
        const uint16_t *kseq = kc + n * Lmax * G * d;    /* sequence n's caches */
        const uint16_t *vseq = vc + n * Lmax * G * d;
        row_attend(q + n * H * d, kseq, vseq, ids + r * G * k, qpos, Ln, H, G, d, B, k, scale,
                   out + r * H * d);
    }
}

/* Decode block scores (steps 1 + 2) of the listed sequences: S[nseqs,G,nbmax] for
 * the query at position seq_len[n]-1 against sequence n's own index-key cache;
 * nbmax >= ceil(seq_len[n]/B) for every listed n, and blocks past the query's own
 * block hold -INFINITY. */
void oracle_decode_block_scores(const uint16_t *iq, const uint16_t *ikc, const int64_t *seq_len,
                                int64_t Lmax, int G, int dI, int B, const int64_t *seqs,
                                int64_t nseqs, int64_t nbmax, float *S)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nseqs; ++r) {
        int64_t n = seqs[r];
        int64_t Ln = seq_len[n];
        int64_t nb = (Ln + B - 1) / B;
        const uint16_t *iks = ikc + n * Lmax * dI;       /* sequence n's index keys */
        float *tmp = (float *)malloc(sizeof(float) * (size_t)(G * nb));
        row_block_scores(iq + n * G * dI, iks, Ln - 1, Ln, G, dI, B, tmp);
        for (int g = 0; g < G; ++g)
            for (int64_t b = 0; b < nbmax; ++b)
                S[(r * G + g) * nbmax + b] = (b < nb) ? tmp[g * nb + b] : -INFINITY;
        free(tmp);
    }
}

/* The value of every E4M3 byte (index = the byte), NaN for the NaN patterns. */
void oracle_e4m3_table(double *out)
{
    for (int x = 0; x < 256; ++x) out[x] = e4m3_to_double((uint8_t)x);
}

/* Decode with an FP8 index-key cache: ik8[N,Lmax,dI] E4M3 bytes and
 * kscale[N,Lmax] fp32; everything else as oracle_decode. */
void oracle_decode_fp8idx(const uint16_t *q, const uint16_t *iq, const uint16_t *kc,
                          const uint16_t *vc, const uint8_t *ik8, const float *kscale,
                          const int64_t *seq_len, int64_t Lmax, int H, int G, int d, int dI,
                          int B, int k, double scale, const int64_t *seqs, int64_t nseqs,
                          int32_t *ids, float *gap, double *out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nseqs; ++r) {
        int64_t n = seqs[r];
        int64_t Ln = seq_len[n];
        int64_t i = Ln - 1;
        int64_t nb = (Ln + B - 1) / B;
        float *S = (float *)malloc(sizeof(float) * (size_t)(G * nb));
        row_block_scores_fp8(iq + n * G * dI, ik8 + n * Lmax * dI, kscale + n * Lmax, i, Ln, G,
                             dI, B, S);
        for (int g = 0; g < G; ++g)
            select_one(S + g * nb, i / B, k, ids + (r * G + g) * k, gap + r * G + g);
        row_attend(q + n * H * d, kc + n * Lmax * G * d, vc + n * Lmax * G * d, ids + r * G * k,
                   i, Ln, H, G, d, B, k, scale, out + r * H * d);
        free(S);
    }
}

/* Decode block scores over an FP8 index-key cache (ik8[N,Lmax,dI] E4M3 bytes,
 * kscale[N,Lmax]); layout and conventions as oracle_decode_block_scores. */
void oracle_decode_block_scores_fp8(const uint16_t *iq, const uint8_t *ik8, const float *kscale,
                                    const int64_t *seq_len, int64_t Lmax, int G, int dI, int B,
                                    const int64_t *seqs, int64_t nseqs, int64_t nbmax, float *S)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nseqs; ++r) {
        int64_t n = seqs[r];
        int64_t Ln = seq_len[n];
        int64_t nb = (Ln + B - 1) / B;
        const uint8_t *ik8s = ik8 + n * Lmax * dI;       /* sequence n's E4M3 keys */
        const float *kss = kscale + n * Lmax;            /* and their scales */
        float *tmp = (float *)malloc(sizeof(float) * (size_t)(G * nb));
        row_block_scores_fp8(iq + n * G * dI, ik8s, kss, Ln - 1, Ln, G, dI, B, tmp);
        for (int g = 0; g < G; ++g)
            for (int64_t b = 0; b < nbmax; ++b)
                S[(r * G + g) * nbmax + b] = (b < nb) ? tmp[g * nb + b] : -INFINITY;
        free(tmp);
    }
}

/* Threads an OpenMP parallel region of the oracle uses. */
int oracle_num_threads(void)
{
    return omp_get_max_threads();
}
