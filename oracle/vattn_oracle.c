/*
 * CPU oracle for the verified sparse-attention (vAttention) decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library.  It shares no source
 * with the HIP library: its own Philox, its own pinned dot product, its own
 * exp, its own selection (plain qsort) and plain fp64 loops for the outputs.
 *
 * What the step computes (edgentiq blog post "vAttention: a new approach to
 * sparse attention with guaranteed accuracy", sections "How vAttention Works"
 * and "Introducing vAttention"): for every query head, a deterministic index
 * set (attention sinks, a sliding window, predicted top-k tokens) joined with a
 * uniform random sample of the remaining long tail.  The sample size comes from
 * a central-limit bound so that the softmax-denominator estimate meets a user
 * (eps, delta); the denominator is the quantity whose accuracy is targeted.
 * The sampled tail is weighted by the inverse sampling probability.
 * The top-k predictor ranks tokens with attention scores computed in a
 * low-dimensional key space (pith.science page "Loki: Low-rank Keys for
 * Efficient Sparse Attention", abstract), with exact scores ("oracle top-k",
 * same blog post, section "Performance and Efficiency"), or by hash
 * signatures (HashAttention, named as a top-k method in the same section):
 * here 32 random-hyperplane sign bits of the projected query and key
 * (Charikar's SimHash, untrained), scored by the number of equal bits.
 *
 * The pages fix no arithmetic order.  Every floating-point quantity that
 * decides a discrete outcome (which tokens are top-k, the budget) is defined
 * here by one explicit sequence of IEEE fp32/fp64 operations so that an
 * independent implementation can reproduce it bit for bit:
 *   pdot   blocked dot: fp32 fma chains over blocks of 8 elements, then a
 *          pairwise tree over the block partials;
 *   pexp   Cody-Waite range reduction + degree-7 Taylor polynomial in fma;
 *   stats  exact unsigned integer sums of E_i = trunc(pexp(s_i - m) * 2^40);
 *   budget fp64 expression with a fixed parenthesisation, no contraction;
 *   numerator statistics (the output-level mode) fp64 sums of E_i * V_ic in a
 *          fixed order: ascending tokens within spans of ORC_SPAN tokens from
 *          +0, then the span partials in ascending span order.
 * The attention output itself is computed in fp64 from the chosen index set.
 *
 * Build: gcc -O2 -std=gnu11 -ffp-contract=off -fopenmp -shared -fPIC.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_PAGE 16

typedef unsigned __int128 u128;

/* Configuration as the oracle reads it (its own struct; mirrored by ctypes). */
typedef struct {
    int32_t sinks;        /* first tokens always kept                      */
    int32_t window;       /* last tokens always kept (includes the newest)  */
    int32_t topk_abs;     /* >= 0: absolute k; < 0: use topk_ppm           */
    int32_t topk_ppm;     /* k = ceil(L * ppm / 1e6)                        */
    int32_t base_ppm;     /* base sample = ceil(N_tail * ppm / 1e6), >= 2   */
    int32_t force_budget; /* < 0: CLT budget; >= 0: fixed n = min(N_t, .)   */
    int32_t predictor;    /* 0 exact scores, 1 low-rank keys, 2 signatures */
    int32_t rank;         /* r, low-rank width (32 signature bits for 2)   */
    double eps, delta;    /* accuracy target, failure probability          */
    double z32;           /* Phi^-1(1 - delta/2) rounded to fp32 (caller)  */
    uint64_t seed;        /* Philox key                                    */
    int32_t guarantee;    /* 0 denominator; 1 denominator and numerator    */
} orc_cfg;

/* Tokens per span of the numerator sums' summation order (see decode_head). */
#define ORC_SPAN 1024

/* ------------------------------------------------------------------ */
/* Small exact helpers                                                 */
/* ------------------------------------------------------------------ */

static inline float bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* fp32 -> bf16 with round-to-nearest-even (finite inputs). */
static inline uint16_t f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* Monotone map of a finite fp32 to uint32: a < b  <=>  okey(a) < okey(b);
 * -0 maps just below +0. */
uint32_t orc_okey(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

/* ------------------------------------------------------------------ */
/* Pinned fp32 dot product.                                            */
/* n is a multiple of 8 and n/8 is a power of two.  Block j holds      */
/* elements 8j..8j+7; its partial is an fma chain started from +0.     */
/* Partials are then added pairwise, adjacent pairs first.            */
/* a is read with stride sa, b with stride sb.                         */
/* ------------------------------------------------------------------ */
float orc_pdot(const float* a, int sa, const float* b, int sb, int n) {
    float part[64];
    int nb = n / 8;
    for (int j = 0; j < nb; ++j) {
        float acc = 0.0f;
        for (int e = 0; e < 8; ++e) {
            int c = 8 * j + e;
            acc = fmaf(a[(size_t)c * sa], b[(size_t)c * sb], acc);
        }
        part[j] = acc;
    }
    while (nb > 1) {
        for (int j = 0; j < nb / 2; ++j) part[j] = part[2 * j] + part[2 * j + 1];
        nb /= 2;
    }
    return part[0];
}

/* ------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: */
/* as easy as 1, 2, 3", SC'11): ten rounds of two 32x32->64 multiplies */
/* with the published multipliers, key bumped by the Weyl constants   */
/* between rounds.                                                     */
/* ------------------------------------------------------------------ */
void orc_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += W0;
            k1 += W1;
        }
        uint64_t p0 = (uint64_t)M0 * c0;
        uint64_t p1 = (uint64_t)M1 * c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Uniform key of token i for KV head g of sequence b:
 * counter = (i >> 2, g, b, 0), key = (seed lo, seed hi), word i & 3. */
uint32_t orc_token_key(uint64_t seed, int b, int g, int i) {
    uint32_t ctr[4] = {(uint32_t)i >> 2, (uint32_t)g, (uint32_t)b, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    orc_philox4x32_10(ctr, key, w);
    return w[i & 3];
}

/* ------------------------------------------------------------------ */
/* Pinned exp for x in [-28, 0] (Cody & Waite, "Software Manual for    */
/* the Elementary Functions", 1980: split ln 2 so n*LN2_HI is exact).  */
/* ------------------------------------------------------------------ */
static float g_ln2_hi, g_ln2_lo, g_log2e, g_c[8];
static int g_init = 0;

static void orc_init_constants(void) {
    if (g_init) return;
    /* ln 2 rounded to 15 significant bits: n*LN2_HI is exact for |n| < 2^9 */
    double hi = ldexp(nearbyint(ldexp(M_LN2, 15)), -15);
    g_ln2_hi = (float)hi;
    g_ln2_lo = (float)(M_LN2 - hi);
    g_log2e = (float)(1.0 / M_LN2);
    double fact = 1.0;
    for (int k = 0; k < 8; ++k) {
        if (k > 0) fact *= (double)k;
        g_c[k] = (float)(1.0 / fact);
    }
    g_init = 1;
}

float orc_pexp(float x) {
    orc_init_constants();
    float t = x * g_log2e;
    float n = rintf(t); /* round half to even (default rounding mode) */
    float r = fmaf(-n, g_ln2_hi, x);
    r = fmaf(-n, g_ln2_lo, r);
    float p = g_c[7];
    for (int k = 6; k >= 0; --k) p = fmaf(p, r, g_c[k]);
    return ldexpf(p, (int)n);
}

/* E = trunc(pexp(x) * 2^40) in [0, 2^40]; 0 below x = -28. */
uint64_t orc_fixed_weight(float x) {
    if (x < -28.0f) return 0;
    float v = orc_pexp(x) * 0x1p40f;
    uint64_t e = (uint64_t)v;
    if (e > (1ull << 40)) e = 1ull << 40;
    return e;
}

/* ------------------------------------------------------------------ */
/* Low-rank keys: Kt[i][j] = bf16(pdot(K_i, P[:, j], d)).              */
/* ------------------------------------------------------------------ */
void orc_project_rows(const float* k_rows, int64_t nrows, int d, const float* proj, int r,
                      uint16_t* out) {
    for (int64_t i = 0; i < nrows; ++i)
        for (int j = 0; j < r; ++j)
            out[i * r + j] = f32_to_bf16(orc_pdot(k_rows + i * d, 1, proj + j, r, d));
}

/* ------------------------------------------------------------------ */
/* Key signatures: bit j of S_i is set when pdot(K_i, P[:, j], d) > 0, */
/* for the 32 columns of P ([d][32]).                                  */
/* ------------------------------------------------------------------ */
void orc_sign_rows(const float* k_rows, int64_t nrows, int d, const float* proj, uint32_t* out) {
    for (int64_t i = 0; i < nrows; ++i) {
        uint32_t w = 0;
        for (int j = 0; j < 32; ++j)
            if (orc_pdot(k_rows + i * d, 1, proj + j, 32, d) > 0.0f) w |= 1u << j;
        out[i] = w;
    }
}

/* Bits set in a word, one at a time. */
static int orc_popcount(uint32_t w) {
    int c = 0;
    for (; w; w >>= 1) c += (int)(w & 1u);
    return c;
}

/* ------------------------------------------------------------------ */
/* Decode                                                               */
/* ------------------------------------------------------------------ */
typedef struct {
    uint64_t k;
    int32_t i;
} orc_item;

/* ascending by k, then ascending by i */
static int cmp_item_asc(const void* pa, const void* pb) {
    const orc_item* a = (const orc_item*)pa;
    const orc_item* b = (const orc_item*)pb;
    if (a->k != b->k) return a->k < b->k ? -1 : 1;
    return (a->i > b->i) - (a->i < b->i);
}

static int cmp_int(const void* pa, const void* pb) {
    int a = *(const int*)pa, b = *(const int*)pb;
    return (a > b) - (a < b);
}

typedef struct {
    const orc_cfg* cfg;
    int B, Hq, Hkv, d, max_blocks, kv_bf16, max_seq_len;
    const float* q;
    const void* k_cache;
    const void* v_cache;
    const float* proj;   /* [proj_heads][d][r]: one basis, or one per KV head */
    int proj_heads;
    const int32_t* block_table;
    const int32_t* seq_lens;
    /* outputs */
    double* out;
    double* lse;
    double* lse_dense;
    double* out_dense;
    int32_t* idx;
    int idx_cap;
    int32_t* counts;
    uint64_t* stats;
    float* pred_scores; /* [B*Hq][max_seq_len] predictor scores, NaN outside the middle */
    double* nstats;     /* [B*Hq][2] numerator statistics TR, NN (output-level mode) or NULL */
} orc_ctx;

/* Copy the L rows of (b, g) out of the paged cache as fp32. */
static void load_rows(const orc_ctx* cx, const void* cache, int b, int g, int L, float* dst) {
    int d = cx->d;
    for (int i = 0; i < L; ++i) {
        int64_t page = cx->block_table[(int64_t)b * cx->max_blocks + i / ORC_PAGE];
        int64_t row = ((page * cx->Hkv + g) * ORC_PAGE + (i % ORC_PAGE)) * (int64_t)d;
        if (cx->kv_bf16) {
            const uint16_t* src = (const uint16_t*)cache + row;
            for (int c = 0; c < d; ++c) dst[(int64_t)i * d + c] = bf16_to_f32(src[c]);
        } else {
            const float* src = (const float*)cache + row;
            memcpy(dst + (int64_t)i * d, src, sizeof(float) * d);
        }
    }
}

/* fp64 softmax attention over a weighted index list (sorted or not). */
static void attend_fp64(const float* q, const float* K, const float* V, int d, const int* list,
                        const double* w, int cnt, double* out, double* lse) {
    double inv_sqrt_d = 1.0 / sqrt((double)d);
    double* sig = (double*)malloc(sizeof(double) * (cnt > 0 ? cnt : 1));
    double M = -INFINITY;
    for (int t = 0; t < cnt; ++t) {
        const float* kr = K + (int64_t)list[t] * d;
        double acc = 0.0;
        for (int c = 0; c < d; ++c) acc += (double)q[c] * (double)kr[c];
        sig[t] = acc * inv_sqrt_d;
        if (sig[t] > M) M = sig[t];
    }
    double D = 0.0;
    for (int c = 0; c < d; ++c) out[c] = 0.0;
    for (int t = 0; t < cnt; ++t) {
        double p = w[t] * exp(sig[t] - M);
        D += p;
        const float* vr = V + (int64_t)list[t] * d;
        for (int c = 0; c < d; ++c) out[c] += p * (double)vr[c];
    }
    if (cnt == 0 || D == 0.0) {
        for (int c = 0; c < d; ++c) out[c] = 0.0;
        *lse = -INFINITY;
    } else {
        for (int c = 0; c < d; ++c) out[c] /= D;
        *lse = M + log(D);
    }
    free(sig);
}

/* One query head h of sequence b (KV head g), given the group's rows. */
static void decode_head(const orc_ctx* cx, int b, int h, int g, int L, const float* K,
                        const float* V, const float* Kt /* [L][r] fp32 or NULL */,
                        const uint32_t* Ks /* [L] key signatures or NULL */) {
    const orc_cfg* cfg = cx->cfg;
    const int d = cx->d, r = cfg->rank;
    const int64_t bh = (int64_t)b * cx->Hq + h;
    double* out = cx->out + bh * d;
    double* lse = cx->lse + bh;
    int32_t* counts = cx->counts ? cx->counts + bh * 6 : NULL;
    uint64_t* stats = cx->stats ? cx->stats + bh * 4 : NULL;
    int32_t* idx = cx->idx ? cx->idx + bh * cx->idx_cap : NULL;
    double* nstats = cx->nstats ? cx->nstats + bh * 2 : NULL;

    if (nstats) nstats[0] = nstats[1] = 0.0;
    if (idx)
        for (int t = 0; t < cx->idx_cap; ++t) idx[t] = -1;
    if (counts) memset(counts, 0, sizeof(int32_t) * 6);
    if (stats) memset(stats, 0, sizeof(uint64_t) * 4);
    if (cx->pred_scores)
        for (int i = 0; i < cx->max_seq_len; ++i) cx->pred_scores[bh * cx->max_seq_len + i] = NAN;

    /* dense reference over all L tokens, weight 1 (exact-reduction target) */
    if (cx->lse_dense || cx->out_dense) {
        int* all = (int*)malloc(sizeof(int) * (L > 0 ? L : 1));
        double* w1 = (double*)malloc(sizeof(double) * (L > 0 ? L : 1));
        double* od = (double*)malloc(sizeof(double) * d);
        double ld;
        for (int i = 0; i < L; ++i) { all[i] = i; w1[i] = 1.0; }
        attend_fp64(cx->q + bh * d, K, V, d, all, w1, L, od, &ld);
        if (cx->lse_dense) cx->lse_dense[bh] = ld;
        if (cx->out_dense) memcpy(cx->out_dense + bh * d, od, sizeof(double) * d);
        free(all); free(w1); free(od);
    }

    if (L == 0) {
        for (int c = 0; c < d; ++c) out[c] = 0.0;
        *lse = -INFINITY;
        return;
    }

    /* query scaled by fl32(1/sqrt(d)), SDPA's scale (blog, intro section) */
    float scale32 = (float)(1.0 / sqrt((double)d));
    float* qs = (float*)malloc(sizeof(float) * d);
    for (int c = 0; c < d; ++c) qs[c] = cx->q[bh * d + c] * scale32;

    /* regions: sinks [0,sp), window [L-wp, L), middle [sp, L-wp) */
    int sp = cfg->sinks < L ? cfg->sinks : L;
    int wp = cfg->window < L - sp ? cfg->window : L - sp;
    int m_lo = sp, m_hi = L - wp, nM = m_hi - m_lo;

    int64_t k64 = cfg->topk_abs >= 0 ? (int64_t)cfg->topk_abs
                                     : ((int64_t)L * cfg->topk_ppm + 999999) / 1000000;
    int k = (int)(k64 < nM ? k64 : nM);

    /* predictor scores over the middle */
    float* qt = NULL;
    uint32_t qsig = 0;
    if (cfg->predictor == 1 || cfg->predictor == 2) {
        qt = (float*)malloc(sizeof(float) * r);
        const float* P = cx->proj + (size_t)(cx->proj_heads > 1 ? g : 0) * d * r;  /* the group's basis */
        for (int j = 0; j < r; ++j) qt[j] = orc_pdot(qs, 1, P + j, r, d);
        /* the query's signature: the same sign test on its projection */
        if (cfg->predictor == 2)
            for (int j = 0; j < 32; ++j)
                if (qt[j] > 0.0f) qsig |= 1u << j;
    }
    orc_item* items = (orc_item*)malloc(sizeof(orc_item) * (nM > 0 ? nM : 1));
    for (int t = 0; t < nM; ++t) {
        int i = m_lo + t;
        float s;
        if (cfg->predictor == 1) s = orc_pdot(qt, 1, Kt + (int64_t)i * r, 1, r);
        else if (cfg->predictor == 2) s = (float)(32 - orc_popcount(qsig ^ Ks[i]));  /* equal bits */
        else s = orc_pdot(qs, 1, K + (int64_t)i * d, 1, d);
        if (cx->pred_scores) cx->pred_scores[bh * cx->max_seq_len + i] = s;
        /* descending score == ascending complement of the order key */
        items[t].k = (uint64_t)(~orc_okey(s));
        items[t].i = i;
    }
    /* top-k: k largest scores, the lower index first among equal scores */
    qsort(items, (size_t)nM, sizeof(orc_item), cmp_item_asc);

    char* in_fixed = (char*)calloc((size_t)L, 1); /* I_f membership */
    for (int i = 0; i < sp; ++i) in_fixed[i] = 1;
    for (int i = m_hi; i < L; ++i) in_fixed[i] = 1;
    for (int t = 0; t < k; ++t) in_fixed[items[t].i] = 1;
    int n_fixed = sp + wp + k;
    int NT = nM - k;

    /* tail in random order: ascending (Philox word, index) */
    orc_item* rho = (orc_item*)malloc(sizeof(orc_item) * (NT > 0 ? NT : 1));
    int nr = 0;
    for (int i = m_lo; i < m_hi; ++i) {
        if (in_fixed[i]) continue;
        rho[nr].k = orc_token_key(cfg->seed, b, g, i);
        rho[nr].i = i;
        ++nr;
    }
    qsort(rho, (size_t)NT, sizeof(orc_item), cmp_item_asc);

    int nb = 0;
    if (NT > 0) {
        int64_t want = ((int64_t)NT * cfg->base_ppm + 999999) / 1000000;
        if (want < 2) want = 2;
        nb = (int)(want < NT ? want : NT);
    }

    /* pinned exact scores of I_f and the base sample, max, fixed-point sums */
    float* s_exact = (float*)malloc(sizeof(float) * L);
    float m = -INFINITY;
    for (int i = 0; i < L; ++i)
        if (in_fixed[i]) {
            s_exact[i] = orc_pdot(qs, 1, K + (int64_t)i * d, 1, d);
            if (s_exact[i] > m) m = s_exact[i];
        }
    for (int t = 0; t < nb; ++t) {
        int i = rho[t].i;
        s_exact[i] = orc_pdot(qs, 1, K + (int64_t)i * d, 1, d);
        if (s_exact[i] > m) m = s_exact[i];
    }
    uint64_t SF = 0, S1 = 0;
    u128 S2 = 0;
    for (int i = 0; i < L; ++i)
        if (in_fixed[i]) SF += orc_fixed_weight(s_exact[i] - m);
    for (int t = 0; t < nb; ++t) {
        uint64_t e = orc_fixed_weight(s_exact[rho[t].i] - m);
        S1 += e;
        S2 += (u128)e * e;
    }

    /* Numerator statistics, output-level mode only.  SkyLight's post ("vAttention
     * Computation") promises (eps, delta) on the intermediate quantities; the
     * edgentiq post ("How vAttention Works") calls the denominator-only budget a
     * relaxation.  Without it the numerator N = sum_i e^{s_i - m} V_i (a vector)
     * is held to the same CLT bound: with y_i = E_i V_i per channel c,
     *   TR = sum_c (n_b T2_c - T1_c^2)   (n_b (n_b - 1) times the summed
     *                                     unbiased per-channel variances of y
     *                                     over the base sample),
     *   NN = sum_c (n_b NF_c + N_t T1_c)^2  (n_b^2 times the squared norm of
     *                                        the estimated numerator),
     * T1, T2 the sums of y and y^2 over the base sample, NF the sum of y over
     * the fixed set.  Every sum is fp64 in one fixed order (ascending tokens
     * within spans of ORC_SPAN, then the spans in order; channels ascending for
     * TR and NN), so an independent implementation reproduces the bits. */
    double TR = 0.0, NN = 0.0;
    const int use_num = cfg->guarantee == 1 && nb > 0;
    if (use_num) {
        char* in_base = (char*)calloc((size_t)L, 1);
        for (int t = 0; t < nb; ++t) in_base[rho[t].i] = 1;
        double* tot = (double*)calloc((size_t)3 * d, sizeof(double)); /* T1, T2, NF */
        double* part = (double*)malloc(sizeof(double) * 3 * d);
        for (int s0 = 0; s0 < L; s0 += ORC_SPAN) {
            for (int c = 0; c < 3 * d; ++c) part[c] = 0.0;
            int s1 = s0 + ORC_SPAN < L ? s0 + ORC_SPAN : L;
            for (int i = s0; i < s1; ++i) {
                if (!in_fixed[i] && !in_base[i]) continue;
                double e = (double)orc_fixed_weight(s_exact[i] - m);
                for (int c = 0; c < d; ++c) {
                    double y = e * (double)V[(int64_t)i * d + c];
                    if (in_fixed[i]) {
                        part[2 * d + c] = part[2 * d + c] + y;
                    } else {
                        part[c] = part[c] + y;
                        part[d + c] = part[d + c] + y * y;
                    }
                }
            }
            for (int c = 0; c < 3 * d; ++c) tot[c] = tot[c] + part[c];
        }
        for (int c = 0; c < d; ++c) {
            double m2 = (double)nb * tot[d + c] - tot[c] * tot[c];
            if (m2 < 0.0) m2 = 0.0;
            double yc = (double)nb * tot[2 * d + c] + (double)NT * tot[c];
            TR = TR + m2;
            NN = NN + yc * yc;
        }
        free(in_base); free(tot); free(part);
        if (nstats) { nstats[0] = TR; nstats[1] = NN; }
    }

    /* CLT budget on the denominator: n = (z * sigma * N_t / (eps * D))^2 with
     * sigma^2 the unbiased variance of the base sample and D the base-sample
     * denominator estimate, rearranged over the exact integers.  In the
     * output-level mode the numerator's budget (the same expression with TR
     * for M2 and NN for Y^2) is taken when larger (flag 8). */
    int n, flags = 0;
    if (cfg->force_budget >= 0) {
        n = cfg->force_budget < NT ? cfg->force_budget : NT;
        flags |= 2;
    } else if (nb == NT) {
        n = NT;
    } else {
        u128 M2 = (u128)nb * S2 - (u128)S1 * S1;
        u128 Y = (u128)nb * SF + (u128)NT * S1;
        double z = cfg->z32;
        double num = (z * z * (double)NT * (double)NT) * ((double)M2 * (double)nb);
        double den = ((double)(nb - 1) * (cfg->eps * cfg->eps)) * ((double)Y * (double)Y);
        double nreal = num / den;
        if (nreal >= (double)NT) {
            n = NT;
        } else {
            n = (int)ceil(nreal);
            if (n < nb) { n = nb; flags |= 4; }
        }
        if (use_num) {
            double numN = (z * z * (double)NT * (double)NT) * (TR * (double)nb);
            double denN = ((double)(nb - 1) * (cfg->eps * cfg->eps)) * NN;
            int nN;
            if (denN == 0.0) {
                nN = numN > 0.0 ? NT : 0; /* a zero numerator estimate: any spread is unbounded relative error */
            } else {
                double r = numN / denN;
                nN = r >= (double)NT ? NT : (int)ceil(r);
            }
            if (nN > n) { n = nN; flags |= 8; }
        }
    }
    if (n == NT) flags |= 1;

    /* final index set I = I_f + first n of the random order, ascending */
    int cnt = n_fixed + n;
    int* list = (int*)malloc(sizeof(int) * (cnt > 0 ? cnt : 1));
    int c = 0;
    for (int i = 0; i < L; ++i)
        if (in_fixed[i]) list[c++] = i;
    for (int t = 0; t < n; ++t) list[c++] = rho[t].i;
    qsort(list, (size_t)cnt, sizeof(int), cmp_int);

    /* weights: 1 on I_f, N_t / n on the sample (inverse inclusion probability) */
    double* w = (double*)malloc(sizeof(double) * (cnt > 0 ? cnt : 1));
    double ws = n > 0 ? (double)NT / (double)n : 0.0;
    for (int t = 0; t < cnt; ++t) w[t] = in_fixed[list[t]] ? 1.0 : ws;
    attend_fp64(cx->q + bh * d, K, V, d, list, w, cnt, out, lse);

    if (idx)
        for (int t = 0; t < cnt && t < cx->idx_cap; ++t) idx[t] = list[t];
    if (counts) {
        counts[0] = n_fixed; counts[1] = NT; counts[2] = nb;
        counts[3] = n; counts[4] = cnt; counts[5] = flags;
    }
    if (stats) {
        stats[0] = SF; stats[1] = S1;
        stats[2] = (uint64_t)(S2 >> 64); stats[3] = (uint64_t)S2;
    }
    free(qs); free(qt); free(items); free(in_fixed); free(rho);
    free(s_exact); free(list); free(w);
}

/* 1 when every one of the n values is finite (the pages define the step on
 * real scores; non-finite inputs have no reading and are refused). */
static int all_finite(const float* x, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) return 0;
    return 1;
}

/* One (b, g) group; returns 0, or 5 when a cached K or V row of the group is
 * not finite (the group's outputs are then left untouched). */
static int decode_group(const orc_ctx* cx, int b, int g) {
    const int d = cx->d, G = cx->Hq / cx->Hkv;
    int L = cx->seq_lens[b];
    float* K = (float*)malloc(sizeof(float) * (size_t)(L > 0 ? L : 1) * d);
    float* V = (float*)malloc(sizeof(float) * (size_t)(L > 0 ? L : 1) * d);
    load_rows(cx, cx->k_cache, b, g, L, K);
    load_rows(cx, cx->v_cache, b, g, L, V);
    if (!all_finite(K, (int64_t)L * d) || !all_finite(V, (int64_t)L * d)) {
        free(K); free(V);
        return 5;
    }
    float* Kt = NULL;
    if (cx->cfg->predictor == 1 && L > 0) {
        int r = cx->cfg->rank;
        uint16_t* kt16 = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)L * r);
        orc_project_rows(K, L, d, cx->proj + (size_t)(cx->proj_heads > 1 ? g : 0) * d * r, r, kt16);
        Kt = (float*)malloc(sizeof(float) * (size_t)L * r);
        for (int64_t t = 0; t < (int64_t)L * r; ++t) Kt[t] = bf16_to_f32(kt16[t]);
        free(kt16);
    }
    uint32_t* Ks = NULL;
    if (cx->cfg->predictor == 2 && L > 0) {
        Ks = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)L);
        orc_sign_rows(K, L, d, cx->proj + (size_t)(cx->proj_heads > 1 ? g : 0) * d * 32, Ks);
    }
    for (int hl = 0; hl < G; ++hl) decode_head(cx, b, g * G + hl, g, L, K, V, Kt, Ks);
    free(K); free(V); free(Kt); free(Ks);
    return 0;
}

/*
 * Full decode over the (b, g) groups in `groups` (b*Hkv + g), or all groups
 * when groups is NULL.  Outputs of groups not evaluated are left untouched.
 * Returns 0 on success, nonzero on invalid arguments: 5 when q, the basis or a
 * cached K or V row that a decode reads is not finite (outputs then undefined).
 */
int orc_decode(const orc_cfg* cfg, int B, int Hq, int Hkv, int d, int max_blocks, int kv_bf16,
               int max_seq_len, const float* q, const void* k_cache, const void* v_cache,
               const float* proj, int proj_heads, const int32_t* block_table, const int32_t* seq_lens,
               const int32_t* groups, int n_groups, int nthreads, double* out, double* lse,
               double* lse_dense, double* out_dense, int32_t* idx, int idx_cap,
               int32_t* counts, uint64_t* stats, float* pred_scores, double* nstats) {
    if (!cfg || !q || !k_cache || !v_cache || !block_table || !seq_lens || !out || !lse) return 1;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || d % 8 != 0 || d > 512) return 2;
    if (cfg->predictor == 1 && (!proj || cfg->rank % 8 != 0 || cfg->rank > d)) return 3;
    if (cfg->predictor == 2 && (!proj || cfg->rank != 32 || cfg->rank > d)) return 3;
    if (cfg->predictor < 0 || cfg->predictor > 2) return 3;
    if (cfg->guarantee != 0 && cfg->guarantee != 1) return 3;
    if (proj_heads != 1 && proj_heads != Hkv) return 3;
    if (idx && idx_cap < max_seq_len) return 4;
    if (!all_finite(q, (int64_t)B * Hq * d)) return 5;
    if ((cfg->predictor == 1 || cfg->predictor == 2) &&
        !all_finite(proj, (int64_t)proj_heads * d * cfg->rank))
        return 5;
    orc_init_constants();
    orc_ctx cx = {cfg, B, Hq, Hkv, d, max_blocks, kv_bf16, max_seq_len, q, k_cache, v_cache,
                  proj, proj_heads, block_table, seq_lens, out, lse, lse_dense, out_dense, idx, idx_cap,
                  counts, stats, pred_scores, nstats};
    int total = groups ? n_groups : B * Hkv;
    if (nthreads < 1) nthreads = 1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : bad)
    for (int t = 0; t < total; ++t) {
        int bg = groups ? groups[t] : t;
        bad |= decode_group(&cx, bg / Hkv, bg % Hkv);
    }
    return bad ? 5 : 0;
}

/*
 * Dense fp64 softmax attention over all L tokens of every query head of the
 * (b, g) groups in `groups` (all when NULL): the exact quantity the sparse
 * estimate approximates (scores q . K_i / sqrt(d), weights 1).  lse_dense
 * [B*Hq]; out_dense [B*Hq][d] or NULL.  Returns 0, 1 or 2 for bad arguments,
 * 5 for a non-finite input.
 */
int orc_dense(int B, int Hq, int Hkv, int d, int max_blocks, int kv_bf16, const float* q, const void* k_cache,
              const void* v_cache, const int32_t* block_table, const int32_t* seq_lens, const int32_t* groups,
              int n_groups, int nthreads, double* lse_dense, double* out_dense) {
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !lse_dense) return 1;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || d <= 0) return 2;
    if (!all_finite(q, (int64_t)B * Hq * d)) return 5;
    orc_ctx cx;
    memset(&cx, 0, sizeof(cx));
    cx.B = B; cx.Hq = Hq; cx.Hkv = Hkv; cx.d = d; cx.max_blocks = max_blocks; cx.kv_bf16 = kv_bf16;
    cx.block_table = block_table; cx.seq_lens = seq_lens;
    const int G = Hq / Hkv;
    int total = groups ? n_groups : B * Hkv;
    if (nthreads < 1) nthreads = 1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : bad)
    for (int t = 0; t < total; ++t) {
        int bg = groups ? groups[t] : t;
        int b = bg / Hkv, g = bg % Hkv, L = seq_lens[b];
        float* K = (float*)malloc(sizeof(float) * (size_t)(L > 0 ? L : 1) * d);
        float* V = (float*)malloc(sizeof(float) * (size_t)(L > 0 ? L : 1) * d);
        int* all = (int*)malloc(sizeof(int) * (L > 0 ? L : 1));
        double* w1 = (double*)malloc(sizeof(double) * (L > 0 ? L : 1));
        double* od = (double*)malloc(sizeof(double) * d);
        load_rows(&cx, k_cache, b, g, L, K);
        load_rows(&cx, v_cache, b, g, L, V);
        if (!all_finite(K, (int64_t)L * d) || !all_finite(V, (int64_t)L * d)) {
            bad |= 5;
        } else {
            for (int i = 0; i < L; ++i) { all[i] = i; w1[i] = 1.0; }
            for (int hl = 0; hl < G; ++hl) {
                int64_t bh = (int64_t)b * Hq + g * G + hl;
                attend_fp64(q + bh * d, K, V, d, all, w1, L, od, &lse_dense[bh]);
                if (out_dense) memcpy(out_dense + bh * d, od, sizeof(double) * d);
            }
        }
        free(K); free(V); free(all); free(w1); free(od);
    }
    return bad ? 5 : 0;
}

/*
 * Key second moments per KV head: gram[g][i][j] = sum over every sequence b
 * and every cached token t < seq_lens[b] of K_ti K_tj, in fp64 (the matrix
 * whose leading eigenvectors are the principal directions of the keys, the
 * PCA basis of the pith.science page "Loki: Low-rank Keys for Efficient
 * Sparse Attention", abstract).  absg (may be NULL) receives the same sums of
 * |K_ti| |K_tj|, the scale against which an fp32 accumulation's error is
 * bounded.  Plain loops: sequences ascending, tokens ascending.  Returns 0, 1
 * or 2 for bad arguments, 5 for a non-finite cached key.
 */
int orc_key_gram(int B, int Hkv, int d, int max_blocks, int kv_bf16, const void* k_cache,
                 const int32_t* block_table, const int32_t* seq_lens, double* gram, double* absg) {
    if (!k_cache || !block_table || !seq_lens || !gram) return 1;
    if (B <= 0 || Hkv <= 0 || d <= 0 || max_blocks <= 0) return 2;
    orc_ctx cx;
    memset(&cx, 0, sizeof(cx));
    cx.B = B; cx.Hkv = Hkv; cx.d = d; cx.max_blocks = max_blocks; cx.kv_bf16 = kv_bf16;
    cx.block_table = block_table; cx.seq_lens = seq_lens;
    memset(gram, 0, sizeof(double) * (size_t)Hkv * d * d);
    if (absg) memset(absg, 0, sizeof(double) * (size_t)Hkv * d * d);
    for (int b = 0; b < B; ++b) {
        int L = seq_lens[b];
        if (L < 0 || L > max_blocks * ORC_PAGE) return 2;
        float* K = (float*)malloc(sizeof(float) * (size_t)(L > 0 ? L : 1) * d);
        for (int g = 0; g < Hkv; ++g) {
            load_rows(&cx, k_cache, b, g, L, K);
            if (!all_finite(K, (int64_t)L * d)) { free(K); return 5; }
            double* G = gram + (size_t)g * d * d;
            double* A = absg ? absg + (size_t)g * d * d : NULL;
            for (int t = 0; t < L; ++t) {
                const float* k = K + (size_t)t * d;
                for (int i = 0; i < d; ++i)
                    for (int j = 0; j < d; ++j) {
                        G[(size_t)i * d + j] += (double)k[i] * (double)k[j];
                        if (A) A[(size_t)i * d + j] += fabs((double)k[i]) * fabs((double)k[j]);
                    }
            }
        }
        free(K);
    }
    return 0;
}
