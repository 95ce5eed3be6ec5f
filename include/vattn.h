/*
 * vattn.h -- C ABI of the MI355X (gfx950) verified sparse-attention decode step.
 *
 * The operation (edgentiq blog post "vAttention: a new approach to sparse
 * attention with guaranteed accuracy", sections "Introducing vAttention" and
 * "How vAttention Works"; SkyLight post "vAttention Computation"):
 * for one decode step and every query head h of every sequence b,
 *   1. a deterministic index set I_f = attention sinks (first `sinks` tokens)
 *      + sliding window (last `window` tokens, the newest included)
 *      + the k best tokens of the middle by a predictor score.  The predictor
 *      is either exact scaled scores ("oracle top-k", same post, section
 *      "Performance and Efficiency"), scores in a rank-r key space (pith.science
 *      page "Loki: Low-rank Keys for Efficient Sparse Attention", abstract),
 *      one basis for all heads or one per KV head, or the shared bits of
 *      32-bit hash signatures (HashAttention-style, same post and section);
 *   2. a uniform sample without replacement of the remaining tail, of N_t tokens.
 *      A base sample of n_b tokens estimates the spread of exp(s - m) over the
 *      tail.  The final size n is the central-limit budget
 *      n = (z * sigma * N_t / (eps * D))^2, with z = Phi^-1(1 - delta/2),
 *      clamped to [n_b, N_t].  It makes the softmax denominator estimate D
 *      relatively eps-accurate with probability >= 1 - delta.  The guarantee
 *      targets the denominator (same post, "How vAttention Works");
 *   3. out = sum_i w_i e^{s_i} V_i / sum_i w_i e^{s_i} over I_f + sample, with
 *      w = 1 on I_f and w = N_t / n (inverse inclusion probability) on the
 *      sample; lse = log sum_i w_i e^{s_i}.  Scores s_i = q . K_i / sqrt(d).
 *
 * Conventions for every entry point:
 *  - Device pointers are caller-owned.  No entry point allocates device or host
 *    memory; scratch space is the caller's workspace.
 *  - Work is enqueued asynchronously on `hip_stream` (a hipStream_t; NULL means
 *    the null stream).  No entry point synchronizes.
 *  - Errors are returned as vattn_status; nothing aborts or throws across the
 *    ABI.  Every host-checkable condition is validated before any launch; on a
 *    non-OK return nothing has been enqueued, except VATTN_E_HIP: a launch
 *    failed, and no kernel that consumes its output was enqueued after it.
 *    VATTN_E_HIP is also returned, before any launch, when the calling thread
 *    already has a HIP error pending from earlier calls (the error stays
 *    pending for the caller to read).
 *  - Thread safety: calls from several host threads may run concurrently as
 *    long as they do not share a workspace or outputs; the library keeps no
 *    mutable state besides a once-per-device kernel attribute flag (atomic).
 *  - Undefined (not checked on the device): seq_lens[b] > max_seq_len,
 *    block_table entries outside [0, num_blocks) for pages below
 *    ceil(seq_lens[b] / 16), non-finite values in q, K, V, P.
 *  - Deterministic: the same inputs and seed give bit-identical index sets,
 *    counts and statistics on any run, and bit-identical out/lse on one GPU.
 */
#ifndef VATTN_H
#define VATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VATTN_PAGE 16          /* tokens per KV page */
#define VATTN_MAX_SEQ (1 << 20) /* longest supported sequence */

typedef enum {
    VATTN_OK = 0,
    VATTN_E_NULL = 1,        /* a required pointer is NULL                         */
    VATTN_E_SHAPE = 2,       /* a size is outside the supported range              */
    VATTN_E_DTYPE = 3,       /* unknown kv dtype                                   */
    VATTN_E_CFG = 4,         /* a vattn_cfg field is out of range                  */
    VATTN_E_WORKSPACE = 5,   /* workspace NULL, too small or not 256-byte aligned  */
    VATTN_E_UNSUPPORTED = 6, /* valid request this build does not implement        */
    VATTN_E_HIP = 7          /* a HIP runtime call or kernel launch failed         */
} vattn_status;

typedef enum { VATTN_F32 = 0, VATTN_BF16 = 1 } vattn_dtype;

/* What the sample size guarantees (vattn_cfg.guarantee). */
typedef enum {
    VATTN_GUARANTEE_DENOMINATOR = 0, /* the softmax denominator (the pages' relaxation)     */
    VATTN_GUARANTEE_OUTPUT = 1       /* the denominator and the numerator sum w e^s V: the   */
                                     /* budget is the larger of the two CLT budgets         */
} vattn_guarantee;

typedef enum {
    VATTN_PRED_EXACT = 0,   /* top-k on exact scores q_s . K_i (reads K)          */
    VATTN_PRED_LOWRANK = 1, /* top-k on (q_s P) . Kt_i with Kt = bf16(K P) (reads Kt) */
    VATTN_PRED_HASH = 2     /* top-k on the bits shared by 32-bit signatures of q_s */
                            /* and K_i (reads k_sig, 4 bytes per token)            */
} vattn_predictor;

/* Decode configuration (host struct, read once per call). */
typedef struct {
    int32_t sinks;        /* >= 0: first tokens always kept                           */
    int32_t window;       /* >= 0: last tokens always kept (the newest included)       */
    int32_t topk_abs;     /* >= 0: k itself; -1: k = ceil(L * topk_ppm / 1e6)          */
    int32_t topk_ppm;     /* used when topk_abs < 0; in [0, 1e6]                       */
    int32_t base_ppm;     /* base sample = max(2, ceil(N_t * base_ppm / 1e6)), <= N_t; */
                          /* in [1, 1e6]; 50000 (5%) is the usual value               */
    int32_t force_budget; /* -1: CLT budget; >= 0: n = min(N_t, force_budget)          */
    int32_t predictor;    /* vattn_predictor                                          */
    int32_t rank;         /* r for VATTN_PRED_LOWRANK: 16, 32 or 64, <= d; 32 for      */
                          /* VATTN_PRED_HASH (signature bits)                         */
    double eps;           /* > 0: relative accuracy target of the denominator         */
    double delta;         /* in (0, 1): failure probability                           */
    uint64_t seed;        /* Philox4x32-10 key; callers vary it per step and layer     */
    int32_t guarantee;    /* vattn_guarantee.  VATTN_GUARANTEE_OUTPUT (SkyLight post   */
                          /* "vAttention Computation": (eps, delta) on the intermediate */
                          /* quantities; edgentiq post, "How vAttention Works": the     */
                          /* denominator-only budget is a relaxation) also holds the    */
                          /* numerator N = sum_i e^{s_i - m} V_i to the CLT bound in L2: */
                          /* n_N = z^2 N_t^2 TR n_b / ((n_b - 1) eps^2 NN) with          */
                          /* TR = sum_c max(n_b T2_c - T1_c^2, 0) and                    */
                          /* NN = sum_c (n_b NF_c + N_t T1_c)^2, where over the base     */
                          /* sample T1_c = sum E_i V_ic, T2_c = sum (E_i V_ic)^2, over   */
                          /* the fixed set NF_c = sum E_i V_ic, E_i the fixed-point      */
                          /* weights of the statistics; every sum in fp64, ascending     */
                          /* tokens within 1024-token spans from +0, the spans in order, */
                          /* channels ascending.  n = max(n_D, n_N) clamped as n_D.      */
                          /* Reads the V rows of the fixed sets and base samples once    */
                          /* more (two more kernels)                                     */
} vattn_cfg;

/* Inputs.  All pointers are device pointers except where noted.  k_cache and
 * v_cache may instead point into pinned host memory that is mapped for the
 * device (hipHostMalloc): the kernels then read only the rows they use over the
 * host link (edgentiq vAttention post, section "Performance and Efficiency":
 * decode with the KV cache hosted on the CPU), while k_lowrank and the workspace
 * stay in device memory. */
typedef struct {
    const float* q;             /* [B, Hq, d] fp32                                   */
    const void* k_cache;        /* [num_blocks, Hkv, 16, d] kv_dtype                  */
    const void* v_cache;        /* [num_blocks, Hkv, 16, d] kv_dtype                  */
    const uint16_t* k_lowrank;  /* [num_blocks, Hkv, 16, r] bf16 bits (LOWRANK only;  */
                                /* produced by vattn_project_keys), else NULL         */
    const float* proj;          /* [d, r] fp32, or [Hkv, d, r] (proj_heads = Hkv)     */
                                /* (LOWRANK and HASH, r = 32 for HASH), else NULL     */
    const int32_t* block_table; /* [B, max_blocks] page ids                           */
    const int32_t* seq_lens;    /* [B] tokens in each sequence, 0 <= L <= max_seq_len  */
    int32_t B;                  /* host: batch, >= 1                                  */
    int32_t Hq, Hkv;            /* host: query / KV heads; Hq / Hkv in {1, 2, 4, 8}   */
    int32_t d;                  /* host: head dim, 64 or 128                          */
    int32_t max_blocks;         /* host: row length of block_table                    */
    int32_t num_blocks;         /* host: pages in the caches                          */
    int32_t max_seq_len;        /* host: bound on seq_lens, 1 .. VATTN_MAX_SEQ,       */
                                /*       <= 16 * max_blocks                            */
    int32_t kv_dtype;           /* host: vattn_dtype of k_cache / v_cache             */
    int32_t proj_heads;         /* host: 0 or 1: one basis for all heads; Hkv: one    */
                                /*   basis per KV head (its query heads' low-rank     */
                                /*   queries and its low-rank keys use it); else      */
                                /*   VATTN_E_SHAPE                                    */
    const uint32_t* k_sig;      /* [num_blocks, Hkv, 16] key signatures (HASH only;   */
                                /* produced by vattn_sign_keys), else ignored         */
} vattn_inputs;

/* Outputs.  out and lse are required; the others are optional (NULL = skip). */
typedef struct {
    float* out;       /* [B, Hq, d] fp32: attention output (0 when L = 0)              */
    float* lse;       /* [B, Hq] fp32: log of the weighted denominator (-inf if L = 0)  */
    int32_t* idx;     /* [B, Hq, idx_cap]: the index set ascending, -1 padded           */
    int32_t idx_cap;  /* >= max_seq_len when idx != NULL                               */
    int32_t* counts;  /* [B, Hq, 6]: n_fixed, N_t, n_b, n, |I|, flags                  */
                      /*   flags bit0: n == N_t (exact), bit1: forced budget,          */
                      /*   bit2: CLT budget below n_b raised to n_b, bit3: the         */
                      /*   numerator's budget exceeded the denominator's (output mode) */
    uint64_t* stats;  /* [B, Hq, 4]: SF, S1, S2 high word, S2 low word: exact sums     */
                      /*   of E_i = trunc(exp(s_i - m) 2^40) over I_f (SF) and over    */
                      /*   the base sample (S1, and S2 of E_i^2 as 128 bits)           */
    int32_t* group_counts; /* [B, Hkv, 2]: tokens whose V row was gathered (the union  */
                      /*   of the group's index sets) and tokens whose K row the base-  */
                      /*   score pass read (union of fixed sets and base samples);      */
                      /*   for byte accounting                                          */
    double z_used;    /* host, written by vattn_decode: fp32-rounded z                  */
    double* num_stats; /* [B, Hq, 2] optional: TR, NN of the output-level mode (0 when   */
                      /*   the head has no base sample); ignored in the denominator mode */
} vattn_outputs;

/* Bytes of device workspace vattn_decode needs for these shapes and cfg
 * (0 if the arguments are invalid).  Depends only on host fields. */
size_t vattn_workspace_size(const vattn_inputs* in, const vattn_cfg* cfg);

/* One decode step (see the top of this file).  `workspace` is a device buffer
 * of at least vattn_workspace_size bytes, 256-byte aligned, not shared with a
 * concurrently running call; its contents need no initialization and are
 * garbage afterwards.  out->z_used is written on the host before launching. */
vattn_status vattn_decode(const vattn_inputs* in, const vattn_cfg* cfg, vattn_outputs* out,
                          void* workspace, size_t ws_bytes, void* hip_stream);

/* Bytes of the library's static device scratch (one copy per GPU, held until
 * the process ends) that vattn_decode_noalloc uses in place of a workspace. */
#define VATTN_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/* vattn_decode without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The kernels' scratch space is a static device array
 * of VATTN_NOALLOC_SCRATCH_BYTES bytes inside the library; its device address
 * is looked up on the first call on each device (with that device current),
 * after which no call makes any allocating HIP or library call.  The caller
 * still passes inputs and outputs exactly as for vattn_decode, with the same
 * results.  Returns VATTN_E_WORKSPACE, before any HIP call, when
 * vattn_workspace_size(in, cfg) exceeds VATTN_NOALLOC_SCRATCH_BYTES (e.g.
 * 8 sequences x 32K tokens x 32 query heads need 64 MiB and fit; 64 x 16K
 * do not); other errors as for vattn_decode.  Every call on one GPU shares that
 * GPU's array and leaves it holding its contents (no call needs it cleared):
 * two calls that overlap on one GPU (other streams, other host threads) race
 * and give undefined results, so such callers serialise them or use
 * vattn_decode with separate workspaces.  Asynchronous on hip_stream. */
vattn_status vattn_decode_noalloc(const vattn_inputs* in, const vattn_cfg* cfg, vattn_outputs* out,
                                  void* hip_stream);

/* Kernels of one decode step, in launch order (for vattn_decode_profiled). */
#define VATTN_NUM_STAGES 7 /* predict, select, base, budget, gather, combine, emit */

/* vattn_decode, additionally recording caller-created hipEvent_t handles on
 * hip_stream: events[0] before the first kernel and events[s + 1] after stage s
 * (stage 6, emit, is empty when out->idx is NULL).  n_events must be
 * VATTN_NUM_STAGES + 1.  For measurement; timing adds event records only. */
vattn_status vattn_decode_profiled(const vattn_inputs* in, const vattn_cfg* cfg,
                                   vattn_outputs* out, void* workspace, size_t ws_bytes,
                                   void* hip_stream, void* const* events, int32_t n_events);

/* Low-rank key cache for the LOWRANK predictor (Loki page, abstract: keys
 * scored in a low-dimensional space): k_lowrank[p][g][t][j] =
 * bf16_rne(pdot(K[p][g][t][:], P_g[:, j])) for every page p < num_blocks,
 * P_g = proj (proj_heads 0 or 1: [d, r] fp32) or proj[g] (proj_heads = Hkv:
 * [Hkv, d, r] fp32); another proj_heads gives VATTN_E_SHAPE.
 * k_cache: [num_blocks, Hkv, 16, d] kv_dtype;
 * k_lowrank: [num_blocks, Hkv, 16, r] bf16 bits (output).  pdot is the
 * blocked fp32 dot product the predictor uses (fma chains over blocks of 8,
 * then a pairwise tree over the block partials).  Asynchronous on hip_stream. */
vattn_status vattn_project_keys(const void* k_cache, int32_t kv_dtype, const float* proj,
                                uint16_t* k_lowrank, int32_t num_blocks, int32_t Hkv,
                                int32_t d, int32_t r, int32_t proj_heads, void* hip_stream);

/* Key-side maintenance for one decode step: writes the newest token of each
 * sequence into the paged caches and, when k_lowrank is given, its low-rank
 * key row, so the predictor stream of the next vattn_decode sees it (the
 * window of the decode step includes this newest token).
 * For every b < B with pos[b] >= 0, page = block_table[b][pos[b] / 16],
 * slot = pos[b] % 16, and every KV head g:
 *   k_cache[page][g][slot][:]   = k_new[b][g][:]
 *   v_cache[page][g][slot][:]   = v_new[b][g][:]
 *   k_lowrank[page][g][slot][j] = bf16_rne(pdot(k_new[b][g][:], P_g[:, j]))
 * with the same pdot and rounding as vattn_project_keys.  pos[b] < 0 leaves
 * sequence b untouched.
 * k_new, v_new: [B, Hkv, d] in kv_dtype (device); pos: [B] int32 (device);
 * block_table: [B, max_blocks] int32 (device); caches as for vattn_decode;
 * k_lowrank and proj are both NULL or both given; proj and proj_heads as for
 * vattn_project_keys (P_g the KV head's basis).  All pointers
 * are caller-owned and 16-byte aligned; the library allocates nothing.
 * Returns VATTN_E_NULL, VATTN_E_DTYPE, VATTN_E_SHAPE or VATTN_E_UNSUPPORTED
 * before any launch for bad arguments, VATTN_E_HIP for a failed launch.
 * pos[b] >= 16 * max_blocks and block ids outside [0, num_blocks) are
 * undefined behaviour (not checked on the device).  Two sequences must not
 * write the same page slot.  Asynchronous on hip_stream. */
vattn_status vattn_append_kv(const void* k_new, const void* v_new, const int32_t* pos,
                             const int32_t* block_table, int32_t B, int32_t max_blocks,
                             void* k_cache, void* v_cache, uint16_t* k_lowrank, const float* proj,
                             int32_t kv_dtype, int32_t num_blocks, int32_t Hkv, int32_t d, int32_t r,
                             int32_t proj_heads, void* hip_stream);

/* Key signatures for the HASH predictor.  HashAttention (named as a top-k
 * method in the edgentiq vAttention post, section "Performance and
 * Efficiency") ranks tokens by bit signatures of query and key; with no
 * trained hash the signatures here are random-hyperplane sign bits (Charikar's
 * SimHash): bit j of k_sig[p][g][t] is set when pdot(K[p][g][t][:], P_g[:, j])
 * > 0, j < 32, with P_g = proj ([d, 32] fp32, proj_heads 0 or 1) or proj[g]
 * ([Hkv, d, 32], proj_heads = Hkv), and the same pdot as vattn_project_keys.
 * The decode signs q_s the same way and scores a token by the number of equal
 * bits (0 .. 32), lower index first among equal scores.
 * k_cache: [num_blocks, Hkv, 16, d] kv_dtype; k_sig: [num_blocks, Hkv, 16]
 * uint32 (output, 16-byte aligned).  Errors as for vattn_project_keys, before
 * any launch.  Asynchronous on hip_stream. */
vattn_status vattn_sign_keys(const void* k_cache, int32_t kv_dtype, const float* proj, uint32_t* k_sig,
                             int32_t num_blocks, int32_t Hkv, int32_t d, int32_t proj_heads,
                             void* hip_stream);

/* vattn_append_kv for the HASH predictor: writes the newest token's K and V
 * rows as vattn_append_kv does, and its signature
 *   k_sig[page][g][slot] = signature of k_new[b][g][:] under P_g
 * exactly as vattn_sign_keys computes it.  Arguments, errors and undefined
 * behaviour as for vattn_append_kv, with k_sig ([num_blocks, Hkv, 16] uint32)
 * and proj ([d, 32] or [Hkv, d, 32]) both required. */
vattn_status vattn_append_kv_sig(const void* k_new, const void* v_new, const int32_t* pos,
                                 const int32_t* block_table, int32_t B, int32_t max_blocks,
                                 void* k_cache, void* v_cache, uint32_t* k_sig, const float* proj,
                                 int32_t kv_dtype, int32_t num_blocks, int32_t Hkv, int32_t d,
                                 int32_t proj_heads, void* hip_stream);

/* Key Gram matrices for a per-head predictor basis.  The Loki page (abstract)
 * finds that key vectors lie in a much lower-dimensional space; a KV head's
 * basis P_g for vattn_project_keys (proj_heads = Hkv) can be taken as the r
 * leading eigenvectors of
 *   gram[g][i][j] = sum over b < B, t < seq_lens[b] of K[b, t, g, i] K[b, t, g, j]
 * (K[b, t, g] the cached key of token t of sequence b, read through
 * block_table as in vattn_decode), the keys' uncentered second moments.  The
 * eigensolve of this d x d matrix is the caller's (host calibration, outside
 * the decode path).  Products and sums are fp32 (matrix-core bf16 products,
 * exact in fp32, then fp32 sums in a fixed order: the result is the same on
 * every call).
 * k_cache: [num_blocks, Hkv, 16, d] bf16 only (VATTN_E_UNSUPPORTED for fp32);
 * block_table [B, max_blocks], seq_lens [B] int32 (device); gram: [Hkv, d, d]
 * fp32 (device, output); workspace: device buffer of at least
 * vattn_key_gram_workspace_size bytes, 256-byte aligned, contents garbage
 * afterwards.  Host-checkable errors are returned before any launch; the
 * library allocates nothing.  Asynchronous on hip_stream. */
size_t vattn_key_gram_workspace_size(int32_t B, int32_t Hkv, int32_t d, int32_t max_seq_len);
vattn_status vattn_key_gram(const void* k_cache, int32_t kv_dtype, const int32_t* block_table,
                            const int32_t* seq_lens, int32_t B, int32_t max_blocks, int32_t num_blocks,
                            int32_t Hkv, int32_t d, int32_t max_seq_len, float* gram, void* workspace,
                            size_t ws_bytes, void* hip_stream);

/* Device read-stream calibration (no part of the method): reads every byte of
 * buf once with 16-byte non-temporal loads, as the decode's streams do, and
 * XORs the buffer's 32-bit words into the VATTN_READ_PROBE_SINK words of sink
 * (one atomic per block, spread over the words; the caller clears sink): the
 * XOR of the sink's words is then the XOR of the buffer's.  Timed over a
 * large buffer it gives the device's read-only streaming rate, the ceiling of
 * the decode's read-dominated kernels (a copy, which also writes,
 * understates it).  buf: device, 16-byte aligned, bytes a positive multiple
 * of 16; sink: VATTN_READ_PROBE_SINK device uint32 words.  VATTN_E_NULL /
 * VATTN_E_SHAPE before any launch.  Asynchronous on hip_stream. */
#define VATTN_READ_PROBE_SINK 1024
vattn_status vattn_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* hip_stream);

/* z = Phi^-1(1 - delta/2) rounded to fp32, as vattn_decode uses it (host). */
double vattn_z_from_delta(double delta);

/* Static string naming a status code. */
const char* vattn_status_string(vattn_status s);

#ifdef __cplusplus
}
#endif
#endif /* VATTN_H */
