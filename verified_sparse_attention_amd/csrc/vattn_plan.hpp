// Internal launch plan shared by the host C ABI and the kernels.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace vattn {

constexpr int kPage = 16;
constexpr int kPredThreads = 1024;   // predictor + chunk top-k
constexpr int kSelectThreads = 1024; // per-head exact top-k and base threshold
constexpr int kBudgetThreads = 1024;  // per-head statistics, budget and final threshold
constexpr int kManyHeads = 1024;     // from this many query heads (B * Hq) on, the per-head
constexpr int kHeadThreadsMany = 256; // select, budget, combine and emit run 256-thread blocks, several per CU
constexpr int kChunkThreads = 256;   // base scores and gather
constexpr int kEmitThreads = 1024;   // index-set emission
constexpr int kEmitQuads = 8;       // token quads per lane and pass of the index-set emission
constexpr int kPredKeys = 32768;     // predictor keys held in LDS per block (128 KiB)
static_assert(kPredKeys <= 65536, "a predictor chunk's token offsets fit 16 bits");
constexpr int kSampBits = 11;        // sampler histogram: top bits of the Philox word
constexpr int kSampBins = 1 << kSampBits;
constexpr int kTopBuckets = 256;     // value-range buckets of the top-k select
constexpr int kListCap = 128;        // boundary-bucket list capacity per head
constexpr int kPremergeParts = 4;    // candidate parts after the pre-merge
constexpr int kPremergeMaxHeads = 128;  // pre-merge when B*Hq is below this ...
constexpr int kPremergeMinChunks = 16;  // ... and there are at least this many predictor chunks
constexpr int kGatherChunk = 4 * kChunkThreads;  // tokens per base/gather block
constexpr int kMaxLds = 160 * 1024;  // LDS per workgroup on gfx950
constexpr int kGramChunk = 4096;     // tokens per partial of the key Gram matrices
constexpr int kGramTile = 128;       // tokens staged in LDS at a time
constexpr int kProbeSink = 1024;     // words of the read probe's sink
#define VATTN_MAX_SEQ_TOKENS (1 << 20)

// Per (sequence, query head) state handed from kernel to kernel.
struct HeadState {
    int32_t L, k, n_fixed, NT, nb, n, flags, pad;
    uint64_t thr_b;  // base sample  = tail tokens with sample key >= thr_b (nb > 0)
    uint64_t thr_n;  // final sample = tail tokens with sample key >= thr_n (n > 0)
    float m;         // max pinned score over I_f and the base sample
    float wsamp;     // N_t / n as fp32
    uint64_t SF, S1, S2hi, S2lo;  // exact sums, written by the budget pass
};

struct Plan {
    // shapes
    int B, Hq, Hkv, G, d, r, max_blocks, max_seq_len, words;
    // configuration
    int sinks, window, topk_abs, topk_ppm, base_ppm, force_budget, predictor, kv_bf16;
    int guarantee;  // 0 denominator; 1 denominator and numerator (output-level mode)
    float scale32;
    double z32, eps;
    uint32_t seed_lo, seed_hi;
    // chunking
    int cp, ncp, kcap;  // predictor chunk (tokens), chunks per sequence, candidate slots
    int cg, ncg;        // gather chunk (tokens), chunks per sequence
    // inputs
    const float* q;
    const void* k;
    const void* v;
    const uint16_t* kt;
    const uint32_t* ksig;  // [num_blocks][Hkv][16] key signatures (signature predictor)
    const float* proj;
    int proj_stride;  // floats between the KV heads' bases (0: one basis for all)
    const int32_t* bt;
    const int32_t* seq_lens;
    // workspace
    uint64_t* cand;  // [B*Hq][ncp][kcap] composite (score key, ~index)
    uint32_t* bits;  // [B*Hq][words] fixed-set membership bitmap
    HeadState* hs;   // [B*Hq]
    float* cmax;     // [B*Hq][ncg] chunk max of pinned scores
    float* part;     // [B*Hq][ncg][d + 2] online-softmax partials (m, l, acc[d])
    uint32_t* soff;  // [B*Hkv][ncp][kSampBins + 1] bin offsets of each chunk's middle tokens
    uint16_t* slist; // [B*Hkv][ncp][cp] each chunk's middle tokens grouped by sample-word bin (offsets in the chunk)
    uint32_t* hh;    // [B*Hq][kSampBins] sampler-word histogram of each head's tail
    float* bsc;      // [B*Hkv][ncg][G][cg] pinned scores of the base-pass members, in list order
                     // (ascending token order within the chunk), one row per head; read by budget and gather
    uint16_t* bmeta; // [B*Hkv][ncg][cg] base mask | fixed mask << 8 (G <= 8 heads: 16 bits)
    int32_t* bcnt;   // [B*Hkv][ncg] members per base chunk
    uint32_t* brow;  // [B*Hkv][ncg][cg] V row of each base-pass member (output-level mode, else null)
    double* npart;   // [B*Hq][ncg][3][d] numerator partials T1, T2, NF per chunk (output-level mode)
    uint32_t* crange;  // [B*Hq][ncp][2] order-key bracket (min, max) of each chunk's candidates
    uint32_t* gw;      // [B*Hkv] gather dispatch weight: max over the group's heads of (n_fixed + n) / L, fp32 bits
    int32_t* gorder;   // [B*Hkv] groups by descending gw (ties to the lower group), for more groups than a gather block has threads
    // pre-merged candidate parts (nparts > 0 only: few heads, many chunks)
    int nparts, kcap2; // parts; key slots per part = min(k bound, cp * chunks in the largest part)
    uint64_t* cand2;   // [B*Hq][nparts][kcap2] each part's exact top-min(k, n) keys
    uint32_t* crange2; // [B*Hq][nparts][2] their order-key brackets
    int32_t* pcount;   // [B*Hq][nparts] keys per part
    uint32_t* hist2;   // [B*Hkv][nparts][kSampBins] tail sample-word histogram per part
    // outputs
    float* out;
    float* lse;
    int32_t* idx;
    int32_t idx_cap;
    int32_t* counts;
    uint64_t* stats;
    int32_t* gcounts;  // [B*Hkv][2] optional
    double* nstats;    // [B*Hq][2] numerator statistics TR, NN (output-level mode), optional
};

// Launches one decode step.  Returns 0 or a hipError_t value.
int launch_decode(const Plan& p, void* stream, void* const* events = nullptr);
int launch_project(const void* k_cache, int kv_bf16, const float* proj, int proj_stride, uint16_t* kt,
                   int num_blocks, int Hkv, int d, int r, void* stream);
size_t predict_lds_bytes(int G, int d, int row, int cp);
int launch_gram(const uint16_t* k_cache, const int32_t* bt, const int32_t* seq_lens, int B, int max_blocks,
                int Hkv, int d, int max_seq_len, float* gram, float* part, void* stream);
int launch_append(const void* k_new, const void* v_new, const int32_t* pos, const int32_t* bt, int B,
                  int max_blocks, void* k_cache, void* v_cache, uint16_t* kt, uint32_t* ksig, const float* proj,
                  int proj_stride, int kv_bf16, int Hkv, int d, int r, void* stream);
int launch_sign(const void* k_cache, int kv_bf16, const float* proj, int proj_stride, uint32_t* ksig,
                int num_blocks, int Hkv, int d, void* stream);
int launch_read_probe(const void* buf, size_t n16, uint32_t* sink, void* stream);

}  // namespace vattn
