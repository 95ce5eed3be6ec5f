// Host side of the C ABI declared in include/vattn.h: argument validation,
// the launch plan, the workspace layout and z = Phi^-1(1 - delta/2).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "vattn.h"
#include "vattn_plan.hpp"

namespace {

constexpr size_t kAlign = 256;
static_assert(VATTN_MAX_SEQ == VATTN_MAX_SEQ_TOKENS, "sequence bound differs from the kernels'");

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Upper-tail standard normal quantile: z with P(Z > z) = p, 0 < p < 1.
// Start from the Abramowitz-Stegun 26.2.23 rational approximation and refine
// with Newton steps on the exact tail 0.5 * erfc(z / sqrt 2).
double normal_isf(double p) {
    const bool upper = p <= 0.5;
    const double pp = upper ? p : 1.0 - p;
    const double t = std::sqrt(-2.0 * std::log(pp));
    double z = t - (2.515517 + 0.802853 * t + 0.010328 * t * t) /
                       (1.0 + 1.432788 * t + 0.189269 * t * t + 0.001308 * t * t * t);
    const double inv_sqrt2 = 0.70710678118654752440;
    const double inv_sqrt2pi = 0.39894228040143267794;
    for (int it = 0; it < 8; ++it) {
        const double tail = 0.5 * std::erfc(z * inv_sqrt2);
        const double dens = inv_sqrt2pi * std::exp(-0.5 * z * z);
        if (!(dens > 0.0)) break;
        const double step = (tail - pp) / dens;
        z += step;
        if (std::fabs(step) <= 1e-17 * std::fabs(z)) break;
    }
    return upper ? z : -z;
}

// Width of the predictor's query rows: r (low rank), 32 (signature bits) or d (exact).
int pred_row(const vattn_inputs* in, const vattn_cfg* cfg) {
    return cfg->predictor == VATTN_PRED_LOWRANK ? cfg->rank : cfg->predictor == VATTN_PRED_HASH ? 32 : in->d;
}

struct Shape {
    int G, cp, ncp, kcap, cg, ncg, words, nparts, kcap2, guarantee;
};

vattn_status check(const vattn_inputs* in, const vattn_cfg* cfg, Shape* sh) {
    if (!in || !cfg) return VATTN_E_NULL;
    if (in->B < 1 || in->Hq < 1 || in->Hkv < 1 || in->Hq % in->Hkv != 0) return VATTN_E_SHAPE;
    const int G = in->Hq / in->Hkv;
    if (G != 1 && G != 2 && G != 4 && G != 8) return VATTN_E_UNSUPPORTED;
    if (in->d != 64 && in->d != 128) return VATTN_E_UNSUPPORTED;
    if (in->max_seq_len < 1 || in->max_seq_len > VATTN_MAX_SEQ) return VATTN_E_SHAPE;
    if (in->max_blocks < 1 || static_cast<long long>(in->max_blocks) * VATTN_PAGE < in->max_seq_len)
        return VATTN_E_SHAPE;
    if (in->num_blocks < 1) return VATTN_E_SHAPE;
    if (static_cast<long long>(in->B) * in->Hkv > 65535) return VATTN_E_SHAPE;
    if (in->kv_dtype != VATTN_F32 && in->kv_dtype != VATTN_BF16) return VATTN_E_DTYPE;
    if (in->proj_heads != 0 && in->proj_heads != 1 && in->proj_heads != in->Hkv) return VATTN_E_SHAPE;
    if (cfg->sinks < 0 || cfg->window < 0 || cfg->topk_abs < -1) return VATTN_E_CFG;
    if (cfg->topk_ppm < 0 || cfg->topk_ppm > 1000000) return VATTN_E_CFG;
    if (cfg->base_ppm < 1 || cfg->base_ppm > 1000000) return VATTN_E_CFG;
    if (cfg->force_budget < -1) return VATTN_E_CFG;
    if (cfg->predictor != VATTN_PRED_EXACT && cfg->predictor != VATTN_PRED_LOWRANK &&
        cfg->predictor != VATTN_PRED_HASH)
        return VATTN_E_CFG;
    if (cfg->predictor == VATTN_PRED_HASH && cfg->rank != 32) return VATTN_E_UNSUPPORTED;
    if (cfg->predictor == VATTN_PRED_LOWRANK) {
        if (cfg->rank != 16 && cfg->rank != 32 && cfg->rank != 64) return VATTN_E_UNSUPPORTED;
        if (cfg->rank > in->d) return VATTN_E_CFG;
    }
    if (!(cfg->eps > 0.0) || !std::isfinite(cfg->eps)) return VATTN_E_CFG;
    if (!(cfg->delta > 0.0 && cfg->delta < 1.0)) return VATTN_E_CFG;
    if (cfg->guarantee != VATTN_GUARANTEE_DENOMINATOR && cfg->guarantee != VATTN_GUARANTEE_OUTPUT) return VATTN_E_CFG;
    if (sh) {
        sh->G = G;
        sh->guarantee = cfg->guarantee;
        // Predictor chunk: the keys of G heads stay in LDS (at most kPredKeys
        // and within the workgroup LDS limit).  Below that bound, aim for one
        // chunk per compute unit over the whole batch, but keep chunks of at
        // least 2048 tokens so the chunk top-k stays a small fraction of them.
        const int prow = pred_row(in, cfg);
        int cpmax = vattn::kPredKeys / G;
        while (cpmax > vattn::kPage &&
               vattn::predict_lds_bytes(G, in->d, prow, cpmax) > static_cast<size_t>(vattn::kMaxLds))
            cpmax -= vattn::kPage;
        const long long spread = (static_cast<long long>(in->max_seq_len) * in->B * in->Hkv + 255) / 256;
        long long cp = (spread + vattn::kPage - 1) / vattn::kPage * vattn::kPage;
        if (cp < 2048) cp = 2048;
        if (cp > cpmax) cp = cpmax;
        sh->cp = static_cast<int>(cp);
        sh->ncp = (in->max_seq_len + sh->cp - 1) / sh->cp;
        const long long kmax = cfg->topk_abs >= 0
                                   ? static_cast<long long>(cfg->topk_abs)
                                   : (static_cast<long long>(in->max_seq_len) * cfg->topk_ppm + 999999) / 1000000;
        long long kc = kmax < sh->cp ? kmax : sh->cp;
        sh->kcap = static_cast<int>(kc < 1 ? 1 : kc);
        sh->cg = vattn::kGatherChunk;
        sh->ncg = (in->max_seq_len + sh->cg - 1) / sh->cg;
        sh->words = (in->max_seq_len + 31) / 32;
        // few heads and many predictor chunks: pre-merge the chunk candidates
        // in parts so the per-head select is not left with every chunk
        sh->nparts = (static_cast<long long>(in->B) * in->Hq < vattn::kPremergeMaxHeads &&
                      sh->ncp >= vattn::kPremergeMinChunks) ? vattn::kPremergeParts : 0;
        // a part keeps min(k, its chunks' candidates): at most k, and at most
        // cp tokens from each of its chunks (the largest part has ceil(ncp / parts))
        if (sh->nparts) {
            const long long per = static_cast<long long>(sh->cp) * ((sh->ncp + sh->nparts - 1) / sh->nparts);
            sh->kcap2 = static_cast<int>(kmax < per ? (kmax < 1 ? 1 : kmax) : per);
        } else {
            sh->kcap2 = 0;
        }
    }
    return VATTN_OK;
}

struct Layout {
    size_t cand, bits, hs, cmax, part, soff, slist, hh, bsc, bmeta, bcnt, crange, gw, cand2, crange2, pcount, hist2,
        brow, npart, total;
};

Layout layout(const vattn_inputs* in, const Shape& s) {
    const size_t BHq = static_cast<size_t>(in->B) * in->Hq;
    const size_t BHkv = static_cast<size_t>(in->B) * in->Hkv;
    Layout L{};
    size_t off = 0;
    L.cand = off;
    off += align_up(BHq * s.ncp * s.kcap * sizeof(uint64_t));
    L.bits = off;
    off += align_up(BHq * s.words * sizeof(uint32_t));
    L.hs = off;
    off += align_up(BHq * sizeof(vattn::HeadState));
    L.cmax = off;
    off += align_up(BHq * s.ncg * sizeof(float));
    L.part = off;
    off += align_up(BHq * s.ncg * static_cast<size_t>(in->d + 2) * sizeof(float));
    L.soff = off;
    off += align_up(BHkv * s.ncp * (vattn::kSampBins + 1) * sizeof(uint32_t));
    L.slist = off;
    off += align_up(BHkv * s.ncp * static_cast<size_t>(s.cp) * sizeof(uint16_t));
    L.hh = off;
    off += align_up(BHq * vattn::kSampBins * sizeof(uint32_t));
    L.bsc = off;
    off += align_up(BHkv * s.ncg * s.cg * s.G * sizeof(float));
    L.bmeta = off;
    off += align_up(BHkv * s.ncg * s.cg * sizeof(uint16_t));
    L.bcnt = off;
    off += align_up(BHkv * s.ncg * sizeof(int32_t));
    L.crange = off;
    off += align_up(BHq * s.ncp * 2 * sizeof(uint32_t));
    L.gw = off;  // gw, then gorder
    off += align_up(2 * BHkv * sizeof(uint32_t));
    L.cand2 = off;
    off += align_up(BHq * s.nparts * static_cast<size_t>(s.kcap2) * sizeof(uint64_t));
    L.crange2 = off;
    off += align_up(BHq * s.nparts * 2 * sizeof(uint32_t));
    L.pcount = off;
    off += align_up(BHq * s.nparts * sizeof(int32_t));
    L.hist2 = off;
    off += align_up(BHkv * s.nparts * vattn::kSampBins * sizeof(uint32_t));
    const bool num = s.guarantee == VATTN_GUARANTEE_OUTPUT;  // the output-level mode's arrays
    L.brow = off;
    off += num ? align_up(BHkv * s.ncg * s.cg * sizeof(uint32_t)) : 0;
    L.npart = off;
    off += num ? align_up(BHq * s.ncg * 3 * static_cast<size_t>(in->d) * sizeof(double)) : 0;
    L.total = off;
    return L;
}

}  // namespace

extern "C" {

double vattn_z_from_delta(double delta) {
    if (!(delta > 0.0 && delta < 1.0)) return NAN;
    return static_cast<double>(static_cast<float>(normal_isf(delta / 2.0)));
}

size_t vattn_workspace_size(const vattn_inputs* in, const vattn_cfg* cfg) {
    Shape s{};
    if (check(in, cfg, &s) != VATTN_OK) return 0;
    return layout(in, s).total;
}

static vattn_status decode_impl(const vattn_inputs* in, const vattn_cfg* cfg, vattn_outputs* out,
                                void* workspace, size_t ws_bytes, void* hip_stream,
                                void* const* events) {
    Shape s{};
    vattn_status st = check(in, cfg, &s);
    if (st != VATTN_OK) return st;
    if (!out || !out->out || !out->lse) return VATTN_E_NULL;
    if (!in->q || !in->k_cache || !in->v_cache || !in->block_table || !in->seq_lens) return VATTN_E_NULL;
    if (cfg->predictor == VATTN_PRED_LOWRANK && (!in->k_lowrank || !in->proj)) return VATTN_E_NULL;
    if (cfg->predictor == VATTN_PRED_HASH && (!in->k_sig || !in->proj)) return VATTN_E_NULL;
    if (!aligned(in->q, 16) || !aligned(in->k_cache, 16) || !aligned(in->v_cache, 16) ||
        (in->k_lowrank && !aligned(in->k_lowrank, 16)) || (in->proj && !aligned(in->proj, 4)) ||
        (cfg->predictor == VATTN_PRED_HASH && !aligned(in->k_sig, 16)))
        return VATTN_E_SHAPE;
    if (out->idx && out->idx_cap < in->max_seq_len) return VATTN_E_SHAPE;
    const Layout L = layout(in, s);
    if (!workspace || !aligned(workspace, kAlign) || ws_bytes < L.total) return VATTN_E_WORKSPACE;
    const int prow = pred_row(in, cfg);
    if (vattn::predict_lds_bytes(s.G, in->d, prow, s.cp) > static_cast<size_t>(vattn::kMaxLds))
        return VATTN_E_UNSUPPORTED;  // unreachable: the chunk is sized to fit

    vattn::Plan p{};
    p.B = in->B;
    p.Hq = in->Hq;
    p.Hkv = in->Hkv;
    p.G = s.G;
    p.d = in->d;
    p.r = prow;
    p.max_blocks = in->max_blocks;
    p.max_seq_len = in->max_seq_len;
    p.words = s.words;
    p.sinks = cfg->sinks;
    p.window = cfg->window;
    p.topk_abs = cfg->topk_abs;
    p.topk_ppm = cfg->topk_ppm;
    p.base_ppm = cfg->base_ppm;
    p.force_budget = cfg->force_budget;
    p.predictor = cfg->predictor;
    p.kv_bf16 = in->kv_dtype == VATTN_BF16;
    p.scale32 = static_cast<float>(1.0 / std::sqrt(static_cast<double>(in->d)));
    p.z32 = vattn_z_from_delta(cfg->delta);
    p.eps = cfg->eps;
    p.seed_lo = static_cast<uint32_t>(cfg->seed);
    p.seed_hi = static_cast<uint32_t>(cfg->seed >> 32);
    p.cp = s.cp;
    p.ncp = s.ncp;
    p.kcap = s.kcap;
    p.cg = s.cg;
    p.ncg = s.ncg;
    p.q = in->q;
    p.k = in->k_cache;
    p.v = in->v_cache;
    p.kt = in->k_lowrank;
    p.ksig = cfg->predictor == VATTN_PRED_HASH ? in->k_sig : nullptr;
    p.proj = in->proj;
    p.proj_stride = (in->proj_heads > 1 && cfg->predictor != VATTN_PRED_EXACT) ? in->d * prow : 0;
    p.bt = in->block_table;
    p.seq_lens = in->seq_lens;
    char* ws = static_cast<char*>(workspace);
    p.cand = reinterpret_cast<uint64_t*>(ws + L.cand);
    p.bits = reinterpret_cast<uint32_t*>(ws + L.bits);
    p.hs = reinterpret_cast<vattn::HeadState*>(ws + L.hs);
    p.cmax = reinterpret_cast<float*>(ws + L.cmax);
    p.part = reinterpret_cast<float*>(ws + L.part);
    p.soff = reinterpret_cast<uint32_t*>(ws + L.soff);
    p.slist = reinterpret_cast<uint16_t*>(ws + L.slist);
    p.hh = reinterpret_cast<uint32_t*>(ws + L.hh);
    p.bsc = reinterpret_cast<float*>(ws + L.bsc);
    p.bmeta = reinterpret_cast<uint16_t*>(ws + L.bmeta);
    p.bcnt = reinterpret_cast<int32_t*>(ws + L.bcnt);
    p.crange = reinterpret_cast<uint32_t*>(ws + L.crange);
    p.gw = reinterpret_cast<uint32_t*>(ws + L.gw);
    p.gorder = reinterpret_cast<int32_t*>(p.gw + static_cast<size_t>(in->B) * in->Hkv);
    p.nparts = s.nparts;
    p.kcap2 = s.kcap2;
    p.cand2 = reinterpret_cast<uint64_t*>(ws + L.cand2);
    p.crange2 = reinterpret_cast<uint32_t*>(ws + L.crange2);
    p.pcount = reinterpret_cast<int32_t*>(ws + L.pcount);
    p.hist2 = reinterpret_cast<uint32_t*>(ws + L.hist2);
    p.guarantee = cfg->guarantee;
    p.brow = s.guarantee == VATTN_GUARANTEE_OUTPUT ? reinterpret_cast<uint32_t*>(ws + L.brow) : nullptr;
    p.npart = s.guarantee == VATTN_GUARANTEE_OUTPUT ? reinterpret_cast<double*>(ws + L.npart) : nullptr;
    p.out = out->out;
    p.lse = out->lse;
    p.idx = out->idx;
    p.idx_cap = out->idx_cap;
    p.counts = out->counts;
    p.stats = out->stats;
    p.gcounts = out->group_counts;
    p.nstats = s.guarantee == VATTN_GUARANTEE_OUTPUT ? out->num_stats : nullptr;
    out->z_used = p.z32;
    const int rc = vattn::launch_decode(p, hip_stream, events);
    return rc == 0 ? VATTN_OK : VATTN_E_HIP;
}

vattn_status vattn_decode(const vattn_inputs* in, const vattn_cfg* cfg, vattn_outputs* out,
                          void* workspace, size_t ws_bytes, void* hip_stream) {
    return decode_impl(in, cfg, out, workspace, ws_bytes, hip_stream, nullptr);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Static device scratch for vattn_decode_noalloc.  In host code `scratch` is
// only a stand-in for the device array: its device address (one per GPU, each
// holding its own copy) is looked up once per device with that device current
// and kept in scratch_ptr, which is what the kernels receive.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[VATTN_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];  // guarded by scratch_mu

// The current device's copy of `scratch`, looked up on its first use.
vattn_status current_scratch(void** ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return VATTN_E_HIP;
    if (dev >= kMaxDevices) return VATTN_E_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return VATTN_E_HIP;
        scratch_ptr[dev] = p;
    }
    *ptr = scratch_ptr[dev];
    return VATTN_OK;
}
}  // namespace

extern "C" {

vattn_status vattn_decode_noalloc(const vattn_inputs* in, const vattn_cfg* cfg, vattn_outputs* out,
                                  void* hip_stream) {
    Shape s{};
    const vattn_status st = check(in, cfg, &s);
    if (st != VATTN_OK) return st;
    if (layout(in, s).total > VATTN_NOALLOC_SCRATCH_BYTES) return VATTN_E_WORKSPACE;  // before any HIP call
    void* ws = nullptr;
    const vattn_status sst = current_scratch(&ws);
    if (sst != VATTN_OK) return sst;
    return decode_impl(in, cfg, out, ws, VATTN_NOALLOC_SCRATCH_BYTES, hip_stream, nullptr);
}

vattn_status vattn_decode_profiled(const vattn_inputs* in, const vattn_cfg* cfg,
                                   vattn_outputs* out, void* workspace, size_t ws_bytes,
                                   void* hip_stream, void* const* events, int32_t n_events) {
    if (!events) return VATTN_E_NULL;
    if (n_events != VATTN_NUM_STAGES + 1) return VATTN_E_SHAPE;
    for (int i = 0; i < n_events; ++i)
        if (!events[i]) return VATTN_E_NULL;
    return decode_impl(in, cfg, out, workspace, ws_bytes, hip_stream, events);
}

vattn_status vattn_project_keys(const void* k_cache, int32_t kv_dtype, const float* proj,
                                uint16_t* k_lowrank, int32_t num_blocks, int32_t Hkv, int32_t d,
                                int32_t r, int32_t proj_heads, void* hip_stream) {
    if (!k_cache || !proj || !k_lowrank) return VATTN_E_NULL;
    if (proj_heads != 0 && proj_heads != 1 && proj_heads != Hkv) return VATTN_E_SHAPE;
    if (kv_dtype != VATTN_F32 && kv_dtype != VATTN_BF16) return VATTN_E_DTYPE;
    if (num_blocks < 1 || Hkv < 1) return VATTN_E_SHAPE;
    if (d != 64 && d != 128) return VATTN_E_UNSUPPORTED;
    if (r != 16 && r != 32 && r != 64) return VATTN_E_UNSUPPORTED;
    if (r > d) return VATTN_E_SHAPE;
    const long long rows = static_cast<long long>(num_blocks) * Hkv * VATTN_PAGE;
    if ((rows + 3) / 4 > 0x7FFFFFFFLL) return VATTN_E_SHAPE;
    const int rc = vattn::launch_project(k_cache, kv_dtype == VATTN_BF16, proj, proj_heads > 1 ? d * r : 0,
                                         k_lowrank, num_blocks, Hkv, d, r, hip_stream);
    return rc == 0 ? VATTN_OK : VATTN_E_HIP;
}

vattn_status vattn_append_kv(const void* k_new, const void* v_new, const int32_t* pos,
                             const int32_t* block_table, int32_t B, int32_t max_blocks, void* k_cache,
                             void* v_cache, uint16_t* k_lowrank, const float* proj, int32_t kv_dtype,
                             int32_t num_blocks, int32_t Hkv, int32_t d, int32_t r, int32_t proj_heads,
                             void* hip_stream) {
    if (!k_new || !v_new || !pos || !block_table || !k_cache || !v_cache) return VATTN_E_NULL;
    if (proj_heads != 0 && proj_heads != 1 && proj_heads != Hkv) return VATTN_E_SHAPE;
    if ((k_lowrank == nullptr) != (proj == nullptr)) return VATTN_E_NULL;
    if (kv_dtype != VATTN_F32 && kv_dtype != VATTN_BF16) return VATTN_E_DTYPE;
    if (B < 1 || max_blocks < 1 || num_blocks < 1 || Hkv < 1) return VATTN_E_SHAPE;
    if (static_cast<long long>(B) * Hkv > 0x7FFFFFFFLL) return VATTN_E_SHAPE;
    if (d != 64 && d != 128) return VATTN_E_UNSUPPORTED;
    if (k_lowrank) {
        if (r != 16 && r != 32 && r != 64) return VATTN_E_UNSUPPORTED;
        if (r > d) return VATTN_E_SHAPE;
    }
    const void* ptrs[] = {k_new, v_new, k_cache, v_cache, k_lowrank, proj};
    for (const void* q : ptrs)
        if (q && (reinterpret_cast<uintptr_t>(q) & 15u)) return VATTN_E_SHAPE;
    const int rc = vattn::launch_append(k_new, v_new, pos, block_table, B, max_blocks, k_cache, v_cache, k_lowrank,
                                        nullptr, proj, (k_lowrank && proj_heads > 1) ? d * r : 0,
                                        kv_dtype == VATTN_BF16, Hkv, d, k_lowrank ? r : 16, hip_stream);
    return rc == 0 ? VATTN_OK : VATTN_E_HIP;
}

vattn_status vattn_sign_keys(const void* k_cache, int32_t kv_dtype, const float* proj, uint32_t* k_sig,
                             int32_t num_blocks, int32_t Hkv, int32_t d, int32_t proj_heads, void* hip_stream) {
    if (!k_cache || !proj || !k_sig) return VATTN_E_NULL;
    if (proj_heads != 0 && proj_heads != 1 && proj_heads != Hkv) return VATTN_E_SHAPE;
    if (kv_dtype != VATTN_F32 && kv_dtype != VATTN_BF16) return VATTN_E_DTYPE;
    if (num_blocks < 1 || Hkv < 1) return VATTN_E_SHAPE;
    if (d != 64 && d != 128) return VATTN_E_UNSUPPORTED;
    if (!aligned(k_sig, 16) || !aligned(proj, 4)) return VATTN_E_SHAPE;
    const long long rows = static_cast<long long>(num_blocks) * Hkv * VATTN_PAGE;
    if ((rows + 7) / 8 > 0x7FFFFFFFLL) return VATTN_E_SHAPE;
    const int rc = vattn::launch_sign(k_cache, kv_dtype == VATTN_BF16, proj, proj_heads > 1 ? d * 32 : 0, k_sig,
                                      num_blocks, Hkv, d, hip_stream);
    return rc == 0 ? VATTN_OK : VATTN_E_HIP;
}

vattn_status vattn_append_kv_sig(const void* k_new, const void* v_new, const int32_t* pos,
                                 const int32_t* block_table, int32_t B, int32_t max_blocks, void* k_cache,
                                 void* v_cache, uint32_t* k_sig, const float* proj, int32_t kv_dtype,
                                 int32_t num_blocks, int32_t Hkv, int32_t d, int32_t proj_heads,
                                 void* hip_stream) {
    if (!k_new || !v_new || !pos || !block_table || !k_cache || !v_cache || !k_sig || !proj) return VATTN_E_NULL;
    if (proj_heads != 0 && proj_heads != 1 && proj_heads != Hkv) return VATTN_E_SHAPE;
    if (kv_dtype != VATTN_F32 && kv_dtype != VATTN_BF16) return VATTN_E_DTYPE;
    if (B < 1 || max_blocks < 1 || num_blocks < 1 || Hkv < 1) return VATTN_E_SHAPE;
    if (static_cast<long long>(B) * Hkv > 0x7FFFFFFFLL) return VATTN_E_SHAPE;
    if (d != 64 && d != 128) return VATTN_E_UNSUPPORTED;
    const void* ptrs[] = {k_new, v_new, k_cache, v_cache, k_sig, proj};
    for (const void* q : ptrs)
        if (reinterpret_cast<uintptr_t>(q) & 15u) return VATTN_E_SHAPE;
    const int rc = vattn::launch_append(k_new, v_new, pos, block_table, B, max_blocks, k_cache, v_cache, nullptr,
                                        k_sig, proj, proj_heads > 1 ? d * 32 : 0, kv_dtype == VATTN_BF16, Hkv, d,
                                        16, hip_stream);
    return rc == 0 ? VATTN_OK : VATTN_E_HIP;
}

size_t vattn_key_gram_workspace_size(int32_t B, int32_t Hkv, int32_t d, int32_t max_seq_len) {
    if (B < 1 || Hkv < 1 || (d != 64 && d != 128) || max_seq_len < 1 || max_seq_len > VATTN_MAX_SEQ) return 0;
    const size_t nchunk = (static_cast<size_t>(max_seq_len) + vattn::kGramChunk - 1) / vattn::kGramChunk;
    return align_up(static_cast<size_t>(B) * Hkv * nchunk * d * d * sizeof(float));
}

vattn_status vattn_key_gram(const void* k_cache, int32_t kv_dtype, const int32_t* block_table,
                            const int32_t* seq_lens, int32_t B, int32_t max_blocks, int32_t num_blocks,
                            int32_t Hkv, int32_t d, int32_t max_seq_len, float* gram, void* workspace,
                            size_t ws_bytes, void* hip_stream) {
    if (!k_cache || !block_table || !seq_lens || !gram) return VATTN_E_NULL;
    if (kv_dtype != VATTN_F32 && kv_dtype != VATTN_BF16) return VATTN_E_DTYPE;
    if (kv_dtype != VATTN_BF16) return VATTN_E_UNSUPPORTED;
    if (d != 64 && d != 128) return VATTN_E_UNSUPPORTED;
    if (B < 1 || Hkv < 1 || num_blocks < 1 || max_blocks < 1) return VATTN_E_SHAPE;
    if (static_cast<long long>(B) * Hkv > 65535) return VATTN_E_SHAPE;
    if (max_seq_len < 1 || max_seq_len > VATTN_MAX_SEQ) return VATTN_E_SHAPE;
    if (static_cast<long long>(max_blocks) * VATTN_PAGE < max_seq_len) return VATTN_E_SHAPE;
    if (!aligned(k_cache, 16) || !aligned(gram, 4)) return VATTN_E_SHAPE;
    const size_t need = vattn_key_gram_workspace_size(B, Hkv, d, max_seq_len);
    if (!workspace || !aligned(workspace, kAlign) || ws_bytes < need) return VATTN_E_WORKSPACE;
    const int rc = vattn::launch_gram(static_cast<const uint16_t*>(k_cache), block_table, seq_lens, B, max_blocks,
                                      Hkv, d, max_seq_len, gram, static_cast<float*>(workspace), hip_stream);
    return rc == 0 ? VATTN_OK : VATTN_E_HIP;
}

static_assert(vattn::kProbeSink == VATTN_READ_PROBE_SINK, "one sink size");

vattn_status vattn_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* hip_stream) {
    if (!buf || !sink) return VATTN_E_NULL;
    if (bytes == 0 || bytes % 16 != 0 || !aligned(buf, 16) || !aligned(sink, 4)) return VATTN_E_SHAPE;
    return vattn::launch_read_probe(buf, bytes / 16, sink, hip_stream) == 0 ? VATTN_OK : VATTN_E_HIP;
}

const char* vattn_status_string(vattn_status s) {
    switch (s) {
        case VATTN_OK: return "VATTN_OK";
        case VATTN_E_NULL: return "VATTN_E_NULL: a required pointer is NULL";
        case VATTN_E_SHAPE: return "VATTN_E_SHAPE: a size or alignment is outside the supported range";
        case VATTN_E_DTYPE: return "VATTN_E_DTYPE: unknown kv dtype";
        case VATTN_E_CFG: return "VATTN_E_CFG: a configuration field is out of range";
        case VATTN_E_WORKSPACE: return "VATTN_E_WORKSPACE: workspace NULL, misaligned or too small";
        case VATTN_E_UNSUPPORTED: return "VATTN_E_UNSUPPORTED: combination not implemented";
        case VATTN_E_HIP: return "VATTN_E_HIP: a HIP launch failed";
    }
    return "unknown vattn_status";
}

}  // extern "C"
