// gfx950 kernels of the verified sparse-attention decode step.
//
// Pipeline for one step (all on the caller's stream):
//   predict  (chunk, b*Hkv)  stream the predictor keys of one context chunk,
//                            score the G query heads of the KV group, keep the
//                            chunk's top-k candidates per head; histogram of the
//                            chunk's sample words
//   select   (b*Hkv)         exact top-k from the candidates, fixed-set bitmap
//                            (sinks, window, top-k), per-head tail histograms,
//                            base-sample threshold in the sample order
//   base     (chunk, b*Hkv)  pinned exact scores of the union of the group's
//                            fixed sets and base samples -> score cache, chunk
//                            maxima, member lists
//   budget   (b*Hkv)         exact fixed-point denominator statistics from the
//                            member lists, CLT budget, final-sample threshold
//   gather   (chunk, b*Hkv)  one pass over the union of the group's index sets:
//                            K row (unless its score is cached) and V row per
//                            token, weighted online softmax for each member head
//   combine  (b*Hq)          merge chunk partials -> out, lse, counts, stats
//   emit     (b*Hq)          optional: the index set in ascending order
//
// The method (edgentiq blog post "vAttention: a new approach to sparse attention
// with guaranteed accuracy", section "How vAttention Works"): sinks + window +
// predicted top-k are kept deterministically, the tail is sampled uniformly
// with a size fixed by a central-limit bound on the denominator estimate, and
// sampled tokens carry the inverse sampling probability as weight.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vattn_device.hpp"
#include "vattn_plan.hpp"

namespace vattn {

constexpr int kUnroll = 4;  // token rows in flight per lane group in the streaming loops
constexpr int kMaxChunks = (VATTN_MAX_SEQ_TOKENS + kGatherChunk - 1) / kGatherChunk;

__device__ __forceinline__ bool bit_of(const uint32_t* row, int i) {
    return (row[i >> 5] >> (i & 31)) & 1u;
}

// Coherent (L2) read of a bitmap word written earlier in the same kernel.
__device__ __forceinline__ bool bit_of_coherent(const uint32_t* row, int i) {
    uint32_t* wp = const_cast<uint32_t*>(row + (i >> 5));
    const uint32_t w = __hip_atomic_load(wp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return (w >> (i & 31)) & 1u;
}

__device__ __forceinline__ size_t row_index(int page, int Hkv, int g, int slot, int width) {
    return ((static_cast<size_t>(page) * Hkv + g) * kPage + slot) * static_cast<size_t>(width);
}

// Cached sample words of group bg (written by the predictor pass for the middle).
__device__ __forceinline__ const uint32_t* group_words(const Plan& P, int bg) {
    return P.uw + static_cast<size_t>(bg) * P.ncg * P.cg;
}

__host__ __device__ __forceinline__ size_t align16(size_t x) { return (x + 15) & ~static_cast<size_t>(15); }

// ===========================================================================
// predict: chunk-local top-k candidates and the chunk's sample-word histogram
// ===========================================================================
size_t predict_lds_bytes(int G, int d, int row, int cp) {
    size_t ts = 0;
    switch (G) {
        case 1: ts = sizeof(TopkShared<1>); break;
        case 2: ts = sizeof(TopkShared<2>); break;
        case 4: ts = sizeof(TopkShared<4>); break;
        default: ts = sizeof(TopkShared<8>); break;
    }
    return align16(ts) + sizeof(uint32_t) * kSampBins + sizeof(int32_t) * (cp / kPage + 2) +
           sizeof(float) * (static_cast<size_t>(G) * d + static_cast<size_t>(G) * row) +
           sizeof(uint32_t) * static_cast<size_t>(G) * cp;
}

template <int ROW, typename T, int G>
__global__ __launch_bounds__(kPredThreads) void k_predict(Plan P) {
    extern __shared__ __align__(16) unsigned char smem[];
    TopkShared<G>& TS = *reinterpret_cast<TopkShared<G>*>(smem);
    size_t off = align16(sizeof(TopkShared<G>));
    uint32_t* shist = reinterpret_cast<uint32_t*>(smem + off);
    off += sizeof(uint32_t) * kSampBins;
    int32_t* pages = reinterpret_cast<int32_t*>(smem + off);  // the chunk's page ids
    off += sizeof(int32_t) * (P.cp / kPage + 2);
    float* qs = reinterpret_cast<float*>(smem + off);  // [G][d]
    float* qv = qs + G * P.d;                           // [G][ROW]
    uint32_t* keys = reinterpret_cast<uint32_t*>(qv + G * ROW);  // [G][cp]

    const int tid = threadIdx.x, nthr = blockDim.x;
    const int lane = tid & 63, wave = tid >> 6, nwaves = nthr >> 6;
    const int bg = blockIdx.y, b = bg / P.Hkv, g = bg % P.Hkv, c = blockIdx.x;
    const int L = P.seq_lens[b];
    const Regions R = regions(P, L);
    const int t0 = max(c * P.cp, R.lo), t1 = min((c + 1) * P.cp, R.hi);
    if (t0 >= t1) return;
    const int d = P.d;

    // sample-word histogram of the chunk's middle tokens (the top-k tokens are
    // taken out per head once they are known)
    const int tb = (t0 / kPage) * kPage;
    const int ntok = ((t1 - 1) / kPage + 1) * kPage - tb;
    const int32_t* btrow = P.bt + static_cast<size_t>(b) * P.max_blocks;
    for (int x = tid; x < kSampBins; x += nthr) shist[x] = 0;
    for (int x = tid; x < ntok / kPage; x += nthr) pages[x] = btrow[tb / kPage + x];
    __syncthreads();
    uint32_t* uwg = P.uw + static_cast<size_t>(bg) * P.ncg * P.cg;
    for (int qd = (t0 >> 2) + tid; 4 * qd < t1; qd += nthr) {
        const uint4 w = philox4x32_10(static_cast<uint32_t>(qd), g, b, 0, P.seed_lo, P.seed_hi);
        *reinterpret_cast<uint4*>(uwg + 4 * qd) = w;  // chunks are disjoint at quad granularity
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 4 * qd + e;
            if (i >= t0 && i < t1) atomicAdd(&shist[word_of(w, e) >> (32 - kSampBits)], 1u);
        }
    }

    if (R.k > 0) {
        // 1) query vectors: q_s = fl32(q * fl32(1/sqrt(d))); low-rank q~ = pdot(q_s, P[:, j])
        for (int x = tid; x < G * d; x += nthr) {
            const int h = x / d, cc = x - h * d;
            qs[x] = P.q[(static_cast<size_t>(b) * P.Hq + g * G + h) * d + cc] * P.scale32;
        }
        __syncthreads();
        if (P.predictor == 1) {
            for (int x = tid; x < G * ROW; x += nthr) {
                const int h = x / ROW, j = x - h * ROW;
                qv[x] = (d == 128) ? pdot_serial<128>(qs + h * d, 1, P.proj + j, ROW)
                                   : pdot_serial<64>(qs + h * d, 1, P.proj + j, ROW);
            }
        } else {
            for (int x = tid; x < G * ROW; x += nthr) qv[x] = qs[x];
        }
        __syncthreads();

        // 2) scores: LPT lanes per token row, 8 elements per lane, kUnroll rows in flight
        constexpr int LPT = ROW / 8, TPW = 64 / LPT;
        const int j = lane % LPT, slot = lane / LPT;
        float qreg[G][8];
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) qreg[h][e] = qv[h * ROW + 8 * j + e];
        const T* src = static_cast<const T*>(P.predictor == 1 ? static_cast<const void*>(P.kt) : P.k);
        const int cbase = c * P.cp;
        uint32_t klo[G], khi[G];  // order-key range of the stored scores
#pragma unroll
        for (int h = 0; h < G; ++h) {
            klo[h] = 0xFFFFFFFFu;
            khi[h] = 0;
        }
        if (tid < G) {
            TS.lo[tid] = 0xFFFFFFFFu;
            TS.hi[tid] = 0;
            TS.aux[tid] = 0;
        }
        for (int base = wave * TPW * kUnroll; base < ntok; base += nwaves * TPW * kUnroll) {
            float kf[kUnroll][8];
            int tt[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                // rows past the chunk's last page reread its last row and are not stored
                const int tl = min(base + u * TPW + slot, ntok - 1);
                tt[u] = tb + tl;
                load8(src + row_index(pages[tl / kPage], P.Hkv, g, tt[u] % kPage, ROW) + 8 * j, kf[u]);
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float s = tree_across_lanes<LPT>(chain8(qreg[h], kf[u]));
                    if (j == LPT - 1 && tt[u] >= t0 && tt[u] < t1) {
                        const uint32_t ok = okey(s);
                        keys[h * P.cp + (tt[u] - cbase)] = ok;
                        klo[h] = min(klo[h], ok);
                        khi[h] = max(khi[h], ok);
                    }
                }
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            uint32_t a = klo[h], bb = khi[h];
            for (int o = 1; o < 64; o <<= 1) {
                a = min(a, static_cast<uint32_t>(__shfl_xor(a, o, 64)));
                bb = max(bb, static_cast<uint32_t>(__shfl_xor(bb, o, 64)));
            }
            if (lane == 0) {
                atomicMin(&TS.lo[h], a);
                atomicMax(&TS.hi[h], bb);
            }
        }
        __syncthreads();

        // 3) chunk top-kp per head, written as candidates (any order)
        const int kp = min(R.k, t1 - t0);
        uint32_t want[G], total[G], lo[G], hi[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            want[h] = static_cast<uint32_t>(kp);
            total[h] = static_cast<uint32_t>(t1 - t0);
            lo[h] = TS.lo[h];
            hi[h] = TS.hi[h];
        }
        const size_t bh0 = static_cast<size_t>(b) * P.Hq + g * G;
        const int cp = P.cp, ncp = P.ncp, kcap = P.kcap;
        uint64_t* __restrict__ cand = P.cand;
        block_topk<G>(TS, want, total, lo, hi, [&](auto&& f) __attribute__((always_inline)) {
            for (int t = t0 + tid; t < t1; t += nthr)
#pragma unroll
                for (int h = 0; h < G; ++h) f(h, keys[h * cp + (t - cbase)], static_cast<uint32_t>(t));
        }, [&](int h, uint64_t key) __attribute__((always_inline)) {
            const uint32_t pos = atomicAdd(&TS.aux[h], 1u);
            if (pos < static_cast<uint32_t>(kp)) cand[((bh0 + h) * ncp + c) * kcap + pos] = key;
        });
        // order-key bracket of the candidates for the merge: [threshold key, chunk max]
        if (tid < G) {
            uint32_t* cr = P.crange + ((bh0 + tid) * P.ncp + c) * 2;
            cr[0] = TS.thr[tid] ? static_cast<uint32_t>(TS.thr[tid] >> 32) : lo[tid];
            cr[1] = hi[tid];
        }
    }
    __syncthreads();
    uint32_t* dst = P.shist + (static_cast<size_t>(bg) * P.ncp + c) * kSampBins;
    for (int x = tid; x < kSampBins; x += nthr) dst[x] = shist[x];
}

// ===========================================================================
// select: exact top-k, fixed-set bitmap, tail histograms, base threshold
// ===========================================================================
__device__ __forceinline__ int chunk_candidates(int cp, const Regions R, int c) {
    const int a = max(c * cp, R.lo), e = min((c + 1) * cp, R.hi);
    return a < e ? min(R.k, e - a) : 0;
}

template <int G>
__global__ __launch_bounds__(kGroupThreads) void k_select(Plan P) {
    __shared__ TopkShared<G> TS;
    __shared__ SampShared<G> SS;
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int bg = blockIdx.x, b = bg / P.Hkv, g = bg % P.Hkv;
    const int L = P.seq_lens[b];
    const Regions R = regions(P, L);
    const size_t bh0 = static_cast<size_t>(b) * P.Hq + g * G;
    const uint32_t* uwg = group_words(P, bg);
    // lambdas below capture these locals, never the kernel argument itself
    const int cp = P.cp, ncp = P.ncp, kcap = P.kcap, words = P.words;
    const uint64_t* __restrict__ cand = P.cand;
    uint32_t* __restrict__ bits = P.bits;
    if (tid == 0 && P.gcounts) {
        P.gcounts[2 * bg] = 0;
        P.gcounts[2 * bg + 1] = 0;
    }

    // 1) bitmap: sinks [0, sp), window [hi, L); tail histogram = middle histogram
    const int wl = (L + 31) >> 5;
    for (int x = tid; x < G * wl; x += nthr) {
        const int h = x / wl, w = x - h * wl;
        uint32_t word = 0;
        const int i0 = 32 * w;
        if (i0 < R.sp) word |= (R.sp - i0 >= 32) ? 0xFFFFFFFFu : ((1u << (R.sp - i0)) - 1u);
        if (i0 + 32 > R.hi) {
            const int a = max(R.hi - i0, 0), e = min(L - i0, 32);  // bits [a, e)
            if (e > a) word |= (e - a >= 32 ? 0xFFFFFFFFu : ((1u << (e - a)) - 1u)) << a;
        }
        P.bits[(bh0 + h) * P.words + w] = word;
    }
    for (int x = tid; x < kSampBins; x += nthr) {
        uint32_t sum = 0;
        for (int c = 0; c < P.ncp; ++c) {
            const int a = max(c * P.cp, R.lo), e = min((c + 1) * P.cp, R.hi);
            if (a < e) sum += P.shist[(static_cast<size_t>(bg) * P.ncp + c) * kSampBins + x];
        }
#pragma unroll
        for (int h = 0; h < G; ++h) SS.hist[h][x] = sum;
    }

    // 2) exact top-k of each head from its chunk candidates: set the bit and
    //    take the token out of the tail histogram (block_topk starts with a barrier)
    if (R.k > 0) {
        uint32_t want[G], total[G], lo[G], hi[G];
        uint32_t tot = 0;
        for (int c = 0; c < P.ncp; ++c) tot += static_cast<uint32_t>(chunk_candidates(cp, R, c));
#pragma unroll
        for (int h = 0; h < G; ++h) {
            want[h] = static_cast<uint32_t>(R.k);
            total[h] = tot;
            lo[h] = 0xFFFFFFFFu;
            hi[h] = 0;
            for (int c = 0; c < P.ncp; ++c) {
                if (chunk_candidates(cp, R, c) == 0) continue;
                const uint32_t* cr = P.crange + ((bh0 + h) * P.ncp + c) * 2;
                lo[h] = min(lo[h], cr[0]);
                hi[h] = max(hi[h], cr[1]);
            }
        }
        const int slots = ncp * kcap;
        constexpr int kBatch = 8;  // candidate keys loaded before any is visited
        block_topk<G>(TS, want, total, lo, hi, [&](auto&& f) __attribute__((always_inline)) {
            for (int x0 = tid; x0 < G * slots; x0 += kBatch * nthr) {
                uint64_t kk[kBatch];
                int hh[kBatch];
#pragma unroll
                for (int t = 0; t < kBatch; ++t) {
                    const int x = x0 + t * nthr;
                    const int h = x / slots, sl = x - h * slots;
                    const int c = sl / kcap, p = sl - c * kcap;
                    const bool ok = x < G * slots && p < chunk_candidates(cp, R, c);
                    hh[t] = ok ? h : -1;
                    kk[t] = ok ? cand[((bh0 + h) * ncp + c) * kcap + p] : 0ull;
                }
#pragma unroll
                for (int t = 0; t < kBatch; ++t)
                    if (hh[t] >= 0) f(hh[t], static_cast<uint32_t>(kk[t] >> 32), ~static_cast<uint32_t>(kk[t]));
            }
        }, [&](int h, uint64_t key) __attribute__((always_inline)) {
            const uint32_t i = ~static_cast<uint32_t>(key);
            atomicOr(&bits[(bh0 + h) * words + (i >> 5)], 1u << (i & 31));
            atomicSub(&SS.hist[h][uwg[i] >> (32 - kSampBits)], 1u);
        });
    } else {
        __syncthreads();
    }
    for (int x = tid; x < G * kSampBins; x += nthr) {
        const int h = x / kSampBins, e = x - h * kSampBins;
        P.hh[(bh0 + h) * kSampBins + e] = SS.hist[h][e];
    }

    // 3) base sample: first nb tail tokens in (word, index) order
    uint32_t rank[G];
#pragma unroll
    for (int h = 0; h < G; ++h) rank[h] = (R.nb > 0 && R.nb < R.NT) ? static_cast<uint32_t>(R.nb) : 0u;
    block_sample_threshold<G>(SS, TS.S, R, uwg, rank, [&](int h, int i) __attribute__((always_inline)) {
        return bit_of_coherent(bits + (bh0 + h) * words, i);
    });

    if (tid < G) {
        HeadState hs{};
        hs.L = L;
        hs.k = R.k;
        hs.n_fixed = R.sp + R.wp + R.k;
        hs.NT = R.NT;
        hs.nb = R.nb;
        hs.thr_b = (R.nb > 0 && R.nb < R.NT) ? SS.thr[tid] : 0;  // nb == N_t: the whole tail
        P.hs[bh0 + tid] = hs;
    }
}

// ===========================================================================
// base: pinned exact scores of the union of fixed sets and base samples
// ===========================================================================
struct HeadView {
    uint64_t thr_b, thr_n;
    int nb, n;
    float wsamp;
};

template <int D, typename KVT, int G>
__global__ __launch_bounds__(kChunkThreads) void k_base(Plan P) {
    __shared__ int tok[kGatherChunk];
    __shared__ uint32_t tmeta[kGatherChunk];
    __shared__ uint32_t trow[kGatherChunk];
    __shared__ uint32_t wsum[kChunkThreads / 64];
    __shared__ float wmax[kChunkThreads / 64][G];
    __shared__ HeadView hv[G];
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int lane = tid & 63, wave = tid >> 6, nwaves = nthr >> 6;
    const int bg = blockIdx.y, b = bg / P.Hkv, g = bg % P.Hkv, c = blockIdx.x;
    const int L = P.seq_lens[b];
    const int T0 = c * P.cg;
    if (T0 >= L) return;
    const Regions R = regions(P, L);
    const size_t bh0 = static_cast<size_t>(b) * P.Hq + g * G;
    if (tid < G) {
        const HeadState& s = P.hs[bh0 + tid];
        hv[tid] = HeadView{s.thr_b, 0, s.nb, 0, 0.f};
    }
    __syncthreads();

    // membership (one Philox call per 4 tokens): meta = base mask | fixed mask << 8
    const int T1 = min(T0 + P.cg, L);
    uint32_t m4[4] = {0, 0, 0, 0};
    uint32_t mine = 0;
    const int qd = (T0 >> 2) + tid;
    const int32_t* btrow = P.bt + static_cast<size_t>(b) * P.max_blocks;
    const uint32_t row0 = 4 * qd < T1 ? (static_cast<uint32_t>(btrow[qd >> 2]) * P.Hkv + g) * kPage : 0u;
    if (4 * qd < T1) {
        uint4 w = make_uint4(0, 0, 0, 0);
        if (4 * qd + 3 >= R.lo && 4 * qd < R.hi) w = *reinterpret_cast<const uint4*>(group_words(P, bg) + 4 * qd);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 4 * qd + e;
            if (i >= T1) continue;
            const bool inM = i >= R.lo && i < R.hi;
            const uint64_t key = sample_key(word_of(w, e), static_cast<uint32_t>(i));
            uint32_t bm = 0, fm = 0;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const bool fx = bit_of(P.bits + (bh0 + h) * P.words, i);
                const bool bs = inM && !fx && hv[h].nb > 0 && key >= hv[h].thr_b;
                bm |= (fx || bs) ? (1u << h) : 0u;
                fm |= fx ? (1u << h) : 0u;
            }
            m4[e] = bm ? (bm | (fm << 8)) : 0u;
            mine += bm ? 1u : 0u;
        }
    }
    uint32_t cnt;
    uint32_t pos = block_excl_scan(mine, wsum, cnt);
    int32_t* ltok = P.btok + (static_cast<size_t>(bg) * P.ncg + c) * P.cg;
    uint32_t* lmeta = P.bmeta + (static_cast<size_t>(bg) * P.ncg + c) * P.cg;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (m4[e]) {
            tok[pos] = 4 * qd + e;
            tmeta[pos] = m4[e];
            trow[pos] = row0 + ((4 * qd + e) & (kPage - 1));
            ltok[pos] = 4 * qd + e;
            lmeta[pos] = m4[e];
            ++pos;
        }
    if (tid == 0) {
        P.bcnt[static_cast<size_t>(bg) * P.ncg + c] = static_cast<int32_t>(cnt);
        if (P.gcounts && cnt) atomicAdd(&P.gcounts[2 * bg + 1], static_cast<int>(cnt));
    }
    __syncthreads();

    // pinned scores for all G heads of each listed token
    constexpr int LPT = D / 8, TPW = 64 / LPT;
    const int j = lane % LPT, slot = lane / LPT;
    float qreg[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) qreg[h][e] = P.q[(bh0 + h) * D + 8 * j + e] * P.scale32;
    float lmax[G];
#pragma unroll
    for (int h = 0; h < G; ++h) lmax[h] = -__builtin_inff();
    const KVT* kbase = static_cast<const KVT*>(P.k);
    float* scrow = P.sc + static_cast<size_t>(bg) * P.max_seq_len * G;
    const int n = static_cast<int>(cnt);
    for (int base = wave * TPW * kUnroll; base < n; base += nwaves * TPW * kUnroll) {
        float kf[kUnroll][8];
        int tk[kUnroll];
        uint32_t mk[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int x = base + u * TPW + slot;
            const bool act = x < n;
            const int xs = act ? x : 0;
            tk[u] = tok[xs];
            mk[u] = act ? tmeta[xs] : 0u;
            load8(kbase + static_cast<size_t>(trow[xs]) * D + 8 * j, kf[u]);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float s[G];
#pragma unroll
            for (int h = 0; h < G; ++h) s[h] = tree_across_lanes<LPT>(chain8(qreg[h], kf[u]));
            if (j == LPT - 1) {  // the lane holding the pinned sums
#pragma unroll
                for (int h = 0; h < G; ++h)
                    if ((mk[u] >> h) & 1u) lmax[h] = fmaxf(lmax[h], s[h]);
                if (mk[u]) {
#pragma unroll
                    for (int h = 0; h < G; ++h) scrow[static_cast<size_t>(tk[u]) * G + h] = s[h];
                }
            }
        }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float v = lmax[h];
        for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
        if (lane == 0) wmax[wave][h] = v;
    }
    __syncthreads();
    if (tid < G) {
        float v = -__builtin_inff();
        for (int w = 0; w < nwaves; ++w) v = fmaxf(v, wmax[w][tid]);
        P.cmax[(bh0 + tid) * P.ncg + c] = v;
    }
}

// ===========================================================================
// budget: exact fixed-point statistics, CLT budget, final-sample threshold
// ===========================================================================
template <int G>
__global__ __launch_bounds__(kGroupThreads) void k_budget(Plan P) {
    __shared__ SampShared<G> SS;
    __shared__ SelShared<G> FS;
    __shared__ float smax[G];
    __shared__ uint64_t red[kGroupThreads / 64][G][4];
    __shared__ int nsel[G], nfin[G];
    __shared__ int coff[kMaxChunks + 1];
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int lane = tid & 63, wave = tid >> 6, nwaves = nthr >> 6;
    const int bg = blockIdx.x, b = bg / P.Hkv, g = bg % P.Hkv;
    const int L = P.seq_lens[b];
    const Regions R = regions(P, L);
    const size_t bh0 = static_cast<size_t>(b) * P.Hq + g * G;
    if (L == 0) {
        if (tid < G) {
            HeadState hs{};
            P.hs[bh0 + tid] = hs;
        }
        return;
    }
    const int nc = (L + P.cg - 1) / P.cg;
    if (tid < G) {
        float m = -__builtin_inff();
        for (int c = 0; c < nc; ++c) m = fmaxf(m, P.cmax[(bh0 + tid) * P.ncg + c]);
        smax[tid] = m;
    }
    for (int x = tid; x < G * kSampBins; x += nthr) {
        const int h = x / kSampBins, e = x - h * kSampBins;
        SS.hist[h][e] = P.hh[(bh0 + h) * kSampBins + e];
    }
    __syncthreads();

    // fixed-point sums over the base pass's member lists: SF over I_f, S1 and
    // S2 over the base sample
    uint64_t sf[G], s1[G];
    unsigned __int128 s2[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        sf[h] = 0;
        s1[h] = 0;
        s2[h] = 0;
    }
    const float* scrow = P.sc + static_cast<size_t>(bg) * P.max_seq_len * G;
    // members of all base chunks as one flat range: a prefix over the chunk
    // counts, then every thread loads its members' tokens and scores before use
    {
        const int32_t* cnts = P.bcnt + static_cast<size_t>(bg) * P.ncg;
        for (int c = tid; c < nc; c += nthr) coff[c] = cnts[c];
        __syncthreads();
        if (wave == 0) {  // exclusive prefix over nc <= kMaxChunks counts, 64 at a time
            uint32_t carry = 0;
            for (int c0 = 0; c0 < nc; c0 += 64) {
                const uint32_t v = c0 + lane < nc ? static_cast<uint32_t>(coff[c0 + lane]) : 0u;
                const uint32_t inc = wave_incl_scan(v);
                if (c0 + lane < nc) coff[c0 + lane] = static_cast<int>(carry + inc - v);
                carry += __shfl(inc, 63, 64);
            }
            if (lane == 0) coff[nc] = static_cast<int>(carry);
        }
        __syncthreads();
        const int total = coff[nc];
        constexpr int kMemBatch = G <= 4 ? 4 : 2;
        for (int y0 = tid; y0 < total; y0 += kMemBatch * nthr) {
            int ti[kMemBatch];
            uint32_t tm[kMemBatch];
#pragma unroll
            for (int v = 0; v < kMemBatch; ++v) {
                const int y = y0 + v * nthr;
                ti[v] = -1;
                tm[v] = 0u;
                if (y < total) {
                    int lo = 0, hi = nc - 1;  // chunk c with coff[c] <= y < coff[c + 1]
                    while (lo < hi) {
                        const int mid = (lo + hi + 1) >> 1;
                        if (coff[mid] <= y) lo = mid; else hi = mid - 1;
                    }
                    const size_t at = (static_cast<size_t>(bg) * P.ncg + lo) * P.cg + (y - coff[lo]);
                    ti[v] = P.btok[at];
                    tm[v] = P.bmeta[at];
                }
            }
            float sv[kMemBatch][G];
#pragma unroll
            for (int v = 0; v < kMemBatch; ++v)
#pragma unroll
                for (int h = 0; h < G; ++h)
                    sv[v][h] = ((tm[v] >> h) & 1u) ? scrow[static_cast<size_t>(ti[v]) * G + h] : 0.0f;
#pragma unroll
            for (int v = 0; v < kMemBatch; ++v)
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const uint64_t E = ((tm[v] >> h) & 1u) ? fixed_weight(sv[v][h] - smax[h]) : 0ull;
                    if ((tm[v] >> (8 + h)) & 1u) {
                        sf[h] += E;
                    } else {
                        s1[h] += E;
                        s2[h] += static_cast<unsigned __int128>(E) * E;
                    }
                }
        }
    }
    // exact reduction (integer sums are order independent)
#pragma unroll
    for (int h = 0; h < G; ++h) {
        uint64_t a = sf[h], b1 = s1[h];
        uint64_t lo = static_cast<uint64_t>(s2[h]), hi = static_cast<uint64_t>(s2[h] >> 64);
        for (int o = 32; o >= 1; o >>= 1) {
            a += shfl_xor_u64(a, o);
            b1 += shfl_xor_u64(b1, o);
            const uint64_t olo = shfl_xor_u64(lo, o), ohi = shfl_xor_u64(hi, o);
            const uint64_t nlo = lo + olo;
            hi = hi + ohi + (nlo < lo ? 1u : 0u);
            lo = nlo;
        }
        if (lane == 0) {
            red[wave][h][0] = a;
            red[wave][h][1] = b1;
            red[wave][h][2] = hi;
            red[wave][h][3] = lo;
        }
    }
    __syncthreads();
    if (tid < G) {
        const int h = tid;
        uint64_t SF = 0, S1 = 0;
        unsigned __int128 S2 = 0;
        for (int w = 0; w < nwaves; ++w) {
            SF += red[w][h][0];
            S1 += red[w][h][1];
            S2 += (static_cast<unsigned __int128>(red[w][h][2]) << 64) | red[w][h][3];
        }
        const int NT = R.NT, nb = R.nb;
        int n, flags = 0;
        if (P.force_budget >= 0) {
            n = min(NT, P.force_budget);
            flags |= 2;
        } else if (nb == NT) {
            n = NT;
        } else {
            // n = (z sigma N_t / (eps D))^2 over exact integers:
            //   sigma^2 = M2 / (nb (nb - 1)),  D = Y / nb,
            //   M2 = nb S2 - S1^2,  Y = nb SF + N_t S1
            const unsigned __int128 M2 = static_cast<unsigned __int128>(nb) * S2 -
                                         static_cast<unsigned __int128>(S1) * S1;
            const unsigned __int128 Y = static_cast<unsigned __int128>(nb) * SF +
                                        static_cast<unsigned __int128>(NT) * S1;
            const double z = P.z32;
            const double num = (z * z * static_cast<double>(NT) * static_cast<double>(NT)) *
                               (u128_to_f64(M2) * static_cast<double>(nb));
            const double den = (static_cast<double>(nb - 1) * (P.eps * P.eps)) *
                               (u128_to_f64(Y) * u128_to_f64(Y));
            const double nreal = num / den;
            if (nreal >= static_cast<double>(NT)) {
                n = NT;
            } else {
                n = static_cast<int>(__builtin_ceil(nreal));
                if (n < nb) {
                    n = nb;
                    flags |= 4;
                }
            }
        }
        if (n == NT) flags |= 1;
        HeadState& hs = P.hs[bh0 + h];
        hs.n = n;
        hs.flags = flags;
        hs.m = smax[h];
        hs.wsamp = n > 0 ? static_cast<float>(static_cast<double>(NT) / static_cast<double>(n)) : 0.0f;
        hs.SF = SF;
        hs.S1 = S1;
        hs.S2hi = static_cast<uint64_t>(S2 >> 64);
        hs.S2lo = static_cast<uint64_t>(S2);
        // a new threshold unless the sample is empty, the whole tail or the base sample
        nsel[h] = (n > 0 && n < NT && n != nb) ? n : 0;
        nfin[h] = n;
    }
    __syncthreads();

    uint32_t rank[G];
#pragma unroll
    for (int h = 0; h < G; ++h) rank[h] = static_cast<uint32_t>(nsel[h]);
    const uint32_t* __restrict__ bits = P.bits;
    const int words = P.words;
    block_sample_threshold<G>(SS, FS, R, group_words(P, bg), rank, [&](int h, int i) __attribute__((always_inline)) {
        return bit_of(bits + (bh0 + h) * words, i);
    });
    if (tid < G) {
        const int h = tid, n = nfin[h];
        HeadState& hs = P.hs[bh0 + h];
        uint64_t thr = 0;  // n == N_t: the whole tail (n == 0: unused)
        if (nsel[h] > 0) thr = SS.thr[h];
        else if (n > 0 && n == R.nb) thr = hs.thr_b;
        hs.thr_n = thr;
    }
}

// ===========================================================================
// gather: weighted softmax over the union of the group's index sets, in two
// passes over the listed tokens: (1) scores (score cache or K row) into LDS,
// then per head the block max and the weights p = w exp(s - max); (2) a pure
// stream of V rows accumulating sum_i p_i V_i.  Every weight is computed once.
// ===========================================================================
constexpr int kGatherUnrollV = 4;  // V rows per batch and lane group (two batches in flight)

template <int D, typename KVT, int G>
__global__ __launch_bounds__(kChunkThreads) void k_gather(Plan P) {
    constexpr int NW = kChunkThreads / 64;
    __shared__ int tok[kGatherChunk];
    __shared__ uint32_t tmeta[kGatherChunk];
    __shared__ uint32_t trow[kGatherChunk];
    __shared__ float sp[G][kGatherChunk];  // scores, then weights
    __shared__ uint32_t wsum[NW];
    __shared__ HeadView hv[G];
    __shared__ float wred[NW][G];
    __shared__ float hmax[G], hsum[G];
    __shared__ float wacc[NW][G][D];
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int lane = tid & 63, wave = tid >> 6, nwaves = nthr >> 6;
    const int bg = blockIdx.y, b = bg / P.Hkv, g = bg % P.Hkv, c = blockIdx.x;
    const int L = P.seq_lens[b];
    const int T0 = c * P.cg;
    if (T0 >= L) return;
    const Regions R = regions(P, L);
    const size_t bh0 = static_cast<size_t>(b) * P.Hq + g * G;
    if (tid < G) {
        const HeadState& s = P.hs[bh0 + tid];
        hv[tid] = HeadView{s.thr_b, s.thr_n, s.nb, s.n, s.wsamp};
    }
    __syncthreads();

    // membership: meta = final mask | fixed mask << 8 | score cached << 16
    const int T1 = min(T0 + P.cg, L);
    uint32_t m4[4] = {0, 0, 0, 0};
    uint32_t mine = 0;
    const int qd = (T0 >> 2) + tid;
    const int32_t* btrow = P.bt + static_cast<size_t>(b) * P.max_blocks;
    const uint32_t row0 = 4 * qd < T1 ? (static_cast<uint32_t>(btrow[qd >> 2]) * P.Hkv + g) * kPage : 0u;
    if (4 * qd < T1) {
        uint4 w = make_uint4(0, 0, 0, 0);
        if (4 * qd + 3 >= R.lo && 4 * qd < R.hi) w = *reinterpret_cast<const uint4*>(group_words(P, bg) + 4 * qd);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 4 * qd + e;
            if (i >= T1) continue;
            const bool inM = i >= R.lo && i < R.hi;
            const uint64_t key = sample_key(word_of(w, e), static_cast<uint32_t>(i));
            uint32_t fin = 0, fxm = 0, cached = 0;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const bool fx = bit_of(P.bits + (bh0 + h) * P.words, i);
                const bool tail = inM && !fx;
                const bool sn = tail && hv[h].n > 0 && key >= hv[h].thr_n;
                const bool sb = tail && hv[h].nb > 0 && key >= hv[h].thr_b;
                fin |= (fx || sn) ? (1u << h) : 0u;
                fxm |= fx ? (1u << h) : 0u;
                cached |= (fx || sb) ? 1u : 0u;
            }
            m4[e] = fin ? (fin | (fxm << 8) | (cached << 16)) : 0u;
            mine += fin ? 1u : 0u;
        }
    }
    uint32_t cnt;
    uint32_t pos = block_excl_scan(mine, wsum, cnt);
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (m4[e]) {
            tok[pos] = 4 * qd + e;
            tmeta[pos] = m4[e];
            trow[pos] = row0 + ((4 * qd + e) & (kPage - 1));
            ++pos;
        }
    if (tid == 0 && P.gcounts && cnt) atomicAdd(&P.gcounts[2 * bg], static_cast<int>(cnt));
    __syncthreads();
    const int n = static_cast<int>(cnt);

    // (1) scores into LDS (-inf for heads the token does not belong to).
    // Tokens of the base pass take their cached pinned scores (independent
    // loads, one pass); the others are scored from their K rows below.
    constexpr int LPT = D / 8, TPW = 64 / LPT;
    const int j = lane % LPT, slot = lane / LPT;
    const float* scrow = P.sc + static_cast<size_t>(bg) * P.max_seq_len * G;
    const KVT* kbase = static_cast<const KVT*>(P.k);
    for (int x = tid; x < n; x += nthr) {
        const uint32_t m = tmeta[x];
        if ((m >> 16) & 1u) {
            float v[G];
#pragma unroll
            for (int h = 0; h < G; ++h) v[h] = scrow[static_cast<size_t>(tok[x]) * G + h];
#pragma unroll
            for (int h = 0; h < G; ++h) sp[h][x] = ((m >> h) & 1u) ? v[h] : -__builtin_inff();
        }
    }
    if constexpr (sizeof(KVT) == 2) {
        // bf16 keys: 16-token tiles on the matrix cores.  A = K rows (16 x D),
        // B = the scaled query split into three bf16 terms q_hi + q_lo + q_lo2
        // (residual ~2^-25 |q|), three columns per head, four heads per column
        // block; bf16 x bf16 products are exact and accumulate in fp32.
        constexpr int KB = D / 32, NCB = (G + 3) / 4;
        const int col = lane & 15, kq = lane >> 4;
        bf16x8 qb[NCB][KB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int hh = cb * 4 + col / 3, term = col % 3;
            const bool live = col < 12 && hh < G;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float part = 0.0f;
                    if (live) {
                        const float qsv = P.q[(bh0 + hh) * D + 32 * kb + 8 * kq + e] * P.scale32;
                        const float hi = bf16_round(qsv);
                        const float lo = bf16_round(qsv - hi);
                        part = term == 0 ? hi : term == 1 ? lo : bf16_round((qsv - hi) - lo);
                    }
                    qb[cb][kb][e] = static_cast<__bf16>(part);
                }
        }
        const int ntile = (n + 15) / 16;
        auto tile_row = [&](int x0) __attribute__((always_inline)) {
            // row of this lane's token; cached or absent tokens read a row that
            // is already needed (their result is not used)
            const int x = x0 + col;
            const int xr = x < n ? x : x0;
            const uint32_t m = tmeta[xr];
            return ((m >> 16) & 1u) ? trow[x0] : trow[xr];
        };
        struct KTile {
            uint4 a[KB];
        };
        auto issue = [&](KTile& t, int x0) __attribute__((always_inline)) {
            const KVT* rp = kbase + static_cast<size_t>(tile_row(x0)) * D + 8 * kq;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) t.a[kb] = *reinterpret_cast<const uint4*>(rp + 32 * kb);
        };
        auto score = [&](const KTile& t, int x0) __attribute__((always_inline)) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, t.a[kb]), qb[cb][kb],
                                                                 acc, 0, 0, 0);
                const int hh = cb * 4 + col / 3;
                const bool writer = col < 12 && col % 3 == 0 && hh < G;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float sv = acc[r] + dpp<0x101>(acc[r]) + dpp<0x102>(acc[r]);  // row_shl:1, :2
                    const int x = x0 + 4 * kq + r;
                    if (writer && x < n) {
                        const uint32_t m = tmeta[x];
                        if (!((m >> 16) & 1u)) sp[hh][x] = ((m >> hh) & 1u) ? sv : -__builtin_inff();
                    }
                }
            }
        };
        int tI = wave;
        KTile A, B;
        if (tI < ntile) issue(A, 16 * tI);
        while (tI < ntile) {
            if (tI + nwaves < ntile) issue(B, 16 * (tI + nwaves));
            score(A, 16 * tI);
            tI += nwaves;
            if (tI >= ntile) break;
            if (tI + nwaves < ntile) issue(A, 16 * (tI + nwaves));
            score(B, 16 * tI);
            tI += nwaves;
        }
    } else {
        float qreg[G][8];
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) qreg[h][e] = P.q[(bh0 + h) * D + 8 * j + e] * P.scale32;
        for (int base = wave * TPW * kUnroll; base < n; base += nwaves * TPW * kUnroll) {
            Raw8 kr[kUnroll];
            uint32_t mk[kUnroll];
            int xs[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int x = base + u * TPW + slot;
                xs[u] = x < n ? x : -1;
                mk[u] = x < n ? tmeta[x] : 0u;
                load_raw(kbase + static_cast<size_t>(trow[x < n ? x : 0]) * D + 8 * j, kr[u]);
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const bool cached = (mk[u] >> 16) & 1u;
                float kf[8];
                widen<KVT>(kr[u], kf);
                float sv[G];
#pragma unroll
                for (int h = 0; h < G; ++h) sv[h] = tree_across_lanes<LPT>(chain8(qreg[h], kf));
                if (j == LPT - 1 && xs[u] >= 0 && !cached) {
                    const int x = xs[u];
#pragma unroll
                    for (int h = 0; h < G; ++h) sp[h][x] = ((mk[u] >> h) & 1u) ? sv[h] : -__builtin_inff();
                }
            }
        }
    }
    __syncthreads();
    // per-head block max, then weights and their sum
    {
        float mx[G];
#pragma unroll
        for (int h = 0; h < G; ++h) mx[h] = -__builtin_inff();
        for (int x = tid; x < n; x += nthr)
#pragma unroll
            for (int h = 0; h < G; ++h) mx[h] = fmaxf(mx[h], sp[h][x]);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float v = mx[h];
            for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
            if (lane == 0) wred[wave][h] = v;
        }
        __syncthreads();
        if (tid < G) {
            float v = -__builtin_inff();
            for (int w = 0; w < NW; ++w) v = fmaxf(v, wred[w][tid]);
            hmax[tid] = v;
        }
        __syncthreads();
        float hm[G], ls[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            hm[h] = hmax[h];
            ls[h] = 0.f;
        }
        for (int x = tid; x < n; x += nthr) {
            const uint32_t meta = tmeta[x];
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float sv = sp[h][x];
                const float w = ((meta >> (8 + h)) & 1u) ? 1.0f : hv[h].wsamp;
                const float p = (sv == -__builtin_inff()) ? 0.0f : w * __expf(sv - hm[h]);
                sp[h][x] = p;
                ls[h] += p;
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float v = ls[h];
            for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
            if (lane == 0) wred[wave][h] = v;
        }
        __syncthreads();
        if (tid < G) {
            float v = 0.f;
            for (int w = 0; w < NW; ++w) v += wred[w][tid];
            hsum[tid] = v;
        }
    }
    __syncthreads();

    // (2) sum_i p_i V_i, V rows streamed kGatherUnrollV deep and double-buffered
    float acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    {
        const KVT* vbase = static_cast<const KVT*>(P.v);
        struct VBatch {
            Raw8 vr[kGatherUnrollV];
            int x0;
        };
        // rows past the list end reread the last row with weight 0 (no branches)
        auto issue = [&](VBatch& bt, int b0) __attribute__((always_inline)) {
            bt.x0 = b0;
#pragma unroll
            for (int u = 0; u < kGatherUnrollV; ++u) {
                const int x = min(b0 + u * TPW + slot, n - 1);
                load_raw(vbase + static_cast<size_t>(trow[x]) * D + 8 * j, bt.vr[u]);
            }
        };
        auto accumulate = [&](const VBatch& bt) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < kGatherUnrollV; ++u) {
                const int x = bt.x0 + u * TPW + slot;
                const int xc = min(x, n - 1);
                float vf[8];
                widen<KVT>(bt.vr[u], vf);
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float pw = x < n ? sp[h][xc] : 0.0f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[h][e] = __builtin_fmaf(pw, vf[e], acc[h][e]);
                }
            }
        };
        const int stride = nwaves * TPW * kGatherUnrollV;
        int base = wave * TPW * kGatherUnrollV;
        VBatch A, B;
        if (base < n) issue(A, base);
        while (base < n) {
            if (base + stride < n) issue(B, base + stride);
            accumulate(A);
            base += stride;
            if (base >= n) break;
            if (base + stride < n) issue(A, base + stride);
            accumulate(B);
            base += stride;
        }
    }
    // token slots of the wave hold the same dims: plain sums
#pragma unroll
    for (int o = LPT; o < 64; o <<= 1)
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] += __shfl_xor(acc[h][e], o, 64);
    if (slot == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) wacc[wave][h][8 * j + e] = acc[h][e];
    }
    __syncthreads();
    for (int x = tid; x < G * (D + 2); x += nthr) {
        const int h = x / (D + 2), e = x - h * (D + 2);
        float v;
        if (e == 0) {
            v = hmax[h];
        } else if (e == 1) {
            v = hsum[h];
        } else {
            v = 0.f;
            for (int w = 0; w < NW; ++w) v += wacc[w][h][e - 2];
        }
        P.part[((bh0 + h) * P.ncg + c) * (D + 2) + e] = v;
    }
}

// ===========================================================================
// combine: merge chunk partials; counts and statistics
// ===========================================================================
constexpr int kCombineThreads = 128;

__global__ __launch_bounds__(kCombineThreads) void k_combine(Plan P) {
    __shared__ float wsh[kMaxChunks];
    __shared__ float rm[kCombineThreads / 64], rl[kCombineThreads / 64];
    const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63, wave = tid >> 6;
    const int bh = blockIdx.x, b = bh / P.Hq;
    const int L = P.seq_lens[b];
    const int D = P.d;
    const int nc = (L + P.cg - 1) / P.cg;
    const float* pp = P.part + static_cast<size_t>(bh) * P.ncg * (D + 2);
    float mloc = -__builtin_inff();
    for (int c = tid; c < nc; c += nthr) mloc = fmaxf(mloc, pp[static_cast<size_t>(c) * (D + 2)]);
    for (int o = 1; o < 64; o <<= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, o, 64));
    if (lane == 0) rm[wave] = mloc;
    __syncthreads();
    float M = -__builtin_inff();
    for (int w = 0; w < nthr / 64; ++w) M = fmaxf(M, rm[w]);
    float lloc = 0.f;
    for (int c = tid; c < nc; c += nthr) {
        const float* q = pp + static_cast<size_t>(c) * (D + 2);
        const float wgt = (M == -__builtin_inff()) ? 0.0f : __expf(q[0] - M);
        wsh[c] = wgt;
        lloc += wgt * q[1];
    }
    for (int o = 1; o < 64; o <<= 1) lloc += __shfl_xor(lloc, o, 64);
    if (lane == 0) rl[wave] = lloc;
    __syncthreads();
    float l = 0.f;
    for (int w = 0; w < nthr / 64; ++w) l += rl[w];
    const bool ok = M != -__builtin_inff() && l > 0.f;
    for (int e = tid; e < D; e += nthr) {
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
        int c = 0;
        for (; c + 4 <= nc; c += 4) {
            a0 += wsh[c] * pp[static_cast<size_t>(c) * (D + 2) + 2 + e];
            a1 += wsh[c + 1] * pp[static_cast<size_t>(c + 1) * (D + 2) + 2 + e];
            a2 += wsh[c + 2] * pp[static_cast<size_t>(c + 2) * (D + 2) + 2 + e];
            a3 += wsh[c + 3] * pp[static_cast<size_t>(c + 3) * (D + 2) + 2 + e];
        }
        for (; c < nc; ++c) a0 += wsh[c] * pp[static_cast<size_t>(c) * (D + 2) + 2 + e];
        const float a = (a0 + a1) + (a2 + a3);
        P.out[static_cast<size_t>(bh) * D + e] = ok ? a / l : 0.0f;
    }
    if (tid == 0) {
        P.lse[bh] = ok ? M + __logf(l) : -__builtin_inff();
        const HeadState& hs = P.hs[bh];
        if (P.counts) {
            int32_t* ct = P.counts + static_cast<size_t>(bh) * 6;
            if (L == 0) {
                for (int x = 0; x < 6; ++x) ct[x] = 0;
            } else {
                ct[0] = hs.n_fixed;
                ct[1] = hs.NT;
                ct[2] = hs.nb;
                ct[3] = hs.n;
                ct[4] = hs.n_fixed + hs.n;
                ct[5] = hs.flags;
            }
        }
        if (P.stats) {
            uint64_t* st = P.stats + static_cast<size_t>(bh) * 4;
            st[0] = L ? hs.SF : 0;
            st[1] = L ? hs.S1 : 0;
            st[2] = L ? hs.S2hi : 0;
            st[3] = L ? hs.S2lo : 0;
        }
    }
}

// ===========================================================================
// emit: the index set of one head, ascending, -1 padded
// ===========================================================================
__global__ __launch_bounds__(kEmitThreads) void k_emit(Plan P) {
    __shared__ uint32_t wsum[kEmitThreads / 64];
    const int bh = blockIdx.x, b = bh / P.Hq, h = bh % P.Hq;
    const int G = P.G, g = h / G;
    const int L = P.seq_lens[b];
    const Regions R = regions(P, L);
    const HeadState hs = P.hs[bh];
    const uint32_t* bits = P.bits + static_cast<size_t>(bh) * P.words;
    int32_t* out = P.idx + static_cast<size_t>(bh) * P.idx_cap;
    int written = 0;
    for (int T0 = 0; T0 < L; T0 += 4 * blockDim.x) {
        const int qd = (T0 >> 2) + threadIdx.x;
        bool mem[4] = {false, false, false, false};
        uint32_t mine = 0;
        if (4 * qd < L) {
            uint4 w = make_uint4(0, 0, 0, 0);
            if (4 * qd + 3 >= R.lo && 4 * qd < R.hi)
                w = *reinterpret_cast<const uint4*>(group_words(P, b * P.Hkv + g) + 4 * qd);
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * qd + e;
                if (i >= L) continue;
                const bool fx = bit_of(bits, i);
                const bool inM = i >= R.lo && i < R.hi;
                const bool sn = inM && !fx && hs.n > 0 &&
                                sample_key(word_of(w, e), static_cast<uint32_t>(i)) >= hs.thr_n;
                mem[e] = fx || sn;
                mine += mem[e] ? 1u : 0u;
            }
        }
        uint32_t tot;
        uint32_t pos = block_excl_scan(mine, wsum, tot) + written;
        for (int e = 0; e < 4; ++e)
            if (mem[e]) {
                if (pos < static_cast<uint32_t>(P.idx_cap)) out[pos] = 4 * qd + e;
                ++pos;
            }
        written += static_cast<int>(tot);
    }
    written = min(written, P.idx_cap);
    for (int x = written + threadIdx.x; x < P.idx_cap; x += blockDim.x) out[x] = -1;
}

// ===========================================================================
// low-rank key projection: Kt = bf16(pdot(K_i, P[:, j]))
// ===========================================================================
template <typename KVT, int D, int RK>
__global__ __launch_bounds__(256) void k_project(const KVT* __restrict__ k, const float* __restrict__ proj,
                                                 uint16_t* __restrict__ kt, long long nrows) {
    constexpr int RPB = 256 / RK;  // rows per block
    __shared__ float ps[D * RK];
    __shared__ float kr[RPB][D];
    for (int x = threadIdx.x; x < D * RK; x += 256) ps[x] = proj[x];
    const long long r0 = static_cast<long long>(blockIdx.x) * RPB;
    for (int x = threadIdx.x; x < RPB * D; x += 256) {
        const int rr = x / D, e = x - rr * D;
        const long long row = r0 + rr;
        float v = 0.f;
        if (row < nrows) {
            if constexpr (sizeof(KVT) == 2) {
                v = __uint_as_float(static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(k)[row * D + e]) << 16);
            } else {
                v = reinterpret_cast<const float*>(k)[row * D + e];
            }
        }
        kr[rr][e] = v;
    }
    __syncthreads();
    const int rr = threadIdx.x / RK, jj = threadIdx.x % RK;
    const long long row = r0 + rr;
    if (row >= nrows) return;
    const float s = pdot_serial<D>(kr[rr], 1, ps + jj, RK);
    uint32_t u = __float_as_uint(s);
    u += 0x7FFFu + ((u >> 16) & 1u);  // round to nearest even
    kt[row * RK + jj] = static_cast<uint16_t>(u >> 16);
}

// ===========================================================================
// host-side dispatch
// ===========================================================================
// Records events[k] (when profiling) after the k-th stage.
struct Marks {
    void* const* ev;
    hipStream_t st;
    int mark(int k) const {
        return ev ? static_cast<int>(hipEventRecord(static_cast<hipEvent_t>(ev[k]), st)) : 0;
    }
};

template <int D, typename KVT, int G>
static int launch_chunk_kernels(const Plan& p, hipStream_t st, const Marks& mk) {
    const dim3 grid_c(p.ncg, p.B * p.Hkv);
    int rc = 0;
    hipLaunchKernelGGL((k_base<D, KVT, G>), grid_c, dim3(kChunkThreads), 0, st, p);
    if ((rc = mk.mark(3))) return rc;
    hipLaunchKernelGGL((k_budget<G>), dim3(p.B * p.Hkv), dim3(kGroupThreads), 0, st, p);
    if ((rc = mk.mark(4))) return rc;
    hipLaunchKernelGGL((k_gather<D, KVT, G>), grid_c, dim3(kChunkThreads), 0, st, p);
    return mk.mark(5);
}

template <int ROW, typename T, int G>
static int launch_predict(const Plan& p, hipStream_t st) {
    const size_t lds = predict_lds_bytes(G, p.d, ROW, p.cp);
    auto kern = k_predict<ROW, T, G>;
    static bool attr_set = false;  // per kernel instance; the limit never changes
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
        if (e != hipSuccess) return static_cast<int>(e);
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3(p.ncp, p.B * p.Hkv), dim3(kPredThreads), lds, st, p);
    return 0;
}

template <int G>
static int launch_g(const Plan& p, hipStream_t st, const Marks& mk) {
    int rc = 0;
    if ((rc = mk.mark(0))) return rc;
    // 1. predictor + chunk candidates
    if (p.predictor == 1) {
        switch (p.r) {
            case 16: rc = launch_predict<16, uint16_t, G>(p, st); break;
            case 32: rc = launch_predict<32, uint16_t, G>(p, st); break;
            default: rc = launch_predict<64, uint16_t, G>(p, st); break;
        }
    } else {
        if (p.d == 128) rc = p.kv_bf16 ? launch_predict<128, uint16_t, G>(p, st) : launch_predict<128, float, G>(p, st);
        else rc = p.kv_bf16 ? launch_predict<64, uint16_t, G>(p, st) : launch_predict<64, float, G>(p, st);
    }
    if (rc) return rc;
    if ((rc = mk.mark(1))) return rc;
    // 2. exact top-k, bitmap, base threshold
    hipLaunchKernelGGL((k_select<G>), dim3(p.B * p.Hkv), dim3(kGroupThreads), 0, st, p);
    if ((rc = mk.mark(2))) return rc;
    // 3-5. base scores, budget, gather
    if (p.d == 128)
        rc = p.kv_bf16 ? launch_chunk_kernels<128, uint16_t, G>(p, st, mk)
                       : launch_chunk_kernels<128, float, G>(p, st, mk);
    else
        rc = p.kv_bf16 ? launch_chunk_kernels<64, uint16_t, G>(p, st, mk)
                       : launch_chunk_kernels<64, float, G>(p, st, mk);
    return rc;
}

int launch_decode(const Plan& p, void* stream, void* const* events) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const Marks mk{events, st};
    int rc = 0;
    switch (p.G) {
        case 1: rc = launch_g<1>(p, st, mk); break;
        case 2: rc = launch_g<2>(p, st, mk); break;
        case 4: rc = launch_g<4>(p, st, mk); break;
        default: rc = launch_g<8>(p, st, mk); break;
    }
    if (rc) return rc;
    hipLaunchKernelGGL(k_combine, dim3(p.B * p.Hq), dim3(kCombineThreads), 0, st, p);
    if ((rc = mk.mark(6))) return rc;
    if (p.idx) hipLaunchKernelGGL(k_emit, dim3(p.B * p.Hq), dim3(kEmitThreads), 0, st, p);
    if ((rc = mk.mark(7))) return rc;
    return static_cast<int>(hipGetLastError());
}

template <typename KVT, int D>
static void launch_project_t(const void* k, const float* proj, uint16_t* kt, long long nrows, int r,
                             hipStream_t st) {
    switch (r) {
        case 16: {
            const long long nb = (nrows + 15) / 16;
            hipLaunchKernelGGL((k_project<KVT, D, 16>), dim3(static_cast<unsigned>(nb)), dim3(256), 0, st,
                               static_cast<const KVT*>(k), proj, kt, nrows);
            break;
        }
        case 32: {
            const long long nb = (nrows + 7) / 8;
            hipLaunchKernelGGL((k_project<KVT, D, 32>), dim3(static_cast<unsigned>(nb)), dim3(256), 0, st,
                               static_cast<const KVT*>(k), proj, kt, nrows);
            break;
        }
        default: {
            const long long nb = (nrows + 3) / 4;
            hipLaunchKernelGGL((k_project<KVT, D, 64>), dim3(static_cast<unsigned>(nb)), dim3(256), 0, st,
                               static_cast<const KVT*>(k), proj, kt, nrows);
            break;
        }
    }
}

int launch_project(const void* k_cache, int kv_bf16, const float* proj, uint16_t* kt, int num_blocks,
                   int Hkv, int d, int r, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const long long nrows = static_cast<long long>(num_blocks) * Hkv * kPage;
    if (d == 128) {
        if (kv_bf16) launch_project_t<uint16_t, 128>(k_cache, proj, kt, nrows, r, st);
        else launch_project_t<float, 128>(k_cache, proj, kt, nrows, r, st);
    } else {
        if (kv_bf16) launch_project_t<uint16_t, 64>(k_cache, proj, kt, nrows, r, st);
        else launch_project_t<float, 64>(k_cache, proj, kt, nrows, r, st);
    }
    return static_cast<int>(hipGetLastError());
}

}  // namespace vattn
