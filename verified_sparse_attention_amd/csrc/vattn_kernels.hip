// gfx950 kernels of the verified sparse-attention decode step.
//
// Pipeline for one step (all on the caller's stream):
//   predict  (chunk, b*Hkv)  stream the predictor keys of one context chunk,
//                            score the G query heads of the KV group, keep the
//                            chunk's top-k candidates per head; the chunk's
//                            sample words, grouped by their top bits
//   premerge (b*Hq, part)    only with few heads and many chunks: each part's
//                            chunk candidates reduced to its exact top-k
//   select   (b*Hq)          exact top-k from the candidates, fixed-set bitmap
//                            (sinks, window, top-k), tail histogram,
//                            base-sample threshold in the sample order
//   base     (b*Hkv, chunk)  pinned exact scores of the union of the group's
//                            fixed sets and base samples -> score cache, chunk
//                            maxima, member lists
//   budget   (b*Hq)          exact fixed-point denominator statistics of the
//                            head's fixed set and base sample, CLT budget,
//                            final-sample threshold, the group's dispatch weight
//                            (output-level mode: statistics, then numstat
//                            (b*Hkv, chunk) numerator partials, then
//                            budget_num (b*Hq) the larger budget and threshold)
//   gather   (chunk, b*Hkv)  over the union of the group's index sets, groups
//                            densest first: K row (unless its score is cached)
//                            and V row per token, weighted softmax partials
//                            per chunk
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

#include <atomic>
#include <type_traits>

#include "vattn_device.hpp"
#include "vattn_plan.hpp"

namespace vattn {

constexpr int kUnroll = 4;      // token rows in flight per lane group in the predictor stream
constexpr int kBaseUnroll = 8;  // K rows in flight per lane group in the base pass (fp32 K)
constexpr int kBaseUnrollBf16 = 12;  // the same for bf16 K (a lane's slice of a bf16 row takes half the registers)
constexpr int kKeyPad = 16;     // words between the predictor's per-head key rows
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
    return align16(ts) + sizeof(uint32_t) * (kSampBins + kPredThreads / 64) + align16(sizeof(int32_t) * (cp / kPage + 2)) +
           sizeof(float) * (static_cast<size_t>(G) * d + static_cast<size_t>(G) * row) +
           sizeof(uint32_t) * static_cast<size_t>(G) * (cp + kKeyPad);
}

// q~[h][j] = pdot(q_s[h], P[:, j]) in two steps: every chain of 8 (one per
// thread, consecutive threads on consecutive j so the projection loads
// coalesce) into `part`, then one thread per output adds the D / 8 chain sums
// in the pairwise tree order.  Ends with a barrier.
template <int D, int ROW, int G>
__device__ __forceinline__ void low_rank_query(const float* qs, const float* __restrict__ proj, float* qv,
                                               float* part, int tid, int nthr) {
    constexpr int NB = D / 8;
    for (int x = tid; x < G * NB * ROW; x += nthr) {
        const int j = x % ROW, hb = x / ROW, h = hb / NB, e = hb - h * NB;
        float a[8], pb[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            a[k] = qs[h * D + 8 * e + k];
            pb[k] = proj[(8 * e + k) * ROW + j];
        }
        part[(h * ROW + j) * NB + e] = chain8(a, pb);
    }
    __syncthreads();
    for (int o = tid; o < G * ROW; o += nthr) {
        float t[NB];
#pragma unroll
        for (int e = 0; e < NB; ++e) t[e] = part[o * NB + e];
#pragma unroll
        for (int w = NB; w > 1; w >>= 1)
#pragma unroll
            for (int e = 0; e < w / 2; ++e) t[e] = t[2 * e] + t[2 * e + 1];
        qv[o] = t[0];
    }
    __syncthreads();
}

// T = uint32_t selects the signature predictor: one 32-bit word per token,
// scored by the bits it shares with the query's signature (ROW = 32).
template <int ROW, typename T, int G>
__global__ __launch_bounds__(kPredThreads) void k_predict(Plan P) {
    constexpr bool kSig = std::is_same<T, uint32_t>::value;
    static_assert(!kSig || ROW == 32, "signatures have 32 bits");
    extern __shared__ __align__(16) unsigned char smem[];
    TopkShared<G>& TS = *reinterpret_cast<TopkShared<G>*>(smem);
    size_t off = align16(sizeof(TopkShared<G>));
    uint32_t* shist = reinterpret_cast<uint32_t*>(smem + off);
    uint32_t* wsum = shist + kSampBins;  // scan scratch, one word per wave
    off += sizeof(uint32_t) * (kSampBins + kPredThreads / 64);
    int32_t* pages = reinterpret_cast<int32_t*>(smem + off);  // the chunk's page ids
    off += align16(sizeof(int32_t) * (P.cp / kPage + 2));      // keys below start 16-byte aligned
    float* qs = reinterpret_cast<float*>(smem + off);  // [G][d]
    float* qv = qs + G * P.d;                           // [G][ROW]
    uint32_t* keys = reinterpret_cast<uint32_t*>(qv + G * ROW);  // [G][ks]
    const int ks = P.cp + kKeyPad;  // head stride of the keys: the G rows of a token in distinct banks

    const int tid = threadIdx.x, nthr = blockDim.x;
    const int lane = tid & 63, wave = tid >> 6, nwaves = nthr >> 6;
    const int bg = blockIdx.y, b = bg / P.Hkv, g = bg % P.Hkv, c = blockIdx.x;
    const int L = P.seq_lens[b];
    const Regions R = regions(P, L);
    const int t0 = max(c * P.cp, R.lo), t1 = min((c + 1) * P.cp, R.hi);
    if (t0 >= t1) return;
    const int d = P.d;

    // sample words of the chunk's middle tokens, their histogram over the top
    // kSampBits, and the tokens grouped by that bin (a counting sort): the
    // sampler later reads one bin's tokens instead of scanning the tail
    const int tb = (t0 / kPage) * kPage;
    const int ntok = ((t1 - 1) / kPage + 1) * kPage - tb;
    const int32_t* btrow = P.bt + static_cast<size_t>(b) * P.max_blocks;
    for (int x = tid; x < kSampBins; x += nthr) shist[x] = 0;
    for (int x = tid; x < ntok / kPage; x += nthr) pages[x] = btrow[tb / kPage + x];
    // scaled queries of the group's heads: q_s = fl32(q * fl32(1/sqrt(d)))
    for (int x = tid; x < G * d; x += nthr) {
        const int h = x / d, cc = x - h * d;
        qs[x] = P.q[(static_cast<size_t>(b) * P.Hq + g * G + h) * d + cc] * P.scale32;
    }
    __syncthreads();
    // a chunk spans at most kPredKeys / G tokens: kPhx quads per thread, their
    // words kept in registers for the scatter after the score stream.  With a
    // low-rank or exact score stream the quads are computed inside it, one
    // per iteration while the rows are in flight.
    constexpr int kPhx = kPredKeys / G / 4 / kPredThreads;
    static_assert(kPhx >= 1, "a quad per thread");
    constexpr bool kKeep = kPhx <= 2;  // words held through the stream (else computed again)
    uint4 wq[kKeep ? kPhx : 1];
    auto sample_quad = [&](int e) __attribute__((always_inline)) {
        const int qd = (t0 >> 2) + tid + e * nthr;
        if (4 * qd < t1) {
            const uint4 w = quad_words(static_cast<uint32_t>(qd), g, b, P.seed_lo, P.seed_hi);
            if constexpr (kKeep) wq[e] = w;
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const int i = 4 * qd + f;
                if (i >= t0 && i < t1) atomicAdd(&shist[word_of(w, f) >> (32 - kSampBits)], 1u);
            }
        }
    };
    int phx = 0;  // quads done (wave-uniform)
    if (kSig || R.k == 0) {
#pragma unroll
        for (int e = 0; e < kPhx; ++e) sample_quad(e);
        phx = kPhx;
    }

    if (R.k > 0) {
        // the heads' order-key brackets, reset before the barrier that ends
        // step 1 (the stream's atomics follow it)
        if (tid < G) {
            TS.lo[tid] = 0xFFFFFFFFu;
            TS.hi[tid] = 0;
        }
        // 1) low-rank queries q~ = pdot(q_s, P[:, j]) (the signature predictor
        //    signs these)
        if (P.predictor != 0) {
            float* part = reinterpret_cast<float*>(keys);  // free until the score stream
            const float* pg = P.proj + static_cast<size_t>(g) * P.proj_stride;  // the group's basis
            if (d == 128) low_rank_query<128, ROW, G>(qs, pg, qv, part, tid, nthr);
            else low_rank_query<64, ROW, G>(qs, pg, qv, part, tid, nthr);
        } else {
            for (int x = tid; x < G * ROW; x += nthr) qv[x] = qs[x];
            __syncthreads();
        }

        const int cbase = c * P.cp;
        if constexpr (kSig) {
            // 2') signature scores: bit j of the query's signature is q~_j > 0,
            //     the test the key signatures were made with; a token scores
            //     the number of equal bits.  A page's 16 words are 64
            //     contiguous bytes: 4 tokens per lane and load.
            uint32_t qsig[G], klo[G], khi[G];
#pragma unroll
            for (int h = 0; h < G; ++h) {
                uint32_t w = 0;
#pragma unroll
                for (int jj = 0; jj < 32; ++jj) w |= (qv[h * 32 + jj] > 0.0f ? 1u : 0u) << jj;
                qsig[h] = w;
                klo[h] = 0xFFFFFFFFu;
                khi[h] = 0;
            }
            const uint32_t* ssrc = P.ksig + static_cast<size_t>(g) * kPage;
            const uint32_t pstride = static_cast<uint32_t>(P.Hkv) * kPage;  // words per page
            constexpr int SU = 4;  // loads in flight per lane
            for (int base = 4 * tid; base < ntok; base += 4 * nthr * SU) {
                uint4 wv[SU];
#pragma unroll
                for (int u = 0; u < SU; ++u) {
                    const int tl = base + 4 * nthr * u;
                    if (tl < ntok) {
                        const uint32_t pg = static_cast<uint32_t>(pages[tl / kPage]);
                        wv[u] = *reinterpret_cast<const uint4*>(ssrc + static_cast<uint64_t>(pg) * pstride +
                                                                tl % kPage);
                    }
                }
#pragma unroll
                for (int u = 0; u < SU; ++u) {
                    const int tl = base + 4 * nthr * u;
                    if (tl >= ntok) continue;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int tt = tb + tl + e;
                        if (tt < t0 || tt >= t1) continue;
                        const uint32_t kw = word_of(wv[u], e);
#pragma unroll
                        for (int h = 0; h < G; ++h) {
                            const uint32_t ok = okey(static_cast<float>(32 - __popc(qsig[h] ^ kw)));
                            keys[h * ks + tt - cbase] = ok;
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
        } else {
        // 2) scores: LPT lanes per token row, 8 elements per lane; the G sums
        //    of a row are spread over its lanes, each finished by one lane
        constexpr int LPT = ROW / 8, TPW = 64 / LPT;
        using SP = Spread<G, LPT>;
        constexpr int NH = SP::NH;
        const int j = lane % LPT, slot = lane / LPT;
        float qreg[G][8];
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) qreg[h][e] = qv[h * ROW + 8 * j + e];
        const T* src = static_cast<const T*>(P.predictor == 1 ? static_cast<const void*>(P.kt) : P.k);
        const bool fin = SP::finisher(j);
        int kst[NH];  // this lane's heads' score rows, offset by the chunk start
        uint32_t klo[NH], khi[NH];  // order-key range of the stored scores
#pragma unroll
        for (int e = 0; e < NH; ++e) {
            kst[e] = SP::head(j, e) * ks - cbase;
            klo[e] = 0xFFFFFFFFu;
            khi[e] = 0;
        }
        // Rows past the chunk's last page reread a row of that page and are
        // not stored.  Each iteration requests its whole batch before scoring
        // any of it (no loads carried across iterations, so the waits stay
        // exact).  Token offsets are non-negative: unsigned page arithmetic.
        const uint32_t pstride = static_cast<uint32_t>(P.Hkv) * kPage * ROW;  // elements per page
        const T* gsrc = src + static_cast<size_t>(g) * kPage * ROW + 8 * j;
        const uint32_t tlast = static_cast<uint32_t>(ntok - 1);
        // rows per lane group and batch: fewer when the G query registers are many
        constexpr int PU = G * sizeof(T) >= 32 ? 2 : G * sizeof(T) >= 16 ? 4 : 2 * kUnroll;
        for (int sb = wave * TPW * PU; sb < ntok; sb += nwaves * TPW * PU) {
            Raw8 kr[PU];
#pragma unroll
            for (int u = 0; u < PU; ++u) {
                const uint32_t tl = min(static_cast<uint32_t>(sb + u * TPW + slot), tlast);
                const uint32_t pg = static_cast<uint32_t>(pages[tl / kPage]);
                load_raw_nt(gsrc + static_cast<uint64_t>(pg) * pstride + (tl % kPage) * ROW, kr[u]);
            }
#pragma unroll
            for (int e = 0; e < kPhx; ++e)
                if (e == phx) sample_quad(e);
            phx += phx < kPhx ? 1 : 0;
#pragma unroll
            for (int u = 0; u < PU; ++u) {
                const int tt = tb + sb + u * TPW + slot;
                float kf[8];
                widen<T>(kr[u], kf);
                float part[G], sv[NH];
#pragma unroll
                for (int h = 0; h < G; ++h) part[h] = chain8(qreg[h], kf);
                spread_across_lanes<G, LPT>(part, sv, j);
                if (fin && tt >= t0 && tt < t1) {
#pragma unroll
                    for (int e = 0; e < NH; ++e) {
                        const uint32_t ok = okey(sv[e]);
                        keys[kst[e] + tt] = ok;
                        klo[e] = min(klo[e], ok);
                        khi[e] = max(khi[e], ok);
                    }
                }
            }
        }
        // lanes with the same j hold the same heads: reduce over the others
#pragma unroll
        for (int e = 0; e < NH; ++e) {
            uint32_t a = klo[e], bb = khi[e];
            for (int o = LPT; o < 64; o <<= 1) {
                a = min(a, static_cast<uint32_t>(__shfl_xor(a, o, 64)));
                bb = max(bb, static_cast<uint32_t>(__shfl_xor(bb, o, 64)));
            }
            if (lane < LPT && fin) {
                atomicMin(&TS.lo[SP::head(j, e)], a);
                atomicMax(&TS.hi[SP::head(j, e)], bb);
            }
        }
        }  // score stream
        __syncthreads();
    }
    // the quads a short stream left (their histogram counts are complete at
    // the barrier that opens the top-k or the counting sort)
#pragma unroll
    for (int e = 0; e < kPhx; ++e)
        if (e >= phx) sample_quad(e);

    if (R.k > 0) {
        // 3) chunk top-kp per head, written as candidates (any order)
        const int cbase = c * P.cp;
        const int kp = min(R.k, t1 - t0);
        const size_t bh0 = static_cast<size_t>(b) * P.Hq + g * G;
        if constexpr (kSig) {
            // 3') integer scores 0..32: the boundary score s* (the largest v
            //     with at least kp keys >= v) by a search on block-wide counts
            //     (three thresholds per sweep), then every key above s* and the kp - above tokens at
            //     s* with the lowest indices.  Each thread owns a contiguous
            //     token range, so a block scan ranks the ties in index order.
            const int o0 = t0 - cbase, o1 = t1 - cbase, oa = o0 & ~3;
            const int span = (((o1 - oa) + nthr - 1) / nthr + 3) & ~3;
            const int my0 = oa + tid * span, my1 = min(my0 + span, o1);
            uint32_t* red = &TS.S.hist[0][0];  // [2][nwaves][3G] partial counts (free here)
            auto count_cmp = [&](const uint32_t (&th)[G], uint32_t (&above)[G], uint32_t (&equal)[G]) {
#pragma unroll
                for (int h = 0; h < G; ++h) above[h] = equal[h] = 0;
                for (int o = my0; o < my1; o += 4) {
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        const uint4 kk = *reinterpret_cast<const uint4*>(keys + h * ks + o);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t k = word_of(kk, e);
                            const bool in = o + e >= o0 && o + e < o1;
                            above[h] += (in && k > th[h]) ? 1u : 0u;
                            equal[h] += (in && k == th[h]) ? 1u : 0u;
                        }
                    }
                }
            };
            // block-wide sums of 3G per-thread counts (double-buffered by pass)
            constexpr int NC = 3 * G;
            auto block_sum = [&](uint32_t (&v)[NC], int buf) {
#pragma unroll
                for (int x = 0; x < NC; ++x) {
                    uint32_t y = v[x];
                    for (int m = 1; m < 64; m <<= 1) y += static_cast<uint32_t>(__shfl_xor(y, m, 64));
                    if (lane == 0) red[(buf * nwaves + wave) * NC + x] = y;
                }
                __syncthreads();
#pragma unroll
                for (int x = 0; x < NC; ++x) v[x] = 0;
                for (int w2 = 0; w2 < nwaves; ++w2)
#pragma unroll
                    for (int x = 0; x < NC; ++x) v[x] += red[(buf * nwaves + w2) * NC + x];
            };
            int slo[G], shi[G];
            uint32_t th[G], ca[G], ce[G];
#pragma unroll
            for (int h = 0; h < G; ++h) {
                slo[h] = 0;   // count(score >= 0) = all >= kp
                shi[h] = 33;  // count(score >= 33) = 0 < kp
            }
            // three probes per pass split [slo, shi) in quarters: 33 -> 9 -> 3 -> 1
            for (int it = 0; it < 3; ++it) {
                uint32_t pth[NC], cnt[NC];
#pragma unroll
                for (int h = 0; h < G; ++h)
#pragma unroll
                    for (int j = 0; j < 3; ++j)
                        pth[3 * h + j] = okey(static_cast<float>(slo[h] + (shi[h] - slo[h]) * (j + 1) / 4));
#pragma unroll
                for (int x = 0; x < NC; ++x) cnt[x] = 0;
                for (int o = my0; o < my1; o += 4) {
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        const uint4 kk = *reinterpret_cast<const uint4*>(keys + h * ks + o);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t k = word_of(kk, e);
                            const bool in = o + e >= o0 && o + e < o1;
#pragma unroll
                            for (int j = 0; j < 3; ++j) cnt[3 * h + j] += (in && k >= pth[3 * h + j]) ? 1u : 0u;
                        }
                    }
                }
                block_sum(cnt, it & 1);
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    int nlo = slo[h], nhi = shi[h];
#pragma unroll
                    for (int j = 0; j < 3; ++j) {
                        const int m = slo[h] + (shi[h] - slo[h]) * (j + 1) / 4;
                        if (cnt[3 * h + j] >= static_cast<uint32_t>(kp)) nlo = max(nlo, m);
                        else nhi = min(nhi, m);
                    }
                    slo[h] = nlo;
                    shi[h] = nhi;
                }
            }
#pragma unroll
            for (int h = 0; h < G; ++h) th[h] = okey(static_cast<float>(slo[h]));
            count_cmp(th, ca, ce);
            uint64_t* __restrict__ cand = P.cand;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                uint32_t tot;
                const uint32_t ex = block_excl_scan(ca[h] | (ce[h] << 16), wsum, tot);
                const uint32_t need = static_cast<uint32_t>(kp) - (tot & 0xFFFFu);  // ties to take, >= 1
                uint32_t pos = (ex & 0xFFFFu) + min(ex >> 16, need);
                uint32_t tie = ex >> 16;  // ties before this thread's range
                uint64_t* out = cand + ((bh0 + h) * P.ncp + c) * P.kcap;
                for (int o = my0; o < my1; o += 4) {
                    const uint4 kk = *reinterpret_cast<const uint4*>(keys + h * ks + o);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t k = word_of(kk, e);
                        if (o + e < o0 || o + e >= o1) continue;
                        const bool take = k > th[h] || (k == th[h] && tie++ < need);
                        if (take && pos < static_cast<uint32_t>(kp))
                            out[pos++] = topk_key(k, static_cast<uint32_t>(cbase + o + e));
                    }
                }
                if (tid == 0) {
                    uint32_t* cr = P.crange + ((bh0 + h) * P.ncp + c) * 2;
                    cr[0] = th[h];  // the smallest emitted order key
                    cr[1] = TS.hi[h];
                }
            }
        } else {
        uint32_t want[G], total[G], lo[G], hi[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            want[h] = static_cast<uint32_t>(kp);
            total[h] = static_cast<uint32_t>(t1 - t0);
            lo[h] = TS.lo[h];
            hi[h] = TS.hi[h];
        }
        const int ncp = P.ncp, kcap = P.kcap;
        uint64_t* __restrict__ cand = P.cand;
        // each thread's keys sit at fixed slots: iteration it, head h, token
        // e of the quad at offset o = o0 + 4 (tid + it nthr) take slot
        // (it G + h) 4 + e (G cp <= kPredKeys: at most 8 / G iterations);
        // each visit reads 4 consecutive keys of every head with one 16-byte
        // LDS load per head (offsets from the 16-byte aligned chunk start)
        constexpr int NIT = 8 / G;
        static_assert(4 * kPredThreads * 8 >= kPredKeys, "a chunk's keys fit 32 slots per thread");
        const int o0 = (t0 - cbase) & ~3, o1 = t1 - cbase;
        block_topk_slots<G, 32>(TS, want, total, lo, hi, [&](auto&& f) __attribute__((always_inline)) {
#pragma unroll
            for (int it = 0; it < NIT; ++it) {
                const int o = o0 + 4 * (tid + it * nthr);
                if (o >= o1) continue;
                uint4 kk[G];
#pragma unroll
                for (int h = 0; h < G; ++h) kk[h] = *reinterpret_cast<const uint4*>(keys + h * ks + o);
                if (cbase + o >= t0 && o + 4 <= o1) {  // all four tokens in the chunk: no checks
#pragma unroll
                    for (int h = 0; h < G; ++h)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            f((it * G + h) * 4 + e, word_of(kk[h], e), static_cast<uint32_t>(cbase + o + e));
                } else {
#pragma unroll
                    for (int h = 0; h < G; ++h)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int t = cbase + o + e;
                            if (t >= t0 && t < t1) f((it * G + h) * 4 + e, word_of(kk[h], e), static_cast<uint32_t>(t));
                        }
                }
            }
        }, [&](int s, auto&& g) __attribute__((always_inline)) {
            const int it = s / (4 * G), h = (s / 4) % G, e = s % 4;
            const int o = o0 + 4 * (tid + it * nthr) + e;
            g(keys[h * ks + o], static_cast<uint32_t>(cbase + o));
        }, [&](int h, uint32_t pos, uint64_t key) __attribute__((always_inline)) {
            if (pos < static_cast<uint32_t>(kp)) cand[((bh0 + h) * ncp + c) * kcap + pos] = key;
        });
        // order-key bracket of the candidates for the merge: [threshold key, chunk max]
        if (tid < G) {
            uint32_t* cr = P.crange + ((bh0 + tid) * P.ncp + c) * 2;
            cr[0] = TS.thr[tid] ? static_cast<uint32_t>(TS.thr[tid] >> 32) : lo[tid];
            cr[1] = hi[tid];
        }
        }  // chunk top-k
    }
    // 4) the counting sort of the chunk's middle tokens by bin: offsets of
    //    every bin (soff), the tokens staged in their bins' ranges in LDS
    //    (the score area is free after the top-k), then one coalesced copy
    __syncthreads();
    {
        static_assert(kSampBins % kPredThreads == 0, "bins per thread");
        constexpr int PER = kSampBins / kPredThreads;
        uint32_t v[PER], sum = 0;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            v[e] = shist[PER * tid + e];
            sum += v[e];
        }
        uint32_t total;
        uint32_t run = block_excl_scan(sum, wsum, total);
        uint32_t* so = P.soff + (static_cast<size_t>(bg) * P.ncp + c) * (kSampBins + 1);
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            shist[PER * tid + e] = run;  // bin cursor for the scatter below
            so[PER * tid + e] = run;
            run += v[e];
        }
        if (tid == 0) so[kSampBins] = total;
        __syncthreads();
        int32_t* stage = reinterpret_cast<int32_t*>(keys);
#pragma unroll
        for (int e = 0; e < kPhx; ++e) {
            const int qd = (t0 >> 2) + tid + e * nthr;
            if (4 * qd < t1) {
                uint4 w;
                if constexpr (kKeep) w = wq[e];
                else w = quad_words(static_cast<uint32_t>(qd), g, b, P.seed_lo, P.seed_hi);
#pragma unroll
                for (int f = 0; f < 4; ++f) {
                    const int i = 4 * qd + f;
                    if (i >= t0 && i < t1) stage[atomicAdd(&shist[word_of(w, f) >> (32 - kSampBits)], 1u)] = i;
                }
            }
        }
        __syncthreads();
        // stored as 16-bit offsets from the chunk's first token (a chunk spans
        // at most kPredKeys tokens)
        uint16_t* sl = P.slist + (static_cast<size_t>(bg) * P.ncp + c) * P.cp;
        const int cfirst = c * P.cp;
        for (int x = tid; x < t1 - t0; x += nthr) sl[x] = static_cast<uint16_t>(stage[x] - cfirst);
    }
}

// Candidates a predictor chunk emits for one head: min(k, its middle tokens).
__device__ __forceinline__ int chunk_candidates(int cp, const Regions R, int c) {
    const int a = max(c * cp, R.lo), e = min((c + 1) * cp, R.hi);
    return a < e ? min(R.k, e - a) : 0;
}

// ===========================================================================
// pre-merge (few heads, many predictor chunks): block (head, part) merges the
// candidates of its share of the chunks into that share's exact top-min(k, n)
// (the global top-k is within the union of the parts' top-k), and the group's
// first head sums the share's sample-word histograms; the select then merges
// kPremergeParts parts instead of every chunk.
// ===========================================================================
__global__ __launch_bounds__(kSelectThreads) void k_premerge(Plan P) {
    __shared__ TopkShared<1> TS;
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int bh = blockIdx.x, s = blockIdx.y, b = bh / P.Hq, h = bh % P.Hq, g = h / P.G;
    const int bg = b * P.Hkv + g;
    const int L = P.seq_lens[b];
    const Regions R = regions(P, L);
    const int cp = P.cp, ncp = P.ncp, kcap = P.kcap, np = P.nparts;
    const int c0 = s * ncp / np, c1 = (s + 1) * ncp / np;  // the part's chunks
    if (h % P.G == 0) {  // the group's tail histogram over the part's chunks
        const uint32_t* soffg = P.soff + static_cast<size_t>(bg) * ncp * (kSampBins + 1);
        uint32_t* h2 = P.hist2 + (static_cast<size_t>(bg) * np + s) * kSampBins;
        for (int x = tid; x < kSampBins; x += nthr) {
            uint32_t sum = 0;
            for (int c = c0; c < c1; ++c) {
                if (max(c * cp, R.lo) >= min((c + 1) * cp, R.hi)) continue;
                const uint32_t* off = soffg + static_cast<size_t>(c) * (kSampBins + 1) + x;
                sum += off[1] - off[0];
            }
            h2[x] = sum;
        }
    }
    uint32_t tot = 0, lo = 0xFFFFFFFFu, hi = 0;
    for (int c = c0; c < c1; ++c) {
        const int nc = chunk_candidates(cp, R, c);
        if (!nc) continue;
        const uint32_t* cr = P.crange + (static_cast<size_t>(bh) * ncp + c) * 2;
        tot += static_cast<uint32_t>(nc);
        lo = min(lo, cr[0]);
        hi = max(hi, cr[1]);
    }
    const uint32_t keep = min(static_cast<uint32_t>(R.k), tot);
    const uint64_t* __restrict__ cand = P.cand + (static_cast<size_t>(bh) * ncp + c0) * kcap;
    uint64_t* __restrict__ out = P.cand2 + (static_cast<size_t>(bh) * np + s) * P.kcap2;  // keep <= kcap2
    const int slots = (c1 - c0) * kcap;
    const uint32_t want[1] = {keep}, total[1] = {tot}, lo1[1] = {lo}, hi1[1] = {hi};
    constexpr int kBatch = 8;
    block_topk<1>(TS, want, total, lo1, hi1, [&](auto&& f) __attribute__((always_inline)) {
        for (int x0 = tid; x0 < slots; x0 += kBatch * nthr) {
            uint64_t kk[kBatch];
            bool ok[kBatch];
#pragma unroll
            for (int t = 0; t < kBatch; ++t) {
                const int x = x0 + t * nthr;
                const int c = x / kcap, p = x - c * kcap;
                ok[t] = x < slots && p < chunk_candidates(cp, R, c0 + c);
                kk[t] = ok[t] ? cand[x] : 0ull;
            }
#pragma unroll
            for (int t = 0; t < kBatch; ++t)
                if (ok[t]) f(0, static_cast<uint32_t>(kk[t] >> 32), ~static_cast<uint32_t>(kk[t]));
        }
    }, [&](int, uint32_t pos, uint64_t key) __attribute__((always_inline)) {
        if (pos < keep) out[pos] = key;
    });
    if (tid == 0) {
        P.pcount[static_cast<size_t>(bh) * np + s] = static_cast<int32_t>(keep);
        uint32_t* cr = P.crange2 + (static_cast<size_t>(bh) * np + s) * 2;
        cr[0] = TS.thr[0] ? static_cast<uint32_t>(TS.thr[0] >> 32) : lo;
        cr[1] = hi;
    }
}

// ===========================================================================
// select: exact top-k, fixed-set bitmap, tail histograms, base threshold
// ===========================================================================

constexpr int kSelLdsWords = 4096;  // fixed-set bitmaps of up to 131072 tokens are built in LDS
constexpr int kSelRegKeys = 8;      // candidate keys per thread held in registers (when they all fit)
constexpr int kSelTopList = 2048;   // top-k tokens listed in LDS before their sample words are computed

// PM: the candidates come pre-merged in P.nparts parts.  LB: the head's
// fixed-set bitmap is built in LDS (max_seq_len <= 32 * kSelLdsWords) and
// stored once at the end; otherwise it is built in place in global memory.
template <bool PM, bool LB>
__global__ __launch_bounds__(kSelectThreads) void k_select(Plan P) {
    __shared__ TopkShared<1> TS;
    __shared__ HeadSamp SS;
    __shared__ uint32_t lbits[LB ? kSelLdsWords : 1];
    __shared__ int32_t ltop[kSelTopList];
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int bh = blockIdx.x, b = bh / P.Hq, h = bh % P.Hq, g = h / P.G;
    const int bg = b * P.Hkv + g;
    const int L = P.seq_lens[b];
    const Regions R = regions(P, L);
    const uint32_t slo = P.seed_lo, shi = P.seed_hi;
    // lambdas below capture these locals, never the kernel argument itself
    const int cp = P.cp, ncp = P.ncp, kcap = P.kcap;
    // candidate parts: the predictor chunks, or (few heads, many chunks) the
    // pre-merged groups of chunks with explicit counts and histograms
    const int np = PM ? P.nparts : 0, nparts = PM ? np : ncp;
    const int pk = PM ? P.kcap2 : kcap;  // key slots per part
    const uint64_t* __restrict__ cand = PM ? P.cand2 + static_cast<size_t>(bh) * np * pk
                                           : P.cand + static_cast<size_t>(bh) * ncp * kcap;
    const uint32_t* __restrict__ crng = PM ? P.crange2 + static_cast<size_t>(bh) * np * 2
                                           : P.crange + static_cast<size_t>(bh) * ncp * 2;
    const int32_t* __restrict__ pcnt = PM ? P.pcount + static_cast<size_t>(bh) * np : nullptr;
    auto part_count = [&](int c) __attribute__((always_inline)) {
        if constexpr (PM) return static_cast<int>(pcnt[c]);
        else return chunk_candidates(cp, R, c);
    };
    uint32_t* __restrict__ gbits = P.bits + static_cast<size_t>(bh) * P.words;
    uint32_t* __restrict__ bits = LB ? lbits : gbits;
    const uint32_t* soffg = P.soff + static_cast<size_t>(bg) * ncp * (kSampBins + 1);
    if (tid == 0 && P.gcounts && h % P.G == 0) {
        P.gcounts[2 * bg] = 0;
        P.gcounts[2 * bg + 1] = 0;
    }
    if (tid == 0 && h % P.G == 0) P.gw[bg] = 0u;  // the budgets raise it

    // the candidates are requested first, so their loads overlap the tail
    // histogram's: into registers when every slot fits, with the parts' key
    // brackets
    const int slots = nparts * pk;
    const bool inreg = R.k > 0 && slots <= kSelRegKeys * nthr;  // block-uniform
    uint64_t rk[kSelRegKeys];
    bool rv[kSelRegKeys];
#pragma unroll
    for (int t = 0; t < kSelRegKeys; ++t) {
        const int x = tid + t * nthr;
        const int c = x / pk, p = x - c * pk;
        rv[t] = inreg && x < slots && p < part_count(c);
        rk[t] = rv[t] ? cand[x] : 0ull;
    }
    constexpr int kCB = 4;  // chunks whose loads are issued together
    uint32_t tot = 0, lo = 0xFFFFFFFFu, hi = 0;
    if (R.k > 0) {
        for (int c0 = 0; c0 < nparts; c0 += kCB) {
            uint32_t clo[kCB], chi[kCB];
#pragma unroll
            for (int t = 0; t < kCB; ++t) {
                const int c = c0 + t;
                const int nc = c < nparts ? part_count(c) : 0;
                tot += static_cast<uint32_t>(nc);
                const uint32_t* cr = crng + static_cast<size_t>(nc ? c : 0) * 2;
                clo[t] = nc ? cr[0] : 0xFFFFFFFFu;
                chi[t] = nc ? cr[1] : 0u;
            }
#pragma unroll
            for (int t = 0; t < kCB; ++t) {
                lo = min(lo, clo[t]);
                hi = max(hi, chi[t]);
            }
        }
    }

    // 1) bitmap: sinks [0, sp), window [hi, L); tail histogram = middle histogram
    const int wl = (L + 31) >> 5;
    for (int w = tid; w < wl; w += nthr) {
        uint32_t word = 0;
        const int i0 = 32 * w;
        if (i0 < R.sp) word |= (R.sp - i0 >= 32) ? 0xFFFFFFFFu : ((1u << (R.sp - i0)) - 1u);
        if (i0 + 32 > R.hi) {
            const int a = max(R.hi - i0, 0), e = min(L - i0, 32);  // bits [a, e)
            if (e > a) word |= (e - a >= 32 ? 0xFFFFFFFFu : ((1u << (e - a)) - 1u)) << a;
        }
        bits[w] = word;
    }
    if constexpr (PM) {
        const uint32_t* h2 = P.hist2 + static_cast<size_t>(bg) * np * kSampBins;
        for (int x = tid; x < kSampBins; x += nthr) {
            uint32_t sum = 0;
            for (int c = 0; c < np; ++c) sum += h2[static_cast<size_t>(c) * kSampBins + x];
            SS.hist[x] = sum;
        }
    }
    if constexpr (!PM) {  // two bins of this thread and kCB chunks requested at once
        constexpr int PER = 2;
        for (int x0 = tid; x0 < kSampBins; x0 += PER * nthr) {
            uint32_t sum[PER] = {};
            for (int c0 = 0; c0 < ncp; c0 += kCB) {
                uint32_t a[PER][kCB], e[PER][kCB];
#pragma unroll
                for (int u = 0; u < PER; ++u)
#pragma unroll
                    for (int t = 0; t < kCB; ++t) {
                        const int x = x0 + u * nthr, c = c0 + t;
                        const bool live = x < kSampBins && c < ncp && max(c * cp, R.lo) < min((c + 1) * cp, R.hi);
                        const uint32_t* off = soffg + static_cast<size_t>(live ? c : 0) * (kSampBins + 1) + (live ? x : 0);
                        a[u][t] = live ? off[0] : 0u;
                        e[u][t] = live ? off[1] : 0u;
                    }
#pragma unroll
                for (int u = 0; u < PER; ++u)
#pragma unroll
                    for (int t = 0; t < kCB; ++t) sum[u] += e[u][t] - a[u][t];
            }
#pragma unroll
            for (int u = 0; u < PER; ++u)
                if (x0 + u * nthr < kSampBins) SS.hist[x0 + u * nthr] = sum[u];
        }
    }

    // 2) exact top-k from the chunk candidates: set the bit and take the token
    //    out of the tail histogram (block_topk starts with a barrier)
    if (R.k > 0) {
        const uint32_t want[1] = {static_cast<uint32_t>(R.k)}, total[1] = {tot}, lo1[1] = {lo}, hi1[1] = {hi};
        const bool listed = R.k <= kSelTopList;  // block-uniform; positions are < R.k
        auto emit = [&](int, uint32_t pos, uint64_t key) __attribute__((always_inline)) {
            const uint32_t i = ~static_cast<uint32_t>(key);
            atomicOr(&bits[i >> 5], 1u << (i & 31));
            if (listed) ltop[pos] = static_cast<int32_t>(i);  // its sample word below, all lanes busy
            else atomicSub(&SS.hist[token_word(i, g, b, slo, shi) >> (32 - kSampBits)], 1u);
        };
        constexpr int kBatch = 8;  // candidate keys loaded before any is visited
        block_topk<1>(TS, want, total, lo1, hi1, [&](auto&& f) __attribute__((always_inline)) {
            if (inreg) {
#pragma unroll
                for (int t = 0; t < kSelRegKeys; ++t)
                    if (rv[t]) f(0, static_cast<uint32_t>(rk[t] >> 32), ~static_cast<uint32_t>(rk[t]));
                return;
            }
            for (int x0 = tid; x0 < slots; x0 += kBatch * nthr) {
                uint64_t kk[kBatch];
                bool ok[kBatch];
#pragma unroll
                for (int t = 0; t < kBatch; ++t) {
                    const int x = x0 + t * nthr;
                    const int c = x / pk, p = x - c * pk;
                    ok[t] = x < slots && p < part_count(c);
                    kk[t] = ok[t] ? cand[x] : 0ull;
                }
#pragma unroll
                for (int t = 0; t < kBatch; ++t)
                    if (ok[t]) f(0, static_cast<uint32_t>(kk[t] >> 32), ~static_cast<uint32_t>(kk[t]));
            }
        }, emit);
        if (listed) {  // block_topk ends with a barrier
            for (int x = tid; x < R.k; x += nthr) {
                const uint32_t i = static_cast<uint32_t>(ltop[x]);
                atomicSub(&SS.hist[token_word(i, g, b, slo, shi) >> (32 - kSampBits)], 1u);
            }
            __syncthreads();
        }
    } else {
        __syncthreads();
    }
    for (int x = tid; x < kSampBins; x += nthr) P.hh[static_cast<size_t>(bh) * kSampBins + x] = SS.hist[x];

    // 3) base sample: first nb tail tokens in (word, index) order
    const uint32_t rank = (R.nb > 0 && R.nb < R.NT) ? static_cast<uint32_t>(R.nb) : 0u;
    const BinLists BL{soffg, P.slist + static_cast<size_t>(bg) * ncp * cp, ncp, cp, R.lo, R.hi};
    head_sample_threshold(SS, TS.S, BL, [&](int i) __attribute__((always_inline)) {
        return token_word(static_cast<uint32_t>(i), g, b, slo, shi);
    }, rank, [&](int i) __attribute__((always_inline)) {
        if constexpr (LB) return bit_of(lbits, i);   // complete after block_topk's closing barrier
        else return bit_of_coherent(gbits, i);
    });
    if constexpr (LB)
        for (int w = tid; w < wl; w += nthr) gbits[w] = lbits[w];
    if (tid == 0) {
        HeadState hs{};  // statistics, budget and thresholds are filled in by the budget pass
        hs.L = L;
        hs.k = R.k;
        hs.n_fixed = R.sp + R.wp + R.k;
        hs.NT = R.NT;
        hs.nb = R.nb;
        hs.thr_b = rank ? SS.thr : 0;  // nb == N_t: the whole tail
        P.hs[bh] = hs;
    }
}

// ===========================================================================
// base: pinned exact scores of the union of fixed sets and base samples
// ===========================================================================
struct HeadView {
    uint64_t thr_b, thr_n;
    int nb, n;
    float wsamp, m;
};

template <int D, typename KVT, int G>
__global__ __launch_bounds__(kChunkThreads) void k_base(Plan P) {
    __shared__ uint32_t tmeta[kGatherChunk];
    __shared__ uint32_t trow[kGatherChunk];
    __shared__ float tsc[G][kGatherChunk];  // the scores, stored to bsc one head row at a time
    __shared__ uint32_t wsum[kChunkThreads / 64];
    __shared__ float wmax[kChunkThreads / 64][G];
    __shared__ HeadView hv[G];
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int lane = tid & 63, wave = tid >> 6, nwaves = nthr >> 6;
    // KV heads fastest: the blocks of one (sequence, chunk) launch together and
    // read the same pages, whose KV heads are adjacent in memory
    const int g = blockIdx.x, c = blockIdx.y, b = blockIdx.z, bg = b * P.Hkv + g;
    const int L = P.seq_lens[b];
    const int T0 = c * P.cg;
    if (T0 >= L) return;
    const Regions R = regions(P, L);
    const size_t bh0 = static_cast<size_t>(b) * P.Hq + g * G;
    // the heads' state, the quad's page, sample words and each head's bitmap
    // word (a quad never straddles a 32-token word) are requested together
    if (tid < G) {
        const HeadState& s = P.hs[bh0 + tid];
        hv[tid] = HeadView{s.thr_b, 0, s.nb, 0, 0.f, 0.f};
    }
    const int T1 = min(T0 + P.cg, L);
    const int qd = (T0 >> 2) + tid;
    const bool live4 = 4 * qd < T1;
    const int32_t* btrow = P.bt + static_cast<size_t>(b) * P.max_blocks;
    const uint32_t row0 = live4 ? (static_cast<uint32_t>(btrow[qd >> 2]) * P.Hkv + g) * kPage : 0u;
    const bool anyM = live4 && 4 * qd + 3 >= R.lo && 4 * qd < R.hi;
    const uint4 w = anyM ? quad_words(static_cast<uint32_t>(qd), g, b, P.seed_lo, P.seed_hi) : make_uint4(0, 0, 0, 0);
    uint32_t fw[G];
#pragma unroll
    for (int h = 0; h < G; ++h) fw[h] = live4 ? P.bits[(bh0 + h) * P.words + (qd >> 3)] : 0u;
    __syncthreads();

    // membership (one Philox word per token): meta = base mask | fixed mask << 8
    uint32_t m4[4] = {0, 0, 0, 0};
    uint32_t mine = 0;
    if (live4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 4 * qd + e;
            const bool inM = i >= R.lo && i < R.hi;
            const uint64_t key = sample_key(word_of(w, e), static_cast<uint32_t>(i));
            uint32_t bm = 0, fm = 0;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const bool fx = (fw[h] >> (i & 31)) & 1u;
                const bool bs = inM && !fx && hv[h].nb > 0 && key >= hv[h].thr_b;
                bm |= (fx || bs) ? (1u << h) : 0u;
                fm |= fx ? (1u << h) : 0u;
            }
            const bool live = i < T1 && bm;
            m4[e] = live ? (bm | (fm << 8)) : 0u;
            mine += live ? 1u : 0u;
        }
    }
    uint32_t cnt;
    uint32_t pos = block_excl_scan(mine, wsum, cnt);
    uint16_t* lmeta = P.bmeta + (static_cast<size_t>(bg) * P.ncg + c) * P.cg;
    uint32_t* lrow = P.brow ? P.brow + (static_cast<size_t>(bg) * P.ncg + c) * P.cg : nullptr;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (m4[e]) {
            const uint32_t rw = row0 + ((4 * qd + e) & (kPage - 1));
            tmeta[pos] = m4[e];
            trow[pos] = rw;
            lmeta[pos] = static_cast<uint16_t>(m4[e]);
            if (lrow) lrow[pos] = rw;  // the V row, for the output-level statistics
            ++pos;
        }
    if (tid == 0) {
        P.bcnt[static_cast<size_t>(bg) * P.ncg + c] = static_cast<int32_t>(cnt);
        if (P.gcounts && cnt) atomicAdd(&P.gcounts[2 * bg + 1], static_cast<int>(cnt));
    }
    __syncthreads();

    // pinned scores for all G heads of each listed token: the G sums of a row
    // are spread over its lanes, each finished (max, store) by one lane.  The
    // scores are stored once, in list order: the budget reads them so, and the
    // gather finds a token's scores at its position in this (ascending) list
    constexpr int LPT = D / 8, TPW = 64 / LPT;
    using SP = Spread<G, LPT>;
    constexpr int NH = SP::NH;
    const int j = lane % LPT, slot = lane / LPT;
    const bool fin = SP::finisher(j);
    int hsel[NH];
    float lmax[NH];
#pragma unroll
    for (int e = 0; e < NH; ++e) {
        hsel[e] = SP::head(j, e);
        lmax[e] = -__builtin_inff();
    }
    float qreg[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) qreg[h][e] = P.q[(bh0 + h) * D + 8 * j + e] * P.scale32;
    const KVT* kbase = static_cast<const KVT*>(P.k);
    float* lsc = P.bsc + (static_cast<size_t>(bg) * P.ncg + c) * P.cg * G;
    const int n = static_cast<int>(cnt);
    constexpr int kBU = std::is_same<KVT, uint16_t>::value ? kBaseUnrollBf16 : kBaseUnroll;
    for (int base = wave * TPW * kBU; base < n; base += nwaves * TPW * kBU) {
        Raw8 kr[kBU];
        int xl[kBU];
        uint32_t mk[kBU];
#pragma unroll
        for (int u = 0; u < kBU; ++u) {
            const int x = base + u * TPW + slot;
            const bool act = x < n;
            const int xs = act ? x : 0;
            xl[u] = xs;
            mk[u] = act ? tmeta[xs] : 0u;
            load_raw_nt(kbase + static_cast<size_t>(trow[xs]) * D + 8 * j, kr[u]);
        }
#pragma unroll
        for (int u = 0; u < kBU; ++u) {
            float kf[8];
            widen<KVT>(kr[u], kf);
            float part[G], sv[NH];
#pragma unroll
            for (int h = 0; h < G; ++h) part[h] = chain8(qreg[h], kf);
            spread_across_lanes<G, LPT>(part, sv, j);
            if (fin && mk[u]) {
#pragma unroll
                for (int e = 0; e < NH; ++e) {
                    if ((mk[u] >> hsel[e]) & 1u) lmax[e] = fmaxf(lmax[e], sv[e]);
                    tsc[hsel[e]][xl[u]] = sv[e];
                }
            }
        }
    }
    // per head maximum: lanes with the same j hold the same heads
#pragma unroll
    for (int e = 0; e < NH; ++e)
        for (int o = LPT; o < 64; o <<= 1) lmax[e] = fmaxf(lmax[e], __shfl_xor(lmax[e], o, 64));
    if (lane < LPT && fin) {
#pragma unroll
        for (int e = 0; e < NH; ++e) wmax[wave][hsel[e]] = lmax[e];
    }
    __syncthreads();
    for (int h = 0; h < G; ++h)
        for (int x = tid; x < n; x += nthr) lsc[static_cast<size_t>(h) * P.cg + x] = tsc[h][x];
    if (tid < G) {
        float v = -__builtin_inff();
        for (int w = 0; w < nwaves; ++w) v = fmaxf(v, wmax[w][tid]);
        P.cmax[(bh0 + tid) * P.ncg + c] = v;
    }
}

// ===========================================================================
// budget: exact statistics of the head's base sample, CLT budget, final-sample
// threshold.  One block per query head.  The statistics are fixed-point
// integer sums (order independent) over the base members of every chunk of
// the head's group; each block reduces its own head, so no cross-block
// accumulation is needed.
// ===========================================================================
constexpr int kStatsBatch = 4;  // entries of each of a wave's two chunks requested per lane at once

// The final sample's threshold in the sample order (rank > 0: a new one; else
// the whole tail, or the base sample's when n == n_b).  S.hist holds the
// head's tail histogram.  All threads call.
__device__ __forceinline__ void final_sample_threshold(const Plan& P, HeadSamp& SS, SelShared<1>& FS, HeadState* hsp,
                                                       int bh, int bg, const Regions& R, uint32_t rank, int n,
                                                       uint64_t thr_b) {
    const uint32_t* __restrict__ bits = P.bits + static_cast<size_t>(bh) * P.words;
    const BinLists BL{P.soff + static_cast<size_t>(bg) * P.ncp * (kSampBins + 1),
                      P.slist + static_cast<size_t>(bg) * P.ncp * P.cp, P.ncp, P.cp, R.lo, R.hi};
    const uint32_t b = static_cast<uint32_t>(bg / P.Hkv), g = static_cast<uint32_t>(bg % P.Hkv);
    const uint32_t slo = P.seed_lo, shi = P.seed_hi;
    head_sample_threshold(SS, FS, BL, [&](int i) __attribute__((always_inline)) {
        return token_word(static_cast<uint32_t>(i), g, b, slo, shi);
    }, rank, [&](int i) __attribute__((always_inline)) {
        return bit_of(bits, i);
    });
    if (threadIdx.x == 0) {  // n and the base threshold are thread 0's
        uint64_t thr = 0;  // n == N_t: the whole tail (n == 0: unused)
        if (rank > 0) thr = SS.thr;
        else if (n > 0 && n == R.nb) thr = thr_b;
        hsp->thr_n = thr;
    }
}

// The head's final budget is set (hsp->n): the sample weight, the group's
// gather dispatch weight (expected member density; non-negative fp32 values
// order as their bit patterns) and the rank of a new threshold, 0 unless the
// sample is neither empty, the whole tail nor the base sample.  Thread 0.
__device__ __forceinline__ int settle_budget(const Plan& P, HeadState* hsp, int bg, const Regions& R, int L, int n) {
    const int NT = R.NT, nb = R.nb;
    atomicMax(&P.gw[bg], __float_as_uint(static_cast<float>(R.sp + R.wp + R.k + n) / static_cast<float>(L)));
    hsp->wsamp = n > 0 ? static_cast<float>(static_cast<double>(NT) / static_cast<double>(n)) : 0.0f;
    return (n > 0 && n < NT && n != nb) ? n : 0;
}

// DEFER (output-level mode): statistics, m and the denominator's budget only;
// k_numstat and k_budget_num finish the budget and the threshold.
template <int kThreads, bool DEFER>  // per block
__global__ __launch_bounds__(kThreads) void k_budget(Plan P) {
    constexpr int NW = kThreads / 64;
    __shared__ HeadSamp SS;
    __shared__ SelShared<1> FS;
    __shared__ uint64_t red[NW][5];
    __shared__ int s_nsel;
    __shared__ float s_m;
    const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63, wave = tid >> 6;
    const int bh = blockIdx.x, b = bh / P.Hq, h = bh % P.Hq, g = h / P.G, hg = h % P.G;
    const int bg = b * P.Hkv + g;
    const int L = P.seq_lens[b];
    const Regions R = regions(P, L);
    HeadState* hsp = P.hs + bh;
    if (L == 0) {
        if (tid == 0) {
            const HeadState z{};
            *hsp = z;
        }
        return;
    }
    const uint64_t thr_b = tid == 0 ? hsp->thr_b : 0;  // the base threshold (the select's), for thread 0
    int nfin = 0;                                       // the final budget, thread 0's
    const int nc = (L + P.cg - 1) / P.cg;
    if constexpr (!DEFER) {  // every load of the histogram requested before any is stored
        constexpr int PER = (kSampBins + kThreads - 1) / kThreads;
        uint32_t hv[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int x = tid + e * nthr;
            hv[e] = x < kSampBins ? P.hh[static_cast<size_t>(bh) * kSampBins + x] : 0u;
        }
#pragma unroll
        for (int e = 0; e < PER; ++e)
            if (tid + e * nthr < kSampBins) SS.hist[tid + e * nthr] = hv[e];
    }
    // each wave's first two chunks: member counts, masks and scores requested
    // now, with the histogram and the chunk maxima (they need no m)
    const int G = P.G;
    const uint16_t* bmeta = P.bmeta + static_cast<size_t>(bg) * P.ncg * P.cg;
    const float* bsc = P.bsc + static_cast<size_t>(bg) * P.ncg * P.cg * G + static_cast<size_t>(hg) * P.cg;
    const int32_t* bcnt = P.bcnt + static_cast<size_t>(bg) * P.ncg;
    auto request = [&](int ca, int y0, int na, int nb2, uint32_t (&tm)[2][kStatsBatch],
                       float (&sv)[2][kStatsBatch]) __attribute__((always_inline)) {
        const int cb = ca + NW;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int cc = q ? cb : ca, ncc = q ? nb2 : na;
#pragma unroll
            for (int v = 0; v < kStatsBatch; ++v) {
                const int y = y0 + lane + 64 * v;
                const size_t at = static_cast<size_t>(cc) * P.cg + y;
                tm[q][v] = y < ncc ? static_cast<uint32_t>(bmeta[at]) : 0u;
                sv[q][v] = y < ncc ? bsc[static_cast<size_t>(cc) * P.cg * G + y] : 0.0f;  // head hg's row of the chunk
            }
        }
    };
    const int na0 = wave < nc ? bcnt[wave] : 0, nb0 = wave + NW < nc ? bcnt[wave + NW] : 0;
    uint32_t tm0[2][kStatsBatch];
    float sv0[2][kStatsBatch];
    request(wave, 0, na0, nb0, tm0, sv0);
    if (wave == 0) {  // m: max pinned score over I_f and the base sample
        float m = -__builtin_inff();
        for (int c = lane; c < nc; c += 64) m = fmaxf(m, P.cmax[static_cast<size_t>(bh) * P.ncg + c]);
        for (int o = 1; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
        if (lane == 0) s_m = m;
    }
    __syncthreads();

    // E_i = fixed_weight(s_i - m) over this head's members: SF over the fixed
    // set, S1 and S2 (128-bit) over the base sample.  Each wave takes whole
    // chunks, two at a time, every entry's mask and score requested before any
    // is used.
    {
        const float m = s_m;
        // S2 = sum E^2 < 2^80 per entry, from E = a 2^20 + b: sums of a^2,
        // a b and b^2 (each below 2^40 per entry, so below 2^60 over any
        // sequence) are exact in 64 bits and give S2 = A2 2^40 + AB 2^21 + B2
        uint64_t sf = 0, s1 = 0, a2 = 0, ab = 0, b2 = 0;
        auto add = [&](const uint32_t (&tm)[2][kStatsBatch], const float (&sv)[2][kStatsBatch]) __attribute__((always_inline)) {
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int v = 0; v < kStatsBatch; ++v) {
                    const bool mem = (tm[q][v] >> hg) & 1u, fx = (tm[q][v] >> (8 + hg)) & 1u;
                    const uint64_t E = mem ? fixed_weight(sv[q][v] - m) : 0ull;
                    const uint64_t Es = fx ? 0ull : E;
                    sf += fx ? E : 0ull;
                    s1 += Es;
                    const uint32_t ea = static_cast<uint32_t>(Es >> 20), eb = static_cast<uint32_t>(Es) & 0xFFFFFu;
                    a2 += static_cast<uint64_t>(ea) * ea;
                    ab += static_cast<uint64_t>(ea) * eb;
                    b2 += static_cast<uint64_t>(eb) * eb;
                }
        };
        add(tm0, sv0);
        for (int cw = wave; cw < nc; cw += 2 * NW) {
            const int na = cw == wave ? na0 : bcnt[cw];
            const int nb2 = cw == wave ? nb0 : (cw + NW < nc ? bcnt[cw + NW] : 0);
            const int nmax = max(na, nb2);
            for (int y0 = cw == wave ? 64 * kStatsBatch : 0; y0 < nmax; y0 += 64 * kStatsBatch) {
                uint32_t tm[2][kStatsBatch];
                float sv[2][kStatsBatch];
                request(cw, y0, na, nb2, tm, sv);
                add(tm, sv);
            }
        }
        for (int o = 32; o >= 1; o >>= 1) {
            sf += shfl_xor_u64(sf, o);
            s1 += shfl_xor_u64(s1, o);
            a2 += shfl_xor_u64(a2, o);
            ab += shfl_xor_u64(ab, o);
            b2 += shfl_xor_u64(b2, o);
        }
        if (lane == 0) {
            red[wave][0] = sf;
            red[wave][1] = s1;
            red[wave][2] = a2;
            red[wave][3] = ab;
            red[wave][4] = b2;
        }
    }
    __syncthreads();
    // lanes 0..4 of wave 0 sum one statistic each over the waves; thread 0
    // then holds all five (wave-uniform values)
    uint64_t col = 0;
    if (wave == 0 && lane < 5)
        for (int w = 0; w < NW; ++w) col += red[w][lane];
    auto lane_u64 = [&](int l) __attribute__((always_inline)) {
        const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(col), l));
        const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(col >> 32), l));
        return (static_cast<uint64_t>(hi) << 32) | lo;
    };
    const uint64_t SF = lane_u64(0), S1 = lane_u64(1), A2 = lane_u64(2), AB = lane_u64(3), B2 = lane_u64(4);
    if (tid == 0) {
        const float m = s_m;
        const unsigned __int128 S2 = (static_cast<unsigned __int128>(A2) << 40) +
                                     (static_cast<unsigned __int128>(AB) << 21) + B2;
        hsp->SF = SF;
        hsp->S1 = S1;
        hsp->S2hi = static_cast<uint64_t>(S2 >> 64);
        hsp->S2lo = static_cast<uint64_t>(S2);
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
        hsp->n = n;
        hsp->flags = flags;
        hsp->m = m;
        if constexpr (!DEFER) s_nsel = settle_budget(P, hsp, bg, R, L, n);
        nfin = n;
    }
    if constexpr (DEFER) return;
    __syncthreads();
    final_sample_threshold(P, SS, FS, hsp, bh, bg, R, static_cast<uint32_t>(s_nsel), nfin, thr_b);
}

// ===========================================================================
// Output-level mode.  SkyLight's post ("vAttention Computation") promises
// (eps, delta) on the intermediate quantities and the edgentiq post ("How
// vAttention Works") calls the denominator-only budget a relaxation; without
// it the numerator N = sum_i e^{s_i - m} V_i is held to the same CLT bound.
// With y_i = E_i V_i per channel (E_i the exact fixed-point weights of the
// statistics), over each head's base sample T1 = sum y, T2 = sum y^2 and over
// its fixed set NF = sum y, all fp64 in one order: ascending tokens within each
// gather chunk from +0 (k_numstat, per chunk), then the chunk partials in
// ascending chunk order (k_budget_num).  Then
//   TR = sum_c max(n_b T2_c - T1_c^2, 0),  NN = sum_c (n_b NF_c + N_t T1_c)^2
// (channels ascending) and the numerator's budget is the denominator's
// expression with TR for M2 and NN for Y^2; the larger budget is taken.
// ===========================================================================
constexpr int kNumTile = 64;  // base-list members whose V rows are staged at once

// One block per (gather chunk, group): the chunk's base list (ascending tokens)
// is walked in tiles of kNumTile members whose V rows are staged raw in LDS;
// the next tile's rows are requested before the current tile is summed.  Per
// tile and head, one wave ballot lists the head's base-sample members and its
// fixed members, each ascending; each thread owns (head, channel) chains and
// adds to them the members of the head's lists in order (T1 and T2 over the
// base-sample list, NF over the fixed list).
template <int D, typename KVT, int G>
__global__ __launch_bounds__(kChunkThreads) void k_numstat(Plan P) {
    static_assert(kNumTile == 64, "one wave ballot per tile");
    constexpr int NW = kChunkThreads / 64;
    constexpr int RPL = sizeof(KVT) * 8 / 16;                 // 16-byte loads per 8 elements
    constexpr int LPM = D / 8 * RPL;                          // 16-byte loads per member row
    constexpr int VPT = (kNumTile * LPM + kChunkThreads - 1) / kChunkThreads;  // per thread and tile
    constexpr int EPT = (kNumTile * G + kChunkThreads - 1) / kChunkThreads;
    __shared__ __align__(16) KVT vs[kNumTile][D];  // the tile's V rows as stored
    __shared__ double es[kNumTile][G];           // E_i of each member for each head
    __shared__ uint32_t tm[kNumTile];            // base mask | fixed mask << 8 of each member
    __shared__ uint8_t lst[2][G][kNumTile];      // per head: base-sample members, fixed members
    __shared__ int lcnt[2][G];
    __shared__ uint32_t rows[kGatherChunk];      // V rows of the chunk's members
    __shared__ float hm[G];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = blockIdx.x, c = blockIdx.y, b = blockIdx.z, bg = b * P.Hkv + g;
    const int L = P.seq_lens[b];
    if (c * P.cg >= L) return;  // block-uniform; no partial for chunks past the end
    const size_t bh0 = static_cast<size_t>(b) * P.Hq + g * G;
    const size_t lb = (static_cast<size_t>(bg) * P.ncg + c) * P.cg;  // the chunk's base list
    const int n = P.bcnt[static_cast<size_t>(bg) * P.ncg + c];
    if (tid < G) hm[tid] = P.hs[bh0 + tid].m;
    for (int x = tid; x < n; x += kChunkThreads) rows[x] = P.brow[lb + x];
    // a wave covers one head's channels, CPT consecutive ones per lane (a
    // member's weight is read once for all of them), and heads wave,
    // wave + NW, ... in turn
    constexpr int CPT = D / 64, NHT = (G + NW - 1) / NW;
    static_assert(D % 64 == 0, "a wave covers a head's channels");
    const int cc = lane * CPT;
    double p1[NHT][CPT], p2[NHT][CPT], pf[NHT][CPT];
#pragma unroll
    for (int t = 0; t < NHT; ++t)
#pragma unroll
        for (int k = 0; k < CPT; ++k) p1[t][k] = p2[t][k] = pf[t][k] = 0.0;
    const uint4* vbase = static_cast<const uint4*>(P.v);
    __syncthreads();
    uint4 vr[VPT];
    float sr[EPT];
    uint32_t mr[EPT];
    auto request = [&](int t0) __attribute__((always_inline)) {
        const int tn = min(kNumTile, n - t0);
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int x = tid + u * kChunkThreads, mi = x / LPM, part = x - mi * LPM;
            if (mi < tn) vr[u] = nt_load16(vbase + static_cast<size_t>(rows[t0 + mi]) * LPM + part);
        }
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            const int x = tid + u * kChunkThreads, mi = x / G, h = x - mi * G;
            if (mi < tn) {
                mr[u] = static_cast<uint32_t>(P.bmeta[lb + t0 + mi]);
                sr[u] = P.bsc[lb * G + static_cast<size_t>(h) * P.cg + t0 + mi];
            }
        }
    };
    if (n > 0) request(0);
    for (int t0 = 0; t0 < n; t0 += kNumTile) {
        const int tn = min(kNumTile, n - t0);
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int x = tid + u * kChunkThreads, mi = x / LPM, part = x - mi * LPM;
            if (mi < tn) reinterpret_cast<uint4*>(&vs[mi][0])[part] = vr[u];
        }
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            const int x = tid + u * kChunkThreads, mi = x / G, h = x - mi * G;
            if (mi < tn) {
                es[mi][h] = static_cast<double>(fixed_weight(sr[u] - hm[h]));
                if (h == 0) tm[mi] = mr[u];
            }
        }
        __syncthreads();
        for (int h = wave; h < G; h += NW) {  // lane = member of the tile
            const uint32_t meta = lane < tn ? tm[lane] : 0u;
            const bool mem = (meta >> h) & 1u, fix = (meta >> (8 + h)) & 1u;
            const uint64_t bb = __ballot(mem && !fix), bf = __ballot(mem && fix);
            const uint64_t below = (1ull << lane) - 1ull;
            if (mem && !fix) lst[0][h][__popcll(bb & below)] = static_cast<uint8_t>(lane);
            if (mem && fix) lst[1][h][__popcll(bf & below)] = static_cast<uint8_t>(lane);
            if (lane == 0) {
                lcnt[0][h] = __popcll(bb);
                lcnt[1][h] = __popcll(bf);
            }
        }
        __syncthreads();
        if (t0 + kNumTile < n) request(t0 + kNumTile);  // block-uniform
#pragma unroll
        for (int t = 0; t < NHT; ++t) {
            const int h = wave + t * NW;
            if (h >= G) break;  // wave-uniform
#pragma unroll
            for (int q = 0; q < 2; ++q) {  // q = 0: base sample (T1, T2); q = 1: fixed set (NF)
                const int nl = lcnt[q][h];
                for (int j0 = 0; j0 < nl; j0 += 8) {
                    double e[8];
                    float vf[8][CPT];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int mi = lst[q][h][min(j0 + u, nl - 1)];
                        e[u] = es[mi][h];
#pragma unroll
                        for (int k = 0; k < CPT; ++k) {
                            if constexpr (sizeof(KVT) == 2) vf[u][k] = __uint_as_float(static_cast<uint32_t>(vs[mi][cc + k]) << 16);
                            else vf[u][k] = vs[mi][cc + k];
                        }
                    }
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        if (j0 + u >= nl) break;  // wave-uniform
#pragma unroll
                        for (int k = 0; k < CPT; ++k) {
                            const double y = e[u] * static_cast<double>(vf[u][k]);
                            if (q == 0) {
                                p1[t][k] = p1[t][k] + y;
                                p2[t][k] = p2[t][k] + y * y;
                            } else {
                                pf[t][k] = pf[t][k] + y;
                            }
                        }
                    }
                }
            }
        }
        __syncthreads();  // the tile and its lists are restaged
    }
#pragma unroll
    for (int t = 0; t < NHT; ++t) {
        const int h = wave + t * NW;
        if (h >= G) break;
        double* out = P.npart + ((bh0 + h) * P.ncg + c) * 3 * D;
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            out[cc + k] = p1[t][k];
            out[D + cc + k] = p2[t][k];
            out[2 * D + cc + k] = pf[t][k];
        }
    }
}

template <int kThreads>  // per block
__global__ __launch_bounds__(kThreads) void k_budget_num(Plan P) {
    __shared__ HeadSamp SS;
    __shared__ SelShared<1> FS;
    __shared__ double tot[3][128];  // T1, T2, NF per channel (d <= 128)
    __shared__ int s_nsel;
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int bh = blockIdx.x, b = bh / P.Hq, h = bh % P.Hq, g = h / P.G;
    const int bg = b * P.Hkv + g;
    const int L = P.seq_lens[b];
    const int D = P.d;
    HeadState* hsp = P.hs + bh;
    if (L == 0) {
        if (tid == 0 && P.nstats) P.nstats[2 * bh] = P.nstats[2 * bh + 1] = 0.0;
        return;
    }
    const Regions R = regions(P, L);
    const int NT = R.NT, nb = R.nb;
    const uint64_t thr_b = tid == 0 ? hsp->thr_b : 0;  // thread 0's: the base threshold and
    int nfin = tid == 0 ? hsp->n : 0;                   // the denominator's budget
    for (int x = tid; x < kSampBins; x += nthr) SS.hist[x] = P.hh[static_cast<size_t>(bh) * kSampBins + x];
    if (nb > 0) {  // the chunk partials, summed in chunk order
        const int nc = (L + P.cg - 1) / P.cg;
        const double* pp = P.npart + static_cast<size_t>(bh) * P.ncg * 3 * D;
        for (int x = tid; x < 3 * D; x += nthr) {
            double t = 0.0;
            for (int cc = 0; cc < nc; ++cc) t = t + pp[static_cast<size_t>(cc) * 3 * D + x];
            tot[x / D][x % D] = t;
        }
    }
    __syncthreads();
    if (tid == 0) {
        double TR = 0.0, NN = 0.0;
        if (nb > 0) {
            for (int c = 0; c < D; ++c) {
                double m2 = static_cast<double>(nb) * tot[1][c] - tot[0][c] * tot[0][c];
                if (m2 < 0.0) m2 = 0.0;
                const double yc = static_cast<double>(nb) * tot[2][c] + static_cast<double>(NT) * tot[0][c];
                TR = TR + m2;
                NN = NN + yc * yc;
            }
        }
        if (P.nstats) {
            P.nstats[2 * bh] = TR;
            P.nstats[2 * bh + 1] = NN;
        }
        if (P.force_budget < 0 && nb > 0 && nb < NT) {  // the CLT branch
            const double z = P.z32;
            const double num = (z * z * static_cast<double>(NT) * static_cast<double>(NT)) *
                               (TR * static_cast<double>(nb));
            const double den = (static_cast<double>(nb - 1) * (P.eps * P.eps)) * NN;
            int nN;
            if (den == 0.0) {
                nN = num > 0.0 ? NT : 0;
            } else {
                const double r = num / den;
                nN = r >= static_cast<double>(NT) ? NT : static_cast<int>(__builtin_ceil(r));
            }
            if (nN > nfin) {
                nfin = nN;
                hsp->n = nN;
                hsp->flags = hsp->flags | 8 | (nN == NT ? 1 : 0);
            }
        }
        s_nsel = settle_budget(P, hsp, bg, R, L, nfin);
    }
    __syncthreads();
    final_sample_threshold(P, SS, FS, hsp, bh, bg, R, static_cast<uint32_t>(s_nsel), nfin, thr_b);
}

// ===========================================================================
// gather: weighted softmax over the union of the group's index sets, in two
// passes over the listed tokens: (1) scores (score cache or K row) into LDS,
// then per head the block max and the weights p = w exp(s - max); (2) a pure
// stream of V rows accumulating sum_i p_i V_i.  Every weight is computed once.
// ===========================================================================
constexpr float kRescale = 16.0f;  // reference-maximum headroom for the weights (e^16)
constexpr int kGatherUnrollV = 6;  // V rows per batch and lane group (4 with eight heads per group)
constexpr int kGatherUnrollK = 8;  // K rows per batch and lane group (VALU scoring)

// Group of a gather block.  Block row y takes the group of rank y when the
// groups are ordered by expected member density (n_fixed + n) / L of their
// densest head, descending, ties to the lower group: the groups with the most
// rows per chunk are dispatched first, so the blocks still running at the end
// of the kernel are the light ones and the tail, where too few blocks are left
// to keep HBM busy, stays short.  Every block derives the same order from the
// group weights the budgets wrote.  With more groups than threads the rows
// keep their own groups.
// With more groups than a gather block has threads (up to kOrderMaxGroups), one
// block ranks them once, into gorder, before the gather.
constexpr int kOrderMaxGroups = 4096;
constexpr int kOrderThreads = 1024;

__global__ __launch_bounds__(kOrderThreads) void k_order(Plan P) {
    __shared__ float w[kOrderMaxGroups];
    const int ngr = P.B * P.Hkv;  // kChunkThreads < ngr <= kOrderMaxGroups
    for (int x = threadIdx.x; x < ngr; x += blockDim.x) w[x] = __uint_as_float(P.gw[x]);
    __syncthreads();
    for (int x = threadIdx.x; x < ngr; x += blockDim.x) {
        const float mine = w[x];
        int rank = 0;
        for (int u = 0; u < ngr; ++u) {
            const float o = w[u];
            rank += (o > mine || (o == mine && u < x)) ? 1 : 0;
        }
        P.gorder[rank] = x;
    }
}

__device__ __forceinline__ int gather_group(const Plan& P, int tid) {
    __shared__ float gw[kChunkThreads];
    __shared__ int s_bg;
    const int ngr = P.B * P.Hkv, y = blockIdx.y;
    if (ngr > kChunkThreads) return ngr <= kOrderMaxGroups ? P.gorder[y] : y;  // uniform over the grid
    if (tid == 0) s_bg = y;
    const float mine = tid < ngr ? __uint_as_float(P.gw[tid]) : 0.0f;
    if (tid < ngr) gw[tid] = mine;
    __syncthreads();
    if (tid < ngr) {  // thread tid ranks group tid
        int rank = 0;
        for (int u = 0; u < ngr; ++u) {
            const float o = gw[u];
            rank += (o > mine || (o == mine && u < tid)) ? 1 : 0;
        }
        if (rank == y) s_bg = tid;
    }
    __syncthreads();
    return s_bg;
}

template <int D, typename KVT, int G>
__global__ __launch_bounds__(kChunkThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_gather(Plan P) {
    constexpr int NW = kChunkThreads / 64;
    __shared__ uint32_t tmeta[kGatherChunk];
    __shared__ uint32_t trow[kGatherChunk];
    __shared__ float sp[G][kGatherChunk];  // scores, then weights
    __shared__ uint32_t wsum[NW];
    __shared__ HeadView hv[G];
    __shared__ float wred[NW][G];
    __shared__ float hmax[G], hsum[G];
    __shared__ int s_over;  // some member score exceeds its head's reference by kRescale
    __shared__ int wfin[NW];
    static_assert(NW * D <= kGatherChunk, "per-wave sums fit in the weight array");
    float (*wacc)[G][D] = reinterpret_cast<float (*)[G][D]>(&sp[0][0]);  // reuses sp after the V pass
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int lane = tid & 63, wave = tid >> 6, nwaves = nthr >> 6;
    const int bg = gather_group(P, tid), b = bg / P.Hkv, g = bg % P.Hkv, c = blockIdx.x;
    const int L = P.seq_lens[b];
    const int T0 = c * P.cg;
    if (T0 >= L) return;
    if (tid == 0) s_over = 0;
    const Regions R = regions(P, L);
    const size_t bh0 = static_cast<size_t>(b) * P.Hq + g * G;
    // the row passes walk the member list from a block-dependent start
    // (cyclically): with the pages of the sequences laid out alike, blocks that
    // run together would otherwise read rows at the same page offsets in step
    const int rot = static_cast<int>(((static_cast<uint32_t>(c) * 2654435761u) ^ (static_cast<uint32_t>(bg) * 40503u)) >> 22);
    // the heads' state, the quad's page, sample words and each head's bitmap
    // word are requested together
    if (tid < G) {
        const HeadState& s = P.hs[bh0 + tid];
        hv[tid] = HeadView{s.thr_b, s.thr_n, s.nb, s.n, s.wsamp, s.m};
    }
    const int T1 = min(T0 + P.cg, L);
    const int qd = (T0 >> 2) + tid;
    const bool live4 = 4 * qd < T1;
    const int32_t* btrow = P.bt + static_cast<size_t>(b) * P.max_blocks;
    const uint32_t row0 = live4 ? (static_cast<uint32_t>(btrow[qd >> 2]) * P.Hkv + g) * kPage : 0u;
    const bool anyM = live4 && 4 * qd + 3 >= R.lo && 4 * qd < R.hi;
    const uint4 w = anyM ? quad_words(static_cast<uint32_t>(qd), g, b, P.seed_lo, P.seed_hi) : make_uint4(0, 0, 0, 0);
    uint32_t fw[G];
#pragma unroll
    for (int h = 0; h < G; ++h) fw[h] = live4 ? P.bits[(bh0 + h) * P.words + (qd >> 3)] : 0u;
    __syncthreads();

    // membership: meta = final mask | fixed mask << 8 | score cached << 16.
    // "Cached" is the base pass's own membership test (fixed, or base sample,
    // for some head of the group), so the cached tokens of the chunk, ascending,
    // are exactly the base pass's list and a cached token's scores sit at its
    // rank among them.  Every cached token is listed, even one that no head's
    // final set holds (a forced budget below the base sample): it then carries
    // weight 0.
    uint32_t m4[4] = {0, 0, 0, 0};
    uint32_t mine = 0;
    if (live4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 4 * qd + e;
            const bool inM = i >= R.lo && i < R.hi && i < T1;
            const uint64_t key = sample_key(word_of(w, e), static_cast<uint32_t>(i));
            uint32_t fin = 0, fxm = 0, cached = 0;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const bool fx = i < T1 && ((fw[h] >> (i & 31)) & 1u);
                const bool tail = inM && !fx;
                const bool sn = tail && hv[h].n > 0 && key >= hv[h].thr_n;
                const bool sb = tail && hv[h].nb > 0 && key >= hv[h].thr_b;
                fin |= (fx || sn) ? (1u << h) : 0u;
                fxm |= fx ? (1u << h) : 0u;
                cached |= (fx || sb) ? 1u : 0u;
            }
            m4[e] = (fin || cached) ? (fin | (fxm << 8) | (cached << 16)) : 0u;
            mine += cached ? 0x10000u : (fin ? 1u : 0u);  // uncached count | cached count << 16
        }
    }
    // list: the members whose scores still need their K rows first, [0, nu),
    // then the cached tokens in the base pass's order, [nu, n); both counts fit
    // 16 bits
    uint32_t cnt;
    const uint32_t pre = block_excl_scan(mine, wsum, cnt);
    const int nu = static_cast<int>(cnt & 0xFFFFu);
    uint32_t pu = pre & 0xFFFFu, pc = static_cast<uint32_t>(nu) + (pre >> 16);
    int nfin = 0;  // members of some head's final set, for the byte accounting
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (m4[e]) {
            const uint32_t pos = ((m4[e] >> 16) & 1u) ? pc++ : pu++;
            tmeta[pos] = m4[e];
            trow[pos] = row0 + ((4 * qd + e) & (kPage - 1));
            nfin += (m4[e] & 0xFFu) ? 1 : 0;
        }
    const int n = nu + static_cast<int>(cnt >> 16);
    if (P.gcounts) {  // block-uniform: one atomic per block, after the barrier below
        for (int o = 32; o >= 1; o >>= 1) nfin += __shfl_xor(nfin, o, 64);
        if (lane == 0) wfin[wave] = nfin;
    }
    __syncthreads();
    if (P.gcounts && tid == 0) {
        int t = 0;
        for (int w2 = 0; w2 < NW; ++w2) t += wfin[w2];
        if (t) atomicAdd(&P.gcounts[2 * bg], t);
    }

    // (1) scores into LDS (-inf for heads the token does not belong to).
    // Tokens of the base pass take their pinned scores from its list (entry
    // x - nu, contiguous loads, one pass); the others are scored from their K
    // rows below.
    constexpr int LPT = D / 8, TPW = 64 / LPT;
    const int j = lane % LPT, slot = lane / LPT;
    const float* bsc = P.bsc + (static_cast<size_t>(bg) * P.ncg + c) * P.cg * G;
    const KVT* kbase = static_cast<const KVT*>(P.k);
    {
        constexpr int PER = kGatherChunk / kChunkThreads;  // list entries per thread
        float v[PER][G];
        uint32_t mm[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int x = nu + tid + e * nthr;
            mm[e] = x < n ? tmeta[x] : 0u;
            const size_t at = static_cast<size_t>(x < n ? x - nu : 0);
#pragma unroll
            for (int h = 0; h < G; ++h) v[e][h] = x < n ? bsc[static_cast<size_t>(h) * P.cg + at] : 0.0f;
        }
        bool over = false;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int x = nu + tid + e * nthr;
            if ((mm[e] >> 16) & 1u) {
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const bool mem = (mm[e] >> h) & 1u;
                    over |= mem && v[e][h] > hv[h].m + kRescale;
                    sp[h][x] = mem ? v[e][h] : -__builtin_inff();
                }
            }
        }
        if (over) s_over = 1;
    }
    {
        // LPT lanes per K row (8 elements each), the G pinned-order sums
        // spread over the row's lanes; each batch of rows is requested before
        // any is scored
        using SP = Spread<G, LPT>;
        constexpr int NH = SP::NH, KU = kGatherUnrollK;
        const bool fin = SP::finisher(j);
        int hsel[NH];
#pragma unroll
        for (int e = 0; e < NH; ++e) hsel[e] = SP::head(j, e);
        float qreg[G][8];
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) qreg[h][e] = P.q[(bh0 + h) * D + 8 * j + e] * P.scale32;
        bool over = false;
        const int rk = nu > 0 ? rot % nu : 0;
        for (int base = wave * TPW * KU; base < nu; base += nwaves * TPW * KU) {
            Raw8 kr[KU];
            uint32_t mk[KU];
#pragma unroll
            for (int u = 0; u < KU; ++u) {
                const int x = base + u * TPW + slot;
                const int xr = x < nu ? (x + rk < nu ? x + rk : x + rk - nu) : 0;
                mk[u] = x < nu ? tmeta[xr] : 0u;
                load_raw_nt(kbase + static_cast<size_t>(trow[xr]) * D + 8 * j, kr[u]);
            }
#pragma unroll
            for (int u = 0; u < KU; ++u) {
                float kf[8];
                widen<KVT>(kr[u], kf);
                float part[G], sv[NH];
#pragma unroll
                for (int h = 0; h < G; ++h) part[h] = chain8(qreg[h], kf);
                spread_across_lanes<G, LPT>(part, sv, j);
                const int x = base + u * TPW + slot;
                const int xr = x + rk < nu ? x + rk : x + rk - nu;
                if (fin && x < nu) {
#pragma unroll
                    for (int e = 0; e < NH; ++e) {
                        const int h = hsel[e];
                        const bool mem = (mk[u] >> h) & 1u;
                        over |= mem && sv[e] > hv[h].m + kRescale;
                        sp[h][xr] = mem ? sv[e] : -__builtin_inff();
                    }
                }
            }
        }
        if (over) s_over = 1;
    }
    __syncthreads();
    // weights against each head's base-pass maximum (the pinned maximum over
    // its fixed set and base sample); only when some score here exceeds that
    // by more than kRescale is the block's own maximum taken instead
    {
        if (s_over) {  // block-uniform: read after the barrier closing the score pass
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
        } else if (tid < G) {
            hmax[tid] = hv[tid].m;
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

    // (2) sum_i p_i V_i over the V rows
    float acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    {
        // eight heads keep 8 x 8 accumulators per lane: 4 rows per batch keep the
        // kernel at 3 waves per SIMD (146 VGPRs; 6 rows take 182, 2 waves)
        constexpr int VU = G == 8 ? 4 : kGatherUnrollV;
        const KVT* vbase = static_cast<const KVT*>(P.v);
        struct VBatch {
            Raw8 vr[VU];
            int x0;
        };
        // rows past the list end reread the last row with weight 0 (no branches)
        const int rv = n > 0 ? rot % n : 0;
        auto issue = [&](VBatch& bt, int b0) __attribute__((always_inline)) {
            bt.x0 = b0;
#pragma unroll
            for (int u = 0; u < VU; ++u) {
                const int x = b0 + u * TPW + slot;
                const int xc = x < n ? (x + rv < n ? x + rv : x + rv - n) : n - 1;
                load_raw_nt(vbase + static_cast<size_t>(trow[xc]) * D + 8 * j, bt.vr[u]);
            }
        };
        auto accumulate = [&](const VBatch& bt) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < VU; ++u) {
                const int x = bt.x0 + u * TPW + slot;
                const int xc = x < n ? (x + rv < n ? x + rv : x + rv - n) : n - 1;
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
        // one batch of VU rows per lane group per iteration, all
        // requested before any is accumulated (rows past the end reread the
        // last row with weight 0)
        for (int b0 = wave * TPW * VU; b0 < n; b0 += nwaves * TPW * VU) {
            VBatch bt;
            issue(bt, b0);
            accumulate(bt);
        }
    }
    // token slots of the wave hold the same dims: plain sums
#pragma unroll
    for (int o = LPT; o < 64; o <<= 1)
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] += __shfl_xor(acc[h][e], o, 64);
    __syncthreads();  // every wave is done with the weights before their space is reused
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
// 1024 threads: the weighted sum over chunks takes one round of loads per
// thread for up to 64 chunks at d = 128 (8 groups of chunks per dimension)
constexpr int kCombineThreads = 1024;

template <int kThreads>  // per block
__global__ __launch_bounds__(kThreads) void k_combine(Plan P) {
    constexpr int NW = kThreads / 64;
    constexpr int U = 8;  // chunk loads in flight per thread
    __shared__ float wsh[kMaxChunks];
    __shared__ float rm[NW], rl[NW];
    __shared__ float accs[kThreads];
    const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63, wave = tid >> 6;
    const int bh = blockIdx.x, b = bh / P.Hq;
    const int D = P.d, ncg = P.ncg;
    const float* pp = P.part + static_cast<size_t>(bh) * ncg * (D + 2);
    // nthr / D groups of chunks per dimension
    const int ngrp = nthr / D, e = tid % D, grp = tid / D;
    // one round of loads at entry: the sequence length, this thread's chunk
    // maximum and sum, the first U chunks' partial sums of its dimension and
    // the head state (slots past the sequence's chunks hold stale values, which
    // are dropped once its length is known)
    const int L = P.seq_lens[b];
    const float m0 = tid < ncg ? pp[static_cast<size_t>(tid) * (D + 2)] : -__builtin_inff();
    const float l0 = tid < ncg ? pp[static_cast<size_t>(tid) * (D + 2) + 1] : 0.0f;
    float v0[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = grp + u * ngrp;
        v0[u] = c < ncg ? pp[static_cast<size_t>(c) * (D + 2) + 2 + e] : 0.0f;
    }
    HeadState hs{};
    if (tid == 0) hs = P.hs[bh];
    const int nc = (L + P.cg - 1) / P.cg;
    float mloc = tid < nc ? m0 : -__builtin_inff();
    for (int c = tid + nthr; c < nc; c += nthr) mloc = fmaxf(mloc, pp[static_cast<size_t>(c) * (D + 2)]);
    for (int o = 1; o < 64; o <<= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, o, 64));
    if (lane == 0) rm[wave] = mloc;
    __syncthreads();
    float M = -__builtin_inff();
    for (int w = 0; w < NW; ++w) M = fmaxf(M, rm[w]);
    float lloc = 0.f;
    for (int c = tid; c < nc; c += nthr) {
        const float mc = c == tid ? m0 : pp[static_cast<size_t>(c) * (D + 2)];
        const float lc = c == tid ? l0 : pp[static_cast<size_t>(c) * (D + 2) + 1];
        const float wgt = (M == -__builtin_inff()) ? 0.0f : __expf(mc - M);
        wsh[c] = wgt;
        lloc += wgt * lc;
    }
    for (int o = 1; o < 64; o <<= 1) lloc += __shfl_xor(lloc, o, 64);
    if (lane == 0) rl[wave] = lloc;
    __syncthreads();
    float l = 0.f;
    for (int w = 0; w < NW; ++w) l += rl[w];
    const bool ok = M != -__builtin_inff() && l > 0.f;
    float a = 0.f;
    for (int c0 = grp; c0 < nc; c0 += U * ngrp) {
        float v[U], wv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u * ngrp;
            v[u] = c < nc ? (c0 == grp ? v0[u] : pp[static_cast<size_t>(c) * (D + 2) + 2 + e]) : 0.f;
            wv[u] = c < nc ? wsh[c] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) a = __builtin_fmaf(wv[u], v[u], a);
    }
    accs[tid] = a;
    __syncthreads();
    if (tid < D) {
        float t = 0.f;
        for (int gi = 0; gi < ngrp; ++gi) t += accs[gi * D + tid];
        P.out[static_cast<size_t>(bh) * D + tid] = ok ? t / l : 0.0f;
    }
    if (tid == 0) {
        P.lse[bh] = ok ? M + __logf(l) : -__builtin_inff();
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
template <int kThreads>  // per block
__global__ __launch_bounds__(kThreads) void k_emit(Plan P) {
    // A span of 4 * kEmitQuads * kThreads tokens is one pass: wave w owns
    // quads [w * 64 * kEmitQuads, (w + 1) * 64 * kEmitQuads) of it and lane l
    // the quads l + 64 k (coalesced loads), so the wave's tokens ascend in
    // (k, lane) order; one wave prefix sum per k and one block scan of the
    // wave totals place every member.
    constexpr int NW = kThreads / 64, KQ = kEmitQuads, SPAN = 4 * KQ * kThreads;
    __shared__ uint32_t wtot[NW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bh = blockIdx.x, b = bh / P.Hq, h = bh % P.Hq;
    const int G = P.G, g = h / G;
    const int L = P.seq_lens[b];
    const Regions R = regions(P, L);
    const HeadState hs = P.hs[bh];
    const uint32_t* bits = P.bits + static_cast<size_t>(bh) * P.words;
    int32_t* out = P.idx + static_cast<size_t>(bh) * P.idx_cap;
    const int cap = P.idx_cap;
    int written = 0;
    for (int S0 = 0; S0 < L; S0 += SPAN) {
        const int q0 = (S0 >> 2) + wave * 64 * KQ + lane;
        uint4 w[KQ];
        uint32_t fw[KQ];
#pragma unroll
        for (int k = 0; k < KQ; ++k) {  // every load of the span first
            const int qd = q0 + 64 * k;
            const bool live = 4 * qd < L;
            const bool anyM = live && 4 * qd + 3 >= R.lo && 4 * qd < R.hi;
            w[k] = anyM ? quad_words(static_cast<uint32_t>(qd), g, b, P.seed_lo, P.seed_hi) : make_uint4(0, 0, 0, 0);
            fw[k] = live ? bits[qd >> 3] : 0u;
        }
        uint32_t m[KQ], ex[KQ], run = 0;
#pragma unroll
        for (int k = 0; k < KQ; ++k) {
            const int qd = q0 + 64 * k;
            uint32_t mk = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * qd + e;
                const bool fx = i < L && ((fw[k] >> (i & 31)) & 1u);
                const bool inM = i >= R.lo && i < R.hi;
                const bool sn = inM && !fx && hs.n > 0 &&
                                sample_key(word_of(w[k], e), static_cast<uint32_t>(i)) >= hs.thr_n;
                mk |= (fx || sn) ? (1u << e) : 0u;
            }
            m[k] = mk;
            const uint32_t c = static_cast<uint32_t>(__builtin_popcount(mk));
            const uint32_t inc = wave_incl_scan(c);
            ex[k] = run + inc - c;
            run += static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(inc), 63));
        }
        if (lane == 0) wtot[wave] = run;
        __syncthreads();
        uint32_t woff = 0, stot = 0;
#pragma unroll
        for (int x = 0; x < NW; ++x) {
            const uint32_t t = wtot[x];
            woff += x < wave ? t : 0u;
            stot += t;
        }
        __syncthreads();  // the totals are rewritten by the next span
#pragma unroll
        for (int k = 0; k < KQ; ++k) {
            uint32_t pos = static_cast<uint32_t>(written) + woff + ex[k];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if ((m[k] >> e) & 1u) {
                    if (pos < static_cast<uint32_t>(cap)) out[pos] = 4 * (q0 + 64 * k) + e;
                    ++pos;
                }
        }
        written += static_cast<int>(stot);
    }
    written = min(written, cap);
    for (int x = written + tid; x < cap; x += kThreads) out[x] = -1;
}

// ===========================================================================
// low-rank key projection: Kt = bf16(pdot(K_i, P[:, j]))
// ===========================================================================
template <typename KVT, int D, int RK>
__global__ __launch_bounds__(256) void k_project(const KVT* __restrict__ k, const float* __restrict__ proj,
                                                 uint16_t* __restrict__ kt, long long nrows, int Hkv,
                                                 int proj_stride) {
    constexpr int RPB = 256 / RK;  // rows per block, all of one (page, KV head): RPB divides 16
    static_assert(kPage % RPB == 0, "a block's rows share their KV head");
    __shared__ float ps[D * RK];
    __shared__ float kr[RPB][D];
    const long long r0 = static_cast<long long>(blockIdx.x) * RPB;
    const float* pg = proj + static_cast<size_t>((r0 / kPage) % Hkv) * proj_stride;  // the head's basis
    for (int x = threadIdx.x; x < D * RK; x += 256) ps[x] = pg[x];
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
// key signatures: bit j of S_i is pdot(K_i, P[:, j]) > 0 for the 32 columns of
// P, with the pdot of the projection above.  A block holds 8 rows of one
// (page, KV head); a wave's 64 lanes are the 32 hyperplanes of two rows, so
// one ballot forms both signatures.
// ===========================================================================
template <typename KVT, int D>
__global__ __launch_bounds__(256) void k_sign(const KVT* __restrict__ k, const float* __restrict__ proj,
                                              uint32_t* __restrict__ ksig, long long nrows, int Hkv,
                                              int proj_stride) {
    constexpr int RPB = 8;
    static_assert(kPage % RPB == 0, "a block's rows share their KV head");
    __shared__ float ps[D * 32];
    __shared__ float kr[RPB][D];
    const long long r0 = static_cast<long long>(blockIdx.x) * RPB;
    const float* pg = proj + static_cast<size_t>((r0 / kPage) % Hkv) * proj_stride;  // the head's hyperplanes
    for (int x = threadIdx.x; x < D * 32; x += 256) ps[x] = pg[x];
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
    const int rr = threadIdx.x / 32, jj = threadIdx.x % 32;
    const long long row = r0 + rr;
    const float s = pdot_serial<D>(kr[rr], 1, ps + jj, 32);
    const uint64_t m = __ballot(s > 0.0f);  // every lane takes part
    if (jj == 0 && row < nrows) ksig[row] = static_cast<uint32_t>(m >> (32 * (rr & 1)));
}

// ===========================================================================
// append: the newest token of each sequence into the paged caches, with its
// low-rank key row (same pdot and rounding as the projection above)
// ===========================================================================
template <typename KVT, int D, int RK>
__global__ __launch_bounds__(64) void k_append(const KVT* __restrict__ k_new, const KVT* __restrict__ v_new,
                                               const int32_t* __restrict__ pos, const int32_t* __restrict__ bt,
                                               int max_blocks, int Hkv, KVT* __restrict__ kc, KVT* __restrict__ vc,
                                               uint16_t* __restrict__ kt, uint32_t* __restrict__ ksig,
                                               const float* __restrict__ proj, int proj_stride) {
    __shared__ float kr[D];
    const int bg = blockIdx.x, b = bg / Hkv, g = bg % Hkv, lane = threadIdx.x;
    const int p = pos[b];
    if (p < 0) return;
    const long long row = (static_cast<long long>(bt[static_cast<size_t>(b) * max_blocks + p / kPage]) * Hkv + g) *
                              kPage + p % kPage;
    const KVT* ks = k_new + static_cast<size_t>(bg) * D;
    const KVT* vs = v_new + static_cast<size_t>(bg) * D;
    for (int e = lane; e < D; e += 64) {
        const KVT kv = ks[e];
        kc[row * D + e] = kv;
        vc[row * D + e] = vs[e];
        if constexpr (sizeof(KVT) == 2) {
            kr[e] = __uint_as_float(static_cast<uint32_t>(reinterpret_cast<const uint16_t&>(kv)) << 16);
        } else {
            kr[e] = kv;
        }
    }
    if (kt == nullptr && ksig == nullptr) return;  // block-uniform
    __syncthreads();
    if (ksig != nullptr) {  // signature: lanes 0..31 test one hyperplane each
        const float s = lane < 32 ? pdot_serial<D>(kr, 1, proj + static_cast<size_t>(g) * proj_stride + lane, 32)
                                  : 0.0f;
        const uint64_t m = __ballot(s > 0.0f);
        if (lane == 0) ksig[row] = static_cast<uint32_t>(m);
        return;
    }
    for (int j = lane; j < RK; j += 64) {
        const float s = pdot_serial<D>(kr, 1, proj + static_cast<size_t>(g) * proj_stride + j, RK);
        uint32_t u = __float_as_uint(s);
        u += 0x7FFFu + ((u >> 16) & 1u);  // round to nearest even
        kt[row * RK + j] = static_cast<uint16_t>(u >> 16);
    }
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

// Status of the launch just enqueued (clears it): every stage is checked
// before a kernel that consumes its output is enqueued.
static int launched() { return static_cast<int>(hipGetLastError()); }

template <int D, typename KVT, int G>
static int launch_chunk_kernels(const Plan& p, hipStream_t st, const Marks& mk) {
    const dim3 grid_c(p.ncg, p.B * p.Hkv);         // (chunk, group)
    const dim3 grid_h(p.Hkv, p.ncg, p.B);          // (KV head, chunk, sequence)
    int rc = 0;
    hipLaunchKernelGGL((k_base<D, KVT, G>), grid_h, dim3(kChunkThreads), 0, st, p);
    if ((rc = launched()) || (rc = mk.mark(3))) return rc;
    // with many heads the per-head kernels run smaller blocks, several per CU
    const bool many = p.B * p.Hq >= kManyHeads;
    if (p.guarantee == 0) {
        if (many)
            hipLaunchKernelGGL((k_budget<kHeadThreadsMany, false>), dim3(p.B * p.Hq), dim3(kHeadThreadsMany), 0, st, p);
        else
            hipLaunchKernelGGL((k_budget<kBudgetThreads, false>), dim3(p.B * p.Hq), dim3(kBudgetThreads), 0, st, p);
        if ((rc = launched())) return rc;
    } else {  // output-level mode: statistics, numerator partials, then the budget
        if (many)
            hipLaunchKernelGGL((k_budget<kHeadThreadsMany, true>), dim3(p.B * p.Hq), dim3(kHeadThreadsMany), 0, st, p);
        else
            hipLaunchKernelGGL((k_budget<kBudgetThreads, true>), dim3(p.B * p.Hq), dim3(kBudgetThreads), 0, st, p);
        if ((rc = launched())) return rc;
        hipLaunchKernelGGL((k_numstat<D, KVT, G>), grid_h, dim3(kChunkThreads), 0, st, p);
        if ((rc = launched())) return rc;
        if (many)
            hipLaunchKernelGGL(k_budget_num<kHeadThreadsMany>, dim3(p.B * p.Hq), dim3(kHeadThreadsMany), 0, st, p);
        else
            hipLaunchKernelGGL(k_budget_num<kBudgetThreads>, dim3(p.B * p.Hq), dim3(kBudgetThreads), 0, st, p);
        if ((rc = launched())) return rc;
    }
    if ((rc = mk.mark(4))) return rc;
    const int ngr = p.B * p.Hkv;
    if (ngr > kChunkThreads && ngr <= kOrderMaxGroups) {
        hipLaunchKernelGGL(k_order, dim3(1), dim3(kOrderThreads), 0, st, p);
        if ((rc = launched())) return rc;
    }
    hipLaunchKernelGGL((k_gather<D, KVT, G>), grid_c, dim3(kChunkThreads), 0, st, p);
    if ((rc = launched())) return rc;
    return mk.mark(5);
}

template <int ROW, typename T, int G>
static int launch_predict(const Plan& p, hipStream_t st) {
    const size_t lds = predict_lds_bytes(G, p.d, ROW, p.cp);
    auto kern = k_predict<ROW, T, G>;
    // the dynamic LDS limit is raised once per kernel instance and device; the
    // flags are atomics so concurrent callers on several host threads are safe
    // (setting the attribute twice is harmless)
    constexpr int kDevices = 64;
    static std::atomic<bool> attr_set[kDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    if (dev >= kDevices || !attr_set[dev].load(std::memory_order_acquire)) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
        if (e != hipSuccess) return static_cast<int>(e);
        if (dev < kDevices) attr_set[dev].store(true, std::memory_order_release);
    }
    hipLaunchKernelGGL(kern, dim3(p.ncp, p.B * p.Hkv), dim3(kPredThreads), lds, st, p);
    return launched();
}

template <int G>
static int launch_g(const Plan& p, hipStream_t st, const Marks& mk) {
    int rc = 0;
    if ((rc = mk.mark(0))) return rc;
    // 1. predictor + chunk candidates
    if (p.predictor == 2) {
        rc = launch_predict<32, uint32_t, G>(p, st);
    } else if (p.predictor == 1) {
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
    const bool lds_bits = p.words <= kSelLdsWords;
    if (p.nparts > 0) {
        hipLaunchKernelGGL(k_premerge, dim3(p.B * p.Hq, p.nparts), dim3(kSelectThreads), 0, st, p);
        if ((rc = launched())) return rc;
        if (lds_bits) hipLaunchKernelGGL((k_select<true, true>), dim3(p.B * p.Hq), dim3(kSelectThreads), 0, st, p);
        else hipLaunchKernelGGL((k_select<true, false>), dim3(p.B * p.Hq), dim3(kSelectThreads), 0, st, p);
    } else {
        const dim3 blk(p.B * p.Hq >= kManyHeads ? kHeadThreadsMany : kSelectThreads);
        if (lds_bits) hipLaunchKernelGGL((k_select<false, true>), dim3(p.B * p.Hq), blk, 0, st, p);
        else hipLaunchKernelGGL((k_select<false, false>), dim3(p.B * p.Hq), blk, 0, st, p);
    }
    if ((rc = launched()) || (rc = mk.mark(2))) return rc;
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
    // an error the calling thread left pending is reported, not taken for one
    // of this call's launches, and nothing is enqueued behind it
    int rc = static_cast<int>(hipPeekAtLastError());
    if (rc) return rc;
    switch (p.G) {
        case 1: rc = launch_g<1>(p, st, mk); break;
        case 2: rc = launch_g<2>(p, st, mk); break;
        case 4: rc = launch_g<4>(p, st, mk); break;
        default: rc = launch_g<8>(p, st, mk); break;
    }
    if (rc) return rc;
    if (p.B * p.Hq >= kManyHeads)
        hipLaunchKernelGGL(k_combine<kHeadThreadsMany>, dim3(p.B * p.Hq), dim3(kHeadThreadsMany), 0, st, p);
    else
        hipLaunchKernelGGL(k_combine<kCombineThreads>, dim3(p.B * p.Hq), dim3(kCombineThreads), 0, st, p);
    if ((rc = launched()) || (rc = mk.mark(6))) return rc;
    if (p.idx) {
        if (p.B * p.Hq >= kManyHeads)
            hipLaunchKernelGGL(k_emit<kHeadThreadsMany>, dim3(p.B * p.Hq), dim3(kHeadThreadsMany), 0, st, p);
        else
            hipLaunchKernelGGL(k_emit<kEmitThreads>, dim3(p.B * p.Hq), dim3(kEmitThreads), 0, st, p);
        if ((rc = launched())) return rc;
    }
    return mk.mark(7);
}

// ===========================================================================
// key Gram matrices: gram[g] = sum over every cached token of K K^T (fp32),
// from which a caller takes a KV head's predictor basis (its leading
// eigenvectors).  A dense contraction over tokens, so on the matrix cores:
// one block per (sequence, KV head, chunk of kGramChunk tokens) stages
// kGramTile tokens at a time feature-major in LDS and accumulates the d x d
// product in 16 x 16 tiles; a second pass sums the chunk partials in a fixed
// order, so the result does not depend on scheduling.
// ===========================================================================
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

template <int D>
__global__ __launch_bounds__(256) void k_gram_part(const uint16_t* __restrict__ k, const int32_t* __restrict__ bt,
                                                   const int32_t* __restrict__ seq_lens, int max_blocks, int Hkv,
                                                   int nchunk, float* __restrict__ part) {
    constexpr int NT = D / 16;   // 16 x 16 output tiles per side
    constexpr int RPW = NT / 4;  // tile rows per wave (4 waves)
    constexpr int RS = kGramTile + 8;  // LDS row stride (elements), 16-byte aligned rows
    __shared__ __align__(16) __bf16 kf[D * RS];  // [feature][token]
    __shared__ int32_t pgs[kGramChunk / kPage];  // the chunk's page ids
    const int c = blockIdx.x, bg = blockIdx.y, b = bg / Hkv, g = bg % Hkv;
    const int L = min(seq_lens[b], max_blocks * kPage);  // never past the block-table row
    const int t0 = c * kGramChunk;
    if (t0 >= L) return;  // block-uniform; the reduction skips this partial
    const int t1 = min(t0 + kGramChunk, L);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    f32x4_t acc[RPW][NT];
#pragma unroll
    for (int ri = 0; ri < RPW; ++ri)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[ri][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int32_t* btrow = bt + static_cast<size_t>(b) * max_blocks;
    for (int x = tid; x < kGramChunk / kPage; x += 256)
        if (t0 + x * kPage < t1) pgs[x] = btrow[t0 / kPage + x];
    __syncthreads();
    // staging: a thread takes 4 consecutive tokens x 8 features (four 16-byte
    // row pieces) per pair and writes each feature's 4 tokens as one 8-byte
    // word; the next tile's pieces are requested before the current tile's
    // products, so the loads overlap the matrix work
    constexpr int OCT = D / 8;                          // feature octets per token
    constexpr int PAIRS = (kGramTile / 4) * OCT / 256;  // (token quad, octet) pairs per thread
    static_assert(PAIRS >= 1 && (kGramTile / 4) * OCT % 256 == 0, "whole pairs per thread");
    uint4 pre[PAIRS][4];
    auto fetch = [&](int ts) __attribute__((always_inline)) {
#pragma unroll
        for (int pi = 0; pi < PAIRS; ++pi) {
            const int pr = tid + 256 * pi, tq = pr / OCT, fo = pr % OCT;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int t = ts + 4 * tq + u;
                pre[pi][u] = make_uint4(0, 0, 0, 0);
                if (t < t1) {
                    const size_t row = (static_cast<size_t>(pgs[(t - t0) / kPage]) * Hkv + g) * kPage + (t % kPage);
                    pre[pi][u] = *reinterpret_cast<const uint4*>(k + row * D + 8 * fo);
                }
            }
        }
    };
    fetch(t0);
    for (int ts = t0; ts < t1; ts += kGramTile) {
#pragma unroll
        for (int pi = 0; pi < PAIRS; ++pi) {
            const int pr = tid + 256 * pi, tq = pr / OCT, fo = pr % OCT;
            const uint32_t w[4][4] = {{pre[pi][0].x, pre[pi][0].y, pre[pi][0].z, pre[pi][0].w},
                                      {pre[pi][1].x, pre[pi][1].y, pre[pi][1].z, pre[pi][1].w},
                                      {pre[pi][2].x, pre[pi][2].y, pre[pi][2].z, pre[pi][2].w},
                                      {pre[pi][3].x, pre[pi][3].y, pre[pi][3].z, pre[pi][3].w}};
#pragma unroll
            for (int q = 0; q < 8; ++q) {  // feature 8 fo + q of tokens 4 tq .. 4 tq + 3
                const int sh = 16 * (q & 1);
                const uint32_t lo = ((w[0][q >> 1] >> sh) & 0xFFFFu) | (((w[1][q >> 1] >> sh) & 0xFFFFu) << 16);
                const uint32_t hi = ((w[2][q >> 1] >> sh) & 0xFFFFu) | (((w[3][q >> 1] >> sh) & 0xFFFFu) << 16);
                *reinterpret_cast<uint2*>(&kf[(8 * fo + q) * RS + 4 * tq]) = make_uint2(lo, hi);
            }
        }
        __syncthreads();
        if (ts + kGramTile < t1) fetch(ts + kGramTile);  // block-uniform
        // 32 tokens per step: lane l gives row l % 16 of a tile, tokens
        // 8 (l / 16) .. + 8 (one 16-byte LDS read per operand)
        for (int ks = 0; ks < kGramTile; ks += 32) {
            const int tk = ks + 8 * (lane / 16), fr = lane % 16;
            bf16x8_t bop[NT];
#pragma unroll
            for (int j = 0; j < NT; ++j) bop[j] = *reinterpret_cast<const bf16x8_t*>(&kf[(16 * j + fr) * RS + tk]);
#pragma unroll
            for (int ri = 0; ri < RPW; ++ri) {
                const int i = wave * RPW + ri;
                const bf16x8_t aop = *reinterpret_cast<const bf16x8_t*>(&kf[(16 * i + fr) * RS + tk]);
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    acc[ri][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, bop[j], acc[ri][j], 0, 0, 0);
            }
        }
        __syncthreads();  // the tile is restaged
    }
    // tile (i, j): lane l holds rows 16 i + 4 (l / 16) + r, column 16 j + l % 16
    float* out = part + (static_cast<size_t>(bg) * nchunk + c) * D * D;
#pragma unroll
    for (int ri = 0; ri < RPW; ++ri)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                out[(16 * (wave * RPW + ri) + 4 * (lane / 16) + r) * D + 16 * j + lane % 16] = acc[ri][j][r];
}

// gram[g][e] = sum over sequences b, then chunks c (ascending) of the partials
__global__ __launch_bounds__(256) void k_gram_reduce(const float* __restrict__ part, const int32_t* __restrict__ seq_lens,
                                                     int B, int Hkv, int nchunk, int DD, float* __restrict__ gram) {
    const int e = blockIdx.x * 256 + threadIdx.x, g = blockIdx.y;
    if (e >= DD) return;
    float s = 0.f;
    for (int b = 0; b < B; ++b) {
        const int nc = min((seq_lens[b] + kGramChunk - 1) / kGramChunk, nchunk);
        const float* pp = part + (static_cast<size_t>(b) * Hkv + g) * nchunk * DD + e;
        for (int c = 0; c < nc; ++c) s += pp[static_cast<size_t>(c) * DD];
    }
    gram[static_cast<size_t>(g) * DD + e] = s;
}

int launch_gram(const uint16_t* k_cache, const int32_t* bt, const int32_t* seq_lens, int B, int max_blocks,
                int Hkv, int d, int max_seq_len, float* gram, float* part, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (const int rc = static_cast<int>(hipPeekAtLastError())) return rc;  // pending from the caller
    const int nchunk = (max_seq_len + kGramChunk - 1) / kGramChunk;
    const dim3 grid(static_cast<unsigned>(nchunk), static_cast<unsigned>(B * Hkv));
    if (d == 128)
        hipLaunchKernelGGL(k_gram_part<128>, grid, dim3(256), 0, st, k_cache, bt, seq_lens, max_blocks, Hkv, nchunk, part);
    else
        hipLaunchKernelGGL(k_gram_part<64>, grid, dim3(256), 0, st, k_cache, bt, seq_lens, max_blocks, Hkv, nchunk, part);
    const int DD = d * d;
    hipLaunchKernelGGL(k_gram_reduce, dim3(static_cast<unsigned>((DD + 255) / 256), static_cast<unsigned>(Hkv)),
                       dim3(256), 0, st, part, seq_lens, B, Hkv, nchunk, DD, gram);
    return static_cast<int>(hipGetLastError());
}

template <typename KVT, int D>
static void launch_project_t(const void* k, const float* proj, uint16_t* kt, long long nrows, int r,
                             int Hkv, int proj_stride, hipStream_t st) {
    switch (r) {
        case 16: {
            const long long nb = (nrows + 15) / 16;
            hipLaunchKernelGGL((k_project<KVT, D, 16>), dim3(static_cast<unsigned>(nb)), dim3(256), 0, st,
                               static_cast<const KVT*>(k), proj, kt, nrows, Hkv, proj_stride);
            break;
        }
        case 32: {
            const long long nb = (nrows + 7) / 8;
            hipLaunchKernelGGL((k_project<KVT, D, 32>), dim3(static_cast<unsigned>(nb)), dim3(256), 0, st,
                               static_cast<const KVT*>(k), proj, kt, nrows, Hkv, proj_stride);
            break;
        }
        default: {
            const long long nb = (nrows + 3) / 4;
            hipLaunchKernelGGL((k_project<KVT, D, 64>), dim3(static_cast<unsigned>(nb)), dim3(256), 0, st,
                               static_cast<const KVT*>(k), proj, kt, nrows, Hkv, proj_stride);
            break;
        }
    }
}

int launch_project(const void* k_cache, int kv_bf16, const float* proj, int proj_stride, uint16_t* kt,
                   int num_blocks, int Hkv, int d, int r, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (const int rc = static_cast<int>(hipPeekAtLastError())) return rc;  // pending from the caller
    const long long nrows = static_cast<long long>(num_blocks) * Hkv * kPage;
    if (d == 128) {
        if (kv_bf16) launch_project_t<uint16_t, 128>(k_cache, proj, kt, nrows, r, Hkv, proj_stride, st);
        else launch_project_t<float, 128>(k_cache, proj, kt, nrows, r, Hkv, proj_stride, st);
    } else {
        if (kv_bf16) launch_project_t<uint16_t, 64>(k_cache, proj, kt, nrows, r, Hkv, proj_stride, st);
        else launch_project_t<float, 64>(k_cache, proj, kt, nrows, r, Hkv, proj_stride, st);
    }
    return static_cast<int>(hipGetLastError());
}

template <typename KVT, int D>
static void launch_append_t(const void* k_new, const void* v_new, const int32_t* pos, const int32_t* bt, int B,
                            int max_blocks, void* kc, void* vc, uint16_t* kt, uint32_t* ksig, const float* proj,
                            int proj_stride, int Hkv, int r, hipStream_t st) {
    const dim3 grid(static_cast<unsigned>(B * Hkv));
    const KVT* kn = static_cast<const KVT*>(k_new);
    const KVT* vn = static_cast<const KVT*>(v_new);
    KVT* kcc = static_cast<KVT*>(kc);
    KVT* vcc = static_cast<KVT*>(vc);
    switch (r) {
        case 16: hipLaunchKernelGGL((k_append<KVT, D, 16>), grid, dim3(64), 0, st, kn, vn, pos, bt, max_blocks, Hkv, kcc, vcc, kt, ksig, proj, proj_stride); break;
        case 32: hipLaunchKernelGGL((k_append<KVT, D, 32>), grid, dim3(64), 0, st, kn, vn, pos, bt, max_blocks, Hkv, kcc, vcc, kt, ksig, proj, proj_stride); break;
        default: hipLaunchKernelGGL((k_append<KVT, D, 64>), grid, dim3(64), 0, st, kn, vn, pos, bt, max_blocks, Hkv, kcc, vcc, kt, ksig, proj, proj_stride); break;
    }
}

int launch_append(const void* k_new, const void* v_new, const int32_t* pos, const int32_t* bt, int B,
                  int max_blocks, void* k_cache, void* v_cache, uint16_t* kt, uint32_t* ksig, const float* proj,
                  int proj_stride, int kv_bf16, int Hkv, int d, int r, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (const int rc = static_cast<int>(hipPeekAtLastError())) return rc;  // pending from the caller
    if (d == 128) {
        if (kv_bf16) launch_append_t<uint16_t, 128>(k_new, v_new, pos, bt, B, max_blocks, k_cache, v_cache, kt, ksig, proj, proj_stride, Hkv, r, st);
        else launch_append_t<float, 128>(k_new, v_new, pos, bt, B, max_blocks, k_cache, v_cache, kt, ksig, proj, proj_stride, Hkv, r, st);
    } else {
        if (kv_bf16) launch_append_t<uint16_t, 64>(k_new, v_new, pos, bt, B, max_blocks, k_cache, v_cache, kt, ksig, proj, proj_stride, Hkv, r, st);
        else launch_append_t<float, 64>(k_new, v_new, pos, bt, B, max_blocks, k_cache, v_cache, kt, ksig, proj, proj_stride, Hkv, r, st);
    }
    return static_cast<int>(hipGetLastError());
}

// ===========================================================================
// read-stream calibration: XOR of a buffer's words, every byte read once
// ===========================================================================
constexpr int kProbeUnroll = 4;  // 16-byte loads in flight per lane

__global__ __launch_bounds__(256) void k_read_probe(const uint4* __restrict__ buf, size_t n16, uint32_t* sink) {
    uint32_t acc = 0;
    const size_t stride = static_cast<size_t>(gridDim.x) * 256 * kProbeUnroll;
    for (size_t base = static_cast<size_t>(blockIdx.x) * 256 * kProbeUnroll + threadIdx.x; base < n16;
         base += stride) {
        uint4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const size_t i = base + static_cast<size_t>(u) * 256;
            v[u] = i < n16 ? nt_load16(buf + i) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (int o = 32; o >= 1; o >>= 1) acc ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), o, 64));
    // one atomic per block, spread over the sink's words (one address would
    // serialize them)
    __shared__ uint32_t wx[4];
    if ((threadIdx.x & 63) == 0) wx[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) atomicXor(sink + blockIdx.x % kProbeSink, wx[0] ^ wx[1] ^ wx[2] ^ wx[3]);
}

int launch_read_probe(const void* buf, size_t n16, uint32_t* sink, void* stream) {
    const size_t want = (n16 + 256 * kProbeUnroll - 1) / (256 * kProbeUnroll);
    const int grid = static_cast<int>(want < 4096 ? want : 4096);
    hipLaunchKernelGGL(k_read_probe, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4*>(buf), n16, sink);
    return launched();
}

int launch_sign(const void* k_cache, int kv_bf16, const float* proj, int proj_stride, uint32_t* ksig,
                int num_blocks, int Hkv, int d, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (const int rc = static_cast<int>(hipPeekAtLastError())) return rc;  // pending from the caller
    const long long nrows = static_cast<long long>(num_blocks) * Hkv * kPage;
    const dim3 grid(static_cast<unsigned>((nrows + 7) / 8));
    if (d == 128) {
        if (kv_bf16) hipLaunchKernelGGL((k_sign<uint16_t, 128>), grid, dim3(256), 0, st, static_cast<const uint16_t*>(k_cache), proj, ksig, nrows, Hkv, proj_stride);
        else hipLaunchKernelGGL((k_sign<float, 128>), grid, dim3(256), 0, st, static_cast<const float*>(k_cache), proj, ksig, nrows, Hkv, proj_stride);
    } else {
        if (kv_bf16) hipLaunchKernelGGL((k_sign<uint16_t, 64>), grid, dim3(256), 0, st, static_cast<const uint16_t*>(k_cache), proj, ksig, nrows, Hkv, proj_stride);
        else hipLaunchKernelGGL((k_sign<float, 64>), grid, dim3(256), 0, st, static_cast<const float*>(k_cache), proj, ksig, nrows, Hkv, proj_stride);
    }
    return static_cast<int>(hipGetLastError());
}

}  // namespace vattn
