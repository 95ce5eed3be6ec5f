// gfx950 kernels of the verified sparse-attention decode step.
//
// Pipeline for one step (one workgroup grid each, all on the caller's stream):
//   predict  (chunk, b*Hkv)  stream predictor keys of one context chunk, score
//                            the G query heads of the KV group, keep the chunk's
//                            top-k candidates per head (radix select in LDS)
//   select   (b*Hkv)         merge candidates into the exact top-k, write the
//                            fixed-set bitmap (sinks, window, top-k), pick the
//                            base sample threshold in the Philox order
//   base     (chunk, b*Hkv)  pinned exact scores of every token in the union of
//                            the group's fixed sets and base samples -> score
//                            cache; chunk maxima
//   budget   (b*Hkv)         exact fixed-point denominator statistics, CLT
//                            budget, final sample threshold
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

__device__ __forceinline__ bool bit_of(const uint32_t* row, int i) {
    return (row[i >> 5] >> (i & 31)) & 1u;
}

// Coherent (L2) read of a bitmap word written earlier in the same kernel.
__device__ __forceinline__ bool bit_of_coherent(const uint32_t* row, int i) {
    uint32_t* wp = const_cast<uint32_t*>(row + (i >> 5));
    const uint32_t w = __hip_atomic_load(wp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return (w >> (i & 31)) & 1u;
}

__device__ __forceinline__ const void* row_ptr(const void* base, size_t esize, int page, int Hkv,
                                               int g, int slot, int width) {
    const size_t off = ((static_cast<size_t>(page) * Hkv + g) * kPage + slot) * static_cast<size_t>(width);
    return static_cast<const char*>(base) + off * esize;
}

// ===========================================================================
// predict: chunk-local top-k candidates
// ===========================================================================
size_t predict_lds_bytes(int G, int d, int row, int cp) {
    size_t sel = 0;
    switch (G) {
        case 1: sel = sizeof(SelShared<1>); break;
        case 2: sel = sizeof(SelShared<2>); break;
        case 4: sel = sizeof(SelShared<4>); break;
        default: sel = sizeof(SelShared<8>); break;
    }
    sel = (sel + 15) & ~static_cast<size_t>(15);
    return sel + sizeof(float) * (static_cast<size_t>(G) * d + static_cast<size_t>(G) * row) +
           sizeof(uint32_t) * (static_cast<size_t>(G) * cp + 8);
}

template <int ROW, typename T, int G>
__global__ __launch_bounds__(kPredThreads) void k_predict(Plan P) {
    extern __shared__ __align__(16) unsigned char smem[];
    SelShared<G>& S = *reinterpret_cast<SelShared<G>*>(smem);
    const size_t sel = (sizeof(SelShared<G>) + 15) & ~static_cast<size_t>(15);
    float* qs = reinterpret_cast<float*>(smem + sel);  // [G][d]
    float* qv = qs + G * P.d;                           // [G][ROW]
    uint32_t* keys = reinterpret_cast<uint32_t*>(qv + G * ROW);  // [G][cp]
    uint32_t* wcnt = keys + G * P.cp;                            // [G] output counters

    const int tid = threadIdx.x, nthr = blockDim.x;
    const int lane = tid & 63, wave = tid >> 6, nwaves = nthr >> 6;
    const int bg = blockIdx.y, b = bg / P.Hkv, g = bg % P.Hkv, c = blockIdx.x;
    const int L = P.seq_lens[b];
    const Regions R = regions(P, L);
    const int t0 = max(c * P.cp, R.lo), t1 = min((c + 1) * P.cp, R.hi);
    if (t0 >= t1 || R.k == 0) return;
    const int kp = min(R.k, t1 - t0);
    const int d = P.d;

    // 1) query vectors: q_s = fl32(q * fl32(1/sqrt(d))); low-rank q~ = pdot(q_s, P[:, j])
    for (int x = tid; x < G * d; x += nthr) {
        const int h = x / d, cc = x - h * d;
        qs[x] = P.q[(static_cast<size_t>(b) * P.Hq + g * G + h) * d + cc] * P.scale32;
    }
    if (tid < G) wcnt[tid] = 0;
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

    // 2) scores: LPT lanes per token row, 8 elements per lane
    constexpr int LPT = ROW / 8, TPW = 64 / LPT;
    const int j = lane % LPT, slot = lane / LPT;
    float qreg[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) qreg[h][e] = qv[h * ROW + 8 * j + e];
    const T* src = static_cast<const T*>(P.predictor == 1 ? static_cast<const void*>(P.kt) : P.k);
    const int tb = (t0 / kPage) * kPage;
    const int ntok = ((t1 - 1) / kPage + 1) * kPage - tb;
    const int cbase = c * P.cp;
    const int32_t* btrow = P.bt + static_cast<size_t>(b) * P.max_blocks;
    for (int base = wave * TPW; base < ntok; base += nwaves * TPW) {
        // rows past the chunk's last page (TPW > 16) reread the last row and are not stored
        const int t = tb + min(base + slot, ntok - 1);
        const int page = btrow[t / kPage];
        const T* rowp = static_cast<const T*>(row_ptr(src, sizeof(T), page, P.Hkv, g, t % kPage, ROW)) + 8 * j;
        float kf[8];
        load8(rowp, kf);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float s = tree_across_lanes<LPT>(chain8(qreg[h], kf));
            if (j == 0 && t >= t0 && t < t1) keys[h * P.cp + (t - cbase)] = okey(s);
        }
    }
    __syncthreads();

    // 3) chunk top-kp per head
    uint32_t want[G];
#pragma unroll
    for (int h = 0; h < G; ++h) want[h] = static_cast<uint32_t>(kp);
    block_select<G>(S, want, [&](auto&& visit) {
        for (int t = t0 + tid; t < t1; t += nthr)
#pragma unroll
            for (int h = 0; h < G; ++h) visit(h, topk_key(keys[h * P.cp + (t - cbase)], static_cast<uint32_t>(t)));
    });

    // 4) write the kp candidates of each head (any order)
    uint64_t thr[G];
#pragma unroll
    for (int h = 0; h < G; ++h) thr[h] = S.thr[h];
    for (int t = t0 + tid; t < t1; t += nthr) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const uint64_t key = topk_key(keys[h * P.cp + (t - cbase)], static_cast<uint32_t>(t));
            if (key >= thr[h]) {
                const uint32_t pos = atomicAdd(&wcnt[h], 1u);
                const size_t bh = static_cast<size_t>(b) * P.Hq + g * G + h;
                if (pos < static_cast<uint32_t>(kp)) P.cand[(bh * P.ncp + c) * P.kcap + pos] = key;
            }
        }
    }
}

// ===========================================================================
// select: exact top-k, fixed-set bitmap, base-sample threshold
// ===========================================================================
__device__ __forceinline__ int chunk_candidates(const Plan& P, const Regions& R, int c) {
    const int a = max(c * P.cp, R.lo), e = min((c + 1) * P.cp, R.hi);
    return a < e ? min(R.k, e - a) : 0;
}

template <int G>
__global__ __launch_bounds__(kGroupThreads) void k_select(Plan P) {
    __shared__ SelShared<G> S;
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int bg = blockIdx.x, b = bg / P.Hkv, g = bg % P.Hkv;
    const int L = P.seq_lens[b];
    const Regions R = regions(P, L);
    const size_t bh0 = static_cast<size_t>(b) * P.Hq + g * G;

    // 1) merge the chunk candidates into the exact top-k of each head
    uint64_t thrT[G];
    if (R.k > 0) {
        uint32_t want[G];
#pragma unroll
        for (int h = 0; h < G; ++h) want[h] = static_cast<uint32_t>(R.k);
        const int slots = P.ncp * P.kcap;
        block_select<G>(S, want, [&](auto&& visit) {
            for (int x = tid; x < slots; x += nthr) {
                const int c = x / P.kcap, p = x - c * P.kcap;
                if (p >= chunk_candidates(P, R, c)) continue;
#pragma unroll
                for (int h = 0; h < G; ++h) visit(h, P.cand[((bh0 + h) * P.ncp + c) * P.kcap + p]);
            }
        });
#pragma unroll
        for (int h = 0; h < G; ++h) thrT[h] = S.thr[h];
    }

    // 2) bitmap: sinks [0, sp), window [hi, L), then the top-k bits
    const int wl = (L + 31) >> 5;
    for (int x = tid; x < G * wl; x += nthr) {
        const int h = x / wl, w = x - h * wl;
        uint32_t word = 0;
        for (int e = 0; e < 32; ++e) {
            const int i = 32 * w + e;
            if (i < L && (i < R.sp || i >= R.hi)) word |= 1u << e;
        }
        P.bits[(bh0 + h) * P.words + w] = word;
    }
    __syncthreads();
    if (R.k > 0) {
        const int slots = P.ncp * P.kcap;
        for (int x = tid; x < slots; x += nthr) {
            const int c = x / P.kcap, p = x - c * P.kcap;
            if (p >= chunk_candidates(P, R, c)) continue;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const uint64_t key = P.cand[((bh0 + h) * P.ncp + c) * P.kcap + p];
                if (key >= thrT[h]) {
                    const uint32_t i = ~static_cast<uint32_t>(key);
                    atomicOr(&P.bits[(bh0 + h) * P.words + (i >> 5)], 1u << (i & 31));
                }
            }
        }
    }
    __syncthreads();

    // 3) base sample: first nb tail tokens in (Philox word, index) order
    uint64_t thrB[G];
    if (R.nb > 0) {
        uint32_t want[G];
#pragma unroll
        for (int h = 0; h < G; ++h) want[h] = static_cast<uint32_t>(R.nb);
        const int q0 = R.lo >> 2, q1 = (R.hi - 1) >> 2;
        block_select<G>(S, want, [&](auto&& visit) {
            for (int qd = q0 + tid; qd <= q1; qd += nthr) {
                const uint4 w = philox4x32_10(static_cast<uint32_t>(qd), g, b, 0, P.seed_lo, P.seed_hi);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 4 * qd + e;
                    if (i < R.lo || i >= R.hi) continue;
                    const uint64_t key = sample_key(word_of(w, e), static_cast<uint32_t>(i));
#pragma unroll
                    for (int h = 0; h < G; ++h)
                        if (!bit_of_coherent(P.bits + (bh0 + h) * P.words, i)) visit(h, key);
                }
            }
        });
#pragma unroll
        for (int h = 0; h < G; ++h) thrB[h] = S.thr[h];
    }

    if (tid == 0 && P.gcounts) {
        P.gcounts[2 * bg] = 0;
        P.gcounts[2 * bg + 1] = 0;
    }
    if (tid < G) {
        HeadState hs{};
        hs.L = L;
        hs.k = R.k;
        hs.n_fixed = R.sp + R.wp + R.k;
        hs.NT = R.NT;
        hs.nb = R.nb;
        hs.thr_b = R.nb > 0 ? thrB[tid] : 0;
        P.hs[bh0 + tid] = hs;
    }
}

// ===========================================================================
// Membership of one token for the G heads of its group.
// ===========================================================================
struct HeadView {
    uint64_t thr_b, thr_n;
    int nb, n;
    float wsamp;
};

// ===========================================================================
// base: pinned exact scores of the union of fixed sets and base samples
// ===========================================================================
template <int D, typename KVT, int G>
__global__ __launch_bounds__(kChunkThreads) void k_base(Plan P) {
    __shared__ int tok[1024];
    __shared__ uint32_t tmask[1024];
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

    // membership (one Philox call per 4 tokens)
    const int T1 = min(T0 + P.cg, L);
    uint32_t m4[4] = {0, 0, 0, 0};
    uint32_t mine = 0;
    const int qd = (T0 >> 2) + tid;
    if (4 * qd < T1) {
        uint4 w = make_uint4(0, 0, 0, 0);
        if (4 * qd + 3 >= R.lo && 4 * qd < R.hi)
            w = philox4x32_10(static_cast<uint32_t>(qd), g, b, 0, P.seed_lo, P.seed_hi);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 4 * qd + e;
            if (i >= T1) continue;
            const bool inM = i >= R.lo && i < R.hi;
            const uint64_t key = sample_key(word_of(w, e), static_cast<uint32_t>(i));
            uint32_t mask = 0;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const bool fx = bit_of(P.bits + (bh0 + h) * P.words, i);
                const bool bs = inM && !fx && hv[h].nb > 0 && key >= hv[h].thr_b;
                mask |= (fx || bs) ? (1u << h) : 0u;
            }
            m4[e] = mask;
            mine += mask ? 1u : 0u;
        }
    }
    uint32_t cnt;
    uint32_t pos = block_excl_scan(mine, wsum, cnt);
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (m4[e]) {
            tok[pos] = 4 * qd + e;
            tmask[pos] = m4[e];
            ++pos;
        }
    if (tid == 0 && P.gcounts && cnt) atomicAdd(&P.gcounts[2 * bg + 1], static_cast<int>(cnt));
    __syncthreads();

    // pinned scores for all G heads of each listed token
    constexpr int LPT = D / 8, TPW = 64 / LPT;
    const int j = lane % LPT, slot = lane / LPT;
    float qreg[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            qreg[h][e] = P.q[(bh0 + h) * D + 8 * j + e] * P.scale32;
    float lmax[G];
#pragma unroll
    for (int h = 0; h < G; ++h) lmax[h] = -__builtin_inff();
    const int32_t* btrow = P.bt + static_cast<size_t>(b) * P.max_blocks;
    float* scrow = P.sc + static_cast<size_t>(bg) * P.max_seq_len * G;
    for (int base = 0; base < static_cast<int>(cnt); base += nwaves * TPW) {
        const int x = base + wave * TPW + slot;
        const bool act = x < static_cast<int>(cnt);
        const int i = act ? tok[x] : tok[0];
        const uint32_t mask = act ? tmask[x] : 0u;
        const int page = btrow[i / kPage];
        const KVT* rowp = static_cast<const KVT*>(row_ptr(P.k, sizeof(KVT), page, P.Hkv, g, i % kPage, D)) + 8 * j;
        float kf[8];
        load8(rowp, kf);
        float s[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            s[h] = tree_across_lanes<LPT>(chain8(qreg[h], kf));
            if ((mask >> h) & 1u) lmax[h] = fmaxf(lmax[h], s[h]);
        }
        if (act && j == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) scrow[static_cast<size_t>(i) * G + h] = s[h];
        }
    }
    // block max per head
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
    __shared__ SelShared<G> S;
    __shared__ float smax[G];
    __shared__ uint64_t red[kGroupThreads / 64][G][4];
    __shared__ HeadView hv[G];
    __shared__ int nsel[G];
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
    if (tid < G) {
        const HeadState& s = P.hs[bh0 + tid];
        hv[tid] = HeadView{s.thr_b, 0, s.nb, 0, 0.f};
        const int nc = (L + P.cg - 1) / P.cg;
        float m = -__builtin_inff();
        for (int c = 0; c < nc; ++c) m = fmaxf(m, P.cmax[(bh0 + tid) * P.ncg + c]);
        smax[tid] = m;
    }
    __syncthreads();

    // fixed-point sums: SF over I_f, S1 and S2 over the base sample
    uint64_t sf[G], s1[G];
    unsigned __int128 s2[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        sf[h] = 0;
        s1[h] = 0;
        s2[h] = 0;
    }
    const float* scrow = P.sc + static_cast<size_t>(bg) * P.max_seq_len * G;
    const int nq = (L + 3) >> 2;
    for (int qd = tid; qd < nq; qd += nthr) {
        uint4 w = make_uint4(0, 0, 0, 0);
        if (4 * qd + 3 >= R.lo && 4 * qd < R.hi)
            w = philox4x32_10(static_cast<uint32_t>(qd), g, b, 0, P.seed_lo, P.seed_hi);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 4 * qd + e;
            if (i >= L) continue;
            const bool inM = i >= R.lo && i < R.hi;
            const uint64_t key = sample_key(word_of(w, e), static_cast<uint32_t>(i));
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const bool fx = bit_of(P.bits + (bh0 + h) * P.words, i);
                const bool bs = inM && !fx && hv[h].nb > 0 && key >= hv[h].thr_b;
                if (fx || bs) {
                    const uint64_t E = fixed_weight(scrow[static_cast<size_t>(i) * G + h] - smax[h]);
                    if (fx) {
                        sf[h] += E;
                    } else {
                        s1[h] += E;
                        s2[h] += static_cast<unsigned __int128>(E) * E;
                    }
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
        // a new selection unless the sample is empty, the whole tail or the base sample
        nsel[h] = (n > 0 && n < NT && n != nb) ? n : 0;
        hv[h].n = n;
    }
    __syncthreads();

    uint32_t want[G];
    bool any = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        want[h] = static_cast<uint32_t>(nsel[h]);
        any |= nsel[h] > 0;
    }
    if (any) {
        const int q0 = R.lo >> 2, q1 = (R.hi - 1) >> 2;
        block_select<G>(S, want, [&](auto&& visit) {
            for (int qd = q0 + tid; qd <= q1; qd += nthr) {
                const uint4 w = philox4x32_10(static_cast<uint32_t>(qd), g, b, 0, P.seed_lo, P.seed_hi);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 4 * qd + e;
                    if (i < R.lo || i >= R.hi) continue;
                    const uint64_t key = sample_key(word_of(w, e), static_cast<uint32_t>(i));
#pragma unroll
                    for (int h = 0; h < G; ++h)
                        if (!bit_of(P.bits + (bh0 + h) * P.words, i)) visit(h, key);
                }
            }
        });
    }
    if (tid < G) {
        const int h = tid, n = hv[h].n;
        uint64_t thr = 0;
        if (nsel[h] > 0) thr = S.thr[h];
        else if (n > 0 && n == hv[h].nb) thr = hv[h].thr_b;
        else thr = 0;  // n == N_t: the whole tail (or n == 0: unused)
        P.hs[bh0 + h].thr_n = thr;
    }
}

// ===========================================================================
// gather: weighted online softmax over the union of the group's index sets
// ===========================================================================
template <int D, typename KVT, int G>
__global__ __launch_bounds__(kChunkThreads) void k_gather(Plan P) {
    constexpr int NW = kChunkThreads / 64;
    __shared__ int tok[1024];
    __shared__ uint32_t tmeta[1024];
    __shared__ uint32_t wsum[NW];
    __shared__ HeadView hv[G];
    __shared__ float wm[NW][G], wl[NW][G];
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

    // membership: meta = final mask | fixed mask << 8 | cached << 16
    const int T1 = min(T0 + P.cg, L);
    uint32_t m4[4] = {0, 0, 0, 0};
    uint32_t mine = 0;
    const int qd = (T0 >> 2) + tid;
    if (4 * qd < T1) {
        uint4 w = make_uint4(0, 0, 0, 0);
        if (4 * qd + 3 >= R.lo && 4 * qd < R.hi)
            w = philox4x32_10(static_cast<uint32_t>(qd), g, b, 0, P.seed_lo, P.seed_hi);
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
            const uint32_t meta = fin | (fxm << 8) | (cached << 16);
            m4[e] = fin ? meta : 0u;
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
            ++pos;
        }
    if (tid == 0 && P.gcounts && cnt) atomicAdd(&P.gcounts[2 * bg], static_cast<int>(cnt));
    __syncthreads();

    constexpr int LPT = D / 8, TPW = 64 / LPT;
    const int j = lane % LPT, slot = lane / LPT;
    float qreg[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            qreg[h][e] = P.q[(bh0 + h) * D + 8 * j + e] * P.scale32;
    float ws[G];
#pragma unroll
    for (int h = 0; h < G; ++h) ws[h] = hv[h].wsamp;
    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -__builtin_inff();
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    }
    const int32_t* btrow = P.bt + static_cast<size_t>(b) * P.max_blocks;
    const float* scrow = P.sc + static_cast<size_t>(bg) * P.max_seq_len * G;
    for (int base = 0; base < static_cast<int>(cnt); base += nwaves * TPW) {
        const int x = base + wave * TPW + slot;
        const bool act = x < static_cast<int>(cnt);
        const int i = act ? tok[x] : tok[0];
        const uint32_t meta = act ? tmeta[x] : 0u;
        const bool cached = (meta >> 16) & 1u;
        const int page = btrow[i / kPage];
        const size_t roff = ((static_cast<size_t>(page) * P.Hkv + g) * kPage + (i % kPage)) * D + 8 * j;
        float vf[8], kf[8];
        load8(static_cast<const KVT*>(P.v) + roff, vf);
        if (!cached) {
            load8(static_cast<const KVT*>(P.k) + roff, kf);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) kf[e] = 0.f;
        }
        float s[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float st = tree_across_lanes<LPT>(chain8(qreg[h], kf));
            s[h] = cached ? scrow[static_cast<size_t>(i) * G + h] : st;
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const bool on = act && ((meta >> h) & 1u);
            const float w = ((meta >> (8 + h)) & 1u) ? 1.0f : ws[h];
            const float mn = on ? fmaxf(m[h], s[h]) : m[h];
            const float alpha = (mn == -__builtin_inff()) ? 1.0f : __expf(m[h] - mn);
            const float p = on ? w * __expf(s[h] - mn) : 0.0f;
            l[h] = l[h] * alpha + p;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = acc[h][e] * alpha + p * vf[e];
            m[h] = mn;
        }
    }
    // merge the TPW token slots of the wave (lanes with equal j)
#pragma unroll
    for (int o = LPT; o < 64; o <<= 1) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mo = __shfl_xor(m[h], o, 64), lo = __shfl_xor(l[h], o, 64);
            const float mn = fmaxf(m[h], mo);
            const float a = (mn == -__builtin_inff()) ? 0.0f : __expf(m[h] - mn);
            const float bo = (mn == -__builtin_inff()) ? 0.0f : __expf(mo - mn);
            l[h] = l[h] * a + lo * bo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float ao = __shfl_xor(acc[h][e], o, 64);
                acc[h][e] = acc[h][e] * a + ao * bo;
            }
            m[h] = mn;
        }
    }
    if (slot == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            if (j == 0) {
                wm[wave][h] = m[h];
                wl[wave][h] = l[h];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) wacc[wave][h][8 * j + e] = acc[h][e];
        }
    }
    __syncthreads();
    for (int x = tid; x < G * (D + 2); x += nthr) {
        const int h = x / (D + 2), e = x - h * (D + 2);
        float M = -__builtin_inff();
        for (int w = 0; w < NW; ++w) M = fmaxf(M, wm[w][h]);
        float v = 0.f;
        if (e == 0) {
            v = M;
        } else if (M != -__builtin_inff()) {
            for (int w = 0; w < NW; ++w) {
                const float sc = __expf(wm[w][h] - M);
                v += (e == 1 ? wl[w][h] : wacc[w][h][e - 2]) * sc;
            }
        }
        P.part[((bh0 + h) * P.ncg + c) * (D + 2) + e] = v;
    }
}

// ===========================================================================
// combine: merge chunk partials; counts and statistics
// ===========================================================================
__global__ __launch_bounds__(256) void k_combine(Plan P) {
    const int bh = blockIdx.x, b = bh / P.Hq;
    const int L = P.seq_lens[b];
    const int D = P.d;
    const int nc = (L + P.cg - 1) / P.cg;
    const float* pp = P.part + static_cast<size_t>(bh) * P.ncg * (D + 2);
    float M = -__builtin_inff();
    for (int c = 0; c < nc; ++c) M = fmaxf(M, pp[static_cast<size_t>(c) * (D + 2)]);
    float l = 0.f;
    if (M != -__builtin_inff())
        for (int c = 0; c < nc; ++c) {
            const float* q = pp + static_cast<size_t>(c) * (D + 2);
            l += q[1] * __expf(q[0] - M);
        }
    for (int e = threadIdx.x; e < D; e += blockDim.x) {
        float a = 0.f;
        if (M != -__builtin_inff() && l > 0.f) {
            for (int c = 0; c < nc; ++c) {
                const float* q = pp + static_cast<size_t>(c) * (D + 2);
                a += q[2 + e] * __expf(q[0] - M);
            }
            a = a / l;
        }
        P.out[static_cast<size_t>(bh) * D + e] = a;
    }
    if (threadIdx.x == 0) {
        P.lse[bh] = (M != -__builtin_inff() && l > 0.f) ? M + __logf(l) : -__builtin_inff();
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
                w = philox4x32_10(static_cast<uint32_t>(qd), g, b, 0, P.seed_lo, P.seed_hi);
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
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return static_cast<int>(e);
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
    hipLaunchKernelGGL(k_combine, dim3(p.B * p.Hq), dim3(p.d), 0, st, p);
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
