// Device building blocks for the gfx950 decode step: Philox, the pinned fp32
// dot product and exp, exact fixed-point weights, wavefront/block scans and a
// block-wide multi-problem radix select.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vattn_plan.hpp"

namespace vattn {

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC'11).  One call yields the sample keys of four consecutive
// tokens: counter (i >> 2, g, b, 0), key = seed, token i takes word i & 3.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                               uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        if (round) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint32_t hi0 = __umulhi(0xD2511F53u, c0), lo0 = 0xD2511F53u * c0;
        const uint32_t hi1 = __umulhi(0xCD9E8D57u, c2), lo1 = 0xCD9E8D57u * c2;
        const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
    }
    return make_uint4(c0, c1, c2, c3);
}

__device__ __forceinline__ uint32_t word_of(const uint4& w, int e) {
    return e == 0 ? w.x : e == 1 ? w.y : e == 2 ? w.z : w.w;
}

// Sample words of the token quad qd (tokens 4 qd .. 4 qd + 3) of sequence b,
// KV head g: one Philox4x32-10 block, recomputed wherever a pass needs them
// (cheaper than storing 4 bytes per token and reading them back).
__device__ __forceinline__ uint4 quad_words(uint32_t qd, uint32_t g, uint32_t b, uint32_t seed_lo, uint32_t seed_hi) {
    return philox4x32_10(qd, g, b, 0, seed_lo, seed_hi);
}

__device__ __forceinline__ uint32_t token_word(uint32_t i, uint32_t g, uint32_t b, uint32_t seed_lo, uint32_t seed_hi) {
    return word_of(quad_words(i >> 2, g, b, seed_lo, seed_hi), static_cast<int>(i & 3u));
}

// Sample order: ascending (Philox word u, token index i).  Stored complemented
// so that "first n of the order" == "n largest keys".
__device__ __forceinline__ uint64_t sample_key(uint32_t u, uint32_t i) {
    return ~((static_cast<uint64_t>(u) << 32) | i);
}

// Top-k order: descending score, then ascending index; also "n largest keys".
__device__ __forceinline__ uint32_t okey(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint64_t topk_key(uint32_t ok, uint32_t i) {
    return (static_cast<uint64_t>(ok) << 32) | static_cast<uint32_t>(~i);
}

// ---------------------------------------------------------------------------
// Pinned arithmetic.  Every score that decides a discrete outcome is the same
// sequence of IEEE fp32 operations: for each block of 8 elements an fma chain
// from +0 in element order, then the block partials added pairwise (adjacent
// pairs first).  On the GPU a block is one lane's 16-byte slice and the tree is
// an xor butterfly across the lanes of a row; IEEE addition is commutative, so
// both lanes of a pair hold the identical sum.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float chain8(const float (&a)[8], const float (&b)[8]) {
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(a[e], b[e], acc);
    return acc;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// The pairwise tree over the LPT lane partials of a row, adjacent pairs first,
// with DPP lane moves: quad_perm [1,0,3,2] and [2,3,0,1] pair lanes 2k/2k+1
// and the two halves of each quad; row_ror:4 then adds quad q-1 to quad q and
// row_ror:8 adds lanes 4-7 to lanes 12-15 of each 16-lane row.  IEEE addition
// commutes, so each sum equals the tree's.  The result is valid in the lanes
// with lane % LPT == LPT - 1 (in every lane when LPT <= 4).
template <int LPT>
__device__ __forceinline__ float tree_across_lanes(float v) {
    static_assert(LPT == 1 || LPT == 2 || LPT == 4 || LPT == 8 || LPT == 16, "row of 8..128 elements");
    if constexpr (LPT >= 2) v = v + dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    if constexpr (LPT >= 4) v = v + dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    if constexpr (LPT >= 8) v = dpp<0x124>(v) + v;  // row_ror:4
    if constexpr (LPT >= 16) v = dpp<0x128>(v) + v; // row_ror:8
    return v;
}

// The same tree for G heads at once, with the sums spread over the row's
// lanes.  On each quad level (partners lane ^ 1, then lane ^ 2) that still
// has more than one head per lane, a lane keeps half of its heads and adds its
// partner's partials of them: G/2 + G/4 adds and G + G/2 selects in place of
// 2G adds, and each sum then needs finishing (order key, store) in one lane
// only.  Levels past that, and the row_ror levels of rows over 4 lanes, add as
// tree_across_lanes does.  Every sum is the tree's (IEEE addition commutes).
template <int G, int LPT>
struct Spread {
    static constexpr int lg(int x) { return x <= 1 ? 0 : 1 + lg(x / 2); }
    // quad levels that split the heads
    static constexpr int NS = lg(G) < lg(LPT) ? (lg(G) < 2 ? lg(G) : 2) : (lg(LPT) < 2 ? lg(LPT) : 2);
    static constexpr int NH = G >> NS;  // heads held per lane
    // head of slot e in row lane j
    __device__ static __forceinline__ int head(int j, int e) {
        int h = e;
        if constexpr (NS >= 1) h += (j & 1) * (G / 2);
        if constexpr (NS >= 2) h += ((j >> 1) & 1) * (G / 4);
        return h;
    }
    // the lanes whose sums are complete and not duplicated in another lane
    __device__ static __forceinline__ bool finisher(int j) { return (j | ((1 << NS) - 1)) == LPT - 1; }
};

template <int G, int LPT>
__device__ __forceinline__ void spread_across_lanes(const float (&v)[G], float (&out)[Spread<G, LPT>::NH], int j) {
    static_assert(LPT == 1 || LPT == 2 || LPT == 4 || LPT == 8 || LPT == 16, "row of 8..128 elements");
    constexpr int NS = Spread<G, LPT>::NS;
    float a[G];
#pragma unroll
    for (int h = 0; h < G; ++h) a[h] = v[h];
    if constexpr (NS >= 1) {  // lane ^ 1: keep the lower or upper half of the heads
        const bool up = j & 1;
#pragma unroll
        for (int k = 0; k < G / 2; ++k) {
            const float keep = up ? a[k + G / 2] : a[k];
            const float send = up ? a[k] : a[k + G / 2];
            a[k] = keep + dpp<0xB1>(send);
        }
    } else if constexpr (LPT >= 2) {
        a[0] = a[0] + dpp<0xB1>(a[0]);
    }
    if constexpr (NS >= 2) {  // lane ^ 2
        const bool up = (j >> 1) & 1;
#pragma unroll
        for (int k = 0; k < G / 4; ++k) {
            const float keep = up ? a[k + G / 4] : a[k];
            const float send = up ? a[k] : a[k + G / 4];
            a[k] = keep + dpp<0x4E>(send);
        }
    } else if constexpr (LPT >= 4) {
#pragma unroll
        for (int k = 0; k < (G >> NS); ++k) a[k] = a[k] + dpp<0x4E>(a[k]);
    }
#pragma unroll
    for (int k = 0; k < (G >> NS); ++k) {
        if constexpr (LPT >= 8) a[k] = dpp<0x124>(a[k]) + a[k];   // row_ror:4
        if constexpr (LPT >= 16) a[k] = dpp<0x128>(a[k]) + a[k];  // row_ror:8
        out[k] = a[k];
    }
}

// Sequential form of the same blocked dot (one thread), N a multiple of 8 with
// N / 8 a power of two.
template <int N>
__device__ __forceinline__ float pdot_serial(const float* a, int sa, const float* b, int sb) {
    constexpr int NB = N / 8;
    float part[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        float acc = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(a[(8 * j + e) * sa], b[(8 * j + e) * sb], acc);
        part[j] = acc;
    }
#pragma unroll
    for (int w = NB; w > 1; w >>= 1) {
#pragma unroll
        for (int j = 0; j < w / 2; ++j) part[j] = part[2 * j] + part[2 * j + 1];
    }
    return part[0];
}

// exp(x) for x in [-28, 0]: Cody-Waite reduction with ln 2 split into a 15-bit
// head (n * LN2_HI exact for |n| < 2^9) and an fp32 tail, then the degree-7
// Taylor polynomial with coefficients fl32(1/k!) in Horner form, scaled by 2^n.
__device__ __forceinline__ float pinned_exp(float x) {
    const float kLog2e = 0x1.715476p+0f;   // fl32(1 / ln 2)
    const float kLn2Hi = 0x1.62e4p-1f;     // 22713 / 32768
    const float kLn2Lo = 0x1.7f7d1cp-20f;  // fl32(ln 2 - kLn2Hi)
    const float t = x * kLog2e;
    const float n = __builtin_rintf(t);
    float r = __builtin_fmaf(-n, kLn2Hi, x);
    r = __builtin_fmaf(-n, kLn2Lo, r);
    float p = 0x1.a01a02p-13f;                 // 1/7!
    p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);  // 1/6!
    p = __builtin_fmaf(p, r, 0x1.111112p-7f);   // 1/5!
    p = __builtin_fmaf(p, r, 0x1.555556p-5f);   // 1/4!
    p = __builtin_fmaf(p, r, 0x1.555556p-3f);   // 1/3!
    p = __builtin_fmaf(p, r, 0x1p-1f);          // 1/2!
    p = __builtin_fmaf(p, r, 1.0f);             // 1/1!
    p = __builtin_fmaf(p, r, 1.0f);             // 1/0!
    return __builtin_ldexpf(p, static_cast<int>(n));
}

// E = trunc(exp(x) * 2^40), 0 below x = -28, at most 2^40.  The fp32 product is
// exact (power-of-two scale); the truncation is done on the bits.
__device__ __forceinline__ uint64_t fixed_weight(float x) {
    if (!(x >= -28.0f)) return 0;
    const float v = pinned_exp(x) * 0x1p40f;
    const uint32_t bits = __float_as_uint(v);
    const int ex = static_cast<int>((bits >> 23) & 0xFFu);
    if (ex == 0) return 0;
    const uint64_t mant = (bits & 0x7FFFFFu) | 0x800000u;
    const int sh = ex - 150;
    uint64_t e = sh >= 0 ? (mant << sh) : (sh > -24 ? (mant >> -sh) : 0);
    return e > (1ull << 40) ? (1ull << 40) : e;
}

// Unsigned 128-bit integer to fp64, round to nearest even.
__device__ __forceinline__ double u128_to_f64(unsigned __int128 x) {
    if (x == 0) return 0.0;
    const uint64_t hi = static_cast<uint64_t>(x >> 64), lo = static_cast<uint64_t>(x);
    const int msb = hi ? 127 - __clzll(hi) : 63 - __clzll(lo);
    if (msb <= 52) return static_cast<double>(lo);  // exact
    int s = msb - 52;
    unsigned __int128 m = x >> s;
    const unsigned __int128 rem = x & ((static_cast<unsigned __int128>(1) << s) - 1);
    const unsigned __int128 half = static_cast<unsigned __int128>(1) << (s - 1);
    if (rem > half || (rem == half && (m & 1))) m += 1;
    if (m >> 53) {
        m >>= 1;
        s += 1;
    }
    return __builtin_ldexp(static_cast<double>(static_cast<uint64_t>(m)), s);
}

// ---------------------------------------------------------------------------
// Loads of 8 consecutive elements (one lane's block) as fp32.
// ---------------------------------------------------------------------------
struct Raw8 {  // one lane's 8 elements as loaded (bf16: one uint4; fp32: two float4)
    uint4 a, b;
};
// A lane's 8 elements of a K, V or K~ row.  Every row is read once per step,
// so the loads are non-temporal: they do not displace the step's small
// intermediate arrays from the caches (measured: the gather 10% faster).
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
__device__ __forceinline__ uint4 nt_load16(const void* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void load_raw_nt(const uint16_t* p, Raw8& r) { r.a = nt_load16(p); }
__device__ __forceinline__ void load_raw_nt(const float* p, Raw8& r) {
    r.a = nt_load16(p);
    r.b = nt_load16(p + 4);
}
template <typename T>
__device__ __forceinline__ void widen(const Raw8& r, float (&f)[8]) {
    if constexpr (sizeof(T) == 2) {
        const uint32_t ws[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            f[2 * k] = __uint_as_float(ws[k] << 16);
            f[2 * k + 1] = __uint_as_float(ws[k] & 0xFFFF0000u);
        }
    } else {
        f[0] = __uint_as_float(r.a.x); f[1] = __uint_as_float(r.a.y);
        f[2] = __uint_as_float(r.a.z); f[3] = __uint_as_float(r.a.w);
        f[4] = __uint_as_float(r.b.x); f[5] = __uint_as_float(r.b.y);
        f[6] = __uint_as_float(r.b.z); f[7] = __uint_as_float(r.b.w);
    }
}

// ---------------------------------------------------------------------------
// Sequence regions (sinks, window, middle), k, tail size and base-sample size.
// ---------------------------------------------------------------------------
struct Regions {
    int sp, wp, lo, hi, k, NT, nb;
};

__device__ __forceinline__ Regions regions(const Plan& P, int L) {
    Regions R;
    R.sp = min(P.sinks, L);
    R.wp = min(P.window, L - R.sp);
    R.lo = R.sp;
    R.hi = L - R.wp;
    const int nM = R.hi - R.lo;
    const long long k64 = P.topk_abs >= 0 ? static_cast<long long>(P.topk_abs)
                                          : (static_cast<long long>(L) * P.topk_ppm + 999999) / 1000000;
    R.k = static_cast<int>(k64 < nM ? k64 : nM);
    R.NT = nM - R.k;
    if (R.NT > 0) {
        long long want = (static_cast<long long>(R.NT) * P.base_ppm + 999999) / 1000000;
        if (want < 2) want = 2;
        R.nb = static_cast<int>(want < R.NT ? want : R.NT);
    } else {
        R.nb = 0;
    }
    return R;
}

// ---------------------------------------------------------------------------
// Scans and reductions.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    // row_shr:1, 2, 4, 8 within each 16-lane row (update_dpp with old = 0
    // reads 0 before the row start), then the totals of the rows below from
    // lanes 15, 31 and 47; no LDS traffic.  The whole wave must be active.
    const int lane = threadIdx.x & 63;
    v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x111, 0xF, 0xF, false));
    v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x112, 0xF, 0xF, false));
    v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x114, 0xF, 0xF, false));
    v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x118, 0xF, 0xF, false));
    const uint32_t r0 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 15));
    const uint32_t r1 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 31));
    const uint32_t r2 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 47));
    const int row = lane >> 4;
    return v + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// Exclusive prefix over the block in thread order; `total` gets the block sum.
// `wsum` is LDS scratch of >= blockDim.x / 64 words.  All threads must call.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const uint32_t inc = wave_incl_scan(v);
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    uint32_t before = 0, tot = 0;
    for (int w = 0; w < nw; ++w) {
        const uint32_t x = wsum[w];
        before += (w < wave) ? x : 0u;
        tot += x;
    }
    __syncthreads();
    total = tot;
    return before + inc - v;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), m, 64);
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), m, 64);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// ---------------------------------------------------------------------------
// Block-wide radix select for NH independent problems at once.
// For problem h it finds thr[h] such that exactly want[h] of its keys are
// >= thr[h] (keys are unique 64-bit values).  Digits of 8 bits from the top;
// a problem stops as soon as its whole bucket is inside the answer.  Keys are
// produced by `items(visit)`, which calls visit(h, key) for every key assigned
// to this thread; it is called once per pass, so keys may be recomputed.
// want[h] must not exceed the number of keys of problem h (if it does, thr[h]
// selects all keys seen).  want[h] == 0 leaves problem h inactive.
// ---------------------------------------------------------------------------
template <int NH>
struct SelShared {
    uint32_t hist[NH][256];
    uint64_t prefix[NH];
    uint64_t thr[NH];
    uint32_t rem[NH];
    uint32_t first[NH];  // the pass at which each problem starts
    uint32_t active;
};

// With `exact`, thr[h] is raised to the smallest selected key itself: needed
// when `items` enumerates only part of a larger population (one bucket of it),
// where a prefix threshold could also admit keys that were never visited.
// With `kand` / `kor` (the AND and the OR of problem h's keys, in LDS), the
// digits above the highest bit where its keys differ are known already: the
// problem starts at the digit holding that bit.
template <int NH, class Items>
__device__ __forceinline__ void block_select(SelShared<NH>& S, const uint32_t (&want)[NH], Items&& items,
                             bool exact = false, const uint64_t* kand = nullptr,
                             const uint64_t* kor = nullptr) {
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int lane = tid & 63, wave = tid >> 6, nwaves = nthr >> 6;
    if (tid == 0) {
        uint32_t act = 0;
        for (int h = 0; h < NH; ++h) {
            uint64_t pre = 0;
            uint32_t p0 = 0;
            if (kand != nullptr && want[h] > 0) {
                const uint64_t diff = kand[h] ^ kor[h];
                const int hb = diff ? 63 - __clzll(static_cast<long long>(diff)) : 0;
                p0 = static_cast<uint32_t>((63 - hb) / 8);  // digit 56 - 8 p0 .. 63 - 8 p0 holds hb
                if (p0 > 0) pre = kand[h] & ~((1ull << (64 - 8 * p0)) - 1ull);
            }
            S.prefix[h] = pre;
            S.first[h] = p0;
            S.thr[h] = 0;
            S.rem[h] = want[h];
            if (want[h] > 0) act |= 1u << h;
        }
        S.active = act;
    }
    __syncthreads();
    for (int pass = 0; pass < 8; ++pass) {
        const uint32_t live = S.active;
        if (live == 0) break;  // block-uniform: read after a barrier
        uint32_t act = 0;      // the live problems whose first digit has come
#pragma unroll
        for (int h = 0; h < NH; ++h)
            if (((live >> h) & 1u) && S.first[h] <= static_cast<uint32_t>(pass)) act |= 1u << h;
        if (act == 0) continue;  // block-uniform
        const int shift = 56 - 8 * pass;
        for (int x = tid; x < NH * 256; x += nthr) (&S.hist[0][0])[x] = 0;
        uint64_t pre[NH];
#pragma unroll
        for (int h = 0; h < NH; ++h) pre[h] = S.prefix[h];
        __syncthreads();
        items([&](int h, uint64_t key) __attribute__((always_inline)) {
            if (!((act >> h) & 1u)) return;
            if (pass > 0 && ((key ^ pre[h]) >> (shift + 8)) != 0) return;
            atomicAdd(&S.hist[h][static_cast<uint32_t>(key >> shift) & 255u], 1u);
        });
        __syncthreads();
        for (int h = wave; h < NH; h += nwaves) {
            if (!((act >> h) & 1u)) continue;
            const uint32_t rem = S.rem[h];
            const int top = 255 - 4 * lane;  // this lane's bins: top, top-1, top-2, top-3
            const uint32_t c0 = S.hist[h][top], c1 = S.hist[h][top - 1];
            const uint32_t c2 = S.hist[h][top - 2], c3 = S.hist[h][top - 3];
            const uint32_t cnt = c0 + c1 + c2 + c3;
            const uint32_t inc = wave_incl_scan(cnt);
            const unsigned long long ball = __ballot(inc >= rem);
            if (ball == 0ull) {
                if (lane == 0) {  // fewer keys than wanted: take all of this prefix
                    S.thr[h] = S.prefix[h];
                    atomicAnd(&S.active, ~(1u << h));
                }
                continue;
            }
            const int owner = __ffsll(static_cast<long long>(ball)) - 1;
            if (lane == owner) {
                const uint32_t cs[4] = {c0, c1, c2, c3};
                uint32_t above = inc - cnt;
                int dg = top - 3;
                for (int e = 0; e < 4; ++e) {
                    if (above + cs[e] >= rem) {
                        dg = top - e;
                        break;
                    }
                    above += cs[e];
                }
                const uint32_t r2 = rem - above;
                const uint64_t p = S.prefix[h] | (static_cast<uint64_t>(dg) << shift);
                S.prefix[h] = p;
                S.rem[h] = r2;
                if (S.hist[h][dg] == r2 || shift == 0) {
                    S.thr[h] = p;
                    atomicAnd(&S.active, ~(1u << h));
                }
            }
        }
        __syncthreads();
    }
    if (exact) {
        uint32_t wmask = 0;
#pragma unroll
        for (int h = 0; h < NH; ++h) wmask |= want[h] > 0 ? (1u << h) : 0u;
        if (tid < NH) S.prefix[tid] = S.thr[tid];  // the prefix threshold, kept for the pass
        __syncthreads();
        if (tid < NH) S.thr[tid] = ~0ull;
        __syncthreads();
        items([&](int h, uint64_t key) __attribute__((always_inline)) {
            if (((wmask >> h) & 1u) && key >= S.prefix[h]) atomicMin(&S.thr[h], key);
        });
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// One wavefront finds the bin holding the rank-th element (1-based) when the
// NBINS bins are visited in ascending order, or descending when `desc`.
// bin_out = -1 when the histogram holds fewer than `rank` elements.
// ---------------------------------------------------------------------------
template <int NBINS>
__device__ __forceinline__ void wave_rank_bin(const uint32_t* hist, uint32_t rank, bool desc,
                                              int& bin_out, uint32_t& before_out) {
    constexpr int PER = NBINS / 64;
    const int lane = threadIdx.x & 63;
    uint32_t c[PER];
    uint32_t sum = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const int pos = lane * PER + e;
        c[e] = hist[desc ? NBINS - 1 - pos : pos];
        sum += c[e];
    }
    const uint32_t inc = wave_incl_scan(sum);
    const unsigned long long ball = __ballot(inc >= rank);
    if (ball == 0ull) {
        bin_out = -1;
        before_out = 0;
        return;
    }
    const int owner = __ffsll(static_cast<long long>(ball)) - 1;
    int bin = -1;
    uint32_t before = 0;
    if (lane == owner) {
        uint32_t acc = inc - sum;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            if (bin < 0 && acc + c[e] >= rank) {
                const int pos = lane * PER + e;
                bin = desc ? NBINS - 1 - pos : pos;
                before = acc;
            }
            acc += c[e];
        }
    }
    bin_out = __shfl(bin, owner, 64);
    before_out = __shfl(before, owner, 64);
}

// Element x of list[0, n) is the r-th largest (1-based) iff exactly r - 1
// elements exceed it (keys are unique).  One thread per element.
__device__ __forceinline__ void list_rank_pick(const uint64_t* list, int n, uint32_t r, int x,
                                               uint64_t* out) {
    if (x >= n) return;
    const uint64_t v = list[x];
    uint32_t above = 0;
    for (int y = 0; y < n; ++y) above += list[y] > v ? 1u : 0u;
    if (above + 1 == r) *out = v;
}

// ---------------------------------------------------------------------------
// Block-wide exact top-k for NH heads at once, without contended atomics:
// (B) histogram over kTopBuckets value-range buckets of the score (a
// monotone map of the key, so bucket order is key order) between the given
// bracket [lo_ok, hi_ok] of the heads' order keys, (C) one pass that emits
// every key above the boundary bucket and lists the boundary bucket's keys,
// which are then ranked exactly.  Only a boundary bucket larger than
// kListCap falls back to the radix select.  items(f) calls f(h, okey, index)
// for every key of head h on this thread; emit(h, pos, key) is called exactly
// once for each of the want[h] largest keys topk_key(okey, index) of head h
// (for every key when want[h] >= total[h]), with distinct positions
// pos < want[h].  On return thr[h] is the smallest emitted key (0 when
// everything was emitted).
// ---------------------------------------------------------------------------
template <int NH>
struct TopkShared {
    SelShared<NH> S;  // S.hist doubles as the bucket histogram
    uint64_t list[NH][kListCap];
    uint64_t thr[NH];
    uint32_t above[NH], cnt[NH], aux[NH], lo[NH], hi[NH];
    int bstar[NH];
    float vmin[NH], scale[NH];  // per-head bucket map, read by the visitors
    uint32_t mode[NH];          // 0 idle, 1 select, 2 emit everything
    uint32_t want[NH];
    uint64_t kand[NH], kor[NH];  // AND / OR of a crowded boundary bucket's keys
};

// Score back from its order key.
__device__ __forceinline__ float okey_value(uint32_t ok) {
    return __uint_as_float((ok & 0x80000000u) ? (ok & 0x7FFFFFFFu) : ~ok);
}

// Bucket linear in the score: (s - s_lo) * 256 / (s_hi - s_lo), clamped.
// Each step (fp32 subtract, multiply by a positive constant, truncate) is
// monotone non-decreasing, so bucket order never contradicts key order.
__device__ __forceinline__ int topk_bucket(uint32_t ok, float vmin, float scale) {
    const float f = (okey_value(ok) - vmin) * scale;
    const int bk = f > 0.0f ? static_cast<int>(f) : 0;
    return bk < kTopBuckets - 1 ? bk : kTopBuckets - 1;
}

// Per-head setup of a top-k: bucket maps, modes and counters in LDS, the
// bucket histograms cleared.  Ends with a barrier; returns whether any head
// needs the selection (mode 1).
template <int NH>
__device__ __forceinline__ bool topk_setup(TopkShared<NH>& T, const uint32_t (&want)[NH], const uint32_t (&total)[NH],
                                           const uint32_t (&lo_ok)[NH], const uint32_t (&hi_ok)[NH]) {
    const int tid = threadIdx.x, nthr = blockDim.x;
    // per-head parameters live in LDS: the visitors index them by a head number
    // that need not be a compile-time constant after inlining
#pragma unroll
    for (int h = 0; h < NH; ++h) {  // compile-time head numbers: no indexing of the caller's arrays
        if (tid != h) continue;
        const bool act = want[h] > 0 && want[h] < total[h];
        const bool all = want[h] > 0 && want[h] >= total[h];
        T.want[h] = want[h];
        const float vmin = okey_value(lo_ok[h]), vmax = okey_value(hi_ok[h]);
        const float range = vmax - vmin;
        const float scale = static_cast<float>(kTopBuckets) / range;
        // a zero or non-finite range puts every key in bucket 0
        const bool ok = range > 0.0f && range < __builtin_inff() && scale < __builtin_inff();
        T.vmin[h] = vmin;
        T.scale[h] = ok ? scale : 0.0f;
        T.mode[h] = act ? 1u : all ? 2u : 0u;
        T.cnt[h] = 0;
        T.aux[h] = 0;  // emission positions
        T.thr[h] = 0;
        T.bstar[h] = -1;
        T.above[h] = 0;
    }
    bool any = false;
#pragma unroll
    for (int h = 0; h < NH; ++h) any |= want[h] > 0 && want[h] < total[h];
    for (int x = tid; x < NH * kTopBuckets; x += nthr) (&T.S.hist[0][0])[x] = 0;
    __syncthreads();
    return any;
}

// The boundary bucket of every selecting head from its histogram: bstar, and
// the number of keys above it.  Ends with a barrier.
template <int NH>
__device__ __forceinline__ void topk_rank(TopkShared<NH>& T) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
    for (int h = wave; h < NH; h += nwaves) {
        if (T.mode[h] != 1u) continue;
        int bin;
        uint32_t before;
        wave_rank_bin<kTopBuckets>(T.S.hist[h], T.want[h], true, bin, before);
        if (lane == 0) {
            T.bstar[h] = bin;
            T.above[h] = before;
        }
    }
    __syncthreads();
}

// After the keys above the boundary buckets are emitted and the buckets'
// keys listed (and a barrier): rank each listed bucket and emit its keys
// that belong to the top-k; a bucket too large for the list is ranked by the
// radix select over boundary(f), which calls f(h, okey, index) for every key
// of head h's boundary bucket on this thread.
template <int NH, class Boundary, class Emit>
__device__ __forceinline__ void topk_finish(TopkShared<NH>& T, Boundary&& boundary, Emit&& emit) {
    const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63;
    uint32_t fmask = 0;
#pragma unroll
    for (int h = 0; h < NH; ++h)
        if (T.mode[h] == 1u && T.bstar[h] >= 0 && T.cnt[h] > static_cast<uint32_t>(kListCap)) fmask |= 1u << h;
    for (int x = tid; x < NH * kListCap; x += nthr) {
        const int h = x / kListCap, e = x - h * kListCap;
        if (T.mode[h] == 1u && T.bstar[h] >= 0 && !((fmask >> h) & 1u))
            list_rank_pick(T.list[h], static_cast<int>(T.cnt[h]), T.want[h] - T.above[h], e, &T.thr[h]);
    }
    __syncthreads();
    for (int x = tid; x < NH * kListCap; x += nthr) {
        const int h = x / kListCap, e = x - h * kListCap;
        if (T.mode[h] == 1u && T.bstar[h] >= 0 && !((fmask >> h) & 1u) && e < static_cast<int>(T.cnt[h]) &&
            T.list[h][e] >= T.thr[h])
            emit(h, atomicAdd(&T.aux[h], 1u), T.list[h][e]);
    }
    if (fmask) {  // rare: a crowded boundary bucket, ranked by the radix select
        uint32_t fw[NH];
#pragma unroll
        for (int h = 0; h < NH; ++h) fw[h] = ((fmask >> h) & 1u) ? T.want[h] - T.above[h] : 0u;
        if (tid < NH) {
            T.kand[tid] = ~0ull;
            T.kor[tid] = 0ull;
        }
        __syncthreads();
        // the bits the bucket's keys share (equal scores share the whole score
        // half): the radix select skips the digits above the first that differs
        {
            uint64_t ka[NH], ko[NH];
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                ka[h] = ~0ull;
                ko[h] = 0ull;
            }
            boundary([&](int h, uint32_t ok, uint32_t idx) __attribute__((always_inline)) {
                if ((fmask >> h) & 1u) {
                    const uint64_t key = topk_key(ok, idx);
                    ka[h] &= key;
                    ko[h] |= key;
                }
            });
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                if (!((fmask >> h) & 1u)) continue;
                uint64_t a = ka[h], o = ko[h];
                for (int m = 1; m < 64; m <<= 1) {
                    a &= shfl_xor_u64(a, m);
                    o |= shfl_xor_u64(o, m);
                }
                if (lane == 0) {
                    atomicAnd(reinterpret_cast<unsigned long long*>(&T.kand[h]), static_cast<unsigned long long>(a));
                    atomicOr(reinterpret_cast<unsigned long long*>(&T.kor[h]), static_cast<unsigned long long>(o));
                }
            }
        }
        __syncthreads();
        block_select<NH>(T.S, fw, [&](auto&& visit) __attribute__((always_inline)) {
            boundary([&](int h, uint32_t ok, uint32_t idx) __attribute__((always_inline)) {
                if ((fmask >> h) & 1u) visit(h, topk_key(ok, idx));
            });
        }, true, T.kand, T.kor);
        __syncthreads();
        boundary([&](int h, uint32_t ok, uint32_t idx) __attribute__((always_inline)) {
            if (((fmask >> h) & 1u) && topk_key(ok, idx) >= T.S.thr[h])
                emit(h, atomicAdd(&T.aux[h], 1u), topk_key(ok, idx));
        });
        if (tid < NH && ((fmask >> tid) & 1u)) T.thr[tid] = T.S.thr[tid];
    }
    __syncthreads();
}

template <int NH, class Items, class Emit>
__device__ __forceinline__ void block_topk(TopkShared<NH>& T, const uint32_t (&want)[NH], const uint32_t (&total)[NH],
                           const uint32_t (&lo_ok)[NH], const uint32_t (&hi_ok)[NH], Items&& items,
                           Emit&& emit) {
    const bool any = topk_setup<NH>(T, want, total, lo_ok, hi_ok);
    // the heads' bucket maps in registers (the visitors' head numbers are
    // compile-time constants once inlined)
    uint32_t md[NH];
    float vmn[NH], scl[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        md[h] = T.mode[h];
        vmn[h] = T.vmin[h];
        scl[h] = T.scale[h];
    }
    if (any) {
        // (B) bucket histogram
        items([&](int h, uint32_t ok, uint32_t) __attribute__((always_inline)) {
            if (md[h] == 1u) atomicAdd(&T.S.hist[h][topk_bucket(ok, vmn[h], scl[h])], 1u);
        });
        __syncthreads();
        topk_rank<NH>(T);
    }
    // (C) emit the keys above the boundary bucket, list the boundary bucket
    int bst[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) bst[h] = T.bstar[h];
    items([&](int h, uint32_t ok, uint32_t idx) __attribute__((always_inline)) {
        if (md[h] == 2u) {
            emit(h, atomicAdd(&T.aux[h], 1u), topk_key(ok, idx));
        } else if (md[h] == 1u) {
            const int bk = topk_bucket(ok, vmn[h], scl[h]);
            const int bs = bst[h];
            if (bk > bs) {
                emit(h, atomicAdd(&T.aux[h], 1u), topk_key(ok, idx));
            } else if (bk == bs) {
                const uint32_t pos = atomicAdd(&T.cnt[h], 1u);
                if (pos < static_cast<uint32_t>(kListCap)) T.list[h][pos] = topk_key(ok, idx);
            }
        }
    });
    __syncthreads();
    if (!any) return;
    topk_finish<NH>(T, [&](auto&& f) __attribute__((always_inline)) {
        items([&](int h, uint32_t ok, uint32_t idx) __attribute__((always_inline)) {
            if (md[h] == 1u && topk_bucket(ok, vmn[h], scl[h]) == bst[h]) f(h, ok, idx);
        });
    }, emit);
}

// The same selection for keys at fixed per-thread slots, NS (a multiple of 4,
// at most 32) per thread, slot s holding a key of head (s / 4) % NH.  items(f) calls
// f(s, okey, index) for every key on this thread (the head is the slot's);
// fetch(s, g) calls g(okey, index) for slot s's key again.  The histogram
// pass keeps each key's bucket (a byte per slot), so classing a key later is
// one compare; the keys above the boundary bucket get positions from a block
// scan of per-thread counts and only those slots are visited to emit them.
template <int NH>
__host__ __device__ constexpr uint32_t topk_head_slots(int h) {
    uint32_t m = 0;
    for (int s = 0; s < 32; ++s)
        if ((s / 4) % NH == h) m |= 1u << s;
    return m;
}

template <int NH, int NS, class Items, class Fetch, class Emit>
__device__ __forceinline__ void block_topk_slots(TopkShared<NH>& T, const uint32_t (&want)[NH],
                                                 const uint32_t (&total)[NH], const uint32_t (&lo_ok)[NH],
                                                 const uint32_t (&hi_ok)[NH], Items&& items, Fetch&& fetch,
                                                 Emit&& emit) {
    const bool any = topk_setup<NH>(T, want, total, lo_ok, hi_ok);
    uint32_t md[NH];
    float vmn[NH], scl[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        md[h] = T.mode[h];
        vmn[h] = T.vmin[h];
        scl[h] = T.scale[h];
    }
    static_assert(NS % 4 == 0 && NS <= 32, "slots in words of four");
    // (B) bucket histogram; every key's bucket kept
    uint32_t pk[NS / 4];  // byte s % 4 of word s / 4: slot s's bucket
    uint32_t have = 0;
#pragma unroll
    for (int w = 0; w < NS / 4; ++w) pk[w] = 0;
    items([&](int s, uint32_t ok, uint32_t) __attribute__((always_inline)) {
        const int h = (s / 4) % NH;
        const int bk = topk_bucket(ok, vmn[h], scl[h]);
        if (md[h] == 1u) atomicAdd(&T.S.hist[h][bk], 1u);
        pk[s / 4] |= static_cast<uint32_t>(bk) << (8 * (s % 4));
        have |= 1u << s;
    });
    if (any) {
        __syncthreads();
        topk_rank<NH>(T);
    }
    // (C) classes: above the boundary bucket (emitted), in it (listed); a
    //     head emitting everything has bst -1, an idle head 256
    int bst[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) bst[h] = md[h] == 2u ? -1 : md[h] == 1u ? T.bstar[h] : kTopBuckets;
    uint32_t emask = 0, lmask = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int bk = static_cast<int>((pk[s / 4] >> (8 * (s % 4))) & 0xFFu);
        emask |= bk > bst[(s / 4) % NH] ? 1u << s : 0u;
        lmask |= bk == bst[(s / 4) % NH] ? 1u << s : 0u;
    }
    emask &= have;
    lmask &= have;
    // positions of the emitted keys: a wave scan of the per-thread counts and
    // one counter add per wave and head (T.aux starts at 0; it ends at the
    // number of keys above the boundary buckets, where the list stage goes on)
    uint32_t cnt[NH];
    {
        const int lane = threadIdx.x & 63;
        uint32_t c[NH], incl[NH], wb[NH];
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            c[h] = static_cast<uint32_t>(__builtin_popcount(emask & topk_head_slots<NH>(h)));
            incl[h] = wave_incl_scan(c[h]);
            const uint32_t tot = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl[h]), 63));
            wb[h] = (lane == 0 && tot) ? atomicAdd(&T.aux[h], tot) : 0u;
        }
#pragma unroll
        for (int h = 0; h < NH; ++h)
            cnt[h] = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(wb[h]), 0)) + incl[h] - c[h];
    }
    // (D) list the boundary buckets' keys, then emit the keys above them: one
    //     pass over each mask, a key's position its wave's base plus the
    //     head's emitted slots below it on this thread
    {
        uint32_t m = lmask;
        while (m) {
            const int s = __builtin_ctz(m);
            m &= m - 1;
            const int h = (s / 4) % NH;
            fetch(s, [&](uint32_t ok, uint32_t idx) __attribute__((always_inline)) {
                const uint32_t p = atomicAdd(&T.cnt[h], 1u);
                if (p < static_cast<uint32_t>(kListCap)) T.list[h][p] = topk_key(ok, idx);
            });
        }
        m = emask;
        while (m) {
            const int s = __builtin_ctz(m);
            m &= m - 1;
            const int h = (s / 4) % NH;
            uint32_t p = cnt[0];
#pragma unroll
            for (int hh = 1; hh < NH; ++hh) p = h == hh ? cnt[hh] : p;
            p += static_cast<uint32_t>(__builtin_popcount(emask & (topk_head_slots<NH>(0) << (4 * h)) & ((1u << s) - 1u)));
            fetch(s, [&](uint32_t ok, uint32_t idx) __attribute__((always_inline)) { emit(h, p, topk_key(ok, idx)); });
        }
    }
    __syncthreads();
    if (!any) return;
    topk_finish<NH>(T, [&](auto&& f) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int h = (s / 4) % NH;
            if (((lmask >> s) & 1u) && md[h] == 1u)
                fetch(s, [&](uint32_t ok, uint32_t idx) __attribute__((always_inline)) { f(h, ok, idx); });
        }
    }, emit);
}

// ---------------------------------------------------------------------------
// Sampler threshold of one head from the histogram of the Philox words' top
// kSampBits.  S.hist holds the head's tail histogram.  For rank > 0 the result
// S.thr = sample_key of the rank-th smallest (word, index) of the tail, so the
// first `rank` tail tokens of the sample order are exactly those with
// sample_key >= S.thr.  The tokens of the boundary bin come from the
// predictor's bin-sorted chunk lists (BinLists); `in_fixed(i)` tells whether
// token i is in the head's fixed set (those are not in the tail).
// ---------------------------------------------------------------------------
struct HeadSamp {
    uint32_t hist[kSampBins];
    uint64_t list[kListCap];
    uint64_t thr;
    uint32_t before, cnt;
    int bin;
};

// Chunk c of the middle holds its tokens grouped by bin: bin x of chunk c is
// slist[c * cp + soff[c][x] .. c * cp + soff[c][x + 1]), each entry the token's
// offset from the chunk's first token, c * cp.  Chunks are the
// predictor's; only those overlapping the middle [lo, hi) were written.
struct BinLists {
    const uint32_t* soff;  // [nchunks][kSampBins + 1]
    const uint16_t* slist;  // [nchunks][cp] token offsets within the chunk
    int nchunks, cp, lo, hi;
};

template <class WordOf, class InFixed>
__device__ __forceinline__ void head_sample_threshold(HeadSamp& S, SelShared<1>& F, const BinLists BL,
                                                      WordOf&& word_of_token, uint32_t rank,
                                                      InFixed&& in_fixed) {
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int lane = tid & 63, wave = tid >> 6, nwaves = nthr >> 6;
    if (tid == 0) {
        S.cnt = 0;
        S.thr = 0;
    }
    if (rank == 0) {  // block-uniform
        __syncthreads();
        return;
    }
    if (wave == 0) {
        int bin;
        uint32_t before;
        wave_rank_bin<kSampBins>(S.hist, rank, false, bin, before);
        if (lane == 0) {
            S.bin = bin;
            S.before = before;
        }
    }
    __syncthreads();
    const int bn = S.bin;
    if (bn < 0) return;  // fewer tail tokens than `rank`: excluded by the callers
    const uint32_t r = rank - S.before;
    // every tail token of the boundary bin, wave per chunk
    auto each = [&](auto&& f) __attribute__((always_inline)) {
        for (int c = wave; c < BL.nchunks; c += nwaves) {
            if (max(c * BL.cp, BL.lo) >= min((c + 1) * BL.cp, BL.hi)) continue;
            const uint32_t* off = BL.soff + static_cast<size_t>(c) * (kSampBins + 1) + bn;
            const uint32_t a = off[0], e = off[1];
            const uint16_t* lst = BL.slist + static_cast<size_t>(c) * BL.cp;
            for (uint32_t p = a + lane; p < e; p += 64) {
                const int i = c * BL.cp + static_cast<int>(lst[p]);
                if (!in_fixed(i)) f(sample_key(word_of_token(i), static_cast<uint32_t>(i)));
            }
        }
    };
    each([&](uint64_t key) __attribute__((always_inline)) {
        const uint32_t pos = atomicAdd(&S.cnt, 1u);
        if (pos < static_cast<uint32_t>(kListCap)) S.list[pos] = key;
    });
    __syncthreads();
    const uint32_t cnt = S.cnt;
    if (cnt <= static_cast<uint32_t>(kListCap)) {
        for (int x = tid; x < static_cast<int>(cnt); x += nthr) list_rank_pick(S.list, static_cast<int>(cnt), r, x, &S.thr);
        __syncthreads();
    } else {  // rare: a crowded bin, ranked by the radix select over its tokens
        const uint32_t fw[1] = {r};
        block_select<1>(F, fw, [&](auto&& visit) __attribute__((always_inline)) {
            each([&](uint64_t key) __attribute__((always_inline)) { visit(0, key); });
        }, true);
        if (tid == 0) S.thr = F.thr[0];
        __syncthreads();
    }
}

}  // namespace vattn
