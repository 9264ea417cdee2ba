// Device helpers shared by the libspecv kernels (gfx950, wave64): the
// Philox4x32-10 generator, hand-off words, row loads into registers, and
// DPP wave reductions / scans.  Included by each kernel source.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "specv_internal.hpp"

namespace specv {
namespace {

// uniform purposes (third Philox counter word)
enum Purpose { PURPOSE_DRAFT = 0, PURPOSE_ACCEPT = 1, PURPOSE_RESIDUAL = 2, PURPOSE_BONUS = 3 };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kInf = __builtin_huge_valf();
constexpr int kSpinLimit = kDefaultWaitLimit;

// Polls a bounded wait makes before it gives up (the row is flagged
// INTERNAL).  kSpinLimit, unless a failure-path test lowers it through
// specv_debug_set_wait_limit; each translation unit holds its own copy.
__device__ int g_wait_limit = kSpinLimit;

__host__ inline hipError_t set_wait_limit_here(int n) {
    return hipMemcpyToSymbol(HIP_SYMBOL(g_wait_limit), &n, sizeof(int));
}

// ---------------------------------------------------------------- Philox
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two
// 32x32->64 multiplies, key bumped by the Weyl constants between rounds.
__device__ inline uint4 philox4x32_10(uint4 c, unsigned k0, unsigned k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const unsigned lo0 = 0xD2511F53u * c.x;
        const unsigned hi0 = __umulhi(0xD2511F53u, c.x);
        const unsigned lo1 = 0xCD9E8D57u * c.z;
        const unsigned hi1 = __umulhi(0xCD9E8D57u, c.z);
        c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
    }
    return c;
}

// u = (word0 >> 8) * 2^-24 for counter (b, i, purpose, step).
__device__ inline float uniform24(unsigned long long seed, unsigned b, unsigned i,
                                  unsigned purpose, unsigned step) {
    const uint4 r = philox4x32_10(make_uint4(b, i, purpose, step), (unsigned)seed,
                                  (unsigned)(seed >> 32));
    return (float)(r.x >> 8) * 5.9604644775390625e-08f;
}

// ---------------------------------------------------------------- helpers
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Hand-off between workgroups of one launch.  Published values are written
// and read with agent-scope atomic accesses, which are coherent across the
// XCDs' L2 caches by themselves, so no L2 write-back / invalidate is needed
// (a __threadfence() would flush the whole L2 of the XCD).  ``wait_stores``
// makes this wave's outstanding stores complete before a later atomic, and
// keeps the compiler from moving memory accesses across it.
template <typename T>
__device__ inline void publish(T* p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ inline T published(const T* p) {
    return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Bump an arrival counter; returns the previous count.  With ``ordered`` the
// thread's earlier stores complete first, for readers that do not check
// epoch tags; without it the atomic goes out behind them at once.
__device__ inline unsigned arrive(unsigned* counter, bool ordered) {
    if (ordered) wait_stores();
    return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Epoch-tagged 64-bit words: (epoch << 32) | value.
__device__ inline void put_tagged(unsigned long long* p, unsigned v, unsigned epoch) {
    publish(p, ((unsigned long long)epoch << 32) | v);
}
__device__ inline bool tag_is(unsigned long long w, unsigned epoch) {
    return (unsigned)(w >> 32) == epoch;
}

__device__ inline unsigned long long readlane64(unsigned long long v, int lane) {
    const unsigned lo = __builtin_amdgcn_readlane((unsigned)v, lane);
    const unsigned hi = __builtin_amdgcn_readlane((unsigned)(v >> 32), lane);
    return ((unsigned long long)hi << 32) | lo;
}

__device__ inline float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

template <bool BF16>
__device__ inline float load_elem(const void* row, long long v) {
    if constexpr (BF16) {
        const unsigned short h = static_cast<const unsigned short*>(row)[v];
        return __uint_as_float((unsigned)h << 16);
    } else {
        return static_cast<const float*>(row)[v];
    }
}

template <bool BF16>
__device__ inline const void* row_ptr(const void* base, long long stride_b, long long stride_p,
                                      int b, int i) {
    const long long off = (long long)b * stride_b + (long long)i * stride_p;
    if constexpr (BF16) {
        return static_cast<const unsigned short*>(base) + off;
    } else {
        return static_cast<const float*>(base) + off;
    }
}

template <bool BF16>
__device__ inline void unpack16(const uint4& q, float* x) {
    if constexpr (BF16) {
        x[0] = bf16_lo(q.x);
        x[1] = bf16_hi(q.x);
        x[2] = bf16_lo(q.y);
        x[3] = bf16_hi(q.y);
        x[4] = bf16_lo(q.z);
        x[5] = bf16_hi(q.z);
        x[6] = bf16_lo(q.w);
        x[7] = bf16_hi(q.w);
    } else {
        x[0] = __uint_as_float(q.x);
        x[1] = __uint_as_float(q.y);
        x[2] = __uint_as_float(q.z);
        x[3] = __uint_as_float(q.w);
    }
}

// Index (within the chunk) of entry k of this thread's x[]: 16-byte groups,
// group g = j * kBlock + tid holds entries [g * G, g * G + G), so each load
// instruction of the workgroup covers one contiguous 4 KB span.
template <bool BF16>
__device__ inline int chunk_index(int k) {
    constexpr int G = BF16 ? 8 : 4;
    return ((k / G) * kBlock + (int)threadIdx.x) * G + (k % G);
}

// w[i] for a per-lane index i, by a tree of selects over the register array
// (indexing it directly would put the array in private memory).
template <int N>
__device__ inline unsigned pick_word(const unsigned (&w)[N], int i) {
    unsigned t[N];
#pragma unroll
    for (int j = 0; j < N; ++j) t[j] = w[j];
#pragma unroll
    for (int s = 1; s < N; s <<= 1) {
        const bool hi = (i & s) != 0;
#pragma unroll
        for (int j = 0; j + s < N; j += 2 * s) t[j] = hi ? t[j + s] : t[j];
    }
    return t[0];
}

// One chunk of one logits row held in registers, in chunk_index's layout;
// entries past the row's end read as -inf.
//   VEC:  packed 16-byte groups (bfloat16: 8 entries, float32: 4); every
//         load is issued before any is used (``issue``), groups past the last
//         whole group load group 0 and are overwritten by ``finish``, which
//         also fills a partial last group with scalar loads.
//   !VEC: scalar loads (rows not 16-byte aligned), held as float.
template <bool BF16, bool VEC>
struct ChunkRegs;

template <bool BF16>
struct ChunkRegs<BF16, true> {
    static constexpr int G = BF16 ? 8 : 4;
    static constexpr int NG = kPerThread / G;
    uint4 q[NG];

    __device__ inline void issue(const void* row, int v0, int len) {
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const char*>(row) +
                                                        (size_t)v0 * (BF16 ? 2 : 4));
        const int full = len / G;
        if (full == 0) return;                   // nothing 16-byte loadable (tiny tail)
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            const int g = j * kBlock + (int)threadIdx.x;
            q[j] = p[g < full ? g : 0];
        }
    }
    __device__ inline void finish(const void* row, int v0, int len) {
        const int full = len / G;
        const int rem = len - full * G;
        const unsigned ninf = BF16 ? 0xFF80FF80u : 0xFF800000u;
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            const int g = j * kBlock + (int)threadIdx.x;
            if (g >= full) {
                q[j] = make_uint4(ninf, ninf, ninf, ninf);
                if (g == full && rem) {
                    unsigned w[4] = {ninf, ninf, ninf, ninf};
#pragma unroll
                    for (int e = 0; e < G; ++e) {
                        if (e < rem) {
                            if constexpr (BF16) {
                                const unsigned h = static_cast<const unsigned short*>(row)[v0 + full * G + e];
                                w[e / 2] = (e & 1) ? ((w[e / 2] & 0xFFFFu) | (h << 16))
                                                   : ((w[e / 2] & 0xFFFF0000u) | h);
                            } else {
                                w[e] = __float_as_uint(static_cast<const float*>(row)[v0 + full * G + e]);
                            }
                        }
                    }
                    q[j] = make_uint4(w[0], w[1], w[2], w[3]);
                }
            }
        }
    }
    __device__ inline void get(float (&x)[kPerThread]) const {
#pragma unroll
        for (int j = 0; j < NG; ++j) unpack16<BF16>(q[j], &x[j * G]);
    }
    // entry i (a compile-time constant in unrolled loops) unpacked on the fly
    __device__ inline float elem(int i) const {
        const uint4& g = q[i / G];
        const int e = i % G;
        if constexpr (BF16) {
            const unsigned w = (e / 2) == 0 ? g.x : (e / 2) == 1 ? g.y : (e / 2) == 2 ? g.z : g.w;
            return (e & 1) ? bf16_hi(w) : bf16_lo(w);
        } else {
            return __uint_as_float(e == 0 ? g.x : e == 1 ? g.y : e == 2 ? g.z : g.w);
        }
    }
    // entry i for a per-lane i
    __device__ inline float elem_dyn(int i) const {
        unsigned w[4 * NG];
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            w[4 * j] = q[j].x;
            w[4 * j + 1] = q[j].y;
            w[4 * j + 2] = q[j].z;
            w[4 * j + 3] = q[j].w;
        }
        if constexpr (BF16) {
            const unsigned x = pick_word(w, i >> 1);
            return (i & 1) ? bf16_hi(x) : bf16_lo(x);
        } else {
            return __uint_as_float(pick_word(w, i));
        }
    }
};

template <bool BF16>
struct ChunkRegs<BF16, false> {
    static constexpr int G = BF16 ? 8 : 4;
    static constexpr int NG = kPerThread / G;
    float x[kPerThread];

    __device__ inline void issue(const void* row, int v0, int len) {
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) {
            const int v = chunk_index<BF16>(k);
            x[k] = load_elem<BF16>(row, (long long)v0 + (v < len ? v : len - 1));
        }
    }
    __device__ inline void finish(const void*, int, int len) {
#pragma unroll
        for (int k = 0; k < kPerThread; ++k)
            if (chunk_index<BF16>(k) >= len) x[k] = -kInf;
    }
    __device__ inline void get(float (&y)[kPerThread]) const {
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) y[k] = x[k];
    }
    __device__ inline float elem(int i) const { return x[i]; }
    __device__ inline float elem_dyn(int i) const {
        unsigned w[kPerThread];
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) w[k] = __float_as_uint(x[k]);
        return __uint_as_float(pick_word(w, i));
    }
};

// Merge (m, s) statistics: s is relative to m in units of exp2(. * scale).
__device__ inline void merge_ms(float& m, float& s, float m2, float s2, float scale) {
    const float M = fmaxf(m, m2);
    if (M == -kInf) {            // both empty; keep NaN visible
        s = s + s2;
        m = M;
        return;
    }
    s = s * fast_exp2((m - M) * scale) + s2 * fast_exp2((m2 - M) * scale);
    m = M;
}

// ---------------------------------------------------------------- wave64 DPP
// Cross-lane moves by DPP (VALU-speed, no LDS round trip).  Lanes whose
// source is outside the pattern or masked off receive ``old``, the identity
// of the operation being built.
constexpr int kDppQuad1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuad2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15 - i within 16
constexpr int kDppBcast15 = 0x142;    // lane 15 of a row -> the next row
constexpr int kDppBcast31 = 0x143;    // lane 31 -> rows 2 and 3
constexpr int kDppShr = 0x110;        // + n: row_shr:n

template <int CTRL, int ROW_MASK = 0xF>
__device__ inline int dpp_i(int v, int old) {
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ inline float dpp_f(float v, float old) {
    return __int_as_float(dpp_i<CTRL, ROW_MASK>(__float_as_int(v), __float_as_int(old)));
}

// Wave reduction of a value pair with a combine functor: quads, half rows,
// rows, then rows 0+1 -> 1, 2+3 -> 3, rows 0..2 -> 3; the total ends in lane
// 63 and is broadcast.
template <typename Comb>
__device__ inline void wave_reduce2(float& x, int& y, float idx, int idy, Comb comb) {
#define SPECV_DPP_STEP(CTRL, MASK)                                          \
    {                                                                       \
        const float x2 = dpp_f<CTRL, MASK>(x, idx);                         \
        const int y2 = dpp_i<CTRL, MASK>(y, idy);                           \
        comb(x, y, x2, y2);                                                 \
    }
    SPECV_DPP_STEP(kDppQuad1, 0xF)
    SPECV_DPP_STEP(kDppQuad2, 0xF)
    SPECV_DPP_STEP(kDppHalfMirror, 0xF)
    SPECV_DPP_STEP(kDppMirror, 0xF)
    SPECV_DPP_STEP(kDppBcast15, 0xA)
    SPECV_DPP_STEP(kDppBcast31, 0xC)
#undef SPECV_DPP_STEP
    x = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), kWave - 1));
    y = __builtin_amdgcn_readlane(y, kWave - 1);
}

__device__ inline void wave_merge_ms(float& m, float& s, float scale) {
    int si = __float_as_int(s);
    wave_reduce2(m, si, -kInf, 0, [scale](float& m1, int& s1, float m2, int s2) {
        float sa = __int_as_float(s1);
        merge_ms(m1, sa, m2, __int_as_float(s2), scale);
        s1 = __float_as_int(sa);
    });
    s = __int_as_float(si);
}

// (value, index) argmax merge: larger value wins, lower index on ties.
__device__ inline void merge_arg(float& v, int& i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) {
        v = v2;
        i = i2;
    }
}

__device__ inline void wave_merge_arg(float& v, int& i) {
    wave_reduce2(v, i, -kInf, 0x7fffffff, [](float& v1, int& i1, float v2, int i2) {
        merge_arg(v1, i1, v2, i2);
    });
}

__device__ inline float wave_sum(float x) {
    int dummy = 0;
    wave_reduce2(x, dummy, 0.f, 0, [](float& a, int&, float b, int) { a += b; });
    return x;
}

__device__ inline float wave_max(float x) {
    int dummy = 0;
    wave_reduce2(x, dummy, -kInf, 0, [](float& a, int&, float b, int) { a = fmaxf(a, b); });
    return x;
}

__device__ inline unsigned wave_or(unsigned x) {
    float dummy = 0.f;
    int xi = (int)x;
    wave_reduce2(dummy, xi, 0.f, 0, [](float&, int& a, float, int b) { a |= b; });
    return (unsigned)xi;
}

__device__ inline int wave_min_int(int x) {
    float dummy = 0.f;
    wave_reduce2(dummy, x, 0.f, 0x7fffffff, [](float&, int& a, float, int b) { a = min(a, b); });
    return x;
}

__device__ inline int wave_max_int(int x) {
    float dummy = 0.f;
    wave_reduce2(dummy, x, 0.f, (int)0x80000000, [](float&, int& a, float, int b) { a = max(a, b); });
    return x;
}

// Inclusive prefix sums across the wave (lane order).
__device__ inline float wave_scan_incl(float x) {
    x += dpp_f<kDppShr + 1>(x, 0.f);
    x += dpp_f<kDppShr + 2>(x, 0.f);
    x += dpp_f<kDppShr + 4>(x, 0.f);
    x += dpp_f<kDppShr + 8>(x, 0.f);
    x += dpp_f<kDppBcast15, 0xA>(x, 0.f);
    x += dpp_f<kDppBcast31, 0xC>(x, 0.f);
    return x;
}

__device__ inline int wave_scan_incl(int x) {
    x += dpp_i<kDppShr + 1>(x, 0);
    x += dpp_i<kDppShr + 2>(x, 0);
    x += dpp_i<kDppShr + 4>(x, 0);
    x += dpp_i<kDppShr + 8>(x, 0);
    x += dpp_i<kDppBcast15, 0xA>(x, 0);
    x += dpp_i<kDppBcast31, 0xC>(x, 0);
    return x;
}


// A (value, value) pair as two epoch-tagged words, e.g. a chunk's statistics.
__device__ inline void publish_stats(unsigned long long* w, float m, unsigned second, unsigned epoch) {
    put_tagged(w, __float_as_uint(m), epoch);
    put_tagged(w + 1, second, epoch);
}
// Returns false when the words did not carry this call's tag within the bound.
__device__ inline bool published_stats(const unsigned long long* w, unsigned epoch, float& m,
                                       unsigned& second) {
    unsigned long long w0 = 0, w1 = 0;
    bool ok = false;
    for (int spin = 0; spin < g_wait_limit; ++spin) {
        w0 = published(w);
        w1 = published(w + 1);
        if (tag_is(w0, epoch) && tag_is(w1, epoch)) {
            ok = true;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    m = __uint_as_float((unsigned)w0);
    second = (unsigned)w1;
    return ok;
}

// ---------------------------------------------------------------- chunk reductions
// Statistics of the chunk entries a wave holds in registers (any ChunkRegs),
// merged across the wave; every lane gets the result.
//   wave_chunk_ms:     max m and sum of exp2((z - m) * scale); the sum is NaN
//                      when an entry is NaN or +inf, and 0 (m = -inf) when no
//                      entry is finite;
//   wave_chunk_argmax: max and lowest index of the max (v0 + chunk index), and
//                      whether an entry is NaN or +inf.
template <typename Regs>
__device__ __forceinline__ void wave_chunk_ms(const Regs& r, float scale, float& m, float& s,
                                              float* thread_max = nullptr) {
    float cm = -kInf;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) cm = fmaxf(cm, r.elem(i));
    if (thread_max) *thread_max = cm;           // this thread's maximum (NaN ignored)
    const float nms = cm == -kInf ? 0.f : -cm * scale;
    s = 0.f;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) s += fast_exp2(fmaf(r.elem(i), scale, nms));
    m = cm;
    wave_merge_ms(m, s, scale);
}

// wave_chunk_ms's statistics, bit for bit (the same sums in the same
// order), that also leave this thread's maximum and the sums of its NG
// groups of entries (entries i = j * (kPerThread / NG) + e, e ascending), in
// the thread's own units exp2((z - thread max) * scale).
template <int NG, typename Regs>
__device__ __forceinline__ void wave_chunk_ms_groups(const Regs& r, float scale, float& m, float& s,
                                                     float (&gsum)[NG], float& thread_max) {
    constexpr int G = kPerThread / NG;
    float cm = -kInf;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) cm = fmaxf(cm, r.elem(i));
    thread_max = cm;
    const float nms = cm == -kInf ? 0.f : -cm * scale;
    s = 0.f;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
        float g = 0.f;
#pragma unroll
        for (int e = 0; e < G; ++e) {
            const float x = fast_exp2(fmaf(r.elem(j * G + e), scale, nms));
            s += x;
            g += x;
        }
        gsum[j] = g;
    }
    m = cm;
    wave_merge_ms(m, s, scale);
}

template <bool BF16, typename Regs>
__device__ __forceinline__ void wave_chunk_argmax(const Regs& r, int v0, float& best, int& bi,
                                                  unsigned& bad) {
    best = -kInf;
    bi = 0x7fffffff;
    bad = 0;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        const float x = r.elem(i);
        bad |= !(x <= 3.402823466e38f);           // NaN or +inf
        if (x > best) {                           // strict: keeps the lowest index
            best = x;
            bi = v0 + chunk_index<BF16>(i);
        }
    }
    wave_merge_arg(best, bi);
    bad = wave_or(bad);
}

// ---------------------------------------------------------------- chunk draw
// Inverse CDF inside one chunk held in registers by the whole workgroup
// (chunk_index layout): w[] are this thread's entry weights, gw[] the sums
// of its G-entry groups, and the chunk's running sum starts at ``base``.
// Entries are taken in ascending index order.  Returns, to every thread, the
// chunk index of the first entry whose running sum exceeds ``target``, else
// (rounding) the last entry with weight, else -1.  Whole workgroup.
template <bool BF16>
__device__ __forceinline__ int chunk_inverse_cdf(const float (&w)[kPerThread],
                                                 const float (&gw)[kPerThread / (BF16 ? 8 : 4)],
                                                 float base, float target) {
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    constexpr int G = BF16 ? 8 : 4;
    constexpr int NG = kPerThread / G;
    // prefix sums of the group weights in token order: group (j, tid) comes
    // after every group (j', *) with j' < j and every (j, tid') with tid' < tid
    __shared__ float gtot[NG][kWaves];
    __shared__ int tokW[kWaves], lastW[kWaves];
    float incl[NG];
#pragma unroll
    for (int j = 0; j < NG; ++j) {
        incl[j] = wave_scan_incl(gw[j]);
        if (lane == kWave - 1) gtot[j][wave] = incl[j];
    }
    __syncthreads();
    float gbase = base;
    int tok = 0x7fffffff, lastpos = -1;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
        float before = 0.f, tot = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < kWaves; ++w2) {
            const float g = gtot[j][w2];
            if (w2 < wave) before += g;
            tot += g;
        }
        const float start = gbase + before + (incl[j] - gw[j]);
        float run = start;
        int first = -1, lastin = -1;
#pragma unroll
        for (int e = 0; e < G; ++e) {
            const float wk = w[j * G + e];
            run += wk;
            if (wk > 0.f) {
                lastin = e;
                if (first < 0 && run > target) first = e;
            }
        }
        const int g = j * kBlock + tid;
        if (lastin >= 0) lastpos = g * G + lastin;
        if (tok == 0x7fffffff && gw[j] > 0.f && start + gw[j] > target)
            tok = g * G + (first >= 0 ? first : lastin);
        gbase += tot;
    }
    // the first token past u * W, and the last token with weight (for
    // rounding), reduced per wave then across the four waves
    tok = wave_min_int(tok);
    lastpos = wave_max_int(lastpos);
    if (lane == 0) {
        tokW[wave] = tok;
        lastW[wave] = lastpos;
    }
    __syncthreads();
    int t = tokW[0], l = lastW[0];
    for (int w2 = 1; w2 < kWaves; ++w2) {
        t = min(t, tokW[w2]);
        l = max(l, lastW[w2]);
    }
    return t == 0x7fffffff ? l : t;
}

}  // namespace
}  // namespace specv
