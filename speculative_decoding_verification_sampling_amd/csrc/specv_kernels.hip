// libspecv kernels for gfx950 (CDNA4, wave64).
//
// The verify step is bandwidth-bound: every logits row that the round may
// consult is streamed from HBM once with 16-byte loads, reduced to per-chunk
// statistics, and the sequential part of the round (accept tests, stopping
// at the first rejection) runs on those statistics.  Only the one row pair
// that is actually sampled from is read a second time.
//
//   k_rowstats  grid (chunks, B * (2*gamma+1)): one workgroup per 8192-entry
//               chunk of one logits row.  Sampling rows: chunk max and
//               sum of exp2((z - max) * log2(e) / T).  Greedy rows: chunk max
//               and its lowest index.  Rows a round cannot consult (past the
//               cap / first EOS, draft rows of greedy rows) are skipped.
//   k_decide    grid (chunks, B): every workgroup of a batch row combines
//               the statistics, draws the accept uniforms and finds the first
//               rejection (cheap, done redundantly); each then sums the
//               correction weights max(p - q, 0) of its chunk (or takes the
//               bonus row's chunk mass from the statistics).  The last
//               workgroup of the row to finish (atomic counter) picks the
//               chunk that holds u * W, rescans it with a block prefix sum and
//               writes the outputs.
//
// Sources: "11.1 核心原理: Draft + Verify 与 Rejection Sampling" (11.1.1
// alignment, 11.1.2 acceptance / residual / greedy, pseudo-code 10-1) and
// "Fast Inference from Transformers via Speculative Decoding" (speculative
// sampling, bonus token).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "specv_internal.hpp"

namespace specv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kInf = __builtin_huge_valf();

enum Mode { MODE_SAMPLE = 0, MODE_GREEDY = 1, MODE_TRUNC = 2, MODE_SKIP = 3 };
enum Kind { KIND_NONE = 0, KIND_RESIDUAL = 1, KIND_BONUS = 2 };
enum Purpose { PURPOSE_ACCEPT = 1, PURPOSE_RESIDUAL = 2, PURPOSE_BONUS = 3 };

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
// makes this wave's outstanding stores complete before the arrival counter is
// bumped, and keeps the compiler from moving memory accesses across it.
__device__ inline void publish(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void publish(int* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void publish(unsigned* p, unsigned v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float published(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline int published(const int* p) {
    return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline unsigned published(const unsigned* p) {
    return __hip_atomic_load(const_cast<unsigned*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Bump the arrival counter after this thread's published stores completed;
// returns the previous count.
__device__ inline unsigned arrive(unsigned* counter) {
    wait_stores();
    const unsigned old =
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_stores();
    return old;
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

// Load this thread's 32 entries of a chunk into x[]; entries past ``len``
// read as -inf.  Layout: 16-byte groups, group g = j * kBlock + tid, so each
// load instruction of the workgroup covers one contiguous 4 KB span.  Every
// load is issued before any value is used: out-of-range groups load a clamped
// in-range address and are masked afterwards (no branch around a load).
template <bool BF16, bool VEC>
__device__ inline void load_chunk(const void* row, int v0, int len, float (&x)[kPerThread]) {
    const int tid = threadIdx.x;
    constexpr int G = BF16 ? 8 : 4;                 // entries per 16-byte group
    constexpr int NG = kPerThread / G;              // groups per thread
    if constexpr (VEC) {
        const uint4* p = reinterpret_cast<const uint4*>(
            static_cast<const char*>(row) + (size_t)v0 * (BF16 ? 2 : 4));
        if (len == kChunk) {
            uint4 q[NG];
#pragma unroll
            for (int j = 0; j < NG; ++j) q[j] = p[j * kBlock + tid];
#pragma unroll
            for (int j = 0; j < NG; ++j) unpack16<BF16>(q[j], &x[j * G]);
            return;
        }
        if (len >= G) {
            const int full = len / G;               // groups entirely inside the chunk
            uint4 q[NG];
#pragma unroll
            for (int j = 0; j < NG; ++j) {
                const int g = j * kBlock + tid;
                q[j] = p[g < full ? g : 0];
            }
#pragma unroll
            for (int j = 0; j < NG; ++j) {
                unpack16<BF16>(q[j], &x[j * G]);
                if (j * kBlock + tid >= full) {
#pragma unroll
                    for (int e = 0; e < G; ++e) x[j * G + e] = -kInf;
                }
            }
            // entries of the one partial group at the end, if any
            const int rem = len - full * G;
            if (rem && tid == full % kBlock) {
#pragma unroll
                for (int j = 0; j < NG; ++j) {
                    if (j == full / kBlock) {
#pragma unroll
                        for (int e = 0; e < G; ++e)
                            if (e < rem) x[j * G + e] = load_elem<BF16>(row, (long long)v0 + full * G + e);
                    }
                }
            }
            return;
        }
    }
    float t[kPerThread];
#pragma unroll
    for (int j = 0; j < NG; ++j) {
#pragma unroll
        for (int e = 0; e < G; ++e) {
            const int v = (j * kBlock + tid) * G + e;
            t[j * G + e] = load_elem<BF16>(row, (long long)v0 + (v < len ? v : len - 1));
        }
    }
#pragma unroll
    for (int j = 0; j < NG; ++j) {
#pragma unroll
        for (int e = 0; e < G; ++e) {
            const int v = (j * kBlock + tid) * G + e;
            x[j * G + e] = v < len ? t[j * G + e] : -kInf;
        }
    }
}

// Load entries [tid * 32, tid * 32 + 32) of a chunk (contiguous per thread,
// for the in-order prefix sum); entries past ``len`` read as -inf.
template <bool BF16, bool VEC>
__device__ inline void load_contig(const void* row, int v0, int len, float (&x)[kPerThread]) {
    const int tid = threadIdx.x;
    constexpr int G = BF16 ? 8 : 4;
    constexpr int NG = kPerThread / G;
    const int base = tid * kPerThread;
    if constexpr (VEC) {
        if (len >= G) {
            const uint4* p = reinterpret_cast<const uint4*>(
                static_cast<const char*>(row) + (size_t)v0 * (BF16 ? 2 : 4));
            const int full = len / G;
            uint4 q[NG];
#pragma unroll
            for (int j = 0; j < NG; ++j) {
                const int g = base / G + j;
                q[j] = p[g < full ? g : 0];
            }
#pragma unroll
            for (int j = 0; j < NG; ++j) {
                unpack16<BF16>(q[j], &x[j * G]);
                if (base / G + j >= full) {
#pragma unroll
                    for (int e = 0; e < G; ++e) x[j * G + e] = -kInf;
                }
            }
            const int rem = len - full * G;
            if (rem && full * G >= base && full * G < base + kPerThread) {
#pragma unroll
                for (int j = 0; j < NG; ++j) {
                    if (base / G + j == full) {
#pragma unroll
                        for (int e = 0; e < G; ++e)
                            if (e < rem) x[j * G + e] = load_elem<BF16>(row, (long long)v0 + full * G + e);
                    }
                }
            }
            return;
        }
    }
    float t[kPerThread];
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        const int v = base + k;
        t[k] = load_elem<BF16>(row, (long long)v0 + (v < len ? v : len - 1));
    }
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) x[k] = base + k < len ? t[k] : -kInf;
}

// Index (within the chunk) of entry k of this thread's x[] in load_chunk's layout.
template <bool BF16>
__device__ inline int chunk_index(int k) {
    constexpr int G = BF16 ? 8 : 4;
    return ((k / G) * kBlock + (int)threadIdx.x) * G + (k % G);
}

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

__device__ inline int wave_max_i(int x) {
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

// ---------------------------------------------------------------- row plan
// What one batch row needs, from its parameters and draft tokens alone.
struct Plan {
    int mode;
    int cap;        // tokens the round may emit: max_new_tokens and the first EOS
    int nt;         // target rows the round may consult
    int nd;         // draft rows the round may consult
    float scale;    // log2(e) / T
    int top_k;
    float top_p;
    int keff;       // truncated rows: candidates wanted per chunk (top_k, or the handle's
                    // max_top_k for top-p alone)
    int kmode;      // truncated rows: 1 when top-k is on (normaliser over the top-k set)
    unsigned flags;
};

__device__ inline Plan make_plan(const Args& a, int b) {
    Plan p;
    float T = 0.f;
    int k = 0;
    float tp = 1.f;
    int cap = 0;
    if (a.params) {
        const specv_row_params rp = a.params[b];
        T = rp.temperature;
        k = rp.top_k;
        tp = rp.top_p;
        cap = rp.max_new_tokens;
    } else if (a.caps) {
        cap = a.caps[b];
    }
    // emission ends after max_new_tokens tokens and after an emitted EOS; an
    // EOS among the drafts therefore caps the round at its position + 1
    int ce = cap >= 1 ? cap : 0x7fffffff;
    p.flags = 0;
    for (int i = 0; i < a.gamma; ++i) {
        const int d = a.tokens[(long long)b * a.gamma + i];
        if (d < 0 || d >= a.V) p.flags |= SPECV_FLAG_TOKEN_OOR;
        else if (d == a.eos && i + 1 < ce) ce = i + 1;
    }
    p.cap = ce;
    p.top_k = k;
    p.top_p = tp;
    const bool greedy = a.greedy_all || !(T > 0.f);
    const bool topk_on = k > 0 && k < a.V;
    const bool topp_on = tp < 1.f;
    if (p.flags & SPECV_FLAG_TOKEN_OOR) {
        p.mode = MODE_SKIP;
    } else if (greedy) {
        p.mode = MODE_GREEDY;
    } else if (topk_on || topp_on) {
        if (a.cand_cap == 0 || (topk_on && k > a.max_top_k)) {
            p.mode = MODE_SKIP;               // the handle reserved no room for these candidates
            p.flags |= SPECV_FLAG_UNSUPPORTED;
        } else {
            p.mode = MODE_TRUNC;
        }
    } else {
        p.mode = MODE_SAMPLE;
    }
    p.scale = greedy ? 0.f : kLog2e / T;
    p.kmode = topk_on ? 1 : 0;
    p.keff = topk_on ? k : a.max_top_k;
    p.nt = min(ce, a.gamma + 1);
    p.nd = p.mode == MODE_GREEDY ? 0 : min(ce, a.gamma);
    return p;
}

__device__ inline long long part_index(const Args& a, int b, int r, int unit) {
    return ((long long)b * a.R + r) * a.U + unit;
}

// A Part moves as two 64-bit agent-scope accesses.
__device__ inline void publish_part(Part* p, const Part& v) {
    unsigned long long* q = reinterpret_cast<unsigned long long*>(p);
    const unsigned long long lo =
        (unsigned long long)__float_as_uint(v.m) | ((unsigned long long)__float_as_uint(v.s) << 32);
    const unsigned long long hi =
        (unsigned long long)(unsigned)v.arg | ((unsigned long long)v.bad << 32);
    __hip_atomic_store(q, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 1, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline Part published_part(const Part* p) {
    unsigned long long* q = reinterpret_cast<unsigned long long*>(const_cast<Part*>(p));
    const unsigned long long lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    Part v;
    v.m = __uint_as_float((unsigned)lo);
    v.s = __uint_as_float((unsigned)(lo >> 32));
    v.arg = (int)(unsigned)hi;
    v.bad = (unsigned)(hi >> 32);
    return v;
}

__device__ inline void write_diag_nan(const Args& a, int b, int from) {
    for (int i = from; i < a.gamma; ++i) {
        if (a.p_at) a.p_at[(long long)b * a.gamma + i] = __builtin_nanf("");
        if (a.q_at) a.q_at[(long long)b * a.gamma + i] = __builtin_nanf("");
    }
}

// Final outputs of one row: emit[0..nemit) then ``sampled`` (if >= 0), -1 padding.
__device__ inline void write_outputs(const Args& a, int b, const int* emit, int nemit, int nacc,
                                     unsigned flags, bool dead, int sampled, float wres) {
    const int g1 = a.gamma + 1;
    if (dead) {
        nemit = 0;
        nacc = 0;
        sampled = -1;
    }
    for (int j = 0; j < g1; ++j) {
        int t = -1;
        if (j < nemit) t = emit[j];
        else if (j == nemit && sampled >= 0) t = sampled;
        a.out_tok[(long long)b * g1 + j] = t;
    }
    a.out_emit[b] = nemit + (sampled >= 0 ? 1 : 0);
    a.out_acc[b] = nacc;
    if (a.out_flags) a.out_flags[b] = (int)flags;
    if (a.wres) a.wres[b] = wres;
}

// A batch row's decision while it is being taken (LDS of the deciding
// workgroup), and its publication as epoch-tagged words.
struct DecLocal {
    int kind;
    int pos;
    float u;
    int nemit;
    int nacc;
    unsigned flags;
    int emit[SPECV_MAX_GAMMA];
};

__device__ inline void dec_put(Dec* d, int word, unsigned v, unsigned epoch) {
    __hip_atomic_store(&d->w[word], ((unsigned long long)epoch << 32) | v, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Nothing to sample for the row (its outputs are written).
__device__ inline void publish_dec_none(const Args& a, int b) {
    dec_put(&a.ws.dec[b], DW_KIND, (unsigned)KIND_NONE, a.epoch);
}

// A correction / bonus draw for the sampling workgroups of the row.
__device__ inline void publish_dec_draw(const Args& a, int b, const DecLocal& sd, float mt,
                                        float invt, float mq, float invq, float scale) {
    Dec* d = &a.ws.dec[b];
    const unsigned e = a.epoch;
    dec_put(d, DW_KIND, (unsigned)sd.kind, e);
    dec_put(d, DW_POS, (unsigned)sd.pos, e);
    dec_put(d, DW_U, __float_as_uint(sd.u), e);
    dec_put(d, DW_MT, __float_as_uint(mt), e);
    dec_put(d, DW_INVT, __float_as_uint(invt), e);
    dec_put(d, DW_MQ, __float_as_uint(mq), e);
    dec_put(d, DW_INVQ, __float_as_uint(invq), e);
    dec_put(d, DW_SCALE, __float_as_uint(scale), e);
    dec_put(d, DW_NEMIT, (unsigned)sd.nemit, e);
    dec_put(d, DW_NACC, (unsigned)sd.nacc, e);
    dec_put(d, DW_FLAGS, sd.flags, e);
    for (int j = 0; j < a.gamma; ++j) dec_put(d, DW_EMIT + j, (unsigned)(j < sd.nemit ? sd.emit[j] : -1), e);
}

// ---------------------------------------------------------------- decision
// Run by the last streaming workgroup of batch row b, once every consulted
// row's unit statistics are published: combine them, take the accept tests
// in order and stop at the first rejection (pseudo-code 10-1), or follow the
// greedy rule.  Rows that need no sampled token get their outputs here; the
// others publish a decision record for the sampling phase; either way the
// record's kind word carries this call's epoch.
//
// With ``first`` set it runs after the position-0 rows only: if the round
// ends at position 0 the row is decided as above (and the stage flag says
// "stop"); otherwise only the stage flag is published ("go on") and the
// decision is left to the last unit of the later positions.
template <bool BF16>
__device__ void decide_row(const Args& a, int b, const Plan& pl, bool first) {
    __shared__ float sM[kMaxRows], sS[kMaxRows];
    __shared__ int sI[kMaxRows];
    __shared__ unsigned sBad[kMaxRows];
    __shared__ float sP[SPECV_MAX_GAMMA], sQ[SPECV_MAX_GAMMA];
    __shared__ int sQz[SPECV_MAX_GAMMA];
    __shared__ float sUacc[SPECV_MAX_GAMMA], sUres[SPECV_MAX_GAMMA + 1];
    __shared__ DecLocal sd;
    const int tid = threadIdx.x;
    const bool greedy = pl.mode == MODE_GREEDY;
    const float scale = pl.scale;
    const int nt = first ? 1 : pl.nt;                 // rows merged at this point
    const int nd = first ? min(pl.nd, 1) : pl.nd;
    const int nrows = nt + nd;
    // one memory round trip: every unit statistic, every z at d_i, and the
    // uniforms, issued together by different threads
    __shared__ Part sPart[kDecideParts];
    __shared__ float sZt[SPECV_MAX_GAMMA], sZq[SPECV_MAX_GAMMA];
    const int nparts = nrows * a.U;
    for (int k = tid; k < nparts; k += kBlock) {
        const int row = k / a.U;
        const int r = row < nt ? row : a.gamma + 1 + (row - nt);
        if (k < kDecideParts) sPart[k] = published_part(&a.ws.part[part_index(a, b, r, k - row * a.U)]);
    }
    if (!greedy && tid >= kBlock - kWave && tid - (kBlock - kWave) < nd) {
        const int i = tid - (kBlock - kWave);
        const int d = a.tokens[(long long)b * a.gamma + i];
        sZt[i] = load_elem<BF16>(row_ptr<BF16>(a.tgt, a.t_sb, a.t_sp, b, i), d);
        sZq[i] = load_elem<BF16>(row_ptr<BF16>(a.drf, a.d_sb, a.d_sp, b, i), d);
    }
    if (!greedy && tid >= kBlock - 2 * kWave && tid < kBlock - kWave) {
        const int i = tid - (kBlock - 2 * kWave);
        if (i < nd) {
            sUacc[i] = uniform24(a.seed, b, i, PURPOSE_ACCEPT, a.step);
            sUres[i] = uniform24(a.seed, b, i, PURPOSE_RESIDUAL, a.step);
        }
        if (i == kWave - 1) sUres[a.gamma] = uniform24(a.seed, b, a.gamma, PURPOSE_BONUS, a.step);
    }
    __syncthreads();
    // merge the units of each row, one thread per row
    for (int row = tid; row < nrows; row += kBlock) {
        const int r = row < nt ? row : a.gamma + 1 + (row - nt);
        float m = -kInf, s = 0.f;
        int arg = 0x7fffffff;
        unsigned bad = 0;
        for (int u = 0; u < a.U; ++u) {
            const int k = row * a.U + u;
            const Part p = k < kDecideParts ? sPart[k]
                                            : published_part(&a.ws.part[part_index(a, b, r, u)]);
            if (greedy) merge_arg(m, arg, p.m, p.arg);
            else merge_ms(m, s, p.m, p.s, scale);
            bad |= p.bad;
        }
        sM[r] = m;
        sS[r] = s;
        sI[r] = arg;
        sBad[r] = bad || m == -kInf || (!greedy && !(s > 0.f));
    }
    __syncthreads();
    if (!greedy && tid < nd) {
        // p_i(d_i) and q_i(d_i) from the raw logits at d_i
        const int i = tid;
        const int rq = a.gamma + 1 + i;
        sP[i] = fast_exp2((sZt[i] - sM[i]) * scale) / sS[i];
        sQ[i] = fast_exp2((sZq[i] - sM[rq]) * scale) / sS[rq];
        sQz[i] = sZq[i] == -kInf;
    }
    __syncthreads();
    if (tid != 0) return;

    sd.kind = KIND_NONE;
    sd.pos = -1;
    sd.u = 0.f;
    sd.nemit = 0;
    sd.nacc = 0;
    sd.flags = pl.flags;
    bool dead = false;
    bool go_on = false;                                // first stage: the round continues
    int sampled = -1;
    int tested = 0;
    const int* toks = a.tokens + (long long)b * a.gamma;
    if (greedy) {
        for (int i = 0; i <= a.gamma; ++i) {
            if (sd.nemit >= pl.cap) break;
            if (first && i >= 1) {
                go_on = true;
                break;
            }
            if (sBad[i]) {
                dead = true;
                break;
            }
            const int am = sI[i];
            if (i < a.gamma && toks[i] == am) {
                sd.emit[sd.nemit++] = am;
                sd.nacc++;
                continue;
            }
            sampled = am;        // first mismatch, or the bonus position
            break;
        }
    } else {
        int i = 0;
        for (; i < a.gamma; ++i) {
            if (sd.nemit >= pl.cap) break;
            if (first && i >= 1) {
                go_on = true;
                break;
            }
            if (sBad[i] || sBad[a.gamma + 1 + i]) {
                dead = true;
                break;
            }
            if (sQz[i]) sd.flags |= SPECV_FLAG_Q_ZERO;
            tested = i + 1;
            if (sUacc[i] * sQ[i] < sP[i]) {       // accept with probability min(1, p/q)
                sd.emit[sd.nemit++] = toks[i];
                sd.nacc++;
                continue;
            }
            sd.kind = KIND_RESIDUAL;
            sd.pos = i;
            sd.u = sUres[i];
            break;
        }
        if (!go_on && !dead && sd.kind == KIND_NONE && i == a.gamma && sd.nemit < pl.cap) {
            if (first && a.gamma >= 1) {
                go_on = true;                     // the bonus row is a later position
            } else if (sBad[a.gamma]) {
                dead = true;
            } else {
                sd.kind = KIND_BONUS;
                sd.pos = a.gamma;
                sd.u = sUres[a.gamma];
            }
        }
        if (!go_on) {
            for (int j = 0; j < tested; ++j) {
                if (a.p_at) a.p_at[(long long)b * a.gamma + j] = sP[j];
                if (a.q_at) a.q_at[(long long)b * a.gamma + j] = sQ[j];
            }
        }
    }
    if (go_on) {
        publish(&a.ws.stage1[(long long)b * kCounterStride], 2u * a.epoch + 1u);
        return;
    }
    write_diag_nan(a, b, tested);
    if (dead) {
        sd.flags |= SPECV_FLAG_NONFINITE_ROW;
        sd.kind = KIND_NONE;
    }
    if (sd.kind == KIND_NONE) {
        write_outputs(a, b, sd.emit, sd.nemit, sd.nacc, sd.flags, dead, sampled, 0.f);
        publish_dec_none(a, b);
    } else {
        const int pos = sd.pos;
        const bool res = sd.kind == KIND_RESIDUAL;
        publish_dec_draw(a, b, sd, sM[pos], 1.f / sS[pos], res ? sM[a.gamma + 1 + pos] : 0.f,
                         res ? 1.f / sS[a.gamma + 1 + pos] : 0.f, scale);
    }
    if (first) publish(&a.ws.stage1[(long long)b * kCounterStride], 2u * a.epoch);
}

// ---------------------------------------------------------------- truncation
// Top-k / top-p rows ("11.1 核心原理" 11.1.2: p and q are the distributions
// after truncation; q is the truncated proposal actually sampled).
//   per chunk:   each thread keeps its top-j finite values (j = ceil(2k / 256)
//                <= 8); the k-th largest of those 256 j values, L, has at
//                least k chunk entries >= L, so every finite entry >= L is a
//                superset of the chunk's top k (typically ~k entries);
//   per row:     (last unit of the row) the row's top-k threshold is >= every
//                chunk's L, so only candidates >= max L are gathered (at most
//                2048); they are sorted (value desc, index asc), the k-th
//                entry is the top-k threshold (ties kept), and the prefix is
//                scanned for top-p: the first level whose cumulative mass
//                reaches top_p ends the kept set (ties at a level all kept);
//   per batch row: (last row) accept tests from the kept sets, and the
//                correction / bonus sample from the (short) kept list of the
//                sampled row, tokens in ascending index order.

__device__ inline bool finite_logit(float x) { return x > -kInf && x <= 3.402823466e38f; }

__device__ inline void publish_cand(Cand* p, float v, int idx) {
    const unsigned long long w =
        (unsigned long long)__float_as_uint(v) | ((unsigned long long)(unsigned)idx << 32);
    __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), w, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline Cand published_cand(const Cand* p) {
    const unsigned long long w = __hip_atomic_load(
        reinterpret_cast<unsigned long long*>(const_cast<Cand*>(p)), __ATOMIC_RELAXED,
        __HIP_MEMORY_SCOPE_AGENT);
    Cand c;
    c.v = __uint_as_float((unsigned)w);
    c.idx = (int)(unsigned)(w >> 32);
    return c;
}

__device__ inline int pow2_at_least(int n) {
    int p = 1;
    while (p < n) p <<= 1;
    return p;
}

// (value desc, index asc)
__device__ inline bool by_value(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}
// index asc
__device__ inline bool by_index(float, int ia, float, int ib) { return ia < ib; }

// Block-wide bitonic sort of v / idx [0, n), n a power of two <= kKeptCap,
// so that entry x comes before entry y when prec(x, y).  Entries must be
// visible to the block (caller synchronised); result visible on return.
template <typename Prec>
__device__ void bitonic_sort(float* v, int* idx, int n, Prec prec) {
    for (int k = 2; k <= n; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < n; i += kBlock) {
                const int ixj = i ^ j;
                if (ixj > i) {
                    const float va = v[i], vb = v[ixj];
                    const int ia = idx[i], ib = idx[ixj];
                    const bool sw = (i & k) == 0 ? prec(vb, ib, va, ia) : prec(va, ia, vb, ib);
                    if (sw) {
                        v[i] = vb;
                        v[ixj] = va;
                        idx[i] = ib;
                        idx[ixj] = ia;
                    }
                }
            }
            __syncthreads();
        }
    }
}

// Block-wide exclusive scan of one int per thread; returns this thread's
// offset and writes the total to *total (both visible to all threads).
__device__ inline int block_excl_scan(int x, int* scratch /* kWaves + 1 */, int* total) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int incl = wave_scan_incl(x);
    if (lane == kWave - 1) scratch[wave] = incl;
    __syncthreads();
    int base = 0, tot = 0;
    for (int w = 0; w < kWaves; ++w) {
        if (w < wave) base += scratch[w];
        tot += scratch[w];
    }
    *total = tot;
    __syncthreads();
    return base + incl - x;
}

// In-place inclusive prefix sum of w[0, n), n <= kKeptCap: eight consecutive
// entries per thread in order, then across threads.
__device__ void block_inclusive_scan(float* w, int n, float* red) {
    constexpr int per = kKeptCap / kBlock;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int base = threadIdx.x * per;
    float loc[per];
    float run = 0.f;
#pragma unroll
    for (int j = 0; j < per; ++j) {
        run += base + j < n ? w[base + j] : 0.f;
        loc[j] = run;
    }
    const float incl = wave_scan_incl(run);
    if (lane == kWave - 1) red[wave] = incl;
    __syncthreads();
    float wbase = 0.f;
    for (int w2 = 0; w2 < wave; ++w2) wbase += red[w2];
    const float excl = wbase + incl - run;
#pragma unroll
    for (int j = 0; j < per; ++j)
        if (base + j < n) w[base + j] = excl + loc[j];
    __syncthreads();
}

__device__ inline long long cand_base(const Args& a, long long rowid, int c) {
    return (rowid * a.C + c) * a.cand_cap;
}

// Order-preserving key of a raw logit (larger value -> larger key).  bf16
// values are fp32 patterns with zero low halves, so their keys fit 16 bits.
template <bool BF16>
__device__ inline unsigned order_key(float x) {
    unsigned u = __float_as_uint(x);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return BF16 ? (u >> 16) : u;
}

// Candidate f of a row (flat index over its chunks, offsets in sc.off).
__device__ inline Cand row_candidate(const Args& a, long long rowid, const unsigned* off, int f) {
    int lo = 0, hi = a.C - 1;                  // chunk c with off[c] <= f < off[c + 1]
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int)off[mid] <= f) lo = mid;
        else hi = mid - 1;
    }
    return published_cand(a.ws.cand + cand_base(a, rowid, lo) + (f - (int)off[lo]));
}

// Radix select (8-bit digits from the top) of the K-th largest order key
// among the row's candidates with value >= L, read from global memory.
template <bool BF16>
__device__ unsigned select_kth_key(const Args& a, long long rowid, int total, float L, int K,
                                   TruncScratch& sc) {
    constexpr int KB = BF16 ? 16 : 32;
    const int tid = threadIdx.x;
    __shared__ unsigned sPrefix, sDigit;
    __shared__ int sRemaining, sAbove;
    if (tid == 0) {
        sPrefix = 0;
        sRemaining = K;
    }
    for (int pass = 0; pass < KB / 8; ++pass) {
        const int shift = KB - 8 * (pass + 1);
        sc.hist[tid] = 0;                      // kBlock == 256 bins
        __syncthreads();
        const unsigned prefix = sPrefix;
        const unsigned hi_mask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8)) & (BF16 ? 0xFFFFu : 0xFFFFFFFFu);
        for (int f0 = 0; f0 < total; f0 += 4 * kBlock) {
            Cand cv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int f = f0 + q * kBlock + tid;
                cv[q] = f < total ? row_candidate(a, rowid, sc.off, f) : Cand{-kInf, 0};
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (cv[q].v >= L && finite_logit(cv[q].v)) {
                    const unsigned key = order_key<BF16>(cv[q].v);
                    if ((key & hi_mask) == prefix) atomicAdd(&sc.hist[(key >> shift) & 255u], 1u);
                }
            }
        }
        __syncthreads();
        // bin t holds hist[t]; entries in bins >= t: total - (entries in bins < t)
        const int h = (int)sc.hist[tid];
        int binned;
        const int below = block_excl_scan(h, sc.misc, &binned);
        const int ge = binned - below;
        const int need = sRemaining;
        if (ge >= need && ge - h < need) {
            sDigit = (unsigned)tid;
            sAbove = ge - h;
        }
        __syncthreads();
        if (tid == 0) {
            sPrefix |= sDigit << shift;
            sRemaining -= sAbove;
        }
        __syncthreads();
    }
    return sPrefix;
}

// Candidates of one chunk (whole workgroup): every finite entry >= L.
template <bool BF16>
__device__ void chunk_candidates(const Args& a, long long rowid, int c, int keff,
                                 const float (&x)[kPerThread], TruncScratch& sc) {
    const int tid = threadIdx.x;
    // twice as many per-thread tops as needed keeps L close to the k-th value
    const int jj = min(8, (2 * keff + kBlock - 1) / kBlock);
    float tp[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) tp[j] = -kInf;                // this thread's top 8, desc
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        float v = x[k];
        if (!(finite_logit(v) && v > tp[7])) continue;
#pragma unroll
        for (int j = 0; j < 8; ++j) {                       // insertion, larger values first
            if (v > tp[j]) {
                const float s = tp[j];
                tp[j] = v;
                v = s;
            }
        }
    }
    const int n = kBlock * jj;
    const int n2 = pow2_at_least(n);
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (j < jj) {
            sc.v[tid * jj + j] = tp[j];
            sc.idx[tid * jj + j] = 0;
        }
    for (int i = n + tid; i < n2; i += kBlock) {
        sc.v[i] = -kInf;
        sc.idx[i] = 0;
    }
    __syncthreads();
    bitonic_sort(sc.v, sc.idx, n2, by_value);
    const float L = sc.v[keff - 1];        // keff <= 256 * jj / 2 <= n2
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) cnt += finite_logit(x[k]) && x[k] >= L;
    int total;
    const int off = block_excl_scan(cnt, sc.misc, &total);
    if (total <= a.cand_cap) {
        Cand* dst = a.ws.cand + cand_base(a, rowid, c);
        int o = off;
        const int v0 = c * kChunk;
#pragma unroll
        for (int k = 0; k < kPerThread; ++k)
            if (finite_logit(x[k]) && x[k] >= L) publish_cand(dst + o++, x[k], v0 + chunk_index<BF16>(k));
    }
    if (tid == 0)
        publish_cand(a.ws.cand_meta + rowid * a.C + c, L, total <= a.cand_cap ? total : -1);
}

// Row-level truncation (whole workgroup), run by the last unit of the row.
template <bool BF16>
__device__ void row_merge(const Args& a, int b, int r, const Plan& pl, TruncScratch& sc) {
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const long long rowid = (long long)b * a.R + r;
    __shared__ float sL, sM, sS, sZ1;
    __shared__ unsigned sBad, sFlags;
    __shared__ int sTotal, sN, sJ, sLevelStart;
    unsigned* off = sc.off;                // chunk offsets [0, C]
    if (tid == 0) {
        sBad = 0;
        sFlags = 0;
        sN = 0;
        sJ = 0x7fffffff;
        sLevelStart = 0x7fffffff;
    }
    // chunk bounds and counts (lane c holds chunk c; C <= 64), and the row
    // statistics (for top-p alone)
    if (wave == 0) {
        float L = -kInf;
        int cnt = 0;
        bool ovf = false;
        if (lane < a.C) {
            const Cand m = published_cand(a.ws.cand_meta + rowid * a.C + lane);
            L = m.v;
            ovf = m.idx < 0;
            cnt = ovf ? 0 : m.idx;
        }
        L = wave_max(L);
        const int incl = wave_scan_incl(cnt);
        if (lane < a.C) off[lane] = (unsigned)(incl - cnt);
        if (lane == a.C - 1) {
            off[a.C] = (unsigned)incl;
            sTotal = incl;
        }
        const unsigned long long any_ovf = __ballot(ovf);
        if (lane == 0) {
            sL = L;
            if (any_ovf) sFlags |= SPECV_FLAG_CAND_OVERFLOW;
        }
    } else if (wave == 1) {
        float m = -kInf, s = 0.f;
        unsigned bad = 0;
        for (int u = lane; u < a.U; u += kWave) {
            const Part p = published_part(&a.ws.part[part_index(a, b, r, u)]);
            merge_ms(m, s, p.m, p.s, pl.scale);
            bad |= p.bad;
        }
        wave_merge_ms(m, s, pl.scale);
        bad = wave_or(bad);
        if (lane == 0) {
            sM = m;
            sS = s;
            if (bad || m == -kInf) sBad = 1;
        }
    }
    __syncthreads();
    // gather the candidates >= max L into LDS
    const float L = sL;
    const int total = sTotal;
    auto gather = [&](unsigned min_key) {
        for (int f0 = 0; f0 < total; f0 += 4 * kBlock) {
            Cand cv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int f = f0 + q * kBlock + tid;
                cv[q] = f < total ? row_candidate(a, rowid, off, f) : Cand{-kInf, 0};
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (cv[q].v >= L && finite_logit(cv[q].v) && order_key<BF16>(cv[q].v) >= min_key) {
                    const int pos = atomicAdd(&sN, 1);
                    if (pos < kKeptCap) {
                        sc.v[pos] = cv[q].v;
                        sc.idx[pos] = cv[q].idx;
                    }
                }
            }
        }
        __syncthreads();
    };
    gather(0u);
    if (sN > kKeptCap) {
        // too many candidates above the chunk bounds: select the exact top-k
        // key over them in global memory, then keep only entries >= it
        const int K = min(pl.keff, sN);
        const unsigned kkey = select_kth_key<BF16>(a, rowid, total, L, K, sc);
        if (tid == 0) sN = 0;
        __syncthreads();
        gather(kkey);
    }
    const int n1 = sN;
    if (n1 > kKeptCap && tid == 0) sFlags |= SPECV_FLAG_CAND_OVERFLOW;
    __syncthreads();
    TruncRow* tr = &a.ws.trow[rowid];
    if ((sFlags & SPECV_FLAG_CAND_OVERFLOW) || sBad || n1 == 0) {
        if (tid == 0) {
            publish(&tr->bad, (sBad || n1 == 0) ? 1u : 0u);
            publish(&tr->flags, sFlags);
            publish(&tr->n_kept, 0);
        }
        return;
    }
    // sort the gathered entries: value desc, index asc
    const int n2 = pow2_at_least(n1);
    for (int i = n1 + tid; i < n2; i += kBlock) {
        sc.v[i] = -kInf;
        sc.idx[i] = 0x7fffffff;
    }
    __syncthreads();
    bitonic_sort(sc.v, sc.idx, n2, by_value);
    // top-k: the K-th largest (with multiplicity) ends the kept prefix; all
    // entries equal to it are kept
    const int K = min(pl.keff, n1);
    const float tk = sc.v[K - 1];
    // count of entries >= tk (a prefix of the sorted list)
    int cnt = 0;
    for (int i = tid; i < n1; i += kBlock) cnt += sc.v[i] >= tk;
    int nk1;
    (void)block_excl_scan(cnt, sc.misc, &nk1);
    const float zmax = sc.v[0];
    const float scale = pl.scale;
    for (int i = tid; i < nk1; i += kBlock) sc.w[i] = fast_exp2(__fmul_rn(sc.v[i] - zmax, scale));
    __syncthreads();
    block_inclusive_scan(sc.w, nk1, sc.red);
    if (tid == 0) {
        // normaliser of the top-k-renormalised softmax: the kept top-k set, or
        // the whole row when top-k is off
        sZ1 = pl.kmode ? sc.w[nk1 - 1] : sS * fast_exp2(__fmul_rn(sM - zmax, scale));
    }
    __syncthreads();
    const float Z1 = sZ1;
    int jstar = nk1 - 1;
    if (pl.top_p < 1.f) {
        // first level end whose cumulative mass reaches top_p
        for (int i = tid; i < nk1; i += kBlock) {
            const bool level_end = i == nk1 - 1 || sc.v[i + 1] != sc.v[i];
            if (level_end && sc.w[i] / Z1 >= pl.top_p) atomicMin(&sJ, i);
        }
        __syncthreads();
        if (sJ == 0x7fffffff) {
            if (!pl.kmode) {
                // top-p alone: the candidates hold less than top_p of the mass
                if (tid == 0) {
                    sFlags |= SPECV_FLAG_CAND_OVERFLOW;
                    publish(&tr->bad, 0u);
                    publish(&tr->flags, sFlags);
                    publish(&tr->n_kept, 0);
                }
                return;
            }
            jstar = nk1 - 1;                // rounding: keep the whole top-k set
        } else {
            jstar = sJ;
        }
        const float tv = sc.v[jstar];
        for (int i = tid; i <= jstar; i += kBlock)
            if (sc.v[i] == tv) atomicMin(&sLevelStart, i);
        __syncthreads();
        if (tid == 0) {
            const float cum = sc.w[jstar] / Z1;
            const int ls = sLevelStart;
            const float prev = ls > 0 ? sc.w[ls - 1] / Z1 : 0.f;
            if (fabsf(cum - pl.top_p) < 1e-5f || (ls > 0 && fabsf(prev - pl.top_p) < 1e-5f))
                sFlags |= SPECV_FLAG_TOPP_NEAR;
        }
    }
    const int nkept = jstar + 1;
    Cand* kept = a.ws.kept + rowid * a.kept_cap;
    for (int i = tid; i < nkept; i += kBlock) publish_cand(kept + i, sc.v[i], sc.idx[i]);
    __syncthreads();
    if (tid == 0) {
        publish(&tr->zmax, zmax);
        publish(&tr->tstar, sc.v[jstar]);
        publish(&tr->S, sc.w[jstar]);
        publish(&tr->n_kept, nkept);
        publish(&tr->flags, sFlags);
        publish(&tr->bad, 0u);
    }
}

// Decision and sampling of a truncated batch row (whole workgroup), run by
// the last of its consulted rows to finish.
template <bool BF16>
__device__ void decide_trunc(const Args& a, int b, const Plan& pl, TruncScratch& sc) {
    const int tid = threadIdx.x;
    __shared__ float tZ[kMaxRows], tT[kMaxRows], tS[kMaxRows];
    __shared__ int tN[kMaxRows];
    __shared__ unsigned tF[kMaxRows], tBad[kMaxRows];
    __shared__ float sP[SPECV_MAX_GAMMA], sQ[SPECV_MAX_GAMMA];
    __shared__ int sQz[SPECV_MAX_GAMMA];
    __shared__ float sUacc[SPECV_MAX_GAMMA], sUres[SPECV_MAX_GAMMA + 1];
    __shared__ DecLocal sd;
    __shared__ int sDead, sTok, sLastPos;
    __shared__ float sWsum;
    const float scale = pl.scale;
    const int nrows = pl.nt + pl.nd;
    for (int k = tid; k < nrows; k += kBlock) {
        const int r = k < pl.nt ? k : a.gamma + 1 + (k - pl.nt);
        const TruncRow* tr = &a.ws.trow[(long long)b * a.R + r];
        tZ[r] = published(&tr->zmax);
        tT[r] = published(&tr->tstar);
        tS[r] = published(&tr->S);
        tN[r] = published(&tr->n_kept);
        tF[r] = published(&tr->flags);
        tBad[r] = published(&tr->bad);
    }
    __syncthreads();
    // membership in the kept set is decided on the raw value: z >= tstar
    auto prob = [&](int r, float z) -> float {
        if (!(finite_logit(z) && z >= tT[r])) return 0.f;
        return fast_exp2(__fmul_rn(z - tZ[r], scale)) / tS[r];
    };
    auto row_dead = [&](int r) { return tBad[r] != 0 || (tF[r] & SPECV_FLAG_CAND_OVERFLOW) || tN[r] == 0; };
    if (tid < pl.nd) {
        const int i = tid;
        const int d = a.tokens[(long long)b * a.gamma + i];
        const float zt = load_elem<BF16>(row_ptr<BF16>(a.tgt, a.t_sb, a.t_sp, b, i), d);
        const float zq = load_elem<BF16>(row_ptr<BF16>(a.drf, a.d_sb, a.d_sp, b, i), d);
        const int rq = a.gamma + 1 + i;
        sP[i] = row_dead(i) ? 0.f : prob(i, zt);
        sQ[i] = row_dead(rq) ? 0.f : prob(rq, zq);
        sQz[i] = !(finite_logit(zq) && zq >= tT[rq]);
        sUacc[i] = uniform24(a.seed, b, i, PURPOSE_ACCEPT, a.step);
        sUres[i] = uniform24(a.seed, b, i, PURPOSE_RESIDUAL, a.step);
    }
    if (tid == kBlock - 1) sUres[a.gamma] = uniform24(a.seed, b, a.gamma, PURPOSE_BONUS, a.step);
    __syncthreads();
    if (tid == 0) {
        sd.kind = KIND_NONE;
        sd.pos = -1;
        sd.u = 0.f;
        sd.nemit = 0;
        sd.nacc = 0;
        sd.flags = pl.flags;
        int dead = 0, tested = 0;
        const int* toks = a.tokens + (long long)b * a.gamma;
        auto consult = [&](int r) {
            sd.flags |= tF[r] & (SPECV_FLAG_TOPP_NEAR | SPECV_FLAG_CAND_OVERFLOW);
            if (tBad[r]) sd.flags |= SPECV_FLAG_NONFINITE_ROW;
            return !row_dead(r);
        };
        int i = 0;
        for (; i < a.gamma; ++i) {
            if (sd.nemit >= pl.cap) break;
            const bool okt = consult(i), okq = consult(a.gamma + 1 + i);
            if (!okt || !okq) {
                dead = 1;
                break;
            }
            if (sQz[i]) sd.flags |= SPECV_FLAG_Q_ZERO;
            tested = i + 1;
            if (sUacc[i] * sQ[i] < sP[i]) {       // accept with probability min(1, p/q)
                sd.emit[sd.nemit++] = toks[i];
                sd.nacc++;
                continue;
            }
            sd.kind = KIND_RESIDUAL;
            sd.pos = i;
            sd.u = sUres[i];
            break;
        }
        if (!dead && sd.kind == KIND_NONE && i == a.gamma && sd.nemit < pl.cap) {
            if (!consult(a.gamma)) {
                dead = 1;
            } else {
                sd.kind = KIND_BONUS;
                sd.pos = a.gamma;
                sd.u = sUres[a.gamma];
            }
        }
        for (int j = 0; j < tested; ++j) {
            if (a.p_at) a.p_at[(long long)b * a.gamma + j] = sP[j];
            if (a.q_at) a.q_at[(long long)b * a.gamma + j] = sQ[j];
        }
        write_diag_nan(a, b, tested);
        if (dead) sd.kind = KIND_NONE;
        sDead = dead;
        sTok = 0x7fffffff;
        sLastPos = -1;
    }
    __syncthreads();
    int sampled = -1;
    float wres = 0.f;
    if (sd.kind != KIND_NONE) {
        const int pos = sd.pos;
        const bool res = sd.kind == KIND_RESIDUAL;
        const int n = tN[pos];
        const Cand* kept = a.ws.kept + ((long long)b * a.R + pos) * a.kept_cap;
        const void* qrow = res ? row_ptr<BF16>(a.drf, a.d_sb, a.d_sp, b, pos) : nullptr;
        const int rq = a.gamma + 1 + pos;
        // weights over the kept set of p_pos (zero weight elsewhere):
        // sc.v = weight, sc.idx = token, sc.w = p (fallback weight)
        float part = 0.f, partp = 0.f;
        for (int i = tid; i < n; i += kBlock) {
            const Cand cv = published_cand(kept + i);
            const float p = __fmul_rn(fast_exp2(__fmul_rn(cv.v - tZ[pos], scale)), 1.f / tS[pos]);
            float w = p;
            if (res) {
                const float zq = load_elem<BF16>(qrow, cv.idx);
                const float q = (finite_logit(zq) && zq >= tT[rq])
                                    ? __fmul_rn(fast_exp2(__fmul_rn(zq - tZ[rq], scale)), 1.f / tS[rq])
                                    : 0.f;
                w = fmaxf(__fsub_rn(p, q), 0.f);
            }
            sc.v[i] = w;
            sc.w[i] = p;
            sc.idx[i] = cv.idx;
            part += w;
            partp += p;
        }
        part = wave_sum(part);
        if (tid % kWave == 0) sc.red[tid / kWave] = part;
        __syncthreads();
        if (tid == 0) {
            float W = 0.f;
            for (int w2 = 0; w2 < kWaves; ++w2) W += sc.red[w2];
            sWsum = W;
        }
        __syncthreads();
        wres = res ? sWsum : 0.f;
        if (res && (!(sWsum > 0.f) || !__builtin_isfinite(sWsum))) {
            // the correction mass vanished: sample from p at that position
            for (int i = tid; i < n; i += kBlock) sc.v[i] = sc.w[i];
            if (tid == 0) sd.flags |= SPECV_FLAG_RESIDUAL_FALLBACK;
        }
        (void)partp;
        // tokens in ascending index order, then the first running sum > u * W
        const int n2 = pow2_at_least(n);
        for (int i = n + tid; i < n2; i += kBlock) {
            sc.v[i] = 0.f;
            sc.idx[i] = 0x7fffffff;
        }
        __syncthreads();
        bitonic_sort(sc.v, sc.idx, n2, by_index);
        for (int i = tid; i < n; i += kBlock) sc.w[i] = sc.v[i];
        __syncthreads();
        block_inclusive_scan(sc.w, n, sc.red);
        const float target = sd.u * sc.w[n - 1];
        for (int i = tid; i < n; i += kBlock) {
            if (sc.v[i] > 0.f) {
                if (sc.w[i] > target) atomicMin(&sTok, i);
                atomicMax(&sLastPos, i);
            }
        }
        __syncthreads();
        const int j = sTok != 0x7fffffff ? sTok : sLastPos;     // clamp: last positive weight
        sampled = j >= 0 ? sc.idx[j] : -1;
    }
    if (tid == 0) {
        bool dead = sDead;
        unsigned flags = sd.flags;
        if (!dead && sd.kind != KIND_NONE && sampled < 0) {
            dead = true;
            flags |= SPECV_FLAG_NONFINITE_ROW;
        }
        write_outputs(a, b, sd.emit, sd.nemit, sd.nacc, flags, dead, sampled, wres);
        publish_dec_none(a, b);
    }
}

// ---------------------------------------------------------------- streaming
// The 16-byte loads of this thread's groups of chunk entries [v0, v0 + len),
// in load_chunk's layout, split in two halves so that several chunks can be
// in flight at once: ``issue_groups`` only issues the loads (groups past the
// chunk's last whole group load group 0 instead), ``finish_groups`` unpacks
// and masks them.  Needs len >= one group.
template <bool BF16>
__device__ inline void issue_groups(const void* row, int v0, int len,
                                    uint4 (&q)[kPerThread / (BF16 ? 8 : 4)]) {
    constexpr int G = BF16 ? 8 : 4;
    constexpr int NG = kPerThread / G;
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const char*>(row) +
                                                    (size_t)v0 * (BF16 ? 2 : 4));
    const int full = len / G;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
        const int g = j * kBlock + (int)threadIdx.x;
        q[j] = p[g < full ? g : 0];
    }
}

template <bool BF16>
__device__ inline void finish_groups(const void* row, int v0, int len,
                                     const uint4 (&q)[kPerThread / (BF16 ? 8 : 4)],
                                     float (&x)[kPerThread]) {
    constexpr int G = BF16 ? 8 : 4;
    constexpr int NG = kPerThread / G;
    const int tid = threadIdx.x;
    const int full = len / G;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
        unpack16<BF16>(q[j], &x[j * G]);
        if (j * kBlock + tid >= full) {
#pragma unroll
            for (int e = 0; e < G; ++e) x[j * G + e] = -kInf;
        }
    }
    const int rem = len - full * G;                 // entries of a last partial group
    if (rem && tid == full % kBlock) {
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            if (j == full / kBlock) {
#pragma unroll
                for (int e = 0; e < G; ++e)
                    if (e < rem) x[j * G + e] = load_elem<BF16>(row, (long long)v0 + full * G + e);
            }
        }
    }
}

// One streaming unit t = (b, r, unit): up to kUnitChunks chunks of one logits
// row, the loads of all of them (bfloat16) or of the next two (float32) in
// flight before the first is reduced, with per-thread running statistics:
//   sampling rows: running max m and sum s of exp2((z - m) * scale), the sum
//                  rescaled when the max grows (one extra exp2 per chunk);
//   greedy rows:   running max and its lowest index.
// The unit's statistics are published; the last unit of a batch row to
// arrive runs the decision.
//
// Units come in two stages.  Stage 1 holds the position-0 rows (target row 0
// and draft row 0) of every batch row; stage 2 the later positions.  For
// sampling and greedy rows the last stage-1 unit tests position 0; stage-2
// units wait for that result and skip their rows when the round has already
// ended (the rows past the first rejection are never needed), otherwise the
// last stage-2 unit decides the row.  Truncated rows do not wait.
template <bool BF16, bool VEC, bool TRUNC>
__device__ void stream_unit(const Args& a, int t, TruncScratch* sc) {
    constexpr int NG = kPerThread / (BF16 ? 8 : 4);
    const int n1 = a.gamma >= 1 ? 2 : 1;            // position-0 rows per batch row
    const int n2 = a.R - n1;
    const int units1 = a.B * n1 * a.U;
    const bool stage1 = t < units1;
    int b, r, unit;
    if (stage1) {
        unit = t % a.U;
        const int row = t / a.U;
        b = row / n1;
        r = (row - b * n1) == 0 ? 0 : a.gamma + 1;
    } else {
        const int t2 = t - units1;
        unit = t2 % a.U;
        const int row = t2 / a.U;
        b = row / n2;
        const int k = row - b * n2;                  // target rows 1..gamma, then draft rows 1..
        r = k < a.gamma ? 1 + k : a.gamma + 2 + (k - a.gamma);
    }
    const int tid = threadIdx.x;
    const Plan pl = make_plan(a, b);
    if (pl.mode == MODE_SKIP) {
        if (r == 0 && unit == 0 && tid == 0) {
            write_outputs(a, b, nullptr, 0, 0, pl.flags, true, -1, 0.f);
            write_diag_nan(a, b, 0);
            publish_dec_none(a, b);
        }
        return;
    }
    const bool is_target = r <= a.gamma;
    const int pos = is_target ? r : r - a.gamma - 1;
    if (pos >= (is_target ? pl.nt : pl.nd)) return;   // a row this round cannot consult
    const bool staged = pl.mode == MODE_SAMPLE || pl.mode == MODE_GREEDY;
    if (staged && !stage1) {
        __shared__ unsigned sGo;
        if (tid == 0) {
            const unsigned* flag = &a.ws.stage1[(long long)b * kCounterStride];
            unsigned v = 0;
            for (int spin = 0; spin < (1 << 20); ++spin) {
                v = published(flag);
                if ((v >> 1) == a.epoch) break;
                __builtin_amdgcn_s_sleep(2);
            }
            sGo = (v >> 1) == a.epoch ? (v & 1u) : 0u;
            if ((v >> 1) != a.epoch && a.out_flags) atomicOr(&a.out_flags[b], (int)SPECV_FLAG_INTERNAL);
        }
        __syncthreads();
        if (!sGo) return;                              // the round ended at position 0
    }

    const void* rp = is_target ? row_ptr<BF16>(a.tgt, a.t_sb, a.t_sp, b, pos)
                               : row_ptr<BF16>(a.drf, a.d_sb, a.d_sp, b, pos);
    const int c0 = unit * kUnitChunks;
    const bool greedy = pl.mode == MODE_GREEDY;
    const bool trunc = TRUNC && pl.mode == MODE_TRUNC;
    const long long rowid = (long long)b * a.R + r;
    const float scale = pl.scale;
    float m = -kInf, s = 0.f;                          // sampling rows
    float best = -kInf;                                // greedy rows
    int bi = 0x7fffffff;
    unsigned bad = 0;

    constexpr int G = BF16 ? 8 : 4;
    constexpr int DEPTH = BF16 && !TRUNC ? kUnitChunks : 2;   // chunks in flight (registers)
    auto chunk_len = [&](int c) { return c < a.C ? min(kChunk, a.V - c * kChunk) : 0; };
    uint4 q[DEPTH][NG];
#pragma unroll
    for (int u = 0; u < DEPTH; ++u)
        if (VEC && chunk_len(c0 + u) >= G) issue_groups<BF16>(rp, (c0 + u) * kChunk, chunk_len(c0 + u), q[u]);
#pragma unroll
    for (int u = 0; u < kUnitChunks; ++u) {
        const int c = c0 + u;
        if (c >= a.C) continue;                       // (keeps the unrolled trip count)
        const int len = chunk_len(c);
        float x[kPerThread];
        if (VEC && len >= G) {
            finish_groups<BF16>(rp, c * kChunk, len, q[u % DEPTH], x);
            if (u + DEPTH < kUnitChunks && chunk_len(c + DEPTH) >= G)
                issue_groups<BF16>(rp, (c + DEPTH) * kChunk, chunk_len(c + DEPTH), q[u % DEPTH]);
        } else {
            load_chunk<BF16, VEC>(rp, c * kChunk, len, x);
        }
        if (greedy) {
            const int v0 = c * kChunk;
#pragma unroll
            for (int k = 0; k < kPerThread; ++k) {
                bad |= !(x[k] <= 3.402823466e38f);        // NaN or +inf
                if (x[k] > best) {                        // strict: keeps the lowest index
                    best = x[k];
                    bi = v0 + chunk_index<BF16>(k);
                }
            }
        } else {
            float cm = -kInf;
#pragma unroll
            for (int k = 0; k < kPerThread; ++k) cm = fmaxf(cm, x[k]);
            const float nm = fmaxf(m, cm);
            const float nms = nm == -kInf ? 0.f : -nm * scale;
            float cs = s * fast_exp2(fmaf(m, scale, nms));
#pragma unroll
            for (int k = 0; k < kPerThread; ++k) cs += fast_exp2(fmaf(x[k], scale, nms));
            s = cs;
            m = nm;
            if constexpr (TRUNC)
                if (trunc) chunk_candidates<BF16>(a, rowid, c, pl.keff, x, *sc);
        }
    }

    __shared__ float sm[kWaves], ss[kWaves];
    __shared__ int si[kWaves];
    __shared__ unsigned sb[kWaves];
    __shared__ int sLast;
    const int lane = tid % kWave, wave = tid / kWave;
    Part out;
    if (greedy) {
        wave_merge_arg(best, bi);
        bad = wave_or(bad);
        if (lane == 0) {
            sm[wave] = best;
            si[wave] = bi;
            sb[wave] = bad;
        }
        __syncthreads();
        if (tid == 0) {
            for (int w = 1; w < kWaves; ++w) {
                merge_arg(best, bi, sm[w], si[w]);
                bad |= sb[w];
            }
            out.m = best;
            out.s = 0.f;
            out.arg = bi;
            out.bad = bad;
        }
    } else {
        wave_merge_ms(m, s, scale);
        if (lane == 0) {
            sm[wave] = m;
            ss[wave] = s;
        }
        __syncthreads();
        if (tid == 0) {
            for (int w = 1; w < kWaves; ++w) merge_ms(m, s, sm[w], ss[w], scale);
            out.m = m;
            out.s = s;
            out.arg = -1;
            out.bad = __builtin_isnan(s) ? 1u : 0u;      // NaN or +inf in the unit
        }
    }
    if constexpr (TRUNC) if (trunc) {
        // the last unit of the logits row truncates it; the last truncated
        // row of the batch row decides and samples
        if (tid == 0) {
            publish_part(&a.ws.part[part_index(a, b, r, unit)], out);
            sLast = arrive(&a.ws.counter_row[rowid * kCounterStride]) == (unsigned)(a.U - 1);
        }
        __syncthreads();
        if (!sLast) return;
        if (tid == 0) publish(&a.ws.counter_row[rowid * kCounterStride], 0u);
        row_merge<BF16>(a, b, r, pl, *sc);
        __syncthreads();
        if (tid == 0) {
            const unsigned expected = (unsigned)(pl.nt + pl.nd);
            sLast = arrive(&a.ws.counter[(long long)b * kCounterStride]) == expected - 1;
        }
        __syncthreads();
        if (!sLast) return;
        if (tid == 0) publish(&a.ws.counter[(long long)b * kCounterStride], 0u);
        decide_trunc<BF16>(a, b, pl, *sc);
        return;
    }
    unsigned* counter = stage1 ? &a.ws.counter1[(long long)b * kCounterStride]
                               : &a.ws.counter[(long long)b * kCounterStride];
    if (tid == 0) {
        publish_part(&a.ws.part[part_index(a, b, r, unit)], out);
        const int rows = stage1 ? 1 + min(pl.nd, 1) : (pl.nt - 1) + max(pl.nd - 1, 0);
        sLast = arrive(counter) == (unsigned)(rows * a.U) - 1;
    }
    __syncthreads();
    if (!sLast) return;
    if (tid == 0) publish(counter, 0u);               // ready for the next call
    decide_row<BF16>(a, b, pl, stage1);
}

// ---------------------------------------------------------------- sampling
// Correction / bonus weight of entry z (target) and zq (draft) of the row
// pair being sampled.
struct Weights {
    int residual;        // 1: max(p - q, 0); 0: p
    float mt, st, invt;  // target row max, scale, 1 / sum
    float mq, invq;      // draft row max, 1 / sum
    // Products are rounded separately (no fused multiply-add) so that equal
    // p and q rows give exactly zero correction weight.
    __device__ inline float w(float z, float zq) const {
        const float p = __fmul_rn(fast_exp2(__fmul_rn(z - mt, st)), invt);
        if (!residual) return p;
        const float q = __fmul_rn(fast_exp2(__fmul_rn(zq - mq, st)), invq);
        return fmaxf(__fsub_rn(p, q), 0.f);
    }
};

// Sampling item (b, c), once b's decision is published: sum chunk c's
// sampling weight (correction max(p - q, 0) from the two rows, or bonus p)
// and its p mass.  The last item of the row to arrive picks the chunk
// holding u * W, rescans it with a block prefix sum (tokens in ascending
// order, first running sum > u * W) and writes the outputs.
// The workgroup that decides the row was dispatched before every sampling
// workgroup and never waits for one, so the (bounded) wait for the decision
// ends; the bound only guards against a dispatch order other than the
// hardware's in-order one, and its expiry flags the row INTERNAL.
template <bool BF16, bool VEC>
__device__ void sample_item(const Args& a, int b, int c) {
    const int tid = threadIdx.x;
    const int lane = tid % kWave, wave = tid / kWave;
    // the row's decision record: one wave polls every word it needs at once
    // until all carry this call's epoch (or the kind word alone says there
    // is nothing to sample)
    __shared__ unsigned sDw[kDecWords];
    __shared__ int sOk;
    if (wave == 0) {
        const int nw = DW_EMIT + a.gamma;
        unsigned long long* src = a.ws.dec[b].w;
        const unsigned long long tag = (unsigned long long)a.epoch << 32;
        unsigned long long v = tag;
        bool done = false;
        for (int spin = 0; spin < (1 << 20); ++spin) {
            v = lane < nw ? __hip_atomic_load(src + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                          : tag;
            const unsigned long long mine = __ballot((unsigned)(v >> 32) == a.epoch);
            const unsigned kind0 = __builtin_amdgcn_readfirstlane((unsigned)v);
            if ((mine & 1ull) && (kind0 == (unsigned)KIND_NONE || mine == ~0ull)) {
                done = true;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        if (lane < nw) sDw[lane] = (unsigned)v;
        if (lane == 0) sOk = done;
        if (!done && lane == 0 && c == 0 && a.out_flags) atomicOr(&a.out_flags[b], (int)SPECV_FLAG_INTERNAL);
    }
    __syncthreads();
    if (!sOk) return;
    const int kind = (int)sDw[DW_KIND];
    if (kind == KIND_NONE) return;
    const int pos = (int)sDw[DW_POS];
    Weights wt;
    wt.residual = kind == KIND_RESIDUAL;
    wt.mt = __uint_as_float(sDw[DW_MT]);
    wt.st = __uint_as_float(sDw[DW_SCALE]);
    wt.invt = __uint_as_float(sDw[DW_INVT]);
    wt.mq = __uint_as_float(sDw[DW_MQ]);
    wt.invq = __uint_as_float(sDw[DW_INVQ]);
    const float u = __uint_as_float(sDw[DW_U]);
    const void* trow = row_ptr<BF16>(a.tgt, a.t_sb, a.t_sp, b, pos);
    const void* qrow = wt.residual ? row_ptr<BF16>(a.drf, a.d_sb, a.d_sp, b, pos) : nullptr;

    __shared__ float red[2][kWaves];
    __shared__ int sLast;
    {
        const int v0 = c * kChunk;
        const int len = min(kChunk, a.V - v0);
        float x[kPerThread], y[kPerThread];
        load_chunk<BF16, VEC>(trow, v0, len, x);
        if (wt.residual) load_chunk<BF16, VEC>(qrow, v0, len, y);
        float sw = 0.f, sp = 0.f;
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) {
            const float p = __fmul_rn(fast_exp2(__fmul_rn(x[k] - wt.mt, wt.st)), wt.invt);
            sp += p;
            sw += wt.residual ? wt.w(x[k], y[k]) : p;
        }
        sw = wave_sum(sw);
        sp = wave_sum(sp);
        if (lane == 0) {
            red[0][wave] = sw;
            red[1][wave] = sp;
        }
        __syncthreads();
        if (tid == 0) {
            float wc = red[0][0], pc = red[1][0];
            for (int w = 1; w < kWaves; ++w) {
                wc += red[0][w];
                pc += red[1][w];
            }
            float* slot = a.ws.wsum + ((long long)b * a.C + c) * 2;
            publish(slot, wc);
            publish(slot + 1, pc);
            sLast = arrive(&a.ws.counter2[(long long)b * kCounterStride]) == (unsigned)(a.C - 1);
        }
    }
    __syncthreads();
    if (!sLast) return;

    // last item of the row
    __shared__ float sW[kMaxChunks], sPm[kMaxChunks];
    __shared__ float sWres, sBase, sTarget;
    __shared__ int sChunk, sRes, sTok;
    __shared__ unsigned sFlags;
    for (int cc = tid; cc < a.C; cc += kBlock) {
        const float* slot = a.ws.wsum + ((long long)b * a.C + cc) * 2;
        sW[cc] = published(slot);
        sPm[cc] = published(slot + 1);
    }
    __syncthreads();
    if (tid == 0) {
        publish(&a.ws.counter2[(long long)b * kCounterStride], 0u);   // ready for the next call
        unsigned flags = sDw[DW_FLAGS];
        float W = 0.f;
        for (int cc = 0; cc < a.C; ++cc) W += sW[cc];
        float wres = 0.f;
        if (wt.residual) {
            wres = W;
            if (!(W > 0.f) || !__builtin_isfinite(W)) {
                // the correction mass vanished (p == q where the draft was
                // rejected, or rounding): sample from p at that position
                flags |= SPECV_FLAG_RESIDUAL_FALLBACK;
                wt.residual = 0;
                W = 0.f;
                for (int cc = 0; cc < a.C; ++cc) {
                    sW[cc] = sPm[cc];
                    W += sW[cc];
                }
            }
        }
        const float target = u * W;
        float acc = 0.f, base = 0.f, lastbase = 0.f;
        int chosen = -1, lastc = -1;
        for (int cc = 0; cc < a.C; ++cc) {
            const float v = sW[cc];
            if (v > 0.f) {
                lastc = cc;
                lastbase = acc;
            }
            if (chosen < 0 && acc + v > target) {
                chosen = cc;
                base = acc;
            }
            acc += v;
        }
        if (chosen < 0) {        // rounding: clamp to the last chunk with weight
            chosen = lastc;
            base = lastbase;
        }
        sChunk = chosen;
        sBase = base;
        sTarget = target;
        sRes = wt.residual;
        sWres = wres;
        sFlags = flags;
        sTok = 0x7fffffff;
    }
    __syncthreads();
    wt.residual = sRes;
    const int cs = sChunk;
    int sampled = -1;
    if (cs >= 0) {
        const int v0 = cs * kChunk;
        const int len = min(kChunk, a.V - v0);
        float w[kPerThread];
        float tot = 0.f;
        int lastpos = -1;
        {
            float zt[kPerThread], zq[kPerThread];
            load_contig<BF16, VEC>(trow, v0, len, zt);
            if (wt.residual) load_contig<BF16, VEC>(qrow, v0, len, zq);
#pragma unroll
            for (int k = 0; k < kPerThread; ++k) {
                const int v = tid * kPerThread + k;
                const float wk = v < len ? wt.w(zt[k], wt.residual ? zq[k] : 0.f) : 0.f;
                w[k] = wk;
                tot += wk;
                if (wk > 0.f) lastpos = v;
            }
        }
        // inclusive scan of the per-thread totals (thread order = token order)
        const float incl = wave_scan_incl(tot);
        __shared__ float wtot[kWaves];
        __shared__ int wlast[kWaves];
        if (lane == kWave - 1) wtot[wave] = incl;
        __syncthreads();
        float wbase = 0.f;
        for (int w2 = 0; w2 < wave; ++w2) wbase += wtot[w2];
        const float excl = sBase + wbase + (incl - tot);
        const float inc = sBase + wbase + incl;
        const float target = sTarget;
        // the first thread whose range crosses the target finds the token
        const unsigned long long hit = __ballot(inc > target && tot > 0.f);
        if (hit) {
            const int first = __ffsll((unsigned long long)hit) - 1;
            if (lane == first) {
                float run = 0.f;
                int tk = lastpos;
                bool found = false;
#pragma unroll
                for (int k = 0; k < kPerThread; ++k) {
                    run += w[k];
                    if (!found && w[k] > 0.f && excl + run > target) {
                        tk = tid * kPerThread + k;
                        found = true;
                    }
                }
                atomicMin(&sTok, tk);
            }
        }
        const int lp = wave_max_i(lastpos);
        if (lane == 0) wlast[wave] = lp;
        __syncthreads();
        if (tid == 0) {
            int tk = sTok;
            if (tk == 0x7fffffff) {                 // rounding: the last token with weight
                tk = -1;
                for (int w2 = 0; w2 < kWaves; ++w2) tk = max(tk, wlast[w2]);
            }
            sTok = tk < 0 ? -1 : v0 + tk;
        }
        __syncthreads();
        sampled = sTok;
    }
    if (tid == 0) {
        unsigned flags = sFlags;
        const bool dead = sampled < 0;        // no weight anywhere: cannot happen for finite rows
        if (dead) flags |= SPECV_FLAG_NONFINITE_ROW;
        write_outputs(a, b, reinterpret_cast<const int*>(&sDw[DW_EMIT]), (int)sDw[DW_NEMIT],
                      (int)sDw[DW_NACC], flags, dead, sampled, sWres);
    }
    __syncthreads();      // shared state is reused by the next item
}

// ---------------------------------------------------------------- k_verify
// One launch per call, one workgroup per piece of work:
//   blocks [0, units):            streaming unit t = (b, r, unit), in batch-row
//                                 order; the last unit of a row decides it;
//   blocks [units, units + items): sampling item (b, c), waiting for its row's
//                                 decision.
// Workgroups are dispatched in increasing order within each XCD, so every
// streaming workgroup has been dispatched (and never waits) before any
// sampling workgroup that could wait for it: the waits always end.  Sampling
// of early rows overlaps the streaming of later ones.
//
// TRUNC selects the variant with the truncation path (handles created with
// max_top_k > 0); without it truncated rows are flagged unsupported and the
// kernel stays lean (registers and LDS of the streaming path only).
template <bool BF16, bool VEC, bool TRUNC>
__global__ __launch_bounds__(kBlock, 4) void k_verify(Args a) {
    const int units = a.B * a.R * a.U;
    const int t = blockIdx.x;
    if (t < units) {
        if constexpr (TRUNC) {
            __shared__ TruncScratch sc;
            stream_unit<BF16, VEC, true>(a, t, &sc);
        } else {
            stream_unit<BF16, VEC, false>(a, t, nullptr);
        }
    } else {
        sample_item<BF16, VEC>(a, (t - units) / a.C, (t - units) % a.C);
    }
}

using KernelFn = void (*)(Args);

KernelFn pick(bool bf16, bool vec, bool trunc) {
    if (trunc) {
        if (bf16) return vec ? k_verify<true, true, true> : k_verify<true, false, true>;
        return vec ? k_verify<false, true, true> : k_verify<false, false, true>;
    }
    if (bf16) return vec ? k_verify<true, true, false> : k_verify<true, false, false>;
    return vec ? k_verify<false, true, false> : k_verify<false, false, false>;
}

}  // namespace

hipError_t launch_verify(const Args& a, bool bf16, bool vec, hipStream_t stream, hipEvent_t* ev) {
    const int blocks = a.B * a.R * a.U + a.B * a.C;
    if (ev) (void)hipEventRecord(ev[0], stream);
    hipLaunchKernelGGL(pick(bf16, vec, a.cand_cap > 0), dim3(blocks), dim3(kBlock), 0, stream, a);
    if (ev) (void)hipEventRecord(ev[1], stream);
    return hipGetLastError();
}

}  // namespace specv
