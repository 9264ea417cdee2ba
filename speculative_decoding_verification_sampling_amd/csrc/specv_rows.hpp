// Row-level device code shared by the verify and draft-sampler kernels:
// per-row plans (mode, caps, temperature scale), workspace indexing, output
// helpers, and the truncation steps (top-k candidates per chunk, the
// row-level top-k / top-p merge into a kept list, draws from a kept list).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "specv_device.hpp"
#include "specv_internal.hpp"

namespace specv {
namespace {

enum Mode { MODE_SAMPLE = 0, MODE_GREEDY = 1, MODE_TRUNC = 2, MODE_SKIP = 3 };
// What stands for the proposal q (a template parameter, so that each kind
// is a kernel of its own):
//   kPropLogits: draft logits rows, reduced by the stream like the target's;
//   kPropPoint:  q_i is the point mass on d_i, no draft rows exist;
//   kPropStats:  draft logits rows plus the drafter's row statistics (max,
//                sum, kept-set threshold: specv_draft_stats), so the stream
//                reads no draft row: the accept test loads q's entry at d_i,
//                and only the row where the round stops is read, for the
//                correction draw (its kept-list entries, for truncated rows).
constexpr int kPropLogits = 0, kPropPoint = 1, kPropStats = 2;
enum Kind { KIND_NONE = 0, KIND_RESIDUAL = 1, KIND_BONUS = 2 };
// outcome of one pair (low byte of PW_STATE)
enum Outcome { OUT_ACC = 1, OUT_REJ = 2, OUT_BAD = 3, OUT_BONUS = 4 };

// ---------------------------------------------------------------- row plan
// What one batch row needs, from its parameters and draft tokens alone.
struct Plan {
    int mode;
    int cap;        // tokens the round may emit: max_new_tokens and the first EOS
    int nt;         // positions whose target row the round may consult: min(cap, gamma + 1)
    int ntest;      // accept tests the round may run: min(cap, gamma)
    float scale;    // log2(e) / T
    int top_k;
    float top_p;
    int keff;       // truncated rows: candidates wanted per chunk (top_k, or the handle's
                    // max_top_k for top-p alone or a larger top_k, whose rows are
                    // truncated exactly)
    int kmode;      // truncated rows: 1 when top-k is on (normaliser over the top-k set)
    unsigned flags;
    int tok;        // lane i < gamma: draft token d_i
};

// Computed by every wave on its own: lane i loads d_i, so the parameters and
// all the tokens arrive in one memory round trip.
__device__ inline Plan make_plan(const Args& a, int b) {
    const int lane = threadIdx.x % kWave;
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
    const int d = lane < a.gamma ? a.tokens[(long long)b * a.gamma + lane] : 0;
    p.tok = d;
    // emission ends after max_new_tokens tokens and after an emitted EOS; an
    // EOS among the drafts therefore caps the round at its position + 1
    int ce = cap >= 1 ? cap : 0x7fffffff;
    const unsigned long long oor = __ballot(lane < a.gamma && (d < 0 || d >= a.V));
    const unsigned long long eos = __ballot(lane < a.gamma && d == a.eos);
    p.flags = oor ? SPECV_FLAG_TOKEN_OOR : 0u;
    if (eos) ce = min(ce, __builtin_ctzll(eos) + 1);
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
        if (a.cand_cap == 0) {
            p.mode = MODE_SKIP;               // the handle reserved no room for candidates
            p.flags |= SPECV_FLAG_UNSUPPORTED;
        } else {
            p.mode = MODE_TRUNC;
        }
    } else {
        p.mode = MODE_SAMPLE;
    }
    p.scale = greedy ? 0.f : kLog2e / T;
    p.kmode = topk_on ? 1 : 0;
    p.keff = topk_on ? min(k, a.max_top_k) : a.max_top_k;
    p.nt = min(ce, a.gamma + 1);
    p.ntest = min(ce, a.gamma);
    return p;
}


// ---------------------------------------------------------------- workspace
__device__ inline long long pair_id(const Args& a, int b, int k) { return (long long)b * a.P + k; }

// Draft token d_k of row b, by a load from the same (uniform) address in
// every lane.  Never a cross-lane read of the plan's lane-distributed
// tokens: in code that only some lanes execute, the compiler may reload a
// spilled register for the active lanes alone, and a read of another lane
// then returns garbage.
__device__ inline int draft_token(const Args& a, int b, int k) {
    return a.tokens[(long long)b * a.gamma + k];
}
__device__ inline long long side_row(const Args& a, int b, int k, int side) {
    return pair_id(a, b, k) * 2 + side;
}
__device__ inline long long part_index(const Args& a, int b, int k, int side, int c) {
    return side_row(a, b, k, side) * a.C + c;
}

// A chunk's statistics move as two epoch-tagged words: (max, sum) for
// sampling and truncated rows, the sum NaN when the chunk held NaN / +inf;
// (max, argmax) for greedy rows, the max NaN when the chunk held NaN / +inf.
// Readers poll until both tags are this call's, so the writer never waits
// for its stores to complete.
__device__ inline unsigned long long* stats_words(const Args& a, int b, int k, int side, int c) {
    return a.ws.stats + part_index(a, b, k, side, c) * 2;
}

// ---------------------------------------------------------------- call number
// Every launch needs a tag of its own for the words it publishes, and a
// parity that alternates from launch to launch (the record set it uses).
// Both come from a call number kept on the device, so that a launch replayed
// from a captured graph (whose arguments are frozen) still gets a new one:
//   - every workgroup reads the number with a plain load (it changes only
//     between launches, so a cached copy is this launch's), then counts
//     itself in seen[parity][its batch row] with an atomic add whose address
//     depends on what it read, so the count lands after the read;
//   - the launch has one workgroup more than its work needs, the last one,
//     which waits until every row's count is complete, resets the counts,
//     records the launch's extent in dims[parity] and stores number + 1.
// Nothing on a workgroup's own path waits for these atomics.  The closing
// workgroup is dispatched after every other workgroup of its XCD and no
// workgroup waits for it, so its wait ends.
__device__ inline unsigned read_call(const Workspace& ws) { return ws.calls[0]; }

// One thread per workgroup: count this workgroup (batch row b) as having
// read call number e.
__device__ inline void count_call(const Workspace& ws, unsigned e, int b) {
    (void)__hip_atomic_fetch_add(ws.seen + ((long long)(e & 1u) * ws.n_rows + b) * kSlot, 1u, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
}

// A launch's extent: batch rows, positions per row and chunks per row (the
// region of each record array its indexing can reach).
__device__ inline unsigned long long pack_dims(int B, int P, int C) {
    return (unsigned long long)(unsigned)B | ((unsigned long long)(unsigned)P << 32) |
           ((unsigned long long)(unsigned)C << 40);
}

// The closing workgroup of a launch with B rows of per_row workgroups each
// (whole workgroup): waits (bounded) for every row's count, resets the
// counts, records the extent ``dims`` for the launch that clears this
// parity's record set, and advances the call number.
__device__ inline void close_call(const Workspace& ws, int B, unsigned per_row, unsigned long long dims) {
    const unsigned e = read_call(ws);
    unsigned* seen = ws.seen + (long long)(e & 1u) * ws.n_rows * kSlot;
    for (int r = threadIdx.x; r < B; r += kBlock) {
#pragma unroll 1
        for (int spin = 0; spin < kSpinLimit; ++spin) {    // (fixed: bookkeeping, no row waits on it)
            if (published(seen + (long long)r * kSlot) >= per_row) break;
            __builtin_amdgcn_s_sleep(4);
        }
    }
    __syncthreads();
    for (int r = threadIdx.x; r < B; r += kBlock) publish(seen + (long long)r * kSlot, 0u);
    if (threadIdx.x == 0) {
        publish(ws.dims + (e & 1u), dims);
        publish(ws.calls, e + 1u);
    }
}

// The tag of call number e: odd, so never the zero of a cleared word.
__device__ inline unsigned call_tag(unsigned e) { return 2u * e + 1u; }

// The record set of parity par.  Host-numbered workspaces hold one set of
// the tagged records (set sizes 0): only their counters and status words
// come in two sets, and SETS = false leaves the other pointers as they are.
template <bool SETS = true>
__device__ inline Workspace parity_set(const Workspace& ws, unsigned par) {
    Workspace w = ws;
    if constexpr (SETS) {
        w.stats += par * ws.set_stats;
        w.pair += par * ws.set_pair;
        w.rowrec += par * ws.set_rowrec;
        w.wsum += par * ws.set_wsum;
    }
    w.ctr += (long long)par * ws.n_groups * kSlot;
    w.status += (long long)par * ws.n_rows * (kSlot / 2);
    return w;
}

// Share ``wg`` of ``nwg`` workgroups (whole workgroup): zero the record set
// of the parity other than call number e's, over the extent of the last
// launch that used it (its B rows, P positions and C chunks).
__device__ inline void clear_other_set(const Workspace& ws0, unsigned e, long long wg, long long nwg) {
    const unsigned long long d = ws0.dims[(e & 1u) ^ 1u];   // written by an earlier launch
    const long long B = (long long)(unsigned)d, P = (long long)((d >> 32) & 0xffu), C = (long long)((d >> 40) & 0xffu);
    if (B == 0) return;
    const Workspace ws = parity_set(ws0, (e & 1u) ^ 1u);
    const long long stride = nwg * kBlock;
    const long long i0 = wg * kBlock + threadIdx.x;
    const long long n_stats = B * P * 2 * C * 2, n_pair = B * P * kPairWords, n_row = B * kRowWords,
                    n_wsum = B * C * 2, n_ctr = B * P;
    for (long long i = i0; i < n_stats; i += stride) publish(ws.stats + i, 0ull);
    for (long long i = i0; i < n_pair; i += stride) publish(&ws.pair[i / kPairWords].w[i % kPairWords], 0ull);
    for (long long i = i0; i < n_row; i += stride) publish(ws.rowrec + i, 0ull);
    for (long long i = i0; i < n_wsum; i += stride) publish(ws.wsum + i, 0ull);
    for (long long i = i0; i < n_ctr; i += stride) publish(ws.ctr + i * kSlot, 0u);
    for (long long i = i0; i < B; i += stride) publish(ws.status + i * (kSlot / 2), 0ull);
}

// Diagnostics of one row by one wave: lane i holds p_i(d_i), q_i(d_i).
__device__ inline void write_diag_wave(const Args& a, int b, int tested, float p, float q) {
    const int i = threadIdx.x % kWave;
    if (i < a.gamma) {
        const bool t = i < tested;
        if (a.p_at) a.p_at[(long long)b * a.gamma + i] = t ? p : __builtin_nanf("");
        if (a.q_at) a.q_at[(long long)b * a.gamma + i] = t ? q : __builtin_nanf("");
    }
}

// Final outputs of one row by one wave (lane i holds d_i in ``tok``): the
// first nemit drafts, then ``sampled`` (if >= 0), -1 padding.
__device__ inline void write_outputs_wave(const Args& a, int b, int nemit, int nacc, unsigned flags,
                                          bool dead, int sampled, float wres, int tok) {
    const int lane = threadIdx.x % kWave;
    const int g1 = a.gamma + 1;
    if (dead) {
        nemit = 0;
        nacc = 0;
        sampled = -1;
    }
    if (lane < g1) {
        int t = -1;
        if (lane < nemit) t = tok;
        else if (lane == nemit && sampled >= 0) t = sampled;
        a.out_tok[(long long)b * g1 + lane] = t;
    }
    if (lane == 0) {
        a.out_emit[b] = nemit + (sampled >= 0 ? 1 : 0);
        a.out_acc[b] = nacc;
        if (a.out_flags) a.out_flags[b] = (int)flags;
        if (a.wres) a.wres[b] = wres;
    }
}

// ---------------------------------------------------------------- truncation
// Top-k / top-p rows ("11.1 核心原理" 11.1.2: p and q are the distributions
// after truncation; q is the truncated proposal actually sampled).
//   per chunk:   each thread keeps its top-j finite values (j = ceil(2k / 256)
//                <= 8); the k-th largest of those 256 j values, L, has at
//                least k chunk entries >= L, so every finite entry >= L is a
//                superset of the chunk's top k (typically ~k entries);
//   per row:     (the workgroup deciding the position) the row's top-k
//                threshold is >= every chunk's L, so only candidates >= max L
//                are gathered (at most 2048); a radix select finds the k-th
//                largest of them, the top-k threshold (ties kept); the
//                entries at or above it are sorted (value desc, index asc)
//                and scanned for top-p: the first level whose cumulative
//                mass reaches top_p ends the kept set (ties at a level all
//                kept); a pair's target and draft rows go through these steps
//                in lockstep when both take the usual path, and a list of at
//                most 64 entries is sorted, scanned and cut by one wave;
//   per batch row: the accept tests use the kept sets, and the correction /
//                bonus sample is drawn from the (short) kept list of the
//                sampled row, tokens in ascending index order.

__device__ inline bool finite_logit(float x) { return x > -kInf && x <= 3.402823466e38f; }

__device__ inline void publish_cand(Cand* p, float v, int idx) {
    const unsigned long long w =
        (unsigned long long)__float_as_uint(v) | ((unsigned long long)(unsigned)idx << 32);
    publish(reinterpret_cast<unsigned long long*>(p), w);
}

__device__ inline Cand published_cand(const Cand* p) {
    const unsigned long long w = published(reinterpret_cast<const unsigned long long*>(p));
    Cand c;
    c.v = __uint_as_float((unsigned)w);
    c.idx = (int)(unsigned)(w >> 32);
    return c;
}

// Orders for rank_sort, without short-circuit evaluation (a branch there
// would wait on each LDS load in turn).
struct ByValue {      // value desc, index asc
    __device__ bool operator()(float va, int ia, float vb, int ib) const {
        return (va > vb) | ((va == vb) & (ia < ib));
    }
};
struct ByIndex {      // index asc
    __device__ bool operator()(float, int ia, float, int ib) const { return ia < ib; }
};

// Block-wide rank sort of (iv, ii) [0, n) into (ov, oi): entry x lands at
// the number of entries y with prec(y, x), so prec must order the entries
// strictly (ByValue or ByIndex, with distinct indices).  n comparisons per
// entry, split over the waves for short lists (partial ranks summed through
// part, kBlock ints of LDS): for the kept sets here it beats a bitonic
// network, whose log^2 n barrier-separated stages dominate the row merge.
// The inputs are kKeptCap-entry, 16-byte aligned LDS arrays (read four
// entries at a time, up to n rounded up to a multiple of four), visible to
// the block and not aliasing the outputs; the result is visible on return.
template <typename Prec>
__device__ void rank_sort(const float* iv, const int* ii, int n, float* ov, int* oi, Prec prec,
                          int* part) {
    const int J = n <= kWave ? 4 : (n <= 2 * kWave ? 2 : 1);     // comparison ranges per entry
    if (J == 1) {
        for (int i = threadIdx.x; i < n; i += kBlock) {
            const float vi = iv[i];
            const int xi = ii[i];
            int r = 0;
#pragma unroll 4
            for (int j = 0; j < n; j += 4) {
                const float4 v4 = *reinterpret_cast<const float4*>(iv + j);
                const int4 i4 = *reinterpret_cast<const int4*>(ii + j);
                r += (int)prec(v4.x, i4.x, vi, xi);
                r += (int)((j + 1 < n) & prec(v4.y, i4.y, vi, xi));
                r += (int)((j + 2 < n) & prec(v4.z, i4.z, vi, xi));
                r += (int)((j + 3 < n) & prec(v4.w, i4.w, vi, xi));
            }
            ov[r] = vi;
            oi[r] = xi;
        }
        __syncthreads();
        return;
    }
    const int width = kBlock / J;                           // entries per range group
    const int i = (int)threadIdx.x % width, g = (int)threadIdx.x / width;
    const int len = (n + 4 * J - 1) / (4 * J) * 4;          // comparisons per range
    const int j0 = g * len, j1 = min(n, j0 + len);
    float vi = 0.f;
    int xi = 0, r = 0;
    if (i < n) {
        vi = iv[i];
        xi = ii[i];
        for (int j = j0; j < j1; j += 4) {
            const float4 v4 = *reinterpret_cast<const float4*>(iv + j);
            const int4 i4 = *reinterpret_cast<const int4*>(ii + j);
            r += (int)prec(v4.x, i4.x, vi, xi);
            r += (int)((j + 1 < j1) & prec(v4.y, i4.y, vi, xi));
            r += (int)((j + 2 < j1) & prec(v4.z, i4.z, vi, xi));
            r += (int)((j + 3 < j1) & prec(v4.w, i4.w, vi, xi));
        }
    }
    part[threadIdx.x] = r;
    __syncthreads();
    if (g == 0 && i < n) {
        for (int h = 1; h < J; ++h) r += part[h * width + i];
        ov[r] = vi;
        oi[r] = xi;
    }
    __syncthreads();
}

// Slot of this lane's entry in an LDS list whose length is *count (one
// atomic per wave), or -1 when the lane keeps nothing.
__device__ inline int wave_reserve(bool keep, int* count) {
    const unsigned long long m = __ballot(keep);
    if (m == 0) return -1;
    const int lead = __ffsll((long long)m) - 1;
    int base = 0;
    if ((int)(threadIdx.x % kWave) == lead) base = atomicAdd(count, __popcll(m));
    base = __shfl(base, lead, kWave);
    const int below = __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
    return keep ? base + below : -1;
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

// Inclusive prefix sum of in[0, n) into out[0, n) (in == out allowed),
// n <= kKeptCap: eight consecutive entries per thread in order, then across
// threads.
__device__ void block_inclusive_scan(const float* in, float* w, int n, float* red) {
    constexpr int per = kKeptCap / kBlock;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int base = threadIdx.x * per;
    float loc[per];
    float run = 0.f;
#pragma unroll
    for (int j = 0; j < per; ++j) {
        run += base + j < n ? in[base + j] : 0.f;
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

// Value whose order key is ``key`` (the inverse of order_key for keys of
// float32 values); for a key with its low bits cleared, the smallest value
// of that key range.
__device__ inline float key_value(unsigned key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Value whose order key (order_key<BF16>, so bf16 keys are 16 bits) is key.
template <bool BF16>
__device__ inline float value_of_key(unsigned key) {
    if (BF16) {
        const unsigned k32 = key << 16;
        return __uint_as_float((k32 & 0x80000000u) ? (k32 & 0x7fffffffu) : (~k32 & 0xffff0000u));
    }
    return key_value(key);
}

// Wave 0 of the workgroup: the bin t of the 256-bin histogram h (bins in
// ascending key order) that holds the need-th largest entry: *sel = t and
// *rest = need - (entries in the bins above t); *found = 0 when h holds
// fewer than need entries.  h must be visible to the wave.
__device__ inline void wave_find_bin(const unsigned* h, int need, unsigned* sel, int* rest,
                                     int* found) {
    const int lane = threadIdx.x % kWave;
    const uint4 v = *reinterpret_cast<const uint4*>(h + 4 * lane);
    const int cs[4] = {(int)v.x, (int)v.y, (int)v.z, (int)v.w};
    const int own = cs[0] + cs[1] + cs[2] + cs[3];
    const int incl = wave_scan_incl(own);
    const int total = __shfl(incl, kWave - 1, kWave);
    if (lane == 0 && total < need) *found = 0;
    int ge = total - (incl - own);                          // entries in bins >= 4 * lane
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (ge >= need && ge - cs[e] < need) {              // exactly one lane and bin
            *sel = (unsigned)(4 * lane + e);
            *rest = need - (ge - cs[e]);
        }
        ge -= cs[e];
    }
}

// Order key of the K-th largest (with multiplicity) of the finite values
// v[0, n) in LDS, 1 <= K <= n: a radix select over 8-bit digits from the top
// (two passes for bf16 keys, four for float32), one histogram per digit in
// sc.idx2, each bin found by wave 0.  v must be visible to the block; the
// result is returned to every thread.
template <bool BF16>
__device__ unsigned lds_select_kth(const float* v, int n, int K, TruncScratch& sc) {
    constexpr int NP = BF16 ? 2 : 4;
    constexpr int KB = 8 * NP;
    const int tid = threadIdx.x, wave = tid / kWave;
    unsigned* h = reinterpret_cast<unsigned*>(sc.idx2);
    __shared__ unsigned sSel;
    __shared__ int sRest, sFound;
    __syncthreads();                                        // sc.idx2 may still be read
#pragma unroll
    for (int p = 0; p < NP; ++p) h[p * 256 + tid] = 0;      // kBlock == 256 bins
    __syncthreads();
    unsigned prefix = 0;
    int need = K;
#pragma unroll
    for (int pass = 0; pass < NP; ++pass) {
        const int shift = KB - 8 * (pass + 1);
        unsigned* hp = h + 256 * pass;
        for (int i = tid; i < n; i += kBlock) {
            const unsigned key = order_key<BF16>(v[i]);
            if (pass == 0 || (key >> (shift + 8)) == prefix) atomicAdd(&hp[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (wave == 0) wave_find_bin(hp, need, &sSel, &sRest, &sFound);
        __syncthreads();
        // read before wave 0 updates them (after the next pass's barrier)
        prefix = (prefix << 8) | sSel;
        need = sRest;
    }
    return prefix;
}

// This thread's top jj (<= 8) finite entries of a chunk as 16-bit order keys,
// largest first (0: none).
template <typename Regs>
__device__ __forceinline__ void thread_top_keys(const Regs& r, int jj, unsigned (&k16)[8]) {
    float tp[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) tp[j] = -kInf;
    if (jj == 1) {                                          // top_k <= 128: the maximum
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) {
            const float v = r.elem(k);
            if (finite_logit(v)) tp[0] = fmaxf(tp[0], v);
        }
    } else {
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) {
            float v = r.elem(k);
            if (!(finite_logit(v) && v > tp[7])) continue;
#pragma unroll
            for (int j = 0; j < 8; ++j) {                   // insertion, larger values first
                if (v > tp[j]) {
                    const float t = tp[j];
                    tp[j] = v;
                    v = t;
                }
            }
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) k16[j] = j < jj && finite_logit(tp[j]) ? order_key<false>(tp[j]) >> 16 : 0u;
}

// Publishes this thread's entries of a chunk that are finite and >= L into
// dst (slots by a wave prefix sum and one LDS atomic per wave on *count; the
// order within the list is immaterial); slots past cap are only counted.
template <bool BF16, typename Regs>
__device__ __forceinline__ void emit_candidates(const Regs& r, float L, Cand* dst, int cap, int v0,
                                                int* count) {
    const int lane = threadIdx.x % kWave;
    unsigned kept = 0;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        const float x = r.elem(k);
        kept |= (finite_logit(x) && x >= L) ? (1u << k) : 0u;
    }
    const int cnt = __popc(kept);
    const int incl = wave_scan_incl(cnt);
    int base = 0;
    if (lane == kWave - 1) base = atomicAdd(count, incl);
    base = __shfl(base, kWave - 1, kWave);
    int o = base + incl - cnt;
    while (kept) {
        const int k = __ffs(kept) - 1;
        kept &= kept - 1;
        if (o < cap) publish_cand(dst + o, r.elem_dyn(k), v0 + chunk_index<BF16>(k));
        ++o;
    }
}

// Candidates of one chunk (whole workgroup) held in registers, for one row or
// for two at once (a unit's target and draft rows share the barriers): every
// finite entry >= L, where L is a lower bound of the chunk's keff-th largest
// entry: each thread keeps its top jj = ceil(2 keff / 256) <= 8 finite
// entries, so at least keff chunk entries are >= the keff-th largest of those
// 256 jj values; that value is found over the top 16 bits of the values'
// order keys, which for float32 rounds it down to the start of its key range
// (still a lower bound): with one value per thread (jj = 1, keff <= 128) by
// one wave per row, bit by bit from the top (ballot counts of the keys at or
// above each trial prefix: three barriers in all), else by a radix select
// (two 8-bit digits, each from an LDS histogram whose bin one wave finds).
// Both give the same key.  Row 1 (r1) is used only when two.
// max0 / max1: the threads' maxima from the statistics pass when given
// (have_max), used as the tops when jj = 1 (a non-finite maximum means no
// finite top, or a row the merge rejects as bad).
template <bool BF16, typename Regs>
__device__ __forceinline__ void chunk_candidates_pair(const Args& a, long long row0, long long row1, bool two, int c,
                                      int keff, const Regs& r0, const Regs& r1, TruncScratch& sc,
                                      bool have_max = false, float max0 = 0.f, float max1 = 0.f) {
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int jj = min(8, (2 * keff + kBlock - 1) / kBlock);
    unsigned ka[8], kb[8];
    if (have_max && jj == 1) {
#pragma unroll
        for (int j = 0; j < 8; ++j) ka[j] = kb[j] = 0u;
        ka[0] = finite_logit(max0) ? order_key<false>(max0) >> 16 : 0u;
        if (two) kb[0] = finite_logit(max1) ? order_key<false>(max1) >> 16 : 0u;
    } else {
        thread_top_keys(r0, jj, ka);
        if (two) {
            thread_top_keys(r1, jj, kb);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) kb[j] = 0u;
        }
    }
    if (jj == 1) {
        // one key per thread: the keys to LDS (row 0 in sc.hist, row 1 in
        // sc.idx2), then one wave per row finds the keff-th largest bit by
        // bit from the top (ballot counts of keys >= each trial prefix)
        unsigned* ka_s = sc.hist;
        unsigned* kb_s = reinterpret_cast<unsigned*>(sc.idx2);
        __shared__ float sLsel[2];
        __shared__ int sCnt1[2];
        __syncthreads();                                    // sc may still be read
        ka_s[tid] = ka[0];
        kb_s[tid] = kb[0];
        if (tid < 2) sCnt1[tid] = 0;
        __syncthreads();
        if (wave < (two ? 2 : 1)) {
            const uint4 q = *reinterpret_cast<const uint4*>((wave ? kb_s : ka_s) + 4 * lane);
            const unsigned k4[4] = {q.x, q.y, q.z, q.w};
            int nz = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) nz += __popcll(__ballot(k4[e] != 0u));
            float L = -kInf;                                // fewer finite tops than keff
            if (nz >= keff) {
                unsigned T = 0;
#pragma unroll
                for (int bit = 15; bit >= 0; --bit) {
                    const unsigned trial = T | (1u << bit);
                    int cnt = 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) cnt += __popcll(__ballot(k4[e] >= trial));
                    if (cnt >= keff) T = trial;
                }
                L = key_value(T << 16);
            }
            if (lane == 0) sLsel[wave] = L;
        }
        __syncthreads();
        const float La = sLsel[0];
        const float Lb = two ? sLsel[1] : -kInf;
        const int v0 = c * kChunk;
        emit_candidates<BF16>(r0, La, a.ws.cand + cand_base(a, row0, c), a.cand_cap, v0, &sCnt1[0]);
        if (two) emit_candidates<BF16>(r1, Lb, a.ws.cand + cand_base(a, row1, c), a.cand_cap, v0, &sCnt1[1]);
        wait_stores();
        __syncthreads();
        if (tid == 0) {
            const int total = sCnt1[0];
            publish_cand(a.ws.cand_meta + row0 * a.C + c, La, total <= a.cand_cap ? total : -1);
        } else if (two && tid == kWave) {
            const int total = sCnt1[1];
            publish_cand(a.ws.cand_meta + row1 * a.C + c, Lb, total <= a.cand_cap ? total : -1);
        }
        return;
    }
    // first digit: histograms h0a / h0b; second digit: h1a / h1b
    unsigned* h0a = sc.hist;                                // kBlock == 256 bins each
    unsigned* h1a = reinterpret_cast<unsigned*>(sc.idx2);
    unsigned* h0b = h1a + 256;
    unsigned* h1b = h1a + 512;
    __shared__ unsigned sSel[2];
    __shared__ int sRest[2], sFound[2], sCount[2];
    __syncthreads();                                        // sc may still be read
    h0a[tid] = 0;
    h1a[tid] = 0;
    h0b[tid] = 0;
    h1b[tid] = 0;
    if (tid < 2) {
        sFound[tid] = 1;
        sCount[tid] = 0;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (ka[j]) atomicAdd(&h0a[ka[j] >> 8], 1u);
        if (kb[j]) atomicAdd(&h0b[kb[j] >> 8], 1u);
    }
    __syncthreads();
    if (wave == 0) wave_find_bin(h0a, keff, &sSel[0], &sRest[0], &sFound[0]);
    else if (wave == 1 && two) wave_find_bin(h0b, keff, &sSel[1], &sRest[1], &sFound[1]);
    __syncthreads();
    // read before waves 0 / 1 update them below (after the next barrier)
    const unsigned da = sSel[0], db = sSel[1];
    const int na = sRest[0], nb = sRest[1];
    const bool fa = sFound[0] != 0;                         // else fewer finite tops than keff
    const bool fb = two && sFound[1] != 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (fa && ka[j] && (ka[j] >> 8) == da) atomicAdd(&h1a[ka[j] & 255u], 1u);
        if (fb && kb[j] && (kb[j] >> 8) == db) atomicAdd(&h1b[kb[j] & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0 && fa) wave_find_bin(h1a, na, &sSel[0], &sRest[0], &sFound[0]);
    else if (wave == 1 && fb) wave_find_bin(h1b, nb, &sSel[1], &sRest[1], &sFound[1]);
    __syncthreads();
    const float La = fa ? key_value(((da << 8) | sSel[0]) << 16) : -kInf;
    const float Lb = fb ? key_value(((db << 8) | sSel[1]) << 16) : -kInf;
    const int v0 = c * kChunk;
    emit_candidates<BF16>(r0, La, a.ws.cand + cand_base(a, row0, c), a.cand_cap, v0, &sCount[0]);
    if (two) emit_candidates<BF16>(r1, Lb, a.ws.cand + cand_base(a, row1, c), a.cand_cap, v0, &sCount[1]);
    // a barrier does not wait for other waves' stores: each wave completes
    // its own, so that the lists are out before the unit's arrival is counted
    wait_stores();
    __syncthreads();
    if (tid == 0) {
        const int total = sCount[0];
        publish_cand(a.ws.cand_meta + row0 * a.C + c, La, total <= a.cand_cap ? total : -1);
    } else if (two && tid == kWave) {
        const int total = sCount[1];
        publish_cand(a.ws.cand_meta + row1 * a.C + c, Lb, total <= a.cand_cap ? total : -1);
    }
}

// One row's candidates of one chunk (see chunk_candidates_pair).
template <bool BF16, typename Regs>
__device__ inline void chunk_candidates(const Args& a, long long rowid, int c, int keff, const Regs& r,
                                        TruncScratch& sc) {
    chunk_candidates_pair<BF16>(a, rowid, rowid, false, c, keff, r, r, sc);
}

// ---------------------------------------------------------------- exact truncation
// The slow path, for rows whose truncation the candidate lists cannot
// settle: heavy ties at the top-k threshold (a chunk's candidates overflow
// their slots), top-p without top-k on a flat row (the kept set needs more
// entries than the candidates hold), top_k above the handle's max_top_k.
// The top-k threshold (the k-th largest finite value, ties kept) and the
// top-p threshold (the largest value t whose set {z >= t} holds at least
// top_p of the top-k-renormalised mass) come from radix descents over the
// order keys of the whole row, which the deciding workgroup reads from
// global memory: one pass per 8-bit digit (two for bfloat16 keys, four for
// float32), each a 256-bin histogram of the entries still in range.  Counts
// are integers and masses exp2((z - max) * log2(e) / T) are summed in 2^-40
// fixed point, so every sum is exact and independent of the order of
// accumulation.  The row is then kept in threshold form: the kept set
// {z >= tstar} without a list (TruncRow::n_kept == kThresholdForm), its
// normaliser from the same sums; draws from such a row scan the row itself
// (threshold_draw).
constexpr int kThresholdForm = -1;          // TruncRow::n_kept: kept set {z >= tstar}, no list
constexpr int kNeedsExact = -2;             // short_merge_wave: the candidates cannot settle the row
constexpr float kMassUnit = 1099511627776.0f;   // 2^40
constexpr double kInvMassUnit = 1.0 / 1099511627776.0;

__device__ inline unsigned long long mass_fixed(float w) {
    return (unsigned long long)(w * kMassUnit);
}

__device__ inline unsigned long long wave_sum_u64(unsigned long long x) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) x += __shfl_xor(x, o, kWave);
    return x;
}

__device__ inline unsigned long long wave_scan_incl_u64(unsigned long long x) {
    const int lane = threadIdx.x % kWave;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const unsigned long long y = __shfl_up(x, o, kWave);
        if (lane >= o) x += y;
    }
    return x;
}

// Sum over the workgroup (every thread gets it).
__device__ inline unsigned long long block_sum_u64(unsigned long long x) {
    __shared__ unsigned long long red[kWaves];
    x = wave_sum_u64(x);
    __syncthreads();
    if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = x;
    __syncthreads();
    unsigned long long t = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t += red[w];
    __syncthreads();
    return t;
}

// Calls f(z) for every entry of a logits row of length V: coalesced loads
// (thread t reads entries t, t + 256, ...), eight in flight per thread.
template <bool BF16, typename F>
__device__ __forceinline__ void for_row(const void* row, int V, F f) {
    for (int v0 = 0; v0 < V; v0 += 8 * kBlock) {
        float z[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int v = v0 + j * kBlock + (int)threadIdx.x;
            z[j] = v < V ? load_elem<BF16>(row, v) : -kInf;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) f(z[j]);
    }
}

// Radix descent over the finite entries of ``row`` with order key >= kmin,
// each of weight 1 (scale == 0) or of fixed-point mass
// exp2((z - zmax) * scale): the largest key t such that the entries with
// key >= t weigh at least ``need`` (with frac > 0, need = ceil(frac * total
// weight), at least 1).  Returns false, t = kmin, when the total is below
// need.  *above gets the weight of the entries with key > t, *atleast that
// of key >= t, *total the total.  Whole workgroup; the histograms live in
// sc.v (one per wave) and sc.w.
template <bool BF16>
__device__ __forceinline__ bool row_descent(const void* row, int V, unsigned kmin, float zmax, float scale,
                            unsigned long long need, double frac, TruncScratch& sc, unsigned* t,
                            unsigned long long* above, unsigned long long* atleast,
                            unsigned long long* total) {
    constexpr int NP = BF16 ? 2 : 4;
    constexpr int KB = 8 * NP;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const bool weighted = scale != 0.f;
    unsigned long long* hist = reinterpret_cast<unsigned long long*>(sc.v);   // [kWaves][256]
    unsigned long long* tot = reinterpret_cast<unsigned long long*>(sc.w);    // [256]
    __shared__ unsigned dPrefix;
    __shared__ unsigned long long dAbove, dNeed, dTotal, dAtLeast;
    __shared__ int dFound;
    __syncthreads();                                         // sc may still be read
    if (tid == 0) {
        dPrefix = 0;
        dAbove = 0;
        dAtLeast = 0;
        dTotal = 0;
        dNeed = need;
        dFound = 1;
    }
    for (int pass = 0; pass < NP; ++pass) {
        const int shift = KB - 8 * (pass + 1);
#pragma unroll
        for (int w = 0; w < kWaves; ++w) hist[w * 256 + tid] = 0ull;           // kBlock == 256 bins
        __syncthreads();
        const unsigned prefix = dPrefix;
        for_row<BF16>(row, V, [&](float z) {
            const unsigned key = order_key<BF16>(z);
            const bool in = finite_logit(z) && key >= kmin && (pass == 0 || (key >> (shift + 8)) == prefix);
            const unsigned bin = (key >> shift) & 255u;
            const unsigned long long wt = in ? (weighted ? mass_fixed(fast_exp2(__fmul_rn(z - zmax, scale))) : 1ull)
                                             : 0ull;
            // a flat row sends a whole wave to one bin: one atomic for it
            const unsigned long long ins = __ballot(in);
            if (ins == 0) return;
            const unsigned b0 = (unsigned)__shfl((int)bin, __ffsll((long long)ins) - 1, kWave);
            if (__ballot(in && bin != b0) == 0) {
                const unsigned long long s = wave_sum_u64(wt);
                if (lane == 0) atomicAdd(&hist[wave * 256 + b0], s);
            } else if (in) {
                atomicAdd(&hist[wave * 256 + bin], wt);
            }
        });
        __syncthreads();
        unsigned long long h = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) h += hist[w * 256 + tid];
        tot[tid] = h;
        __syncthreads();
        if (tid == 0) {
            if (pass == 0) {
                unsigned long long all = 0;
                for (int d = 0; d < 256; ++d) all += tot[d];
                dTotal = all;
                if (frac > 0.0) {
                    const double n = ceil(frac * (double)all);
                    dNeed = n < 1.0 ? 1ull : (unsigned long long)n;
                }
                if (all < dNeed) dFound = 0;
            }
            if (dFound) {
                unsigned long long run = dAbove;
                unsigned sel = 0;
                for (int d = 255; d >= 0; --d) {
                    if (run + tot[d] >= dNeed) {
                        sel = (unsigned)d;
                        break;
                    }
                    run += tot[d];
                }
                dAbove = run;
                dPrefix = (prefix << 8) | sel;
                dAtLeast = run + tot[sel];
            }
        }
        __syncthreads();
        if (!dFound) break;
    }
    const bool found = dFound != 0;
    *t = found ? dPrefix : kmin;
    *above = dAbove;
    *atleast = dAtLeast;
    *total = dTotal;
    __syncthreads();
    return found;
}

// Fixed-point mass of the finite entries of ``row`` with key >= kmin.
template <bool BF16>
__device__ __forceinline__ unsigned long long row_mass(const void* row, int V, unsigned kmin, float zmax, float scale) {
    unsigned long long part = 0;
    for_row<BF16>(row, V, [&](float z) {
        if (finite_logit(z) && order_key<BF16>(z) >= kmin) part += mass_fixed(fast_exp2(__fmul_rn(z - zmax, scale)));
    });
    return block_sum_u64(part);
}

// The exact truncation of logits row (b, k, side) (whole workgroup), given
// the row's maximum: published as the row's TruncRow in threshold form and
// returned to every thread.  ``flags`` (flags found so far) gains TOPP_NEAR
// when the cumulative mass at the chosen level or the level above lies
// within 1e-5 of top_p.
template <bool BF16>
__device__ __forceinline__ TruncRow row_truncate_exact(const Args& a, int b, int k, int side, const Plan& pl, float zmax,
                                       unsigned flags, TruncScratch& sc) {
    const void* row = side ? row_ptr<BF16>(a.drf, a.d_sb, a.d_sp, b, k) : row_ptr<BF16>(a.tgt, a.t_sb, a.t_sp, b, k);
    TruncRow* tr = &a.ws.trow[side_row(a, b, k, side)];
    unsigned long long above, atleast, total;
    // the top-k threshold: the k-th largest finite value with multiplicity;
    // with fewer finite entries than k every finite entry stays (key 0)
    unsigned kkey = 0;
    if (pl.kmode) {
        unsigned t;
        if (row_descent<BF16>(row, a.V, 0u, zmax, 0.f, (unsigned long long)pl.top_k, 0.0, sc, &t, &above, &atleast,
                              &total))
            kkey = t;
    }
    unsigned key = kkey;
    unsigned long long S2;
    if (pl.top_p < 1.f) {
        // the largest t with mass(key >= t) >= ceil(top_p * mass(key >= kkey))
        row_descent<BF16>(row, a.V, kkey, zmax, pl.scale, 1ull, (double)pl.top_p, sc, &key, &above, &S2, &total);
        const double cj = (double)S2 / (double)total, pv = (double)above / (double)total;
        if (fabs(cj - (double)pl.top_p) < 1e-5 || (above > 0 && fabs(pv - (double)pl.top_p) < 1e-5))
            flags |= SPECV_FLAG_TOPP_NEAR;
    } else {
        S2 = row_mass<BF16>(row, a.V, kkey, zmax, pl.scale);
    }
    __shared__ TruncRow xOut;
    if (threadIdx.x == 0) {
        TruncRow o{};
        o.zmax = zmax;
        // key 0: every finite value is kept
        o.tstar = key ? value_of_key<BF16>(key) : -3.402823466e38f;
        o.S = (float)((double)S2 * kInvMassUnit);
        o.n_kept = kThresholdForm;
        o.flags = flags;
        o.bad = S2 == 0 ? 1u : 0u;
        xOut = o;
        publish(&tr->zmax, o.zmax);
        publish(&tr->tstar, o.tstar);
        publish(&tr->S, o.S);
        publish(&tr->n_kept, o.n_kept);
        publish(&tr->flags, o.flags);
        publish(&tr->bad, o.bad);
    }
    __syncthreads();
    const TruncRow out = xOut;
    __syncthreads();
    return out;
}

// Inverse-CDF draw (whole workgroup) over a whole row of length V in
// ascending token order: weight w(v) = p(v), p from row ``prow`` truncated
// as tP (kept set {z >= tP.tstar}); with ``res``, w(v) = max(p(v) - q(v), 0)
// with q from row ``qrow`` truncated as tQ, or the point mass on token dpm
// when qrow is null.  The token is the first whose running weight exceeds
// u * W; weights are summed in 2^-40 fixed point over tiles of 256 entries
// (a tile per wave at a time, lane i holding entries 4i .. 4i + 3).  When
// the residual weighs nothing the draw falls back to p (*fallback).  *W
// gets the total weight drawn from (before the fallback).  Returns -1 when
// nothing weighs anything.
template <bool BF16>
__device__ __forceinline__ int threshold_draw(const void* prow, const TruncRow& tP, const void* qrow, const TruncRow& tQ, int dpm,
                              bool res, int V, float scale, float u, TruncScratch& sc, float* W, bool* fallback) {
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    constexpr int kTile = 4 * kWave;
    const int ntiles = (V + kTile - 1) / kTile;             // <= 2048 (V <= 524288)
    // tile sums [ntiles] over sc.v and sc.idx (adjacent, 16 KB together)
    static_assert(offsetof(TruncScratch, idx) == offsetof(TruncScratch, v) + sizeof(float) * kKeptCap &&
                      2 * kKeptCap * sizeof(float) >= kMaxChunks * kChunk / (4 * kWave) * sizeof(unsigned long long),
                  "tile sums do not fit sc.v and sc.idx");
    unsigned long long* tsum = reinterpret_cast<unsigned long long*>(sc.v);
    const float invP = 1.f / tP.S, invQ = 1.f / tQ.S;
    auto weight = [&](int v, bool resid) -> unsigned long long {
        if (v >= V) return 0ull;
        const float z = load_elem<BF16>(prow, v);
        const float p = (finite_logit(z) && z >= tP.tstar) ? __fmul_rn(fast_exp2(__fmul_rn(z - tP.zmax, scale)), invP)
                                                           : 0.f;
        if (!resid) return mass_fixed(p);
        float q;
        if (qrow) {
            const float zq = load_elem<BF16>(qrow, v);
            q = (finite_logit(zq) && zq >= tQ.tstar) ? __fmul_rn(fast_exp2(__fmul_rn(zq - tQ.zmax, scale)), invQ)
                                                     : 0.f;
        } else {
            q = v == dpm ? 1.f : 0.f;
        }
        return mass_fixed(fmaxf(__fsub_rn(p, q), 0.f));
    };
    __shared__ unsigned long long xSeg[kBlock / kWave + 1];
    __shared__ int xTile;
    __shared__ unsigned long long xBase;
    __shared__ int xTok;
    auto tile_sums = [&](bool resid) {
        __syncthreads();
        for (int t0 = wave; t0 < ntiles; t0 += 2 * kWaves) {
            unsigned long long s[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int t = t0 + q * kWaves;
                s[q] = 0;
                if (t < ntiles) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) s[q] += weight(t * kTile + 4 * lane + e, resid);
                }
            }
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int t = t0 + q * kWaves;
                const unsigned long long ts = wave_sum_u64(s[q]);
                if (t < ntiles && lane == 0) tsum[t] = ts;
            }
        }
        __syncthreads();
        unsigned long long part = 0;
        for (int t = tid; t < ntiles; t += kBlock) part += tsum[t];
        return block_sum_u64(part);
    };
    unsigned long long Wf = tile_sums(res);
    *W = (float)((double)Wf * kInvMassUnit);
    const bool fb = res && Wf == 0;
    *fallback = fb;
    if (fb) Wf = tile_sums(false);
    if (Wf == 0) return -1;
    const bool resid = res && !fb;
    // the target: floor(u * W), u = m * 2^-24 (exact in two parts)
    const unsigned long long m = (unsigned long long)(u * 16777216.f);
    const unsigned long long target = (Wf >> 24) * m + (((Wf & 0xffffffull) * m) >> 24);
    // the tile holding the first running sum > target: thread t scans its
    // contiguous run of tiles after a block scan of the runs' sums
    const int per = (ntiles + kBlock - 1) / kBlock;
    const int t0 = tid * per, t1 = min(ntiles, t0 + per);
    unsigned long long run = 0;
    for (int t = t0; t < t1; ++t) run += tsum[t];
    const unsigned long long incl = wave_scan_incl_u64(run);
    if (lane == kWave - 1) xSeg[wave] = incl;
    if (tid == 0) xTile = -1;
    __syncthreads();
    unsigned long long before = incl - run;
    for (int w = 0; w < wave; ++w) before += xSeg[w];
    if (before <= target && target < before + run) {
        unsigned long long acc = before;
        for (int t = t0; t < t1; ++t) {
            if (target < acc + tsum[t]) {
                xTile = t;
                xBase = acc;
                break;
            }
            acc += tsum[t];
        }
    }
    __syncthreads();
    const int tile = xTile;                   // found, as target < W (a miss draws nothing)
    if (tile < 0) {
        if (tid == 0) xTok = -1;
    } else if (wave == 0) {
        unsigned long long e[4], ls = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            e[j] = weight(tile * kTile + 4 * lane + j, resid);
            ls += e[j];
        }
        unsigned long long acc = xBase + wave_scan_incl_u64(ls) - ls;
        int hit = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc += e[j];
            if (hit == 0x7fffffff && e[j] > 0 && acc > target) hit = tile * kTile + 4 * lane + j;
        }
        const unsigned long long any = __ballot(hit != 0x7fffffff);
        if (any) {
            const int first = __ffsll((long long)any) - 1;
            const int tok = __shfl(hit, first, kWave);
            if (lane == 0) xTok = tok;
        } else if (lane == 0) {
            xTok = -1;
        }
    }
    __syncthreads();
    const int tok = xTok;
    __syncthreads();
    return tok;
}

// One wave (lane i holding entry i): the kept set of a row from its
// candidates at or above the top-k threshold, (cw, cx)[0, n) with
// 1 <= n <= 64, with cross-lane operations and no block barriers: rank
// (value desc, index asc) by lane reads, order by ds_permute, DPP scan, cut
// at top-p by ballots.  Publishes the kept list and the row's TruncRow,
// leaves the sorted kept list in (kv, kx)[0, n_kept) and the TruncRow in
// *out (lane 0); when the candidates cannot settle the row (top-p alone,
// short of top_p) it publishes nothing and *out has n_kept == kNeedsExact.  rowM / rowS: the whole row's statistics (for top-p alone);
// flags: flags found so far.
__device__ __forceinline__ void short_merge_wave(const Args& a, long long rowid, const Plan& pl,
                                                 const float* cw, const int* cx, int n, float rowM,
                                                 float rowS, unsigned flags, float* kv, int* kx,
                                                 TruncRow* out) {
    const int lane = threadIdx.x % kWave;
    TruncRow* tr = &a.ws.trow[rowid];
    const bool in = lane < n;
    const float vi = in ? cw[lane] : -kInf;
    const int xi = in ? cx[lane] : 0x7fffffff;
    int r = lane;                                   // lanes past the list keep their place
    if (in) r = 0;
    for (int j = 0; j < n; ++j) {                   // rank: value desc, index asc
        const float vj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vi), j));
        const int xj = __builtin_amdgcn_readlane(xi, j);
        r += (int)(in & ByValue{}(vj, xj, vi, xi));
    }
    const float v = __int_as_float(__builtin_amdgcn_ds_permute(r * 4, __float_as_int(vi)));
    const int x = __builtin_amdgcn_ds_permute(r * 4, xi);
    const float zmax = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
    const float scale = pl.scale;
    const float w = in ? fast_exp2(__fmul_rn(v - zmax, scale)) : 0.f;
    const float cum = wave_scan_incl(w);
    const float last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cum), n - 1));
    // normaliser of the top-k-renormalised softmax: the kept top-k set, or
    // the whole row when top-k is off
    const float Z1 = pl.kmode ? last : rowS * fast_exp2(__fmul_rn(rowM - zmax, scale));
    int jstar = n - 1;
    bool none = false;
    if (pl.top_p < 1.f) {
        // first level end whose cumulative mass reaches top_p
        const float vnext = __shfl(v, lane + 1 < kWave ? lane + 1 : lane, kWave);
        const bool level_end = in && (lane == n - 1 || vnext != v);
        const unsigned long long hit = __ballot(level_end && cum / Z1 >= pl.top_p);
        if (hit) jstar = __ffsll((long long)hit) - 1;
        else none = !pl.kmode;                      // top-p alone: candidates short of top_p
        if (!none) {
            const float tv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), jstar));
            const unsigned long long lvl = __ballot(in && lane <= jstar && v == tv);
            const int ls = __ffsll((long long)lvl) - 1;
            const float cj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cum), jstar)) / Z1;
            const float pv =
                ls > 0 ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cum), ls > 0 ? ls - 1 : 0)) / Z1
                       : 0.f;
            if (fabsf(cj - pl.top_p) < 1e-5f || (ls > 0 && fabsf(pv - pl.top_p) < 1e-5f))
                flags |= SPECV_FLAG_TOPP_NEAR;
        }
    }
    if (none) {
        // top-p alone and the candidates hold less than top_p: nothing is
        // published; the caller takes the exact truncation
        if (lane == 0) {
            TruncRow o{};
            o.zmax = -kInf;
            o.tstar = kInf;
            o.flags = flags;
            o.n_kept = kNeedsExact;
            *out = o;
        }
        return;
    }
    const int nkept = jstar + 1;
    const float tstar = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), jstar));
    const float S = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cum), jstar));
    Cand* kept = a.ws.kept + rowid * a.kept_cap;
    if (lane < nkept) {
        publish_cand(kept + lane, v, x);
        kv[lane] = v;
        kx[lane] = x;
    }
    if (lane == 0) {
        TruncRow o{};
        o.zmax = zmax;
        o.tstar = tstar;
        o.S = S;
        o.n_kept = nkept;
        o.flags = flags;
        o.bad = 0;
        *out = o;
        publish(&tr->zmax, zmax);
        publish(&tr->tstar, tstar);
        publish(&tr->S, S);
        publish(&tr->n_kept, nkept);
        publish(&tr->flags, flags);
        publish(&tr->bad, 0u);
    }
}

// Both rows of pair (b, k), target (side 0) and draft (side 1), merged in
// lockstep: every step of row_merge for the two rows shares the barriers,
// and the one-wave kept-set steps run on waves 0 and 1 at once.  Only the
// usual case is taken (top-k <= 64, no candidate overflow, every list within
// its first S slots, at most kKeptCap / 2 gathered and 64 kept per row);
// otherwise it returns false having published nothing, and the caller merges
// the rows one at a time.  On true, out[0] / out[1] hold the rows'
// TruncRows (as row_merge returns them, a row marked kNeedsExact included)
// for every thread.
template <bool BF16>
__device__ __forceinline__ bool row_merge_pair(const Args& a, int b, int k, const Plan& pl,
                                               TruncScratch& sc, TruncRow* out) {
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    if (pl.keff > kWave || (pl.kmode && pl.top_k > pl.keff)) return false;
    constexpr int kHalf = kKeptCap / 2;
    const long long row0 = side_row(a, b, k, 0), row1 = side_row(a, b, k, 1);
    __shared__ float pL[2], pM[2], pS[2];
    __shared__ int pN[2], pMaxCnt[2], pTotal[2];
    __shared__ unsigned pBad;
    __shared__ unsigned pOff[2][kMaxChunks + 1];
    __shared__ TruncRow pOut[2];
    // slots [0, S) of both rows' chunk lists, read with the lists' lengths
    const int S = min(a.cand_cap, max(64, (3 * pl.keff / 2 + 15) & ~15));
    const int nspec = a.C * S;
    const float invS = 1.f / (float)S;
    auto slot_chunk = [&](int p) {          // p / S, exact for p < 2^24
        int c = (int)((float)p * invS);
        c -= c * S > p;
        c += (c + 1) * S <= p;
        return c;
    };
    auto spec_load = [&](int p) {           // p over both rows: side p / nspec
        const int side = p >= nspec ? 1 : 0;
        const int ps = p - side * nspec;
        const int c = slot_chunk(ps);
        const Cand* base = a.ws.cand + cand_base(a, side ? row1 : row0, c);
        return p < 2 * nspec ? published_cand(base + (ps - c * S)) : Cand{-kInf, 0};
    };
    constexpr int NQ = 12;                  // slots per thread a round
    Cand cv[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) cv[q] = spec_load(q * kBlock + tid);
    if (tid == 0) {                         // (one call per workgroup)
        pBad = 0;
        pN[0] = pN[1] = 0;
    }
    // the top-k select's histograms (in idx2: row r, digit d at (r * NP + d)
    // * 256), cleared here: the first digit is counted by the gather
    constexpr int NP = BF16 ? 2 : 4;
    constexpr int KB = 8 * NP;
    unsigned* h = reinterpret_cast<unsigned*>(sc.idx2);
#pragma unroll
    for (int d = 0; d < 2 * NP; ++d) h[d * 256 + tid] = 0;
    __syncthreads();
    // lengths and bounds (waves 0, 2) and row statistics (waves 1, 3)
    {
        const int side = wave >> 1;
        const long long rowid = side ? row1 : row0;
        if ((wave & 1) == 0) {
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
            if (lane < a.C) pOff[side][lane] = (unsigned)(incl - cnt);
            if (lane == a.C - 1) {
                pOff[side][a.C] = (unsigned)incl;
                pTotal[side] = incl;
            }
            const int mc = wave_max_int(cnt);
            const unsigned long long any_ovf = __ballot(ovf);
            if (lane == 0) {
                pL[side] = L;
                pMaxCnt[side] = mc;
                if (any_ovf) atomicOr(&pBad, 1u);
            }
        } else {
            float m = -kInf, sm = 0.f;
            if (lane < a.C) {
                unsigned sw = 0;
                (void)published_stats(stats_words(a, b, k, side, lane), a.epoch, m, sw);
                sm = __uint_as_float(sw);
            }
            wave_merge_ms(m, sm, pl.scale);
            if (lane == 0) {
                pM[side] = m;
                pS[side] = sm;
                if (__builtin_isnan(sm) || m == -kInf) atomicOr(&pBad, 1u);
            }
        }
    }
    __syncthreads();
    if (pBad || pMaxCnt[0] > S || pMaxCnt[1] > S) return false;
    // gather both rows' candidates >= their max L into the halves of (v, idx):
    // the round's kept slots are marked first, then each wave reserves its
    // share of each half with one LDS atomic (the order within a half is
    // immaterial: every later step orders by value, then index)
    const float Lr[2] = {pL[0], pL[1]};
    for (int p0 = 0;;) {
        unsigned km[2] = {0u, 0u};
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int p = p0 + q * kBlock + tid;
            const int side = p >= nspec ? 1 : 0;
            const int ps = p - side * nspec;
            const int c = min(slot_chunk(ps), a.C - 1);
            const bool listed = p < 2 * nspec && ps - c * S < (int)(pOff[side][c + 1] - pOff[side][c]);
            const bool keep = listed && cv[q].v >= Lr[side] && finite_logit(cv[q].v);
            if (keep) km[side] |= 1u << q;
        }
        int o[2];
#pragma unroll
        for (int side = 0; side < 2; ++side) {
            const int cnt = __popc(km[side]);
            const int incl = wave_scan_incl(cnt);
            int base = 0;
            if (lane == kWave - 1 && incl > 0) base = atomicAdd(&pN[side], incl);
            o[side] = __shfl(base, kWave - 1, kWave) + incl - cnt;
        }
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
#pragma unroll
            for (int side = 0; side < 2; ++side) {
                if ((km[side] >> q) & 1u) {
                    if (o[side] < kHalf) {
                        sc.v[side * kHalf + o[side]] = cv[q].v;
                        sc.idx[side * kHalf + o[side]] = cv[q].idx;
                    }
                    atomicAdd(&h[side * NP * 256 + ((order_key<BF16>(cv[q].v) >> (KB - 8)) & 255u)], 1u);
                    ++o[side];
                }
            }
        }
        p0 += NQ * kBlock;
        if (p0 >= 2 * nspec) break;
#pragma unroll
        for (int q = 0; q < NQ; ++q) cv[q] = spec_load(p0 + q * kBlock + tid);
    }
    __syncthreads();
    const int n[2] = {pN[0], pN[1]};
    if (n[0] == 0 || n[1] == 0 || n[0] > kHalf || n[1] > kHalf) return false;
    // the top-k threshold of each row: radix select over 8-bit digits, both
    // rows per pass (the first digit's counts come from the gather)
    __shared__ unsigned pSel[2];
    __shared__ int pRest[2], pFound[2];
    unsigned prefix[2] = {0u, 0u};
    int need[2] = {min(pl.keff, n[0]), min(pl.keff, n[1])};
#pragma unroll
    for (int pass = 0; pass < NP; ++pass) {
        const int shift = KB - 8 * (pass + 1);
        if (pass > 0) {
#pragma unroll
            for (int side = 0; side < 2; ++side) {
                unsigned* hp = h + (side * NP + pass) * 256;
                for (int i = tid; i < n[side]; i += kBlock) {
                    const unsigned key = order_key<BF16>(sc.v[side * kHalf + i]);
                    if ((key >> (shift + 8)) == prefix[side]) atomicAdd(&hp[(key >> shift) & 255u], 1u);
                }
            }
            __syncthreads();
        }
        if (wave < 2)
            wave_find_bin(h + (wave * NP + pass) * 256, wave ? need[1] : need[0], &pSel[wave], &pRest[wave],
                          &pFound[wave]);
        __syncthreads();
        // read before waves 0 / 1 update them (after the next pass's barrier)
#pragma unroll
        for (int side = 0; side < 2; ++side) {
            prefix[side] = (prefix[side] << 8) | pSel[side];
            need[side] = pRest[side];
        }
    }
    const float tk[2] = {value_of_key<BF16>(prefix[0]), value_of_key<BF16>(prefix[1])};
    // the entries at or above each threshold, into the halves of (w, idx2);
    // both counts scanned at once (row 1's in the high 16 bits)
    int cnt = 0;
#pragma unroll
    for (int side = 0; side < 2; ++side)
        for (int i = tid; i < n[side]; i += kBlock) cnt += (sc.v[side * kHalf + i] >= tk[side]) << (16 * side);
    int tot;
    const int o = block_excl_scan(cnt, sc.misc, &tot);
    const int nk[2] = {tot & 0xffff, tot >> 16};
    if (nk[0] > kWave || nk[1] > kWave) return false;
    int oo[2] = {o & 0xffff, o >> 16};
#pragma unroll
    for (int side = 0; side < 2; ++side) {
        for (int i = tid; i < n[side]; i += kBlock) {
            const float x = sc.v[side * kHalf + i];
            if (x >= tk[side]) {
                sc.w[side * kHalf + oo[side]] = x;
                sc.idx2[side * kHalf + oo[side]] = sc.idx[side * kHalf + i];
                ++oo[side];
            }
        }
    }
    __syncthreads();
    if (wave < 2)
        short_merge_wave(a, wave ? row1 : row0, pl, sc.w + wave * kHalf, sc.idx2 + wave * kHalf, wave ? nk[1] : nk[0],
                         pM[wave], pS[wave], 0u, sc.v + wave * kHalf, sc.idx + wave * kHalf, &pOut[wave]);
    __syncthreads();
    if (tid == 0) {
        // top-p alone short of top_p among a row's candidates: that row is
        // marked for the exact truncation, with its maximum
#pragma unroll
        for (int side = 0; side < 2; ++side)
            if (pOut[side].n_kept == kNeedsExact) pOut[side].zmax = pM[side];
    }
    __syncthreads();
    out[0] = pOut[0];
    out[1] = pOut[1];
    __syncthreads();
    return true;
}

// Row-level truncation (whole workgroup) of logits row (b, k, side), once
// every chunk's candidates are published.  Publishes the kept list and the
// row's TruncRow, and returns the TruncRow to every thread; when the row
// keeps n_kept > 0 entries, sc.v / sc.idx [0, n_kept) also hold the kept
// list (value descending, index ascending) on return.  A row the candidates
// cannot settle is returned unpublished with n_kept == kNeedsExact, its
// maximum in zmax and its flags so far: row_settle finishes it.
template <bool BF16>
__device__ __forceinline__ TruncRow row_merge(const Args& a, int b, int k, int side, const Plan& pl,
                              TruncScratch& sc) {
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const long long rowid = side_row(a, b, k, side);
    __shared__ float sL, sM, sS, sZ1;
    __shared__ unsigned sBad, sFlags, sExact;
    __shared__ int sTotal, sN, sJ, sLevelStart, sMaxCnt;
    __shared__ TruncRow sOut;
    unsigned* off = sc.off;                // chunk offsets [0, C]
    // slots [0, S) of every chunk's list are read before the lists' lengths
    // are known, in the same memory round trip (S about 1.5 keff, which
    // covers the usual list of a little over keff; longer lists are finished
    // afterwards); slot p is (chunk p / S, entry p % S)
    const int S = min(a.cand_cap, max(64, (3 * pl.keff / 2 + 15) & ~15));
    const int nspec = a.C * S;
    const float invS = 1.f / (float)S;
    const Cand* cbase = a.ws.cand + cand_base(a, rowid, 0);
    auto slot_chunk = [&](int p) {          // p / S, exact for p < 2^24
        int c = (int)((float)p * invS);
        c -= c * S > p;
        c += (c + 1) * S <= p;
        return c;
    };
    auto spec_load = [&](int p) {
        const int c = slot_chunk(p);
        return p < nspec ? published_cand(cbase + (long long)c * a.cand_cap + (p - c * S)) : Cand{-kInf, 0};
    };
    Cand cv[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) cv[q] = spec_load(q * kBlock + tid);
    __syncthreads();                       // shared state may still be read
    if (tid == 0) {
        sBad = 0;
        sFlags = 0;
        sExact = 0;
        sN = 0;
        sJ = 0x7fffffff;
        sLevelStart = 0x7fffffff;
        sOut.zmax = -kInf;
        sOut.tstar = kInf;
        sOut.S = 0.f;
        sOut.n_kept = 0;
        sOut.flags = 0;
        sOut.bad = 0;
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
        const int mc = wave_max_int(cnt);
        if (lane == 0) sMaxCnt = mc;
        const unsigned long long any_ovf = __ballot(ovf);
        if (lane == 0) {
            sL = L;
            if (any_ovf) sExact = 1;           // a chunk's list overflowed: heavy ties
        }
    } else if (wave == 1) {
        float m = -kInf, s = 0.f;
        if (lane < a.C) {
            unsigned sw = 0;
            (void)published_stats(stats_words(a, b, k, side, lane), a.epoch, m, sw);
            s = __uint_as_float(sw);
        }
        wave_merge_ms(m, s, pl.scale);
        if (lane == 0) {
            sM = m;
            sS = s;
            if (__builtin_isnan(s) || m == -kInf) sBad = 1;
        }
    }
    __syncthreads();
    TruncRow* tr = &a.ws.trow[rowid];
    auto publish_bad = [&]() {
        if (tid == 0) {
            sOut.bad = 1;
            sOut.n_kept = 0;
            publish(&tr->bad, 1u);
            publish(&tr->flags, 0u);
            publish(&tr->n_kept, 0);
        }
        __syncthreads();
        return sOut;
    };
    // a row the candidate lists cannot settle: nothing published; the
    // caller takes the exact truncation (row_settle)
    auto needs_exact = [&](float zmax, unsigned flags) {
        TruncRow o{};
        o.zmax = zmax;
        o.tstar = kInf;
        o.flags = flags;
        o.n_kept = kNeedsExact;
        return o;
    };
    if (sBad) return publish_bad();
    // top_k beyond the candidates, or a list that overflowed: exactly
    if ((pl.kmode && pl.top_k > pl.keff) || sExact) return needs_exact(sM, 0u);
    // gather the candidates >= max L into LDS
    const float L = sL;
    const int total = sTotal;
    auto take = [&](const Cand& x, bool listed, unsigned min_key) {
        const bool keep = listed && x.v >= L && finite_logit(x.v) && order_key<BF16>(x.v) >= min_key;
        const int pos = wave_reserve(keep, &sN);
        if (pos >= 0 && pos < kKeptCap) {
            sc.v[pos] = x.v;
            sc.idx[pos] = x.idx;
        }
    };
    for (int p0 = 0;;) {                   // the speculative slots, 8 per thread a round
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int p = p0 + q * kBlock + tid;
            const int c = min(slot_chunk(p), a.C - 1);
            take(cv[q], p < nspec && p - c * S < (int)(off[c + 1] - off[c]), 0u);
        }
        p0 += 8 * kBlock;
        if (p0 >= nspec) break;
#pragma unroll
        for (int q = 0; q < 8; ++q) cv[q] = spec_load(p0 + q * kBlock + tid);
    }
    // all of a row's candidates from slot ``from`` of each list on
    auto gather = [&](unsigned min_key, int from) {
        for (int f0 = 0; f0 < total; f0 += 4 * kBlock) {
            Cand cw[4];
            bool in[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int f = f0 + q * kBlock + tid;
                in[q] = false;
                cw[q] = Cand{-kInf, 0};
                if (f < total) {
                    int lo = 0, hi = a.C - 1;  // chunk c with off[c] <= f < off[c + 1]
                    while (lo < hi) {
                        const int mid = (lo + hi + 1) >> 1;
                        if ((int)off[mid] <= f) lo = mid;
                        else hi = mid - 1;
                    }
                    if (f - (int)off[lo] >= from) {
                        in[q] = true;
                        cw[q] = published_cand(a.ws.cand + cand_base(a, rowid, lo) + (f - (int)off[lo]));
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) take(cw[q], in[q], min_key);
        }
        __syncthreads();
    };
    if (sMaxCnt > S) gather(0u, S);        // lists longer than the slots read
    else __syncthreads();
    if (sN > kKeptCap) {
        // too many candidates above the chunk bounds: select the exact top-k
        // key over them in global memory, then keep only entries >= it
        const int K = min(pl.keff, sN);
        const unsigned kkey = select_kth_key<BF16>(a, rowid, total, L, K, sc);
        if (tid == 0) sN = 0;
        __syncthreads();
        gather(kkey, 0);
    }
    const int n1 = sN;
    // more candidates above the top-k key than LDS holds (ties): exactly
    if (n1 > kKeptCap) return needs_exact(sM, 0u);
    if (n1 == 0) return publish_bad();
    // top-k: the K-th largest value (with multiplicity) ends the kept set,
    // and every entry equal to it is kept; those entries are moved to
    // (w, idx2), then sorted into (v, idx): value desc, index asc
    const int K = min(pl.keff, n1);
    const float tk = K < n1 ? value_of_key<BF16>(lds_select_kth<BF16>(sc.v, n1, K, sc)) : -kInf;
    int cnt = 0;
    for (int i = tid; i < n1; i += kBlock) cnt += sc.v[i] >= tk;
    int nk1;
    int o = block_excl_scan(cnt, sc.misc, &nk1);
    for (int i = tid; i < n1; i += kBlock) {
        if (sc.v[i] >= tk) {
            sc.w[o] = sc.v[i];
            sc.idx2[o] = sc.idx[i];
            ++o;
        }
    }
    __syncthreads();
    if (nk1 <= kWave) {
        // the usual short list (top-k of a few dozen): one wave
        if (wave == 0) short_merge_wave(a, rowid, pl, sc.w, sc.idx2, nk1, sM, sS, sFlags, sc.v, sc.idx, &sOut);
        __syncthreads();
        if (sOut.n_kept == kNeedsExact) return needs_exact(sM, sOut.flags);
        return sOut;
    }
    rank_sort(sc.w, sc.idx2, nk1, sc.v, sc.idx, ByValue{}, reinterpret_cast<int*>(sc.hist));
    const float zmax = sc.v[0];
    const float scale = pl.scale;
    for (int i = tid; i < nk1; i += kBlock) sc.w[i] = fast_exp2(__fmul_rn(sc.v[i] - zmax, scale));
    __syncthreads();
    block_inclusive_scan(sc.w, sc.w, nk1, sc.red);
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
            // top-p alone: the candidates hold less than top_p of the mass
            if (!pl.kmode) return needs_exact(sM, sFlags);
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
    wait_stores();                         // every wave's entries out before the decision
    __syncthreads();
    if (tid == 0) {
        sOut.zmax = zmax;
        sOut.tstar = sc.v[jstar];
        sOut.S = sc.w[jstar];
        sOut.n_kept = nkept;
        sOut.flags = sFlags;
        sOut.bad = 0;
        publish(&tr->zmax, zmax);
        publish(&tr->tstar, sc.v[jstar]);
        publish(&tr->S, sc.w[jstar]);
        publish(&tr->n_kept, nkept);
        publish(&tr->flags, sFlags);
        publish(&tr->bad, 0u);
    }
    __syncthreads();
    return sOut;
}

// A row that row_merge / row_merge_pair marked kNeedsExact gets the exact
// whole-row truncation (published, returned to every thread); any other row
// is returned as it is.  Each kernel calls this from one place, so that the
// slow path is inlined once.
template <bool BF16>
__device__ __forceinline__ TruncRow row_settle(const Args& a, int b, int k, int side, const Plan& pl,
                                               const TruncRow& t, TruncScratch& sc) {
    if (t.n_kept != kNeedsExact) return t;
    return row_truncate_exact<BF16>(a, b, k, side, pl, t.zmax, t.flags, sc);
}

__device__ inline bool trow_dead(const TruncRow& t) {
    return t.bad != 0 || t.n_kept == 0;
}

// Probability of raw logit z under a truncated row: membership in the kept
// set is decided on the raw value (z >= tstar).
__device__ inline float trunc_prob(const TruncRow& t, float z, float scale) {
    if (!(finite_logit(z) && z >= t.tstar)) return 0.f;
    return fast_exp2(__fmul_rn(z - t.zmax, scale)) / t.S;
}

// A draft row's truncation from the drafter's statistics (specv_draft_stats):
// kept set {z >= threshold}, max, and the kept set's sum (threshold form);
// flags as the drafter found them.  A row the drafter marked non-finite, or
// whose statistics are not valid, is bad.
__device__ inline TruncRow stats_trow(const specv_draft_stats& st) {
    TruncRow t{};
    const unsigned fl = (unsigned)st.flags;
    t.zmax = st.max;
    t.tstar = st.threshold;
    t.S = st.sum;
    t.flags = fl & SPECV_FLAG_TOPP_NEAR;
    const bool valid = st.sum > 0.f && finite_logit(st.max) && !__builtin_isnan(st.threshold);
    t.bad = (fl & SPECV_FLAG_NONFINITE_ROW) || !valid ? 1u : 0u;
    t.n_kept = t.bad ? 0 : kThresholdForm;
    return t;
}

__device__ inline TruncRow published_trow(const TruncRow* p) {
    TruncRow t;
    t.zmax = published(&p->zmax);
    t.tstar = published(&p->tstar);
    t.S = published(&p->S);
    t.n_kept = published(&p->n_kept);
    t.flags = published(&p->flags);
    t.bad = published(&p->bad);
    return t;
}

// Correction / bonus sample of a truncated row (whole workgroup) at position
// pos: weights over the kept set of p_pos (zero weight elsewhere), tokens in
// ascending index order, first running sum > u * W.  Returns the token (-1 if
// no weight anywhere) to every thread; *wres gets W of a correction, and
// *fallback is set when the correction mass vanished and p was used.
template <bool BF16, int PROP>
__device__ int trunc_sample(const Args& a, int b, int pos, bool res, float u, const Plan& pl,
                            TruncScratch& sc, float* wres, bool* fallback) {
    const int tid = threadIdx.x;
    __shared__ TruncRow tT, tQ;
    __shared__ float sWsum;
    __shared__ int sTok, sLastPos, sFb;
    const float scale = pl.scale;
    constexpr bool pm = PROP == kPropPoint;  // q = the point mass on d_pos
    __syncthreads();
    if (tid == 0) {
        tT = published_trow(&a.ws.trow[side_row(a, b, pos, 0)]);
        if (res && !pm)
            tQ = PROP == kPropStats ? stats_trow(a.qstats[(long long)b * a.qs_sb + pos])
                                    : published_trow(&a.ws.trow[side_row(a, b, pos, 1)]);
        sTok = 0x7fffffff;
        sLastPos = -1;
        sFb = 0;
    }
    __syncthreads();
    const int n = tT.n_kept;
    const int dpm = res && pm ? draft_token(a, b, pos) : -1;
    const void* qrow = res && !pm ? row_ptr<BF16>(a.drf, a.d_sb, a.d_sp, b, pos) : nullptr;
    if (n == kThresholdForm) {
        // kept set {z >= tstar} without a list: a scan of the row
        const TruncRow t = tT, q = tQ;
        float W;
        const int tok = threshold_draw<BF16>(row_ptr<BF16>(a.tgt, a.t_sb, a.t_sp, b, pos), t, qrow, q, dpm, res, a.V,
                                             scale, u, sc, &W, fallback);
        *wres = res ? W : 0.f;
        return tok;
    }
    if (n <= 0) return -1;                  // (a dead row is never sampled)
    const Cand* kept = a.ws.kept + side_row(a, b, pos, 0) * a.kept_cap;
    if (n <= kWave) {
        // a short kept list: one wave weighs, orders by token, scans and
        // picks, lane i holding entry i
        if (tid < kWave) {
            const int lane = tid;
            const bool in = lane < n;
            float p = 0.f, w = 0.f;
            int x = 0x7fffffff;
            if (in) {
                const Cand cv = published_cand(kept + lane);
                x = cv.idx;
                p = __fmul_rn(fast_exp2(__fmul_rn(cv.v - tT.zmax, scale)), 1.f / tT.S);
                w = p;
                if (res) {
                    float q;
                    if (pm) {
                        q = cv.idx == dpm ? 1.f : 0.f;
                    } else {
                        const float zq = load_elem<BF16>(qrow, cv.idx);
                        q = (finite_logit(zq) && zq >= tQ.tstar)
                                ? __fmul_rn(fast_exp2(__fmul_rn(zq - tQ.zmax, scale)), 1.f / tQ.S)
                                : 0.f;
                    }
                    w = fmaxf(__fsub_rn(p, q), 0.f);
                }
            }
            const float W = wave_sum(w);
            const bool fb = res && (!(W > 0.f) || !__builtin_isfinite(W));
            if (fb) w = p;                          // the correction mass vanished: p
            int r = lane;                           // lanes past the list keep their place
            if (in) r = 0;
            for (int j = 0; j < n; ++j) r += (int)(in & (__builtin_amdgcn_readlane(x, j) < x));
            const float ws = __int_as_float(__builtin_amdgcn_ds_permute(r * 4, __float_as_int(w)));
            const int xs = __builtin_amdgcn_ds_permute(r * 4, x);
            const float cum = wave_scan_incl(ws);
            const float target = u * __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cum), n - 1));
            const unsigned long long pos = __ballot(lane < n && ws > 0.f);
            const unsigned long long hit = __ballot(lane < n && ws > 0.f && cum > target);
            // the first running sum > u W; clamp: the last positive weight
            const int j = hit ? __ffsll((long long)hit) - 1 : (pos ? 63 - __clzll(pos) : -1);
            const int tok = j >= 0 ? __builtin_amdgcn_readlane(xs, j) : -1;
            if (lane == 0) {
                sTok = tok;
                sWsum = W;
                sFb = fb ? 1 : 0;
            }
        }
        __syncthreads();
        *wres = res ? sWsum : 0.f;
        *fallback = sFb != 0;
        const int tok = sTok;
        __syncthreads();
        return tok;
    }
    // sc.v = weight, sc.idx = token, sc.w = p (fallback weight)
    float part = 0.f;
    for (int i = tid; i < n; i += kBlock) {
        const Cand cv = published_cand(kept + i);
        const float p = __fmul_rn(fast_exp2(__fmul_rn(cv.v - tT.zmax, scale)), 1.f / tT.S);
        float w = p;
        if (res) {
            float q;
            if (pm) {
                q = cv.idx == dpm ? 1.f : 0.f;
            } else {
                const float zq = load_elem<BF16>(qrow, cv.idx);
                q = (finite_logit(zq) && zq >= tQ.tstar)
                        ? __fmul_rn(fast_exp2(__fmul_rn(zq - tQ.zmax, scale)), 1.f / tQ.S)
                        : 0.f;
            }
            w = fmaxf(__fsub_rn(p, q), 0.f);
        }
        sc.v[i] = w;
        sc.w[i] = p;
        sc.idx[i] = cv.idx;
        part += w;
    }
    part = wave_sum(part);
    if (tid % kWave == 0) sc.red[tid / kWave] = part;
    __syncthreads();
    if (tid == 0) {
        float W = 0.f;
        for (int w2 = 0; w2 < kWaves; ++w2) W += sc.red[w2];
        sWsum = W;
        sFb = res && (!(W > 0.f) || !__builtin_isfinite(W));
    }
    __syncthreads();
    *wres = res ? sWsum : 0.f;
    *fallback = sFb != 0;
    if (sFb) {
        // the correction mass vanished: sample from p at that position
        for (int i = tid; i < n; i += kBlock) sc.v[i] = sc.w[i];
    }
    __syncthreads();
    // weights in ascending token order into (w, idx2), running sums into v,
    // then the first running sum > u * W
    rank_sort(sc.v, sc.idx, n, sc.w, sc.idx2, ByIndex{}, reinterpret_cast<int*>(sc.hist));
    block_inclusive_scan(sc.w, sc.v, n, sc.red);
    const float target = u * sc.v[n - 1];
    for (int i = tid; i < n; i += kBlock) {
        if (sc.w[i] > 0.f) {
            if (sc.v[i] > target) atomicMin(&sTok, i);
            atomicMax(&sLastPos, i);
        }
    }
    __syncthreads();
    const int j = sTok != 0x7fffffff ? sTok : sLastPos;     // clamp: last positive weight
    const int tok = j >= 0 ? sc.idx2[j] : -1;
    __syncthreads();
    return tok;
}

}  // namespace
}  // namespace specv
