// libspecv draft-side sampler for gfx950: d_i ~ q_i in one pass over the
// draft logits, plus the row statistics the verifier can reuse.
//
// q_i is the draft model's distribution after its temperature, top-k and
// top-p ("11.1 核心原理" 11.1.2: the proposal is the distribution actually
// sampled; the tutorial's section 3.3 divides the logits by the
// temperature).  The draw is the inverse CDF of q_i at a Philox uniform of
// purpose 0 (DRAFT): tokens in ascending index order, the first whose
// running mass exceeds u * W.
//
// Workgroup (i, b, c), position-major, one per 8192-entry chunk of draft row
// (b, i):
//   1. reads its chunk once (16-byte loads) and reduces it to (max, sum of
//      exp2((z - max) * log2(e) / T)), or (max, lowest argmax) for greedy
//      rows, published as two tagged words; truncated rows also keep
//      their top-k candidates (published before the words);
//   2. untruncated rows: wave 0 reads every chunk's words of the row (lane
//      c: chunk c), merges them into the row's (m, s), and turns them into
//      chunk masses s_c * exp2((m_c - m) * scale) whose prefix sums locate
//      the chunk holding u * W; every workgroup of the row computes the same
//      thing;
//   3. the workgroup owning that chunk finds the token in its registers and
//      writes the token and the row's statistics.  Its in-chunk running sums
//      (in the chunk's own exp2 units) are computed by every workgroup while
//      the statistics are in flight, so that after the hand-off the owner
//      only compares the target with its groups' ranges;
//   2'. truncated rows: chunk 0's workgroup waits for every chunk, merges the
//      candidates into the row's kept list (the verify kernel's row merge:
//      top-k threshold, then top-p) and draws from the kept list.
// One hand-off per row, and the row is read once.  The chunk statistics, the
// row merge and their order are the verify kernel's, so the statistics
// written here equal what the verify step computes from the same row.
//
// Waits: a row's C workgroups have consecutive IDs and each waits only for
// its own row.  Workgroups are dispatched in increasing ID order within each
// XCD, and an XCD holds far more than C of them, so the lowest row with a
// waiting workgroup always has all its workgroups dispatched.  The wait is
// bounded; expiry flags the entry INTERNAL.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "specv_device.hpp"
#include "specv_internal.hpp"
#include "specv_rows.hpp"

namespace specv {
namespace {

__device__ inline void write_draft(const DraftArgs& a, long long o, int tok, float m, float s,
                                   float thr, unsigned flags) {
    a.out_tok[o] = tok;
    if (a.out_stats) {
        specv_draft_stats st;
        st.max = m;
        st.sum = s;
        st.threshold = thr;
        st.flags = (int)flags;
        a.out_stats[o] = st;
    }
}

// The verify kernel's argument view of a sampler call, for the shared
// workspace indexing and truncation steps: draft row (b, i) is side 1 of
// pair (b, i), with n positions per batch row.
__device__ inline Args verify_view(const DraftArgs& a) {
    Args v{};
    v.drf = a.drf;
    v.d_sb = a.d_sb;
    v.d_sp = a.d_sp;
    v.B = a.B;
    v.V = a.V;
    v.C = a.C;
    v.P = a.n;
    v.cand_cap = a.cand_cap;
    v.kept_cap = a.kept_cap;
    v.max_top_k = a.max_top_k;
    v.epoch = a.epoch;
    v.ws = a.ws;
    return v;
}

// Truncated draft row (b, i) after every chunk published its candidates and
// statistics (chunk 0's workgroup, whole workgroup): the kept list by the
// verify kernel's row merge, then the inverse CDF over the kept tokens in
// ascending index order.
template <bool BF16>
__device__ __forceinline__ void draw_truncated(const DraftArgs& a, const Args& va, int b, int i, long long o,
                               const Plan& pl, float u, TruncScratch& sc) {
    const int tid = threadIdx.x;
    const float nan = __builtin_nanf("");
    const TruncRow tr = row_settle<BF16>(va, b, i, 1, pl, row_merge<BF16>(va, b, i, 1, pl, sc), sc);
    if (tr.bad || tr.n_kept == 0) {
        if (tid == 0) write_draft(a, o, -1, nan, nan, nan, tr.flags | SPECV_FLAG_NONFINITE_ROW);
        return;
    }
    if (tr.n_kept == kThresholdForm) {
        // kept set {z >= tstar} without a list: a scan of the row
        float W;
        bool fb;
        const int tok = threshold_draw<BF16>(row_ptr<BF16>(a.drf, a.d_sb, a.d_sp, b, i), tr, nullptr, tr, -1, false,
                                             a.V, pl.scale, u, sc, &W, &fb);
        if (tid == 0) {
            if (tok < 0) write_draft(a, o, -1, nan, nan, nan, tr.flags | SPECV_FLAG_NONFINITE_ROW);
            else write_draft(a, o, tok, tr.zmax, tr.S, tr.tstar, tr.flags);
        }
        return;
    }
    // row_merge leaves the kept list in sc.v / sc.idx (value descending)
    __shared__ int sTok, sLast;
    const int n = tr.n_kept;
    for (int j = tid; j < n; j += kBlock) sc.w[j] = fast_exp2(__fmul_rn(sc.v[j] - tr.zmax, pl.scale));
    if (tid == 0) {
        sTok = 0x7fffffff;
        sLast = -1;
    }
    __syncthreads();
    rank_sort(sc.w, sc.idx, n, sc.v, sc.idx2, ByIndex{}, reinterpret_cast<int*>(sc.hist));   // weights in token order
    block_inclusive_scan(sc.v, sc.w, n, sc.red);            // running sums
    const float target = u * sc.w[n - 1];
    for (int j = tid; j < n; j += kBlock) {
        if (sc.v[j] > 0.f) {
            if (sc.w[j] > target) atomicMin(&sTok, j);
            atomicMax(&sLast, j);
        }
    }
    __syncthreads();
    if (tid == 0) {
        const int j = sTok != 0x7fffffff ? sTok : sLast;     // rounding: last with weight
        if (j < 0) write_draft(a, o, -1, nan, nan, nan, tr.flags | SPECV_FLAG_NONFINITE_ROW);
        else write_draft(a, o, sc.idx2[j], tr.zmax, tr.S, tr.tstar, tr.flags);
    }
}

template <bool BF16, bool VEC, bool TRUNC, bool DEVCALL>
__device__ __forceinline__ void sample_draft_block(const DraftArgs& a0, TruncScratch* sc) {
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int per = a0.B * a0.C;
    const int work = a0.n * per;
    if constexpr (DEVCALL) {
        if ((int)blockIdx.x == work) {
            // the closing workgroup (as in the verify kernel)
            close_call(a0.ws, a0.B, (unsigned)(a0.n * a0.C), pack_dims(a0.B, a0.n, a0.C));
            return;
        }
    }
    const int i = blockIdx.x / per;
    const int rem = blockIdx.x - i * per;
    const int b = rem / a0.C;
    const int c = rem - b * a0.C;
    // the call number (tag and record set, as in the verify kernel); with
    // the device's, every workgroup clears its share of the other parity's
    // set and counts itself once nothing it waits for comes after the count
    // (vector memory operations retire in order)
    const unsigned e = DEVCALL ? read_call(a0.ws) : a0.epoch;
    DraftArgs a = a0;
    a.epoch = DEVCALL ? call_tag(e) : e;
    a.ws = parity_set<DEVCALL>(a0.ws, e & 1u);
    const Args va = verify_view(a);
    const float nan = __builtin_nanf("");
    // the chunk's loads go out first: the row's parameters, read next, share
    // their round trip
    const void* row = row_ptr<BF16>(a.drf, a.d_sb, a.d_sp, b, i);
    const int v0 = c * kChunk;
    const int len = min(kChunk, a.V - v0);
    ChunkRegs<BF16, VEC> r;
    r.issue(row, v0, len);
    const specv_row_params rp = a.params[b];
    const bool greedy = !(rp.temperature > 0.f);
    const bool topk_on = rp.top_k > 0 && rp.top_k < a.V;
    const bool trunc = !greedy && (topk_on || rp.top_p < 1.f);
    const int pos = a.pos0 + i;
    const long long o = (long long)b * a.out_stride + pos;
    if (trunc && (!TRUNC || a.cand_cap == 0)) {
        // the handle reserved no room for candidates
        if (c == 0 && tid == 0) write_draft(a, o, -1, nan, nan, nan, SPECV_FLAG_UNSUPPORTED);
        if constexpr (DEVCALL) {
            clear_other_set(a0.ws, e, blockIdx.x, work);
            if (tid == 0) count_call(a0.ws, e, b);
        }
        return;
    }
    const float scale = greedy ? 0.f : kLog2e / rp.temperature;
    r.finish(row, v0, len);

    // 1. chunk statistics, merged across the four waves as the verify's
    //    streaming units merge them (side 1 of pair (b, i) of the workspace);
    //    sampled rows also keep each thread's group sums (G-entry groups) in
    //    the thread's own units, for the running sums of step 2
    constexpr int G = BF16 ? 8 : 4;
    constexpr int NG = kPerThread / G;
    float gwt[NG], tmax = -kInf;            // (sampled rows without truncation)
    __shared__ float sm[kWaves], ss[kWaves];
    __shared__ int si[kWaves];
    __shared__ unsigned sb[kWaves];
    if (greedy) {
        float best;
        int bi;
        unsigned bad;
        wave_chunk_argmax<BF16>(r, v0, best, bi, bad);
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
            publish_stats(stats_words(va, b, i, 1, c), bad ? nan : best, (unsigned)bi, a.epoch);
        }
    } else {
        float m, s;
        if (TRUNC && trunc) wave_chunk_ms(r, scale, m, s);       // (no step 2)
        else wave_chunk_ms_groups(r, scale, m, s, gwt, tmax);
        if (lane == 0) {
            sm[wave] = m;
            ss[wave] = s;
        }
        if constexpr (TRUNC) {
            if (trunc) {
                // the chunk's top-k candidates, complete before its statistics
                // are published (the statistics words tell the merge they are in)
                chunk_candidates<BF16>(va, side_row(va, b, i, 1), c, topk_on ? min(rp.top_k, a.max_top_k) : a.max_top_k, r,
                                       *sc);
                wait_stores();
            }
        }
        __syncthreads();
        if (tid == 0) {
            m = sm[0];
            s = ss[0];
            for (int w = 1; w < kWaves; ++w) merge_ms(m, s, sm[w], ss[w], scale);
            publish_stats(stats_words(va, b, i, 1, c), m, __float_as_uint(s), a.epoch);
        }
    }
    if constexpr (DEVCALL) {
        // behind the statistics: this workgroup's share of the clearing, and its count
        clear_other_set(a0.ws, e, blockIdx.x, work);
        if (tid == 0) count_call(a0.ws, e, b);
    }
    if constexpr (TRUNC) {
        if (trunc) {
            // 2'. chunk 0's workgroup merges the row and draws
            if (c != 0) return;
            __shared__ int sLate;
            if (wave == 0) {
                float m = -kInf;
                unsigned second = 0;
                bool ok = true;
                if (lane < a.C) ok = published_stats(stats_words(va, b, i, 1, lane), a.epoch, m, second);
                const bool late = __ballot(!ok) != 0;
                if (lane == 0) sLate = late;
            }
            __syncthreads();
            if (sLate) {
                if (tid == 0) write_draft(a, o, -1, nan, nan, nan, SPECV_FLAG_INTERNAL);
                return;
            }
            Plan pl{};
            pl.mode = MODE_TRUNC;
            pl.scale = scale;
            pl.top_k = rp.top_k;
            pl.top_p = rp.top_p;
            pl.kmode = topk_on ? 1 : 0;
            pl.keff = topk_on ? min(rp.top_k, a.max_top_k) : a.max_top_k;
            const float u = uniform24(a.seed, b, pos, PURPOSE_DRAFT, a.step);
            draw_truncated<BF16>(a, va, b, i, o, pl, u, *sc);
            return;
        }
    }

    // 2. (sampled rows) while the other chunks' statistics are on their way:
    //    this chunk's weights in its own units exp2((z - m_c) * scale), as
    //    group sums gw[j] (the thread's group sums of step 1, rescaled from
    //    its maximum to the chunk's) with their starting running sums
    //    gstart[j] (group (j, tid) follows every (j', *) with j' < j and
    //    every (j, tid') with tid' < tid)
    __shared__ float gtot[NG][kWaves];
    __shared__ int lastW[kWaves], sTok;
    float gw[NG], gstart[NG], nms = 0.f;
    if (!greedy) {
        const float mc = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
        nms = mc == -kInf ? 0.f : -mc * scale;
        const float f = tmax == -kInf ? 0.f : fast_exp2((tmax - mc) * scale);
        float incl[NG];
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            gw[j] = gwt[j] * f;
            incl[j] = wave_scan_incl(gw[j]);
            if (lane == kWave - 1) gtot[j][wave] = incl[j];
        }
        if (tid == 0) sTok = 0x7fffffff;
        __syncthreads();
        float gbase = 0.f;
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            float before = 0.f, tot = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < kWaves; ++w2) {
                const float g = gtot[j][w2];
                if (w2 < wave) before += g;
                tot += g;
            }
            gstart[j] = gbase + before + (incl[j] - gw[j]);
            gbase += tot;
        }
    }

    // 3. the row's statistics and the chunk holding u * W (wave 0)
    __shared__ int sChosen, sDone;
    __shared__ float sLocal, sM, sS;
    if (wave == 0) {
        // the uniform does not depend on the statistics: drawn before the wait
        float u = 0.f;
        if (!greedy) {
            u = uniform24(a.seed, b, pos, PURPOSE_DRAFT, a.step);
            asm volatile("" : "+v"(u));
        }
        float m = -kInf;
        unsigned second = 0;
        bool ok = true;
        if (lane < a.C) ok = published_stats(stats_words(va, b, i, 1, lane), a.epoch, m, second);
        const bool late = __ballot(!ok) != 0;
        int chosen = -1, tok = -1;
        unsigned flags = 0;
        float M = nan, S = nan, local = 0.f;
        if (greedy) {
            int arg = lane < a.C ? (int)second : 0x7fffffff;
            const bool isnan_m = lane < a.C && __builtin_isnan(m);
            if (isnan_m || lane >= a.C) m = -kInf;
            wave_merge_arg(m, arg);
            if (__ballot(isnan_m) != 0 || m == -kInf) flags = SPECV_FLAG_NONFINITE_ROW;
            else tok = arg;
        } else {
            const float s = lane < a.C ? __uint_as_float(second) : 0.f;
            if (lane >= a.C) m = -kInf;
            float Mr = m, Sr = s;
            wave_merge_ms(Mr, Sr, scale);
            if (__builtin_isnan(Sr) || Mr == -kInf || !(Sr > 0.f)) {
                flags = SPECV_FLAG_NONFINITE_ROW;
            } else {
                M = Mr;
                S = Sr;
                // chunk masses s_c * exp2((m_c - M) * scale) and their prefix sums
                const float wc = m > -kInf ? s * fast_exp2((m - M) * scale) : 0.f;
                const float incl = wave_scan_incl(wc);
                const float W = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(incl), kWave - 1));
                const float target = u * W;
                const unsigned long long hit = __ballot(wc > 0.f && incl > target);
                const unsigned long long any = __ballot(wc > 0.f);
                // rounding: without a hit, the last chunk with mass
                chosen = hit ? __builtin_ctzll(hit) : (any ? 63 - __builtin_clzll(any) : -1);
                const float before = __int_as_float(
                    __builtin_amdgcn_readlane(__float_as_int(incl), chosen > 0 ? chosen - 1 : 0));
                const float mch = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), chosen > 0 ? chosen : 0));
                // u * W - (mass of the earlier chunks), in the chosen chunk's own
                // units exp2((z - m_c) * scale)
                local = (target - (chosen > 0 ? before : 0.f)) * fast_exp2((M - mch) * scale);
            }
        }
        if (late) {
            // this workgroup gave up on the row: it flags the draw and writes
            // nothing else (another workgroup of the row may have seen every
            // chunk and own the draw; its token is then valid)
            if (lane == 0 && a.out_stats) atomicOr(&a.out_stats[o].flags, (int)SPECV_FLAG_INTERNAL);
            chosen = -1;
        }
        if (lane == 0) {
            sChosen = chosen;
            sDone = chosen < 0;
            sLocal = local;
            sM = M;
            sS = S;
            // rows with nothing left to draw (greedy, bad) are written by chunk
            // 0's workgroup
            if (chosen < 0 && c == 0 && !late) write_draft(a, o, tok, nan, nan, nan, flags);
        }
    }
    __syncthreads();
    if (sDone || sChosen != c) return;

    // 4. the owner of the chunk: the group whose running-sum range holds the
    //    target claims it and scans its entries, recomputing their weights
    //    (the first whose running sum exceeds the target, else, rounding, the
    //    group's last entry with weight); the lowest claimed token wins; with
    //    no claim (rounding), the chunk's last entry with weight
    const float tloc = sLocal;
    int claim = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
        if (claim == 0x7fffffff && gw[j] > 0.f && tloc >= gstart[j] && tloc < gstart[j] + gw[j]) {
            float run = gstart[j];
            int first = -1, lastin = -1;
#pragma unroll
            for (int e = 0; e < G; ++e) {
                const float x = fast_exp2(fmaf(r.elem(j * G + e), scale, nms));
                run += x;
                if (x > 0.f) {
                    lastin = e;
                    if (first < 0 && run > tloc) first = e;
                }
            }
            if (first >= 0 || lastin >= 0) claim = (j * kBlock + tid) * G + (first >= 0 ? first : lastin);
        }
    }
    if (claim != 0x7fffffff) atomicMin(&sTok, claim);
    __syncthreads();
    if (sTok == 0x7fffffff) {
        // no claim: the chunk's last entry with weight
        int lastpos = -1;
#pragma unroll
        for (int j = 0; j < NG; ++j) {
#pragma unroll
            for (int e = 0; e < G; ++e) {
                if (fast_exp2(fmaf(r.elem(j * G + e), scale, nms)) > 0.f) lastpos = (j * kBlock + tid) * G + e;
            }
        }
        lastpos = wave_max_int(lastpos);
        if (lane == 0) lastW[wave] = lastpos;
        __syncthreads();
    }
    if (tid == 0) {
        int t = sTok;
        if (t == 0x7fffffff) t = max(max(lastW[0], lastW[1]), max(lastW[2], lastW[3]));
        if (t < 0) write_draft(a, o, -1, nan, nan, nan, SPECV_FLAG_NONFINITE_ROW);
        else write_draft(a, o, c * kChunk + t, sM, sS, -kInf, 0u);
    }
}

template <bool BF16, bool VEC, bool DEVCALL>
__global__ __launch_bounds__(kBlock) void k_sample_draft(DraftArgs a) {
    sample_draft_block<BF16, VEC, false, DEVCALL>(a, nullptr);
}

// With the truncation path (handles created with max_top_k > 0) and its LDS.
template <bool BF16, bool VEC, bool DEVCALL>
__global__ __launch_bounds__(kBlock) void k_sample_draft_trunc(DraftArgs a) {
    __shared__ TruncScratch sc;
    sample_draft_block<BF16, VEC, true, DEVCALL>(a, &sc);
}

template <bool DEVCALL>
void (*pick_draft(bool bf16, bool vec, bool trunc))(DraftArgs) {
    if (trunc)
        return bf16 ? (vec ? k_sample_draft_trunc<true, true, DEVCALL> : k_sample_draft_trunc<true, false, DEVCALL>)
                    : (vec ? k_sample_draft_trunc<false, true, DEVCALL> : k_sample_draft_trunc<false, false, DEVCALL>);
    return bf16 ? (vec ? k_sample_draft<true, true, DEVCALL> : k_sample_draft<true, false, DEVCALL>)
                : (vec ? k_sample_draft<false, true, DEVCALL> : k_sample_draft<false, false, DEVCALL>);
}

}  // namespace

hipError_t set_wait_limit_draft(int n) { return set_wait_limit_here(n); }

hipError_t launch_sample_draft(const DraftArgs& a, bool bf16, bool vec, bool devcall, hipStream_t stream,
                               hipEvent_t* ev) {
    const long long blocks = (long long)a.n * a.B * a.C + (devcall ? 1 : 0);   // + the closing workgroup
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    void (*fn)(DraftArgs) = devcall ? pick_draft<true>(bf16, vec, a.cand_cap > 0)
                                    : pick_draft<false>(bf16, vec, a.cand_cap > 0);
    if (ev)
        hipExtLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(kBlock), 0, stream, ev[0], ev[1], 0, a);
    else
        hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(kBlock), 0, stream, a);   // also under capture
    return hipGetLastError();
}

}  // namespace specv
