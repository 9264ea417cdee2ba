// libspecv kernels for gfx950 (CDNA4, wave64).
//
// The verify step is bandwidth-bound, and the round it computes is
// sequential: draft d_k only matters while every earlier draft was accepted
// (pseudo-code 10-1 stops at the first rejection), so rows past the first
// rejection need not be read.  One launch does the whole step with two kinds
// of workgroup:
//
//   streaming unit (k, b, c), position-major, P x B x C of them: reads chunk
//            c (8192 entries) of target row k and, for sampling and
//            truncated rows below gamma, of draft row k, with 16-byte loads;
//            reduces it to chunk statistics (max / sum of exp2 for sampling
//            rows, max / lowest argmax for greedy rows, top-k candidates for
//            truncated rows), published as tagged words; bumps the
//            pair's arrival counter.  The last of the C units to arrive
//            merges the statistics and takes position k's accept test,
//            publishes the pair record and sets the position's bit in the
//            row's status word.  Units of position k >= 2 first read that
//            word and skip their chunk when the round stopped before k; the
//            stream itself never waits for a decision, so positions that are
//            still open are read speculatively.
//   row finish: the decider whose bit resolves the row (first rejection, a
//            bad row, the cap, or the bonus position reached) gathers the
//            consulted pair records, writes diagnostics and, for greedy,
//            capped, dead and truncated rows, the outputs; for sampling rows
//            it publishes the row record (where the round stopped and that
//            position's normalisers).
//   sampling workgroup (b, c), B x C of them after the stream: waits for
//            the row record, reads chunk c of the stopping position's target
//            (and draft) row, sums the correction weight max(p - q, 0) (or
//            the bonus weight p), publishes the sum, reads every chunk's sum,
//            and the workgroup whose chunk holds u * W finds the token with a
//            block prefix sum.
//
// Hand-offs use agent-scope atomics on words tagged with the launch's call
// number, polled with a bound (the expiry flags the row, it never hangs the
// launch).  The call number is taken on the device (a ticket per workgroup,
// specv_rows.hpp), so a launch replayed from a captured graph gets its own.  Workgroups
// are dispatched in increasing ID order within each XCD, and every wait is
// for words that a workgroup with a lower ID writes (the stream's decisions,
// for the sampling workgroups) or that were stored before the status bit the
// waiter saw (pair records, for the row finish), so the waits end.
//
// Sources: "11.1 核心原理: Draft + Verify 与 Rejection Sampling" (11.1.1
// alignment, 11.1.2 acceptance / residual / greedy / processed proposals,
// pseudo-code 10-1) and "Fast Inference from Transformers via Speculative
// Decoding" (speculative sampling, bonus token).

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "specv_device.hpp"
#include "specv_internal.hpp"
#include "specv_rows.hpp"

namespace specv {
namespace {

// ---------------------------------------------------------------- row status
// Row status word (one per batch row and call parity):
//   bit k        accept test of position k passed        (k < gamma <= 31)
//   bit 31       bonus row merged and usable
//   bit 32 + k   position k stopped the round: rejected, or a consulted row is bad
//   bit 63       bonus row bad
constexpr unsigned long long kBonusOk = 1ull << 31;
constexpr unsigned long long kBonusBad = 1ull << 63;

// Where the round stands, from a row status word.
enum How { H_OPEN = 0, H_STOP, H_CAPPED, H_BONUS, H_BONUS_BAD };
struct Res {
    int how;
    int n;          // H_STOP: the stopping position; H_CAPPED: accepted drafts
};

__device__ inline Res resolve(unsigned long long st, const Plan& pl, int gamma) {
    const unsigned acc = (unsigned)st & 0x7fffffffu;
    const unsigned stop = (unsigned)(st >> 32) & 0x7fffffffu;
    Res r;
    const int j = __builtin_ctz(~acc);          // first position not (yet) accepted; <= 31
    if (j < pl.ntest) {
        r.n = j;
        r.how = ((stop >> j) & 1u) ? H_STOP : H_OPEN;
        return r;
    }
    r.n = pl.ntest;
    if (pl.nt <= gamma) r.how = H_CAPPED;       // the cap leaves no bonus position
    else if (st & kBonusOk) r.how = H_BONUS;
    else if (st & kBonusBad) r.how = H_BONUS_BAD;
    else r.how = H_OPEN;
    return r;
}

__device__ inline bool stopped_before(unsigned long long st, int k) {
    const unsigned stop = (unsigned)(st >> 32) & 0x7fffffffu;
    return (stop & ((1u << k) - 1u)) != 0;      // k <= 31
}

// (a.ws is the launch's record set: parity_set of the call number's parity)
__device__ inline unsigned* pair_counter(const Args& a, int b, int k) {
    return a.ws.ctr + pair_id(a, b, k) * kSlot;
}
__device__ inline unsigned long long* status_word(const Args& a, int b) {
    return a.ws.status + (long long)b * (kSlot / 2);
}

// ---------------------------------------------------------------- row finish
// A pair record in registers.
struct PairVals {
    unsigned state;
    float p, q;
    int arg;
    float mt, invt, mq, invq;
};

// Run by the workgroup whose status update resolved row b (whole
// workgroup; wave 0 does the row's bookkeeping, lane i for position i): the
// records of the positions the round consulted give the flags and the
// diagnostics; greedy, capped and dead rows get their outputs here,
// truncated rows draw their token here from the kept lists, and sampling rows
// hand the draw to their sampling workgroups through the row record.
template <bool BF16, bool TRUNC, int PROP>
__device__ __forceinline__ void finish_row(const Args& a, int b, int k, const PairVals& own, const Plan& pl,
                           unsigned long long st, TruncScratch* sc) {
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const Res r = resolve(st, pl, a.gamma);
    const bool greedy = pl.mode == MODE_GREEDY;
    // highest position whose record is read
    const int last = r.how == H_STOP ? r.n : (r.how == H_CAPPED ? r.n - 1 : a.gamma);
    const int nacc = r.how == H_STOP || r.how == H_CAPPED ? r.n : a.gamma;
    __shared__ int fKind, fDead, fAt;
    __shared__ unsigned fFlags;
    unsigned long long* rowrec = a.ws.rowrec + (long long)b * kRowWords;
    if (wave == 0) {
        // A sampling row whose round ends at this position hands its draw to
        // its sampling workgroups at once: the kind, the position and this
        // pair's normalisers do not depend on the other positions' records,
        // which only add flags (RW_FLAGS, published once gathered).
        const int at = r.how == H_STOP ? r.n : a.gamma;
        const bool early = pl.mode == MODE_SAMPLE && at == k &&
                           ((r.how == H_STOP && (own.state & 0xffu) == OUT_REJ) || r.how == H_BONUS);
        if (early) {
            const unsigned rec = (unsigned)(r.how == H_STOP ? KIND_RESIDUAL : KIND_BONUS) | ((unsigned)at << 3);
            const unsigned v = lane == RW_MT ? __float_as_uint(own.mt) : lane == RW_INVT ? __float_as_uint(own.invt)
                             : lane == RW_MQ ? __float_as_uint(own.mq) : lane == RW_INVQ ? __float_as_uint(own.invq)
                             : rec;
            if (lane <= RW_INVQ) put_tagged(&rowrec[lane], v, a.epoch);
        }
        unsigned long long w[kPairWords];
#pragma unroll
        for (int i = 0; i < kPairWords; ++i) w[i] = 0;
        bool ok = true;
        if (lane <= last) {
            if (lane == k) {
                w[PW_STATE] = own.state;
                w[PW_P] = __float_as_uint(own.p);
                w[PW_Q] = __float_as_uint(own.q);
                w[PW_ARG] = (unsigned)own.arg;
                w[PW_MT] = __float_as_uint(own.mt);
                w[PW_INVT] = __float_as_uint(own.invt);
                w[PW_MQ] = __float_as_uint(own.mq);
                w[PW_INVQ] = __float_as_uint(own.invq);
            } else {
                const PairRec* pr = &a.ws.pair[pair_id(a, b, lane)];
                ok = false;
#pragma unroll 1
                for (int spin = 0; spin < g_wait_limit; ++spin) {
                    bool all = true;
#pragma unroll
                    for (int i = 0; i < kPairWords; ++i) {
                        w[i] = published(&pr->w[i]);
                        all = all && tag_is(w[i], a.epoch);
                    }
                    if (all) {
                        ok = true;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
            }
        }
        const unsigned rs = (unsigned)w[PW_STATE];
        unsigned flags = pl.flags | wave_or(lane < nacc ? (rs >> 8) : 0u);
        if (__ballot(!ok)) flags |= SPECV_FLAG_INTERNAL;
        int kind = KIND_NONE, sampled = -1, tested = nacc;
        bool dead = false;
        // the record of the position that ended the round, read from its lane
        // here, with every lane active (a cross-lane read inside a branch that
        // only some lanes take can see registers the branch never restored)
        const unsigned s_at = __builtin_amdgcn_readlane(rs, at);
        const int a_at = __builtin_amdgcn_readlane((int)(unsigned)w[PW_ARG], at);
        const unsigned mt_at = __builtin_amdgcn_readlane((unsigned)w[PW_MT], at);
        const unsigned invt_at = __builtin_amdgcn_readlane((unsigned)w[PW_INVT], at);
        const unsigned mq_at = __builtin_amdgcn_readlane((unsigned)w[PW_MQ], at);
        const unsigned invq_at = __builtin_amdgcn_readlane((unsigned)w[PW_INVQ], at);
        if (r.how == H_STOP || r.how == H_BONUS || r.how == H_BONUS_BAD) {
            flags |= s_at >> 8;
            if (r.how == H_BONUS_BAD || (s_at & 0xffu) == OUT_BAD) {
                dead = true;
            } else {
                if (r.how == H_STOP) tested = r.n + 1;
                if (greedy) sampled = a_at;
                else kind = r.how == H_STOP ? KIND_RESIDUAL : KIND_BONUS;
            }
        }
        if (greedy) tested = 0;
        write_diag_wave(a, b, tested, __uint_as_float((unsigned)w[PW_P]),
                        __uint_as_float((unsigned)w[PW_Q]));
        const bool samp = pl.mode == MODE_SAMPLE && kind != KIND_NONE;
        if (kind == KIND_NONE) write_outputs_wave(a, b, nacc, nacc, flags, dead, sampled, 0.f, pl.tok);
        if (pl.mode == MODE_SAMPLE) {
            // the row record (lane i writes word i), unless handed over above,
            // and the row's flags
            const unsigned rec = (unsigned)(samp ? kind : KIND_NONE) | ((unsigned)(samp ? at : 0) << 3);
            const unsigned v = lane == RW_MT ? mt_at : lane == RW_INVT ? invt_at
                             : lane == RW_MQ ? mq_at : lane == RW_INVQ ? invq_at
                             : lane == RW_FLAGS ? (flags & 0xffu) : rec;
            if ((lane <= RW_INVQ && !early) || lane == RW_FLAGS) put_tagged(&rowrec[lane], v, a.epoch);
        }
        if (lane == 0) {
            fKind = kind;
            fDead = dead;
            fFlags = flags;
            fAt = at;
        }
    }
    __syncthreads();
    if constexpr (TRUNC) {
        if (pl.mode == MODE_TRUNC && fKind != KIND_NONE) {
            const bool res = fKind == KIND_RESIDUAL;
            const int pos = fAt;
            const float u = uniform24(a.seed, b, pos, res ? PURPOSE_RESIDUAL : PURPOSE_BONUS, a.step);
            float wres;
            bool fb;
            const int tok = trunc_sample<BF16, PROP>(a, b, pos, res, u, pl, *sc, &wres, &fb);
            if (wave == 0) {
                unsigned flags = fFlags | (fb ? SPECV_FLAG_RESIDUAL_FALLBACK : 0u);
                bool dead = fDead;
                if (tok < 0) {
                    dead = true;
                    flags |= SPECV_FLAG_NONFINITE_ROW;
                }
                write_outputs_wave(a, b, nacc, nacc, flags, dead, tok, wres, pl.tok);
            }
        }
    }
}

// ---------------------------------------------------------------- pair decision
// Run by the last unit of pair (k, b) to arrive (whole workgroup): merge the
// chunk statistics of target row k (and draft row k), or truncate the two
// rows, and take the accept test of position k (pseudo-code 10-1: accept
// with probability min(1, p / q), i.e. u * q < p; greedy rows compare with the
// argmax); publish the pair record, set the pair's status bit, and finish
// the row when that resolves it.  Readers of the pair record check its tags,
// so its stores need not complete first, except for truncated rows, whose
// kept lists and TruncRows are read untagged.
template <bool BF16, bool TRUNC, int PROP>
__device__ __forceinline__ void decide_pair(const Args& a, int b, int k, const Plan& pl, TruncScratch* sc) {
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const bool greedy = pl.mode == MODE_GREEDY;
    const bool trunc = TRUNC && pl.mode == MODE_TRUNC;
    const bool test = k < a.gamma;
    constexpr bool pm = PROP == kPropPoint;  // q_k is the point mass on d_k
    constexpr bool qs = PROP == kPropStats;  // q_k's statistics come from the drafter
    const bool zneed = !greedy && test;     // z at d_k and the accept uniform
    const bool qside = zneed && !pm;        // the draft row's entry at d_k is consulted
    const bool two = qside && !qs;          // the draft row's chunk statistics are merged
    const float scale = pl.scale;
    __shared__ float dM[2], dS[2], dZ[2], dU;
    __shared__ int dA, dBad[2], dLate[2];
    __shared__ TruncRow dT[2];
    __shared__ int dFinish;
    __shared__ unsigned long long dNew;
    __shared__ PairVals dOwn;
    const int d = test ? draft_token(a, b, k) : 0;
    if (trunc) {
        if constexpr (TRUNC) {
            // z at d_k, requested before the merge by lane k (which holds
            // d_k from the plan) and kept in its registers until the
            // decision
            float zt = 0.f, zq = 0.f;
            if (zneed && tid == k) {
                zt = load_elem<BF16>(row_ptr<BF16>(a.tgt, a.t_sb, a.t_sp, b, k), pl.tok);
                if (qside) zq = load_elem<BF16>(row_ptr<BF16>(a.drf, a.d_sb, a.d_sp, b, k), pl.tok);
            }
            // both rows in lockstep when they take the usual path, else one
            // after the other
            __shared__ TruncRow dPair[2];
            TruncRow t0, t1;
            if (two && row_merge_pair<BF16>(a, b, k, pl, *sc, dPair)) {
                t0 = dPair[0];
                t1 = dPair[1];
            } else {
                t0 = row_merge<BF16>(a, b, k, 0, pl, *sc);
                t1 = t0;
                if (two) t1 = row_merge<BF16>(a, b, k, 1, pl, *sc);
            }
            // rows the candidates could not settle: the exact truncation,
            // from one call site
#pragma unroll 1
            for (int side = 0; side < (two ? 2 : 1); ++side) {
                const TruncRow t = row_settle<BF16>(a, b, k, side, pl, side ? t1 : t0, *sc);
                if (side) t1 = t;
                else t0 = t;
            }
            if (!two) t1 = t0;
            if (tid == 0) {
                dT[0] = t0;
                dT[1] = qs && qside ? stats_trow(a.qstats[(long long)b * a.qs_sb + k]) : t1;
                dLate[0] = dLate[1] = 0;
                if (zneed) dU = uniform24(a.seed, b, k, PURPOSE_ACCEPT, a.step);
            }
            if (zneed && tid == k) {
                dZ[0] = zt;
                dZ[1] = zq;
            }
        }
    } else {
        // one wave per row merges the chunk statistics (lane c: chunk c);
        // wave 2 fetches z at d_k and draws the accept uniform meanwhile
        if (wave < (two ? 2 : 1)) {
            const int side = wave;
            float m = -kInf;
            unsigned second = 0;
            bool ok = true;
            if (lane < a.C) ok = published_stats(stats_words(a, b, k, side, lane), a.epoch, m, second);
            float s = 0.f;
            int arg = 0x7fffffff;
            bool nan = false;
            if (lane < a.C) {
                if (greedy) {
                    arg = (int)second;
                    nan = __builtin_isnan(m);
                    if (nan) m = -kInf;
                } else {
                    s = __uint_as_float(second);
                }
            }
            if (greedy) wave_merge_arg(m, arg);
            else wave_merge_ms(m, s, scale);
            const bool anybad = __ballot(nan) != 0;
            const bool late = __ballot(!ok) != 0;
            if (lane == 0) {
                dM[side] = m;
                dS[side] = s;
                dBad[side] = anybad || (greedy ? false : __builtin_isnan(s));
                dLate[side] = late;
                if (side == 0) dA = arg;
            }
        } else if (wave == 2 && zneed) {
            // both rows' z at d_k from lane k, which holds d_k from the
            // plan (its own register: no wait for the token's load), and the
            // drafter's statistics (lanes 3, 4), in one round trip
            if (lane == k) {
                dZ[0] = load_elem<BF16>(row_ptr<BF16>(a.tgt, a.t_sb, a.t_sp, b, k), pl.tok);
                if (qside) dZ[1] = load_elem<BF16>(row_ptr<BF16>(a.drf, a.d_sb, a.d_sp, b, k), pl.tok);
            }
            if (lane == 2) dU = uniform24(a.seed, b, k, PURPOSE_ACCEPT, a.step);
            if (qs && (lane == 3 || lane == 4)) {
                const specv_draft_stats* st = &a.qstats[(long long)b * a.qs_sb + k];
                const float x = lane == 3 ? st->max : st->sum;
                if (lane == 3) {
                    dM[1] = x;
                    dLate[1] = 0;
                } else {
                    dS[1] = x;
                    dBad[1] = __builtin_isnan(x);
                }
            }
        }
    }
    // the truncation steps' untagged words (kept lists, row records) are
    // trusted once the status bit is seen: every wave's stores complete
    // before the barrier that precedes the status update
    if (trunc) wait_stores();
    __syncthreads();
    if (tid == 0) {
        PairVals v{};
        unsigned outcome, flags = 0;
        if (greedy) {
            const bool bad = dBad[0] || dM[0] == -kInf;
            if (bad) {
                outcome = OUT_BAD;
                flags = SPECV_FLAG_NONFINITE_ROW;
            } else {
                outcome = !test ? OUT_BONUS : (d == dA ? OUT_ACC : OUT_REJ);
            }
            v.arg = dA;
        } else if (trunc) {
            const TruncRow& t0 = dT[0];
            const TruncRow& t1 = dT[1];
            flags = (t0.flags | (qside ? t1.flags : 0u)) & SPECV_FLAG_TOPP_NEAR;
            if (t0.bad || (qside && t1.bad)) flags |= SPECV_FLAG_NONFINITE_ROW;
            if (trow_dead(t0) || (qside && trow_dead(t1))) {
                outcome = OUT_BAD;
            } else if (!test) {
                outcome = OUT_BONUS;
            } else {
                v.p = trunc_prob(t0, dZ[0], scale);
                v.q = pm ? 1.f : trunc_prob(t1, dZ[1], scale);
                if (!pm && !(finite_logit(dZ[1]) && dZ[1] >= t1.tstar)) flags |= SPECV_FLAG_Q_ZERO;
                outcome = dU * v.q < v.p ? OUT_ACC : OUT_REJ;
            }
        } else {
            const bool badT = dBad[0] || dM[0] == -kInf || !(dS[0] > 0.f);
            const bool badQ = qside && (dBad[1] || dM[1] == -kInf || !(dS[1] > 0.f));
            v.mt = dM[0];
            v.invt = 1.f / dS[0];
            if (qside) {
                v.mq = dM[1];
                v.invq = 1.f / dS[1];
            }
            if (badT || badQ) {
                outcome = OUT_BAD;
                flags = SPECV_FLAG_NONFINITE_ROW;
            } else if (!test) {
                outcome = OUT_BONUS;
            } else {
                v.p = fast_exp2((dZ[0] - dM[0]) * scale) / dS[0];
                v.q = pm ? 1.f : fast_exp2((dZ[1] - dM[1]) * scale) / dS[1];
                if (!pm && dZ[1] == -kInf) flags |= SPECV_FLAG_Q_ZERO;
                outcome = dU * v.q < v.p ? OUT_ACC : OUT_REJ;
            }
        }
        if (dLate[0] || (two && dLate[1])) {
            // statistics that never arrived (a dispatch order other than the
            // hardware's): the row emits nothing
            outcome = OUT_BAD;
            flags |= SPECV_FLAG_INTERNAL;
        }
        v.state = outcome | (flags << 8);
        PairRec* pr = &a.ws.pair[pair_id(a, b, k)];
        const unsigned e = a.epoch;
        put_tagged(&pr->w[PW_P], __float_as_uint(v.p), e);
        put_tagged(&pr->w[PW_Q], __float_as_uint(v.q), e);
        put_tagged(&pr->w[PW_ARG], (unsigned)v.arg, e);
        put_tagged(&pr->w[PW_MT], __float_as_uint(v.mt), e);
        put_tagged(&pr->w[PW_INVT], __float_as_uint(v.invt), e);
        put_tagged(&pr->w[PW_MQ], __float_as_uint(v.mq), e);
        put_tagged(&pr->w[PW_INVQ], __float_as_uint(v.invq), e);
        put_tagged(&pr->w[PW_STATE], v.state, e);
        dOwn = v;
        unsigned long long bit;
        if (test) bit = outcome == OUT_ACC ? (1ull << k) : (1ull << (32 + k));
        else bit = outcome == OUT_BONUS ? kBonusOk : kBonusBad;
        if (trunc) wait_stores();
        const unsigned long long old = __hip_atomic_fetch_or(
            status_word(a, b), bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const unsigned long long now = old | bit;
        dNew = now;
        dFinish = resolve(old, pl, a.gamma).how == H_OPEN && resolve(now, pl, a.gamma).how != H_OPEN;
    }
    __syncthreads();
    if (dFinish) finish_row<BF16, TRUNC, PROP>(a, b, k, dOwn, pl, dNew, sc);
}

// ---------------------------------------------------------------- sampling
// Correction / bonus weight of entry z (target) and zq (draft) of the row
// pair being sampled.
struct Weights {
    int residual;        // 1: max(p - q, 0); 0: p
    int dpm;             // point-mass proposal: q = delta(dpm), so the correction weight
                         // is p except 0 at dpm; -1 otherwise
    float mt, st, invt;  // target row max, scale, 1 / sum
    float mq, invq;      // draft row max, 1 / sum
    // Products are rounded separately (no fused multiply-add) so that equal
    // p and q rows give exactly zero correction weight.
    __device__ inline float p(float z) const {
        return __fmul_rn(fast_exp2(__fmul_rn(z - mt, st)), invt);
    }
    __device__ inline float w(float z, float zq) const {
        const float pz = p(z);
        if (!residual) return pz;
        const float q = __fmul_rn(fast_exp2(__fmul_rn(zq - mq, st)), invq);
        return fmaxf(__fsub_rn(pz, q), 0.f);
    }
};

// Correction (position k < gamma) or bonus (k == gamma) sample of row b, by
// its C sampling workgroups, each holding chunk c of the sampled row pair in
// registers: each publishes its chunk's weight sum and p mass, reads all of
// them, and the workgroup whose chunk holds u * W scans it (tokens in
// ascending order, first running sum > u * W) and writes the outputs.
// The row's flags (RW_FLAGS of the row record) are read with the chunk sums.
// Whole workgroup.
template <bool BF16, bool VEC, int PROP>
__device__ void sample_from_regs(const Args& a, int b, int k, int c, const Plan& pl, Weights wt,
                                 const ChunkRegs<BF16, VEC>& rt,
                                 const ChunkRegs<BF16, VEC>& rd) {
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    constexpr int G = BF16 ? 8 : 4;
    constexpr int NG = kPerThread / G;
    const float u = uniform24(a.seed, b, k, wt.residual ? PURPOSE_RESIDUAL : PURPOSE_BONUS, a.step);
    // the weights of this thread's entries (kept for the scan), their group
    // sums, and the p mass
    float w[kPerThread], gw[NG], sw = 0.f, sp = 0.f;
    if (PROP == kPropPoint && wt.dpm >= 0) {
        // point-mass proposal: p, except 0 at the proposed token
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < G; ++e) {
                const int i = j * G + e;
                const float pz = wt.p(rt.elem(i));
                sp += pz;
                w[i] = c * kChunk + chunk_index<BF16>(i) == wt.dpm ? 0.f : pz;
                s += w[i];
            }
            gw[j] = s;
            sw += s;
        }
    } else {
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < G; ++e) {
                const int i = j * G + e;
                const float pz = wt.p(rt.elem(i));
                sp += pz;
                w[i] = wt.residual ? wt.w(rt.elem(i), rd.elem(i)) : pz;
                s += w[i];
            }
            gw[j] = s;
            sw += s;
        }
    }
    __shared__ float red[2][kWaves];
    sw = wave_sum(sw);
    sp = wave_sum(sp);
    if (lane == 0) {
        red[0][wave] = sw;
        red[1][wave] = sp;
    }
    __syncthreads();

    // wave 0 publishes this chunk's sums, reads every chunk's (lane c: chunk
    // c) and picks the chunk holding u * W from their prefix sums; the same
    // arithmetic in every workgroup of the row, so all pick the same chunk
    __shared__ float sBase, sTarget, sWres;
    __shared__ int sChunk, sRes, sOk;
    __shared__ unsigned sFlags;
    if (wave == 0) {
        float wc = red[0][0], pc = red[1][0];
        for (int w2 = 1; w2 < kWaves; ++w2) {
            wc += red[0][w2];
            pc += red[1][w2];
        }
        unsigned long long* base = a.ws.wsum + (long long)b * a.C * 2;
        if (lane < 2) put_tagged(base + c * 2 + lane, __float_as_uint(lane == 0 ? wc : pc), a.epoch);
        const unsigned long long* rflags = a.ws.rowrec + (long long)b * kRowWords + RW_FLAGS;
        bool done = false;
        unsigned long long w0 = 0, w1 = 0, wf = 0;
#pragma unroll 1
        for (int spin = 0; spin < g_wait_limit; ++spin) {
            if (lane < a.C) {
                w0 = published(base + lane * 2);
                w1 = published(base + lane * 2 + 1);
            }
            if (lane == 0) wf = published(rflags);
            const bool mine = (lane >= a.C || (tag_is(w0, a.epoch) && tag_is(w1, a.epoch))) &&
                              (lane != 0 || tag_is(wf, a.epoch));
            if (__ballot(mine) == ~0ull) {
                done = true;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        float vw = lane < a.C ? __uint_as_float((unsigned)w0) : 0.f;
        const float vp = lane < a.C ? __uint_as_float((unsigned)w1) : 0.f;
        unsigned flags = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)wf) & 0xffu;
        int res = wt.residual;
        float W = wave_sum(vw);
        const float wres = res ? W : 0.f;
        if (res && (!(W > 0.f) || !__builtin_isfinite(W))) {
            // the correction mass vanished (p == q where the draft was
            // rejected, or rounding): sample from p at that position
            flags |= SPECV_FLAG_RESIDUAL_FALLBACK;
            res = 0;
            vw = vp;
            W = wave_sum(vw);
        }
        const float target = u * W;
        const float incl = wave_scan_incl(vw);
        const unsigned long long hit = __ballot(lane < a.C && vw > 0.f && incl > target);
        const unsigned long long pos = __ballot(lane < a.C && vw > 0.f);
        // rounding: without a hit, the last chunk with weight
        const int chosen = hit ? __builtin_ctzll(hit) : (pos ? 63 - __builtin_clzll(pos) : -1);
        const float before = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(incl), chosen > 0 ? chosen - 1 : 0));
        if (lane == 0) {
            sOk = done;
            sChunk = chosen;
            sBase = chosen > 0 ? before : 0.f;
            sTarget = target;
            sRes = res;
            sWres = wres;
            sFlags = flags;
            if (!done && a.out_flags) atomicOr(&a.out_flags[b], (int)SPECV_FLAG_INTERNAL);
        }
    }
    __syncthreads();
    if (!sOk) return;
    const int chosen = sChunk;
    if (chosen < 0) {
        // no weight anywhere: cannot happen for finite rows
        if (c == 0 && wave == 0)
            write_outputs_wave(a, b, k, k, sFlags | SPECV_FLAG_NONFINITE_ROW, true, -1, sWres, pl.tok);
        return;
    }
    if (chosen != c) return;
    if (sRes != wt.residual) {
        // fallback weights p
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < G; ++e) {
                w[j * G + e] = wt.p(rt.elem(j * G + e));
                s += w[j * G + e];
            }
            gw[j] = s;
        }
    }
    const int t = chunk_inverse_cdf<BF16>(w, gw, sBase, sTarget);
    if (wave == 0) {
        const bool dead = t < 0;
        unsigned flags = sFlags;
        if (dead) flags |= SPECV_FLAG_NONFINITE_ROW;
        write_outputs_wave(a, b, k, k, flags, dead, dead ? -1 : c * kChunk + t, sWres, pl.tok);
    }
}

// ---------------------------------------------------------------- streaming
// Unit (k, b, c): chunk c of target row k and (sampling and truncated rows,
// k < gamma) of draft row k, reduced to chunk statistics that are published
// for the pair's decision; the last unit of the pair to arrive decides it.
// A unit at position k >= kSkipFrom skips its chunk when its row's status
// (st, read with the ticket) shows that the round stopped before k;
// otherwise it reads (speculatively when earlier positions are undecided),
// so the stream never waits for a decision.
#ifndef SPECV_SKIP_FROM
#define SPECV_SKIP_FROM 2
#endif
constexpr int kSkipFrom = SPECV_SKIP_FROM;

template <bool BF16, bool VEC, bool TRUNC, int PROP, bool DEVCALL>
__device__ __forceinline__ void stream_unit(const Args& a0, int k, int b, int c, TruncScratch* sc) {
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    // the call number (the host's, or a plain load of the device's, with the
    // plan's loads) and, for units that may skip, the row's status word (of
    // both parities when the number comes from the device), in one round
    // trip.  A device-numbered workgroup counts itself only where nothing it
    // still waits for was issued after the count (vector memory operations
    // retire in order): on its way out, or right before the arrival, whose
    // own round trip covers it.
    const bool check = k >= kSkipFrom;
    const unsigned e = DEVCALL ? read_call(a0.ws) : a0.epoch;
    unsigned long long st0 = 0, st1 = 0;
    if (check && tid == 0) {
        if constexpr (DEVCALL) {
            st0 = published(a0.ws.status + (long long)b * (kSlot / 2));
            st1 = published(a0.ws.status + ((long long)a0.ws.n_rows + b) * (kSlot / 2));
        } else {
            st0 = published(a0.ws.status + ((long long)(e & 1u) * a0.ws.n_rows + b) * (kSlot / 2));
        }
    }
    const Plan pl = make_plan(a0, b);
    Args a = a0;
    a.epoch = DEVCALL ? call_tag(e) : e;
    a.ws = parity_set<DEVCALL>(a0.ws, e & 1u);
    __shared__ int sSkip;
    if (pl.mode == MODE_SKIP) {
        if (k == 0 && c == 0 && wave == 0) {
            write_outputs_wave(a, b, 0, 0, pl.flags, true, -1, 0.f, pl.tok);
            write_diag_wave(a, b, 0, 0.f, 0.f);
        }
        if (DEVCALL && tid == 0) count_call(a0.ws, e, b);
        return;
    }
    if (k >= pl.nt) {                               // a position the round cannot consult
        if (DEVCALL && tid == 0) count_call(a0.ws, e, b);
        return;
    }
    if (check) {
        if (tid == 0) sSkip = stopped_before((DEVCALL && (e & 1u)) ? st1 : st0, k);
        __syncthreads();
        if (sSkip) {
            if (DEVCALL && tid == 0) count_call(a0.ws, e, b);
            return;
        }
    }
    const bool greedy = pl.mode == MODE_GREEDY;
    const bool trunc = TRUNC && pl.mode == MODE_TRUNC;
    const bool two = !greedy && k < a.gamma && PROP == kPropLogits;
    const void* trow = row_ptr<BF16>(a.tgt, a.t_sb, a.t_sp, b, k);
    const void* drow = two ? row_ptr<BF16>(a.drf, a.d_sb, a.d_sp, b, k) : nullptr;
    const int v0 = c * kChunk;
    const int len = min(kChunk, a.V - v0);
    ChunkRegs<BF16, VEC> rt, rd;
    rt.issue(trow, v0, len);
    if (two) rd.issue(drow, v0, len);
    rt.finish(trow, v0, len);
    if (two) rd.finish(drow, v0, len);

    __shared__ float sm[2][kWaves], ss[2][kWaves];
    __shared__ int si[kWaves];
    __shared__ unsigned sb[kWaves];
    __shared__ int sLast;
    const float scale = pl.scale;
    if (greedy) {
        float best;
        int bi;
        unsigned bad;
        wave_chunk_argmax<BF16>(rt, v0, best, bi, bad);
        if (lane == 0) {
            sm[0][wave] = best;
            si[wave] = bi;
            sb[wave] = bad;
        }
        __syncthreads();
        if (tid == 0) {
            for (int w = 1; w < kWaves; ++w) {
                merge_arg(best, bi, sm[0][w], si[w]);
                bad |= sb[w];
            }
            publish_stats(stats_words(a, b, k, 0, c), bad ? __builtin_nanf("") : best, (unsigned)bi,
                          a.epoch);
        }
    } else {
        // one call per side on its own registers (selecting between rt and
        // rd by reference would put both in private memory)
        auto side_stats = [&](int side, const ChunkRegs<BF16, VEC>& r, float& tmax) {
            float m, s;
            wave_chunk_ms(r, scale, m, s, &tmax);
            if (lane == 0) {
                sm[side][wave] = m;
                ss[side][wave] = s;
            }
        };
        float tmax0 = -kInf, tmax1 = -kInf;     // the threads' maxima, the top-k tops when k <= 128
        side_stats(0, rt, tmax0);
        if (two) side_stats(1, rd, tmax1);
        if constexpr (TRUNC) {
            if (trunc)
                chunk_candidates_pair<BF16>(a, side_row(a, b, k, 0), side_row(a, b, k, 1), two, c, pl.keff,
                                            rt, rd, *sc, true, tmax0, tmax1);
        }
        __syncthreads();
        if (tid == 0) {
            for (int side = 0; side < (two ? 2 : 1); ++side) {
                float m = sm[side][0], s = ss[side][0];
                for (int w = 1; w < kWaves; ++w) merge_ms(m, s, sm[side][w], ss[side][w], scale);
                publish_stats(stats_words(a, b, k, side, c), m, __float_as_uint(s), a.epoch);
            }
        }
    }
    if (tid == 0) {
        if (DEVCALL) count_call(a0.ws, e, b);
        sLast = arrive(pair_counter(a, b, k), trunc) == (unsigned)(a.C - 1);
    }
    __syncthreads();
    if (sLast) decide_pair<BF16, TRUNC, PROP>(a, b, k, pl, sc);
}

// Sampling workgroup (b, c) of a sampling row: waits for the row record,
// then reads chunk c of the target (and draft) row of the position the round
// stopped at, or of the bonus row, and takes part in the sample.  Rows of
// other modes never need one.
template <bool BF16, bool VEC, int PROP, bool DEVCALL>
__device__ __forceinline__ void sample_item(const Args& a0, int b, int c) {
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const unsigned e = DEVCALL ? read_call(a0.ws) : a0.epoch;
    // with the host's call number the record set is known at once: the
    // record's first poll goes out with the plan's loads
    unsigned long long first = 0;
    if constexpr (!DEVCALL) {
        if (wave == 0 && lane <= RW_INVQ) first = published(a0.ws.rowrec + (long long)b * kRowWords + lane);
    }
    const Plan pl = make_plan(a0, b);
    if constexpr (DEVCALL) {
        // the sampling workgroups clear the other parity's record set between
        // them (they have time: most wait for their row's record), then count
        // themselves before their first poll
        clear_other_set(a0.ws, e, (long long)b * a0.C + c, (long long)a0.B * a0.C);
        if (tid == 0) count_call(a0.ws, e, b);
    }
    if (pl.mode != MODE_SAMPLE) return;
    Args a = a0;
    a.epoch = DEVCALL ? call_tag(e) : e;
    a.ws = parity_set<DEVCALL>(a0.ws, e & 1u);
    __shared__ unsigned sRec[kRowWords];
    __shared__ int sGo;
    if (wave == 0) {
        const unsigned long long* rr = a.ws.rowrec + (long long)b * kRowWords;
        int go = 0;
        unsigned long long v = 0;
#pragma unroll 1
        for (int spin = 0; spin < g_wait_limit; ++spin) {
            v = !DEVCALL && spin == 0 ? first : lane <= RW_INVQ ? published(rr + lane) : 0ull;
            if ((__ballot(lane <= RW_INVQ && tag_is(v, a.epoch)) & 0x1full) == 0x1full) {
                go = 1;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        if (lane < kRowWords) sRec[lane] = (unsigned)v;
        if (lane == 0) sGo = go;
        if (!go && lane == 0 && a.out_flags) atomicOr(&a.out_flags[b], (int)SPECV_FLAG_INTERNAL);
    }
    __syncthreads();
    if (!sGo) return;
    const unsigned rec = sRec[RW_REC];
    const int kind = (int)(rec & 7u);
    if (kind != KIND_RESIDUAL && kind != KIND_BONUS) return;
    const int k = (int)((rec >> 3) & 31u);
    const bool two = kind == KIND_RESIDUAL && PROP != kPropPoint;  // the draft row is read
    const void* trow = row_ptr<BF16>(a.tgt, a.t_sb, a.t_sp, b, k);
    const void* drow = two ? row_ptr<BF16>(a.drf, a.d_sb, a.d_sp, b, k) : nullptr;
    const int v0 = c * kChunk;
    const int len = min(kChunk, a.V - v0);
    ChunkRegs<BF16, VEC> rt, rd;
    rt.issue(trow, v0, len);
    if (two) rd.issue(drow, v0, len);
    rt.finish(trow, v0, len);
    if (two) rd.finish(drow, v0, len);
    Weights wt;
    wt.residual = kind == KIND_RESIDUAL;
    wt.dpm = PROP == kPropPoint && kind == KIND_RESIDUAL ? draft_token(a, b, k) : -1;
    wt.mt = __uint_as_float(sRec[RW_MT]);
    wt.invt = __uint_as_float(sRec[RW_INVT]);
    wt.mq = __uint_as_float(sRec[RW_MQ]);
    wt.invq = __uint_as_float(sRec[RW_INVQ]);
    wt.st = pl.scale;
    sample_from_regs<BF16, VEC, PROP>(a, b, k, c, pl, wt, rt, rd);
}

// ---------------------------------------------------------------- k_verify
// One launch per call:
//   blocks [0, P * B * C):        streaming unit (k, b, c), position-major;
//   blocks [P * B * C, + B * C):  sampling workgroup (b, c);
// and, when the call number comes from the device (DEVCALL: launches that
// may be replayed from a captured graph), one more:
//   block P * B * C + B * C:      the closing workgroup, which advances the
//                                 call number once every other one read it.
// The call number gives the tag of the words a launch publishes and the
// parity of its counters, status words and (DEVCALL) record set.  With the
// host's number every workgroup clears its share of the other parity's
// counters and status words; with the device's the sampling workgroups
// clear the other parity's whole record set.  The next launch starts from
// what was cleared.  k_verify_trunc carries the truncation path (handles
// created with max_top_k > 0) and its LDS scratch; without it truncated rows
// are flagged unsupported and the kernel stays lean.
__device__ inline void clear_other_parity(const Args& a) {
    const unsigned other = (a.epoch & 1u) ^ 1u;
    const long long stride = (long long)gridDim.x * kBlock;
    for (long long i = (long long)blockIdx.x * kBlock + threadIdx.x; i < a.ws.n_groups; i += stride)
        publish(a.ws.ctr + ((long long)other * a.ws.n_groups + i) * kSlot, 0u);
    for (long long i = (long long)blockIdx.x * kBlock + threadIdx.x; i < a.ws.n_rows; i += stride)
        publish(a.ws.status + ((long long)other * a.ws.n_rows + i) * (kSlot / 2), 0ull);
}

template <bool BF16, bool VEC, bool TRUNC, int PROP, bool DEVCALL>
__device__ inline void verify_block(const Args& a, TruncScratch* sc) {
    const int per_pos = a.B * a.C;
    const int t = blockIdx.x;
    if constexpr (DEVCALL) {
        if (t == (a.P + 1) * per_pos) {
            close_call(a.ws, a.B, (unsigned)((a.P + 1) * a.C), pack_dims(a.B, a.P, a.C));
            return;
        }
    } else {
        clear_other_parity(a);
    }
    const int k = t / per_pos;
    const int rem = t - k * per_pos;
    const int b = rem / a.C;
    const int c = rem - b * a.C;
    if (k < a.P) stream_unit<BF16, VEC, TRUNC, PROP, DEVCALL>(a, k, b, c, sc);
    else sample_item<BF16, VEC, PROP, DEVCALL>(a, b, c);
}

template <bool BF16, bool VEC, int PROP, bool DEVCALL>
__global__ __launch_bounds__(kBlock) void k_verify(Args a) {
    verify_block<BF16, VEC, false, PROP, DEVCALL>(a, nullptr);
}

// k_verify held to six resident workgroups per CU (80 VGPRs, a few of them
// spilled to private memory), for launches of many units: when most of a
// grid's units are skipped past early rejections, their dispatch and status
// round trips rather than the read bound the launch, and the sixth workgroup
// per CU pays for the spills (eager launches of bfloat16 target and draft
// logits).
__global__ __launch_bounds__(kBlock, 6) void k_verify_wide(Args a) {
    verify_block<true, true, false, kPropLogits, false>(a, nullptr);
}

template <bool BF16, bool VEC, int PROP, bool DEVCALL>
__global__ __launch_bounds__(kBlock) void k_verify_trunc(Args a) {
    __shared__ TruncScratch sc;
    verify_block<BF16, VEC, true, PROP, DEVCALL>(a, &sc);
}

using KernelFn = void (*)(Args);

// Each proposal kind (and call-number source) is a separate instantiation,
// so that the two-model kernels carry none of the other kinds' code.
template <int PROP, bool DEVCALL>
KernelFn pick_prop(bool bf16, bool vec, bool trunc, bool wide) {
    if constexpr (!DEVCALL && PROP == kPropLogits) {
        if (wide && !trunc && bf16 && vec) return k_verify_wide;
    }
    if (trunc) {
        if (bf16) return vec ? k_verify_trunc<true, true, PROP, DEVCALL> : k_verify_trunc<true, false, PROP, DEVCALL>;
        return vec ? k_verify_trunc<false, true, PROP, DEVCALL> : k_verify_trunc<false, false, PROP, DEVCALL>;
    }
    if (bf16) return vec ? k_verify<true, true, PROP, DEVCALL> : k_verify<true, false, PROP, DEVCALL>;
    return vec ? k_verify<false, true, PROP, DEVCALL> : k_verify<false, false, PROP, DEVCALL>;
}

template <bool DEVCALL>
KernelFn pick(bool bf16, bool vec, bool trunc, int prop, bool wide) {
    if (prop == kPropPoint) return pick_prop<kPropPoint, DEVCALL>(bf16, vec, trunc, wide);
    if (prop == kPropStats) return pick_prop<kPropStats, DEVCALL>(bf16, vec, trunc, wide);
    return pick_prop<kPropLogits, DEVCALL>(bf16, vec, trunc, wide);
}

// Launches with at least this many streaming units take k_verify_wide
// (measured: the mixed batch, 36,864 units, 114.5 -> 109.5 us; the serving
// batch, 6,144 units, is 0.5-1 us slower with it).
constexpr long long kWideUnits = 16384;

}  // namespace

hipError_t set_wait_limit_verify(int n) { return set_wait_limit_here(n); }

hipError_t launch_verify(const Args& a, bool bf16, bool vec, bool devcall, hipStream_t stream, hipEvent_t* ev) {
    const long long blocks = (long long)(a.P + 1) * a.B * a.C + (devcall ? 1 : 0);   // + the closing workgroup
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    const bool wide = (long long)a.P * a.B * a.C >= kWideUnits;
    KernelFn fn = devcall ? pick<true>(bf16, vec, a.cand_cap > 0, a.prop, wide)
                          : pick<false>(bf16, vec, a.cand_cap > 0, a.prop, wide);
    // the events (when profiling) are attached to the dispatch itself, so
    // that they time the kernel and not the packets around it
    if (ev)
        hipExtLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(kBlock), 0, stream, ev[0], ev[1], 0, a);
    else
        hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(kBlock), 0, stream, a);   // also under capture
    return hipGetLastError();
}

}  // namespace specv
