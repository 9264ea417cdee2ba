// Internal declarations shared by the libspecv host code and its kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specv.h"

namespace specv {

constexpr int kBlock = 256;             // threads per workgroup (4 wave64)
constexpr int kWave = 64;
constexpr int kWaves = kBlock / kWave;
constexpr int kChunk = 8192;            // vocabulary entries per chunk (32 per thread)
constexpr int kPerThread = kChunk / kBlock;
constexpr int kMaxChunks = 64;          // V <= 64 * 8192 = 524288
constexpr int kMaxPos = SPECV_MAX_GAMMA + 1;   // positions 0 .. gamma (gamma = bonus)
constexpr int kSlot = 64;               // 32-bit words per 256-byte slot: every arrival
                                        // counter has a cache line of its own (atomics on
                                        // one line serialize device-wide)
constexpr int kTieSlack = 256;          // candidates per chunk beyond top_k (ties)
constexpr int kKeptCap = 2048;          // kept set per row after the row-level top-k

struct Cand {
    float v;        // raw logit
    int idx;        // token index
};

// Result of the row-level truncation (top-k then top-p) for one logits row.
// The kept set is {v : z_v >= tstar}, stored sorted (value desc, index asc).
struct TruncRow {
    float zmax;     // largest raw logit
    float tstar;    // raw value of the last kept level
    float S;        // sum over the kept set of exp2((z - zmax) * scale)
    int n_kept;     // entries in Workspace::kept for the row
    unsigned flags; // SPECV_FLAG_* bits found while truncating (overflow, top-p near)
    unsigned bad;   // 1: NaN / +inf in the row, or no finite value
    int pad0, pad1;
};

// LDS scratch of the truncation steps (one per workgroup, reused).
struct alignas(16) TruncScratch {   // 8-byte LDS atomics on v and w
    float v[kKeptCap];
    int idx[kKeptCap];
    float w[kKeptCap];
    int idx2[kKeptCap];
    unsigned hist[256];
    unsigned off[kMaxChunks + 1];
    float red[kBlock / 64];
    int misc[8];
};

// Outcome of one position of one batch row (its "pair": target row k and,
// below gamma, draft row k), published by the workgroup that decided it.
// Every word holds (tag << 32) | value with the launch's tag (never 0), so a
// reader knows a word is this launch's when its tag matches.
enum PairWord {
    PW_STATE = 0,         // outcome | (SPECV_FLAG_* bits << 8)
    PW_P, PW_Q,           // p_k(d_k), q_k(d_k) (float bits)
    PW_ARG,               // target argmax (greedy rows)
    PW_MT, PW_INVT,       // target row max and 1 / sum (exp2 units)
    PW_MQ, PW_INVQ,       // draft row max and 1 / sum
    kPairWords
};
struct PairRec {
    unsigned long long w[kPairWords];
};

// How a sampling row's round ended, for its sampling workgroups: which
// position draws the correction / bonus token, the row's flags so far, and
// that position's normalisers.  Tagged words like PairRec.
enum RowWord {
    RW_REC = 0,           // kind | (position << 3)
    RW_MT, RW_INVT, RW_MQ, RW_INVQ,
    RW_FLAGS,             // the row's flags from the consulted positions (published once
                          // they are gathered, possibly after the words above)
    kRowWords = 8
};

// The records the workgroups of one launch exchange come in two sets, one
// per parity of the call number.  A launch uses its parity's set and clears
// the other set over the extent of the launch that used it last, which the
// next launch then finds zeroed: every word a launch reads is either zero or
// written by that launch.  The call number itself lives on the device, in
// ``calls``, so that launches replayed from a captured graph still advance
// it (the kernels' protocol: specv_rows.hpp, "call number").
struct Workspace {
    unsigned long long* stats;  // [2][max_batch * max_pos * 2 * max_chunks][2]: per (row,
                                // chunk) tagged (max, sum) or (max, argmax)
    PairRec* pair;              // [2][max_batch * max_pos]
    unsigned long long* rowrec; // [2][max_batch * kRowWords]
    unsigned long long* wsum;   // [2][max_batch * max_chunks * 2]: chunk sampling weight, p mass
    unsigned* ctr;              // [2][max_batch * max_pos][kSlot]: arrivals per pair
    unsigned long long* status; // [2][max_batch][kSlot / 2]: per-row accept / stop bits
    long long set_stats;        // words in one set of stats
    long long set_pair;         // records in one set of pair
    long long set_rowrec;       // words in one set of rowrec
    long long set_wsum;         // words in one set of wsum
    unsigned* calls;            // [kSlot]: word 0 is the call number of the next launch
    unsigned* seen;             // [2][max_batch][kSlot]: per parity and batch row, workgroups
                                // of the running launch that have read the call number
    unsigned long long* dims;   // [2] (16-byte aligned, in a slot of its own): per parity,
                                // the extent (B, positions, chunks) of the last launch of
                                // that parity
    int n_groups;               // max_batch * max_pos
    int n_rows;                 // max_batch
    Cand* cand;                 // [max_batch * max_pos * 2 * max_chunks * cand_cap]
    Cand* cand_meta;            // [max_batch * max_pos * 2 * max_chunks]: (bound L, count);
                                // count -1 when the chunk's candidates overflowed
    TruncRow* trow;             // [max_batch * max_pos * 2]
    Cand* kept;                 // [max_batch * max_pos * 2 * kept_cap]
};

struct Args {
    const void* tgt;
    long long t_sb, t_sp;         // element strides of target rows
    const void* drf;
    long long d_sb, d_sp;
    int B, gamma, V;
    int C;                        // chunks per row
    int P;                        // positions per batch row: gamma + 1
    int greedy_all;               // specv_verify_greedy
    int prop;                     // the proposal: 0 draft logits; 1 (specv_verify_point_mass)
                                  // q_i is the point mass on d_i and no draft logits are read;
                                  // 2 (specv_verify_sample_qstats) draft logits plus the
                                  // drafter's row statistics
    const specv_draft_stats* qstats;  // prop 2: [B][qs_sb] statistics of draft row (b, i)
    long long qs_sb;
    int cand_cap;                 // candidates per (row, chunk); 0: no truncation
    int kept_cap;                 // kept-set entries per row: min(kKeptCap, max_vocab)
    int max_top_k;
    const int* tokens;            // [B, gamma]
    const specv_row_params* params;
    const int* caps;              // greedy entry point caps or nullptr
    unsigned long long seed;
    unsigned step;
    int eos;
    unsigned epoch;               // the launch's tag, set on the device from the call number
                                  // (the host leaves it 0)
    int* out_acc;
    int* out_tok;
    int* out_emit;
    int* out_flags;
    float* p_at;
    float* q_at;
    float* wres;
    Workspace ws;
};

// The draft-side sampler (specv_sample_draft): draws positions pos0 ..
// pos0 + n - 1 of B batch rows.
struct DraftArgs {
    const void* drf;
    long long d_sb, d_sp;         // element strides of draft rows: row (b, i) is position pos0 + i
    int B, n, V;
    int C;                        // chunks per row
    int pos0;
    long long out_stride;         // entries per batch row of the outputs
    const specv_row_params* params;
    unsigned long long seed;
    unsigned step;
    unsigned epoch;               // the launch's tag, set on the device (as Args::epoch)
    int* out_tok;                 // [B][out_stride]
    specv_draft_stats* out_stats; // [B][out_stride] or nullptr
    Workspace ws;                 // the handle's: chunk statistics and, for truncated rows,
                                  // candidates and kept lists of draft row (b, i) = side 1 of
                                  // pair (b, i) with n positions per batch row
    int cand_cap, kept_cap, max_top_k;
};

hipError_t launch_sample_draft(const DraftArgs& a, bool bf16, bool vec, bool devcall, hipStream_t stream,
                               hipEvent_t* ev);

// Launch the whole verify step on ``stream`` as one kernel: one streaming
// workgroup per (position, batch row, chunk), position-major, then one
// sampling workgroup per (batch row, chunk).  ``bf16`` selects the element
// type, ``vec`` the 16-byte vector-load variant (row starts 16-byte aligned);
// the truncation-capable variant is used when a.cand_cap > 0.  ``ev``
// (nullable) holds two events that the launch records at the kernel's start
// and end.
hipError_t launch_verify(const Args& a, bool bf16, bool vec, bool devcall, hipStream_t stream, hipEvent_t* ev);
// The bounded waits' poll limit in the verify and draft kernels (failure-path tests).
constexpr int kDefaultWaitLimit = 1 << 18;
hipError_t set_wait_limit_verify(int n);
hipError_t set_wait_limit_draft(int n);

// The sizes a workspace is laid out for, and its truncation capacity.
struct Limits {
    int max_batch, max_gamma, max_vocab, max_top_k;
    int cand_cap;                 // candidates per (row, chunk); 0: no truncation workspace
    int kept_cap;
};

// Checks the arguments of a stochastic verify call against ``lim`` (prop:
// kPropLogits draft logits, kPropPoint point-mass drafts, kPropStats the
// drafter's statistics) and packs them into *out, all but the workspace and
// the epoch; *out_vec tells whether every row start allows 16-byte loads.
// Returns the status the entry point reports; with B == 0 there is nothing
// to launch.
specv_status verify_sampling_args(const Limits& lim, const void* target_logits, int64_t t_stride_b,
                                  int64_t t_stride_pos, const void* draft_logits, int64_t d_stride_b,
                                  int64_t d_stride_pos, const specv_draft_stats* draft_stats,
                                  int64_t s_stride_b, specv_dtype dtype, int B, int gamma, int V,
                                  const int32_t* draft_tokens, const specv_row_params* row_params,
                                  uint64_t seed, uint32_t step, int32_t eos_id,
                                  int32_t* out_num_accepted, int32_t* out_tokens,
                                  int32_t* out_num_emitted, int32_t* out_row_flags,
                                  const specv_diag* diag, int prop, Args* out, bool* out_vec);

// A plain streaming read of n16 16-byte words (measurement aid): ``grid``
// workgroups, each folding its share into one word of sink[grid].
hipError_t launch_read_ceiling(const void* buf, long long n16, int grid, unsigned* sink,
                               hipStream_t stream);

}  // namespace specv
