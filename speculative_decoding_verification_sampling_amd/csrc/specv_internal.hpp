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
constexpr int kUnitChunks = 4;          // chunks streamed by one workgroup (one "unit")
constexpr int kDecideParts = 512;       // unit statistics a decision stages in LDS at once
constexpr int kMaxChunks = 64;          // V <= 64 * 8192 = 524288
constexpr int kMaxRows = 2 * SPECV_MAX_GAMMA + 1;
constexpr int kCounterStride = 64;     // one arrival counter per 256-byte slot: atomics
                                        // on one cache line serialize across the device
constexpr int kTieSlack = 256;          // candidates per chunk beyond top_k (ties)
constexpr int kKeptCap = 2048;          // kept set per row after the row-level top-k

// Per (row, unit) statistics from the streaming pass.
//  sampling rows: m = max raw logit, s = sum exp2((z - m) * scale)
//  greedy rows:   m = max raw logit, arg = its lowest index
struct Part {
    float m;
    float s;
    int arg;
    unsigned bad;   // 1: NaN / +inf seen
};

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
struct TruncScratch {
    float v[kKeptCap];
    int idx[kKeptCap];
    float w[kKeptCap];
    unsigned hist[256];
    unsigned off[kMaxChunks + 1];
    float red[kBlock / 64];
    int misc[8];
};

// Outcome of one batch row's accept tests, handed from the workgroup that
// decides the row to its sampling workgroups.  Every word holds
// (epoch << 32) | value, written with one 64-bit store, so a reader polls all
// the words it needs at once and knows each is this call's when its epoch
// matches: no separate ready flag, no ordering between the words.
enum DecWord {
    DW_KIND = 0,          // 0: nothing to sample (outputs written); 1: correction; 2: bonus
    DW_POS,               // rejected position, or gamma for the bonus
    DW_U,                 // uniform of the correction / bonus draw (float bits)
    DW_MT, DW_INVT,       // target row max and 1 / sum (exp2 units)
    DW_MQ, DW_INVQ,       // draft row max and 1 / sum (correction only)
    DW_SCALE,             // log2(e) / T
    DW_NEMIT,             // tokens emitted before the sampled one
    DW_NACC,
    DW_FLAGS,
    DW_EMIT,              // emitted tokens, gamma words (-1 past nemit)
};
constexpr int kDecWords = DW_EMIT + SPECV_MAX_GAMMA;
static_assert(kDecWords <= 64, "one wave64 polls the whole record");
struct Dec {
    unsigned long long w[48];
};

struct Workspace {
    Part* part;           // [max_batch * max_rows * max_chunks]
    float* wsum;          // [max_batch * max_chunks * 2]: per chunk (sampling weight, p mass)
    unsigned* counter;    // [max_batch * kCounterStride] arrivals in the streaming kernel
    unsigned* counter2;   // [max_batch * kCounterStride] arrivals in the sampling kernel;
                          // both zero between calls
    Dec* dec;             // [max_batch], zero before the first call
    unsigned* counter1;   // [max_batch * kCounterStride] arrivals of position-0 units
    unsigned* stage1;     // [max_batch * kCounterStride]: 2 * epoch + 1 when the round goes on
                          // past position 0, 2 * epoch when it ended there
    Cand* cand;           // [max_batch * rows * max_chunks * cand_cap] chunk candidates
    Cand* cand_meta;      // [max_batch * rows * max_chunks]: (lower bound L, count); count -1
                          // when the chunk's candidates overflowed
    TruncRow* trow;       // [max_batch * rows]
    Cand* kept;           // [max_batch * rows * kept_cap]
    unsigned* counter_row;// [max_batch * rows * kCounterStride] unit arrivals per truncated row
};

struct Args {
    const void* tgt;
    long long t_sb, t_sp;         // element strides of target rows
    const void* drf;
    long long d_sb, d_sp;
    int B, gamma, V;
    int C;                        // chunks per row
    int U;                        // streaming units per row: ceil(C / kUnitChunks)
    int R;                        // logits rows per batch row: 2 * gamma + 1
    int greedy_all;               // specv_verify_greedy
    int cand_cap;                 // candidates per (row, chunk); 0: no truncation
    int kept_cap;                 // kept-set entries per row: min(kKeptCap, max_vocab)
    int max_top_k;
    const int* tokens;            // [B, gamma]
    const specv_row_params* params;
    const int* caps;              // greedy entry point caps or nullptr
    unsigned long long seed;
    unsigned step;
    int eos;
    unsigned epoch;               // per-handle call number (never 0)
    int* out_acc;
    int* out_tok;
    int* out_emit;
    int* out_flags;
    float* p_at;
    float* q_at;
    float* wres;
    Workspace ws;
};

// Launch the whole verify step on ``stream`` as one kernel (one workgroup per
// streaming unit and per sampling item).  ``bf16`` selects the element type,
// ``vec`` the 16-byte vector-load variant (row starts 16-byte aligned); the
// truncation-capable variant is used when a.cand_cap > 0.  ``ev`` (nullable)
// receives two event records around the launch.
hipError_t launch_verify(const Args& a, bool bf16, bool vec, hipStream_t stream, hipEvent_t* ev);

}  // namespace specv
