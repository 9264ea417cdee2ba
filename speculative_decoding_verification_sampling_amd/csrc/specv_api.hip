// libspecv C ABI: argument validation, workspace ownership, launches.
//
// Every argument error is returned before anything is enqueued.  Calls are
// asynchronous on the caller's stream and allocate nothing: the workspace is
// allocated once in specv_create, sized from the handle's maxima.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <new>
#include <vector>

#include "specv.h"
#include "specv_internal.hpp"

struct specv_ctx {
    specv_config cfg;
    int max_chunks;
    int cand_cap;      // candidates per (row, chunk); 0 without truncation support
    int kept_cap;      // kept-set entries per row
    // The exchange records, in two forms.  Eager calls use ``ws``: the host
    // numbers them (``epoch``), tagged records in one set, counters and
    // status words in two sets by parity.  Calls made while the stream is
    // being captured into a graph use ``ws_dev``: the launch takes its number
    // on the device (every replay a new one), all records in two sets.  The
    // truncation storage (written before it is read within each launch) is
    // shared.
    specv::Workspace ws;
    specv::Workspace ws_dev;
    unsigned epoch = 0;             // the host's call number (eager calls)
    // profiling: a ring of event triples, drained by specv_get_profile or
    // when the ring wraps
    bool prof = false;
    std::vector<hipEvent_t> ev;     // 2 * kProfRing
    std::vector<char> ev_live;      // kProfRing
    size_t ev_next = 0;
    int prof_calls = 0;
    double ms_kernel = 0.0;
    std::vector<float> samples;     // per-call kernel milliseconds since the last reset
};

namespace {
constexpr size_t kProfRing = 512;
constexpr size_t kMaxSamples = 1 << 16;

hipError_t drain_slot(specv_ctx* h, size_t slot) {
    if (!h->ev_live[slot]) return hipSuccess;
    hipEvent_t* e = &h->ev[2 * slot];
    hipError_t err = hipEventSynchronize(e[1]);
    if (err != hipSuccess) return err;
    float ms = 0.f;
    err = hipEventElapsedTime(&ms, e[0], e[1]);
    if (err != hipSuccess) return err;
    h->ms_kernel += ms;
    h->prof_calls += 1;
    if (h->samples.size() < kMaxSamples) h->samples.push_back(ms);
    h->ev_live[slot] = 0;
    return hipSuccess;
}

// Event triple for the next call, or nullptr when profiling is off.
hipEvent_t* next_events(specv_ctx* h) {
    if (!h->prof) return nullptr;
    const size_t slot = h->ev_next % kProfRing;
    if (drain_slot(h, slot) != hipSuccess) return nullptr;
    h->ev_next++;
    h->ev_live[slot] = 1;
    return &h->ev[2 * slot];
}
}  // namespace

namespace {

template <typename T>
hipError_t alloc(T** p, size_t count) {
    *p = nullptr;
    return hipMalloc(reinterpret_cast<void**>(p), count * sizeof(T) + 256);
}

// The records of one workspace form (not the shared truncation storage).
void free_records(specv::Workspace& ws) {
    if (ws.stats) (void)hipFree(ws.stats);
    if (ws.pair) (void)hipFree(ws.pair);
    if (ws.rowrec) (void)hipFree(ws.rowrec);
    if (ws.status) (void)hipFree(ws.status);
    if (ws.wsum) (void)hipFree(ws.wsum);
    if (ws.ctr) (void)hipFree(ws.ctr);
    if (ws.calls) (void)hipFree(ws.calls);
    if (ws.seen) (void)hipFree(ws.seen);
    if (ws.dims) (void)hipFree(ws.dims);
}

void free_ws(specv_ctx* h) {
    free_records(h->ws);
    free_records(h->ws_dev);
    specv::Workspace& ws = h->ws;
    if (ws.cand) (void)hipFree(ws.cand);
    if (ws.cand_meta) (void)hipFree(ws.cand_meta);
    if (ws.trow) (void)hipFree(ws.trow);
    if (ws.kept) (void)hipFree(ws.kept);
    h->ws = specv::Workspace{};
    h->ws_dev = specv::Workspace{};
}

// Allocates the records of one workspace form: ``sets`` sets of the tagged
// records (1: host-numbered, 2: device-numbered), two sets of counters and
// status words, and (device-numbered) the call number's words.
bool alloc_records(specv::Workspace& ws, const specv_config* cfg, int max_chunks, int sets) {
    const size_t groups = (size_t)cfg->max_batch * (cfg->max_gamma + 1);
    ws.n_groups = (int)groups;
    ws.n_rows = cfg->max_batch;
    const long long n_stats = (long long)groups * 2 * max_chunks * 2;
    const long long n_pair = (long long)groups;
    const long long n_rowrec = (long long)cfg->max_batch * specv::kRowWords;
    const long long n_wsum = (long long)cfg->max_batch * max_chunks * 2;
    // the kernels address set p at base + p * set size: one set means size 0
    ws.set_stats = sets == 2 ? n_stats : 0;
    ws.set_pair = sets == 2 ? n_pair : 0;
    ws.set_rowrec = sets == 2 ? n_rowrec : 0;
    ws.set_wsum = sets == 2 ? n_wsum : 0;
    bool ok = alloc(&ws.stats, sets * (size_t)n_stats) == hipSuccess &&
              alloc(&ws.pair, sets * (size_t)n_pair) == hipSuccess &&
              alloc(&ws.rowrec, sets * (size_t)n_rowrec) == hipSuccess &&
              alloc(&ws.wsum, sets * (size_t)n_wsum) == hipSuccess &&
              alloc(&ws.ctr, 2 * groups * specv::kSlot) == hipSuccess &&
              alloc(&ws.status, (size_t)2 * cfg->max_batch * (specv::kSlot / 2)) == hipSuccess;
    if (ok && sets == 2)
        ok = alloc(&ws.calls, (size_t)specv::kSlot) == hipSuccess &&
             alloc(&ws.seen, (size_t)2 * cfg->max_batch * specv::kSlot) == hipSuccess &&
             alloc(&ws.dims, (size_t)specv::kSlot) == hipSuccess;
    return ok;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Validation shared by the verify entry points, against the sizes a
// workspace was laid out for.
specv_status check_common(const specv::Limits& lim, const void* target, int64_t t_sb, int64_t t_sp,
                          specv_dtype dtype, int B, int gamma, int V, const int32_t* tokens,
                          int32_t* out_acc, int32_t* out_tok, int32_t* out_emit,
                          int32_t* out_flags) {
    if (dtype != SPECV_F32 && dtype != SPECV_BF16) return SPECV_E_DTYPE;
    if (B < 0 || gamma < 0 || gamma > SPECV_MAX_GAMMA || V < 1) return SPECV_E_SHAPE;
    if (t_sb < 0 || t_sp < 0) return SPECV_E_SHAPE;
    if (B > lim.max_batch || gamma > lim.max_gamma || V > lim.max_vocab) return SPECV_E_CAPACITY;
    if (B == 0) return SPECV_OK;
    if (!target || !out_acc || !out_tok || !out_emit) return SPECV_E_NULL;
    if (gamma > 0 && !tokens) return SPECV_E_NULL;
    const size_t es = dtype == SPECV_BF16 ? 2 : 4;
    if (!aligned(target, es)) return SPECV_E_ALIGN;
    if (!aligned(out_acc, 4) || !aligned(out_tok, 4) || !aligned(out_emit, 4) ||
        (out_flags && !aligned(out_flags, 4)) || (tokens && !aligned(tokens, 4)))
        return SPECV_E_ALIGN;
    return SPECV_OK;
}

specv::Limits handle_limits(specv_handle h) {
    specv::Limits l;
    l.max_batch = h->cfg.max_batch;
    l.max_gamma = h->cfg.max_gamma;
    l.max_vocab = h->cfg.max_vocab;
    l.max_top_k = h->cfg.max_top_k;
    l.cand_cap = h->cand_cap;
    l.kept_cap = h->kept_cap;
    return l;
}

bool rows_vec_aligned(const void* base, int64_t sb, int64_t sp, size_t es) {
    return aligned(base, 16) && ((sb * (int64_t)es) % 16) == 0 && ((sp * (int64_t)es) % 16) == 0;
}

specv::Args base_args(const specv::Limits& lim, int B, int gamma, int V) {
    specv::Args a{};
    a.B = B;
    a.gamma = gamma;
    a.V = V;
    a.C = (V + specv::kChunk - 1) / specv::kChunk;
    a.P = gamma + 1;
    a.cand_cap = lim.cand_cap;
    a.kept_cap = lim.kept_cap;
    a.max_top_k = lim.max_top_k;
    return a;
}

// Zero the records of one workspace form.  Fresh allocations may hold
// anything, another handle's tagged words included.
hipError_t clear_records(const specv::Workspace& ws, const specv_config& cfg, int max_chunks, hipStream_t stream) {
    const size_t groups = (size_t)cfg.max_batch * (cfg.max_gamma + 1);
    const size_t rows = (size_t)cfg.max_batch;
    const int sets = ws.set_stats ? 2 : 1;
    hipError_t e = hipMemsetAsync(ws.stats, 0, sets * groups * 2 * max_chunks * 2 * sizeof(unsigned long long), stream);
    if (e == hipSuccess) e = hipMemsetAsync(ws.pair, 0, sets * groups * sizeof(specv::PairRec), stream);
    if (e == hipSuccess)
        e = hipMemsetAsync(ws.rowrec, 0, sets * rows * specv::kRowWords * sizeof(unsigned long long), stream);
    if (e == hipSuccess)
        e = hipMemsetAsync(ws.wsum, 0, sets * rows * max_chunks * 2 * sizeof(unsigned long long), stream);
    if (e == hipSuccess) e = hipMemsetAsync(ws.ctr, 0, 2 * groups * specv::kSlot * sizeof(unsigned), stream);
    if (e == hipSuccess)
        e = hipMemsetAsync(ws.status, 0, 2 * rows * specv::kSlot * sizeof(unsigned), stream);
    if (e == hipSuccess && ws.calls) e = hipMemsetAsync(ws.calls, 0, specv::kSlot * sizeof(unsigned), stream);
    if (e == hipSuccess && ws.seen) e = hipMemsetAsync(ws.seen, 0, 2 * rows * specv::kSlot * sizeof(unsigned), stream);
    if (e == hipSuccess && ws.dims) e = hipMemsetAsync(ws.dims, 0, 2 * specv::kSlot * sizeof(unsigned), stream);
    return e;
}

// The host's number of the next eager call, clearing the eager records
// first when the tags would repeat.  Verify calls advance it by 1: a verify
// call clears the counters and status words of the other parity for the
// next one, so consecutive verify calls must alternate parity.  Sampler
// calls touch no counters or status words and advance it by 2, keeping the
// parity the next verify call expects; they share the tagged chunk
// statistics with verify calls, so every call's tag is distinct.
bool next_epoch(specv_handle h, hipStream_t s, unsigned step, unsigned* out) {
    unsigned next = h->epoch + step;
    if (next >= 0x7fffffffu) {
        if (clear_records(h->ws, h->cfg, h->max_chunks, s) != hipSuccess) return false;
        next = step;
    }
    *out = next;
    return true;
}

// True while ``s`` is being captured into a graph: such a call takes its
// number on the device, so that each replay of it gets a new one.
bool capturing(hipStream_t s) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(s, &st) == hipSuccess && st == hipStreamCaptureStatusActive;
}

// One launch of the verify kernel: numbered by the host (eager; the number
// advances only when the launch succeeded) or, under capture, on the device.
specv_status launch(specv_handle h, specv::Args& a, bool bf16, bool vec, void* stream) {
    if (hipSetDevice(h->cfg.device) != hipSuccess) return SPECV_E_HIP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (capturing(s)) {
        a.ws = h->ws_dev;
        a.epoch = 0;
        return specv::launch_verify(a, bf16, vec, true, s, nullptr) == hipSuccess ? SPECV_OK : SPECV_E_HIP;
    }
    unsigned next;
    if (!next_epoch(h, s, 1, &next)) return SPECV_E_HIP;
    a.ws = h->ws;
    a.epoch = next;
    if (specv::launch_verify(a, bf16, vec, false, s, next_events(h)) != hipSuccess) return SPECV_E_HIP;
    h->epoch = next;
    return SPECV_OK;
}

}  // namespace

extern "C" {

const char* specv_status_string(specv_status s) {
    switch (s) {
        case SPECV_OK: return "ok";
        case SPECV_E_NULL: return "null pointer argument";
        case SPECV_E_SHAPE: return "invalid shape or stride";
        case SPECV_E_DTYPE: return "unsupported dtype";
        case SPECV_E_ALIGN: return "misaligned pointer";
        case SPECV_E_CAPACITY: return "size above the handle's configured maximum";
        case SPECV_E_PARAM: return "invalid configuration";
        case SPECV_E_NOMEM: return "device allocation failed";
        case SPECV_E_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

specv_status specv_create(const specv_config* cfg, specv_handle* out) {
    if (!cfg || !out) return SPECV_E_NULL;
    if (cfg->max_batch < 1 || cfg->max_gamma < 0 || cfg->max_gamma > SPECV_MAX_GAMMA ||
        cfg->max_vocab < 1 || cfg->max_vocab > SPECV_MAX_VOCAB || cfg->max_top_k < 0 ||
        cfg->max_top_k > SPECV_MAX_TOP_K)
        return SPECV_E_PARAM;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || cfg->device < 0 || cfg->device >= ndev)
        return SPECV_E_PARAM;
    if (hipSetDevice(cfg->device) != hipSuccess) return SPECV_E_HIP;

    specv_ctx* h = new (std::nothrow) specv_ctx{};
    if (!h) return SPECV_E_NOMEM;
    h->cfg = *cfg;
    h->max_chunks = (cfg->max_vocab + specv::kChunk - 1) / specv::kChunk;
    h->cand_cap = cfg->max_top_k > 0 ? 2 * cfg->max_top_k + specv::kTieSlack : 0;
    h->cand_cap = std::min(h->cand_cap, std::min(specv::kChunk, cfg->max_vocab));
    h->kept_cap = std::min(specv::kKeptCap, cfg->max_vocab);
    const size_t groups = (size_t)cfg->max_batch * (cfg->max_gamma + 1);   // (b, position) pairs
    const size_t rows = groups * 2;                                         // logits rows
    const size_t rc = rows * h->max_chunks;
    specv::Workspace& ws = h->ws;
    bool ok = alloc_records(h->ws, cfg, h->max_chunks, 1) && alloc_records(h->ws_dev, cfg, h->max_chunks, 2);
    // candidate storage for truncated rows, reserved only when asked for
    if (ok && h->cand_cap > 0)
        ok = alloc(&ws.cand, rc * h->cand_cap) == hipSuccess &&
             alloc(&ws.cand_meta, rc) == hipSuccess && alloc(&ws.trow, rows) == hipSuccess &&
             alloc(&ws.kept, rows * h->kept_cap) == hipSuccess;
    h->ws_dev.cand = ws.cand;
    h->ws_dev.cand_meta = ws.cand_meta;
    h->ws_dev.trow = ws.trow;
    h->ws_dev.kept = ws.kept;
    if (ok) ok = clear_records(h->ws, *cfg, h->max_chunks, nullptr) == hipSuccess &&
                 clear_records(h->ws_dev, *cfg, h->max_chunks, nullptr) == hipSuccess;
    if (ok) ok = hipDeviceSynchronize() == hipSuccess;
    if (!ok) {
        free_ws(h);
        delete h;
        (void)hipGetLastError();
        return SPECV_E_NOMEM;
    }
    *out = h;
    return SPECV_OK;
}

specv_status specv_set_profiling(specv_handle h, int enable) {
    if (!h) return SPECV_E_NULL;
    if (enable && h->ev.empty()) {
        if (hipSetDevice(h->cfg.device) != hipSuccess) return SPECV_E_HIP;
        h->ev.assign(2 * kProfRing, nullptr);
        h->ev_live.assign(kProfRing, 0);
        for (auto& e : h->ev)
            if (hipEventCreate(&e) != hipSuccess) return SPECV_E_HIP;
    }
    h->prof = enable != 0;
    return SPECV_OK;
}

specv_status specv_get_profile(specv_handle h, int reset, int* calls, double* ms_kernel) {
    if (!h) return SPECV_E_NULL;
    for (size_t s = 0; s < h->ev_live.size(); ++s)
        if (drain_slot(h, s) != hipSuccess) return SPECV_E_HIP;
    if (calls) *calls = h->prof_calls;
    if (ms_kernel) *ms_kernel = h->ms_kernel;
    if (reset) {
        h->prof_calls = 0;
        h->ms_kernel = 0.0;
        h->samples.clear();
    }
    return SPECV_OK;
}

specv_status specv_get_profile_samples(specv_handle h, int max_samples, float* ms_out, int* n_out) {
    if (!h || !n_out || (max_samples > 0 && !ms_out)) return SPECV_E_NULL;
    for (size_t s = 0; s < h->ev_live.size(); ++s)
        if (drain_slot(h, s) != hipSuccess) return SPECV_E_HIP;
    const int n = (int)std::min<size_t>(h->samples.size(), (size_t)std::max(max_samples, 0));
    for (int i = 0; i < n; ++i) ms_out[i] = h->samples[i];
    *n_out = n;
    return SPECV_OK;
}

specv_status specv_read_ceiling(void* stream, const void* buf, int64_t bytes, int grid, uint32_t* sink) {
    if (!buf || !sink) return SPECV_E_NULL;
    if (bytes < 16 || (bytes % 16) != 0 || grid < 1) return SPECV_E_SHAPE;
    if ((reinterpret_cast<uintptr_t>(buf) % 16) != 0 || (reinterpret_cast<uintptr_t>(sink) % 4) != 0)
        return SPECV_E_ALIGN;
    if (specv::launch_read_ceiling(buf, bytes / 16, grid, sink, static_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return SPECV_E_HIP;
    return SPECV_OK;
}

specv_status specv_debug_set_wait_limit(int device, int32_t polls) {
    if (polls < 0) return SPECV_E_PARAM;
    const int n = polls == 0 ? specv::kDefaultWaitLimit : polls;
    if (hipSetDevice(device) != hipSuccess) return SPECV_E_HIP;
    if (hipDeviceSynchronize() != hipSuccess) return SPECV_E_HIP;
    if (specv::set_wait_limit_verify(n) != hipSuccess || specv::set_wait_limit_draft(n) != hipSuccess)
        return SPECV_E_HIP;
    return SPECV_OK;
}

specv_status specv_destroy(specv_handle h) {
    if (!h) return SPECV_OK;
    (void)hipSetDevice(h->cfg.device);
    (void)hipDeviceSynchronize();
    for (auto& e : h->ev)
        if (e) (void)hipEventDestroy(e);
    free_ws(h);
    delete h;
    return SPECV_OK;
}

}  // extern "C"

namespace specv {

// Stochastic verification.  prop: 0 draft logits (specv_verify_sample);
// 1 no draft logits, q_i is the point mass on d_i (specv_verify_point_mass);
// 2 draft logits plus the drafter's row statistics (specv_verify_sample_qstats).
specv_status verify_sampling_args(const specv::Limits& lim, const void* target_logits,
                             int64_t t_stride_b, int64_t t_stride_pos, const void* draft_logits,
                             int64_t d_stride_b, int64_t d_stride_pos,
                             const specv_draft_stats* draft_stats,
                             int64_t s_stride_b, specv_dtype dtype, int B, int gamma, int V,
                             const int32_t* draft_tokens, const specv_row_params* row_params,
                             uint64_t seed, uint32_t step, int32_t eos_id, int32_t* out_num_accepted,
                             int32_t* out_tokens, int32_t* out_num_emitted, int32_t* out_row_flags,
                             const specv_diag* diag, int prop, specv::Args* out, bool* out_vec) {
    const bool point_mass = prop == 1;
    specv_status st = check_common(lim, target_logits, t_stride_b, t_stride_pos, dtype, B, gamma, V,
                                   draft_tokens, out_num_accepted, out_tokens, out_num_emitted,
                                   out_row_flags);
    if (st != SPECV_OK || B == 0) return st;
    if (!row_params) return SPECV_E_NULL;
    const size_t es = dtype == SPECV_BF16 ? 2 : 4;
    if (!point_mass) {
        if (gamma > 0 && !draft_logits) return SPECV_E_NULL;
        if (d_stride_b < 0 || d_stride_pos < 0) return SPECV_E_SHAPE;
        if (gamma > 0 && !aligned(draft_logits, es)) return SPECV_E_ALIGN;
    }
    if (prop == 2 && gamma > 0) {
        if (!draft_stats) return SPECV_E_NULL;
        if (s_stride_b < gamma) return SPECV_E_SHAPE;
        if (!aligned(draft_stats, 16)) return SPECV_E_ALIGN;
    }
    if (!aligned(row_params, 16)) return SPECV_E_ALIGN;
    if (diag && ((diag->p_at_draft && !aligned(diag->p_at_draft, 4)) ||
                 (diag->q_at_draft && !aligned(diag->q_at_draft, 4)) ||
                 (diag->residual_sum && !aligned(diag->residual_sum, 4))))
        return SPECV_E_ALIGN;

    specv::Args a = base_args(lim, B, gamma, V);
    a.tgt = target_logits;
    a.t_sb = t_stride_b;
    a.t_sp = t_stride_pos;
    a.drf = point_mass ? nullptr : draft_logits;
    a.d_sb = point_mass ? 0 : d_stride_b;
    a.d_sp = point_mass ? 0 : d_stride_pos;
    a.greedy_all = 0;
    a.prop = prop;
    a.qstats = prop == 2 ? draft_stats : nullptr;
    a.qs_sb = prop == 2 ? s_stride_b : 0;
    a.tokens = draft_tokens;
    a.params = row_params;
    a.caps = nullptr;
    a.seed = seed;
    a.step = step;
    a.eos = eos_id;
    a.out_acc = out_num_accepted;
    a.out_tok = out_tokens;
    a.out_emit = out_num_emitted;
    a.out_flags = out_row_flags;
    a.p_at = diag ? diag->p_at_draft : nullptr;
    a.q_at = diag ? diag->q_at_draft : nullptr;
    a.wres = diag ? diag->residual_sum : nullptr;
    *out_vec = rows_vec_aligned(target_logits, t_stride_b, t_stride_pos, es) &&
               (point_mass || gamma == 0 || rows_vec_aligned(draft_logits, d_stride_b, d_stride_pos, es));
    *out = a;
    return SPECV_OK;
}

}  // namespace specv

namespace {

specv_status verify_sampling(specv_handle h, void* stream, const void* target_logits,
                             int64_t t_stride_b, int64_t t_stride_pos, const void* draft_logits,
                             int64_t d_stride_b, int64_t d_stride_pos,
                             const specv_draft_stats* draft_stats,
                             int64_t s_stride_b, specv_dtype dtype, int B, int gamma, int V,
                             const int32_t* draft_tokens, const specv_row_params* row_params,
                             uint64_t seed, uint32_t step, int32_t eos_id, int32_t* out_num_accepted,
                             int32_t* out_tokens, int32_t* out_num_emitted, int32_t* out_row_flags,
                             const specv_diag* diag, int prop) {
    if (!h) return SPECV_E_NULL;
    specv::Args a;
    bool vec = false;
    const specv_status st = verify_sampling_args(
        handle_limits(h), target_logits, t_stride_b, t_stride_pos, draft_logits, d_stride_b, d_stride_pos,
        draft_stats, s_stride_b, dtype, B, gamma, V, draft_tokens, row_params, seed, step, eos_id,
        out_num_accepted, out_tokens, out_num_emitted, out_row_flags, diag, prop, &a, &vec);
    if (st != SPECV_OK || B == 0) return st;
    a.ws = h->ws;
    return launch(h, a, dtype == SPECV_BF16, vec, stream);
}

}  // namespace

extern "C" {

specv_status specv_verify_sample(specv_handle h, void* stream, const void* target_logits,
                                 int64_t t_stride_b, int64_t t_stride_pos, const void* draft_logits,
                                 int64_t d_stride_b, int64_t d_stride_pos, specv_dtype dtype, int B,
                                 int gamma, int V, const int32_t* draft_tokens,
                                 const specv_row_params* row_params, uint64_t seed, uint32_t step,
                                 int32_t eos_id, int32_t* out_num_accepted, int32_t* out_tokens,
                                 int32_t* out_num_emitted, int32_t* out_row_flags,
                                 const specv_diag* diag) {
    return verify_sampling(h, stream, target_logits, t_stride_b, t_stride_pos, draft_logits, d_stride_b,
                           d_stride_pos, nullptr, 0, dtype, B, gamma, V, draft_tokens, row_params, seed,
                           step, eos_id, out_num_accepted, out_tokens, out_num_emitted, out_row_flags,
                           diag, 0);
}

specv_status specv_verify_sample_qstats(specv_handle h, void* stream, const void* target_logits,
                                        int64_t t_stride_b, int64_t t_stride_pos,
                                        const void* draft_logits, int64_t d_stride_b,
                                        int64_t d_stride_pos, const specv_draft_stats* draft_stats,
                                        int64_t s_stride_b, specv_dtype dtype, int B, int gamma, int V,
                                        const int32_t* draft_tokens,
                                        const specv_row_params* row_params, uint64_t seed,
                                        uint32_t step, int32_t eos_id, int32_t* out_num_accepted,
                                        int32_t* out_tokens, int32_t* out_num_emitted,
                                        int32_t* out_row_flags, const specv_diag* diag) {
    return verify_sampling(h, stream, target_logits, t_stride_b, t_stride_pos, draft_logits, d_stride_b,
                           d_stride_pos, draft_stats, s_stride_b, dtype, B, gamma, V, draft_tokens,
                           row_params, seed, step, eos_id, out_num_accepted, out_tokens, out_num_emitted,
                           out_row_flags, diag, 2);
}

specv_status specv_verify_point_mass(specv_handle h, void* stream, const void* target_logits,
                                     int64_t t_stride_b, int64_t t_stride_pos, specv_dtype dtype, int B,
                                     int gamma, int V, const int32_t* draft_tokens,
                                     const specv_row_params* row_params, uint64_t seed, uint32_t step,
                                     int32_t eos_id, int32_t* out_num_accepted, int32_t* out_tokens,
                                     int32_t* out_num_emitted, int32_t* out_row_flags,
                                     const specv_diag* diag) {
    return verify_sampling(h, stream, target_logits, t_stride_b, t_stride_pos, nullptr, 0, 0, nullptr, 0,
                           dtype, B, gamma, V, draft_tokens, row_params, seed, step, eos_id,
                           out_num_accepted, out_tokens, out_num_emitted, out_row_flags, diag, 1);
}

specv_status specv_sample_draft(specv_handle h, void* stream, const void* draft_logits,
                                int64_t d_stride_b, int64_t d_stride_pos, specv_dtype dtype, int B,
                                int n_pos, int V, int pos0, const specv_row_params* row_params,
                                uint64_t seed, uint32_t step, int32_t* out_tokens,
                                specv_draft_stats* out_stats, int64_t out_stride) {
    if (!h) return SPECV_E_NULL;
    if (dtype != SPECV_F32 && dtype != SPECV_BF16) return SPECV_E_DTYPE;
    if (B < 0 || n_pos < 0 || V < 1 || pos0 < 0 || d_stride_b < 0 || d_stride_pos < 0)
        return SPECV_E_SHAPE;
    if (out_stride < (int64_t)pos0 + n_pos) return SPECV_E_SHAPE;
    if (B > h->cfg.max_batch || n_pos > std::max(h->cfg.max_gamma, 1) || V > h->cfg.max_vocab)
        return SPECV_E_CAPACITY;
    if (B == 0 || n_pos == 0) return SPECV_OK;
    if (!draft_logits || !row_params || !out_tokens) return SPECV_E_NULL;
    const size_t es = dtype == SPECV_BF16 ? 2 : 4;
    if (!aligned(draft_logits, es) || !aligned(row_params, 16) || !aligned(out_tokens, 4) ||
        (out_stats && !aligned(out_stats, 16)))
        return SPECV_E_ALIGN;
    if (hipSetDevice(h->cfg.device) != hipSuccess) return SPECV_E_HIP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    specv::DraftArgs a{};
    a.drf = draft_logits;
    a.d_sb = d_stride_b;
    a.d_sp = d_stride_pos;
    a.B = B;
    a.n = n_pos;
    a.V = V;
    a.C = (V + specv::kChunk - 1) / specv::kChunk;
    a.pos0 = pos0;
    a.out_stride = out_stride;
    a.params = row_params;
    a.seed = seed;
    a.step = step;
    a.out_tok = out_tokens;
    a.out_stats = out_stats;
    a.ws = h->ws;
    a.cand_cap = h->cand_cap;
    a.kept_cap = h->kept_cap;
    a.max_top_k = h->cfg.max_top_k;
    const bool vec = rows_vec_aligned(draft_logits, d_stride_b, d_stride_pos, es);
    if (capturing(s)) {
        a.ws = h->ws_dev;
        a.epoch = 0;
        return specv::launch_sample_draft(a, dtype == SPECV_BF16, vec, true, s, nullptr) == hipSuccess
                   ? SPECV_OK
                   : SPECV_E_HIP;
    }
    unsigned next;
    if (!next_epoch(h, s, 2, &next)) return SPECV_E_HIP;
    a.epoch = next;
    if (specv::launch_sample_draft(a, dtype == SPECV_BF16, vec, false, s, next_events(h)) != hipSuccess)
        return SPECV_E_HIP;
    h->epoch = next;
    return SPECV_OK;
}

specv_status specv_verify_greedy(specv_handle h, void* stream, const void* target_logits,
                                 int64_t t_stride_b, int64_t t_stride_pos, specv_dtype dtype, int B,
                                 int gamma, int V, const int32_t* draft_tokens,
                                 const int32_t* max_new_tokens, int32_t eos_id,
                                 int32_t* out_num_accepted, int32_t* out_tokens,
                                 int32_t* out_num_emitted, int32_t* out_row_flags) {
    if (!h) return SPECV_E_NULL;
    const specv::Limits lim = handle_limits(h);
    specv_status st = check_common(lim, target_logits, t_stride_b, t_stride_pos, dtype, B, gamma, V,
                                   draft_tokens, out_num_accepted, out_tokens, out_num_emitted,
                                   out_row_flags);
    if (st != SPECV_OK || B == 0) return st;
    if (max_new_tokens && !aligned(max_new_tokens, 4)) return SPECV_E_ALIGN;
    const size_t es = dtype == SPECV_BF16 ? 2 : 4;
    specv::Args a = base_args(lim, B, gamma, V);
    a.ws = h->ws;
    a.tgt = target_logits;
    a.t_sb = t_stride_b;
    a.t_sp = t_stride_pos;
    a.drf = nullptr;
    a.greedy_all = 1;
    a.tokens = draft_tokens;
    a.params = nullptr;
    a.caps = max_new_tokens;
    a.eos = eos_id;
    a.out_acc = out_num_accepted;
    a.out_tok = out_tokens;
    a.out_emit = out_num_emitted;
    a.out_flags = out_row_flags;
    const bool vec = rows_vec_aligned(target_logits, t_stride_b, t_stride_pos, es);
    return launch(h, a, dtype == SPECV_BF16, vec, stream);
}

}  // extern "C"
