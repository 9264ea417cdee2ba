// specv_verify_sample_noalloc: specv_verify_sample for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  The records the verify kernels exchange
// live in one file-scope device array, ``scratch``, laid out for calls of at
// most kNaBatch rows, kNaGamma drafts and kNaVocab vocabulary entries;
// nothing is allocated, ever.
//
// Each device the library runs on holds its own copy of the array until the
// process ends.  Its address is taken once per device, with that device
// current, by hipGetSymbolAddress; host code uses only that address (the
// array's name on the host is a stand-in, not a device address).  Every
// call on a device shares the device's array, so calls that overlap on one
// device (other streams, other host threads without ordering) race and
// their outputs are undefined.  The array keeps the last call's contents:
// the first call on a device zeroes it with a fill kernel on the caller's
// stream, and every launch after that clears on the device what the next
// one needs (the record set of the other parity), and takes its call number
// from the array itself, as a handle's launches do.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "specv.h"
#include "specv_internal.hpp"

namespace specv {
namespace {

constexpr int kNaBatch = SPECV_NOALLOC_MAX_BATCH;
constexpr int kNaGamma = SPECV_NOALLOC_MAX_GAMMA;
constexpr int kNaVocab = SPECV_NOALLOC_MAX_VOCAB;
constexpr int kNaPos = kNaGamma + 1;
constexpr int kNaChunks = (kNaVocab + kChunk - 1) / kChunk;

constexpr size_t round256(size_t n) { return (n + 255) & ~size_t(255); }

// The workspace's parts, at 256-byte aligned offsets (the same parts a
// handle allocates, two record sets included; no truncation candidates).
constexpr long long kSetStats = (long long)kNaBatch * kNaPos * 2 * kNaChunks * 2;
constexpr long long kSetPair = (long long)kNaBatch * kNaPos;
constexpr long long kSetRowrec = (long long)kNaBatch * kRowWords;
constexpr long long kSetWsum = (long long)kNaBatch * kNaChunks * 2;
constexpr size_t kStatsOff = 0;
constexpr size_t kStatsBytes = 2 * (size_t)kSetStats * sizeof(unsigned long long);
constexpr size_t kPairOff = round256(kStatsOff + kStatsBytes);
constexpr size_t kPairBytes = 2 * (size_t)kSetPair * sizeof(PairRec);
constexpr size_t kRowrecOff = round256(kPairOff + kPairBytes);
constexpr size_t kRowrecBytes = 2 * (size_t)kSetRowrec * sizeof(unsigned long long);
constexpr size_t kWsumOff = round256(kRowrecOff + kRowrecBytes);
constexpr size_t kWsumBytes = 2 * (size_t)kSetWsum * sizeof(unsigned long long);
constexpr size_t kCtrOff = round256(kWsumOff + kWsumBytes);
constexpr size_t kCtrBytes = (size_t)2 * kNaBatch * kNaPos * kSlot * sizeof(unsigned);
constexpr size_t kStatusOff = round256(kCtrOff + kCtrBytes);
constexpr size_t kStatusBytes = (size_t)2 * kNaBatch * (kSlot / 2) * sizeof(unsigned long long);
constexpr size_t kCallsOff = round256(kStatusOff + kStatusBytes);
constexpr size_t kCallsBytes = (size_t)kSlot * sizeof(unsigned);
constexpr size_t kSeenOff = round256(kCallsOff + kCallsBytes);
constexpr size_t kSeenBytes = (size_t)2 * kNaBatch * kSlot * sizeof(unsigned);
constexpr size_t kDimsOff = round256(kSeenOff + kSeenBytes);
constexpr size_t kDimsBytes = (size_t)kSlot * sizeof(unsigned long long);
constexpr size_t kScratchBytes = round256(kDimsOff + kDimsBytes);
static_assert(kScratchBytes == SPECV_NOALLOC_SCRATCH_BYTES, "scratch size differs from the header's");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Zero n16 16-byte words (the whole scratch array, through its device
// address): a kernel, not a memset, so that it is an ordinary kernel node
// when the caller captures the call.
__global__ __launch_bounds__(kBlock) void k_zero(uint4* p, long long n16) {
    for (long long i = (long long)blockIdx.x * kBlock + threadIdx.x; i < n16;
         i += (long long)gridDim.x * kBlock)
        p[i] = make_uint4(0, 0, 0, 0);
}

hipError_t zero_scratch(void* ptr, hipStream_t s) {
    const long long n16 = (long long)(kScratchBytes / 16);
    hipLaunchKernelGGL(k_zero, dim3(1024), dim3(kBlock), 0, s, static_cast<uint4*>(ptr), n16);
    return hipGetLastError();
}

constexpr int kMaxDevices = 64;
struct DeviceScratch {
    void* ptr = nullptr;     // the device's copy of ``scratch``, from hipGetSymbolAddress
};
std::mutex g_mutex;
DeviceScratch g_dev[kMaxDevices];

Workspace carve(void* ptr) {
    unsigned char* base = static_cast<unsigned char*>(ptr);
    Workspace ws{};
    ws.stats = reinterpret_cast<unsigned long long*>(base + kStatsOff);
    ws.pair = reinterpret_cast<PairRec*>(base + kPairOff);
    ws.rowrec = reinterpret_cast<unsigned long long*>(base + kRowrecOff);
    ws.wsum = reinterpret_cast<unsigned long long*>(base + kWsumOff);
    ws.ctr = reinterpret_cast<unsigned*>(base + kCtrOff);
    ws.status = reinterpret_cast<unsigned long long*>(base + kStatusOff);
    ws.calls = reinterpret_cast<unsigned*>(base + kCallsOff);
    ws.seen = reinterpret_cast<unsigned*>(base + kSeenOff);
    ws.dims = reinterpret_cast<unsigned long long*>(base + kDimsOff);
    ws.set_stats = kSetStats;
    ws.set_pair = kSetPair;
    ws.set_rowrec = kSetRowrec;
    ws.set_wsum = kSetWsum;
    ws.n_groups = kNaBatch * kNaPos;
    ws.n_rows = kNaBatch;
    return ws;
}

// Restores the calling thread's current device on scope exit.
struct DeviceGuard {
    int prev = -1;
    bool set(int device) {
        if (hipGetDevice(&prev) != hipSuccess) return false;
        return prev == device || hipSetDevice(device) == hipSuccess;
    }
    ~DeviceGuard() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

}  // namespace
}  // namespace specv

extern "C" SPECV_API specv_status specv_verify_sample_noalloc(
    int device, void* stream, const void* target_logits, int64_t t_stride_b, int64_t t_stride_pos,
    const void* draft_logits, int64_t d_stride_b, int64_t d_stride_pos, specv_dtype dtype, int B,
    int gamma, int V, const int32_t* draft_tokens, const specv_row_params* row_params, uint64_t seed,
    uint32_t step, int32_t eos_id, int32_t* out_num_accepted, int32_t* out_tokens,
    int32_t* out_num_emitted, int32_t* out_row_flags, const specv_diag* diag) {
    using namespace specv;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess) return SPECV_E_HIP;
    if (device < 0 || device >= ndev || device >= kMaxDevices) return SPECV_E_PARAM;
    Limits lim{};
    lim.max_batch = kNaBatch;
    lim.max_gamma = kNaGamma;
    lim.max_vocab = kNaVocab;
    lim.max_top_k = 0;             // no truncation workspace: truncated rows are unsupported
    lim.cand_cap = 0;
    lim.kept_cap = 0;
    Args a;
    bool vec = false;
    specv_status st = verify_sampling_args(
        lim, target_logits, t_stride_b, t_stride_pos, draft_logits, d_stride_b, d_stride_pos, nullptr, 0,
        dtype, B, gamma, V, draft_tokens, row_params, seed, step, eos_id, out_num_accepted, out_tokens,
        out_num_emitted, out_row_flags, diag, 0, &a, &vec);
    if (st != SPECV_OK || B == 0) return st;

    std::lock_guard<std::mutex> lock(g_mutex);
    DeviceGuard guard;
    if (!guard.set(device)) return SPECV_E_HIP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    DeviceScratch& d = g_dev[device];
    if (!d.ptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SPECV_E_HIP;
        if (zero_scratch(p, s) != hipSuccess) return SPECV_E_HIP;
        d.ptr = p;
    }
    a.ws = carve(d.ptr);
    // numbered on the device, captured or not: the array keeps no host state
    if (launch_verify(a, dtype == SPECV_BF16, vec, true, s, nullptr) != hipSuccess) return SPECV_E_HIP;
    return SPECV_OK;
}
