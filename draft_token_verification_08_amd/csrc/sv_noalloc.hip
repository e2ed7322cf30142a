// sv_noalloc.hip -- spec_verify_sample_ex_noalloc(): spec_verify_sample_ex()
// with its workspace in a file-scope device array instead of caller memory, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// The array `scratch` is SV_NOALLOC_SCRATCH_BYTES bytes; every GPU the library
// runs on holds its own copy until the process ends.  Host code never passes
// the array's name to a kernel (in host code it is only a stand-in for the
// symbol): its device address on the current device is looked up once per
// device with hipGetSymbolAddress and kept, and only that address is used.
// The verify kernels need the workspace zero-filled and leave it zero-filled
// after every call that completes, so the array is cleared (a fill kernel on
// the caller's stream) on its first use on a device and after a call that
// failed with some of its kernels possibly enqueued.
#include <mutex>

#include "sv_internal.h"

namespace {

constexpr size_t kScratchBytes = SV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // scratch's device address on each device (null: not looked up yet)
bool g_dirty[kMaxDevices];     // clear before the next call's kernels

}  // namespace

extern "C" sv_status_t spec_verify_sample_ex_noalloc(
    const void* target_logits, const void* draft_logits, sv_dtype_t dt, const int32_t* draft_tokens,
    const int32_t* draft_lens, const float* temperature, const float* uniforms, const float* draft_stats, int B,
    int n, int V, int32_t* accepted_len, int32_t* emitted, float* row_lse, uint32_t* err_flags, int32_t* tokens,
    const void* hidden_src, void* hidden_dst, int H, void* stream) {
    // sizes first: a call that cannot fit touches nothing
    const size_t need = sv_workspace_bytes(B, n, V, dt);
    if (need == 0) return SV_EINVAL;
    if (need > kScratchBytes) return SV_EWORKSPACE;
    if (B == 0) return SV_OK;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return sv::hip_status(e);
    if (dev < 0 || dev >= kMaxDevices) return SV_EINVAL;
    void* ws = nullptr;
    bool clear = false;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        if (g_scratch[dev] == nullptr) {
            void* p = nullptr;
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || p == nullptr) return sv::hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol);
            g_scratch[dev] = p;
            g_dirty[dev] = true;
        }
        ws = g_scratch[dev];
        clear = g_dirty[dev];
    }
    hipStream_t s = (hipStream_t)stream;
    if (clear) {
        e = sv::launch_clear(ws, kScratchBytes, s);
        if (e != hipSuccess) return sv::hip_status(e);
    }
    const sv_status_t st = sv::sample_ex(target_logits, draft_logits, dt, draft_tokens, draft_lens, temperature,
                                         uniforms, draft_stats, B, n, V, accepted_len, emitted, row_lse, err_flags,
                                         tokens, hidden_src, hidden_dst, H, ws, kScratchBytes, stream);
    {
        std::lock_guard<std::mutex> lock(g_mu);
        // SV_EHIP: a launch failed after others may have been enqueued, so the
        // array may not be zero-filled any more; other statuses enqueue nothing
        if (st == SV_EHIP) g_dirty[dev] = true;
        else if (clear) g_dirty[dev] = false;
    }
    return st;
}
