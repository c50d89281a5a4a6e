// kda_chunk_fwd_noalloc: kda_chunk_fwd with its workspace in a file-scope
// device array, for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid allocation).
//
// Every GPU the library runs on holds one copy of `scratch` (in the loaded
// code object) until the process ends.  Its device address is resolved once
// per device with hipGetSymbolAddress, with that device current, and kept:
// in host code the array's name is only a host-side stand-in, so only the
// resolved pointer is ever passed to a kernel.  Every call on a GPU shares
// that GPU's array and the array keeps the last call's contents; the chunked
// path writes every workspace byte it reads (work items, segment maps,
// staged states) earlier in the same call, so nothing has to start at zero.
// Calls that overlap on one GPU (two streams, two host threads) race on the
// array and must be serialised by the caller.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <mutex>

#include "../../include/kda.h"

namespace {

constexpr size_t kScratchBytes = KDA_CHUNK_FWD_NOALLOC_MAX_WORKSPACE;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte blocks");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// This device's copy of `scratch` (the current device's), resolved on first use.
kda_status device_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KDA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            (void)hipGetLastError();  // leave no sticky error behind for the caller
            return KDA_ERR_HIP;
        }
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return KDA_OK;
}

}  // namespace

extern "C" kda_status kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                            const float* g, const float* beta, float scale,
                                            const float* initial_state, const int32_t* cu_seqlens,
                                            const int32_t* cu_seqlens_host, int32_t B, int32_t T,
                                            int32_t H, int32_t d_k, int32_t d_v, int32_t N,
                                            kda_dtype in_dtype, kda_dtype out_dtype, void* o,
                                            float* final_state, kda_variant variant,
                                            void* stream) {
    // Size check on the host first.  AUTO may choose the segment scan, whose
    // maps grow with the sequence length; when they do not fit, the plain
    // chunked kernel (one work item per sequence) is used instead.  A size of
    // 0 also stands for arguments kda_chunk_fwd rejects, which it then reports.
    kda_variant var = variant;
    size_t need = kda_chunk_fwd_workspace_size(B, T, H, d_k, d_v, N, cu_seqlens_host, in_dtype, var);
    if (need > kScratchBytes && var == KDA_VARIANT_AUTO) {
        const size_t plain = kda_chunk_fwd_workspace_size(B, T, H, d_k, d_v, N, cu_seqlens_host,
                                                          in_dtype, KDA_VARIANT_CHUNK);
        if (plain > 0 && plain <= kScratchBytes) {
            var = KDA_VARIANT_CHUNK;
            need = plain;
        }
    }
    if (need > kScratchBytes) return KDA_ERR_WORKSPACE;
    void* ws = nullptr;
    const kda_status s = device_scratch(&ws);
    if (s != KDA_OK) return s;
    return kda_chunk_fwd(q, k, v, g, beta, scale, initial_state, cu_seqlens, cu_seqlens_host, B, T,
                         H, d_k, d_v, N, in_dtype, out_dtype, o, final_state, ws, kScratchBytes, var,
                         stream);
}
