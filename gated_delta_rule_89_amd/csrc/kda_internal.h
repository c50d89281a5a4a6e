// Internal launcher interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

namespace kda {

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    float scale;
    const float* h0;     // [N, H, dk, dv] or nullptr
    const int32_t* cu;   // device [N+1] or nullptr (then sequences are rows of length T)
    const int32_t* cu_host;
    int B, T, H, dk, dv, N;
    bool in_bf16, out_bf16;
    void* o;
    float* hT;           // [N, H, dk, dv] or nullptr
    float* snaps;        // [total snapshots, H, dk, dv] or nullptr
    int snap_interval;   // tokens between snapshots (multiple of 64) when snaps
    const int32_t* snap_base;  // device [N]: row of each sequence's first snapshot
    const void* ogate;   // [B, T, H, dv] in_dtype output gate, or nullptr (plain o)
    const float* nweight;  // [dv] RMSNorm weight (with ogate)
    float neps;          // RMSNorm eps (with ogate)
    void* ws;
    size_t ws_bytes;
    hipStream_t stream;
};

// One workgroup's work in the chunked kernels: tokens [t0, t1) of one
// sequence, for head blockIdx % H.
struct ChunkItem {
    int64_t t0, t1;
    int32_t sin;   // initial state: >= 0 row of h0, <= -2 row (-sin - 2) of the staged states, -1 zero
    int32_t sout;  // final state: >= 0 row of the output (the map slot in MAP mode),
                   // <= -2 row (-sout - 2) of the segment-state buffer, -1 none
    int64_t p0;    // tokens of the sequence before t0
    int32_t snap;  // row of the sequence's first state snapshot, -1 none
    int32_t fin;   // FULL, last segment of a split sequence: row of the final state,
                   // written here instead of the segment-state row when its map vanished
};

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    float scale;
    float* state;
    int N, H, dk, dv;
    int T;            // tokens per sequence (1 for a decode step)
    bool in_bf16, out_bf16;
    void* o;
    hipStream_t stream;
};

// Calls f(integral_constant<int, DK>, integral_constant<int, DV>) for the
// supported head sizes; returns hipErrorInvalidValue for anything else.
template <typename F>
hipError_t dispatch_head_sizes(int dk, int dv, F&& f) {
    auto inner = [&](auto DK) -> hipError_t {
        switch (dv) {
            case 16: return f(DK, std::integral_constant<int, 16>{});
            case 32: return f(DK, std::integral_constant<int, 32>{});
            case 64: return f(DK, std::integral_constant<int, 64>{});
            case 128: return f(DK, std::integral_constant<int, 128>{});
            default: return hipErrorInvalidValue;
        }
    };
    switch (dk) {
        case 16: return inner(std::integral_constant<int, 16>{});
        case 32: return inner(std::integral_constant<int, 32>{});
        case 64: return inner(std::integral_constant<int, 64>{});
        case 128: return inner(std::integral_constant<int, 128>{});
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_copy_or_zero(float* dst, const float* src, int64_t n, hipStream_t stream);
hipError_t launch_recurrent(const PrefillArgs& a);
hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_steps(const DecodeArgs& a);
// d_k = d_v = 128: the run in 8-token sub-chunks on fp32 MFMA.
hipError_t launch_steps_mfma(const DecodeArgs& a);
// g = -softplus(z W + b) (bf16 MFMA up-projection), beta = sigmoid(u).
hipError_t launch_fused_gate(const void* z, const void* w, const float* bias, const float* u,
                             int64_t M, int r, int H, float* g, float* beta, hipStream_t stream);
// o <- gate * w * o / sqrt(mean(o^2) + eps) over d_v, in place, for every (token, head).
hipError_t launch_gate_norm(const PrefillArgs& a);

// Chunked MFMA prefill (bf16 inputs, d_k = d_v = 128).  With scan = true long
// sequences are cut into segments whose (B, M) maps are composed by a scan.
// cu_host may be null (then the N sequences are rows of length T).
int chunk_chains_per_cu();  // full-mode chunk workgroups resident per CU
// Row of each sequence's first snapshot (floor(length / interval) each).
hipError_t launch_snap_base(const int32_t* cu, int N, int T, int interval, int32_t* out,
                            hipStream_t stream);
int chunk_segment_tokens(int B, int T, int H, int N, const int32_t* cu_host);
size_t chunk_workspace_bytes(int B, int T, int H, int N, const int32_t* cu_host, bool scan);
// scan: segment-scan path; c64: single-role kernel on 64-token chunks.
hipError_t launch_chunk(const PrefillArgs& a, bool scan, bool c64);
// One item per sequence (whole sequence, its own h0/hT rows and first
// snapshot row), longest first when cu is given and N is at most 16384.
hipError_t launch_plan_sequences(const PrefillArgs& a, ChunkItem* items);
// Any supported head size and input dtype: the chunk form on 8-token
// sub-chunks in fp32 MFMA.  Workspace: chunk8_workspace_bytes(N).
size_t chunk8_workspace_bytes(int N);
hipError_t launch_chunk8(const PrefillArgs& a);

}  // namespace kda
