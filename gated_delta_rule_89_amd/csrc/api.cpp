// C ABI of the KDA operator: argument validation, variant choice, launches.
// Every check runs on the host before anything is enqueued.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "../../include/kda.h"
#include "kda_internal.h"

namespace {

using kda::DecodeArgs;
using kda::PrefillArgs;

bool head_size_ok(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool dtype_ok(kda_dtype t) { return t == KDA_F32 || t == KDA_BF16; }
size_t esize(kda_dtype t) { return t == KDA_BF16 ? 2 : 4; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};
Range range(const void* p, size_t bytes) {
    uintptr_t b = reinterpret_cast<uintptr_t>(p);
    return Range{b, b + bytes};
}
bool overlap(Range a, Range b) {
    if (a.lo == a.hi || b.lo == b.hi || a.lo == 0 || b.lo == 0) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

// The chunked kernels take bf16 q/k/v with d_k = d_v = 128.
bool chunk_supported(int32_t dk, int32_t dv, kda_dtype in) {
    return in == KDA_BF16 && dk == 128 && dv == 128;
}

// Compute units of the current device, cached per device id (threads that
// race on the first call store the same value).
int cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// AUTO: the chunked kernel, with the segment scan when the longest sequence
// alone would take well over the average work per CU (one chain per
// workgroup runs sequentially over its chunks).
kda_variant resolve_variant(kda_variant v, int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                            int32_t N, kda_dtype in, const int32_t* cu_host) {
    if (v != KDA_VARIANT_AUTO) return v;
    if (!chunk_supported(dk, dv, in)) return KDA_VARIANT_CHUNK8;
    int64_t longest = 0, chunks = 0;
    for (int32_t n = 0; n < N; ++n) {
        const int64_t len = cu_host ? cu_host[n + 1] - cu_host[n] : T;
        longest = len > longest ? len : longest;
        chunks += (len + 31) / 32;
    }
    (void)B;
    // Chunks per resident chain if the work were spread evenly; a sequence
    // much longer than that would leave most of the GPU idle at the end.
    const int64_t per_slot = chunks * H / (static_cast<int64_t>(cu_count()) * kda::chunk_chains_per_cu());
    return (longest + 31) / 32 > 2 * per_slot + 16 ? KDA_VARIANT_CHUNK_SCAN : KDA_VARIANT_CHUNK;
}

size_t workspace_for(kda_variant v, int32_t B, int32_t T, int32_t H, int32_t N, const int32_t* cu_host) {
    if (v == KDA_VARIANT_CHUNK || v == KDA_VARIANT_CHUNK_SCAN || v == KDA_VARIANT_CHUNK64)
        return kda::chunk_workspace_bytes(B, T, H, N, cu_host, v == KDA_VARIANT_CHUNK_SCAN);
    if (v == KDA_VARIANT_CHUNK8) return kda::chunk8_workspace_bytes(N);
    return 0;
}

size_t align256_(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Snapshots over all sequences: floor(length / interval) each.
int64_t snapshot_count(const int32_t* cu_host, int32_t N, int32_t T, int32_t interval) {
    int64_t c = 0;
    for (int32_t n = 0; n < N; ++n) c += (cu_host ? cu_host[n + 1] - cu_host[n] : T) / interval;
    return c;
}

bool seqlens_ok(const int32_t* cu_host, int32_t N, int32_t T) {
    if (cu_host[0] != 0 || cu_host[N] != T) return false;
    for (int32_t i = 0; i < N; ++i)
        if (cu_host[i + 1] < cu_host[i]) return false;
    return true;
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_str(kda_status s) {
    switch (s) {
        case KDA_OK: return "ok";
        case KDA_ERR_NULL: return "a required pointer is NULL";
        case KDA_ERR_SHAPE: return "a size is negative or inconsistent";
        case KDA_ERR_DTYPE: return "unknown dtype";
        case KDA_ERR_UNSUPPORTED: return "unsupported head size, dtype or variant";
        case KDA_ERR_SEQLENS: return "cu_seqlens must satisfy 0 = c0 <= c1 <= ... <= cN = T";
        case KDA_ERR_ALIAS: return "an output overlaps an input or another output";
        case KDA_ERR_ALIGN: return "a pointer is not aligned as required";
        case KDA_ERR_WORKSPACE: return "workspace missing or too small";
        case KDA_ERR_HIP: return "a HIP launch failed";
    }
    return "unknown status";
}

size_t kda_chunk_fwd_workspace_size(int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                                    int32_t N, const int32_t* cu_seqlens_host, kda_dtype in_dtype,
                                    kda_variant variant) {
    if (B < 0 || T < 0 || H < 0 || N < 0 || !head_size_ok(d_k) || !head_size_ok(d_v) ||
        !dtype_ok(in_dtype) || variant < KDA_VARIANT_AUTO || variant > KDA_VARIANT_CHUNK8)
        return 0;
    if (cu_seqlens_host ? (B != 1 || !seqlens_ok(cu_seqlens_host, N, T)) : N != B) return 0;
    const kda_variant v = resolve_variant(variant, B, T, H, d_k, d_v, N, in_dtype, cu_seqlens_host);
    return workspace_for(v, B, T, H, N, cu_seqlens_host);
}

}  // extern "C"

namespace {

// kda_chunk_fwd and kda_chunk_fwd_snapshots; snap_mode selects the latter.
kda_status chunk_fwd_impl(const void* q, const void* k, const void* v, const float* g,
                          const float* beta, float scale, const float* initial_state,
                          const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int32_t B,
                          int32_t T, int32_t H, int32_t d_k, int32_t d_v, int32_t N,
                          kda_dtype in_dtype, kda_dtype out_dtype, void* o, float* final_state,
                          void* workspace, size_t workspace_bytes, kda_variant variant,
                          void* stream, bool snap_mode, int32_t snap_interval, float* snapshots,
                          bool gated = false, const void* out_gate = nullptr,
                          const float* norm_weight = nullptr, float norm_eps = 0.f) {
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return KDA_ERR_DTYPE;
    if (gated && !(norm_eps >= 0.f && norm_eps < 3.0e38f)) return KDA_ERR_SHAPE;  // also NaN
    if (snap_mode && snap_interval <= 0) return KDA_ERR_SHAPE;
    if (snap_mode && snap_interval % 64 != 0) return KDA_ERR_UNSUPPORTED;
    if (B < 0 || T < 0 || H < 0 || N < 0 || d_k <= 0 || d_v <= 0) return KDA_ERR_SHAPE;
    if (!head_size_ok(d_k) || !head_size_ok(d_v)) return KDA_ERR_UNSUPPORTED;
    if (variant < KDA_VARIANT_AUTO || variant > KDA_VARIANT_CHUNK8) return KDA_ERR_UNSUPPORTED;
    if ((cu_seqlens == nullptr) != (cu_seqlens_host == nullptr)) return KDA_ERR_NULL;
    if (cu_seqlens) {
        if (B != 1) return KDA_ERR_SHAPE;
        if (!seqlens_ok(cu_seqlens_host, N, T)) return KDA_ERR_SEQLENS;
    } else if (N != B) {
        return KDA_ERR_SHAPE;
    }
    if (!aligned(initial_state, 16) || !aligned(final_state, 16)) return KDA_ERR_ALIGN;
    const int64_t tokens = static_cast<int64_t>(B) * T;
    if (tokens == 0 || N == 0 || H == 0) {
        // No token to process; a requested final state equals the initial one.
        if (N > 0 && H > 0 && final_state) {
            const int64_t n = static_cast<int64_t>(N) * H * d_k * d_v;
            if (initial_state && initial_state != final_state &&
                overlap(range(initial_state, n * 4), range(final_state, n * 4)))
                return KDA_ERR_ALIAS;
            if (kda::launch_copy_or_zero(final_state, initial_state, n,
                                         static_cast<hipStream_t>(stream)) != hipSuccess)
                return KDA_ERR_HIP;
        }
        return KDA_OK;
    }
    if (!q || !k || !v || !g || !beta || !o) return KDA_ERR_NULL;
    if (gated && (!out_gate || !norm_weight)) return KDA_ERR_NULL;
    if (gated && (!aligned(out_gate, 16) || !aligned(norm_weight, 16))) return KDA_ERR_ALIGN;
    if (static_cast<int64_t>(N) * H * 8 > INT32_MAX || H > 65535) return KDA_ERR_SHAPE;

    const kda_variant var = resolve_variant(variant, B, T, H, d_k, d_v, N, in_dtype, cu_seqlens_host);
    if ((var == KDA_VARIANT_CHUNK || var == KDA_VARIANT_CHUNK_SCAN || var == KDA_VARIANT_CHUNK64) &&
        !chunk_supported(d_k, d_v, in_dtype))
        return KDA_ERR_UNSUPPORTED;

    for (const void* p : {q, k, v, static_cast<const void*>(g), static_cast<const void*>(o),
                          static_cast<const void*>(initial_state),
                          static_cast<const void*>(final_state)})
        if (!aligned(p, 16)) return KDA_ERR_ALIGN;
    if (!aligned(beta, 4) || !aligned(cu_seqlens, 4) || !aligned(workspace, 256))
        return KDA_ERR_ALIGN;

    const int64_t nsnap = snap_mode ? snapshot_count(cu_seqlens_host, N, T, snap_interval) : 0;
    if (nsnap > 0 && !snapshots) return KDA_ERR_NULL;
    if (!aligned(snapshots, 16)) return KDA_ERR_ALIGN;
    if (nsnap > INT32_MAX / 2) return KDA_ERR_SHAPE;
    const size_t ws_plain = workspace_for(var, B, T, H, N, cu_seqlens_host);
    const size_t ws_need = nsnap > 0 ? align256_(ws_plain) + align256_(static_cast<size_t>(N) * 4) : ws_plain;
    if (ws_need > 0 && (!workspace || workspace_bytes < ws_need)) return KDA_ERR_WORKSPACE;

    const size_t th = static_cast<size_t>(tokens) * H;
    const size_t state_bytes = static_cast<size_t>(N) * H * d_k * d_v * sizeof(float);
    const Range in_r[] = {range(q, th * d_k * esize(in_dtype)), range(k, th * d_k * esize(in_dtype)),
                          range(v, th * d_v * esize(in_dtype)), range(g, th * d_k * 4),
                          range(beta, th * 4), range(initial_state, initial_state ? state_bytes : 0),
                          range(cu_seqlens, cu_seqlens ? (static_cast<size_t>(N) + 1) * 4 : 0)};
    const Range o_r = range(o, th * d_v * esize(out_dtype));
    const Range f_r = range(final_state, final_state ? state_bytes : 0);
    const Range w_r = range(workspace, ws_need > 0 ? workspace_bytes : 0);
    for (const Range& r : in_r) {
        if (overlap(o_r, r) || overlap(w_r, r)) return KDA_ERR_ALIAS;
        const bool same_state = final_state && r.lo == reinterpret_cast<uintptr_t>(initial_state) &&
                                static_cast<const void*>(final_state) == initial_state;
        if (!same_state && overlap(f_r, r)) return KDA_ERR_ALIAS;
    }
    if (overlap(o_r, f_r) || overlap(o_r, w_r) || overlap(f_r, w_r)) return KDA_ERR_ALIAS;
    if (gated) {
        const Range g_r = range(out_gate, th * d_v * esize(in_dtype));
        const Range nw_r = range(norm_weight, static_cast<size_t>(d_v) * 4);
        for (const Range& r : {g_r, nw_r})
            if (overlap(o_r, r) || overlap(f_r, r) || overlap(w_r, r)) return KDA_ERR_ALIAS;
    }
    if (nsnap > 0) {
        const Range s_r = range(snapshots, static_cast<size_t>(nsnap) * H * d_k * d_v * 4);
        for (const Range& r : in_r)
            if (overlap(s_r, r)) return KDA_ERR_ALIAS;
        if (overlap(s_r, o_r) || overlap(s_r, f_r) || overlap(s_r, w_r)) return KDA_ERR_ALIAS;
    }

    PrefillArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.scale = scale;
    a.h0 = initial_state;
    a.cu = cu_seqlens;
    a.cu_host = cu_seqlens_host;
    a.B = B;
    a.T = T;
    a.H = H;
    a.dk = d_k;
    a.dv = d_v;
    a.N = N;
    a.in_bf16 = in_dtype == KDA_BF16;
    a.out_bf16 = out_dtype == KDA_BF16;
    a.o = o;
    a.hT = final_state;
    a.ws = workspace;
    a.ws_bytes = workspace_bytes;
    a.stream = static_cast<hipStream_t>(stream);
    if (nsnap > 0) {
        int32_t* base = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + align256_(ws_plain));
        a.snaps = snapshots;
        a.snap_interval = snap_interval;
        a.snap_base = base;
        if (kda::launch_snap_base(cu_seqlens, N, T, snap_interval, base, a.stream) != hipSuccess)
            return KDA_ERR_HIP;
    }

    if (gated) {
        a.ogate = out_gate;
        a.nweight = norm_weight;
        a.neps = norm_eps;
    }

    hipError_t e = hipErrorInvalidValue;
    switch (var) {
        case KDA_VARIANT_RECURRENT: e = kda::launch_recurrent(a); break;
        case KDA_VARIANT_CHUNK: e = kda::launch_chunk(a, false, false); break;
        case KDA_VARIANT_CHUNK_SCAN: e = kda::launch_chunk(a, true, false); break;
        case KDA_VARIANT_CHUNK64: e = kda::launch_chunk(a, false, true); break;
        case KDA_VARIANT_CHUNK8: e = kda::launch_chunk8(a); break;
        default: return KDA_ERR_UNSUPPORTED;
    }
    // The 12-wave kernel (CHUNK, CHUNK_SCAN) fuses the gated RMSNorm into its o
    // store; the other variants write o and the epilogue rewrites it in place.
    if (e == hipSuccess && gated &&
        (var == KDA_VARIANT_RECURRENT || var == KDA_VARIANT_CHUNK64 || var == KDA_VARIANT_CHUNK8))
        e = kda::launch_gate_norm(a);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

extern "C" {

kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, float scale, const float* initial_state,
                         const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int32_t B,
                         int32_t T, int32_t H, int32_t d_k, int32_t d_v, int32_t N,
                         kda_dtype in_dtype, kda_dtype out_dtype, void* o, float* final_state,
                         void* workspace, size_t workspace_bytes, kda_variant variant,
                         void* stream) {
    return chunk_fwd_impl(q, k, v, g, beta, scale, initial_state, cu_seqlens, cu_seqlens_host, B, T,
                          H, d_k, d_v, N, in_dtype, out_dtype, o, final_state, workspace,
                          workspace_bytes, variant, stream, false, 0, nullptr);
}

size_t kda_chunk_fwd_snapshots_workspace_size(int32_t B, int32_t T, int32_t H, int32_t d_k,
                                              int32_t d_v, int32_t N,
                                              const int32_t* cu_seqlens_host, kda_dtype in_dtype,
                                              kda_variant variant, int32_t snap_interval) {
    if (snap_interval <= 0 || snap_interval % 64 != 0) return 0;
    if (B < 0 || T < 0 || H < 0 || N < 0 || !head_size_ok(d_k) || !head_size_ok(d_v) ||
        !dtype_ok(in_dtype) || variant < KDA_VARIANT_AUTO || variant > KDA_VARIANT_CHUNK8)
        return 0;
    if (cu_seqlens_host ? (B != 1 || !seqlens_ok(cu_seqlens_host, N, T)) : N != B) return 0;
    const kda_variant v = resolve_variant(variant, B, T, H, d_k, d_v, N, in_dtype, cu_seqlens_host);
    const size_t plain = workspace_for(v, B, T, H, N, cu_seqlens_host);
    if (static_cast<int64_t>(B) * T == 0 || snapshot_count(cu_seqlens_host, N, T, snap_interval) == 0)
        return plain;
    return align256_(plain) + align256_(static_cast<size_t>(N) * 4);
}

kda_status kda_fused_gate(const void* z, const void* w_up, const float* b_up, const float* u,
                          int32_t M, int32_t r, int32_t H, int32_t d_k, kda_dtype in_dtype,
                          float* g, float* beta, void* stream) {
    if (!dtype_ok(in_dtype)) return KDA_ERR_DTYPE;
    if (M < 0 || r <= 0 || H < 0 || d_k <= 0) return KDA_ERR_SHAPE;
    if (in_dtype != KDA_BF16 || d_k != 128 || (r != 32 && r != 64 && r != 128 && r != 256))
        return KDA_ERR_UNSUPPORTED;
    if (M == 0 || H == 0) return KDA_OK;
    if (!z || !w_up || !u || !g || !beta) return KDA_ERR_NULL;
    if (H > 65535) return KDA_ERR_SHAPE;  // one grid row per head; 32-bit row offsets within 32 rows of g
    for (const void* p : {z, w_up, static_cast<const void*>(g)})
        if (!aligned(p, 16)) return KDA_ERR_ALIGN;
    if (!aligned(b_up, 16) || !aligned(u, 4) || !aligned(beta, 4)) return KDA_ERR_ALIGN;
    const size_t n = static_cast<size_t>(H) * d_k, m = static_cast<size_t>(M);
    const Range in_r[] = {range(z, m * r * 2), range(w_up, static_cast<size_t>(r) * n * 2),
                          range(b_up, b_up ? n * 4 : 0), range(u, m * H * 4)};
    const Range g_r = range(g, m * n * 4), b_r = range(beta, m * H * 4);
    for (const Range& x : in_r)
        if (overlap(g_r, x) || overlap(b_r, x)) return KDA_ERR_ALIAS;
    if (overlap(g_r, b_r)) return KDA_ERR_ALIAS;
    return kda::launch_fused_gate(z, w_up, b_up, u, M, r, H, g, beta,
                                  static_cast<hipStream_t>(stream)) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_chunk_fwd_gated(const void* q, const void* k, const void* v, const float* g,
                               const float* beta, float scale, const float* initial_state,
                               const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                               int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                               int32_t N, kda_dtype in_dtype, kda_dtype out_dtype,
                               const void* out_gate, const float* norm_weight, float norm_eps,
                               void* o, float* final_state, void* workspace,
                               size_t workspace_bytes, kda_variant variant, void* stream) {
    return chunk_fwd_impl(q, k, v, g, beta, scale, initial_state, cu_seqlens, cu_seqlens_host, B, T,
                          H, d_k, d_v, N, in_dtype, out_dtype, o, final_state, workspace,
                          workspace_bytes, variant, stream, false, 0, nullptr, true, out_gate,
                          norm_weight, norm_eps);
}

kda_status kda_chunk_fwd_snapshots(const void* q, const void* k, const void* v, const float* g,
                                   const float* beta, float scale, const float* initial_state,
                                   const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                   int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                                   int32_t N, kda_dtype in_dtype, kda_dtype out_dtype, void* o,
                                   float* final_state, int32_t snap_interval, float* snapshots,
                                   void* workspace, size_t workspace_bytes, kda_variant variant,
                                   void* stream) {
    return chunk_fwd_impl(q, k, v, g, beta, scale, initial_state, cu_seqlens, cu_seqlens_host, B, T,
                          H, d_k, d_v, N, in_dtype, out_dtype, o, final_state, workspace,
                          workspace_bytes, variant, stream, true, snap_interval, snapshots);
}

kda_status kda_decode_step(const void* q, const void* k, const void* v, const float* g,
                           const float* beta, float scale, float* state, int32_t N, int32_t H,
                           int32_t d_k, int32_t d_v, kda_dtype in_dtype, kda_dtype out_dtype,
                           void* o, void* stream) {
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return KDA_ERR_DTYPE;
    if (N < 0 || H < 0 || d_k <= 0 || d_v <= 0) return KDA_ERR_SHAPE;
    if (!head_size_ok(d_k) || !head_size_ok(d_v)) return KDA_ERR_UNSUPPORTED;
    if (N == 0 || H == 0) return KDA_OK;
    if (!q || !k || !v || !g || !beta || !state || !o) return KDA_ERR_NULL;
    if (static_cast<int64_t>(N) * H > INT32_MAX) return KDA_ERR_SHAPE;
    for (const void* p : {q, k, v, static_cast<const void*>(g), static_cast<const void*>(state), static_cast<const void*>(o)})
        if (!aligned(p, 16)) return KDA_ERR_ALIGN;
    if (!aligned(beta, 4)) return KDA_ERR_ALIGN;
    const size_t nh = static_cast<size_t>(N) * H;
    const Range in_r[] = {range(q, nh * d_k * esize(in_dtype)), range(k, nh * d_k * esize(in_dtype)),
                          range(v, nh * d_v * esize(in_dtype)), range(g, nh * d_k * 4),
                          range(beta, nh * 4)};
    const Range s_r = range(state, nh * d_k * d_v * 4);
    const Range o_r = range(o, nh * d_v * esize(out_dtype));
    for (const Range& r : in_r)
        if (overlap(o_r, r) || overlap(s_r, r)) return KDA_ERR_ALIAS;
    if (overlap(o_r, s_r)) return KDA_ERR_ALIAS;

    DecodeArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.scale = scale;
    a.state = state;
    a.N = N;
    a.H = H;
    a.dk = d_k;
    a.dv = d_v;
    a.in_bf16 = in_dtype == KDA_BF16;
    a.out_bf16 = out_dtype == KDA_BF16;
    a.o = o;
    a.T = 1;
    a.stream = static_cast<hipStream_t>(stream);
    return kda::launch_decode(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_fused_recurrent_fwd(const void* q, const void* k, const void* v, const float* g,
                                   const float* beta, float scale, float* state, int32_t N,
                                   int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                                   kda_dtype in_dtype, kda_dtype out_dtype, void* o,
                                   void* stream) {
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return KDA_ERR_DTYPE;
    if (N < 0 || T < 0 || H < 0 || d_k <= 0 || d_v <= 0) return KDA_ERR_SHAPE;
    if (!head_size_ok(d_k) || !head_size_ok(d_v)) return KDA_ERR_UNSUPPORTED;
    if (T > KDA_FUSED_RECURRENT_MAX_T) return KDA_ERR_UNSUPPORTED;
    if (N == 0 || H == 0 || T == 0) return KDA_OK;
    if (!q || !k || !v || !g || !beta || !state || !o) return KDA_ERR_NULL;
    if (static_cast<int64_t>(N) * H > INT32_MAX) return KDA_ERR_SHAPE;
    for (const void* p : {q, k, v, static_cast<const void*>(g), static_cast<const void*>(state), static_cast<const void*>(o)})
        if (!aligned(p, 16)) return KDA_ERR_ALIGN;
    if (!aligned(beta, 4)) return KDA_ERR_ALIGN;
    const size_t nh = static_cast<size_t>(N) * H, nth = nh * static_cast<size_t>(T);
    const Range in_r[] = {range(q, nth * d_k * esize(in_dtype)), range(k, nth * d_k * esize(in_dtype)),
                          range(v, nth * d_v * esize(in_dtype)), range(g, nth * d_k * 4),
                          range(beta, nth * 4)};
    const Range s_r = range(state, nh * d_k * d_v * 4);
    const Range o_r = range(o, nth * d_v * esize(out_dtype));
    for (const Range& r : in_r)
        if (overlap(o_r, r) || overlap(s_r, r)) return KDA_ERR_ALIAS;
    if (overlap(o_r, s_r)) return KDA_ERR_ALIAS;

    DecodeArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.scale = scale;
    a.state = state;
    a.N = N;
    a.H = H;
    a.dk = d_k;
    a.dv = d_v;
    a.T = T;
    a.in_bf16 = in_dtype == KDA_BF16;
    a.out_bf16 = out_dtype == KDA_BF16;
    a.o = o;
    a.stream = static_cast<hipStream_t>(stream);
    return kda::launch_steps(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
