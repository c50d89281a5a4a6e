// Output gate after RMSNorm, applied to a written o in place ("kimi delta
// attn from first principles", section "three gates": RMSNorm of o_t, then
// the elementwise product with the output gate).  The 12-wave chunk kernel
// fuses this into its o store; this kernel serves the other prefill variants.
//
// One wave per (token, head): lane l holds channels l, l + 64 (d_v <= 128),
// the sum of squares is a wave butterfly, and each value is rewritten as
// gate * w * o / sqrt(mean(o^2) + eps).
#include "dev_common.h"
#include "kda_internal.h"

namespace kda {

template <int DV, typename Tin, typename Tout>
__global__ __launch_bounds__(256) void gate_norm_kernel(Tout* __restrict__ o, const Tin* __restrict__ gate,
                                                        const float* __restrict__ w, float eps,
                                                        int64_t rows) {
    constexpr int PER = DV >= 64 ? DV / 64 : 1;
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;  // whole wave leaves together
    const int64_t base = row * DV;
    float x[PER];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int c = lane + 64 * i;
        x[i] = c < DV ? ld(o, base + c) : 0.f;
        ss += x[i] * x[i];
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) ss += __shfl_xor(ss, m);
    const float rinv = __builtin_amdgcn_rsqf(ss * (1.f / DV) + eps);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int c = lane + 64 * i;
        if (c < DV) st(o, base + c, x[i] * rinv * w[c] * ld(gate, base + c));
    }
}

template <int DV, typename Tin, typename Tout>
static hipError_t launch_gn(const PrefillArgs& a) {
    const int64_t rows = static_cast<int64_t>(a.B) * a.T * a.H;
    hipLaunchKernelGGL((gate_norm_kernel<DV, Tin, Tout>), dim3(static_cast<uint32_t>((rows + 3) / 4)),
                       dim3(256), 0, a.stream, static_cast<Tout*>(a.o), static_cast<const Tin*>(a.ogate),
                       a.nweight, a.neps, rows);
    return hipGetLastError();
}

template <int DV>
static hipError_t launch_gn_d(const PrefillArgs& a) {
    if (a.in_bf16) return a.out_bf16 ? launch_gn<DV, bf16_t, bf16_t>(a) : launch_gn<DV, bf16_t, float>(a);
    return a.out_bf16 ? launch_gn<DV, float, bf16_t>(a) : launch_gn<DV, float, float>(a);
}

hipError_t launch_gate_norm(const PrefillArgs& a) {
    switch (a.dv) {
        case 16: return launch_gn_d<16>(a);
        case 32: return launch_gn_d<32>(a);
        case 64: return launch_gn_d<64>(a);
        case 128: return launch_gn_d<128>(a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
