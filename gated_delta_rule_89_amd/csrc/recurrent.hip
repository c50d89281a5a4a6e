// Token-sequential (fused recurrent) KDA prefill for any supported head size
// and dtype.  It computes the recurrence of "Understanding Kimi Delta
// Attention" (section "The KDA Recurrence") one token at a time, the
// "fused recurrent mode" of that page's section "Two execution modes".
//
// Columns of the state are independent given (q, k, g, beta): column j of
// S_t depends only on column j of S_{t-1} and v_t[j].  A wave therefore owns
// 8 columns; its 64 lanes are 8 row groups x 8 columns, each lane holding
// DK/8 rows of one column in registers for the whole chain.  Per token the
// two reductions over the key channels (S^T k and S^T q) are a lane-local sum
// plus three cross-lane butterflies; nothing goes through LDS.
#include "dev_common.h"
#include "kda_internal.h"

namespace kda {

template <int DK, int DV, int WAVES, typename Tin, typename Tout>
__global__ __launch_bounds__(64 * WAVES) void recurrent_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, float scale,
    const float* __restrict__ h0, const int32_t* __restrict__ cu, int T, int H,
    Tout* __restrict__ o, float* __restrict__ hT, float* __restrict__ snaps, int interval,
    const int32_t* __restrict__ snap_base) {
    constexpr int R = DK / 8;  // rows per lane
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rg = lane >> 3;
    constexpr int XS = DV / (8 * WAVES);  // column slices per chain
    const int n = blockIdx.x / XS;
    const int j = ((blockIdx.x % XS) * WAVES + wave) * 8 + (lane & 7);
    const int h = blockIdx.y;

    int64_t t0, t1;
    if (cu) {
        t0 = cu[n];
        t1 = cu[n + 1];
    } else {
        t0 = static_cast<int64_t>(n) * T;
        t1 = t0 + T;
    }
    const int64_t sbase = (static_cast<int64_t>(n) * H + h) * DK * DV;

    float s[R];
#pragma unroll
    for (int i = 0; i < R; ++i) s[i] = h0 ? h0[sbase + static_cast<int64_t>(rg * R + i) * DV + j] : 0.f;

    // Next token's operands are fetched one step ahead to hide load latency.
    float nk[R], nq[R], ng[R], nv = 0.f, nb = 0.f;
    auto fetch = [&](int64_t t) {
        const int64_t kb = (t * H + h) * DK + rg * R;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            nk[i] = ld(k, kb + i);
            nq[i] = ld(q, kb + i);
            ng[i] = g[kb + i];
        }
        nv = ld(v, (t * H + h) * DV + j);
        nb = beta[t * H + h];
    };
    if (t0 < t1) fetch(t0);
    int64_t next_snap = interval, snap_row = snaps ? snap_base[n] : 0;
    for (int64_t t = t0; t < t1; ++t) {
        float kk[R], qq[R], gg[R];
#pragma unroll
        for (int i = 0; i < R; ++i) {
            kk[i] = nk[i];
            qq[i] = nq[i];
            gg[i] = ng[i];
        }
        const float vt = nv, bt = nb;
        if (t + 1 < t1) fetch(t + 1);
        float p = 0.f;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            s[i] *= gate_exp(gg[i]);  // decay row by its own gate
            p += s[i] * kk[i];
        }
        p += __shfl_xor(p, 8);
        p += __shfl_xor(p, 16);
        p += __shfl_xor(p, 32);
        const float u = bt * (vt - p);  // delta-rule error on the decayed state
        float r = 0.f;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            s[i] += kk[i] * u;  // rank-1 write
            r += s[i] * qq[i];
        }
        r += __shfl_xor(r, 8);
        r += __shfl_xor(r, 16);
        r += __shfl_xor(r, 32);
        if (rg == 0) st(o, (t * H + h) * DV + j, scale * r);
        if (snaps && t + 1 - t0 == next_snap) {  // state after `interval` more tokens
            float* dst = snaps + (snap_row * H + h) * DK * DV;
#pragma unroll
            for (int i = 0; i < R; ++i) dst[static_cast<int64_t>(rg * R + i) * DV + j] = s[i];
            next_snap += interval;
            ++snap_row;
        }
    }
    if (hT) {
#pragma unroll
        for (int i = 0; i < R; ++i) hT[sbase + static_cast<int64_t>(rg * R + i) * DV + j] = s[i];
    }
}

template <int DK, int DV, typename Tin, typename Tout>
static hipError_t launch_recurrent_t(const PrefillArgs& a) {
    constexpr int WAVES = (DV / 8) >= 4 ? 4 : (DV / 8);
    dim3 grid(a.N * (DV / (8 * WAVES)), a.H);
    hipLaunchKernelGGL((recurrent_kernel<DK, DV, WAVES, Tin, Tout>), grid, dim3(64 * WAVES), 0,
                       a.stream, static_cast<const Tin*>(a.q), static_cast<const Tin*>(a.k),
                       static_cast<const Tin*>(a.v), a.g, a.beta, a.scale, a.h0, a.cu, a.T, a.H,
                       static_cast<Tout*>(a.o), a.hT, a.snaps, a.snap_interval, a.snap_base);
    return hipGetLastError();
}

template <int DK, int DV>
static hipError_t launch_recurrent_d(const PrefillArgs& a) {
    if (a.in_bf16) {
        return a.out_bf16 ? launch_recurrent_t<DK, DV, bf16_t, bf16_t>(a)
                          : launch_recurrent_t<DK, DV, bf16_t, float>(a);
    }
    return a.out_bf16 ? launch_recurrent_t<DK, DV, float, bf16_t>(a)
                      : launch_recurrent_t<DK, DV, float, float>(a);
}

hipError_t launch_recurrent(const PrefillArgs& a) {
    return dispatch_head_sizes(a.dk, a.dv, [&](auto DK, auto DV) {
        return launch_recurrent_d<decltype(DK)::value, decltype(DV)::value>(a);
    });
}

}  // namespace kda
