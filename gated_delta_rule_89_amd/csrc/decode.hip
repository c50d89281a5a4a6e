// Single-token KDA step with the state updated in place: the fused recurrent
// step of "Understanding Kimi Delta Attention" (section "Two execution
// modes"; recurrence of section "The KDA Recurrence").
//
// For one (sequence, head) with decay alpha = exp(g):
//   s_k = (Diag(alpha) S)^T k,  s_q = (Diag(alpha) S)^T q     (one pass over S)
//   u   = beta (v - s_k)
//   S  <- Diag(alpha) S + k u^T                               (written back)
//   o   = scale * (s_q + (q . k) u)                            (= scale S_t^T q)
// The read-out identity follows from S_t^T q = (Diag(alpha) S)^T q + u (k . q).
//
// The step is bound by HBM: per (sequence, head) it reads and writes the
// d_k x d_v fp32 state once and touches a few hundred bytes else.  One
// workgroup owns one state; each thread keeps R rows x 4 columns in
// registers between the read and the write, so the state makes exactly one
// trip in and one trip out, with 16-byte accesses that let a wave cover whole
// 512-byte rows.  Reads are ordinary cached loads and writes are non-temporal
// stores: on this GPU that pairing streams the in-place update measurably
// faster than non-temporal loads or cached stores.
#include "dev_common.h"
#include "kda_internal.h"

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// NT threads per (sequence, head): TPR threads cover a row in 16-byte pieces,
// RGS row groups of R rows each.  A single step streams the state once and
// wants many requests in flight (512 threads measured faster); a run of
// tokens crosses a barrier per token and wants fewer, fuller threads (256).
template <int DK, int DV, int NT = 256>
struct DecodeShape {
    static constexpr int TPR = DV / 4;                                    // threads per row
    static constexpr int RGS = (NT / TPR) < DK ? (NT / TPR) : DK;        // row groups
    static constexpr int THREADS = TPR * RGS;
    static constexpr int R = DK / RGS;                                    // rows per thread
};
constexpr int kDecodeThreads = 512;

template <int DK, int DV, typename Tin, typename Tout>
__global__ __launch_bounds__((DecodeShape<DK, DV, kDecodeThreads>::THREADS)) void decode_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, float scale,
    float* __restrict__ state, Tout* __restrict__ o) {
    using Sh = DecodeShape<DK, DV, kDecodeThreads>;
    constexpr int TPR = Sh::TPR, RGS = Sh::RGS, R = Sh::R;
    __shared__ float red_k[RGS][DV];
    __shared__ float red_q[RGS][DV];
    __shared__ float red_qk[RGS];

    const int c4 = threadIdx.x % TPR;
    const int rg = threadIdx.x / TPR;
    const int64_t nh = blockIdx.x;  // n * H + h
    float* S = state + nh * DK * DV;
    const int64_t vb = nh * DK;

    f32x4 s[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int r = rg + RGS * i;
        s[i] = *(reinterpret_cast<const f32x4*>(S + r * DV) + c4);
    }
    float kr[R], a[R];
    f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
    float qk = 0.f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int r = rg + RGS * i;
        kr[i] = ld(k, vb + r);
        const float qr = ld(q, vb + r);
        a[i] = gate_exp(g[vb + r]);
        s[i] *= a[i];  // decay row r
        pk += s[i] * kr[i];
        pq += s[i] * qr;
        qk += qr * kr[i];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        red_k[rg][4 * c4 + c] = pk[c];
        red_q[rg][4 * c4 + c] = pq[c];
    }
    if (c4 == 0) red_qk[rg] = qk;
    __syncthreads();

    f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sq = {0.f, 0.f, 0.f, 0.f};
    float qk_all = 0.f;
#pragma unroll
    for (int x = 0; x < RGS; ++x) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            sk[c] += red_k[x][4 * c4 + c];
            sq[c] += red_q[x][4 * c4 + c];
        }
        qk_all += red_qk[x];
    }
    const float bt = beta[nh];
    f32x4 u;
#pragma unroll
    for (int c = 0; c < 4; ++c) u[c] = bt * (ld(v, nh * DV + 4 * c4 + c) - sk[c]);

#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int r = rg + RGS * i;
        s[i] += kr[i] * u;  // rank-1 write
        __builtin_nontemporal_store(s[i], reinterpret_cast<f32x4*>(S + r * DV) + c4);
    }
    if (rg == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) st(o, nh * DV + 4 * c4 + c, scale * (sq[c] + qk_all * u[c]));
    }
}

template <int DK, int DV, typename Tin, typename Tout>
static hipError_t launch_decode_t(const DecodeArgs& a) {
    const int64_t blocks = static_cast<int64_t>(a.N) * a.H;
    hipLaunchKernelGGL((decode_kernel<DK, DV, Tin, Tout>), dim3(static_cast<uint32_t>(blocks)),
                       dim3(DecodeShape<DK, DV, kDecodeThreads>::THREADS), 0, a.stream,
                       static_cast<const Tin*>(a.q), static_cast<const Tin*>(a.k),
                       static_cast<const Tin*>(a.v), a.g, a.beta, a.scale, a.state,
                       static_cast<Tout*>(a.o));
    return hipGetLastError();
}

template <int DK, int DV>
static hipError_t launch_decode_d(const DecodeArgs& a) {
    if (a.in_bf16) {
        return a.out_bf16 ? launch_decode_t<DK, DV, bf16_t, bf16_t>(a)
                          : launch_decode_t<DK, DV, bf16_t, float>(a);
    }
    return a.out_bf16 ? launch_decode_t<DK, DV, float, bf16_t>(a)
                      : launch_decode_t<DK, DV, float, float>(a);
}

hipError_t launch_decode(const DecodeArgs& a) {
    return dispatch_head_sizes(a.dk, a.dv, [&](auto DK, auto DV) {
        return launch_decode_d<decltype(DK)::value, decltype(DV)::value>(a);
    });
}

// T consecutive tokens per (sequence, head) with the state in place: the
// same step as decode_kernel, repeated while the state stays in registers,
// so the state still makes one trip in and one trip out for the whole run
// (the fused recurrent mode over a short run of tokens).  Token t's inputs
// sit at ((n T + t) H + h) of the [N, T, H, .] tensors.  The two reductions
// over the rows go through double-buffered LDS partials, one barrier per
// token; the next token's row inputs are read before that barrier.
template <int DK, int DV, typename Tin, typename Tout>
__global__ __launch_bounds__((DecodeShape<DK, DV>::THREADS)) void steps_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, float scale,
    float* __restrict__ state, Tout* __restrict__ o, int T, int H) {
    using Sh = DecodeShape<DK, DV>;
    constexpr int TPR = Sh::TPR, RGS = Sh::RGS, R = Sh::R;
    __shared__ float red_k[2][RGS][DV];
    __shared__ float red_q[2][RGS][DV];
    __shared__ float red_qk[2][RGS];

    const int c4 = threadIdx.x % TPR;
    const int rg = threadIdx.x / TPR;
    const int64_t nh = blockIdx.x;  // n * H + h
    const int64_t n = nh / H, h = nh % H;
    float* S = state + nh * DK * DV;

    f32x4 s[R];
#pragma unroll
    for (int i = 0; i < R; ++i) s[i] = *(reinterpret_cast<const f32x4*>(S + (rg + RGS * i) * DV) + c4);

    // row inputs of the token being processed (kr, qr, a) and of the next one
    float kr[R], qr[R], a[R], nk[R], nq[R], na[R];
    auto fetch = [&](int t, float* fk, float* fq, float* fa) {
        const int64_t b = ((n * T + t) * H + h) * DK;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int r = rg + RGS * i;
            fk[i] = ld(k, b + r);
            fq[i] = ld(q, b + r);
            fa[i] = gate_exp(g[b + r]);
        }
    };
    fetch(0, kr, qr, a);
    for (int t = 0; t < T; ++t) {
        const int buf = t & 1;
        const int64_t tv = (n * T + t) * H + h;  // token row of v, beta, o
        f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
        float qk = 0.f;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            s[i] *= a[i];  // decay row
            pk += s[i] * kr[i];
            pq += s[i] * qr[i];
            qk += qr[i] * kr[i];
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            red_k[buf][rg][4 * c4 + c] = pk[c];
            red_q[buf][rg][4 * c4 + c] = pq[c];
        }
        if (c4 == 0) red_qk[buf][rg] = qk;
        f32x4 vt;
#pragma unroll
        for (int c = 0; c < 4; ++c) vt[c] = ld(v, tv * DV + 4 * c4 + c);
        const float bt = beta[tv];
        if (t + 1 < T) fetch(t + 1, nk, nq, na);
        __syncthreads();

        f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sq = {0.f, 0.f, 0.f, 0.f};
        float qk_all = 0.f;
#pragma unroll
        for (int x = 0; x < RGS; ++x) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                sk[c] += red_k[buf][x][4 * c4 + c];
                sq[c] += red_q[buf][x][4 * c4 + c];
            }
            qk_all += red_qk[buf][x];
        }
        const f32x4 u = bt * (vt - sk);
#pragma unroll
        for (int i = 0; i < R; ++i) s[i] += kr[i] * u;  // rank-1 write
        if (rg == 0) {
#pragma unroll
            for (int c = 0; c < 4; ++c) st(o, tv * DV + 4 * c4 + c, scale * (sq[c] + qk_all * u[c]));
        }
#pragma unroll
        for (int i = 0; i < R; ++i) {
            kr[i] = nk[i];
            qr[i] = nq[i];
            a[i] = na[i];
        }
    }
#pragma unroll
    for (int i = 0; i < R; ++i)
        __builtin_nontemporal_store(s[i], reinterpret_cast<f32x4*>(S + (rg + RGS * i) * DV) + c4);
}

template <int DK, int DV, typename Tin, typename Tout>
static hipError_t launch_steps_t(const DecodeArgs& a) {
    const int64_t blocks = static_cast<int64_t>(a.N) * a.H;
    hipLaunchKernelGGL((steps_kernel<DK, DV, Tin, Tout>), dim3(static_cast<uint32_t>(blocks)),
                       dim3(DecodeShape<DK, DV>::THREADS), 0, a.stream,
                       static_cast<const Tin*>(a.q), static_cast<const Tin*>(a.k),
                       static_cast<const Tin*>(a.v), a.g, a.beta, a.scale, a.state,
                       static_cast<Tout*>(a.o), a.T, a.H);
    return hipGetLastError();
}

template <int DK, int DV>
static hipError_t launch_steps_d(const DecodeArgs& a) {
    if (a.in_bf16) {
        return a.out_bf16 ? launch_steps_t<DK, DV, bf16_t, bf16_t>(a)
                          : launch_steps_t<DK, DV, bf16_t, float>(a);
    }
    return a.out_bf16 ? launch_steps_t<DK, DV, float, bf16_t>(a)
                      : launch_steps_t<DK, DV, float, float>(a);
}

hipError_t launch_steps(const DecodeArgs& a) {
    return dispatch_head_sizes(a.dk, a.dv, [&](auto DK, auto DV) {
        return launch_steps_d<decltype(DK)::value, decltype(DV)::value>(a);
    });
}

}  // namespace kda
