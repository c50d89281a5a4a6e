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
// wants many requests in flight (512 threads measured faster than 256).
template <int DK, int DV, int NT>
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

// T consecutive tokens per (sequence, head) with the state in place (the
// fused recurrent mode over a short run of tokens): the state is read once,
// kept in registers for the whole run and written once.  Token t's inputs
// sit at ((n T + t) H + h) of the [N, T, H, .] tensors.
//
// One wave owns CW (<= 32) columns of one state: lane l holds rows
// R rg .. R rg + R - 1 (rg = l / TPR) of 4 columns (16-byte pieces, so a row
// segment of the wave is CW * 4 contiguous bytes).
//
// The decay is not applied to the registers token by token.  With G_t the
// per-channel sum of the log-gates since a reference point and
// E_t = Diag(exp G_t), the wave holds S' = E_t^-1 S.  Then
//   (Diag(alpha_t) S_{t-1})^T k = S'^T (E_t k),  likewise for q,
//   S_t = E_t (S' + (E_t^-1 k) u^T),
// so a token costs three fp32 operations per state element (two dot
// products and the rank-1 write) instead of four.  Every term of S' is
// scaled back by exp(G_T - G_t) <= 1 when E_T is applied, so rounding stays
// relative to the terms, as in the plain recurrence.  The per-channel
// vectors E_t k, E_t^-1 k and E_t q are formed once per wave (NE channels
// per lane) and shared through the wave's own slice of LDS: the lanes of a
// row group hold the same rows, so forming them per lane would repeat the
// work TPR times.  Once a channel's |G_t| passes FOLD (log2), E_t^-1 would
// leave fp32 range: the wave folds E_t into its rows (the plain decay) and
// restarts G from zero, which also turns a gate of -inf into an exact zero.
// E_T is folded in before the state is written back.
//
// The two reductions over rows (and q . k over channels) stay inside the
// wave: DPP row rotations inside each 16-lane row, then the row-pair swaps
// v_permlane16_swap / v_permlane32_swap across rows.  Only this wave touches
// its LDS slice and its LDS operations complete in order, so no barrier is
// needed; the next token's inputs are loaded at the start of each token.
template <int CTRL>
__device__ __forceinline__ float add_dpp(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}

// Sum over the four 16-lane rows of the wave (lanes that share l % 16).
__device__ __forceinline__ float sum_across_rows(float x) {
    const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
    const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
}

template <int TPR>
__device__ __forceinline__ float sum_row_groups(float x) {
    // lanes that share l % TPR; TPR in {4, 8}
    if (TPR == 4) x = add_dpp<0x124>(x);  // row_ror:4
    x = add_dpp<0x128>(x);                // row_ror:8
    return sum_across_rows(x);
}

__device__ __forceinline__ float sum_wave(float x) {
    x = add_dpp<0x121>(add_dpp<0x122>(add_dpp<0x124>(add_dpp<0x128>(x))));
    return sum_across_rows(x);
}

// NE consecutive channels from element i (i a multiple of NE).
template <int NE, typename T>
__device__ __forceinline__ void load_chan(const T* __restrict__ p, int64_t i, float (&x)[NE]) {
    static_assert(NE == 1 || NE == 2, "one or two channels per lane");
    if constexpr (NE == 2 && std::is_same<T, bf16_t>::value) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(p + i);
        x[0] = __uint_as_float(w << 16);
        x[1] = __uint_as_float(w & 0xffff0000u);
    } else if constexpr (NE == 2) {
        const float2 w = *reinterpret_cast<const float2*>(p + i);
        x[0] = w.x;
        x[1] = w.y;
    } else {
        x[0] = ld(p, i);
    }
}

template <int DK, int DV, typename Tin, typename Tout>
__global__ __launch_bounds__(256) void steps_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, float scale,
    float* __restrict__ state, Tout* __restrict__ o, int T, int H, int64_t items) {
    constexpr int CW = DV < 32 ? DV : 32;   // columns per wave
    constexpr int TPR = CW / 4;              // lanes per row
    constexpr int RG = 64 / TPR;             // row groups per wave
    constexpr int R = DK / RG;               // rows per lane
    constexpr int NCB = DV / CW;             // waves per state
    constexpr int NE = DK > 64 ? DK / 64 : 1;  // channels per lane in the per-channel phase
    constexpr int CL = DK / NE;                // lanes that hold channels
    constexpr float LOG2E = 1.4426950408889634f;
    constexpr float FOLD = 64.f;  // bound on |G| (log2) before E is folded into the rows
    static_assert(TPR == 4 || TPR == 8, "4 or 8 lanes per row");
    static_assert(R >= 1 && DK % RG == 0, "rows split evenly over the row groups");
    const int l = threadIdx.x & 63;
    const int64_t item = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (item >= items) return;  // whole wave
    const int64_t nh = item / NCB;
    const int col = static_cast<int>(item % NCB) * CW + 4 * (l % TPR);
    const int r0 = (l / TPR) * R;
    const int64_t n = nh / H, h = nh % H;
    float* S = state + nh * DK * DV + col;
    const bool chan = CL == 64 || l < CL;
    const int c0 = NE * l;

    // The wave's LDS slice: E k, E^-1 k, E q, and E when it is folded.
    __shared__ __align__(16) float xs[4][4][DK];
    float(*const xw)[DK] = xs[threadIdx.x >> 6];

    f32x4 s[R];
#pragma unroll
    for (int i = 0; i < R; ++i) s[i] = *reinterpret_cast<const f32x4*>(S + (r0 + i) * DV);

    float kc[NE], qc[NE], gc[NE], nk[NE], nq[NE], ng[NE], G[NE];
    f32x4 vt, nv;
    float bt, nb;
    auto fetch = [&](int t) {
        const int64_t tv = (n * T + t) * H + h;
        if (chan) {
            load_chan<NE>(k, tv * DK + c0, nk);
            load_chan<NE>(q, tv * DK + c0, nq);
            load_chan<NE>(g, tv * DK + c0, ng);
        } else {
#pragma unroll
            for (int j = 0; j < NE; ++j) nk[j] = nq[j] = ng[j] = 0.f;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) nv[c] = ld(v, tv * DV + col + c);
        nb = beta[tv];
    };
    // E of the current G into slot 3 and onto this lane's rows of S'.
    auto fold = [&]() {
        if (chan) {
#pragma unroll
            for (int j = 0; j < NE; ++j) xw[3][c0 + j] = __builtin_amdgcn_exp2f(G[j]);
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < R; ++i) s[i] *= xw[3][r0 + i];
#pragma unroll
        for (int j = 0; j < NE; ++j) G[j] = 0.f;
        __builtin_amdgcn_wave_barrier();
    };
#pragma unroll
    for (int j = 0; j < NE; ++j) G[j] = 0.f;
    if (T > 0) fetch(0);
    for (int t = 0; t < T; ++t) {
        const int64_t tv = (n * T + t) * H + h;
#pragma unroll
        for (int j = 0; j < NE; ++j) {
            kc[j] = nk[j];
            qc[j] = nq[j];
            gc[j] = ng[j];
        }
        vt = nv;
        bt = nb;
        fetch(t + 1 < T ? t + 1 : t);  // every iteration loads: exact load counting
        bool deep = false;
#pragma unroll
        for (int j = 0; j < NE; ++j) {
            G[j] += gc[j] * LOG2E;
            deep = deep || fabsf(G[j]) > FOLD;
        }
        if (__any(deep)) fold();
        float qk = 0.f;
        if (chan) {
#pragma unroll
            for (int j = 0; j < NE; ++j) {
                const float e = __builtin_amdgcn_exp2f(G[j]), ei = __builtin_amdgcn_exp2f(-G[j]);
                xw[0][c0 + j] = kc[j] * e;
                xw[1][c0 + j] = kc[j] * ei;
                xw[2][c0 + j] = qc[j] * e;
                qk += qc[j] * kc[j];
            }
        }
        __builtin_amdgcn_wave_barrier();
        f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < R; ++i) {
            pk += s[i] * xw[0][r0 + i];
            pq += s[i] * xw[2][r0 + i];
        }
        qk = sum_wave(qk);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            pk[c] = sum_row_groups<TPR>(pk[c]);
            pq[c] = sum_row_groups<TPR>(pq[c]);
        }
        const f32x4 u = bt * (vt - pk);
#pragma unroll
        for (int i = 0; i < R; ++i) s[i] += xw[1][r0 + i] * u;  // rank-1 write
        if (l < TPR) {
#pragma unroll
            for (int c = 0; c < 4; ++c) st(o, tv * DV + col + c, scale * (pq[c] + qk * u[c]));
        }
        __builtin_amdgcn_wave_barrier();  // this token's slice reads before the next token's writes
    }
    fold();
#pragma unroll
    for (int i = 0; i < R; ++i) __builtin_nontemporal_store(s[i], reinterpret_cast<f32x4*>(S + (r0 + i) * DV));
}

template <int DK, int DV, typename Tin, typename Tout>
static hipError_t launch_steps_t(const DecodeArgs& a) {
    constexpr int NCB = DV / (DV < 32 ? DV : 32);
    const int64_t items = static_cast<int64_t>(a.N) * a.H * NCB;
    hipLaunchKernelGGL((steps_kernel<DK, DV, Tin, Tout>), dim3(static_cast<uint32_t>((items + 3) / 4)),
                       dim3(256), 0, a.stream, static_cast<const Tin*>(a.q), static_cast<const Tin*>(a.k),
                       static_cast<const Tin*>(a.v), a.g, a.beta, a.scale, a.state,
                       static_cast<Tout*>(a.o), a.T, a.H, items);
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
    // the matrix-core form: its per-sub-chunk buffer ranges and offsets
    // (up to 8 H d_k 4 bytes) stay below 2^31 for H <= 2^18
    if (a.dk == 128 && a.dv == 128 && a.H <= (1 << 18)) return launch_steps_mfma(a);
    return dispatch_head_sizes(a.dk, a.dv, [&](auto DK, auto DV) {
        return launch_steps_d<decltype(DK)::value, decltype(DV)::value>(a);
    });
}

}  // namespace kda
