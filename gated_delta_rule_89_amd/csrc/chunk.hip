// Chunkwise KDA prefill on gfx950 MFMA (bf16 q/k/v, d_k = d_v = 128).
//
// Math ("Understanding Kimi Delta Attention", section "The Chunkwise DPLR
// Algorithm": fixed-size chunks, small matrix products, results equal to the
// sequential recurrence of section "The KDA Recurrence").  For one chain and
// a chunk of C tokens starting from state S (rows = key channels), with
// Gamma_r = sum_{s<=r} g_s (per channel, inside the chunk) and Lambda_r =
// exp(Gamma_r):
//
//   A    = StrictLower(Diag(beta) (Lambda k)(k / Lambda)^T)     C x C
//   P    = Lower_incl((Lambda q)(k / Lambda)^T)                 C x C
//   T    = (I + A)^-1 Diag(beta)
//   W    = T (Lambda k),   U = T v
//   Delta = U - W S
//   O    = scale (Q~ S + P Delta),             Q~ = Lambda q
//   S   <- Diag(Lambda_last) S + K-bar^T Delta,  K-bar = (Lambda_last / Lambda) k
//
// so one chunk maps S to (Diag(Lambda_last) - K-bar^T W) S + K-bar^T U: a
// diagonal-plus-low-rank transition, the structure named on that page.
//
// Design on this GPU:
//  * C = 32 tokens per chunk, split in two 16-token sub-blocks; a workgroup of
//    4 waves owns one (sequence, head) chain; LDS use is ~63 KB so two chains
//    share a CU.
//  * Gate exponents stay in range: inside a sub-block every factor is taken
//    relative to the sub-block start, across sub-blocks relative to the end
//    of the earlier one, so all factors are <= 1 except the in-block
//    exp(-Gamma) of the diagonal Gram blocks.  Those two diagonal blocks run
//    on split bf16 operands (hi + lo, three MFMAs) that keep fp32 range; every
//    other product runs on fp16 MFMA with fp32 accumulation.
//  * Columns of S are independent, so the state pass is split by columns:
//    wave w owns d_v columns [32w, 32w+32) of S, U, Delta and O.  S lives in
//    MFMA accumulators for the whole chain; its fp16 copy and Delta's are fed
//    back as MFMA operands straight from the accumulator registers, using a
//    k-order permutation that the gate-side operands read from LDS follow too.
//  * Value-side fp16 operands (S, v, Delta) carry a per-wave power-of-two scale
//    chosen every chunk from max(|S|, |v|), which keeps them inside fp16 range
//    and away from subnormals; the scale is exact and is removed in fp32.
#include "dev_common.h"
#include "kda_internal.h"

namespace kda {
namespace chunkk {

constexpr int C = 32;   // tokens per chunk
constexpr int SB = 16;  // tokens per sub-block
constexpr int D = 128;  // head size (d_k = d_v)
constexpr int QP = 136; // row stride (halves) of [token][channel] tiles
constexpr int TP = 40;  // row stride (halves) of [x][token] tiles
constexpr int GP = 17;  // row stride (floats) of 16x16 Gram tiles

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// Gram tiles: A00, P00, A11, P11, A10, P10.
enum { GA00 = 0, GP00 = 1, GA11 = 2, GP11 = 3, GA10 = 4, GP10 = 5 };

struct alignas(16) Smem {
    _Float16 qt[C][QP];      // Q~ = Lambda q                 [token][channel]
    _Float16 kbt[D][TP];     // K-bar^T                       [channel][token]
    _Float16 ktt[D][TP];     // K~^T = (Lambda k)^T           [channel][token]
    _Float16 r0[SB][QP];     // k exp(Gamma_end0 - Gamma), tokens 0..15   [token][channel]
    _Float16 t[C][TP];       // T = (I + A)^-1 Diag(beta)     [token][token]
    _Float16 p[C][TP];       // P                             [token][token]
    uint16_t v[C][QP];       // v tile (bf16 bits)            [token][column]
    float gp[2][6][SB][GP];  // Gram partial sums, one per channel half
    float x[2][SB][GP];      // (I + A_II)^-1 for the two diagonal blocks
    float tot[2][D];         // per-channel sum of g over each sub-block
    float lam[D];            // Lambda_last = exp(Gamma over the chunk)
    float beta[C];
};

__device__ __forceinline__ f4 mfma16(h8 a, h8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfmab(b8 a, b8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Value of lane i - n of the same 16-lane DPP row (0 for i < n).
template <int N>
__device__ __forceinline__ float row_shr(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 | N, 0xf, 0xf, true));
}

// Inclusive prefix sum over the 16 lanes of a DPP row.
__device__ __forceinline__ float row_scan16(float x) {
    x += row_shr<1>(x);
    x += row_shr<2>(x);
    x += row_shr<4>(x);
    x += row_shr<8>(x);
    return x;
}

__device__ __forceinline__ float wave_max(float m) {
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) m = fmaxf(m, __shfl_xor(m, s));
    return m;
}

__device__ __forceinline__ h8 cat(h4 a, h4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ void unpack_bf16x8(u4 w, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[2 * i] = __uint_as_float(w[i] << 16);
        out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

template <typename Tout>
__global__ __launch_bounds__(256, 2) void chunk_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ g,
    const float* __restrict__ beta, float scale, const float* __restrict__ h0,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ perm, int T, int H,
    Tout* __restrict__ o, float* __restrict__ hT) {
    __shared__ Smem sm;
    const int tid = threadIdx.x;
    const int w = tid >> 6;      // wave
    const int l = tid & 63;      // lane
    const int r = l & 15;        // MFMA row / column index
    const int g4 = l >> 4;       // MFMA k group
    const int I = w >> 1;        // gate phase: sub-block of this wave
    const int hh = w & 1;        // gate phase: channel half of this wave

    const int rank = blockIdx.x / H;
    const int h = blockIdx.x - rank * H;
    const int n = perm ? perm[rank] : rank;
    int64_t t0, t1;
    if (cu) {
        t0 = cu[n];
        t1 = cu[n + 1];
    } else {
        t0 = static_cast<int64_t>(n) * T;
        t1 = t0 + T;
    }
    const int64_t sbase = (static_cast<int64_t>(n) * H + h) * D * D;
    const int colw = 32 * w;  // first state column of this wave

    // State: S[16 rt + 4 g4 + i][colw + 16 ct + r] in S[rt][ct][i].
    f4 S[8][2];
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[rt][ct][i] = h0 ? h0[sbase + (16 * rt + 4 * g4 + i) * D + colw + 16 * ct + r] : 0.f;

    for (int64_t c0 = t0; c0 < t1; c0 += C) {
        const int valid = static_cast<int>(t1 - c0 < C ? t1 - c0 : C);

        // ---------------- gate phase 1: loads, cumulative gates, diagonal Grams
        const int tok = SB * I + r;
        const bool in = tok < valid;
        const int64_t rowq = ((c0 + tok) * H + h) * D;
        float kf[16], qf[16], gl[16];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int ch = 64 * hh + 32 * ks + 8 * g4;
            u4 kw = {0, 0, 0, 0}, qw = {0, 0, 0, 0};
            f4 ga = {0.f, 0.f, 0.f, 0.f}, gb = {0.f, 0.f, 0.f, 0.f};
            if (in) {
                kw = *reinterpret_cast<const u4*>(k + rowq + ch);
                qw = *reinterpret_cast<const u4*>(q + rowq + ch);
                ga = *reinterpret_cast<const f4*>(g + rowq + ch);
                gb = *reinterpret_cast<const f4*>(g + rowq + ch + 4);
            }
            unpack_bf16x8(kw, kf + 8 * ks);
            unpack_bf16x8(qw, qf + 8 * ks);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                gl[8 * ks + m] = ga[m];
                gl[8 * ks + 4 + m] = gb[m];
            }
        }
        float tot[16], L[16], Lq[16], Rb[16];
        f4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            b8 lh, ll, qh, ql, rh, rl;
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int e = 8 * ks + m;
                const float G = row_scan16(gl[e]);      // Gamma relative to the sub-block start
                tot[e] = __shfl(G, 15, 16);             // sum over the sub-block
                const float e1 = gate_exp(G);           // <= 1
                const float e2 = gate_exp(-G);          // >= 1 (diagonal blocks only)
                const float e3 = gate_exp(tot[e] - G);  // <= 1
                L[e] = kf[e] * e1;
                Lq[e] = qf[e] * e1;
                Rb[e] = kf[e] * e3;
                const float R = kf[e] * e2;
                lh[m] = static_cast<__bf16>(L[e]);
                ll[m] = static_cast<__bf16>(L[e] - static_cast<float>(lh[m]));
                qh[m] = static_cast<__bf16>(Lq[e]);
                ql[m] = static_cast<__bf16>(Lq[e] - static_cast<float>(qh[m]));
                rh[m] = static_cast<__bf16>(R);
                rl[m] = static_cast<__bf16>(R - static_cast<float>(rh[m]));
            }
            accA = mfmab(lh, rh, accA);
            accA = mfmab(lh, rl, accA);
            accA = mfmab(ll, rh, accA);
            accP = mfmab(qh, rh, accP);
            accP = mfmab(qh, rl, accP);
            accP = mfmab(ql, rh, accP);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sm.gp[hh][2 * I][4 * g4 + i][r] = accA[i];
            sm.gp[hh][2 * I + 1][4 * g4 + i][r] = accP[i];
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int ch = 64 * hh + 32 * ks + 8 * g4;
            if (I == 0) {
                h8 rv;
#pragma unroll
                for (int m = 0; m < 8; ++m) rv[m] = static_cast<_Float16>(Rb[8 * ks + m]);
                *reinterpret_cast<h8*>(&sm.r0[r][ch]) = rv;
            }
            if (r == 15) {
#pragma unroll
                for (int m = 0; m < 8; ++m) sm.tot[I][ch + m] = tot[8 * ks + m];
            }
        }
        __syncthreads();  // B1

        // ---------------- gate phase 2: chunk-referenced operands, cross-block Grams, v, beta
        {
            f4 a10 = {0.f, 0.f, 0.f, 0.f}, p10 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int ch = 64 * hh + 32 * ks + 8 * g4;
                h8 qv, l16, q16;
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    const int e = 8 * ks + m;
                    const float t0c = sm.tot[0][ch + m], t1c = sm.tot[1][ch + m];
                    const float base = I ? t0c : 0.f;                   // Gamma at the sub-block start
                    const float fb = gate_exp(base);                    // <= 1
                    const float fl = gate_exp(t0c + t1c - base - tot[e]);  // <= 1
                    qv[m] = static_cast<_Float16>(Lq[e] * fb);
                    sm.ktt[ch + m][tok] = static_cast<_Float16>(L[e] * fb);
                    sm.kbt[ch + m][tok] = static_cast<_Float16>(Rb[e] * fl);
                    if (I == 0 && r == 0) sm.lam[ch + m] = gate_exp(t0c + t1c);
                    l16[m] = static_cast<_Float16>(L[e]);
                    q16[m] = static_cast<_Float16>(Lq[e]);
                }
                *reinterpret_cast<h8*>(&sm.qt[tok][ch]) = qv;
                if (I == 1) {
                    const h8 rv = *reinterpret_cast<const h8*>(&sm.r0[r][ch]);
                    a10 = mfma16(l16, rv, a10);
                    p10 = mfma16(q16, rv, p10);
                }
            }
            if (I == 1) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sm.gp[hh][GA10][4 * g4 + i][r] = a10[i];
                    sm.gp[hh][GP10][4 * g4 + i][r] = p10[i];
                }
            }
            if (tid < C) sm.beta[tid] = tid < valid ? beta[(c0 + tid) * H + h] : 0.f;
            {
                const int vt = tid >> 3, vc = (tid & 7) * 16;
                u4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
                if (vt < valid) {
                    const uint16_t* src = v + ((c0 + vt) * H + h) * D + vc;
                    a = *reinterpret_cast<const u4*>(src);
                    b = *reinterpret_cast<const u4*>(src + 8);
                }
                *reinterpret_cast<u4*>(&sm.v[vt][vc]) = a;
                *reinterpret_cast<u4*>(&sm.v[vt][vc + 8]) = b;
            }
        }
        __syncthreads();  // B2

        // ---------------- solve: diagonal block inverses (waves 0, 1), P (waves 2, 3)
        if (w < 2) {
            const int J = w;  // diagonal block
            const int j = r;  // column of the inverse owned by this lane
            float xcol[SB];
#pragma unroll
            for (int i = 0; i < SB; ++i) {
                float s = (i == j) ? 1.f : 0.f;
                const float bi = sm.beta[SB * J + i];
#pragma unroll
                for (int m = 0; m < i; ++m)
                    s -= bi * (sm.gp[0][2 * J][i][m] + sm.gp[1][2 * J][i][m]) * xcol[m];
                xcol[i] = s;
            }
            if (g4 == 0) {
                const float bj = sm.beta[SB * J + j];
#pragma unroll
                for (int i = 0; i < SB; ++i) {
                    sm.x[J][i][j] = xcol[i];
                    sm.t[SB * J + i][SB * J + j] = static_cast<_Float16>(xcol[i] * bj);
                }
            }
        } else {
            const int t2 = tid - 128;
#pragma unroll
            for (int qq = 0; qq < 8; ++qq) {
                const int e = t2 + 128 * qq;
                const int R = e >> 5, Cc = e & 31;
                float val = 0.f;
                if (Cc <= R) {
                    if (R < SB) val = sm.gp[0][GP00][R][Cc] + sm.gp[1][GP00][R][Cc];
                    else if (Cc >= SB) val = sm.gp[0][GP11][R - SB][Cc - SB] + sm.gp[1][GP11][R - SB][Cc - SB];
                    else val = sm.gp[0][GP10][R - SB][Cc] + sm.gp[1][GP10][R - SB][Cc];
                }
                sm.p[R][Cc] = static_cast<_Float16>(val);
            }
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
                const int e = t2 + 128 * qq;
                sm.t[e >> 4][SB + (e & 15)] = static_cast<_Float16>(0.f);
            }
        }
        __syncthreads();  // B3

        // ---------------- solve: off-diagonal block X10 = -X11 A10 X00 (every wave: 4 columns)
        {
            const int i = r, j = 4 * w + g4;
            const float bi = sm.beta[SB + i];
            float y = 0.f;
#pragma unroll
            for (int m = 0; m < SB; ++m)
                y += bi * (sm.gp[0][GA10][i][m] + sm.gp[1][GA10][i][m]) * sm.x[0][m][j];
            float x10 = 0.f;
#pragma unroll
            for (int m = 0; m < SB; ++m) x10 -= sm.x[1][i][m] * __shfl(y, (l & 48) | m);
            sm.t[SB + i][j] = static_cast<_Float16>(x10 * sm.beta[j]);
        }
        __syncthreads();  // B4

        // ---------------- state pass on this wave's 32 columns
        {
            // W^T = K~^T T^T, kept in registers as the A operand of W S.
            h8 tf[2];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) tf[rt] = *reinterpret_cast<const h8*>(&sm.t[16 * rt + r][8 * g4]);
            h8 wf[2][4];  // A operand of (-W) S: [token tile][channel k-step]
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                f4 wa[2][2];
#pragma unroll
                for (int hx = 0; hx < 2; ++hx) {
                    const h8 kt = *reinterpret_cast<const h8*>(&sm.ktt[16 * (2 * ks + hx) + r][8 * g4]);
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt) wa[hx][rt] = mfma16(kt, tf[rt], f4{0.f, 0.f, 0.f, 0.f});
                }
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        wf[rt][ks][m] = static_cast<_Float16>(-wa[0][rt][m]);
                        wf[rt][ks][4 + m] = static_cast<_Float16>(-wa[1][rt][m]);
                    }
            }

            // Value scale from max(|S|, |v|) over this wave's columns.
            float vv[2][8];
            float mx = 0.f;
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    vv[ct][m] = bf16_to_f32(sm.v[8 * g4 + m][colw + 16 * ct + r]);
                    mx = fmaxf(mx, fabsf(vv[ct][m]));
                }
#pragma unroll
            for (int rt = 0; rt < 8; ++rt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(S[rt][ct][i]));
            mx = wave_max(mx);
            int ex = 0;
            if (mx > 0.f && mx < 3.0e38f) {
                (void)frexpf(mx, &ex);
                ex = 10 - ex;
                ex = ex < -120 ? -120 : (ex > 120 ? 120 : ex);
            }
            const float sig = ldexpf(1.f, ex), isig = ldexpf(1.f, -ex);

            h8 s16[4][2];  // B operand of W S and Q~ S: [channel k-step][column tile]
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        s16[ks][ct][m] = static_cast<_Float16>(S[2 * ks][ct][m] * sig);
                        s16[ks][ct][4 + m] = static_cast<_Float16>(S[2 * ks + 1][ct][m] * sig);
                    }
            h8 v16[2];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int m = 0; m < 8; ++m) v16[ct][m] = static_cast<_Float16>(vv[ct][m] * sig);

            // Delta = T v - W S  (scaled by sig)
            f4 dl[2][2];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    f4 a = mfma16(tf[rt], v16[ct], f4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) a = mfma16(wf[rt][ks], s16[ks][ct], a);
                    dl[rt][ct] = a;
                }
            h8 d16[2];  // B operand (k = tokens, permuted)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    d16[ct][m] = static_cast<_Float16>(dl[0][ct][m]);
                    d16[ct][4 + m] = static_cast<_Float16>(dl[1][ct][m]);
                }

            // O = scale (Q~ S + P Delta)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                h8 qf8[4];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    qf8[ks] = cat(*reinterpret_cast<const h4*>(&sm.qt[16 * rt + r][32 * ks + 4 * g4]),
                                  *reinterpret_cast<const h4*>(&sm.qt[16 * rt + r][32 * ks + 16 + 4 * g4]));
                const h8 pf = cat(*reinterpret_cast<const h4*>(&sm.p[16 * rt + r][4 * g4]),
                                  *reinterpret_cast<const h4*>(&sm.p[16 * rt + r][16 + 4 * g4]));
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    f4 a = mfma16(pf, d16[ct], f4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) a = mfma16(qf8[ks], s16[ks][ct], a);
                    const float os = scale * isig;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int tt = 16 * rt + 4 * g4 + i;
                        if (tt < valid) st(o, ((c0 + tt) * H + h) * D + colw + 16 * ct + r, a[i] * os);
                    }
                }
            }

            // S <- Lambda_last S + K-bar^T Delta
#pragma unroll
            for (int rt = 0; rt < 8; ++rt) {
                const f4 lam = *reinterpret_cast<const f4*>(&sm.lam[16 * rt + 4 * g4]);
                const h8 kb = cat(*reinterpret_cast<const h4*>(&sm.kbt[16 * rt + r][4 * g4]),
                                  *reinterpret_cast<const h4*>(&sm.kbt[16 * rt + r][16 + 4 * g4]));
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    f4 a = S[rt][ct] * (lam * sig);
                    a = mfma16(kb, d16[ct], a);
                    S[rt][ct] = a * isig;
                }
            }
        }
    }

    if (hT) {
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    hT[sbase + (16 * rt + 4 * g4 + i) * D + colw + 16 * ct + r] = S[rt][ct][i];
    }
}

// Longest-sequence-first order of the N sequences (ties by index): the
// dispatcher hands workgroups out in index order, so launching long chains
// first gives a longest-processing-time schedule.
__global__ void lpt_plan_kernel(const int32_t* __restrict__ cu, int N, int32_t* __restrict__ perm) {
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N) return;
    const int len = cu[n + 1] - cu[n];
    int rank = 0;
    for (int m = 0; m < N; ++m) {
        const int lm = cu[m + 1] - cu[m];
        rank += (lm > len) || (lm == len && m < n);
    }
    perm[rank] = n;
}

}  // namespace chunkk

constexpr int kLptMaxSeqs = 16384;

size_t chunk_workspace_bytes(int B, int T, int H, int N, bool scan) {
    (void)B;
    (void)T;
    (void)H;
    (void)scan;
    return N <= kLptMaxSeqs ? ((static_cast<size_t>(N) * 4 + 255) / 256) * 256 : 0;
}

hipError_t launch_chunk(const PrefillArgs& a, bool scan) {
    (void)scan;
    const int32_t* perm = nullptr;
    if (a.cu && a.N > 1 && a.N <= kLptMaxSeqs) {
        int32_t* p = static_cast<int32_t*>(a.ws);
        hipLaunchKernelGGL(chunkk::lpt_plan_kernel, dim3((a.N + 255) / 256), dim3(256), 0, a.stream,
                           a.cu, a.N, p);
        perm = p;
    }
    const dim3 grid(static_cast<uint32_t>(a.N) * a.H);
    if (a.out_bf16) {
        hipLaunchKernelGGL(chunkk::chunk_kernel<bf16_t>, grid, dim3(256), 0, a.stream,
                           static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                           static_cast<const uint16_t*>(a.v), a.g, a.beta, a.scale, a.h0, a.cu, perm,
                           a.T, a.H, static_cast<bf16_t*>(a.o), a.hT);
    } else {
        hipLaunchKernelGGL(chunkk::chunk_kernel<float>, grid, dim3(256), 0, a.stream,
                           static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                           static_cast<const uint16_t*>(a.v), a.g, a.beta, a.scale, a.h0, a.cu, perm,
                           a.T, a.H, static_cast<float*>(a.o), a.hT);
    }
    return hipGetLastError();
}

}  // namespace kda
