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

#ifndef KDA_CHUNK_WG_PER_CU
#define KDA_CHUNK_WG_PER_CU 1  // chains resident per CU (sets the register budget)
#endif

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
    alignas(16) float a[2][SB][20];  // A_II^T: column m of Diag(beta) Gram in row m
    float etot[2][D];        // per-channel exp(sum of g over each sub-block)
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

// Maximum of a non-negative value over the wave: prefix maxima inside each
// 16-lane row, then across rows with the row broadcasts; lane 63 ends up with
// the total, which is read back as a wave-uniform value.
__device__ __forceinline__ float wave_max_nonneg(float m) {
    m = fmaxf(m, row_shr<1>(m));
    m = fmaxf(m, row_shr<2>(m));
    m = fmaxf(m, row_shr<4>(m));
    m = fmaxf(m, row_shr<8>(m));
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(m), __float_as_int(m), 0x142, 0xa, 0xf, false)));
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(m), __float_as_int(m), 0x143, 0xc, 0xf, false)));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 63));
}

__device__ __forceinline__ f4 mfma4(float a, float b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
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
__global__ __launch_bounds__(256, KDA_CHUNK_WG_PER_CU) void chunk_kernel(
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

    // State, kept as S * 2^ex: S[16 rt + 4 g4 + i][colw + 16 ct + r] in S[rt][ct][i].
    // ex is a per-wave exponent that keeps the fp16 copies of S and v in range.
    f4 S[8][2];
    int ex = 0;
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[rt][ct][i] = h0 ? h0[sbase + (16 * rt + 4 * g4 + i) * D + colw + 16 * ct + r] : 0.f;

    // Raw inputs of the next chunk, fetched one chunk ahead: k, q, g of this
    // lane's token and channels (gate layout), its beta, and two 16-byte
    // pieces of the v tile (staging layout).
    const int tok = SB * I + r;
    const int vt = tid >> 3, vc = (tid & 7) * 16;
    u4 kw[2], qw[2], va, vb;
    f4 ga[2], gb[2];
    float bt;
    auto fetch = [&](int64_t cs) {
        const int vld = static_cast<int>(t1 - cs < C ? t1 - cs : C);
        const bool in = tok < vld;
        const int64_t rowq = ((cs + tok) * H + h) * D;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int ch = 64 * hh + 32 * ks + 8 * g4;
            kw[ks] = u4{0, 0, 0, 0};
            qw[ks] = u4{0, 0, 0, 0};
            ga[ks] = f4{0.f, 0.f, 0.f, 0.f};
            gb[ks] = f4{0.f, 0.f, 0.f, 0.f};
            if (in) {
                kw[ks] = *reinterpret_cast<const u4*>(k + rowq + ch);
                qw[ks] = *reinterpret_cast<const u4*>(q + rowq + ch);
                ga[ks] = *reinterpret_cast<const f4*>(g + rowq + ch);
                gb[ks] = *reinterpret_cast<const f4*>(g + rowq + ch + 4);
            }
        }
        bt = in ? beta[(cs + tok) * H + h] : 0.f;
        va = u4{0, 0, 0, 0};
        vb = u4{0, 0, 0, 0};
        if (vt < vld) {
            const uint16_t* src = v + ((cs + vt) * H + h) * D + vc;
            va = *reinterpret_cast<const u4*>(src);
            vb = *reinterpret_cast<const u4*>(src + 8);
        }
    };
    if (t0 < t1) fetch(t0);

    for (int64_t c0 = t0; c0 < t1; c0 += C) {
        const int valid = static_cast<int>(t1 - c0 < C ? t1 - c0 : C);

        // ---------------- gate phase 1: loads, cumulative gates, diagonal Grams
        h8 l16[2], q16[2], rb16[2];  // L, Lq, k exp(tot - G) as fp16 (k-step ks, slot m)
        {
            f4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int ch = 64 * hh + 32 * ks + 8 * g4;
                float kf[8], qf[8];
                unpack_bf16x8(kw[ks], kf);
                unpack_bf16x8(qw[ks], qf);
                b8 lh, ll, qh, ql, rh, rl;
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    const float G = row_scan16(m < 4 ? ga[ks][m] : gb[ks][m - 4]);  // Gamma from the sub-block start
                    const float e1 = gate_exp(G);            // <= 1
                    const float e2 = gate_exp(-G);           // >= 1
                    const float etot = __shfl(e1, 15, 16);   // exp(sum of g over the sub-block)
                    const float L = kf[m] * e1, Lq = qf[m] * e1, R = kf[m] * e2;
                    l16[ks][m] = static_cast<_Float16>(L);
                    q16[ks][m] = static_cast<_Float16>(Lq);
                    rb16[ks][m] = static_cast<_Float16>(R * etot);  // k exp(tot - G) <= 1
                    if (r == 15) sm.etot[I][ch + m] = etot;
                    lh[m] = static_cast<__bf16>(L);
                    ll[m] = static_cast<__bf16>(L - static_cast<float>(lh[m]));
                    qh[m] = static_cast<__bf16>(Lq);
                    ql[m] = static_cast<__bf16>(Lq - static_cast<float>(qh[m]));
                    rh[m] = static_cast<__bf16>(R);
                    rl[m] = static_cast<__bf16>(R - static_cast<float>(rh[m]));
                }
                accA = mfmab(lh, rh, accA);
                accA = mfmab(lh, rl, accA);
                accA = mfmab(ll, rh, accA);
                accP = mfmab(qh, rh, accP);
                accP = mfmab(qh, rl, accP);
                accP = mfmab(ql, rh, accP);
                if (I == 0) *reinterpret_cast<h8*>(&sm.r0[r][ch]) = rb16[ks];
            }
            // Row 4 g4 + i of the Gram tile is token 4 g4 + i of the sub-block: scale A by its beta.
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float bi = __shfl(bt, (l & 48) | (4 * g4 + i));
                sm.gp[hh][2 * I][4 * g4 + i][r] = accA[i] * bi;
                sm.gp[hh][2 * I + 1][4 * g4 + i][r] = accP[i];
            }
            if (hh == 0 && g4 == 0) sm.beta[tok] = bt;
        }
        __syncthreads();  // B1

        // ---------------- gate phase 2: chunk-referenced operands, cross-block Grams, v
        {
            f4 a10 = {0.f, 0.f, 0.f, 0.f}, p10 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int ch = 64 * hh + 32 * ks + 8 * g4;
                const f4 oa = *reinterpret_cast<const f4*>(&sm.etot[1 - I][ch]);
                const f4 ob = *reinterpret_cast<const f4*>(&sm.etot[1 - I][ch + 4]);
                h8 qv;
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    const float other = m < 4 ? oa[m] : ob[m - 4];  // exp(sum of g over the other sub-block)
                    const float L = static_cast<float>(l16[ks][m]), Lq = static_cast<float>(q16[ks][m]);
                    const float Rb = static_cast<float>(rb16[ks][m]);
                    // sub-block 0: Gamma_r = G, K-bar needs exp(tot1); sub-block 1: Gamma_r = tot0 + G
                    const float fq = I ? other : 1.f, fk = I ? 1.f : other;
                    qv[m] = static_cast<_Float16>(Lq * fq);
                    sm.ktt[ch + m][tok] = static_cast<_Float16>(L * fq);
                    sm.kbt[ch + m][tok] = static_cast<_Float16>(Rb * fk);
                }
                *reinterpret_cast<h8*>(&sm.qt[tok][ch]) = qv;
                if (I == 1) {
                    const h8 rv = *reinterpret_cast<const h8*>(&sm.r0[r][ch]);
                    a10 = mfma16(l16[ks], rv, a10);
                    p10 = mfma16(q16[ks], rv, p10);
                }
            }
            if (I == 1) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float bi = sm.beta[SB + 4 * g4 + i];
                    sm.gp[hh][GA10][4 * g4 + i][r] = a10[i] * bi;
                    sm.gp[hh][GP10][4 * g4 + i][r] = p10[i];
                }
            }
            if (tid < D) sm.lam[tid] = sm.etot[0][tid] * sm.etot[1][tid];
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
                const int e = tid + 256 * qq, J = e >> 8, i = (e >> 4) & 15, m = e & 15;
                sm.a[J][m][i] = sm.gp[0][2 * J][i][m] + sm.gp[1][2 * J][i][m];  // stored by column
            }
            *reinterpret_cast<u4*>(&sm.v[vt][vc]) = va;
            *reinterpret_cast<u4*>(&sm.v[vt][vc + 8]) = vb;
        }
        __syncthreads();  // B2

        // ---------------- solve: diagonal block inverses (waves 0, 1), P (waves 2, 3)
        if (w < 2) {
            const int J = w;  // diagonal block
            const int j = r;  // column of the inverse owned by this lane
            // Column j of (I + A_JJ)^-1 by forward substitution, column-oriented:
            // once x_m is final, every later row subtracts A[i][m] x_m (independent
            // updates).  Columns of A are read one step ahead.
            float xcol[SB];
#pragma unroll
            for (int i = 0; i < SB; ++i) xcol[i] = (i == j) ? 1.f : 0.f;
            f4 col[4], ncol[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) col[c] = *reinterpret_cast<const f4*>(&sm.a[J][0][4 * c]);
#pragma unroll
            for (int m = 0; m < SB; ++m) {
                if (m + 1 < SB) {
#pragma unroll
                    for (int c = 0; c < 4; ++c) ncol[c] = *reinterpret_cast<const f4*>(&sm.a[J][m + 1][4 * c]);
                }
                const float xm = xcol[m];
#pragma unroll
                for (int i = m + 1; i < SB; ++i) xcol[i] = fmaf(-col[i >> 2][i & 3], xm, xcol[i]);
#pragma unroll
                for (int c = 0; c < 4; ++c) col[c] = ncol[c];
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

        // ---------------- solve: off-diagonal block X10 = -X11 (A10 X00), fp32 MFMA on wave 0
        if (w == 0) {
            f4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int m = 4 * ks + g4;
                y = mfma4(sm.gp[0][GA10][r][m] + sm.gp[1][GA10][r][m], sm.x[0][m][r], y);
            }
            // y[i] = Y[4 g4 + i][r]; contract X11 Y with k index m = 4 g4 + ks
            f4 x10 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) x10 = mfma4(sm.x[1][r][4 * g4 + ks], y[ks], x10);
            const float bj = sm.beta[r];
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.t[SB + 4 * g4 + i][r] = static_cast<_Float16>(-x10[i] * bj);
        }
        __syncthreads();  // B4

        // ---------------- state pass on this wave's 32 columns
        if (c0 + C < t1) fetch(c0 + C);
        {
            // Exponent for this chunk from max(|S|, |v|) over the wave's columns.
            float mv = 0.f;
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int m = 0; m < 8; ++m)
                    mv = fmaxf(mv, fabsf(bf16_to_f32(sm.v[8 * g4 + m][colw + 16 * ct + r])));
            float ms = 0.f;
#pragma unroll
            for (int rt = 0; rt < 8; ++rt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i) ms = fmaxf(ms, fabsf(S[rt][ct][i]));
            const float mx = wave_max_nonneg(fmaxf(ms * ldexpf(1.f, -ex), mv));
            int nex = ex;
            if (mx > 0.f && mx < 3.0e38f) {
                int e2;
                (void)frexpf(mx, &e2);
                nex = 10 - e2;
                nex = nex < -120 ? -120 : (nex > 120 ? 120 : nex);
            }
            if (nex != ex) {  // wave-uniform
                const float f = ldexpf(1.f, nex - ex);
#pragma unroll
                for (int rt = 0; rt < 8; ++rt)
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) S[rt][ct] *= f;
                ex = nex;
            }
            const float sig = ldexpf(1.f, ex);

            h8 s16[4][2];  // B operand of W S and Q~ S: [channel k-step][column tile]
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        s16[ks][ct][m] = static_cast<_Float16>(S[2 * ks][ct][m]);
                        s16[ks][ct][4 + m] = static_cast<_Float16>(S[2 * ks + 1][ct][m]);
                    }

            // Delta = T v - W S (scaled), W = T K~ built per channel k-step from K~^T T^T.
            h8 tf[2];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) tf[rt] = *reinterpret_cast<const h8*>(&sm.t[16 * rt + r][8 * g4]);
            f4 dl[2][2];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                h8 v16;
#pragma unroll
                for (int m = 0; m < 8; ++m)
                    v16[m] = static_cast<_Float16>(bf16_to_f32(sm.v[8 * g4 + m][colw + 16 * ct + r]) * sig);
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) dl[rt][ct] = mfma16(tf[rt], v16, f4{0.f, 0.f, 0.f, 0.f});
            }
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
                for (int rt = 0; rt < 2; ++rt) {
                    h8 wf;
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        wf[m] = static_cast<_Float16>(-wa[0][rt][m]);
                        wf[4 + m] = static_cast<_Float16>(-wa[1][rt][m]);
                    }
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) dl[rt][ct] = mfma16(wf, s16[ks][ct], dl[rt][ct]);
                }
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
            const float os = scale * ldexpf(1.f, -ex);
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
                    Tout* op = o + ((c0 + 16 * rt + 4 * g4) * H + h) * D + colw + 16 * ct + r;
                    const int64_t stride = static_cast<int64_t>(H) * D;
                    if (valid == C) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) st(op, i * stride, a[i] * os);
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (16 * rt + 4 * g4 + i < valid) st(op, i * stride, a[i] * os);
                    }
                }
            }

            // S <- Lambda_last S + K-bar^T Delta  (all in the scaled units)
#pragma unroll
            for (int rt = 0; rt < 8; ++rt) {
                const f4 lam = *reinterpret_cast<const f4*>(&sm.lam[16 * rt + 4 * g4]);
                const h8 kb = cat(*reinterpret_cast<const h4*>(&sm.kbt[16 * rt + r][4 * g4]),
                                  *reinterpret_cast<const h4*>(&sm.kbt[16 * rt + r][16 + 4 * g4]));
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) S[rt][ct] = mfma16(kb, d16[ct], S[rt][ct] * lam);
            }
        }
    }

    if (hT) {
        const float un = ldexpf(1.f, -ex);
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    hT[sbase + (16 * rt + 4 * g4 + i) * D + colw + 16 * ct + r] = S[rt][ct][i] * un;
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
