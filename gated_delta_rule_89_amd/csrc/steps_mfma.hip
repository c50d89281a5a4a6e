// Short runs (T <= 64 tokens per sequence, state in place) for d_k = d_v = 128
// on the matrix cores: the run is taken 8 tokens at a time in the chunk form
// of the recurrence ("Understanding Kimi Delta Attention", section
// "Understanding the Chunkwise Algorithm"; the fused recurrent mode of
// section "Two execution modes" computes the same values token by token).
//
// For a sub-chunk of C = 8 tokens with start state S (d_k x d_v), per-channel
// cumulative log-gates G_t from the sub-chunk start, gamma_t = exp(G_t):
//   K~ = k gamma,  Q~ = q gamma,  K^ = k / gamma,  K- = k gamma_C / gamma
//   A_ts = beta_t K~_t . K^_s  (s < t),   P_ts = Q~_t . K^_s  (s <= t)
//   U = (I + A)^-1 Diag(beta) (V - K~ S)
//   o = scale (Q~ S + P U),   S <- Diag(gamma_C) S + K-^T U
// (u_t = beta_t (v_t - (Diag(alpha_t) S_{t-1})^T k_t) unrolled over the
// sub-chunk).  Every product is fp32 MFMA (16x16x4) with fp32 accumulation,
// so results agree with the token-by-token recurrence to fp32 rounding.
//
// One workgroup of 4 waves per (sequence, head); wave w owns state columns
// 32 w .. 32 w + 31 as two 16-column MFMA tiles (column 32 w + 2 n + nt of
// tile nt at tile column n, so a lane's two tiles are adjacent columns).
// The state lives in MFMA accumulators, lane l holding rows
// 16 mt + 4 (l / 16) + i of tile column l % 16 (D layout).  Read as the B
// operand of the next sub-chunk's [K~; Q~] S product, register i of tile mt
// is the K-step whose 4 channels are 16 mt + 4 g + i (g = l / 16): the
// contraction runs over the channels in that order, and the A operand
// supplies the same order (a lane's 4 K-steps of a tile are 4 consecutive
// channels, one 16-byte LDS read).  The 16 rows of [K~; Q~] are permuted
// (row 4 j + i: K~ of token j and 4 + j for i = 0, 1, Q~ of j and 4 + j for
// i = 2, 3) so that the product's D tile holds, in lane group g, exactly
// the two tokens g and 4 + g that the next products take as B-operand
// K-steps: no data moves between lanes between the products.
//
// Per sub-chunk: (A) each wave forms the gate factors of 32 channels and
// writes the operand rows to LDS; the channel-split partial Grams (8 MFMAs
// per wave) go to LDS; barrier.  (B) every wave sums the partials, forms
// T = (I + A)^-1 = (I + N)(I + N^2)(I + N^4) with N = -A (A is strictly
// lower, N^8 = 0) and P T by 8 x 8 products on 64 lanes, then runs
// [K~; Q~] S (64 MFMAs), [T; P T] X with X = Diag(beta)(V - K~ S) giving U
// and o together (4 MFMAs), and the state update (32 MFMAs); barrier.
//
// K^ = k / gamma leaves fp32 range when a channel forgets nearly everything
// inside the sub-chunk.  A wave whose channels' gate total passes 2^-110
// (log2 units: -110) forms its partial Grams entry by entry instead, with
// exp(G_t - G_s) <= 1 from the exponents themselves.  Per-token log-gates
// below -100 are taken as -100 (alpha = e^-100 is zero next to any fp32
// state entry) so that every exponent difference stays finite.
#include "kda_internal.h"
#include "mfma_f32.h"

namespace kda {
namespace stepsm {

using namespace f32m;

constexpr int D = 128;     // d_k = d_v
constexpr int C = 8;       // tokens per sub-chunk
constexpr int RS = 132;    // padded stride (floats) of the 128-channel operand rows
constexpr int KBS = 10;    // stride of the K-^T rows (8 token slots; 10 spreads the banks)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float GMIN = -144.26950408889634f;  // -100 nats in log2 units
constexpr float SAFE = 110.f;                 // -G_C (log2) up to which K^ stays in range

struct Smem {
    float kq[16][RS];        // [K~; Q~] rows in the permuted order
    float kc[C][RS];         // K^ by token
    float kb[D][KBS];        // K-^T: channel row, token t at slot 2 (t % 4) + t / 4
    float gc[D];             // gamma_C
    float beta[C];
    float gp[4][16][16];     // the waves' partial Grams: [row of [K~; Q~]][token s]
    float mat[4][4][C * C];  // per wave: the 8 x 8 products
    float raw[4][3][C][32];  // per wave, direct Grams only: k, q, G (log2) of its channels
};

template <typename Tin, typename Tout>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void steps_mfma_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, float scale,
    float* __restrict__ state, Tout* __restrict__ o, int T, int H) {
    __shared__ __align__(16) Smem sm;
    const int tid = threadIdx.x, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = l & 15, g4 = l >> 4;
    const int nh = blockIdx.x;  // n H + h
    const int n = nh / H, h = nh - n * H;
    const int col = 32 * w + 2 * r16;  // tile nt holds column col + nt
    float* S = state + static_cast<int64_t>(nh) * D * D + col;

    f4 acc[8][2];  // acc[mt][nt][i] = S[16 mt + 4 g4 + i][col + nt]
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f2 x = *reinterpret_cast<const f2*>(S + (16 * mt + 4 * g4 + i) * D);
            acc[mt][0][i] = x[0];
            acc[mt][1][i] = x[1];
        }

    const int cl = l & 31, cw = 32 * w + cl;  // phase A: channel cw, tokens 4 hs .. 4 hs + 3
    const int hs = l >> 5;
    const int a8 = l >> 3, b8 = l & 7;        // lane (row, column) of the 8 x 8 matrices
    float* const mw = &sm.mat[w][0][0];
    const int64_t tok0 = static_cast<int64_t>(n) * T;  // token t of the run: ((tok0 + t) H + h)

    for (int t0 = 0; t0 < T; t0 += C) {
        const int nv = T - t0 < C ? T - t0 : C;  // real tokens in this sub-chunk
        // token t of the sub-chunk at element t H D + c from its first token:
        // the buffers end after token nv - 1, so later tokens read zeros
        const int64_t first = (tok0 + t0) * H + h;
        const uint32_t span = static_cast<uint32_t>(nv) * H * D;
        const auto rk = rsrc(k + first * D, span * sizeof(Tin));
        const auto rq = rsrc(q + first * D, span * sizeof(Tin));
        const auto rv = rsrc(v + first * D, span * sizeof(Tin));
        const auto rg = rsrc(g + first * D, span * 4u);
        const auto ro = rsrc(o + first * D, span * sizeof(Tout));
        // ---- (A) gate factors of channel cw, tokens 4 hs + j ----
        float kx[4], qx[4], G2[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t e = static_cast<uint32_t>(4 * hs + j) * H * D + cw;
            kx[j] = bld(rk, e, k);
            qx[j] = bld(rq, e, q);
            G2[j] = fmaxf(bld(rg, e, g) * LOG2E, GMIN);
        }
        G2[1] += G2[0];
        G2[2] += G2[1];
        G2[3] += G2[2];
        // lanes 0-31 hold tokens 0-3 and lanes 32-63 tokens 4-7 of the same channels
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(G2[3]), __float_as_uint(G2[3]), false, false);
        const float lo = __uint_as_float(p[0]), hi = __uint_as_float(p[1]);
        const float GC = lo + hi;
        if (hs) {
#pragma unroll
            for (int j = 0; j < 4; ++j) G2[j] += lo;
        }
        const bool direct = __any(-GC > SAFE);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float e = __builtin_amdgcn_exp2f(G2[j]);
            sm.kq[4 * j + hs][cw] = kx[j] * e;
            sm.kq[4 * j + 2 + hs][cw] = qx[j] * e;
            sm.kc[4 * hs + j][cw] = kx[j] * __builtin_amdgcn_exp2f(-G2[j]);
            sm.kb[cw][2 * j + hs] = kx[j] * __builtin_amdgcn_exp2f(GC - G2[j]);
        }
        if (!hs) sm.gc[cw] = __builtin_amdgcn_exp2f(GC);
        if (w == 0 && l < C) sm.beta[l] = bld(rsrc(beta + first, static_cast<uint32_t>(nv) * H * 4u), l * H, beta);
        if (direct) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sm.raw[w][0][4 * hs + j][cl] = kx[j];
                sm.raw[w][1][4 * hs + j][cl] = qx[j];
                sm.raw[w][2][4 * hs + j][cl] = G2[j];
            }
        }
        __builtin_amdgcn_wave_barrier();  // this wave's rows of the tiles are written

        // partial Grams over this wave's 32 channels: D[4 g4 + i][s = r16]
        f4 gacc = {0.f, 0.f, 0.f, 0.f};
        if (!direct) {
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) {
                const int c0 = 16 * (2 * w + mi) + 4 * g4;
                const f4 av = *reinterpret_cast<const f4*>(&sm.kq[r16][c0]);
                f4 bv = *reinterpret_cast<const f4*>(&sm.kc[r16 & 7][c0]);
                if (r16 >= C) bv = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < 4; ++i) gacc = mfma4(av[i], bv[i], gacc);
            }
        } else {
            // entry by entry: row 4 g4 + i is K~ (i < 2) or Q~ of token
            // g4 + 4 (i & 1); column s = r16; exp(G_t - G_s) <= 1 where used
            const int s = r16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = g4 + 4 * (i & 1);
                const bool use = s < C && ((i < 2) ? s < t : s <= t);
                float acc1 = 0.f;
                if (use) {
                    const float* xt = sm.raw[w][i < 2 ? 0 : 1][t];
                    const float* gt = sm.raw[w][2][t];
                    const float* ks = sm.raw[w][0][s];
                    const float* gs = sm.raw[w][2][s];
#pragma unroll 4
                    for (int c = 0; c < 32; ++c)
                        acc1 += xt[c] * ks[c] * __builtin_amdgcn_exp2f(fminf(gt[c] - gs[c], 0.f));
                }
                gacc[i] = acc1;
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.gp[w][4 * g4 + i][r16] = gacc[i];
        __syncthreads();

        // ---- (B) ----
        // N = -A and P on lane (a8, b8); T = (I + N)(I + N^2)(I + N^4); P T
        {
            const int rk = 4 * (a8 & 3) + (a8 >> 2);  // row of K~ of token a8 in [K~; Q~]
            float gk = 0.f, gq = 0.f;
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) {
                gk += sm.gp[ww][rk][b8];
                gq += sm.gp[ww][rk + 2][b8];
            }
            const float nab = b8 < a8 ? -sm.beta[a8] * gk : 0.f;
            const float pab = b8 <= a8 ? gq : 0.f;
            solve8(mw, nab, pab, a8, b8, l);
        }

        // [K~; Q~] S
        f4 y[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const f4 av = *reinterpret_cast<const f4*>(&sm.kq[r16][16 * mt + 4 * g4]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) y[nt] = mfma4(av[i], acc[mt][nt][i], y[nt]);
        }

        // X = Diag(beta)(V - K~ S) for tokens g4 and 4 + g4; [T; P T] X
        const float bg = sm.beta[g4], b4 = sm.beta[4 + g4];
        const uint32_t eg = static_cast<uint32_t>(g4) * H * D + col;      // token g4, column col
        const uint32_t e4 = static_cast<uint32_t>(4 + g4) * H * D + col;  // token 4 + g4
        const f2 vg = bld2(rv, eg, v), v4 = bld2(rv, e4, v);
        // A operand of [T; P T]: row r16 = 4 g' + i' (i' < 2: T, else P T; token g' + 4 (i' & 1))
        const int ra = (r16 >> 2) + 4 * (r16 & 1);
        const float* const Mt = (r16 & 2) ? mw + 128 : mw + 64;
        const float m0 = Mt[8 * ra + g4], m1 = Mt[8 * ra + 4 + g4];
        f4 z[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const float xg = bg * (vg[nt] - y[nt][0]);
            const float x4 = b4 * (v4[nt] - y[nt][1]);
            z[nt] = f4{0.f, 0.f, y[nt][2], y[nt][3]};
            z[nt] = mfma4(m0, xg, z[nt]);
            z[nt] = mfma4(m1, x4, z[nt]);
        }
        // o of tokens g4 and 4 + g4 (rows 2 and 3), columns col, col + 1
        bst2(ro, eg, f2{scale * z[0][2], scale * z[1][2]}, o);
        bst2(ro, e4, f2{scale * z[0][3], scale * z[1][3]}, o);

        // S <- Diag(gamma_C) S + K-^T U  (U of tokens g4, 4 + g4 in rows 0, 1)
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const f4 gv = *reinterpret_cast<const f4*>(&sm.gc[16 * mt + 4 * g4]);
            const f2 kv = *reinterpret_cast<const f2*>(&sm.kb[16 * mt + r16][2 * g4]);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                acc[mt][nt] *= gv;
                acc[mt][nt] = mfma4(kv[0], z[nt][0], acc[mt][nt]);
                acc[mt][nt] = mfma4(kv[1], z[nt][1], acc[mt][nt]);
            }
        }
        __syncthreads();  // the tiles are rewritten by the next sub-chunk
    }

#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_nontemporal_store(f2{acc[mt][0][i], acc[mt][1][i]},
                                        reinterpret_cast<f2*>(S + (16 * mt + 4 * g4 + i) * D));
}

template <typename Tin, typename Tout>
hipError_t launch_t(const DecodeArgs& a) {
    hipLaunchKernelGGL((steps_mfma_kernel<Tin, Tout>), dim3(static_cast<uint32_t>(a.N * a.H)), dim3(256), 0,
                       a.stream, static_cast<const Tin*>(a.q), static_cast<const Tin*>(a.k),
                       static_cast<const Tin*>(a.v), a.g, a.beta, a.scale, a.state, static_cast<Tout*>(a.o),
                       a.T, a.H);
    return hipGetLastError();
}

}  // namespace stepsm

hipError_t launch_steps_mfma(const DecodeArgs& a) {
    if (a.dk != stepsm::D || a.dv != stepsm::D) return hipErrorInvalidValue;
    if (a.in_bf16) {
        return a.out_bf16 ? stepsm::launch_t<bf16_t, bf16_t>(a) : stepsm::launch_t<bf16_t, float>(a);
    }
    return a.out_bf16 ? stepsm::launch_t<float, bf16_t>(a) : stepsm::launch_t<float, float>(a);
}

}  // namespace kda
