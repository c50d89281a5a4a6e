// Chunked prefill for every supported head size (d_k, d_v in {16, 32, 64,
// 128}) and both input dtypes, in fp32 arithmetic throughout: the chunk form
// of the recurrence ("Understanding Kimi Delta Attention", section
// "Understanding the Chunkwise Algorithm") on sub-chunks of 8 tokens, every
// product on fp32 MFMA (16x16x4) with fp32 accumulation, so that results
// agree with the token-by-token recurrence (section "The KDA Recurrence") to
// fp32 rounding.  The matrix-core prefill on fp16 operands serves bf16 inputs
// at d_k = d_v = 128; this kernel serves fp32 inputs and the other head sizes.
//
// For a sub-chunk with start state S (d_k x d_v), per-channel cumulative
// log-gates G_t from the sub-chunk start and gamma_t = exp(G_t):
//   K~ = k gamma,  Q~ = q gamma,  K^ = k / gamma,  K- = k gamma_C / gamma
//   A_ts = beta_t K~_t . K^_s  (s < t),   P_ts = Q~_t . K^_s  (s <= t)
//   U = (I + A)^-1 Diag(beta) (V - K~ S)
//   o = scale (Q~ S + P U),   S <- Diag(gamma_C) S + K-^T U
//
// Columns of the state evolve independently once the gate-side products
// (A, T, P) are known, so each (sequence, head) chain is split over d_v / W
// workgroups, each owning W columns and forming the gate side itself.  A
// workgroup has three roles:
//   state waves (the first NS): the state columns in MFMA accumulators; for
//     W = 128 wave w owns columns 32 w .. 32 w + 31 as two 16-column tiles
//     (column 32 w + 2 n + nt of tile nt at tile column n), for W <= 64
//     columns 16 w .. 16 w + 15 as one tile.  Lane l holds rows
//     16 mt + 4 (l / 16) + i of tile column l % 16 (the MFMA D layout).
//     Read as the B operand of the next sub-chunk's [K~; Q~] S product,
//     register i of row tile mt is the K-step over channels
//     16 mt + 4 (l / 16) + i, and the A operand supplies the same order (a
//     lane's 4 K-steps of a tile are 4 consecutive channels, one 16-byte LDS
//     read).  The 16 rows of [K~; Q~] are permuted (row 4 j + i: K~ of tokens
//     j and 4 + j for i = 0, 1, Q~ of j and 4 + j for i = 2, 3) so that the D
//     tile of that product holds, in lane group g, exactly the tokens g and
//     4 + g that the next two products take as B-operand K-steps.
//   gate waves (one per 32-channel block): the factors of their block,
//     written to LDS as operand rows, and the partial Grams over those
//     channels (up to 8 MFMAs).
//   the solve (state wave 0, after its own products): sums the partial
//     Grams and forms T = (I + A)^-1 = (I + N)(I + N^2)(I + N^4) with N = -A
//     (strictly lower 8 x 8, N^8 = 0) and P T by 8 x 8 products.
// Iteration i runs them as a pipeline with one barrier: the state waves take
// sub-chunk i ([K~; Q~] S, [T; P T] X with X = Diag(beta)(V - K~ S), which
// gives U and o together, and the state update), then state wave 0 solves
// sub-chunk i + 1; the gate waves take sub-chunk i + 2.  Operand tiles are
// kept for three sub-chunks, partial Grams and solves for two, and every
// input is fetched two sub-chunks ahead.
//
// Strong forgetting: K^ = k / gamma leaves fp32 range when a channel forgets
// nearly everything inside the sub-chunk.  A block whose gate total passes
// 2^-110 forms its partial Grams entry by entry, with exp(G_t - G_s) <= 1
// taken from the exponents themselves.  Per-token log-gates below -100 are
// taken as -100 (alpha = e^-100 vanishes next to any fp32 state entry), so
// that every exponent difference stays finite.
#include "kda_internal.h"
#include "mfma_f32.h"

namespace kda {
namespace c8 {

using namespace f32m;

constexpr int C = 8;      // tokens per sub-chunk
constexpr int KBS = 10;   // stride of the K-^T rows (8 token slots; 10 spreads the banks)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float GMIN = -144.26950408889634f;  // -100 nats in log2 units
constexpr float SAFE = 110.f;                 // -G_C (log2) up to which K^ stays in range

template <int DK>
struct Smem {
    float kq[3][16][DK + 4];  // [K~; Q~] rows in the permuted order, by sub-chunk mod 3
    float kb[3][DK][KBS];     // K-^T: channel row, token t at slot 2 (t % 4) + t / 4
    float gc[3][DK];          // gamma_C
    float beta[3][C];
    float gp[2][4][16][16];   // the blocks' partial Grams: [row of [K~; Q~]][token s], by parity
    float mt[2][4 * C * C];   // the solve's 8 x 8 products (T at 64, P T at 128), by parity
    float kc[C][DK + 4];      // K^ by token (used inside a gate wave's own block only)
    float raw[4][3][C][32];   // per block, direct Grams only: k, q, G (log2) of its channels
};

// Launch configuration of a head size, chosen by measurement on the packed
// varlen shape, where one long sequence sets the time: its chains run
// sub-chunk after sub-chunk, and every other workgroup on their CU slows
// them down, while the total work still has to fit.
//   W    state columns per workgroup (a chain's d_v columns are split over
//        d_v / W workgroups that each form the gate side);
//   OCC  the most workgroups a CU may hold (0: as registers and LDS allow),
//        enforced through the workgroup's LDS size.
template <int DK, int DV>
struct Cfg {
    static constexpr int W = DK == 128 ? (DV >= 64 ? 64 : DV) : (DV < 32 ? DV : 32);
    static constexpr int OCC = DK == 128 ? (W == 64 ? 2 : 1) : (DK == 64 ? (DV == 16 ? 1 : 0) : (DV == 128 ? 0 : 2));
    static constexpr int NS = W == 128 ? 4 : W / 16;                   // state waves
    static constexpr int NBLK = DK < 32 ? 1 : DK / 32;                 // gate waves
    static constexpr int NW = NS + NBLK;                               // waves
    static constexpr int WGS = OCC ? OCC : 3;                           // workgroups per CU aimed at
    static constexpr int WPE = (NW * WGS + 3) / 4 > 2 ? (NW * WGS + 3) / 4 : 2;
    static constexpr int LDS_CU = 160 * 1024;
    static constexpr int PAD = OCC ? LDS_CU / (OCC + 1) + 64 - static_cast<int>(sizeof(Smem<DK>)) : 0;
};

template <int DK, int DV, typename Tin, typename Tout>
__global__ __launch_bounds__((64 * Cfg<DK, DV>::NW)) __attribute__((amdgpu_waves_per_eu(Cfg<DK, DV>::WPE)))
void chunk8_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
                   const float* __restrict__ g, const float* __restrict__ beta, float scale,
                   const ChunkItem* __restrict__ items, int H, int nchains, const float* __restrict__ h0,
                   Tout* __restrict__ o, float* __restrict__ hT, float* __restrict__ snaps, int interval) {
    constexpr int MT = DK / 16;                 // row tiles of the state
    constexpr int CB = DK < 32 ? DK : 32;       // channels of a gate block
    constexpr int NBLK = DK / CB;               // blocks: gate wave j < NBLK takes block j
    constexpr int MI = CB / 16;                 // 16-channel K tiles of a block
    constexpr int W = Cfg<DK, DV>::W;           // state columns of this workgroup
    constexpr int XS = DV / W;
    constexpr int NT = W == 128 ? 2 : 1;        // state tiles per state wave
    constexpr int NS = Cfg<DK, DV>::NS;         // state waves (waves 0 .. NS - 1)
    constexpr int PAD = Cfg<DK, DV>::PAD;
    __shared__ __align__(16) Smem<DK> sm;
    __shared__ char occupancy_pad[PAD > 0 ? PAD : 1];  // caps the workgroups per CU

    const int tid = threadIdx.x, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool state = w < NS;                // then the gate waves, one per block
    const int gw = w - NS;
    const int r16 = l & 15, g4 = l >> 4;
    // Workgroups go to the 8 XCDs in turn (block b to XCD b % 8).  The XS
    // column groups of a chain are placed 8 blocks apart, on one XCD, so that
    // their identical k, q and g reads share its L2; chains still start in
    // the longest-first order of the items.  The grid is rounded up to a
    // multiple of 8 XS blocks; the extra ones have no chain.
    const int round8 = static_cast<int>(blockIdx.x) / 8;
    const int chain = XS == 1 ? static_cast<int>(blockIdx.x) : (round8 / XS) * 8 + static_cast<int>(blockIdx.x) % 8;
    const int xs = XS == 1 ? 0 : round8 % XS;
    if (chain >= nchains) return;
    const ChunkItem it = items[chain / H];
    const int h = chain % H;
    const int64_t t0 = it.t0, t1 = it.t1;
    if (PAD > 0 && t0 < 0) occupancy_pad[tid] = 0;  // never taken (t0 >= 0): keeps the pad allocated
    const int n = static_cast<int>((t1 - t0 + C - 1) / C);  // sub-chunks
    const bool bw = state;
    // tile nt holds column col + nt
    const int col = xs * W + (NT == 2 ? 32 * w + 2 * r16 : 16 * w + r16);
    const int cl = l & 31, hs = l >> 5;        // gate block: channel 32 gw + cl, tokens 4 hs .. 4 hs + 3
    const bool aw = !state && gw < NBLK;
    const bool al = aw && cl < CB;
    const int cw = 32 * gw + cl;
    const int a8 = l >> 3, b8 = l & 7;         // lane (row, column) of the 8 x 8 matrices
    constexpr int64_t SD = static_cast<int64_t>(DK) * DV;

    f4 acc[MT][NT];  // acc[mt][nt][i] = S[16 mt + 4 g4 + i][col + nt]
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f4{0.f, 0.f, 0.f, 0.f};
    if (bw && it.sin >= 0) {
        const float* S0 = h0 + (static_cast<int64_t>(it.sin) * H + h) * SD + col;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * mt + 4 * g4 + i;
                if (NT == 2) {
                    const f2 x = *reinterpret_cast<const f2*>(S0 + row * DV);
                    acc[mt][0][i] = x[0];
                    acc[mt][NT - 1][i] = x[1];
                } else {
                    acc[mt][0][i] = S0[row * DV];
                }
            }
    }

    // Inputs are fetched two sub-chunks ahead into two register sets (sub-chunk
    // j in set j % 2).  Token t of a sub-chunk is at element t H d + c from its
    // first token; the buffers end after its last real token, so later tokens
    // read zeros.
    struct GateIn {
        float k[4], q[4], g[4], b;
    };
    GateIn gin[2] = {};
    float vin[2][2][NT] = {};
    auto span_of = [&](int j) {
        const int64_t left = t1 - (t0 + static_cast<int64_t>(C) * j);
        return static_cast<uint32_t>(left < C ? left : C) * H;  // (token, head) rows
    };
    auto gfetch = [&](int j, GateIn& r) {
        const uint32_t span = span_of(j);
        const int64_t first = (t0 + static_cast<int64_t>(C) * j) * H + h;
        if (al) {
            const auto rk = rsrc(k + first * DK, span * DK * sizeof(Tin));
            const auto rq = rsrc(q + first * DK, span * DK * sizeof(Tin));
            const auto rg = rsrc(g + first * DK, span * DK * 4u);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const uint32_t e = static_cast<uint32_t>(4 * hs + jj) * H * DK + cw;
                r.k[jj] = bld(rk, e, k);
                r.q[jj] = bld(rq, e, q);
                r.g[jj] = bld(rg, e, g);
            }
        }
        if (gw == 0) r.b = bld(rsrc(beta + first, span * 4u), (l & 7) * H, beta);
    };
    auto vfetch = [&](int j, float (&vx)[2][NT]) {
        const uint32_t span = span_of(j);
        const int64_t first = (t0 + static_cast<int64_t>(C) * j) * H + h;
        const auto rv = rsrc(v + first * DV, span * DV * sizeof(Tin));
        const uint32_t eg = static_cast<uint32_t>(g4) * H * DV + col;
        const uint32_t e4 = static_cast<uint32_t>(4 + g4) * H * DV + col;
        if (NT == 2) {
            const f2 a = bld2(rv, eg, v), b = bld2(rv, e4, v);
            vx[0][0] = a[0];
            vx[0][NT - 1] = a[1];
            vx[1][0] = b[0];
            vx[1][NT - 1] = b[1];
        } else {
            vx[0][0] = bld(rv, eg, v);
            vx[1][0] = bld(rv, e4, v);
        }
    };

    // ---- gate side of sub-chunk j: factors of block gw, its partial Grams ----
    auto gate_block = [&](int j, const GateIn& r) {
        const int bj = j % 3;
        float G2[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) G2[jj] = fmaxf(r.g[jj] * LOG2E, GMIN);
        G2[1] += G2[0];
        G2[2] += G2[1];
        G2[3] += G2[2];
        // lanes 0-31 hold tokens 0-3 and lanes 32-63 tokens 4-7 of the same channels
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(G2[3]), __float_as_uint(G2[3]), false,
                                                        false);
        const float lo = __uint_as_float(p[0]), hi = __uint_as_float(p[1]);
        const float GC = lo + hi;
        if (hs) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) G2[jj] += lo;
        }
        const bool direct = __any(-GC > SAFE);
        if (al) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float e = __builtin_amdgcn_exp2f(G2[jj]);
                sm.kq[bj][4 * jj + hs][cw] = r.k[jj] * e;
                sm.kq[bj][4 * jj + 2 + hs][cw] = r.q[jj] * e;
                sm.kc[4 * hs + jj][cw] = r.k[jj] * __builtin_amdgcn_exp2f(-G2[jj]);
                sm.kb[bj][cw][2 * jj + hs] = r.k[jj] * __builtin_amdgcn_exp2f(GC - G2[jj]);
            }
            if (!hs) sm.gc[bj][cw] = __builtin_amdgcn_exp2f(GC);
            if (direct) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    sm.raw[gw][0][4 * hs + jj][cl] = r.k[jj];
                    sm.raw[gw][1][4 * hs + jj][cl] = r.q[jj];
                    sm.raw[gw][2][4 * hs + jj][cl] = G2[jj];
                }
            }
        }
        if (gw == 0 && l < C) sm.beta[bj][l] = r.b;
        __builtin_amdgcn_wave_barrier();  // this wave's rows of the tiles are written

        // partial Grams over this block's channels: D[4 g4 + i][s = r16]
        f4 gacc = {0.f, 0.f, 0.f, 0.f};
        if (!direct) {
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
                const int c0 = 32 * gw + 16 * mi + 4 * g4;
                const f4 av = *reinterpret_cast<const f4*>(&sm.kq[bj][r16][c0]);
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
                    const float* xt = sm.raw[gw][i < 2 ? 0 : 1][t];
                    const float* gt = sm.raw[gw][2][t];
                    const float* ks = sm.raw[gw][0][s];
                    const float* gs = sm.raw[gw][2][s];
#pragma unroll 4
                    for (int c = 0; c < CB; ++c)
                        acc1 += xt[c] * ks[c] * __builtin_amdgcn_exp2f(fminf(gt[c] - gs[c], 0.f));
                }
                gacc[i] = acc1;
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.gp[j & 1][gw][4 * g4 + i][r16] = gacc[i];
    };

    // ---- the solve of sub-chunk j (state wave 0): N = -A and P on lane (a8, b8);
    // T = (I + N)(I + N^2)(I + N^4), P T ----
    auto solve = [&](int j) {
        const int rk = 4 * (a8 & 3) + (a8 >> 2);  // row of K~ of token a8 in [K~; Q~]
        float gk = 0.f, gq = 0.f;
#pragma unroll
        for (int ww = 0; ww < NBLK; ++ww) {
            gk += sm.gp[j & 1][ww][rk][b8];
            gq += sm.gp[j & 1][ww][rk + 2][b8];
        }
        const float nab = b8 < a8 ? -sm.beta[j % 3][a8] * gk : 0.f;
        const float pab = b8 <= a8 ? gq : 0.f;
        solve8(sm.mt[j & 1], nab, pab, a8, b8, l);
    };

    // ---- state side of sub-chunk i (state waves owning columns) ----
    int64_t next_snap = interval;
    int64_t snap_row = it.snap;
    auto state_step = [&](int i, const float (&vc)[2][NT]) {
        const int bi = i % 3;
        const int64_t s0 = t0 + static_cast<int64_t>(C) * i;
        // [K~; Q~] S over the row tiles in up to four accumulators (shorter
        // dependent MFMA chains), summed at the end
        constexpr int NY = MT >= 4 ? 4 : MT;
        f4 y2[NY][NT];
#pragma unroll
        for (int e = 0; e < NY; ++e)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) y2[e][nt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const f4 av = *reinterpret_cast<const f4*>(&sm.kq[bi][r16][16 * mt + 4 * g4]);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) y2[mt % NY][nt] = mfma4(av[ii], acc[mt][nt][ii], y2[mt % NY][nt]);
        }
        f4 y[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            y[nt] = y2[0][nt];
#pragma unroll
            for (int e = 1; e < NY; ++e) y[nt] += y2[e][nt];
        }

        // X = Diag(beta)(V - K~ S) for tokens g4 and 4 + g4; [T; P T] X
        const float bg = sm.beta[bi][g4], b4 = sm.beta[bi][4 + g4];
        // A operand of [T; P T]: row r16 = 4 g' + i' (i' < 2: T, else P T; token g' + 4 (i' & 1))
        const int ra = (r16 >> 2) + 4 * (r16 & 1);
        const float* const Mt = sm.mt[i & 1] + ((r16 & 2) ? 128 : 64);
        const float m0 = Mt[8 * ra + g4], m1 = Mt[8 * ra + 4 + g4];
        f4 z[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const float xg = bg * (vc[0][nt] - y[nt][0]);
            const float x4 = b4 * (vc[1][nt] - y[nt][1]);
            z[nt] = f4{0.f, 0.f, y[nt][2], y[nt][3]};
            z[nt] = mfma4(m0, xg, z[nt]);
            z[nt] = mfma4(m1, x4, z[nt]);
        }
        // o of tokens g4 and 4 + g4 (rows 2 and 3)
        {
            const auto ro = rsrc(o + (s0 * H + h) * DV, span_of(i) * DV * sizeof(Tout));
            const uint32_t eg = static_cast<uint32_t>(g4) * H * DV + col;
            const uint32_t e4 = static_cast<uint32_t>(4 + g4) * H * DV + col;
            if (NT == 2) {
                bst2(ro, eg, f2{scale * z[0][2], scale * z[NT - 1][2]}, o);
                bst2(ro, e4, f2{scale * z[0][3], scale * z[NT - 1][3]}, o);
            } else {
                bst(ro, eg, scale * z[0][2], o);
                bst(ro, e4, scale * z[0][3], o);
            }
        }

        // S <- Diag(gamma_C) S + K-^T U  (U of tokens g4, 4 + g4 in rows 0, 1)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const f4 gv = *reinterpret_cast<const f4*>(&sm.gc[bi][16 * mt + 4 * g4]);
            const f2 kv = *reinterpret_cast<const f2*>(&sm.kb[bi][16 * mt + r16][2 * g4]);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                acc[mt][nt] *= gv;
                acc[mt][nt] = mfma4(kv[0], z[nt][0], acc[mt][nt]);
                acc[mt][nt] = mfma4(kv[1], z[nt][1], acc[mt][nt]);
            }
        }

        // the state after each `interval` tokens of the sequence
        const int64_t done = (s0 + C < t1 ? s0 + C : t1) - t0;
        if (snaps && done == next_snap) {
            float* dst = snaps + (snap_row * H + h) * SD + col;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int row = 16 * mt + 4 * g4 + ii;
                    if (NT == 2)
                        *reinterpret_cast<f2*>(dst + row * DV) = f2{acc[mt][0][ii], acc[mt][NT - 1][ii]};
                    else
                        dst[row * DV] = acc[mt][0][ii];
                }
            next_snap += interval;
            ++snap_row;
        }
    };

    // Iteration i: the state waves run sub-chunk i and state wave 0 then
    // solves sub-chunk i + 1 (its partial Grams were written one iteration
    // earlier); the gate waves form the factors and partial Grams of
    // sub-chunk i + 2.  Tiles of
    // sub-chunk j live in buffer j % 3 (partial Grams and solves: j % 2), so
    // one barrier per iteration orders every producer before its consumer
    // and every consumer before the overwrite.
    auto iteration = [&](int i, GateIn& r, float (&vx)[2][NT]) {
        if (state) {
            if (bw) {
                state_step(i, vx);
                if (i + 2 < n) vfetch(i + 2, vx);
            }
            if (w == 0 && i + 1 < n) solve(i + 1);
        } else {
            if (aw && i + 2 < n) {
                gate_block(i + 2, r);
                if (i + 4 < n) gfetch(i + 4, r);
            }
        }
        __syncthreads();
    };

    // prologue: inputs of sub-chunks 0-3 in flight, gate side of 0 and 1, solve of 0
    if (state) {
        if (bw) {
            if (0 < n) vfetch(0, vin[0]);
            if (1 < n) vfetch(1, vin[1]);
        }
    } else if (aw) {
        if (0 < n) gfetch(0, gin[0]);
        if (1 < n) gfetch(1, gin[1]);
        if (0 < n) {
            gate_block(0, gin[0]);
            if (2 < n) gfetch(2, gin[0]);
        }
        if (1 < n) {
            gate_block(1, gin[1]);
            if (3 < n) gfetch(3, gin[1]);
        }
    }
    __syncthreads();
    if (w == 0 && 0 < n) solve(0);
    __syncthreads();

    for (int i = 0; i < n; i += 2) {
        iteration(i, gin[0], vin[0]);
        if (i + 1 >= n) break;
        iteration(i + 1, gin[1], vin[1]);
    }

    if (bw && it.sout >= 0) {
        float* S1 = hT + (static_cast<int64_t>(it.sout) * H + h) * SD + col;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * mt + 4 * g4 + i;
                if (NT == 2)
                    *reinterpret_cast<f2*>(S1 + row * DV) = f2{acc[mt][0][i], acc[mt][NT - 1][i]};
                else
                    S1[row * DV] = acc[mt][0][i];
            }
    }
}

template <int DK, int DV, typename Tin, typename Tout>
hipError_t launch_t(const PrefillArgs& a, const ChunkItem* items) {
    using K = Cfg<DK, DV>;
    constexpr int XS = DV / K::W;
    const uint32_t nch = static_cast<uint32_t>(a.N) * a.H;
    const uint32_t blocks = XS == 1 ? nch : (nch + 7) / 8 * 8 * XS;
    hipLaunchKernelGGL((chunk8_kernel<DK, DV, Tin, Tout>), dim3(blocks),
                       dim3(64 * K::NW), 0, a.stream, static_cast<const Tin*>(a.q), static_cast<const Tin*>(a.k),
                       static_cast<const Tin*>(a.v), a.g, a.beta, a.scale, items, a.H, static_cast<int>(nch), a.h0,
                       static_cast<Tout*>(a.o), a.hT, a.snaps, a.snap_interval);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_d(const PrefillArgs& a, const ChunkItem* items) {
    if (a.in_bf16)
        return a.out_bf16 ? launch_t<DK, DV, bf16_t, bf16_t>(a, items) : launch_t<DK, DV, bf16_t, float>(a, items);
    return a.out_bf16 ? launch_t<DK, DV, float, bf16_t>(a, items) : launch_t<DK, DV, float, float>(a, items);
}

}  // namespace c8

size_t chunk8_workspace_bytes(int N) {
    return (static_cast<size_t>(N) * sizeof(ChunkItem) + 255) / 256 * 256;
}

hipError_t launch_chunk8(const PrefillArgs& a) {
    ChunkItem* items = static_cast<ChunkItem*>(a.ws);
    const hipError_t e = launch_plan_sequences(a, items);
    if (e != hipSuccess) return e;
    return dispatch_head_sizes(a.dk, a.dv, [&](auto DK, auto DV) {
        return c8::launch_d<decltype(DK)::value, decltype(DV)::value>(a, items);
    });
}

}  // namespace kda
