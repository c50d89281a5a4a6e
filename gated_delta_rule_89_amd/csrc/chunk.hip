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
//   Delta = U - W S = T (v - K~ S),            K~ = Lambda k
//   O    = scale (Q~ S + P Delta),             Q~ = Lambda q
//   S   <- Diag(Lambda_last) S + K-bar^T Delta,  K-bar = (Lambda_last / Lambda) k
//
// so one chunk maps S to (Diag(Lambda_last) - K-bar^T W) S + K-bar^T U: a
// diagonal-plus-low-rank transition, the structure named on that page.  A run
// of chunks therefore maps S_in to M S_in + B, with B the run's result from a
// zero state and M the transitions' product; by linearity the read-out from
// S_in is the zero-start read-out plus that of the propagated S_in alone
// (v = 0).  Long sequences are cut into segments on that basis (the
// propagation modes of the 12-wave kernel and segment_scan_kernel).
//
// Design on this GPU:
//  * A chunk is NSB sub-blocks of 16 tokens (C = 16 NSB: 32 tokens in the
//    12-wave kernel, 64 in the single-role one); a workgroup owns one chain
//    segment (one sequence, one head).  Gate-side work (cumulative gates,
//    Grams, the triangular solves) is split over the waves by sub-block and
//    channel part; the state pass is split by state columns (columns of S
//    are independent), 16 NCT columns per wave.
//  * Gate exponents stay in range: inside a sub-block every factor is taken
//    relative to the sub-block start, across sub-blocks relative to sub-block
//    ends, so every factor is <= 1 except in the diagonal Gram blocks.  Those
//    take operands referenced to half the sub-block's gate total: fp16 MFMA
//    when the wave's exponents stay within +-8, fp32 MFMA while they stay
//    within +-120 (log2 units), and beyond that (a channel that forgets
//    almost everything inside 16 tokens) every factor from its own exponent
//    and the diagonal blocks entry by entry (phase1_direct), so any g <= 0
//    is handled.  Every other product runs on fp16 MFMA with fp32
//    accumulation; factors below the fp16 range underflow to zero, which
//    only drops terms smaller than 2^-24 of the ones kept.
//  * T is kept as its diagonal blocks T_JJ = (I + A_JJ)^-1 Diag(beta_J) and
//    the raw cross Grams G_JK (A_JK = Diag(beta_J) G_JK); Delta = T X is then
//    forward block substitution, Delta_J = T_JJ (X_J - sum_K<J G_JK Delta_K).
//  * S lives in MFMA accumulators for the whole segment; its fp16 copy and
//    Delta's are fed back as MFMA operands straight from the accumulator
//    registers, using a k-order permutation that the gate-side operands read
//    from LDS follow too.
//  * Value-side fp16 operands (S, v, Delta) carry a per-wave power-of-two scale
//    chosen every chunk from max(|S|, |v|), which keeps them inside fp16 range
//    and away from subnormals; the scale is exact and is removed in fp32.
//  * The next chunk's inputs are fetched into registers a chunk ahead, right
//    after the current chunk's have been unpacked (v after it is staged).
#include <utility>

#include "dev_common.h"
#include "kda_internal.h"

namespace kda {

// Scan over the segment maps of one sequence (all heads).
struct ScanItem {
    int32_t first_seg;  // index of the sequence's first segment
    int32_t nseg;       // its number of segments (a single one needs no scan)
    int32_t h0;         // row of h0 or -1 for zero
    int32_t hT;         // row of the final state or -1 for none
};

namespace chunkk {

constexpr int SB = 16;    // tokens per sub-block
constexpr int CSEG = 64;  // segment boundaries are multiples of every chunk size
// Exponent headroom of the propagated matrices: X (scaled into [2^9, 2^10)
// at its start) is dropped once its fp16 copy at no more than 2^6 above its
// first exponent rounds to zero, i.e. once max|X| < 2^-25-6-9 max|X_0|:
// 2^-40 of the map or initial state it started from, far below the fp32
// resolution of anything that state contributes to at full strength.
#ifndef PROP_HEADROOM
#define PROP_HEADROOM 6
#endif
constexpr int D = 128;    // head size (d_k = d_v)
constexpr int QP = 136;   // row stride (halves) of [token][channel] tiles
constexpr int GP = 20;    // row stride (floats) of 16x16 Gram tiles (16-byte rows)
constexpr int BP = 20;    // row stride (halves) of 16x16 fp16 blocks
// Largest |G - tot/2| (log2 units) over a wave's k-step for which the
// half-total reference keeps every factor and its inverse in fp32 range;
// beyond it phase 1 takes the entry-by-entry form (phase1_direct).
constexpr float SAFE_SPAN = 120.f;

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// MFMA A operands read from LDS ([row][k] tiles with k = channels or tokens
// in 32-wide blocks) store each 32-wide k block in operand order: position
// 8 j + m holds k index 4 j + m (m < 4) or 16 + 4 j + m - 4 (m >= 4), the
// order in which the B operands built from accumulator registers come.  A
// lane's 8 k values are then one aligned 16-byte read.
__device__ __forceinline__ int kpos(int c) {
    return (c & ~31) + 8 * ((c & 15) >> 2) + 4 * ((c >> 4) & 1) + (c & 3);
}

// Cross (off-diagonal) sub-block pair (I, J), I > J, in row order.
__host__ __device__ constexpr int xidx(int I, int J) { return I * (I - 1) / 2 + J; }

// Per-workgroup LDS for NSB sub-blocks and NP channel parts per sub-block
// (one Gram partial each).  Gram tiles: 2 J (A_JJ), 2 J + 1 (P_JJ), then
// 2 NSB + 2 x (G_x) and 2 NSB + 2 x + 1 (P_x) for cross pair x.
template <int NSB, int NP>
struct alignas(16) Smem {
    static constexpr int C = 16 * NSB;
    static constexpr int NX = NSB * (NSB - 1) / 2;
    static constexpr int TP = C + 8;  // row stride (halves) of [x][token] tiles
    _Float16 qt[C][QP];                // Q~ = Lambda q        [token][channel, operand order]
    _Float16 kt[C][QP];                // K~ = Lambda k        [token][channel, operand order]
    _Float16 kbt[D][TP];               // K-bar^T              [channel][token, operand order]
    _Float16 rbs[NSB - 1][SB][QP];     // k exp(tot_J - G) of sub-blocks 0 .. NSB-2   [token][channel]
    _Float16 tb[NSB + NX][SB][BP];     // T_JJ, then -G_x (raw cross Grams)           [token][token]
    _Float16 p[C][TP];                 // P                    [token][token, operand order]
    uint16_t v[C][QP];                 // v tile (bf16 bits)   [token][column]
    float gp[NP][2 * NSB + 2 * NX][SB][GP];
    float a[NSB][SB][20];              // A_JJ = Diag(beta) G_JJ, strictly lower, by row
    float etot[NSB][D];                // per-channel exp(sum of g over each sub-block)
    float lam[D];                      // Lambda_last = exp(Gamma over the chunk)
    float beta[C];
};

__device__ __forceinline__ f4 mfma16(h8 a, h8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfma16k16(h4 a, h4 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfmab(b8 a, b8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfma4(float a, float b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Value of lane i - n of the same 16-lane DPP row (0 for i < n).
template <int N>
__device__ __forceinline__ float row_shr(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 | N, 0xf, 0xf, true));
}

// Value of lane M of the same 16-lane DPP row, in every lane of the row.
template <int M>
__device__ __forceinline__ float row_bcast16(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 | M, 0xf, 0xf, true));
}

// One step of a column-oriented substitution with rows across the 16 lanes
// of a DPP row: x_i -= a_i x_M for four columns, a_i = A[i][M] of this lane's row.
template <int M>
__device__ __forceinline__ void subst_step(float (&x)[4], const f4 (&arow)[4]) {
    float xb[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) xb[qq] = row_bcast16<M>(x[qq]);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) x[qq] = fmaf(-arow[M >> 2][M & 3], xb[qq], x[qq]);
}
template <int... M>
__device__ __forceinline__ void subst_all(float (&x)[4], const f4 (&arow)[4], std::integer_sequence<int, M...>) {
    (subst_step<M>(x, arow), ...);
}

// The same step for two columns, and steps M0 .. M0 + n - 1.
template <int M>
__device__ __forceinline__ void subst_step2(float (&x)[2], const f4 (&arow)[4]) {
    float xb[2];
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) xb[qq] = row_bcast16<M>(x[qq]);
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) x[qq] = fmaf(-arow[M >> 2][M & 3], xb[qq], x[qq]);
}
template <int M0, int... M>
__device__ __forceinline__ void subst_range2(float (&x)[2], const f4 (&arow)[4], std::integer_sequence<int, M...>) {
    (subst_step2<M0 + M>(x, arow), ...);
}

// Inclusive prefix sum over the 16 lanes of a DPP row.
__device__ __forceinline__ float row_scan16(float x) {
    x += row_shr<1>(x);
    x += row_shr<2>(x);
    x += row_shr<4>(x);
    x += row_shr<8>(x);
    return x;
}

// Sum over the four 16-lane rows of the wave (every lane gets the total):
// the gfx950 row-pair swaps exchange rows 0/1 and 2/3, then the two halves.
__device__ __forceinline__ float sum_rows4(float x) {
    const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
    const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
}

// Gate phase 1 for one 32-channel k-step whose exponents leave the fp32
// range of the half-total reference (a channel's 16-token gate sum below
// about -166): every factor from its own exponent, so nothing overflows.
// Lane (r, g4) holds token r of the sub-block and channels 8 g4 .. 8 g4 + 7:
// k (kf), q (qf) and the raw log-gates (gr, natural units).  Log-gates are
// clamped at -100 first: alpha = e^-100 (about 4e-44) is zero next to any
// fp32 state entry, and the clamp keeps the fp32 cumulative sums within
// about 2^-12 of their exponents (no cancellation against a huge total).
// Outputs: the fp16 operands k exp(G), q exp(G), k exp(tot - G), exp(tot)
// per channel, and the diagonal Gram blocks entry by entry,
//   A[r][j] = sum_c k_rc k_jc exp(G_rc - G_jc),  P[r][j] = sum_c q_rc k_jc exp(G_rc - G_jc),
// over this lane group's channels, summed over the wave's four row groups;
// lane (r, g4) adds columns j = 4 g4 .. 4 g4 + 3 of row r into oa and op.
// Entries on or above the diagonal of A and above it for P are not used;
// their exponent is capped at 0 so they stay finite.
template <bool WITHQ>
__device__ __forceinline__ void phase1_direct(const float (&kf)[8], const float (&qf)[8],
                                              const float (&gr)[8], int g4, h8& l16, h8& q16,
                                              h8& rb16, float (&et)[8], f4& oa, f4& op) {
    constexpr float LOG2E = 1.4426950408889634f;
    float Gc[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        Gc[m] = row_scan16(fmaxf(gr[m], -100.f) * LOG2E);
        const float tot = row_bcast16<15>(Gc[m]);
        const float e = __builtin_amdgcn_exp2f(Gc[m]);
        l16[m] = static_cast<_Float16>(kf[m] * e);
        if (WITHQ) q16[m] = static_cast<_Float16>(qf[m] * e);
        rb16[m] = static_cast<_Float16>(kf[m] * __builtin_amdgcn_exp2f(tot - Gc[m]));
        et[m] = __builtin_amdgcn_exp2f(tot);
    }
    // Token j's values come from lane j of the same 16-lane row (a rolled
    // loop with lane-indexed reads keeps this rarely taken path small).
    const int rowbase = (__lane_id() & 48);
#pragma unroll 1
    for (int j = 0; j < SB; ++j) {
        float a = 0.f, p = 0.f;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const float gj = __shfl(Gc[m], rowbase | j);
            const float kj = __shfl(kf[m], rowbase | j);
            const float t = kj * __builtin_amdgcn_exp2f(fminf(Gc[m] - gj, 0.f));
            a = fmaf(kf[m], t, a);
            if (WITHQ) p = fmaf(qf[m], t, p);
        }
        a = sum_rows4(a);
        if (WITHQ) p = sum_rows4(p);
        const bool mine = g4 == (j >> 2);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool sel = mine && (j & 3) == e;
            oa[e] += sel ? a : 0.f;
            if (WITHQ) op[e] += sel ? p : 0.f;
        }
    }
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

// Raw buffer resource over `bytes` bytes from `base` (a uniform address); the
// per-lane part of an access goes in a 32-bit vector offset, so no 64-bit
// per-lane address has to stay live across the chunk loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ u4 bload16(__amdgpu_buffer_rsrc_t r, int voff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
}
__device__ __forceinline__ float bload4(__amdgpu_buffer_rsrc_t r, int voff) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
}
__device__ __forceinline__ void bstore(__amdgpu_buffer_rsrc_t r, int voff, int soff, float x, float*) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, voff, soff, 0);
}
// 8 consecutive outputs of one lane as 16-byte buffer stores (two for fp32).
__device__ __forceinline__ void store8(__amdgpu_buffer_rsrc_t r, int voff, const float* y, float*) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
        __builtin_amdgcn_raw_buffer_store_b128(
            u4{__float_as_uint(y[4 * j]), __float_as_uint(y[4 * j + 1]), __float_as_uint(y[4 * j + 2]),
               __float_as_uint(y[4 * j + 3])}, r, voff + 16 * j, 0, 0);
}
__device__ __forceinline__ void store8(__amdgpu_buffer_rsrc_t r, int voff, const float* y, bf16_t*) {
    u4 p;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        p[e] = static_cast<uint32_t>(f32_to_bf16(y[2 * e])) | (static_cast<uint32_t>(f32_to_bf16(y[2 * e + 1])) << 16);
    __builtin_amdgcn_raw_buffer_store_b128(p, r, voff, 0, 0);
}
__device__ __forceinline__ void bstore(__amdgpu_buffer_rsrc_t r, int voff, int soff, float x, bf16_t*) {
    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(x), r, voff, soff, 0);
}

// 4 consecutive outputs of one lane as one buffer store (16 bytes fp32, 8 bytes bf16).
__device__ __forceinline__ void store4(__amdgpu_buffer_rsrc_t r, int voff, f4 y, float*) {
    __builtin_amdgcn_raw_buffer_store_b128(
        u4{__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]), __float_as_uint(y[3])}, r, voff, 0, 0);
}
__device__ __forceinline__ void store4(__amdgpu_buffer_rsrc_t r, int voff, f4 y, bf16_t*) {
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    const u2 p = {static_cast<uint32_t>(f32_to_bf16(y[0])) | (static_cast<uint32_t>(f32_to_bf16(y[1])) << 16),
                  static_cast<uint32_t>(f32_to_bf16(y[2])) | (static_cast<uint32_t>(f32_to_bf16(y[3])) << 16)};
    __builtin_amdgcn_raw_buffer_store_b64(p, r, voff, 0, 0);
}

// 4 consecutive values of one lane (16 bytes fp32, 8 bytes bf16), widened to fp32.
__device__ __forceinline__ f4 load4(__amdgpu_buffer_rsrc_t r, int voff, float*) {
    const u4 w = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
    return f4{__uint_as_float(w[0]), __uint_as_float(w[1]), __uint_as_float(w[2]), __uint_as_float(w[3])};
}
__device__ __forceinline__ f4 load4(__amdgpu_buffer_rsrc_t r, int voff, bf16_t*) {
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    const u2 w = __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0);
    return f4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
              __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)};
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

// Exponent e for max(|S|, |v|) = mx: the current one while mx * 2^ex stays
// in [2^8, 2^11), else the one that puts it in [2^9, 2^10).  The fp16 copies
// of the value-side operands then stay far from both ends of the fp16 range
// (K~ S with unit keys is at most sqrt(128) 2^11 < 2^15), and the state is
// rescaled only when its magnitude has drifted by a factor of two or more.
__device__ __forceinline__ int value_exponent(float mx, int ex) {
    if (!(mx > 0.f) || !(mx < 3.0e38f)) return ex;
    int e2;
    (void)frexpf(mx, &e2);  // mx in [2^(e2-1), 2^e2)
    if (e2 - 1 + ex >= 8 && e2 + ex <= 11) return ex;
    const int e = 10 - e2;
    return e < -120 ? -120 : (e > 120 ? 120 : e);
}

// State snapshots: the state after every `interval` tokens of a sequence
// (a multiple of 64, so every snapshot falls on a chunk boundary).  Snapshot j
// of a sequence holds the state after tokens 0 .. (j + 1) interval - 1.
struct SnapCursor {
    int64_t next;  // sequence position of the next snapshot
    int64_t row;   // its row in the snapshot output
    __device__ void init(const ChunkItem& it, int interval) {
        next = (it.p0 / interval + 1) * interval;
        row = it.snap + it.p0 / interval;
    }
};

// Writes the state columns a wave holds (S[rt][ct][i] at row 16 rt + 4 g4 + i,
// column col + 16 ct + r, scaled by un) to a row-major d_k x d_v fp32 matrix.
// Buffer stores: one lane offset, the rest in scalar offsets (few registers).
template <int NCT>
__device__ __forceinline__ void store_state(float* __restrict__ dst, const f4 (&S)[8][NCT], float un,
                                            int g4, int r, int col) {
    const auto rd = rsrc(dst, D * D * 4);
    int vo = ((4 * g4) * D + col + r) * 4;
    asm volatile("" : "+v"(vo));  // computed here, not held in a register across the chunk loop
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) bstore(rd, vo, ((16 * rt + i) * D + 16 * ct) * 4, S[rt][ct][i] * un, dst);
}

// Adds the state columns a wave holds (as store_state) to a d_k x d_v matrix.
template <int NCT>
__device__ __forceinline__ void add_state(float* __restrict__ dst, const f4 (&S)[8][NCT], float un,
                                          int g4, int r, int col) {
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float* p = dst + (16 * rt + 4 * g4 + i) * D + col + 16 * ct + r;
                *p += S[rt][ct][i] * un;
            }
}

// Single-role chunked prefill: NW waves do the gate-side work of each chunk
// and then its state pass, each wave owning NCT 16-column tiles of S
// (NW * 16 NCT = 128 columns); chunks of NSB sub-blocks.  Writes o, the final
// state and the snapshots.  WPC workgroups share a CU (it sets the register
// budget).
template <int NW, int NSB, int NCT, int WPC, typename Tout, bool SNAP = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4 * WPC)))
void chunk_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ g,
    const float* __restrict__ beta, float scale, const ChunkItem* __restrict__ items, int H,
    const float* __restrict__ h0, const float* __restrict__ staged, Tout* __restrict__ o,
    float* __restrict__ out_state, float* __restrict__ snaps, int interval) {
    constexpr int C = 16 * NSB;         // tokens per chunk
    constexpr int NP = NW / NSB;        // channel parts per sub-block
    constexpr int CPG = D / NP;         // channels per gate wave
    constexpr int KS = CPG / 32;        // 32-channel k-steps per gate wave
    constexpr int NKB = C / 32;         // 32-token k blocks of a chunk
    constexpr int CPW = 16 * NCT;       // state columns per wave
    constexpr int NT = NW * 64;         // threads
    constexpr int VU = (C * D / 8) / NT;  // 16-byte pieces of the v tile per thread
    constexpr int NX = NSB * (NSB - 1) / 2;
    static_assert(NSB == 2 || NSB == 4, "chunks of 32 or 64 tokens");
    static_assert(NP >= 1 && NW % NSB == 0 && KS >= 1 && VU >= 1 && NW > NSB, "unsupported wave split");
    static_assert(NW * CPW == D, "the waves' columns cover the state");
    __shared__ Smem<NSB, NP> sm;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave (uniform: scalar register)
    const int l = tid & 63;      // lane
    const int r = l & 15;        // MFMA row / column index
    const int g4 = l >> 4;       // MFMA k group
    const int I = w / NP;        // gate phases: sub-block of this wave
    const int part = w % NP;     // gate phases: channel part of this wave

    const ChunkItem it = items[blockIdx.x / H];
    const int h = blockIdx.x % H;
    const int64_t t0 = it.t0, t1 = it.t1;
    const int col = CPW * w;  // first state column of this wave

    // State, kept as S * 2^ex: S[16 rt + 4 g4 + i][col + 16 ct + r] in S[rt][ct][i].
    f4 S[8][NCT];
    int ex = 0;
    {
        const float* src = nullptr;
        if (it.sin >= 0 && h0) src = h0 + (static_cast<int64_t>(it.sin) * H + h) * D * D;
        else if (it.sin <= -2) src = staged + (static_cast<int64_t>(-it.sin - 2) * H + h) * D * D;
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) S[rt][ct] = f4{0.f, 0.f, 0.f, 0.f};
        if (src) {
#pragma unroll
            for (int rt = 0; rt < 8; ++rt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        S[rt][ct][i] = src[(16 * rt + 4 * g4 + i) * D + col + 16 * ct + r];
        }
    }

    // Raw inputs of the next chunk, fetched one chunk ahead: k, q, g of this
    // lane's token and channels (gate layout), its beta, and pieces of the v
    // tile (staging layout).  Every chunk issues the same buffer loads; tokens
    // at or past the end of the sequence lie outside the buffer range (valid
    // tokens x row bytes) and read zeros, so the compiler counts outstanding
    // loads exactly and waits only for the ones it consumes.
    const int tok = SB * I + r;
    const int rowe = H * D;  // elements per token row
    u4 kw[KS], qw[KS], vp[VU];
    f4 ga[KS], gb[KS];
    float bt;
    auto valid_at = [&](int64_t cs) {
        const int64_t nv = t1 - cs;
        return static_cast<uint32_t>(nv < 0 ? 0 : nv < C ? nv : C);
    };
    auto fetch_gate = [&](int64_t cs) {
        const uint32_t vld = valid_at(cs);
        const int64_t cb = (cs * H + h) * D;
        const auto rk = rsrc(k + cb, vld * rowe * 2);
        const auto rq = rsrc(q + cb, vld * rowe * 2);
        const auto rg = rsrc(g + cb, vld * rowe * 4);
        const auto rb = rsrc(beta + cs * H + h, vld * H * 4);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int off = tok * rowe + CPG * part + 32 * ks + 8 * g4;
            kw[ks] = bload16(rk, 2 * off);
            qw[ks] = bload16(rq, 2 * off);
            const u4 a0 = bload16(rg, 4 * off), a1 = bload16(rg, 4 * off + 16);
            ga[ks] = f4{__uint_as_float(a0[0]), __uint_as_float(a0[1]), __uint_as_float(a0[2]), __uint_as_float(a0[3])};
            gb[ks] = f4{__uint_as_float(a1[0]), __uint_as_float(a1[1]), __uint_as_float(a1[2]), __uint_as_float(a1[3])};
        }
        bt = bload4(rb, 4 * tok * H);
    };
    auto fetch_v = [&](int64_t cs) {
        const auto rv = rsrc(v + (cs * H + h) * D, valid_at(cs) * rowe * 2);
#pragma unroll
        for (int j = 0; j < VU; ++j) {
            const int e = tid + NT * j, vt = e >> 4, vc = (e & 15) * 8;
            vp[j] = bload16(rv, 2 * (vt * rowe + vc));
        }
    };
    fetch_gate(t0);
    fetch_v(t0);
    const bool snapping = SNAP && snaps != nullptr && it.snap >= 0;
    SnapCursor sc{};
    if (snapping) sc.init(it, interval);

    for (int64_t c0 = t0; c0 < t1; c0 += C) {
        const int valid = static_cast<int>(t1 - c0 < C ? t1 - c0 : C);

        // ---------------- gate phase 1: cumulative gates, diagonal Grams
        h8 l16[KS], q16[KS], rb16[KS];  // L, Lq, k exp(tot - G) as fp16 (k-step ks, slot m)
        {
            constexpr float LOG2E = 1.4426950408889634f;
            // Diagonal Gram operands are referenced to half the sub-block total,
            // k exp(G - tot/2) and k exp(tot/2 - G) (their products are unchanged).
            // A k-step whose exponents all stay within +-8 (natural units) over
            // the wave feeds them to fp16 MFMA; otherwise fp32 MFMA keeps fp32 range.
            constexpr float FAST_SPAN = 8.f * LOG2E;
            // This chunk's raw inputs are unpacked first (Gamma from the
            // sub-block start, in log2 units), so the next chunk's fetch into
            // the same registers goes out a whole chunk ahead of its use.
            float kf[KS][8], qf[KS][8], G[KS][8];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                unpack_bf16x8(kw[ks], kf[ks]);
                unpack_bf16x8(qw[ks], qf[ks]);
#pragma unroll
                for (int m = 0; m < 8; ++m)
                    G[ks][m] = row_scan16((m < 4 ? ga[ks][m] : gb[ks][m - 4]) * LOG2E);
            }
            if (part == 0 && g4 == 0) sm.beta[tok] = bt;
            fetch_gate(c0 + C);
            f4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
            bool redo = false;  // wave-uniform: a k-step beyond the reference's range
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int ch = CPG * part + 32 * ks + 8 * g4;
                float Gt[8];  // sub-block total (lane 15)
#pragma unroll
                for (int m = 0; m < 8; ++m) Gt[m] = row_bcast16<15>(G[ks][m]);
                // a = exp(G - tot/2), 1/a, and the channel's exp(tot/2) (a at the
                // last token): exp(G) = a exp(tot/2), exp(tot - G) = exp(tot/2) / a.
                float La[8], Ra[8], Qa[8], hh[8];
                float span = 0.f;
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    const float xa = fmaf(-0.5f, Gt[m], G[ks][m]);
                    span = fmaxf(span, fabsf(xa));
                    const float a = __builtin_amdgcn_exp2f(xa);
                    const float ia = __builtin_amdgcn_exp2f(-xa);
                    La[m] = kf[ks][m] * a;
                    Ra[m] = kf[ks][m] * ia;
                    Qa[m] = qf[ks][m] * a;
                    hh[m] = row_bcast16<15>(a);
                }
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    l16[ks][m] = static_cast<_Float16>(La[m] * hh[m]);   // k exp(G) <= |k|
                    rb16[ks][m] = static_cast<_Float16>(Ra[m] * hh[m]);  // k exp(tot - G)
                    q16[ks][m] = static_cast<_Float16>(Qa[m] * hh[m]);
                }
                if (!__any(span > FAST_SPAN)) {  // wave-uniform
                    h8 la, ra, qa;
#pragma unroll
                    for (int m = 0; m < 8; ++m) {
                        la[m] = static_cast<_Float16>(La[m]);
                        ra[m] = static_cast<_Float16>(Ra[m]);
                        qa[m] = static_cast<_Float16>(Qa[m]);
                    }
                    accA = mfma16(la, ra, accA);
                    accP = mfma16(qa, ra, accP);
                } else {
                    // MFMA m contracts channel 8 g4 + m (k index g4).
#pragma unroll
                    for (int m = 0; m < 8; ++m) {
                        accA = mfma4(La[m], Ra[m], accA);
                        accP = mfma4(Qa[m], Ra[m], accP);
                    }
                    redo = redo || __any(span > SAFE_SPAN);
                }
                if (r == 15) {  // exp(sum of g over the sub-block) = exp(tot/2)^2
                    *reinterpret_cast<f4*>(&sm.etot[I][ch]) =
                        f4{hh[0] * hh[0], hh[1] * hh[1], hh[2] * hh[2], hh[3] * hh[3]};
                    *reinterpret_cast<f4*>(&sm.etot[I][ch + 4]) =
                        f4{hh[4] * hh[4], hh[5] * hh[5], hh[6] * hh[6], hh[7] * hh[7]};
                }
                if (I < NSB - 1) *reinterpret_cast<h8*>(&sm.rbs[I][r][ch]) = rb16[ks];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sm.gp[part][2 * I][4 * g4 + i][r] = accA[i];  // beta of row i is applied in the sum
                sm.gp[part][2 * I + 1][4 * g4 + i][r] = accP[i];
            }
            if (redo) {
                // Exponents beyond the fp32 range of the half-total reference: the
                // wave's phase 1 again, entry by entry from its raw inputs (read
                // again, so nothing stays live for this rare case), over
                // everything written above (the same wave's LDS writes complete
                // in order).
                const uint32_t vld = valid_at(c0);
                const int64_t cb = (c0 * H + h) * D;
                const auto rk = rsrc(k + cb, vld * rowe * 2), rq = rsrc(q + cb, vld * rowe * 2);
                const auto rg = rsrc(g + cb, vld * rowe * 4);
                f4 oa = {0.f, 0.f, 0.f, 0.f}, op = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int ch = CPG * part + 32 * ks + 8 * g4;
                    const int off = tok * rowe + ch;
                    const u4 a0 = bload16(rg, 4 * off), a1 = bload16(rg, 4 * off + 16);
                    float gr[8], et[8], kr[8], qr[8];
                    unpack_bf16x8(bload16(rk, 2 * off), kr);
                    unpack_bf16x8(bload16(rq, 2 * off), qr);
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        gr[m] = __uint_as_float(a0[m]);
                        gr[4 + m] = __uint_as_float(a1[m]);
                    }
                    phase1_direct<true>(kr, qr, gr, g4, l16[ks], q16[ks], rb16[ks], et, oa, op);
                    if (r == 15) {
                        *reinterpret_cast<f4*>(&sm.etot[I][ch]) = f4{et[0], et[1], et[2], et[3]};
                        *reinterpret_cast<f4*>(&sm.etot[I][ch + 4]) = f4{et[4], et[5], et[6], et[7]};
                    }
                    if (I < NSB - 1) *reinterpret_cast<h8*>(&sm.rbs[I][r][ch]) = rb16[ks];
                }
                *reinterpret_cast<f4*>(&sm.gp[part][2 * I][r][4 * g4]) = oa;
                *reinterpret_cast<f4*>(&sm.gp[part][2 * I + 1][r][4 * g4]) = op;
            }
        }
        __syncthreads();  // B1

        // ---------------- gate phase 2: chunk-referenced operands, cross-block Grams, v
        {
            f4 ax[NSB - 1], px[NSB - 1];  // cross Grams with sub-blocks J < I
#pragma unroll
            for (int J = 0; J < NSB - 1; ++J) ax[J] = px[J] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int ch = CPG * part + 32 * ks + 8 * g4;
                // Per-channel exp(sum of g) of every sub-block; products of these
                // (all <= 1, an fp16 underflow to zero drops terms below 2^-24 of
                // the kept ones) move the sub-block's factors to chunk reference:
                // Q~, K~ take those of the sub-blocks before I, K-bar those after.
                float et[NSB][8];
#pragma unroll
                for (int J = 0; J < NSB; ++J) {
                    const f4 a0 = *reinterpret_cast<const f4*>(&sm.etot[J][ch]);
                    const f4 a1 = *reinterpret_cast<const f4*>(&sm.etot[J][ch + 4]);
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        et[J][m] = a0[m];
                        et[J][4 + m] = a1[m];
                    }
                }
                h8 fb, fa;
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    float pb = 1.f, pa = 1.f;
#pragma unroll
                    for (int J = 0; J < NSB; ++J) {
                        if (J < I) pb *= et[J][m];
                        if (J > I) pa *= et[J][m];
                    }
                    fb[m] = static_cast<_Float16>(pb);
                    fa[m] = static_cast<_Float16>(pa);
                }
                h8 kv = l16[ks], qv = q16[ks], bv = rb16[ks];
                if (I > 0) {
                    kv *= fb;
                    qv *= fb;
                }
                if (I < NSB - 1) bv *= fa;
                // channels 8 g4 .. 8 g4 + 7 of the block go to two 4-wide runs
                const int cb = ch & ~31, p0 = cb + (g4 < 2 ? 16 * g4 : 16 * g4 - 28), p1 = p0 + 8;
                *reinterpret_cast<h4*>(&sm.kt[tok][p0]) = __builtin_shufflevector(kv, kv, 0, 1, 2, 3);
                *reinterpret_cast<h4*>(&sm.kt[tok][p1]) = __builtin_shufflevector(kv, kv, 4, 5, 6, 7);
                {
                    *reinterpret_cast<h4*>(&sm.qt[tok][p0]) = __builtin_shufflevector(qv, qv, 0, 1, 2, 3);
                    *reinterpret_cast<h4*>(&sm.qt[tok][p1]) = __builtin_shufflevector(qv, qv, 4, 5, 6, 7);
                }
                const int tp = kpos(tok);
#pragma unroll
                for (int m = 0; m < 8; ++m) sm.kbt[ch + m][tp] = bv[m];
                // Cross Grams G_IJ (J < I): k exp(G) of I against k exp(tot_J - G) of J
                // times the totals of the sub-blocks strictly between them.
#pragma unroll
                for (int J = 0; J < NSB - 1; ++J) {
                    if (J < I) {
                        h8 rv = *reinterpret_cast<const h8*>(&sm.rbs[J][r][ch]);
                        if (J + 1 < I) {
                            h8 fm;
#pragma unroll
                            for (int m = 0; m < 8; ++m) {
                                float pm = 1.f;
#pragma unroll
                                for (int K = 1; K < NSB - 1; ++K)
                                    if (K > J && K < I) pm *= et[K][m];
                                fm[m] = static_cast<_Float16>(pm);
                            }
                            rv *= fm;
                        }
                        ax[J] = mfma16(l16[ks], rv, ax[J]);
                        px[J] = mfma16(q16[ks], rv, px[J]);
                    }
                }
            }
#pragma unroll
            for (int J = 0; J < NSB - 1; ++J) {
                if (J < I) {
                    const int x = xidx(I, J);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        sm.gp[part][2 * NSB + 2 * x][4 * g4 + i][r] = ax[J][i];  // raw (beta applied in the state pass)
                        sm.gp[part][2 * NSB + 2 * x + 1][4 * g4 + i][r] = px[J][i];
                    }
                }
            }
            if (tid < D) {
                float lm = 1.f;
#pragma unroll
                for (int J = 0; J < NSB; ++J) lm *= sm.etot[J][tid];
                sm.lam[tid] = lm;
            }
            for (int e = tid; e < NSB * SB * SB; e += NT) {
                const int J = e >> 8, i = (e >> 4) & 15, m = e & 15;
                float s = 0.f;
#pragma unroll
                for (int pp = 0; pp < NP; ++pp) s += sm.gp[pp][2 * J][i][m];
                sm.a[J][i][m] = m < i ? s * sm.beta[SB * J + i] : 0.f;  // A_JJ by row, strictly lower
            }
#pragma unroll
            for (int j = 0; j < VU; ++j) {
                const int e = tid + NT * j, vt = e >> 4, vc = (e & 15) * 8;
                *reinterpret_cast<u4*>(&sm.v[vt][vc]) = vp[j];
            }
            fetch_v(c0 + C);
        }
        __syncthreads();  // B2

        // ---------------- solve: diagonal block inverses (waves 0 .. NSB-1); P and -G_x (others)
        if (w < NSB) {
            // T_JJ = (I + A_JJ)^-1 Diag(beta_J) by column-oriented substitution:
            // lane (i, g4) holds row i of columns 4 g4 .. 4 g4 + 3 and row i of A.
            const int J = w;  // diagonal block
            f4 arow[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) arow[c] = *reinterpret_cast<const f4*>(&sm.a[J][r][4 * c]);
            const f4 bcol = *reinterpret_cast<const f4*>(&sm.beta[SB * J + 4 * g4]);
            float x[4];
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) x[qq] = (r == 4 * g4 + qq) ? 1.f : 0.f;
            subst_all(x, arow, std::make_integer_sequence<int, SB>{});
            h4 tv;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) tv[qq] = static_cast<_Float16>(x[qq] * bcol[qq]);
            *reinterpret_cast<h4*>(&sm.tb[J][r][4 * g4]) = tv;
        } else {
            // Sums of the channel-part partials, 4 consecutive entries per step:
            // P (causal blocks, plus the zero blocks inside the 32-token k blocks
            // that the state pass reads) as fp16 in operand order, and -G_x.
            const int t2 = tid - 64 * NSB;
            constexpr int NT2 = NT - 64 * NSB;
            constexpr int NPB = NSB + NX + NKB;  // P blocks written: diagonal, cross, upper-in-k-block
            constexpr int NQ = NPB * 64 + NX * 64;  // 4-entry quads
#pragma unroll
            for (int q0 = 0; q0 < NQ; q0 += NT2) {
                const int qi = q0 + t2;
                if (qi < NQ) {
                    const int blk = qi >> 6, i = (qi >> 2) & 15, m4 = (qi & 3) * 4;
                    const bool isp = blk < NPB;
                    int tile = -1, bi = 0, bj = 0;
                    if (isp) {
                        if (blk < NSB) { bi = bj = blk; tile = 2 * blk + 1; }
                        else if (blk < NSB + NX) {
                            const int x = blk - NSB;
                            bi = 1; while (xidx(bi + 1, 0) <= x) ++bi;
                            bj = x - xidx(bi, 0);
                            tile = 2 * NSB + 2 * x + 1;
                        } else { bi = 2 * (blk - NSB - NX); bj = bi + 1; }  // upper block of a 32-token k block
                    } else {
                        tile = 2 * NSB + 2 * (blk - NPB);
                    }
                    f4 val = {0.f, 0.f, 0.f, 0.f};
                    if (tile >= 0) {
#pragma unroll
                        for (int pp = 0; pp < NP; ++pp) val += *reinterpret_cast<const f4*>(&sm.gp[pp][tile][i][m4]);
                    }
                    if (isp) {
                        h4 hv;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            hv[e] = static_cast<_Float16>((bi > bj || m4 + e <= i) ? val[e] : 0.f);
                        const int R = 16 * bi + i;
                        *reinterpret_cast<h4*>(&sm.p[R][kpos(16 * bj + m4)]) = hv;
                    } else {
                        const int x = blk - NPB;
                        h4 hv;
#pragma unroll
                        for (int e = 0; e < 4; ++e) hv[e] = static_cast<_Float16>(-val[e]);
                        *reinterpret_cast<h4*>(&sm.tb[NSB + x][i][m4]) = hv;
                    }
                }
            }
        }
        __syncthreads();  // B3

        // ---------------- state pass on this wave's columns
        {
            // v at token 16 rt + 4 g4 + i, column col + 16 ct + r (accumulator layout).
            float vv[NSB][NCT][4];
#pragma unroll
            for (int rt = 0; rt < NSB; ++rt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        vv[rt][ct][i] = bf16_to_f32(sm.v[16 * rt + 4 * g4 + i][col + 16 * ct + r]);
            // Exponent for this chunk from max(|S|, |v|) over the wave's columns.
            float mv = 0.f;
#pragma unroll
            for (int rt = 0; rt < NSB; ++rt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i) mv = fmaxf(mv, fabsf(vv[rt][ct][i]));
            float ms = 0.f;
#pragma unroll
            for (int rt = 0; rt < 8; ++rt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i) ms = fmaxf(ms, fabsf(S[rt][ct][i]));
            const int nex = value_exponent(wave_max_nonneg(fmaxf(ms * ldexpf(1.f, -ex), mv)), ex);
            if (nex != ex) {  // wave-uniform
                const float f = ldexpf(1.f, nex - ex);
#pragma unroll
                for (int rt = 0; rt < 8; ++rt)
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) S[rt][ct] *= f;
                ex = nex;
            }
            const float sig = ldexpf(1.f, ex);

            h8 s16[4][NCT];  // B operand of K~ S and Q~ S: [channel k-step][column tile]
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        s16[ks][ct][m] = static_cast<_Float16>(S[2 * ks][ct][m]);
                        s16[ks][ct][4 + m] = static_cast<_Float16>(S[2 * ks + 1][ct][m]);
                    }

            // X = sigma v - K~ S (fp32), then Delta = T X (scaled units) by forward
            // block substitution: Delta_J = T_JJ (X_J - sum_{K<J} G_JK Delta_K).
            h4 dh[NSB][NCT];  // Delta_J as fp16 (rows 4 g4 + i of sub-block J)
            {
                f4 y[NSB][NCT];
#pragma unroll
                for (int rt = 0; rt < NSB; ++rt) {
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) y[rt][ct] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        const h8 kf8 = *reinterpret_cast<const h8*>(&sm.kt[16 * rt + r][32 * ks + 8 * g4]);
#pragma unroll
                        for (int ct = 0; ct < NCT; ++ct) y[rt][ct] = mfma16(kf8, s16[ks][ct], y[rt][ct]);
                    }
                }
#pragma unroll
                for (int J = 0; J < NSB; ++J) {
                    const h4 tjj = *reinterpret_cast<const h4*>(&sm.tb[J][r][4 * g4]);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        f4 z;
#pragma unroll
                        for (int m = 0; m < 4; ++m) z[m] = fmaf(vv[J][ct][m], sig, -y[J][ct][m]);
#pragma unroll
                        for (int K = 0; K < NSB - 1; ++K) {
                            if (K < J) {
                                const h4 gjk = *reinterpret_cast<const h4*>(&sm.tb[NSB + xidx(J, K)][r][4 * g4]);
                                z = mfma16k16(gjk, dh[K][ct], z);
                            }
                        }
                        h4 zh;
#pragma unroll
                        for (int m = 0; m < 4; ++m) zh[m] = static_cast<_Float16>(z[m]);
                        const f4 d = mfma16k16(tjj, zh, f4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                        for (int m = 0; m < 4; ++m) dh[J][ct][m] = static_cast<_Float16>(d[m]);
                    }
                }
            }
            h8 d16[NKB][NCT];  // B operand of P Delta and K-bar^T Delta (k = 32 tokens, permuted)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) d16[kb][ct] = cat(dh[2 * kb][ct], dh[2 * kb + 1][ct]);

            // O = scale (Q~ S + P Delta)
            {
                const float os = scale * ldexpf(1.f, -ex);
                const int vlim = valid - 4 * g4;  // rows of this lane group still inside the chunk
                const int64_t stride = static_cast<int64_t>(H) * D;
#pragma unroll
                for (int rt = 0; rt < NSB; ++rt) {
                    h8 qf8[4];
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        qf8[ks] = *reinterpret_cast<const h8*>(&sm.qt[16 * rt + r][32 * ks + 8 * g4]);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        f4 a = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int kb = 0; kb <= rt / 2; ++kb)  // P is causal: k blocks up to this row's
                            a = mfma16(*reinterpret_cast<const h8*>(&sm.p[16 * rt + r][32 * kb + 8 * g4]), d16[kb][ct], a);
#pragma unroll
                        for (int ks = 0; ks < 4; ++ks) a = mfma16(qf8[ks], s16[ks][ct], a);
                        Tout* op = o + ((c0 + 16 * rt + 4 * g4) * H + h) * D + col + 16 * ct + r;
                        if (valid == C) {
#pragma unroll
                            for (int i = 0; i < 4; ++i) st(op, i * stride, a[i] * os);
                        } else {
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                if (16 * rt + i < vlim) st(op, i * stride, a[i] * os);
                        }
                    }
                }
            }

            // S <- Lambda_last S + K-bar^T Delta  (all in the scaled units)
#pragma unroll
            for (int rt = 0; rt < 8; ++rt) {
                const f4 lam = *reinterpret_cast<const f4*>(&sm.lam[16 * rt + 4 * g4]);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) S[rt][ct] *= lam;
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    const h8 kb8 = *reinterpret_cast<const h8*>(&sm.kbt[16 * rt + r][32 * kb + 8 * g4]);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) S[rt][ct] = mfma16(kb8, d16[kb][ct], S[rt][ct]);
                }
            }
        }
        if (snapping && it.p0 + ((c0 + C < t1 ? c0 + C : t1) - t0) == sc.next) {
            store_state<NCT>(snaps + (sc.row * H + h) * D * D, S, ldexpf(1.f, -ex), g4, r, col);
            sc.next += interval;
            ++sc.row;
        }
    }

    // Final state.
    if (it.sout >= 0 && out_state) {
        const float un = ldexpf(1.f, -ex);
        float* dst = out_state + (static_cast<int64_t>(it.sout) * H + h) * D * D;
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dst[(16 * rt + 4 * g4 + i) * D + col + 16 * ct + r] = S[rt][ct][i] * un;
    }
}

// ---------------------------------------------------------------------------
// Full-mode kernel with wave roles: 32-token chunks (two sub-blocks); waves
// 0-3 run the state pass of chunk c on 32 state columns each while waves
// 4-11 prepare the next chunks (cumulative gates, Grams, the diagonal solves,
// P and the cross Grams) into the other half of double-buffered operand tiles.
// Each SIMD then holds one MFMA/LDS-heavy state wave and two VALU-heavy gate
// waves of the same chain, and every A operand is read from LDS by 4 waves.
namespace ws {
constexpr int C = 32, NSB = 2, NX = 1, TP = C + 8;
constexpr int NSW = 4;   // state waves
constexpr int NGW = 8;   // gate waves
constexpr int NW = NSW + NGW;
constexpr int NCT = 2;   // 16-column tiles per state wave
constexpr int NP = NGW / NSB;  // channel parts per sub-block (gate waves per sub-block)
constexpr int CPG = D / NP, KS = CPG / 32;
constexpr int GT = NGW * 64;            // gate threads
constexpr int VU = (C * D / 8) / GT;    // 16-byte pieces of the v tile per gate thread
constexpr bool STAGE_O = true;          // o goes through an LDS tile and leaves as whole rows

struct alignas(16) Tiles {               // operands of one chunk's state pass
    _Float16 qt[C][QP];                  // Q~   [token][channel, operand order]
    _Float16 kt[C][QP];                  // K~   [token][channel, operand order]
    _Float16 kbt[D][TP];                 // K-bar^T [channel][token, operand order]
    _Float16 tb[NSB + NX][SB][BP];       // T00, T11, -G10
    _Float16 p[C][TP];                   // P    [token][token, operand order]
    uint16_t v[C][QP];                   // v tile (bf16 bits) [token][column]
    uint16_t og[C][QP];                  // output gate tile (bf16 bits), gated output only
    float lam[D];                        // Lambda_last
};
struct alignas(16) Smem {
    Tiles tl[2];
    float otile[C][D + 4];               // o of the chunk, for the gated RMSNorm epilogue
    float nw[D];                         // RMSNorm weight
    _Float16 rbs[SB][QP];                // k exp(tot_0 - G), sub-block 0 [token][channel]
    float gp[NP][2 * NSB + 2 * NX][SB][GP];
    float a[NSB][SB][20];                // A_JJ = Diag(beta) G_JJ, strictly lower, by row
    float etot[NSB][D];
    float beta[2][C];                    // beta of the chunks in phases 1-2 and 3 (by chunk parity)
    int alive[NSW];                      // propagation modes: state wave still nonzero in fp16
};
}  // namespace ws

// Modes of the 12-wave kernel.  FULL: the chunked prefill of a sequence or
// segment.  MAP and CORR propagate a d_k x d_k matrix X through a segment with
// v = 0 (X <- Diag(Lambda) X + K-bar^T Delta, Delta = -T K~ X): MAP from the
// identity, storing X at the end (the segment's state map); CORR from the
// segment's true initial state, adding X's read-out scale (Q~ X + P Delta)
// to o (and X to the state snapshots).  Both stop as soon as the fp16 copy
// of X is zero on every state wave: with g <= 0 X can then only shrink and
// every later product it feeds is exactly zero.
enum { MODE_FULL = 0, MODE_MAP = 1, MODE_CORR = 2 };

template <typename Tout, bool SNAP, bool GATED, int MODE = MODE_FULL>
__global__ __launch_bounds__(ws::NW * 64) __attribute__((amdgpu_waves_per_eu(ws::NW / 4)))
void chunk_ws_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ g,
    const float* __restrict__ beta, float scale, const ChunkItem* __restrict__ items, int H,
    const float* __restrict__ h0, const float* __restrict__ staged, Tout* __restrict__ o,
    float* __restrict__ out_state, float* __restrict__ snaps, int interval,
    const uint16_t* __restrict__ ogate, const float* __restrict__ nweight, float neps,
    float* __restrict__ bout, int* __restrict__ mflags) {
    using namespace ws;
    static_assert(MODE == MODE_FULL || !GATED, "the gated epilogue needs the whole read-out");
    constexpr bool PROP = MODE != MODE_FULL;
    __shared__ ws::Smem sm;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, r = l & 15, g4 = l >> 4;
    const bool gate = w >= NSW;  // wave-uniform role

    const ChunkItem it = items[blockIdx.x / H];
    const int h = blockIdx.x % H;
    const int64_t t0 = it.t0, t1 = it.t1;
    const int nch = static_cast<int>((t1 - t0 + C - 1) / C);
    const int rowe = H * D;  // elements per token row

    // The two roles run separate loops with the same trip count and exactly
    // two barriers per iteration (the barriers pair up across the roles).
    // Iteration c: the state waves run chunk c (Y, Delta, o into the LDS o
    // tile, the S update) in interval 1, then store o and prepare chunk c + 1's
    // operands in interval 2; the gate waves solve chunk c + 1's diagonal
    // blocks and run phase 1 of chunk c + 2 in interval 1, and phase 2 of chunk
    // c + 2 in interval 2.  The state waves also sum chunk c + 1's cross-block
    // partials into P10 and -G10 at the start of interval 1.
    // Each role's memory traffic stays inside its own branch, and every
    // iteration issues the same loads (past the end of the sequence they fall
    // outside the buffer range and read zeros): the compiler can then count
    // outstanding loads exactly and never waits for the prefetch of chunk
    // c + 3 before it is consumed.
    if (gate) {
        // ---- gate waves: sub-block I, channel part `part`; raw inputs fetched ahead
        const int gw = w - NSW;
        const int I = gw / NP, part = gw % NP;
        const int gtid = tid - NSW * 64;
        const int tok = SB * I + r;
        u4 kw[KS], qw[KS], vp[VU], gp_[VU];
        f4 ga[KS], gb[KS];
        float bt = 0.f;
        // Tokens at or past the end of the sequence lie outside the buffer range
        // of the chunk (valid tokens x row bytes), so their loads return zeros.
        auto valid_at = [&](int64_t cs) {
            const int64_t n = t1 - cs;
            return static_cast<uint32_t>(n < 0 ? 0 : n < C ? n : C);
        };
        auto fetch_gate = [&](int64_t cs) {  // k, q, g, beta of this lane's token
            const uint32_t vld = valid_at(cs);
            const int64_t cb = (cs * H + h) * D;
            const auto rk = rsrc(k + cb, vld * rowe * 2);
            const auto rq = rsrc(q + cb, MODE == MODE_MAP ? 0u : vld * rowe * 2);  // no read-out in MAP
            const auto rg = rsrc(g + cb, vld * rowe * 4);
            // beta is read by the channel-part-0 waves only (an empty range for the others)
            const auto rb = rsrc(beta + cs * H + h, part == 0 ? vld * H * 4 : 0u);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int off = tok * rowe + CPG * part + 32 * ks + 8 * g4;
                kw[ks] = bload16(rk, 2 * off);
                qw[ks] = bload16(rq, 2 * off);
                const u4 a0 = bload16(rg, 4 * off), a1 = bload16(rg, 4 * off + 16);
                ga[ks] = f4{__uint_as_float(a0[0]), __uint_as_float(a0[1]), __uint_as_float(a0[2]), __uint_as_float(a0[3])};
                gb[ks] = f4{__uint_as_float(a1[0]), __uint_as_float(a1[1]), __uint_as_float(a1[2]), __uint_as_float(a1[3])};
            }
            bt = bload4(rb, 4 * tok * H);
        };
        auto fetch_v = [&](int64_t cs) {  // v (and the output gate) in the staging layout
            if (PROP) return;  // v = 0 when a matrix is propagated
            const auto rv = rsrc(v + (cs * H + h) * D, valid_at(cs) * rowe * 2);
            const auto rog = rsrc(ogate + (cs * H + h) * D, GATED ? valid_at(cs) * rowe * 2 : 0u);
#pragma unroll
            for (int j = 0; j < VU; ++j) {
                const int e = gtid + GT * j, vt = e >> 4, vc = (e & 15) * 8;
                vp[j] = bload16(rv, 2 * (vt * rowe + vc));
                if (GATED) gp_[j] = bload16(rog, 2 * (vt * rowe + vc));
            }
        };
        fetch_gate(t0);
        fetch_v(t0);
        // P01 (tokens of sub-block 0 against sub-block 1) is zero in every chunk:
        // written once into both operand sets, never touched again.
        for (int e = gtid; e < 2 * SB * SB; e += GT)
            sm.tl[e >> 8].p[(e >> 4) & 15][kpos(SB + (e & 15))] = static_cast<_Float16>(0.f);
        h8 l16[KS], q16[KS], rb16[KS];  // gate registers carried from phase 1 to phase 2

        for (int c = -2; c < nch; ++c) {
            const bool gwork = c + 2 < nch;              // phases 1 and 2 of chunk c + 2
            const bool w3 = c + 1 >= 0 && c + 1 < nch;   // the solves of chunk c + 1
            Tiles& nxt = sm.tl[c & 1];                   // chunk c + 2 (chunk c's buffer)
            Tiles& t3 = sm.tl[(c + 1) & 1];
            float* const bnx = sm.beta[c & 1];           // beta of chunk c + 2
            const float* const b3 = sm.beta[(c + 1) & 1];

            constexpr float LOG2E = 1.4426950408889634f;
            // The raw inputs of chunk c + 2 are unpacked first (cumulative
            // gates included).  Sub-block 0 waves then issue the fetch of chunk
            // c + 3 into the same registers at once (after their solves),
            // sub-block 1 waves only after their phase-1 work, so the two
            // groups' loads do not queue together (one fetch site, so the
            // compiler still counts the loads exactly).
            float kf[KS][8], qf[KS][8], G[KS][8];
            if (gwork) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    unpack_bf16x8(kw[ks], kf[ks]);
                    unpack_bf16x8(qw[ks], qf[ks]);
#pragma unroll
                    for (int m = 0; m < 8; ++m)
                        G[ks][m] = row_scan16((m < 4 ? ga[ks][m] : gb[ks][m - 4]) * LOG2E);
                }
                if (part == 0 && g4 == 0) bnx[tok] = bt;
            }
            if (w3 && gw < 2 * NSB) {
                // Column-oriented substitution for T = (I + A_JJ)^-1 of chunk c + 1,
                // two waves per block: columns 8 hh .. 8 hh + 7.  Lane (i, g4) holds
                // row i of columns 8 hh + 2 g4 + {0, 1} and row i of A (zero on and
                // above the diagonal).  Step m broadcasts x_m of each column across
                // its 16-lane row (DPP) and updates every row at once:
                // x_i -= A[i][m] x_m.  Column j has x_m = 0 for m < j, so the right
                // half starts at step 8; step 15 changes nothing.
                const int J = gw & 1, hh = gw >> 1;  // the longer halves on SIMDs 0 and 1
                f4 arow[4];
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) arow[cc] = *reinterpret_cast<const f4*>(&sm.a[J][r][4 * cc]);
                const int cs0 = 8 * hh + 2 * g4;
                const float b0 = b3[SB * J + cs0], b1 = b3[SB * J + cs0 + 1];
                float x[2] = {r == cs0 ? 1.f : 0.f, r == cs0 + 1 ? 1.f : 0.f};
                if (hh == 0) subst_range2<0>(x, arow, std::make_integer_sequence<int, SB - 1>{});
                else subst_range2<8>(x, arow, std::make_integer_sequence<int, SB - 9>{});
                typedef _Float16 h2 __attribute__((ext_vector_type(2)));
                *reinterpret_cast<h2*>(&t3.tb[J][r][cs0]) =
                    h2{static_cast<_Float16>(x[0] * b0), static_cast<_Float16>(x[1] * b1)};
            }
            auto phase1 = [&]() {
                constexpr float FAST_SPAN = 8.f * LOG2E;
                f4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
                bool redo = false;  // wave-uniform: a k-step beyond the reference's range
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int ch = CPG * part + 32 * ks + 8 * g4;
                    float Gt[8];
#pragma unroll
                    for (int m = 0; m < 8; ++m) Gt[m] = row_bcast16<15>(G[ks][m]);
                    // Factors referenced to half the sub-block total: a = exp(G - tot/2),
                    // 1/a, and the channel's exp(tot/2), which is a at the last token.
                    // exp(G) = a exp(tot/2) and exp(tot - G) = exp(tot/2) / a.
                    float xa[8], La[8], Ra[8], Qa[8], hh[8];
                    float span = 0.f;
#pragma unroll
                    for (int m = 0; m < 8; ++m) {
                        xa[m] = fmaf(-0.5f, Gt[m], G[ks][m]);
                        span = fmaxf(span, fabsf(xa[m]));
                        const float a = __builtin_amdgcn_exp2f(xa[m]);
                        const float ia = __builtin_amdgcn_exp2f(-xa[m]);
                        La[m] = kf[ks][m] * a;
                        Ra[m] = kf[ks][m] * ia;
                        Qa[m] = qf[ks][m] * a;
                        hh[m] = row_bcast16<15>(a);
                    }
#pragma unroll
                    for (int m = 0; m < 8; ++m) {
                        l16[ks][m] = static_cast<_Float16>(La[m] * hh[m]);   // k exp(G)
                        rb16[ks][m] = static_cast<_Float16>(Ra[m] * hh[m]);  // k exp(tot - G)
                        q16[ks][m] = static_cast<_Float16>(Qa[m] * hh[m]);   // q exp(G)
                    }
                    if (!__any(span > FAST_SPAN)) {
                        h8 la, ra, qa;
#pragma unroll
                        for (int m = 0; m < 8; ++m) {
                            la[m] = static_cast<_Float16>(La[m]);
                            ra[m] = static_cast<_Float16>(Ra[m]);
                            qa[m] = static_cast<_Float16>(Qa[m]);
                        }
                        accA = mfma16(la, ra, accA);
                        accP = mfma16(qa, ra, accP);
                    } else {
#pragma unroll
                        for (int m = 0; m < 8; ++m) {
                            accA = mfma4(La[m], Ra[m], accA);
                            accP = mfma4(Qa[m], Ra[m], accP);
                        }
                        redo = redo || __any(span > SAFE_SPAN);
                    }
                    if (r == 15) {  // exp(tot) = exp(tot/2)^2
                        *reinterpret_cast<f4*>(&sm.etot[I][ch]) =
                            f4{hh[0] * hh[0], hh[1] * hh[1], hh[2] * hh[2], hh[3] * hh[3]};
                        *reinterpret_cast<f4*>(&sm.etot[I][ch + 4]) =
                            f4{hh[4] * hh[4], hh[5] * hh[5], hh[6] * hh[6], hh[7] * hh[7]};
                    }
                    if (I == 0) *reinterpret_cast<h8*>(&sm.rbs[r][ch]) = rb16[ks];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sm.gp[part][2 * I][4 * g4 + i][r] = accA[i];  // beta of row i is applied in the sum
                    sm.gp[part][2 * I + 1][4 * g4 + i][r] = accP[i];
                }
                if (redo) {
                    // Exponents beyond the fp32 range of the half-total reference:
                    // the wave's phase 1 again, entry by entry from its raw inputs
                    // (read again, so nothing stays live for this rare case), over
                    // everything written above (the same wave's LDS writes
                    // complete in order).
                    const int64_t cs = t0 + static_cast<int64_t>(c + 2) * C;
                    const uint32_t vld = valid_at(cs);
                    const int64_t cb = (cs * H + h) * D;
                    const auto rk = rsrc(k + cb, vld * rowe * 2), rq = rsrc(q + cb, vld * rowe * 2);
                    const auto rg = rsrc(g + cb, vld * rowe * 4);
                    f4 oa = {0.f, 0.f, 0.f, 0.f}, op = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const int ch = CPG * part + 32 * ks + 8 * g4;
                        const int off = tok * rowe + ch;
                        const u4 a0 = bload16(rg, 4 * off), a1 = bload16(rg, 4 * off + 16);
                        float gr[8], et[8], kr[8], qr[8];
                        unpack_bf16x8(bload16(rk, 2 * off), kr);
                        unpack_bf16x8(bload16(rq, 2 * off), qr);
#pragma unroll
                        for (int m = 0; m < 4; ++m) {
                            gr[m] = __uint_as_float(a0[m]);
                            gr[4 + m] = __uint_as_float(a1[m]);
                        }
                        phase1_direct<true>(kr, qr, gr, g4, l16[ks], q16[ks], rb16[ks], et, oa, op);
                        if (r == 15) {
                            *reinterpret_cast<f4*>(&sm.etot[I][ch]) = f4{et[0], et[1], et[2], et[3]};
                            *reinterpret_cast<f4*>(&sm.etot[I][ch + 4]) = f4{et[4], et[5], et[6], et[7]};
                        }
                        if (I == 0) *reinterpret_cast<h8*>(&sm.rbs[r][ch]) = rb16[ks];
                    }
                    *reinterpret_cast<f4*>(&sm.gp[part][2 * I][r][4 * g4]) = oa;
                    *reinterpret_cast<f4*>(&sm.gp[part][2 * I + 1][r][4 * g4]) = op;
                }
            };
            if (gwork && I == 1) phase1();
            fetch_gate(t0 + static_cast<int64_t>(c + 3) * C);
            if (gwork && I == 0) phase1();
            __syncthreads();
            if (gwork && !PROP) {  // v (and the output gate) of chunk c + 2
#pragma unroll
                for (int j = 0; j < VU; ++j) {
                    const int e = gtid + GT * j, vt = e >> 4, vc = (e & 15) * 8;
                    *reinterpret_cast<u4*>(&nxt.v[vt][vc]) = vp[j];
                    if (GATED) *reinterpret_cast<u4*>(&nxt.og[vt][vc]) = gp_[j];
                }
            }
            if (gwork) {
                f4 a10 = {0.f, 0.f, 0.f, 0.f}, p10 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int ch = CPG * part + 32 * ks + 8 * g4;
                    const f4 oa = *reinterpret_cast<const f4*>(&sm.etot[1 - I][ch]);
                    const f4 ob = *reinterpret_cast<const f4*>(&sm.etot[1 - I][ch + 4]);
                    const h8 of = {static_cast<_Float16>(oa[0]), static_cast<_Float16>(oa[1]),
                                   static_cast<_Float16>(oa[2]), static_cast<_Float16>(oa[3]),
                                   static_cast<_Float16>(ob[0]), static_cast<_Float16>(ob[1]),
                                   static_cast<_Float16>(ob[2]), static_cast<_Float16>(ob[3])};
                    h8 kv = l16[ks], qv = q16[ks], bv = rb16[ks];
                    if (I == 1) {
                        kv *= of;
                        qv *= of;
                    } else {
                        bv *= of;
                    }
                    const int cb = ch & ~31, p0 = cb + (g4 < 2 ? 16 * g4 : 16 * g4 - 28), p1 = p0 + 8;
                    *reinterpret_cast<h4*>(&nxt.kt[tok][p0]) = __builtin_shufflevector(kv, kv, 0, 1, 2, 3);
                    *reinterpret_cast<h4*>(&nxt.kt[tok][p1]) = __builtin_shufflevector(kv, kv, 4, 5, 6, 7);
                    *reinterpret_cast<h4*>(&nxt.qt[tok][p0]) = __builtin_shufflevector(qv, qv, 0, 1, 2, 3);
                    *reinterpret_cast<h4*>(&nxt.qt[tok][p1]) = __builtin_shufflevector(qv, qv, 4, 5, 6, 7);
                    const int tp = kpos(tok);
#pragma unroll
                    for (int m = 0; m < 8; ++m) nxt.kbt[ch + m][tp] = bv[m];
                    if (I == 1) {
                        const h8 rv = *reinterpret_cast<const h8*>(&sm.rbs[r][ch]);
                        a10 = mfma16(l16[ks], rv, a10);
                        p10 = mfma16(q16[ks], rv, p10);
                    }
                }
                if (I == 1) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        sm.gp[part][2 * NSB][4 * g4 + i][r] = a10[i];
                        sm.gp[part][2 * NSB + 1][4 * g4 + i][r] = p10[i];
                    }
                }
                // A_JJ on gate waves 0 and 1, lam, P00 and P11 on gate waves 2 and 3
                // (sub-block 0: the lighter phase 2)
                if (gtid >= 128 && gtid < 128 + D) nxt.lam[gtid - 128] = sm.etot[0][gtid - 128] * sm.etot[1][gtid - 128];
                if (gtid < 128) {  // A_JJ = Diag(beta) G_JJ, strictly lower, 4 entries per thread
                    const int J = gtid >> 6, i = (gtid >> 2) & 15, m4 = (gtid & 3) * 4;
                    f4 val = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int pp = 0; pp < NP; ++pp) val += *reinterpret_cast<const f4*>(&sm.gp[pp][2 * J][i][m4]);
                    const float bi = bnx[SB * J + i];
                    f4 av;
#pragma unroll
                    for (int e = 0; e < 4; ++e) av[e] = m4 + e < i ? val[e] * bi : 0.f;
                    *reinterpret_cast<f4*>(&sm.a[J][i][m4]) = av;
                }
                if (gtid >= 128 && gtid < 256) {  // P00 and P11, 4 consecutive entries per thread
                    const int blk = (gtid >> 6) & 1, i = (gtid >> 2) & 15, m4 = (gtid & 3) * 4;
                    f4 val = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int pp = 0; pp < NP; ++pp) val += *reinterpret_cast<const f4*>(&sm.gp[pp][2 * blk + 1][i][m4]);
                    h4 hv;
#pragma unroll
                    for (int e = 0; e < 4; ++e) hv[e] = static_cast<_Float16>(m4 + e <= i ? val[e] : 0.f);
                    *reinterpret_cast<h4*>(&nxt.p[16 * blk + i][kpos(16 * blk + m4)]) = hv;
                }
            }
            fetch_v(t0 + static_cast<int64_t>(c + 3) * C);
            __syncthreads();
            // propagation modes: stop with the state waves once X is zero in fp16
            if (PROP && c + 1 >= 0 && c + 1 < nch && !(sm.alive[0] | sm.alive[1] | sm.alive[2] | sm.alive[3]))
                break;
        }
    } else {
        // ---- state waves: S[16 rt + 4 g4 + i][col + 16 ct + r] * 2^ex in S[rt][ct][i]
        const int col = 32 * (w & 3);
        f4 S[8][NCT];
        int ex = 0;
        // Propagation modes: the exponent may rise at most PROP_HEADROOM above
        // the one X starts at, so X's fp16 copy -- and with it the pass --
        // stops once max|X| has fallen below about 2^-40 of its start.
        int ex_cap = 1 << 20;
        h8 d16[NCT];      // fp16 Delta (B operand of P Delta, K-bar^T Delta), chunk-local
        bool exited = false;  // propagation modes: X became zero in fp16
        {
            const float* src = nullptr;
            if (it.sin >= 0 && h0) {
                src = h0 + (static_cast<int64_t>(it.sin) * H + h) * D * D;
            } else if (it.sin <= -2) {
                // CORR: a segment after one whose map vanished starts from that
                // segment's zero-start final state (the scan staged nothing)
                const int64_t z = -it.sin - 2;
                if (MODE == MODE_CORR && it.p0 > 0 && mflags[(z - 1) * H + h] == 0)
                    src = bout + ((z - 1) * H + h) * D * D;
                else
                    src = staged + (z * H + h) * D * D;
            }
#pragma unroll
            for (int rt = 0; rt < 8; ++rt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i)  // MAP starts from the identity
                        S[rt][ct][i] = (MODE == MODE_MAP && 16 * rt + 4 * g4 + i == col + 16 * ct + r) ? 1.f : 0.f;
            if (src && MODE != MODE_MAP) {
#pragma unroll
                for (int rt = 0; rt < 8; ++rt)
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                        for (int i = 0; i < 4; ++i) S[rt][ct][i] = src[(16 * rt + 4 * g4 + i) * D + col + 16 * ct + r];
            }
        }
        // Operands of the next chunk's state pass (interval 2; interval 1 for
        // max|S| with the gated epilogue): max|S| over the wave and fp16 S at
        // the current exponent, then chunk c + 1's v (staged two intervals
        // earlier), the scale exponent from max(|S|, |v|), and -- only when
        // the exponent moves -- the rescaled S and its fp16 copy again.
        float vv[NSB][NCT][4];
        h8 s16[4][NCT];
        float sig = 1.f;
        auto to_fp16 = [&]() {  // B operand of both K~ S and Q~ S
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        s16[ks][ct][m] = static_cast<_Float16>(S[2 * ks][ct][m]);
                        s16[ks][ct][4 + m] = static_cast<_Float16>(S[2 * ks + 1][ct][m]);
                    }
        };
        auto state_max = [&]() {  // max|S| * 2^ex over the wave, with fp16 S at exponent ex
            float ms = 0.f;
#pragma unroll
            for (int rt = 0; rt < 8; ++rt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i) ms = fmaxf(ms, fabsf(S[rt][ct][i]));
            to_fp16();
            return wave_max_nonneg(ms);
        };
        auto prepare = [&](const Tiles& t, float msw) {
#pragma unroll
            for (int rt = 0; rt < NSB; ++rt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        vv[rt][ct][i] = PROP ? 0.f : bf16_to_f32(t.v[16 * rt + 4 * g4 + i][col + 16 * ct + r]);
            float mv = 0.f;
#pragma unroll
            for (int rt = 0; rt < NSB; ++rt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i) mv = fmaxf(mv, fabsf(vv[rt][ct][i]));
            int nex = value_exponent(fmaxf(msw * ldexpf(1.f, -ex), wave_max_nonneg(mv)), ex);
            if (PROP) {
                if (ex_cap == (1 << 20)) ex_cap = nex + PROP_HEADROOM;  // X's first exponent
                nex = nex < ex_cap ? nex : ex_cap;
            }
            if (nex != ex) {
                const float f = ldexpf(1.f, nex - ex);
#pragma unroll
                for (int rt = 0; rt < 8; ++rt)
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) S[rt][ct] *= f;
                ex = nex;
                to_fp16();
            }
            sig = ldexpf(1.f, ex);
        };
        const bool snapping = SNAP && snaps != nullptr && it.snap >= 0;
        SnapCursor sc{};
        if (snapping) sc.init(it, interval);
        if (GATED && tid < D) sm.nw[tid] = nweight[tid];  // read after several barriers
        // Gated epilogue: this wave normalises tokens 8 w .. 8 w + 7 of the chunk;
        // lane l takes token 8 w + l / 8, channels 16 (l % 8) .. 16 (l % 8) + 15.
        // The indices are rebuilt where used instead of held across the loop.
        auto epi_lane = [&]() {
            int x = l;
            asm volatile("" : "+v"(x));
            return x;
        };
        u4 ogr[2];  // gated output: this lane's output gate, read in interval 1
        f4 opre[4];  // CORR: this wave's o rows of chunk c, read an interval before the add
        for (int c = -2; c < nch; ++c) {
            const bool swork = c >= 0;        // run chunk c
            const int64_t c0 = t0 + static_cast<int64_t>(c) * C;
            const Tiles& cur = sm.tl[c & 1];
            Tiles& nxt = sm.tl[(c + 1) & 1];
            const int valid = static_cast<int>(t1 - c0 < C ? t1 - c0 : C);
            if (c + 1 >= 0 && c + 1 < nch && w >= 2) {
                // P10 (wave 2) and -G10 (wave 3) of chunk c + 1 from the cross-Gram
                // partials of its phase 2, 4 consecutive entries per lane (SIMDs 2
                // and 3 carry the shorter halves of the diagonal solves).
                const int i = (l >> 2) & 15, m4 = (l & 3) * 4;
                const int tile = w == 2 ? 2 * NSB + 1 : 2 * NSB;
                f4 val = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int pp = 0; pp < NP; ++pp) val += *reinterpret_cast<const f4*>(&sm.gp[pp][tile][i][m4]);
                h4 hv;
                const float sgn = w == 2 ? 1.f : -1.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) hv[e] = static_cast<_Float16>(sgn * val[e]);
                if (w == 2) *reinterpret_cast<h4*>(&nxt.p[SB + i][kpos(m4)]) = hv;
                else *reinterpret_cast<h4*>(&nxt.tb[2][i][m4]) = hv;
            }
            if (MODE == MODE_CORR && swork) {
                const auto ro = rsrc(o + (c0 * H + h) * D, static_cast<uint32_t>(valid) * rowe * sizeof(Tout));
                const int el = epi_lane(), c4 = 4 * (el & 31);
#pragma unroll
                for (int k2 = 0; k2 < 4; ++k2) {
                    const int row = 8 * (w & 3) + 2 * k2 + (el >> 5);
                    opre[k2] = load4(ro, (row * rowe + c4) * static_cast<int>(sizeof(Tout)), o);
                }
            }
            if (swork) {
                f4 y[NSB][NCT];
#pragma unroll
                for (int rt = 0; rt < NSB; ++rt) {
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) y[rt][ct] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        const h8 kf8 = *reinterpret_cast<const h8*>(&cur.kt[16 * rt + r][32 * ks + 8 * g4]);
#pragma unroll
                        for (int ct = 0; ct < NCT; ++ct) y[rt][ct] = mfma16(kf8, s16[ks][ct], y[rt][ct]);
                    }
                }
                const h4 t00 = *reinterpret_cast<const h4*>(&cur.tb[0][r][4 * g4]);
                const h4 t11 = *reinterpret_cast<const h4*>(&cur.tb[1][r][4 * g4]);
                const h4 g10 = *reinterpret_cast<const h4*>(&cur.tb[2][r][4 * g4]);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    h4 x0;
                    f4 x1;
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        x0[m] = static_cast<_Float16>(fmaf(vv[0][ct][m], sig, -y[0][ct][m]));
                        x1[m] = fmaf(vv[1][ct][m], sig, -y[1][ct][m]);
                    }
                    const f4 d0 = mfma16k16(t00, x0, f4{0.f, 0.f, 0.f, 0.f});
                    h4 d0h;
#pragma unroll
                    for (int m = 0; m < 4; ++m) d0h[m] = static_cast<_Float16>(d0[m]);
                    const f4 z = mfma16k16(g10, d0h, x1);
                    h4 zh;
#pragma unroll
                    for (int m = 0; m < 4; ++m) zh[m] = static_cast<_Float16>(z[m]);
                    const f4 d1 = mfma16k16(t11, zh, f4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        d16[ct][m] = d0h[m];
                        d16[ct][4 + m] = static_cast<_Float16>(d1[m]);
                    }
                }
                // o of chunk c, right after its Delta (no read-out in MAP mode)
                const float os = scale * ldexpf(1.f, -ex);
                const int vlim = valid - 4 * g4;  // rows of this lane group still inside the chunk
                const auto ro = rsrc(o + (c0 * H + h) * D, static_cast<uint32_t>(valid) * rowe * sizeof(Tout));
                const int vo = static_cast<int>(((4 * g4) * rowe + col + r) * sizeof(Tout));
#pragma unroll
                for (int rt = 0; rt < (MODE == MODE_MAP ? 0 : NSB); ++rt) {
                    h8 qf8[4];
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        qf8[ks] = *reinterpret_cast<const h8*>(&cur.qt[16 * rt + r][32 * ks + 8 * g4]);
                    const h8 pf = *reinterpret_cast<const h8*>(&cur.p[16 * rt + r][8 * g4]);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        f4 a = mfma16(pf, d16[ct], f4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                        for (int ks = 0; ks < 4; ++ks) a = mfma16(qf8[ks], s16[ks][ct], a);
                        const int voc = vo + static_cast<int>(16 * ct * sizeof(Tout));
                        if (GATED || STAGE_O) {
#pragma unroll
                            for (int i = 0; i < 4; ++i) sm.otile[16 * rt + 4 * g4 + i][col + 16 * ct + r] = a[i] * os;
                        } else if (valid == C) {
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                bstore(ro, voc, static_cast<int>((16 * rt + i) * rowe * sizeof(Tout)), a[i] * os, o);
                        } else {
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                if (16 * rt + i < vlim)
                                    bstore(ro, voc, static_cast<int>((16 * rt + i) * rowe * sizeof(Tout)), a[i] * os, o);
                        }
                    }
                }
                if (GATED) {  // the output gate of this wave's epilogue rows, before its tile is reused
                    const int el = epi_lane(), erow = 8 * (w & 3) + (el >> 3), ecol = 16 * (el & 7);
                    ogr[0] = *reinterpret_cast<const u4*>(&cur.og[erow][ecol]);
                    ogr[1] = *reinterpret_cast<const u4*>(&cur.og[erow][ecol + 8]);
                }
#pragma unroll
                for (int rt = 0; rt < 8; ++rt) {
                    const f4 lam = *reinterpret_cast<const f4*>(&cur.lam[16 * rt + 4 * g4]);
                    const h8 kb8 = *reinterpret_cast<const h8*>(&cur.kbt[16 * rt + r][8 * g4]);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) S[rt][ct] = mfma16(kb8, d16[ct], S[rt][ct] * lam);
                }
                if (snapping && it.p0 + (c0 + valid - t0) == sc.next) {
                    float* dst = snaps + (sc.row * H + h) * D * D;
                    if (MODE == MODE_CORR) add_state<NCT>(dst, S, ldexpf(1.f, -ex), g4, r, col);
                    else store_state<NCT>(dst, S, ldexpf(1.f, -ex), g4, r, col);
                    sc.next += interval;
                    ++sc.row;
                }
            }
            // The gated epilogue makes interval 2 the longer one for these waves:
            // take max|S| and fp16 S there only without it.
            float msw = 0.f;
            if (GATED && c + 1 >= 0 && c + 1 < nch) msw = state_max();
            __syncthreads();
            if (swork) {
                if (!GATED && STAGE_O) {
                    // o rows of chunk c from the LDS tile: this wave stores tokens
                    // 8 w .. 8 w + 7, two whole rows per 16-byte-per-lane store.
                    // Rows past the end of the sequence fall outside the buffer range.
                    // CORR adds to the o the zero-start pass wrote; MAP has no o.
                    const auto ro = rsrc(o + (c0 * H + h) * D, static_cast<uint32_t>(valid) * rowe * sizeof(Tout));
                    const int el = epi_lane(), c4 = 4 * (el & 31);
#pragma unroll
                    for (int k2 = 0; k2 < (MODE == MODE_MAP ? 0 : 4); ++k2) {
                        const int row = 8 * (w & 3) + 2 * k2 + (el >> 5);
                        const int off = (row * rowe + c4) * static_cast<int>(sizeof(Tout));
                        f4 y = *reinterpret_cast<const f4*>(&sm.otile[row][c4]);
                        if (MODE == MODE_CORR) y += opre[k2];
                        store4(ro, off, y, o);
                    }
                }
                if (GATED) {
                    // y = gate * w * o / sqrt(mean(o^2) + eps) over the token's d_v channels;
                    // two passes over the LDS row keep few values live.
                    const int el = epi_lane(), erow = 8 * (w & 3) + (el >> 3), ecol = 16 * (el & 7);
                    float ss = 0.f;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const f4 x = *reinterpret_cast<const f4*>(&sm.otile[erow][ecol + 4 * j]);
                        ss += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
                    }
                    ss += __shfl_xor(ss, 1);
                    ss += __shfl_xor(ss, 2);
                    ss += __shfl_xor(ss, 4);
                    const float rinv = __builtin_amdgcn_rsqf(ss * (1.f / D) + neps);
                    const auto ro = rsrc(o + (c0 * H + h) * D, static_cast<uint32_t>(valid) * rowe * sizeof(Tout));
                    const int vo = (erow * rowe + ecol) * static_cast<int>(sizeof(Tout));
#pragma unroll
                    for (int j2 = 0; j2 < 2; ++j2) {  // 8 channels per step
                        float gf[8], yv[8];
                        unpack_bf16x8(ogr[j2], gf);
#pragma unroll
                        for (int jj = 0; jj < 2; ++jj) {
                            const int c4 = ecol + 8 * j2 + 4 * jj;
                            const f4 x = *reinterpret_cast<const f4*>(&sm.otile[erow][c4]);
                            const f4 wv = *reinterpret_cast<const f4*>(&sm.nw[c4]);
#pragma unroll
                            for (int e = 0; e < 4; ++e) yv[4 * jj + e] = x[e] * rinv * wv[e] * gf[4 * jj + e];
                        }
                        store8(ro, vo + 8 * j2 * static_cast<int>(sizeof(Tout)), yv, o);
                    }
                }
            }
            if (c + 1 >= 0 && c + 1 < nch) {  // v of chunk c + 1 staged two intervals ago
                if (!PROP) {
                    prepare(nxt, GATED ? msw : state_max());
                } else {
                    // X is dead on this wave once its fp16 copy (at the new exponent)
                    // rounds to zero everywhere: max below 2^-25.
                    const float m0 = state_max();
                    const int e0 = ex;
                    prepare(nxt, m0);
                    if (l == 0) sm.alive[w] = m0 * ldexpf(1.f, ex - e0) >= 0x1p-25f ? 1 : 0;
                }
            }
            __syncthreads();
            if (PROP && c + 1 >= 0 && c + 1 < nch && !(sm.alive[0] | sm.alive[1] | sm.alive[2] | sm.alive[3])) {
                exited = true;
                break;
            }
        }
        // Final state (FULL: sout >= 0 a row of the output, <= -2 a row of the
        // segment-state buffer); MAP: the segment's map, or only its zero flag.
        float* dst = nullptr;
        if (MODE == MODE_FULL && it.sout >= 0 && out_state)
            dst = out_state + (static_cast<int64_t>(it.sout) * H + h) * D * D;
        else if (MODE == MODE_FULL && it.sout <= -2 && it.fin >= 0 && out_state && mflags &&
                 mflags[static_cast<int64_t>(-it.sout - 2) * H + h] == 0)
            dst = out_state + (static_cast<int64_t>(it.fin) * H + h) * D * D;  // final = B (map vanished)
        else if (MODE == MODE_FULL && it.sout <= -2 && bout)
            dst = bout + (static_cast<int64_t>(-it.sout - 2) * H + h) * D * D;
        else if (MODE == MODE_MAP && it.sout >= 0) {
            if (w == 0 && l == 0) mflags[static_cast<int64_t>(it.sout) * H + h] = exited ? 0 : 1;
            if (!exited) dst = out_state + (static_cast<int64_t>(it.sout) * H + h) * D * D;
        }
        if (dst) {
            const float un = ldexpf(1.f, -ex);
#pragma unroll
            for (int rt = 0; rt < 8; ++rt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        dst[(16 * rt + 4 * g4 + i) * D + col + 16 * ct + r] = S[rt][ct][i] * un;
        }
    }


}

// The true initial state of every segment of a sequence cut into segments:
// S_0 = h0 (or zero), S_{j+1} = B_j + M_j S_j, where B_j is segment j's
// final state from a zero start and M_j its state map.  A map the map pass
// found zero in fp16 (or did not compute: M_0 with a zero h0, the last map
// without a final state) has flag 0 and then S_{j+1} = B_j: the correction
// pass reads B_j itself, so only runs of nonzero maps are walked here, one
// segment after the other, and their states staged.  S_0 = h0 is staged for
// the first segment's correction, and the last state is the final state.
// The caller's h0 is read only here, before any final state is written, so
// an in-place final state cannot race.  One workgroup of 4 waves per
// (sequence, head); wave w owns state columns [32 w, 32 w + 32).  The
// 128 x 128 products run on split bf16 MFMA (hi + lo on both operands, three
// products), about 16 significant bits per operand, fp32 accumulation.
constexpr int SCAN_FLAGS = 1024;

__global__ __launch_bounds__(256, 1) void segment_scan_kernel(
    const ScanItem* __restrict__ sitems, int H, const float* __restrict__ h0,
    const float* __restrict__ bst, const float* __restrict__ maps, const int* __restrict__ mflags,
    float* __restrict__ staged, float* __restrict__ final_state, int inplace) {
    const ScanItem it = sitems[blockIdx.x / H];
    if (it.nseg < 2) return;  // whole workgroup: a single segment ran with its own states
    const int h = blockIdx.x % H;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63, r = l & 15, g4 = l >> 4;
    const int col = 32 * w;
    auto row_of = [&](const float* base, int64_t slot) { return base + (slot * H + h) * D * D; };
    auto mrow_of = [&](float* base, int64_t slot) { return base + (slot * H + h) * D * D; };
    f4 S[8][2];
    // A state row block through a buffer resource over one 64 KB state: the
    // lane's part of the offset in a vector register, the element's row and
    // column block in the scalar offset (no 64-bit address per element).
    constexpr uint32_t SB = D * D * sizeof(float);
    const int vo = ((4 * g4) * D + col + r) * 4;
    auto soff = [](int rt, int ct, int i) { return ((16 * rt + i) * D + 16 * ct) * 4; };
    auto load = [&](const float* src) {
        const auto rs = rsrc(src, SB);
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S[rt][ct][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, vo, soff(rt, ct, i), 0));
    };
    auto put = [&](float* dst) {
        const auto rs = rsrc(dst, SB);
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(S[rt][ct][i]), rs, vo, soff(rt, ct, i), 0);
    };
    const float* hsrc = (it.h0 >= 0 && h0) ? h0 + (static_cast<int64_t>(it.h0) * H + h) * D * D : nullptr;
    bool have = false;  // S holds S_j
    if (inplace && hsrc) {  // the final states overwrite h0: stage it for the correction pass
        load(hsrc);
        put(mrow_of(staged, it.first_seg));
        have = true;
    }
    // the map flags of up to SCAN_FLAGS segments at a time, read in parallel
    // (read one after the other, each waited for a full memory round trip)
    __shared__ int fl[SCAN_FLAGS];
    for (int j = 0; j < it.nseg; ++j) {
        const int64_t sj = it.first_seg + j;
        if (j % SCAN_FLAGS == 0) {
            __syncthreads();
            const int nb = it.nseg - j < SCAN_FLAGS ? it.nseg - j : SCAN_FLAGS;
            for (int x = threadIdx.x; x < nb; x += 256) fl[x] = mflags[(sj + x) * H + h];
            __syncthreads();
        }
        const bool last = j + 1 == it.nseg;
        if (last && it.hT < 0) break;  // no final state wanted
        float* dst = last ? final_state + (static_cast<int64_t>(it.hT) * H + h) * D * D : mrow_of(staged, sj + 1);
        // a vanished map (wave-uniform): S_{j+1} = B_j, which the correction
        // pass reads from the segment-state buffer and (unless in place) the
        // full pass already wrote as the final state
        if (fl[j % SCAN_FLAGS] == 0) {
            if (last && inplace) {
                load(row_of(bst, sj));
                put(dst);
            }
            have = false;
            continue;
        }
        if (!have) {
            if (j > 0) {
                load(row_of(bst, sj - 1));  // S_j = B_{j-1}
            } else if (hsrc) {
                load(hsrc);  // S_0 = h0
            } else {
#pragma unroll
                for (int rt = 0; rt < 8; ++rt)
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) S[rt][ct] = f4{0.f, 0.f, 0.f, 0.f};
            }
        }
        const float* bj = row_of(bst, sj);
        const float* mp = row_of(maps, sj);
        // S_{j+1} = B_j + M_j S_j in fp32 MFMA (16x16x4): the K-step (mt, i)
        // takes rows 16 mt + 4 g4 + i of S, i.e. S[mt][ct][i] as it is held,
        // and the A operand the same 4 consecutive columns of M's row, one
        // 16-byte read.
        const auto rb = rsrc(bj, SB), rm = rsrc(mp, SB);
        const int mo = (r * D + 4 * g4) * 4;  // lane part of row 16 rt + r, columns 16 mt + 4 g4 ..
        f4 N[8][2];
#pragma unroll
        for (int rt = 0; rt < 8; ++rt) {
            f4 acc[2];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[ct][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, vo, soff(rt, ct, i), 0));
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) {  // row 16 rt + r of M
                const u4 mw = __builtin_amdgcn_raw_buffer_load_b128(rm, mo, (16 * rt * D + 16 * mt) * 4, 0);
                const f4 am = {__uint_as_float(mw[0]), __uint_as_float(mw[1]), __uint_as_float(mw[2]),
                               __uint_as_float(mw[3])};
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct)
                        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(am[i], S[mt][ct][i], acc[ct], 0, 0, 0);
            }
            N[rt][0] = acc[0];
            N[rt][1] = acc[1];
            __builtin_amdgcn_sched_barrier(0);  // one row block's loads in flight at a time
        }
#pragma unroll
        for (int rt = 0; rt < 8; ++rt) {
            S[rt][0] = N[rt][0];
            S[rt][1] = N[rt][1];
        }
        put(dst);
        have = true;
    }
}

// Longest-sequence-first order of the N sequences (ties by index): the
// dispatcher hands workgroups out in index order, so launching long chains
// first gives a longest-processing-time schedule.  One item per sequence.
__global__ void plan_sequences_kernel(const int32_t* __restrict__ cu, int N, int T, int lpt,
                                      int has_h0, int has_hT, const int32_t* __restrict__ snap_base,
                                      ChunkItem* __restrict__ items) {
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N) return;
    const int64_t a = cu ? cu[n] : static_cast<int64_t>(n) * T;
    const int64_t b = cu ? cu[n + 1] : a + T;
    int rank = n;
    if (lpt) {
        const int len = static_cast<int>(b - a);
        rank = 0;
        for (int m = 0; m < N; ++m) {
            const int lm = cu[m + 1] - cu[m];
            rank += (lm > len) || (lm == len && m < n);
        }
    }
    items[rank] = ChunkItem{a, b, has_h0 ? n : -1, has_hT ? n : -1, 0, snap_base ? snap_base[n] : -1, -1};
}

// Work items of the segmented path.  Each sequence is cut into segments of
// seg tokens (the last one shorter); a sequence with a single segment runs as
// one FULL item with its own initial and final states.  For the others,
// segment j (state slot z, numbered over the split sequences only) gets: a
// FULL item from a zero state writing its final state to row z of the
// segment-state buffer (sout = -2 - z), or, for the last segment, to the
// final state when its map vanished (fin); a MAP item (sout = z) when its
// map is needed (j > 0 or h0 given; j < last or a final state wanted), else
// an empty one (no tokens, sout = -1); a CORR item when the segment's
// initial state can be nonzero (j > 0 or h0 given) -- from h0 for j = 0,
// else from staged state z (sin = -2 - z) -- else an empty one.  Items are
// numbered over all segments; one scan item per sequence.
//
// A single workgroup walks the sequences in blocks of 256: a block scan of
// the segment counts places every sequence's items, then the segments are
// written one per thread, sequence after sequence.
__device__ __forceinline__ void write_segment(int j, int G, int64_t a, int64_t b, int seg, int si, int zi,
                                              int h0row, int hTrow, int snap, int H, int has_h0,
                                              int has_hT, int inplace, ChunkItem* __restrict__ full_items,
                                              ChunkItem* __restrict__ map_items,
                                              ChunkItem* __restrict__ corr_items, int* __restrict__ mflags) {
    const int64_t sa = a + static_cast<int64_t>(j) * seg;
    const int64_t sb = sa + seg < b ? sa + seg : b;
    if (G == 1) {
        full_items[si] = ChunkItem{sa, sb, h0row, hTrow, 0, snap, -1};
        map_items[si] = ChunkItem{sa, sa, -1, -1, 0, -1, -1};
        corr_items[si] = ChunkItem{sa, sa, -1, -1, 0, -1, -1};
        return;
    }
    const bool live_in = j > 0 || has_h0;
    const bool lastj = j + 1 == G;
    for (int hh = 0; hh < H; ++hh) mflags[static_cast<int64_t>(zi) * H + hh] = 0;  // set by the map pass
    // in place (the final states overwrite h0): h0 is read from its staged
    // copy and every final state is written by the scan, after that copy
    full_items[si] = ChunkItem{sa, sb, -1, -2 - zi, sa - a, snap, (lastj && !inplace) ? hTrow : -1};
    map_items[si] = (live_in && (!lastj || has_hT)) ? ChunkItem{sa, sb, -1, zi, sa - a, -1, -1}
                                                    : ChunkItem{sa, sa, -1, -1, sa - a, -1, -1};
    corr_items[si] = live_in ? ChunkItem{sa, sb, (j == 0 && !inplace) ? h0row : -2 - zi, -1, sa - a, snap, -1}
                             : ChunkItem{sa, sa, -1, -1, sa - a, -1, -1};
}

__global__ __launch_bounds__(256) void plan_segments_kernel(
    const int32_t* __restrict__ cu, int N, int T, int seg, int has_h0, int has_hT, int inplace,
    const int32_t* __restrict__ snap_base, ChunkItem* __restrict__ full_items,
    ChunkItem* __restrict__ map_items, ChunkItem* __restrict__ corr_items,
    ScanItem* __restrict__ scan_items, int H, int* __restrict__ mflags) {
    __shared__ int sc[256], sc2[256], gs[256];
    __shared__ int64_t sa_[256], sb_[256];
    __shared__ int base, base2;
    if (threadIdx.x == 0) base = base2 = 0;
    __syncthreads();
    for (int n0 = 0; n0 < N; n0 += 256) {
        const int n = n0 + threadIdx.x;
        int64_t a = 0, b = 0;
        int G = 0;
        if (n < N) {
            a = cu ? cu[n] : static_cast<int64_t>(n) * T;
            b = cu ? cu[n + 1] : a + T;
            const int64_t len = b - a;
            G = len > 0 ? static_cast<int>((len + seg - 1) / seg) : 1;
        }
        const int Gs = G > 1 ? G : 0;  // state slots (split sequences only)
        sc[threadIdx.x] = G;
        sc2[threadIdx.x] = Gs;
        gs[threadIdx.x] = G;
        sa_[threadIdx.x] = a;
        sb_[threadIdx.x] = b;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {  // inclusive scans of G and Gs
            const int x = threadIdx.x >= off ? sc[threadIdx.x - off] : 0;
            const int y = threadIdx.x >= off ? sc2[threadIdx.x - off] : 0;
            __syncthreads();
            sc[threadIdx.x] += x;
            sc2[threadIdx.x] += y;
            __syncthreads();
        }
        if (n < N)
            scan_items[n] = ScanItem{base2 + sc2[threadIdx.x] - Gs, G, has_h0 ? n : -1, has_hT ? n : -1};
        const int nb = N - n0 < 256 ? N - n0 : 256;
        for (int m = 0; m < nb; ++m) {  // sequence n0 + m: its segments over the threads
            const int Gm = gs[m];
            const int s0 = base + sc[m] - Gm, z0 = base2 + sc2[m] - (Gm > 1 ? Gm : 0);
            const int nm = n0 + m;
            for (int j = threadIdx.x; j < Gm; j += 256)
                write_segment(j, Gm, sa_[m], sb_[m], seg, s0 + j, z0 + j, has_h0 ? nm : -1,
                              has_hT ? nm : -1, snap_base ? snap_base[nm] : -1, H, has_h0, has_hT,
                              inplace, full_items, map_items, corr_items, mflags);
        }
        __syncthreads();
        if (threadIdx.x == 255) {
            base += sc[255];
            base2 += sc2[255];
        }
        __syncthreads();
    }
}

}  // namespace chunkk

namespace {

constexpr int kLptMaxSeqs = 16384;
constexpr int kWpc = 1;  // full-mode chains resident per CU (LDS bound)

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Row of every sequence's first snapshot: an exclusive prefix sum of
// floor(length / interval) over the sequences, one workgroup in blocks of 256.
__global__ __launch_bounds__(256) void snap_base_kernel(const int32_t* __restrict__ cu, int N, int T,
                                                        int interval, int32_t* __restrict__ base_out) {
    __shared__ int sc[256];
    __shared__ int base;
    if (threadIdx.x == 0) base = 0;
    __syncthreads();
    for (int n0 = 0; n0 < N; n0 += 256) {
        const int n = n0 + threadIdx.x;
        int cnt = 0;
        if (n < N) {
            const int64_t len = cu ? cu[n + 1] - cu[n] : T;
            cnt = static_cast<int>(len / interval);
        }
        sc[threadIdx.x] = cnt;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {  // inclusive scan
            const int x = threadIdx.x >= off ? sc[threadIdx.x - off] : 0;
            __syncthreads();
            sc[threadIdx.x] += x;
            __syncthreads();
        }
        if (n < N) base_out[n] = base + sc[threadIdx.x] - cnt;
        __syncthreads();
        if (threadIdx.x == 255) base += sc[255];
        __syncthreads();
    }
}

// Host mirror of the segment plan (same formulas as plan_segments_kernel):
// items (all segments), state slots (segments of split sequences) and the
// number of split sequences.
struct SegCount {
    int64_t nseg, nslot, nsplit;
};
SegCount count_segments(const int32_t* cu_host, int N, int T, int seg) {
    SegCount c{0, 0, 0};
    for (int n = 0; n < N; ++n) {
        const int64_t len = cu_host ? cu_host[n + 1] - cu_host[n] : T;
        const int64_t G = len > 0 ? (len + seg - 1) / seg : 1;
        c.nseg += G;
        if (G > 1) {
            c.nslot += G;
            ++c.nsplit;
        }
    }
    return c;
}

struct ScanLayout {
    size_t full_items, map_items, corr_items, scan_items, flags, bst, maps, staged, total;
};

ScanLayout scan_layout(const SegCount& c, int N, int H) {
    ScanLayout L{};
    const size_t state = static_cast<size_t>(c.nslot) * H * chunkk::D * chunkk::D * sizeof(float);
    size_t off = 0;
    auto take = [&](size_t& at, size_t bytes) {
        at = off;
        off = align256(off + bytes);
    };
    take(L.full_items, c.nseg * sizeof(ChunkItem));
    take(L.map_items, c.nseg * sizeof(ChunkItem));
    take(L.corr_items, c.nseg * sizeof(ChunkItem));
    take(L.scan_items, static_cast<size_t>(N) * sizeof(ScanItem));
    take(L.flags, static_cast<size_t>(c.nslot) * H * sizeof(int));
    take(L.bst, state);
    take(L.maps, state);
    take(L.staged, state);
    L.total = off;
    return L;
}

}  // namespace

int chunk_chains_per_cu() { return kWpc; }

hipError_t launch_plan_sequences(const PrefillArgs& a, ChunkItem* items) {
    const int lpt = (a.cu && a.N > 1 && a.N <= kLptMaxSeqs) ? 1 : 0;
    hipLaunchKernelGGL(chunkk::plan_sequences_kernel, dim3((a.N + 255) / 256), dim3(256), 0, a.stream, a.cu, a.N, a.T,
                       lpt, a.h0 ? 1 : 0, a.hT ? 1 : 0, a.snap_base, items);
    return hipGetLastError();
}

hipError_t launch_snap_base(const int32_t* cu, int N, int T, int interval, int32_t* out,
                            hipStream_t stream) {
    hipLaunchKernelGGL(snap_base_kernel, dim3(1), dim3(256), 0, stream, cu, N, T, interval, out);
    return hipGetLastError();
}

#ifndef MIN_SEG64
#define MIN_SEG64 4
#endif
constexpr int kMinSegChunks64 = MIN_SEG64;  // shortest segment, in 64-token units

int chunk_segment_tokens(int B, int T, int H, int N, const int32_t* cu_host) {
    // Long sequences are cut so that four segments (workgroups) per CU of a
    // 256-CU part exist over all heads: a whole number of rounds of resident
    // workgroups.  Segments are a whole number of chunks.
    (void)B;
    int64_t total = 0;
    for (int n = 0; n < N; ++n) total += cu_host ? cu_host[n + 1] - cu_host[n] : T;
    int64_t target_items = 4 * 256 / (H > 0 ? H : 1);
    if (target_items < 1) target_items = 1;
    int64_t seg = (total + target_items - 1) / target_items;
    seg = (seg + chunkk::CSEG - 1) / chunkk::CSEG * chunkk::CSEG;
    if (seg < kMinSegChunks64 * chunkk::CSEG) seg = kMinSegChunks64 * chunkk::CSEG;
    return static_cast<int>(seg > (1 << 30) ? (1 << 30) : seg);
}

size_t chunk_workspace_bytes(int B, int T, int H, int N, const int32_t* cu_host, bool scan) {
    if (!scan) return align256(static_cast<size_t>(N) * sizeof(ChunkItem));
    const int seg = chunk_segment_tokens(B, T, H, N, cu_host);
    return scan_layout(count_segments(cu_host, N, T, seg), N, H).total;
}

hipError_t launch_chunk(const PrefillArgs& a, bool scan, bool c64) {
    using namespace chunkk;
    char* ws = static_cast<char*>(a.ws);
    // FULL items (mode 0), or the MAP (1) / CORR (2) propagation passes of the
    // segmented path; bout and mflags are the segment-state buffer and the
    // map flags.  fuse_gate: apply the gated RMSNorm in the o store.
    auto launch_full = [&](const ChunkItem* items, int64_t nitems, const float* staged, int mode = 0,
                           float* out_state = nullptr, float* bout = nullptr, int* mflags = nullptr,
                           bool fuse_gate = true) {
        const dim3 grid(static_cast<uint32_t>(nitems * a.H));
        const auto q = static_cast<const uint16_t*>(a.q);
        const auto k = static_cast<const uint16_t*>(a.k);
        const auto v = static_cast<const uint16_t*>(a.v);
        bf16_t* ob = static_cast<bf16_t*>(a.o);
        float* of = static_cast<float*>(a.o);
        const bool sn = a.snaps != nullptr;
        if (c64) {  // single-role kernel, 64-token chunks (a gated output is applied afterwards)
            auto go = [&](auto kernel, auto* o) {
                hipLaunchKernelGGL(kernel, grid, dim3(8 * 64), 0, a.stream, q, k, v, a.g, a.beta, a.scale,
                                   items, a.H, a.h0, staged, o, a.hT, a.snaps, a.snap_interval);
            };
            if (a.out_bf16)
                sn ? go(chunk_kernel<8, 4, 1, 1, bf16_t, true>, ob)
                   : go(chunk_kernel<8, 4, 1, 1, bf16_t, false>, ob);
            else
                sn ? go(chunk_kernel<8, 4, 1, 1, float, true>, of)
                   : go(chunk_kernel<8, 4, 1, 1, float, false>, of);
            return;
        }
        auto go = [&](auto kernel, auto* o) {
            hipLaunchKernelGGL(kernel, grid, dim3(ws::NW * 64), 0, a.stream, q, k, v, a.g, a.beta, a.scale,
                               items, a.H, a.h0, staged, o, mode == MODE_MAP ? out_state : a.hT,
                               a.snaps, a.snap_interval, static_cast<const uint16_t*>(a.ogate), a.nweight,
                               a.neps, bout, mflags);
        };
        if (mode == MODE_MAP) {
            go(chunk_ws_kernel<float, false, false, MODE_MAP>, of);
            return;
        }
        if (mode == MODE_CORR) {
            if (a.out_bf16) sn ? go(chunk_ws_kernel<bf16_t, true, false, MODE_CORR>, ob)
                               : go(chunk_ws_kernel<bf16_t, false, false, MODE_CORR>, ob);
            else sn ? go(chunk_ws_kernel<float, true, false, MODE_CORR>, of)
                    : go(chunk_ws_kernel<float, false, false, MODE_CORR>, of);
            return;
        }
        const bool gt = a.ogate != nullptr && fuse_gate;
        if (a.out_bf16) {
            if (gt) go(chunk_ws_kernel<bf16_t, false, true>, ob);
            else if (sn) go(chunk_ws_kernel<bf16_t, true, false>, ob);
            else go(chunk_ws_kernel<bf16_t, false, false>, ob);
        } else {
            if (gt) go(chunk_ws_kernel<float, false, true>, of);
            else if (sn) go(chunk_ws_kernel<float, true, false>, of);
            else go(chunk_ws_kernel<float, false, false>, of);
        }
    };
    if (!scan) {
        ChunkItem* items = reinterpret_cast<ChunkItem*>(ws);
        const hipError_t e = launch_plan_sequences(a, items);
        if (e != hipSuccess) return e;
        launch_full(items, a.N, nullptr);
        return hipGetLastError();
    }
    // Segmented path: maps (stopping where they vanish), every segment from a
    // zero state, the scan of the true segment states, then the corrections
    // from those states (stopping where they vanish).
    const int seg = chunk_segment_tokens(a.B, a.T, a.H, a.N, a.cu_host);
    const SegCount cnt = count_segments(a.cu_host, a.N, a.T, seg);
    const ScanLayout L = scan_layout(cnt, a.N, a.H);
    ChunkItem* full_items = reinterpret_cast<ChunkItem*>(ws + L.full_items);
    ChunkItem* map_items = reinterpret_cast<ChunkItem*>(ws + L.map_items);
    ChunkItem* corr_items = reinterpret_cast<ChunkItem*>(ws + L.corr_items);
    ScanItem* scan_items = reinterpret_cast<ScanItem*>(ws + L.scan_items);
    int* mflags = reinterpret_cast<int*>(ws + L.flags);
    float* bst = reinterpret_cast<float*>(ws + L.bst);
    float* maps = reinterpret_cast<float*>(ws + L.maps);
    float* staged = reinterpret_cast<float*>(ws + L.staged);
    // final states written over the initial ones (the same or overlapping rows)
    const size_t sbytes = static_cast<size_t>(a.N) * a.H * D * D * sizeof(float);
    const bool inplace = a.h0 && a.hT &&
                         reinterpret_cast<const char*>(a.h0) < reinterpret_cast<const char*>(a.hT) + sbytes &&
                         reinterpret_cast<const char*>(a.hT) < reinterpret_cast<const char*>(a.h0) + sbytes;
    hipLaunchKernelGGL(plan_segments_kernel, dim3(1), dim3(256), 0, a.stream, a.cu, a.N, a.T, seg,
                       a.h0 ? 1 : 0, a.hT ? 1 : 0, inplace ? 1 : 0, a.snap_base, full_items, map_items,
                       corr_items, scan_items, a.H, mflags);
    const bool split = cnt.nsplit > 0;
    if (split) launch_full(map_items, cnt.nseg, nullptr, MODE_MAP, maps, nullptr, mflags);
    launch_full(full_items, cnt.nseg, nullptr, MODE_FULL, nullptr, bst, mflags, !split);
    if (split) {
        hipLaunchKernelGGL(segment_scan_kernel, dim3(static_cast<uint32_t>(a.N) * a.H), dim3(256), 0,
                           a.stream, scan_items, a.H, a.h0, bst, maps, mflags, staged, a.hT, inplace ? 1 : 0);
        launch_full(corr_items, cnt.nseg, staged, MODE_CORR, nullptr, bst, mflags);
        // the gated RMSNorm needs the corrected read-out: applied in place after
        if (a.ogate) {
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            return launch_gate_norm(a);
        }
    }
    return hipGetLastError();
}

}  // namespace kda
