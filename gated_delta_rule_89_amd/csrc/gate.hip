// Fused gate computation: the forget gate's low-rank up-projection with its
// activation, and the update gate's sigmoid ("kimi delta attn from first
// principles", section "three gates": alpha comes from a low-rank projection,
// a down projection to rank r followed by an up projection to the key
// channels; beta is a sigmoid of its projection).
//
//   g[m, h, c]  = -softplus(sum_j z[m, j] W[h d_k + c, j] + b[h d_k + c])   (log alpha <= 0)
//   beta[m, h]  = 1 / (1 + exp(-u[m, h]))
//
// W is [H d_k, r] (a linear layer's weight, output rows): every MFMA operand
// fragment, 8 consecutive j of one row of z or of W, is one 16-byte read.
// The up-projection is a dense contraction (M x r by r x H d_k), so it runs
// on bf16 MFMA (16x16x32, fp32 accumulation), computed transposed (W as the
// A operand, z as B) so that each lane ends with 4 consecutive channels of
// one token: the g tile is written with 16-byte stores.  The write of g
// (4 bytes per element) dominates the traffic: the kernel is bound by HBM
// writes.
#include "dev_common.h"
#include "kda_internal.h"

namespace kda {
namespace gatek {

typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int ROWS = 32;   // rows of z per wave
constexpr int DK = 128;    // key channels per head

__device__ __forceinline__ float neg_softplus(float x) {
    // -(max(x, 0) + log(1 + exp(-|x|))), in base 2 with the hardware exp2/log2
    constexpr float LOG2E = 1.4426950408889634f, LN2 = 0.6931471805599453f;
    const float t = __builtin_amdgcn_exp2f(-fabsf(x) * LOG2E);
    return -(fmaxf(x, 0.f) + __builtin_amdgcn_logf(1.f + t) * LN2);
}

// A workgroup takes one head and NB blocks of 4 x 32 rows of z (one 32-row
// block per wave and step): the head's W rows (DK x R bf16) are read from L2
// once into LDS, where every wave takes its MFMA fragments for all NB row
// blocks.  (One wave per 32 rows reading W from L2 moved twice the bytes of
// the g tile it writes, and the loads, not the stores, stalled the kernel.)
// The z fragments come straight from global memory: rows of z are
// contiguous along j, every fragment is one 16-byte read.  16-byte chunk cc
// of W row r sits at chunk cc ^ (r & (R / 8 - 1)) (at most 16 chunks apart),
// so the 16 rows one fragment read touches fall in different banks.  The k
// loop stays rolled (unrolled, the compiler keeps every fragment in flight
// and occupancy drops).
constexpr int NB = 16;  // row blocks per workgroup

template <int R>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(R == 256 ? 2 : 4))) void fused_gate_kernel(
    const uint16_t* __restrict__ z, const uint16_t* __restrict__ w, const float* __restrict__ bias,
    const float* __restrict__ u, int64_t M, int H, float* __restrict__ g, float* __restrict__ beta) {
    constexpr int RT = ROWS / 16;
    constexpr int CPR = R / 8;                      // 16-byte chunks per W row
    constexpr int SW = CPR < 16 ? CPR - 1 : 15;     // swizzle mask
    __shared__ u4 wl[DK * CPR];
    __shared__ __align__(16) float bl[DK];  // the head's bias (zeros without one)
    const int tid = threadIdx.x, l = tid & 63, r16 = l & 15, g4 = l >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the z buffer base is scalar
    const int h = blockIdx.y;
    const int64_t N = static_cast<int64_t>(H) * DK;
    {
        const u4* wh = reinterpret_cast<const u4*>(w + static_cast<int64_t>(h) * DK * R);
#pragma unroll
        for (int j = 0; j < DK * CPR / 256; ++j) {
            const int ci = tid + 256 * j, row = ci / CPR, cc = ci % CPR;
            wl[row * CPR + (cc ^ (row & SW))] = wh[ci];
        }
        if (tid < DK) bl[tid] = bias ? bias[h * DK + tid] : 0.f;
    }
    __syncthreads();
    const bool lo = r16 < 8;
#pragma unroll 1
    for (int nb = 0; nb < NB; ++nb) {
        const int64_t m0 = (static_cast<int64_t>(blockIdx.x) * NB + nb) * (4 * ROWS) + wave * ROWS;
        if (m0 >= M) break;  // whole wave; no barrier follows
        if (h == 0) {  // beta of these rows, once per row block
            for (int e = l; e < ROWS * H; e += 64) {
                const int64_t idx = m0 * H + e;
                if (idx < M * H) beta[idx] = 1.f / (1.f + __builtin_amdgcn_exp2f(-u[idx] * 1.4426950408889634f));
            }
        }
        f4 acc[RT][DK / 16];
        // this wave's rows of z and of g through range-checked buffers: rows past
        // M read zeros and their stores are dropped
        const int64_t rows = M - m0 < ROWS ? M - m0 : ROWS;
        const auto rz = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(z + m0 * R), 0,
                                                          static_cast<int>(rows * R * 2), 0x00020000);
        const auto rg = __builtin_amdgcn_make_buffer_rsrc(g + m0 * N + h * DK, 0,
                                                          static_cast<int>(((rows - 1) * N + DK) * 4), 0x00020000);
        // k-step ks; with first, the MFMA takes a zero accumulator operand
        auto kstep = [&](int ks, bool first) {
            b8 zf[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                zf[rt] = __builtin_bit_cast(
                    b8, __builtin_amdgcn_raw_buffer_load_b128(rz, ((16 * rt + r16) * R + 32 * ks + 8 * g4) * 2, 0, 0));
#pragma unroll
            for (int ct = 0; ct < DK / 16; ++ct) {
                const int row = 16 * ct + r16, cc = 4 * ks + g4;
                const b8 wf = __builtin_bit_cast(b8, wl[row * CPR + (cc ^ (row & SW))]);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        wf, zf[rt], first ? f4{0.f, 0.f, 0.f, 0.f} : acc[rt][ct], 0, 0, 0);
            }
        };
        if constexpr (R >= 128) {  // (at lower ranks the peeled step costs registers)
            kstep(0, true);
#pragma unroll 1
            for (int ks = 1; ks < R / 32; ++ks) kstep(ks, false);
        } else {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < DK / 16; ++ct) acc[rt][ct] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
            for (int ks = 0; ks < R / 32; ++ks) kstep(ks, false);
        }
        // D layout of the transposed product: lane holds rows 4 g4 + i
        // (channels) of column r16 (token) of each 16 x 16 tile, so one tile
        // covers 64 bytes of a token's g row.  Tiles 2j and 2j + 1 together
        // cover 128 contiguous bytes (a whole cache line) per token: the
        // second tile's values are rotated by 8 lanes inside each 16-lane row
        // (DPP), and each store then writes whole lines of 8 tokens -- lanes
        // r16 < 8 tile 2j of token r16 and lanes r16 >= 8 tile 2j + 1 of token
        // r16 - 8, or the other 8 tokens -- instead of half lines of 16 tokens.
#pragma unroll
        for (int cp = 0; cp < DK / 32; ++cp) {
            const int ca = 32 * cp + 4 * g4, cb = ca + 16;
            const f4 ba = *reinterpret_cast<const f4*>(&bl[ca]);
            const f4 bb = *reinterpret_cast<const f4*>(&bl[cb]);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                f4 ya, yb;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ya[i] = neg_softplus(acc[rt][2 * cp][i] + ba[i]);
                    const float b = neg_softplus(acc[rt][2 * cp + 1][i] + bb[i]);
                    yb[i] = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(b), 0x128, 0xf, 0xf, true));
                }
                f4 x, y;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[i] = lo ? ya[i] : yb[i];
                    y[i] = lo ? yb[i] : ya[i];
                }
                const int t7 = r16 & 7;
                const int tx = 16 * rt + t7, ty = tx + 8;  // rows of the block
                const int cx = lo ? ca : cb, cy = lo ? cb : ca;
                // non-temporal (cache policy nt), rows past M dropped by the range check
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, x), rg, (tx * static_cast<int>(N) + cx) * 4, 0, 2);
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, y), rg, (ty * static_cast<int>(N) + cy) * 4, 0, 2);
            }
        }
    }
}

}  // namespace gatek

hipError_t launch_fused_gate(const void* z, const void* w, const float* bias, const float* u,
                             int64_t M, int r, int H, float* g, float* beta, hipStream_t stream) {
    using namespace gatek;
    const dim3 grid(static_cast<uint32_t>((M + 4 * ROWS * NB - 1) / (4 * ROWS * NB)), static_cast<uint32_t>(H));
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(z),
                           static_cast<const uint16_t*>(w), bias, u, M, H, g, beta);
    };
    switch (r) {
        case 32: go(fused_gate_kernel<32>); break;
        case 64: go(fused_gate_kernel<64>); break;
        case 128: go(fused_gate_kernel<128>); break;
        case 256: go(fused_gate_kernel<256>); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kda
