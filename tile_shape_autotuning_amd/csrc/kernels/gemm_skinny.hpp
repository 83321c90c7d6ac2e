// Skinny-M GEMM for decode-like shapes (M <= 64), bf16 inputs:
//     C = act(A . B + bias),  A [M][K] (activations), B [K][N] (weights).
//
// With a handful of rows there is no reuse of B to capture: every weight is
// read once and the kernel is bound by HBM bandwidth by construction (page
// "Tiling the hierarchy", failure regimes: matrix-vector shapes move
// Theta(N^2) bytes whatever the capacity; page "Compilers and Kernel
// Languages": at 16 tokens every tile ties at the floor set by reading the
// weights).  The design therefore streams B exactly once with many 16-byte
// loads in flight and keeps everything else off the critical path:
//
//   * a workgroup owns a 128-column slice of C and a K range; its W waves
//     take interleaved 32-row chunks of that range (adjacent waves read
//     adjacent rows);
//   * per chunk, a lane loads 8 rows x 8 columns of B (eight 16-byte loads;
//     16 lanes cover 128 columns, 4 lane groups cover 32 rows), transposes
//     the 8x8 block in registers and feeds 8 v_mfma_f32_16x16x32_bf16 whose
//     columns are strided by 8; the A fragment (16 rows x 32 k) is shared by
//     all 8 and comes from L2;
//   * U chunks are issued per step and the next step's loads are issued
//     before the current step's MFMAs (software pipelining);
//   * B is read once by the whole grid, so its loads carry the non-temporal
//     policy (7 % faster on the 16 x 28672 x 8192 decode); A, which every
//     workgroup re-reads, keeps the default one;
//   * the W per-wave partials are summed through LDS; wave 0 runs the
//     bias/activation epilogue and writes 8 consecutive outputs per lane (with
//     split-K, run-time `split` workgroups per slice, it writes raw fp32 sums
//     to the split's workspace slab instead, for the second pass).
#pragma once

#include "common.hpp"

namespace tg {

template <int MT, int W, int U>
struct Skinny {
    static constexpr int T = 64 * W;
    static constexpr int BM = 16 * MT;
    static constexpr int BN = 128;
    static constexpr int RED_BYTES = W > 1 ? W * MT * 8 * 64 * 16 : 16;
    static_assert(MT >= 1 && MT <= 4, "M tiles");
    static_assert(W == 1 || W == 2 || W == 4 || W == 8, "waves");
    static_assert(U == 1 || U == 2 || U == 4, "chunks per step");
};

template <int MT, int W, int U>
__global__ void __launch_bounds__(64 * W)
gemm_skinny_kernel(GemmParams p)
{
    using Cf = Skinny<MT, W, U>;
    constexpr int T = Cf::T;
    __shared__ f32x4_t red[Cf::RED_BYTES / 16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave: scalar registers
    const int l16 = lane & 15, g = lane >> 4;

    int tile, tm, tn, split;
    map_block(blockIdx.x, gridDim.x, 1, p.tiles_n, 1, tile, tm, tn, split);
    const int M = p.M, N = p.N, K = p.K;
    const int n0 = tn * 128;
    const int kbeg = split * p.kps;
    const int kend = min(K, kbeg + p.kps);
    const int nchunks = kend > kbeg ? (kend - kbeg + 31) / 32 : 0;
    // chunks of this wave: wave, wave + W, ...; U per step
    const int my_chunks = nchunks > wave ? (nchunks - wave + W - 1) / W : 0;
    const int nsteps = (my_chunks + U - 1) / U;

    const char* Ab = static_cast<const char*>(p.A);
    const char* Bb = static_cast<const char*>(p.B);
    const int64_t a_total_bytes = (int64_t)M * K * 2;
    const int64_t b_total = (int64_t)K * N;
    const bool col_ok = n0 + l16 * 8 < N;

    // A rows are addressed from A + kbeg
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(Ab + (int64_t)kbeg * 2, a_total_bytes - (int64_t)kbeg * 2);

    f32x4_t acc[MT][8];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < 8; ++t)
            acc[m][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t bufB[2][U][8];
    u32x4_t bufA[2][U][MT];

    auto issue = [&](int step, int slot) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int ci = step * U + u;                  // index among this wave's chunks
            const int q = wave + ci * W;                  // chunk index in the K range
            const bool cv = ci < my_chunks;
            const int krel = q * 32;                      // first row of the chunk, relative to kbeg
            const int64_t b_off = ((int64_t)(kbeg + krel)) * N + n0;
            const __amdgpu_buffer_rsrc_t rB =
                make_rsrc(Bb + b_off * 2, cv ? (b_total - b_off) * 2 : 0);
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int kr = g * 8 + r;
                const bool v = cv && col_ok && (kbeg + krel + kr < kend);
                bufB[slot][u][r] = load16_stream(rB, v ? kr * N * 2 + l16 * 16 : kOOB);
            }
            const int kk = krel + g * 8;
            const bool kv = cv && (kbeg + kk < kend);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const int row = m * 16 + l16;
                const bool v = kv && row < M;
                bufA[slot][u][m] = load16(rA, v ? row * K * 2 + kk * 2 : kOOB);
            }
        }
    };

    auto consume = [&](int slot) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            u32x4_t tr[8];
            transpose8x8_b16(bufB[slot][u], tr);
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    acc[m][t] = mfma_bf16(bufA[slot][u][m], tr[t], acc[m][t]);
        }
    };

    if (nsteps > 0)
        issue(0, 0);
    int s = 0;
    for (; s + 1 < nsteps; s += 2) {
        issue(s + 1, 1);
        consume(0);
        if (s + 2 < nsteps)
            issue(s + 2, 0);
        consume(1);
    }
    if (s < nsteps)
        consume(0);

    // ---- sum the W per-wave partials (fixed wave order)
    if constexpr (W > 1) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int t = 0; t < 8; ++t)
                red[((wave * MT + m) * 8 + t) * 64 + lane] = acc[m][t];
        __syncthreads();
        if (wave != 0)
            return;
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int t = 0; t < 8; ++t)
                acc[m][t] = red[((0 * MT + m) * 8 + t) * 64 + lane];
        // one wave's partials at a time (unrolled, the compiler would load
        // all of them before the first add and spill)
#pragma unroll 1
        for (int w = 1; w < W; ++w)
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    acc[m][t] += red[((w * MT + m) * 8 + t) * 64 + lane];
    }
    // from here on only wave 0 is active

    const OutSpec out = out_spec(p, split);

    // ---- epilogue: lane owns rows 16m + 4g + r, columns n0 + 8*l16 + t (t = 0..7)
    if (!col_ok)
        return;
    const int col0 = n0 + l16 * 8;
    float bv[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
        bv[t] = out.bias ? out.bias[col0 + t] : 0.0f;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = m * 16 + g * 4 + r;
            if (row >= M)
                continue;
            float v[8];
#pragma unroll
            for (int t = 0; t < 8; ++t)
                v[t] = apply_act(acc[m][t][r] + bv[t], out.act);
            const int64_t idx = (int64_t)row * N + col0;
            if (out.bf16) {
                u32x4_t o;
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    o[d] = (unsigned)f32_to_bf16_rne(v[2 * d]) | ((unsigned)f32_to_bf16_rne(v[2 * d + 1]) << 16);
                *reinterpret_cast<u32x4_t*>(static_cast<unsigned short*>(out.dst) + idx) = o;
            } else {
                f32x4_t* dst = reinterpret_cast<f32x4_t*>(static_cast<float*>(out.dst) + idx);
                dst[0] = f32x4_t{v[0], v[1], v[2], v[3]};
                dst[1] = f32x4_t{v[4], v[5], v[6], v[7]};
            }
        }
    }
}

}  // namespace tg
