// Block-tiled GEMM with a fused bias + activation epilogue, loading every
// element on its own: the kernel of the unaligned kind, for pointers or
// shapes (N, K) that are not 16-byte aligned (aligned shapes run the
// direct-to-LDS kernel of gemm_tiled_dma.hpp).
//     C = act(A . B + bias),  A [M][K], B [K][N], C [M][N] row-major.
//
// The decomposition is the one the page "Tile Selection: Cost Models Against
// Measurement" describes in "The structure of the search space": each
// workgroup owns a BM x BN output tile and walks K in steps of BK, staging a
// [BM x BK] panel of A and a [BK x BN] panel of B in on-chip memory; the free
// parameters are the block tile, the reduction step and the per-wave tile
// (WGM x WGN waves, each owning (BM/WGM) x (BN/WGN) outputs).  ST is the LDS
// pipeline depth: 1 = one panel buffer, 2 = double buffering, where the loads
// of step t+1 are in flight while the matrix cores work on step t (page
// "Tiling the hierarchy", double-buffering section).  Split-K (a run-time
// value) gives each of `split` workgroups a contiguous K range; each writes
// its fp32 sums to its split's workspace slab and a second kernel adds the
// slabs in split order and runs the epilogue (deterministic results).
//
// gfx950 specifics:
//   * global loads are 2- or 4-byte buffer loads, one per element
//     (out-of-range lanes read zero, so M, N and K edges need no branches);
//   * bf16: A is kept K-contiguous in LDS; B is transposed in registers (8x8
//     blocks of 16-bit values) on its way to LDS so that both MFMA operands
//     are read with one ds_read_b128 each; 16-byte chunks are XOR-swizzled;
//   * fp32: A as above, B kept N-contiguous with a 4-float row pad; operands
//     feed v_mfma_f32_16x16x4_f32;
//   * accumulation is fp32 on MFMA 16x16 tiles; the epilogue adds the bias,
//     applies ReLU or GELU (erf form) and stores fp32 or bf16 (round to
//     nearest even).
#pragma once

#include "common.hpp"

namespace tg {

template <bool BF, int BM, int BN, int BK, int WGM, int WGN, int ST>
struct Tiled {
    static constexpr int W = WGM * WGN;
    static constexpr int T = 64 * W;
    static constexpr int WM = BM / WGM, WN = BN / WGN;
    static constexpr int FM = WM / 16, FN = WN / 16;
    static constexpr int EB = BF ? 2 : 4;        // bytes per input element
    static constexpr int EPC = 16 / EB;          // elements per 16-byte chunk
    static constexpr int CPR = BK / EPC;         // chunks per K-contiguous LDS row
    static constexpr int KSTEP = BF ? 32 : 16;   // K consumed per fragment step
    static constexpr int A_CH = BM * CPR;        // 16-byte chunks in an A panel
    static constexpr int A_PT = (A_CH + T - 1) / T;
    static constexpr int B_UNITS = BF ? (BK / 8) * (BN / 8) : BK * (BN / 4);
    static constexpr int B_PT = (B_UNITS + T - 1) / T;
    static constexpr int BNP = BN + 4;           // fp32 B row pitch (floats)
    static constexpr int A_SLOTS = BM * CPR;     // 16-byte LDS slots per stage (A)
    static constexpr int B_SLOTS = BF ? BN * CPR : (BK * BNP) / 4;
    static constexpr int STAGE_SLOTS = A_SLOTS + B_SLOTS;
    static constexpr int LDS_BYTES = ST * STAGE_SLOTS * 16;

    static_assert(BM % (16 * WGM) == 0 && BN % (16 * WGN) == 0, "per-wave tile must be whole 16x16 tiles");
    static_assert(BK % KSTEP == 0, "BK must be a multiple of the MFMA K step");
    static_assert(ST == 1 || ST == 2, "pipeline depth");
    static_assert(W <= 16, "at most 1024 threads");
};

template <bool BF, int BM, int BN, int BK, int WGM, int WGN, int ST>
__global__ void __launch_bounds__(64 * WGM * WGN)
gemm_tiled_kernel(GemmParams p)
{
    using Cf = Tiled<BF, BM, BN, BK, WGM, WGN, ST>;
    constexpr int T = Cf::T, CPR = Cf::CPR, EB = Cf::EB;
    constexpr int FM = Cf::FM, FN = Cf::FN;
    __shared__ u32x4_t lds[ST * Cf::STAGE_SLOTS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave: scalar registers
    const int l16 = lane & 15, g = lane >> 4;
    const int wm = wave / WGN, wn = wave % WGN;

    int tile, tm, tn, split;
    map_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tile, tm, tn, split);
    const int M = p.M, N = p.N, K = p.K;
    const int m0 = tm * BM, n0 = tn * BN;
    const int kbeg = split * p.kps;
    const int kend = min(K, kbeg + p.kps);
    const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

    const char* Ab = static_cast<const char*>(p.A);
    const char* Bb = static_cast<const char*>(p.B);
    const int64_t a_total = (int64_t)M * K, b_total = (int64_t)K * N;

    u32x4_t ra[Cf::A_PT];
    u32x4_t rb[Cf::B_PT][BF ? 8 : 1];

    // ---- global -> registers for the K step starting at k0
    auto load_tile = [&](int k0) {
        const int64_t a_off = (int64_t)m0 * K + k0;
        const __amdgpu_buffer_rsrc_t rA = make_rsrc(Ab + a_off * EB, (a_total - a_off) * EB);
#pragma unroll
        for (int i = 0; i < Cf::A_PT; ++i) {
            const int q = tid + i * T;
            if (Cf::A_CH % T == 0 || q < Cf::A_CH) {
                const int row = q / CPR, c = q % CPR;
                const bool rv = m0 + row < M;
                if constexpr (BF) {
                    unsigned h[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const bool v = rv && (k0 + c * 8 + e < kend);
                        h[e] = load2(rA, v ? (row * K + c * 8 + e) * 2 : kOOB);
                    }
#pragma unroll
                    for (int d = 0; d < 4; ++d)
                        ra[i][d] = h[2 * d] | (h[2 * d + 1] << 16);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const bool v = rv && (k0 + c * 4 + e < kend);
                        ra[i][e] = load4(rA, v ? (row * K + c * 4 + e) * 4 : kOOB);
                    }
                }
            }
        }
        const int64_t b_off = (int64_t)k0 * N + n0;
        const __amdgpu_buffer_rsrc_t rB = make_rsrc(Bb + b_off * EB, (b_total - b_off) * EB);
#pragma unroll
        for (int i = 0; i < Cf::B_PT; ++i) {
            const int u = tid + i * T;
            if (Cf::B_UNITS % T == 0 || u < Cf::B_UNITS) {
                if constexpr (BF) {
                    const int nb = u % (BN / 8), kb = u / (BN / 8);
#pragma unroll
                    for (int r = 0; r < 8; ++r) {
                        const int krow = kb * 8 + r;
                        const bool kv = k0 + krow < kend;
                        unsigned h[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const bool v = kv && (n0 + nb * 8 + e < N);
                            h[e] = load2(rB, v ? (krow * N + nb * 8 + e) * 2 : kOOB);
                        }
#pragma unroll
                        for (int d = 0; d < 4; ++d)
                            rb[i][r][d] = h[2 * d] | (h[2 * d + 1] << 16);
                    }
                } else {
                    const int cc = u % (BN / 4), krow = u / (BN / 4);
                    const bool kv = k0 + krow < kend;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const bool v = kv && (n0 + cc * 4 + e < N);
                        rb[i][0][e] = load4(rB, v ? (krow * N + cc * 4 + e) * 4 : kOOB);
                    }
                }
            }
        }
    };

    // ---- registers -> LDS stage s
    auto store_tile = [&](int s) {
        u32x4_t* L = lds + s * Cf::STAGE_SLOTS;
#pragma unroll
        for (int i = 0; i < Cf::A_PT; ++i) {
            const int q = tid + i * T;
            if (Cf::A_CH % T == 0 || q < Cf::A_CH) {
                const int row = q / CPR, c = q % CPR;
                L[row * CPR + (c ^ swz<CPR>(row))] = ra[i];
            }
        }
#pragma unroll
        for (int i = 0; i < Cf::B_PT; ++i) {
            const int u = tid + i * T;
            if (Cf::B_UNITS % T == 0 || u < Cf::B_UNITS) {
                if constexpr (BF) {
                    const int nb = u % (BN / 8), kb = u / (BN / 8);
                    u32x4_t tr[8];
                    transpose8x8_b16(rb[i], tr);
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        const int n = nb * 8 + t;
                        L[Cf::A_SLOTS + n * CPR + (kb ^ swz<CPR>(n))] = tr[t];
                    }
                } else {
                    const int cc = u % (BN / 4), krow = u / (BN / 4);
                    L[Cf::A_SLOTS + (krow * Cf::BNP + cc * 4) / 4] = rb[i][0];
                }
            }
        }
    };

    f32x4_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // ---- MFMA work on LDS stage s
    auto compute = [&](int s) {
        const u32x4_t* L = lds + s * Cf::STAGE_SLOTS;
        if constexpr (BF) {
#pragma unroll
            for (int kk = 0; kk < BK / 32; ++kk) {
                u32x4_t a[FM], b[FN];
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int row = wm * Cf::WM + i * 16 + l16;
                    a[i] = L[row * CPR + ((kk * 4 + g) ^ swz<CPR>(row))];
                }
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int n = wn * Cf::WN + j * 16 + l16;
                    b[j] = L[Cf::A_SLOTS + n * CPR + ((kk * 4 + g) ^ swz<CPR>(n))];
                }
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = mfma_bf16(a[i], b[j], acc[i][j]);
            }
        } else {
            const float* LB = reinterpret_cast<const float*>(L + Cf::A_SLOTS);
#pragma unroll
            for (int kk = 0; kk < BK / 16; ++kk) {
                u32x4_t a[FM];
                float b[FN][4];
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int row = wm * Cf::WM + i * 16 + l16;
                    a[i] = L[row * CPR + ((kk * 4 + g) ^ swz<CPR>(row))];
                }
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4)
                        b[j][s4] = LB[(kk * 16 + g * 4 + s4) * Cf::BNP + wn * Cf::WN + j * 16 + l16];
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
                    for (int i = 0; i < FM; ++i)
#pragma unroll
                        for (int j = 0; j < FN; ++j)
                            // element first, then reinterpret: a bit cast applied to a
                            // vector element lvalue reads element 0 whatever the index
                            acc[i][j] = mfma_f32(__uint_as_float((unsigned)a[i][s4]), b[j][s4], acc[i][j]);
            }
        }
    };

    // ---- main loop
    if (nk > 0) {
        load_tile(kbeg);
        store_tile(0);
    }
    __syncthreads();
    for (int t = 0; t < nk; ++t) {
        const int cur = (ST == 1) ? 0 : (t & 1);
        const bool more = t + 1 < nk;
        if (more)
            load_tile(kbeg + (t + 1) * BK);
        compute(cur);
        if constexpr (ST == 1) {
            __syncthreads();
            if (more)
                store_tile(0);
            __syncthreads();
        } else {
            if (more)
                store_tile(cur ^ 1);
            __syncthreads();
        }
    }

    const OutSpec out = out_spec(p, split);

    // ---- epilogue: bias, activation, convert, store
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn * Cf::WN + j * 16 + l16;
        const bool cv = col < N;
        const float bj = (out.bias && cv) ? out.bias[col] : 0.0f;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm * Cf::WM + i * 16 + g * 4 + r;
                if (cv && row < M) {
                    const float v = apply_act(acc[i][j][r] + bj, out.act);
                    const int64_t idx = (int64_t)row * N + col;
                    if (out.bf16)
                        static_cast<unsigned short*>(out.dst)[idx] = f32_to_bf16_rne(v);
                    else
                        static_cast<float*>(out.dst)[idx] = v;
                }
            }
        }
    }
}

}  // namespace tg
