// Block-tiled bf16 GEMM with an asynchronous multi-stage LDS pipeline:
//     C = act(A . B + bias),  A [M][K], B [K][N] row-major, bf16 in, fp32 accumulate.
//
// Same decomposition as gemm_tiled.hpp (page "Tile Selection: Cost Models
// Against Measurement", "The structure of the search space": BM x BN block
// tile, BK reduction step, WGM x WGN waves each owning a (BM/WGM) x (BN/WGN)
// tile), but the panels travel global -> LDS without passing through
// registers, so the pipeline can be ST stages deep: tiles t+1 .. t+ST-1 are in
// flight while the matrix cores work on tile t.  Page "Tiling the hierarchy"
// (double buffering): the overlap has to be asynchronous to exist at all, a
// compute-bound tile wants at least two stages and a latency-bound one wants
// more; on MI355X one K step of even a 256 x 256 tile is shorter than the
// memory latency under load, so depth is what hides it.
//
// gfx950 specifics:
//   * buffer_load_dwordx4 ... lds: every lane of a wave fetches 16 bytes into
//     consecutive 16-byte LDS slots (slot = wave base + lane); which global
//     chunk a lane fetches decides the LDS layout, so the XOR swizzles below
//     cost nothing; out-of-range lanes (M, N, K edges) write zeros;
//   * completion is tracked with s_waitcnt vmcnt(n) per wave followed by a
//     plain s_barrier: no fence, so loads of later stages stay in flight (the
//     loads are issued as inline assembly so that the compiler does not add
//     its own full drain before the LDS reads);
//   * A [BM][BK] is K-contiguous in LDS and read with ds_read_b128 (8 k values
//     of one row per lane = the A operand of v_mfma_f32_16x16x32_bf16);
//   * B [BK][BN] stays N-contiguous (as in memory) and is read with
//     ds_read_b64_tr_b16: within each 16-lane group, lane L supplies the
//     address of 4 consecutive columns of row (base + L/4) and lane i gets
//     column i of the four rows -- two such reads give the 8 k values of one
//     column that the B operand wants.
#pragma once

#include "common.hpp"

namespace tg {

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
#define TG_LDS(p) ((__attribute__((address_space(3))) void*)(p))

template <int BM, int BN, int BK, int WGM, int WGN, int ST>
struct TiledDma {
    static constexpr int W = WGM * WGN;
    static constexpr int T = 64 * W;
    static constexpr int WM = BM / WGM, WN = BN / WGN;
    static constexpr int FM = WM / 16, FN = WN / 16;
    static constexpr int CPRA = BK / 8;               // 16-byte chunks per A row
    static constexpr int CPRB = BN / 8;               // 16-byte chunks per B row
    static constexpr int A_SLOTS = BM * CPRA;
    static constexpr int B_SLOTS = BK * CPRB;
    static constexpr int STAGE_SLOTS = A_SLOTS + B_SLOTS;
    static constexpr int A_INST = A_SLOTS / 64;       // wave-wide 1 KiB DMA instructions
    static constexpr int B_INST = B_SLOTS / 64;
    static constexpr int INST = A_INST + B_INST;
    static constexpr int LPW_MAX = (INST + W - 1) / W;
    static constexpr int LPW_MIN = INST / W;
    static constexpr int WAIT_N = (ST - 2) * LPW_MIN > 63 ? 63 : (ST - 2) * LPW_MIN;
    static constexpr int LDS_BYTES = ST * STAGE_SLOTS * 16;

    static_assert(BM % (16 * WGM) == 0 && BN % (16 * WGN) == 0, "whole 16x16 tiles per wave");
    static_assert(BK % 32 == 0, "BK is a multiple of the MFMA K (32)");
    static_assert(A_SLOTS % 64 == 0 && B_SLOTS % 64 == 0, "whole wave instructions per panel");
    static_assert(ST >= 2 && ST <= 4, "pipeline depth");
};

// XOR swizzle of B's 16-byte chunks per k row: for the transposed reads, the
// 8 rows a half-wave touches land in distinct 32-byte bank windows.
template <int CPRB>
__device__ __forceinline__ int swz_b(int r)
{
    return (2 * ((r & 3) + 4 * ((r >> 3) & 1))) & (CPRB - 1) & ~1;
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Buffer resource words (base, 32-bit num_records, gfx9 raw-buffer flags).
__device__ __forceinline__ i32x4_t rsrc_words(const void* base, int64_t bytes)
{
    const int64_t n = bytes < 0 ? 0 : (bytes > kMaxRecords ? kMaxRecords : bytes);
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return i32x4_t{(int)(uint32_t)a, (int)((a >> 32) & 0xFFFFu), (int)n, kRsrcWord3};
}

// One wave-wide load of 16 bytes per lane from a buffer straight into LDS
// (lane l writes LDS bytes lds_addr + 16 l .. + 15; out-of-range offsets
// write zeros).  Issued as inline assembly on purpose: the compiler's
// wait-count insertion would otherwise treat every later LDS read as
// dependent on all outstanding transfers and drain the whole pipeline before
// it; completion is tracked explicitly with wait_vmcnt<> instead.
__device__ __forceinline__ void dma16(i32x4_t rsrc, int voff, unsigned lds_addr)
{
    __asm__ __volatile__("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_addr)
                         : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    // expcnt and lgkmcnt at their maxima: wait on vector memory only
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

__device__ __forceinline__ void block_barrier()
{
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ __volatile__("" ::: "memory");
}

template <int BM, int BN, int BK, int WGM, int WGN, int ST>
__global__ void __launch_bounds__(64 * WGM * WGN)
gemm_tiled_dma_kernel(GemmParams p)
{
    using Cf = TiledDma<BM, BN, BK, WGM, WGN, ST>;
    constexpr int T = Cf::T, CPRA = Cf::CPRA, CPRB = Cf::CPRB, FM = Cf::FM, FN = Cf::FN, W = Cf::W;
    __shared__ u32x4_t lds[ST * Cf::STAGE_SLOTS];
    // split-K arrival flag: lives in the (then idle) panel buffers, so the
    // LDS footprint is exactly ST panels
    int& s_last = *reinterpret_cast<int*>(lds);

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

    // per-lane source of each DMA instruction this wave issues (fixed over K):
    // byte offset in the panel rebased at each K step, or kOOB when the lane's
    // row (A) or columns (B) lie outside the matrix
    int voff[Cf::LPW_MAX];
#pragma unroll
    for (int q = 0; q < Cf::LPW_MAX; ++q) {
        const int j = wave + q * W;
        voff[q] = kOOB;
        if (j < Cf::A_INST) {
            const int s = j * 64 + lane;
            const int row = s / CPRA, c = (s % CPRA) ^ swz<CPRA>(s / CPRA);
            if (m0 + row < M)
                voff[q] = row * K * 2 + c * 16;
        } else if (j < Cf::INST) {
            const int s = (j - Cf::A_INST) * 64 + lane;
            const int krow = s / CPRB, cn = (s % CPRB) ^ swz_b<CPRB>(s / CPRB);
            if (n0 + cn * 8 < N)
                voff[q] = krow * N * 2 + cn * 16;
        }
    }
    const unsigned lds_base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) u32x4_t*)lds;

    auto issue = [&](int t, int buf) {
        const int k0 = kbeg + t * BK;
        const int klim = kend - k0;   // k >= klim (relative) lies outside this split
        const int64_t a_off = (int64_t)m0 * K + k0;
        const int64_t b_off = (int64_t)k0 * N + n0;
        const i32x4_t rA = rsrc_words(Ab + a_off * 2, (a_total - a_off) * 2);
        const i32x4_t rB = rsrc_words(Bb + b_off * 2, (b_total - b_off) * 2);
        const unsigned dst0 = lds_base + (unsigned)(buf * Cf::STAGE_SLOTS * 16);
        const bool tail = klim < BK;
#pragma unroll
        for (int q = 0; q < Cf::LPW_MAX; ++q) {
            const int j = wave + q * W;
            if (j < Cf::INST) {
                int vo = voff[q];
                if (tail) {   // last, partial K step: mask the chunks (A) / rows (B) past the end
                    const int s = (j < Cf::A_INST ? j : j - Cf::A_INST) * 64 + lane;
                    const int kp = j < Cf::A_INST ? ((s % CPRA) ^ swz<CPRA>(s / CPRA)) * 8 : s / CPRB;
                    vo = kp < klim ? vo : kOOB;
                }
                dma16(j < Cf::A_INST ? rA : rB, vo, dst0 + (unsigned)(j * 64 * 16));
            }
        }
    };

    f32x4_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // ---- MFMA work on one LDS stage.  Fragment reads run one step ahead of
    // the MFMAs that consume them: the A fragment of row-tile i+1 is read
    // while row-tile i multiplies, and the B fragments of the next 32-wide k
    // slice while the last row-tile of this one multiplies.  sched_barrier
    // pins that order (left alone, the scheduler sinks every read next to its
    // first use and the matrix core waits on each LDS round trip).
    auto compute = [&](int buf) {
        const u32x4_t* LA = lds + buf * Cf::STAGE_SLOTS;
        const char* LB = reinterpret_cast<const char*>(LA + Cf::A_SLOTS);
        constexpr int KK = BK / 32;
        auto read_a = [&](int i, int kk) {
            const int row = wm * Cf::WM + i * 16 + l16;
            return LA[row * CPRA + ((kk * 4 + g) ^ swz<CPRA>(row))];
        };
        auto read_b = [&](int kk, u32x4_t(&b)[FN]) {
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int n = wn * Cf::WN + j * 16 + 4 * (l16 & 3);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int krow = kk * 32 + 8 * g + 4 * h + (l16 >> 2);
                    const int cn = (n >> 3) ^ swz_b<CPRB>(krow);
                    const char* src = LB + krow * (BN * 2) + cn * 16 + (n & 7) * 2;
                    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4_t*)(src));
                    const u32x2_t w = __builtin_bit_cast(u32x2_t, v);
                    b[j][2 * h] = w.x;
                    b[j][2 * h + 1] = w.y;
                }
            }
        };
        u32x4_t b_cur[FN], b_nxt[FN];
        read_b(0, b_cur);
        u32x4_t a_cur = read_a(0, 0);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                u32x4_t a_nxt = a_cur;
                if (i + 1 < FM)
                    a_nxt = read_a(i + 1, kk);
                else if (kk + 1 < KK)
                    a_nxt = read_a(0, kk + 1);
                if (kk + 1 < KK && i == FM - 1)
                    read_b(kk + 1, b_nxt);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = mfma_bf16(a_cur, b_cur[j], acc[i][j]);
                __builtin_amdgcn_sched_barrier(0);
                a_cur = a_nxt;
            }
            if (kk + 1 < KK) {
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    b_cur[j] = b_nxt[j];
            }
        }
    };

    // ---- pipeline: tile t lives in buffer t % ST
#pragma unroll
    for (int t = 0; t < ST - 1; ++t)
        if (t < nk)
            issue(t, t);
    for (int t = 0; t < nk; ++t) {
        if (t + ST - 2 < nk)
            wait_vmcnt<Cf::WAIT_N>();     // this wave's loads of tile t have landed
        else
            wait_vmcnt<0>();
        block_barrier();                  // ... and every wave's; tile t-1's buffer is free
        if (t + ST - 1 < nk)
            issue(t + ST - 1, (t + ST - 1) % ST);
        compute(t % ST);
    }

    // ---- split-K: publish the partial tile; the last arriving block reduces
    if (p.split > 1) {
        f32x4_t* wsp = reinterpret_cast<f32x4_t*>(p.ws) + (int64_t)tile * p.split * (BM * BN / 4);
        f32x4_t* mine = wsp + (int64_t)split * (BM * BN / 4);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                mine[(i * FN + j) * T + tid] = acc[i][j];
        __threadfence();
        __syncthreads();
        if (tid == 0) {
            const unsigned prev = __hip_atomic_fetch_add(p.counters + tile, 1u, __ATOMIC_ACQ_REL,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            s_last = (prev == (unsigned)(p.split - 1));
        }
        __syncthreads();
        if (!s_last)
            return;
        __threadfence();
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < p.split; ++s) {
            const f32x4_t* part = wsp + (int64_t)s * (BM * BN / 4);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] += part[(i * FN + j) * T + tid];
        }
        if (tid == 0)
            __hip_atomic_store(p.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- epilogue: bias, activation, convert, store
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn * Cf::WN + j * 16 + l16;
        const bool cv = col < N;
        const float bj = (p.bias && cv) ? p.bias[col] : 0.0f;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm * Cf::WM + i * 16 + g * 4 + r;
                if (cv && row < M) {
                    const float v = apply_act(acc[i][j][r] + bj, p.act);
                    const int64_t idx = (int64_t)row * N + col;
                    if (p.out_bf16)
                        static_cast<unsigned short*>(p.C)[idx] = f32_to_bf16_rne(v);
                    else
                        static_cast<float*>(p.C)[idx] = v;
                }
            }
        }
    }
}

}  // namespace tg
