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
//     chunk a lane fetches decides the LDS layout, so the layouts below cost
//     nothing to build; out-of-range lanes (M, N, K edges) write zeros;
//   * completion is tracked with s_waitcnt vmcnt(n) per wave followed by a
//     plain s_barrier: no fence, so loads of later stages stay in flight (the
//     loads are issued as inline assembly so that the compiler does not add
//     its own full drain before the LDS reads);
//   * A sits in LDS as 32-wide k sub-panels [BK/32][BM][4 x 16 B], K-contiguous,
//     and is read with ds_read_b128 (8 k values of one row per lane = the A
//     operand of v_mfma_f32_16x16x32_bf16);
//   * B stays N-contiguous in 64-column blocks [BN/64][BK][128 B] whose rows
//     are permuted so that a ds_read_b64_tr_b16 (within each 16-lane group,
//     lane L names 4 consecutive columns of row base + L/4 and lane i receives
//     column i of those four rows) touches 16 consecutive LDS rows; two such
//     reads give the 8 k values of one column that the B operand wants;
//   * 16-byte chunks are XOR-swizzled by row bits that come from the lane
//     index only, so every fragment read is one per-lane base register plus an
//     immediate offset, every transfer one per-lane register plus a scalar
//     offset, and the reads of a half-wave hit 64 distinct banks.
#pragma once

#include "common.hpp"

namespace tg {

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

template <int BM, int BN, int BK, int WGM, int WGN, int ST>
struct TiledDma {
    static constexpr int W = WGM * WGN;
    static constexpr int T = 64 * W;
    static constexpr int WM = BM / WGM, WN = BN / WGN;
    static constexpr int FM = WM / 16, FN = WN / 16;
    static constexpr int KK = BK / 32;                  // 32-wide k slices per step
    static constexpr int A_BYTES = BM * BK * 2;
    static constexpr int QW = BN < 64 ? BN : 64;        // columns per B block
    static constexpr int U = QW / 16;                   // 16-column units per B row
    static constexpr int RB = QW * 2;                   // bytes per B block row
    static constexpr int B_BYTES = BK * BN * 2;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int A_INST = A_BYTES / 1024;       // wave-wide 1 KiB transfers
    static constexpr int B_INST = B_BYTES / 1024;
    static constexpr int INST = A_INST + B_INST;
    static constexpr int LPW_MAX = (INST + W - 1) / W;
    static constexpr int LPW_MIN = INST / W;
    static constexpr int WAIT_N = (ST - 2) * LPW_MIN > 63 ? 63 : (ST - 2) * LPW_MIN;
    static constexpr int PPI = 1024 / RB;               // B rows per transfer (8 or 16)
    static constexpr int SLOTS_PER_ROW = RB / 16;       // 16-byte slots per B block row
    // Read the next k slice's B fragments during the last row-tile of the
    // current one only when the extra FN x 4 registers fit next to the
    // accumulators (at W waves a lane has 512 / max(1, W/4) registers).
    static constexpr int REGS = W <= 4 ? 512 : 512 / (W / 4);
    static constexpr bool PREFETCH_B = KK > 1 && FM * FN * 4 + 8 * FN + 8 + 64 <= REGS;

    static_assert(BM % (16 * WGM) == 0 && BN % (16 * WGN) == 0, "whole 16x16 tiles per wave");
    static_assert(BK % 32 == 0, "BK is a multiple of the MFMA K (32)");
    static_assert(BM % 16 == 0 && BN % 32 == 0, "tile sizes");
    static_assert(ST >= 2 && ST <= 4, "pipeline depth");
};

// A: 64-byte rows (4 chunks of 8 k); chunk c of row r sits at c ^ swz_a(r).
// Uses row bits 1..3 only: 16 consecutive rows read one chunk each without
// bank conflicts (within 128- and 256-byte windows).
__device__ __forceinline__ int swz_a(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

// B: 32-byte unit u (16 columns) of block row p sits at u ^ swz_b(p).
template <int RB>
__device__ __forceinline__ int swz_b(int p)
{
    return RB == 128 ? ((p >> 1) & 3) : ((p >> 2) & 1);
}

// B block rows are stored in the order the transposed reads consume them:
// within each 32-row slice, row 8g + 4h + q (g, h, q = lane group, read half,
// row in the group of four) goes to position 16h + 4g + q.
__device__ __forceinline__ int b_pos_to_row(int p)
{
    return (p & ~31) | (((p >> 4) & 1) << 2) | (((p >> 2) & 3) << 3) | (p & 3);
}

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
// it; completion is tracked explicitly with wait_vmcnt<> instead.  The
// compiler does not insert hazard wait states in front of an asm statement
// for the registers it reads, so the statement carries its own: a vector
// memory instruction that reads an SGPR written by a VALU instruction needs
// 5 wait states on this chip family (the compiler reloads spilled SGPRs with
// v_readlane, and without the wait the load takes a stale offset or
// descriptor word), and an LDS-DMA load needs 1 after M0 is written.
__device__ __forceinline__ void dma16(i32x4_t rsrc, int voff, int soff, unsigned lds_addr)
{
    __asm__ __volatile__("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff),
                         "{m0}"(lds_addr)
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

__device__ __forceinline__ u32x4_t lds_read_b128(unsigned addr)
{
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(addr);
}

__device__ __forceinline__ u32x2_t lds_read_tr(unsigned addr)
{
    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<__attribute__((address_space(3))) i16x4_t*>(addr));
    return __builtin_bit_cast(u32x2_t, v);
}

template <int BM, int BN, int BK, int WGM, int WGN, int ST>
__global__ void __launch_bounds__(64 * WGM * WGN)
gemm_tiled_dma_kernel(GemmParams p)
{
    using Cf = TiledDma<BM, BN, BK, WGM, WGN, ST>;
    constexpr int T = Cf::T, FM = Cf::FM, FN = Cf::FN, W = Cf::W, KK = Cf::KK;
    constexpr int RB = Cf::RB, U = Cf::U, QW = Cf::QW;
    __shared__ u32x4_t lds[ST * Cf::STAGE_BYTES / 16];
    // split-K arrival flag: lives in the (then idle) panel buffers, so the
    // LDS footprint is exactly ST panels
    int& s_last = *reinterpret_cast<int*>(lds);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // uniform per wave (scalar registers); a constant for one-wave blocks, so
    // that the transfer schedule below is resolved at compile time
    const int wave = W == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 6);
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
    const int rows_left = M - m0;      // valid A rows in this tile (may exceed BM)
    const int cols_left = N - n0;      // valid B columns in this tile

    // ---- per-lane parts of the transfers (fixed for the whole K loop)
    // A transfer: 16 rows x 64 bytes of one 32-wide k slice; lane -> row lane/4,
    // physical chunk lane%4 holding logical chunk (lane%4) ^ swz_a(row).
    const int a_row = lane >> 2;
    const int a_chunk = (lane & 3) ^ swz_a(a_row);
    const int voA = a_row * K * 2 + a_chunk * 16;
    // B transfer: PPI block rows x RB bytes; lane -> block row p_l, 16-byte slot
    // s16 (unit s16/2 ^ swz_b, half s16%2).
    const int b_pl = lane / Cf::SLOTS_PER_ROW;
    const int b_s16 = lane % Cf::SLOTS_PER_ROW;
    const int b_col = (((b_s16 >> 1) ^ swz_b<RB>(b_pl)) * 16) + (b_s16 & 1) * 8;   // column within the block
    const int b_krow_lane = b_pos_to_row(b_pl);       // row bits coming from the lane
    const int voB = b_krow_lane * N * 2 + b_col * 2;

    const unsigned lds_base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) u32x4_t*)lds;

    auto issue = [&](int t, int buf) {
        const int k0 = kbeg + t * BK;
        const int klim = kend - k0;   // k >= klim (relative) lies outside this split
        const int64_t a_off = (int64_t)m0 * K + k0;
        const int64_t b_off = (int64_t)k0 * N + n0;
        const i32x4_t rA = rsrc_words(Ab + a_off * 2, (a_total - a_off) * 2);
        const i32x4_t rB = rsrc_words(Bb + b_off * 2, (b_total - b_off) * 2);
        const unsigned dst0 = lds_base + (unsigned)(buf * Cf::STAGE_BYTES);
#pragma unroll
        for (int q = 0; q < Cf::LPW_MAX; ++q) {
            const int j = wave + q * W;
            if (j < Cf::A_INST) {
                // rows rb*16 .. +15 of k slice kk
                const int kk = j / (BM / 16), rb = j % (BM / 16);
                const bool ok = (rb * 16 + a_row < rows_left) && (kk * 32 + a_chunk * 8 < klim);
                dma16(rA, ok ? voA : kOOB, (rb * 16 * K + kk * 32) * 2, dst0 + (unsigned)(j * 1024));
            } else if (j < Cf::INST) {
                const int jb = j - Cf::A_INST;
                const int blk = jb / (BK / Cf::PPI), pblk = jb % (BK / Cf::PPI);
                const int p_unif = pblk * Cf::PPI;                   // block-row bits from the transfer index
                const int krow_unif = b_pos_to_row(p_unif);           // disjoint from the lane's row bits
                const bool ok = (blk * QW + b_col < cols_left) && (krow_unif + b_krow_lane < klim);
                dma16(rB, ok ? voB : kOOB, krow_unif * N * 2 + blk * QW * 2,
                      dst0 + (unsigned)(Cf::A_BYTES + jb * 1024));
            }
        }
    };

    // ---- per-lane LDS read bases (bytes within a stage)
    // A fragment (row-tile i, k slice kk): row wm*WM + 16 i + l16, chunk g.
    const unsigned rdA = (unsigned)((wm * Cf::WM + l16) * 64 + ((g ^ swz_a(l16)) * 16));
    // B fragment (column tile j, k slice kk, half h): block row 16h + 4g + l16/4
    // of slice kk, columns 4 (l16 % 4) .. +3 of the 16-column unit.
    const int b_prow = 4 * g + (l16 >> 2);
    unsigned rdB[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int J = wn * (Cf::WN / 16) + j;          // 16-column unit index within the tile
        const int blk = J / U, jj = J % U;
        rdB[j] = (unsigned)(Cf::A_BYTES + blk * BK * RB + b_prow * RB + ((jj ^ swz_b<RB>(b_prow)) * 32) +
                            (l16 & 3) * 8);
    }

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
        const unsigned st = lds_base + (unsigned)(buf * Cf::STAGE_BYTES);
        const unsigned a0 = st + rdA;
        auto read_a = [&](int i, int kk) { return lds_read_b128(a0 + (unsigned)(kk * BM * 64 + i * 1024)); };
        auto read_b = [&](int kk, u32x4_t(&b)[FN]) {
#pragma unroll
            for (int j = 0; j < FN; ++j) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const u32x2_t w = lds_read_tr(st + rdB[j] + (unsigned)((kk * 32 + h * 16) * RB));
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
            if (!Cf::PREFETCH_B && kk > 0)
                read_b(kk, b_cur);
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                u32x4_t a_nxt = a_cur;
                if (i + 1 < FM)
                    a_nxt = read_a(i + 1, kk);
                else if (kk + 1 < KK)
                    a_nxt = read_a(0, kk + 1);
                if (Cf::PREFETCH_B && kk + 1 < KK && i == FM - 1)
                    read_b(kk + 1, b_nxt);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = mfma_bf16(a_cur, b_cur[j], acc[i][j]);
                __builtin_amdgcn_sched_barrier(0);
                a_cur = a_nxt;
            }
            if (Cf::PREFETCH_B && kk + 1 < KK) {
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
        constexpr int TV = BM * BN / 4;            // 16-byte values per partial tile
        const __amdgpu_buffer_rsrc_t ws = ws_rsrc(p.ws, tile, p.split, TV);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                ws_store(ws, split * TV + (i * FN + j) * T + tid, acc[i][j]);
        wait_vm_all();
        __syncthreads();
        if (tid == 0)
            s_last = (ws_arrive(p.counters, tile) == (unsigned)(p.split - 1));
        __syncthreads();
        if (!s_last)
            return;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < p.split; ++s) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] += ws_load(ws, s * TV + (i * FN + j) * T + tid);
        }
        if (tid == 0)
            ws_reset(p.counters, tile);
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
