// Block-tiled GEMM with an asynchronous multi-stage LDS pipeline:
//     C = act(A . B + bias),  A [M][K], B [K][N] row-major, bf16 or fp32 in,
//     fp32 accumulate.
//
// Same decomposition as gemm_tiled.hpp (page "Tile Selection: Cost Models
// Against Measurement", "The structure of the search space": BM x BN block
// tile, BK reduction step, WGM x WGN waves each owning a (BM/WGM) x (BN/WGN)
// tile), but the panels travel global -> LDS without passing through
// registers, so the pipeline can be ST stages deep (page "Tiling the
// hierarchy", double buffering: the overlap must be asynchronous to exist,
// and a latency-bound tile wants more than two stages; on MI355X one K step
// of even a 256 x 256 tile is shorter than the memory latency under load).
//
// Schedule.  A stage (one BK step) is KK slices of 64 bytes of an A row (32
// bf16 or 16 fp32 k); with K groups (WK > 1) a wave takes KK/WK of them.  A wave's
// fragment registers are double buffered per slice, and while the matrix
// core works through the FM x FN MFMAs of slice s the wave reads slice s+1's
// fragments and, in the last slice of a stage, issues the transfers of the
// tile ST steps ahead -- one or two such instructions after each MFMA, in an
// order pinned with sched_barrier, so the matrix core is never left waiting
// on an instruction burst.  There is one block barrier per stage, at the
// start of its last slice: by then every read of the stage's buffer has
// returned (its fragments are in registers) and the next tile has landed, so
// after the barrier the buffer can be refilled and the next stage's first
// fragments read while the last slice multiplies.  Tiles past the end of the
// K range are issued as fully out-of-range transfers (they write zeros that
// nothing reads), which keeps every stage -- and every wait count -- the same.
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
//   * A sits in LDS as whole rows [BM][BK elements], K-contiguous (a transfer
//     carries 16, 8 or 4 complete rows, so rows of 128 bytes or more request
//     whole lines), and is read with ds_read_b128 (8 bf16 k of one row per
//     lane = the A operand of v_mfma_f32_16x16x32_bf16; 4 fp32 k, one per
//     v_mfma_f32_16x16x4_f32 of the slice);
//   * bf16 B stays N-contiguous in 64-column blocks [BN/64][BK][128 B] whose
//     rows are permuted so that a ds_read_b64_tr_b16 (within each 16-lane
//     group, lane L names 4 consecutive columns of row base + L/4 and lane i
//     receives column i of those four rows) touches 16 consecutive LDS rows;
//     two such reads give the 8 k values of one column that the B operand
//     wants; fp32 B sits in 64-column blocks of 256-byte rows (32 columns of
//     128 bytes for 32-wide tiles) in K order and
//     is read one float per lane and MFMA;
//   * 16-byte chunks are XOR-swizzled by row bits 1..3, which for fragment
//     reads come from the lane index only: every fragment read is a per-lane
//     base register (one per slice) plus an immediate offset, and the
//     reads of a half-wave hit 64 distinct banks; every transfer is a per-lane
//     offset register fixed for the whole K loop.
#pragma once

#include "common.hpp"

namespace tg {

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

template <int BM, int BN, int BK, int WGM, int WGN, int ST, bool F32 = false, int WK = 1>
struct TiledDma {
    // WK groups of WGM x WGN waves: group kg multiplies slices kg KKW ..
    // (kg + 1) KKW - 1 of every stage into its own sums, which are added
    // through LDS after the K loop (K split among the waves of one workgroup,
    // so no second launch); every wave takes part in the transfers
    static constexpr int WO = WGM * WGN;                // waves per K group
    static constexpr int W = WO * WK;
    static constexpr int T = 64 * W;
    static constexpr int WM = BM / WGM, WN = BN / WGN;
    static constexpr int FM = WM / 16, FN = WN / 16;
    static constexpr int EB = F32 ? 4 : 2;              // bytes per input element
    static constexpr int EPS = 16 / EB;                 // elements per 16-byte slot
    static constexpr int KSL = 64 / EB;                 // k per slice: 64 bytes of an A row
    static constexpr int KK = BK / KSL;                 // slices per step
    static constexpr int KKW = KK / WK;                 // slices per step of one wave
    static constexpr int MPS = F32 ? 4 : 1;             // MFMAs per (A, B) fragment pair
    static constexpr int A_BYTES = BM * BK * EB;
    static constexpr int ROWB = BK * EB;                // bytes of one A row in LDS (all KK slices)
    static constexpr int RPA = 1024 / ROWB;             // A rows per transfer (16, 8 or 4)
    static constexpr int LPR = ROWB / 16;               // lanes per A row
    static constexpr int QW = BN < 64 ? BN : 64;        // columns per B block
    static constexpr int U = QW / 16;                   // 16-column units per B row
    static constexpr int RB = QW * EB;                  // bytes per B block row
    static constexpr int B_BYTES = BK * BN * EB;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int A_INST = A_BYTES / 1024;       // wave-wide 1 KiB transfers
    static constexpr int B_INST = B_BYTES / 1024;
    static constexpr int INST = A_INST + B_INST;
    static constexpr int LPW_MAX = (INST + W - 1) / W;   // transfers per wave per stage
    static constexpr int LPW_MIN = INST / W;
    static constexpr int cap63(int n) { return n > 63 ? 63 : n; }
    // outstanding transfers a wave may still have when tile t+1 must have
    // landed (tiles t+2 .. t+ST-1), and after the prologue (tiles 1 .. ST-1)
    static constexpr int WAIT_N = cap63((ST - 2) * LPW_MIN);
    static constexpr int WAIT_P = cap63((ST - 1) * LPW_MIN);
    static constexpr int PPI = 1024 / RB;               // B rows per transfer (4, 8 or 16)
    static constexpr int SLOTS_PER_ROW = RB / 16;       // 16-byte slots per B block row
    static constexpr int NMF = FM * FN;                 // fragment pairs per wave per slice
    static constexpr int RDB = F32 ? 4 : 2;             // LDS reads per B fragment
    static constexpr int NRD = FM + RDB * FN;           // LDS reads per wave per slice
    // fp32 waves with fewer than four output tiles keep KA partial sums per
    // tile (MFMA e of a slice adds into partial e % KA), so that consecutive
    // MFMAs never wait for each other's result; the partials are added in a
    // fixed order after the K loop
    static constexpr int KA = F32 && NMF < 4 ? 4 / NMF : 1;
    // every wave's transfers split into A and B ones the same way: which
    // operand a transfer loads is then known at compile time
    static constexpr bool STATIC_AB = A_INST % W == 0 && B_INST % W == 0;
    // the epilogue stages one 16-row slab per wave through LDS when it fits
    static constexpr bool EPI_LDS = W * 16 * (WN + 4) * 4 <= ST * STAGE_BYTES;

    static_assert(BM % (16 * WGM) == 0 && BN % (16 * WGN) == 0, "whole 16x16 tiles per wave");
    static_assert(BK % KSL == 0, "BK is a multiple of the slice (32 bf16 or 16 fp32 k)");
    static_assert(BM % 16 == 0 && BN % 32 == 0, "tile sizes");
    static_assert(A_BYTES % 1024 == 0 && B_BYTES % 1024 == 0, "whole 1 KiB transfers");
    static_assert(ST >= 2 && ST <= 8, "pipeline depth");
    static_assert(WK >= 1 && KK % WK == 0, "whole slices per K group");
    static_assert(W <= 16, "at most 1024 threads");
    // the K groups' sums meet in the stage buffers
    static_assert(WK == 1 || (WK - 1) * BM * BN * 4 <= ST * STAGE_BYTES, "LDS for the cross-group sums");
};

// A: rows of BK elements (all k of the stage: KK slices of 64 bytes, each
// four 16-byte chunks of 8 bf16 or 4 fp32 k); chunk c of row r sits at
// c ^ swz_a<KK>(r).  16 consecutive rows reading one logical
// chunk land in 16 distinct 16-byte slots of a 256-byte window (no bank
// conflicts): with 64- and 128-byte rows (BK = 32, 64) two or four rows share
// a window and the swizzle uses row bits 1..3; a 256-byte row (bf16 BK = 128,
// fp32 BK = 64) is a window of its own and the swizzle is the row within its
// 16-row group.  With rows of 128 bytes or more every A transfer requests
// whole lines (half-line requests halve what the L2 delivers per request).
template <int KK>
__device__ __forceinline__ int swz_a(int r)
{
    static_assert(KK == 1 || KK == 2 || KK == 4, "rows of 64, 128 or 256 bytes");
    r &= 15;   // a function of the row within its 16-row group (what a fragment read sees)
    return KK == 1 ? (((r >> 1) ^ (r >> 3)) & 3) : KK == 2 ? ((r >> 1) & 7) : r;
}

// B: 32-byte unit u (16 columns) of block row p sits at u ^ swz_b(p).
template <int RB>
__device__ __forceinline__ int swz_b(int p)
{
    return RB == 128 ? ((p >> 1) & 3) : ((p >> 2) & 1);
}

// fp32 B: 64-byte unit u (16 columns) of block row r sits at u ^ swz_bf<U>(r).
// A fragment read takes one float per lane from rows 4g + e of a slice (g =
// lane group, e = 0..3): with 256-byte rows the four groups then read four
// different 64-byte windows (row bits 2..3 pick the unit), with 128-byte rows
// two (a two-way conflict; only 32-column tiles have them).
template <int U>
__device__ __forceinline__ int swz_bf(int r)
{
    static_assert(U == 2 || U == 4, "32 or 64 columns per B block");
    return (r >> 2) & (U - 1);
}

// bf16 B block rows are stored in the order the transposed reads consume them:
// within each 32-row slice, row 8g + 4h + q (g, h, q = lane group, read half,
// row in the group of four) goes to position 16h + 4g + q.
__device__ __forceinline__ int b_pos_to_row(int p)
{
    return (p & ~31) | (((p >> 4) & 1) << 2) | (((p >> 2) & 3) << 3) | (p & 3);
}

// Buffer resource words (base, 32-bit num_records, gfx9 raw-buffer flags).
// Uniform by construction; readfirstlane states it, so the words always land
// in the scalar registers the transfer instruction takes (where the
// compiler's uniformity analysis loses track of them it would otherwise pick
// vector registers, which the instruction cannot encode).
__device__ __forceinline__ i32x4_t rsrc_words(const void* base, int64_t bytes)
{
    const int64_t n = bytes < 0 ? 0 : (bytes > kMaxRecords ? kMaxRecords : bytes);
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return i32x4_t{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                   __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xFFFFu)),
                   __builtin_amdgcn_readfirstlane((int)n), kRsrcWord3};
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
// NT sets the non-temporal cache policy: for data the grid reads exactly
// once, which then does not displace lines that other workgroups re-read.
template <bool NT = false>
__device__ __forceinline__ void dma16(i32x4_t rsrc, int voff, unsigned lds_addr)
{
    if constexpr (NT)
        __asm__ __volatile__("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voff), "s"(rsrc),
                             "{m0}"(lds_addr)
                             : "memory");
    else
        __asm__ __volatile__("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc),
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

// Wait until every LDS read this wave issued has returned.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

template <int N>
struct IntC {
    static constexpr int value = N;
};

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

__device__ __forceinline__ unsigned lds_read_b32(unsigned addr)
{
    return *reinterpret_cast<const __attribute__((address_space(3))) unsigned*>(addr);
}

__device__ __forceinline__ u32x2_t lds_read_tr(unsigned addr)
{
    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<__attribute__((address_space(3))) i16x4_t*>(addr));
    return __builtin_bit_cast(u32x2_t, v);
}

// One output tile (tm, tn) over the K range [kbeg, kend): the transfers, the
// pipelined MFMA loop and the epilogue into `out`.  `lds` is the workgroup's
// ST * STAGE_BYTES of LDS.  Every lane of the workgroup calls it.  F32: fp32
// operands on v_mfma_f32_16x16x4_f32 (a slice is 16 k: each lane's 16-byte A
// chunk holds k = 4g .. 4g+3 of its row, and MFMA e of the slice takes
// element e of it, with the B values of the same four k read one float at a
// time); otherwise bf16 on v_mfma_f32_16x16x32_bf16.
template <int BM, int BN, int BK, int WGM, int WGN, int ST, bool NTB, bool F32 = false, int WK = 1>
__device__ __forceinline__ void dma_tile(const GemmParams& p, u32x4_t* lds, int tm, int tn, int kbeg, int kend,
                                         const OutSpec& out)
{
    using Cf = TiledDma<BM, BN, BK, WGM, WGN, ST, F32, WK>;
    constexpr int T = Cf::T, FM = Cf::FM, FN = Cf::FN, W = Cf::W, KK = Cf::KK, KKW = Cf::KKW, WO = Cf::WO;
    constexpr int RB = Cf::RB, U = Cf::U, QW = Cf::QW, EB = Cf::EB, EPS = Cf::EPS;

    // an opaque copy of the thread index: where the tile body is used more
    // than once in a kernel, nothing derived from it is shared between the
    // uses (and held in registers from one to the next)
    int tid = threadIdx.x;
    __asm__ __volatile__("" : "+v"(tid));
    const int lane = tid & 63;
    // uniform per wave (scalar registers); a constant for one-wave blocks, so
    // that the transfer schedule below is resolved at compile time
    const int wave = W == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g = lane >> 4;
    const int kg = WK == 1 ? 0 : wave / WO;       // K group: slices kg KKW .. of every stage
    const int wo = WK == 1 ? wave : wave % WO;
    const int wm = wo / WGN, wn = wo % WGN;

    const int M = p.M, N = p.N, K = p.K;
    const int m0 = tm * BM, n0 = tn * BN;
    const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
    const char* Ab = static_cast<const char*>(p.A);
    const char* Bb = static_cast<const char*>(p.B);
    // B may hold fewer rows than K (the padded path on a ragged K only pads A):
    // the range check then reads its missing rows as zero
    const int64_t a_total = (int64_t)M * K, b_total = (int64_t)(p.kb > 0 ? p.kb : K) * N;
    const int rows_left = M - m0;      // valid A rows in this tile (may exceed BM)
    const int cols_left = N - n0;      // valid B columns in this tile

    // ---- per-lane parts of the transfers (fixed for the whole K loop)
    // A transfer: RPA whole rows (ROWB bytes each); lane -> row lane / LPR,
    // physical chunk lane % LPR holding logical chunk (lane % LPR) ^ swz_a(row).
    const int a_row = lane / Cf::LPR;
    const int a_p = lane % Cf::LPR;
    // B transfer: PPI block rows x RB bytes; lane -> block row p_l, 16-byte
    // slot s16.  bf16: unit s16/2 ^ swz_b(p_l), half s16%2, rows permuted
    // (b_pos_to_row); fp32: unit s16/4 ^ swz_bf(row), quarter s16%4, rows in
    // order (the swizzle then depends on the transfer's rows, see below).
    const int b_pl = lane / Cf::SLOTS_PER_ROW;
    const int b_s16 = lane % Cf::SLOTS_PER_ROW;
    const int b_col = F32 ? 0 : (((b_s16 >> 1) ^ swz_b<RB>(b_pl)) * 16) + (b_s16 & 1) * 8;   // column within the block
    const int b_krow_lane = F32 ? b_pl : b_pos_to_row(b_pl);       // row bits coming from the lane
    const int voB = b_krow_lane * N * EB + b_col * EB;

    // Transfer q of this wave is number j = wave + q W of the stage: A
    // transfers first (rows j RPA ..), then B (block blk, row group pblk).  Its
    // lane offset within the tile, with the M / N edge folded in, does not
    // change from stage to stage; only the K edge is checked per stage (ak8:
    // first k of the lane's A chunk).
    auto is_a = [&](int q) { return Cf::STATIC_AB ? q < Cf::A_INST / W : wave + q * W < Cf::A_INST; };
    auto exists = [&](int q) { return Cf::STATIC_AB || wave + q * W < Cf::INST; };
    auto krow_of = [&](int pblk) { return F32 ? pblk * Cf::PPI : b_pos_to_row(pblk * Cf::PPI); };
    int vo[Cf::LPW_MAX], ak8[Cf::LPW_MAX];
#pragma unroll
    for (int q = 0; q < Cf::LPW_MAX; ++q) {
        const int j = wave + q * W;
        ak8[q] = 0;
        if (is_a(q)) {
            const int row = j * Cf::RPA + a_row;
            const int c = a_p ^ swz_a<KK>(row);
            ak8[q] = c * EPS;
            vo[q] = (row < rows_left) ? (row * K + c * EPS) * EB : kOOB;
        } else {
            const int jb = j - Cf::A_INST;
            const int blk = jb / (BK / Cf::PPI), pblk = jb % (BK / Cf::PPI);
            const int krow_unif = krow_of(pblk);    // disjoint from the lane's row bits
            if constexpr (F32) {
                const int col = (((b_s16 >> 2) ^ swz_bf<U>(krow_unif + b_pl)) * 16) + (b_s16 & 3) * 4;
                vo[q] = (blk * QW + col < cols_left) ? ((krow_unif + b_pl) * N + blk * QW + col) * EB : kOOB;
            } else {
                vo[q] = (blk * QW + b_col < cols_left) ? voB + (krow_unif * N + blk * QW) * EB : kOOB;
            }
        }
    }

    const unsigned lds_base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) u32x4_t*)lds;

    // Everything the transfers of tile t need: buffer descriptors whose base is
    // the tile's corner (so lane offsets stay small), its LDS buffer, and how
    // many k of it lie inside this split's K range (<= 0 past the end).
    struct Tile {
        i32x4_t rA, rB;
        unsigned dst;
        int klim;
    };
    auto tile_desc = [&](int t, int buf) {
        Tile d;
        const int k0 = kbeg + t * BK;
        d.klim = kend - k0;
        const int64_t a_off = (int64_t)m0 * K + k0;
        const int64_t b_off = (int64_t)k0 * N + n0;
        d.rA = rsrc_words(Ab + a_off * EB, (a_total - a_off) * EB);
        d.rB = rsrc_words(Bb + b_off * EB, (b_total - b_off) * EB);
        d.dst = lds_base + (unsigned)(buf * Cf::STAGE_BYTES);
        return d;
    };
    auto dma_op = [&](int q, const Tile& d) {
        if (!exists(q))
            return;
        const int j = wave + q * W;
        if (is_a(q)) {
            dma16(d.rA, (ak8[q] < d.klim) ? vo[q] : kOOB, d.dst + (unsigned)(j * 1024));
        } else {
            const int jb = j - Cf::A_INST;
            const int krow_unif = krow_of(jb % (BK / Cf::PPI));
            dma16<NTB>(d.rB, (b_krow_lane < d.klim - krow_unif) ? vo[q] : kOOB,
                  d.dst + (unsigned)(Cf::A_BYTES + jb * 1024));
        }
    };

    // ---- per-lane LDS read bases (bytes within a stage)
    // A fragment (row-tile i, the wave's k slice kk = slice kg KKW + kk of the
    // stage): row wm*WM + 16 i + l16, logical chunk 4 (kg KKW + kk) + g; the
    // swizzle only sees row bits 1..3, i.e. l16.
    unsigned rdA[KKW];
#pragma unroll
    for (int kk = 0; kk < KKW; ++kk)
        rdA[kk] = (unsigned)((wm * Cf::WM + l16) * Cf::ROWB + ((((kg * KKW + kk) * 4 + g) ^ swz_a<KK>(l16)) * 16));
    // B fragment (column tile j, k slice kk).  bf16, read half h: block row
    // 16h + 4g + l16/4 of slice kk, columns 4 (l16 % 4) .. +3 of the 16-column
    // unit.  fp32, read e: block row 4g + e of slice kk, column l16 of the
    // unit (the unit's swizzle sees row bits 2..3, i.e. g only).
    // (+ the rows of the slices before the wave's first: KSL rows a slice)
    const int b_prow = (F32 ? 4 * g : 4 * g + (l16 >> 2)) + kg * KKW * Cf::KSL;
    unsigned rdB[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int J = wn * (Cf::WN / 16) + j;          // 16-column unit index within the tile
        const int blk = J / U, jj = J % U;
        if constexpr (F32)
            rdB[j] = (unsigned)(Cf::A_BYTES + blk * BK * RB + b_prow * RB + ((jj ^ swz_bf<U>(b_prow)) * 64) +
                                l16 * 4);
        else
            rdB[j] = (unsigned)(Cf::A_BYTES + blk * BK * RB + b_prow * RB + ((jj ^ swz_b<RB>(b_prow)) * 32) +
                                (l16 & 3) * 8);
    }

    // Accumulators live in AGPRs from here to the end of the K loop: the
    // empty asm statements pin them there at both ends (left alone, the
    // register allocator splits them between AGPRs and VGPRs and shuffles
    // them on every iteration).
    constexpr int KA = Cf::KA;
    f32x4_t acc[KA][FM][FN];
#pragma unroll
    for (int ka = 0; ka < KA; ++ka)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                acc[ka][i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                __asm__ __volatile__("" : "+a"(acc[ka][i][j]));
            }

    // fragment registers of two slices
    u32x4_t a[2][FM], b[2][FN];
    // read o of a slice, in the order its MFMAs first need them: A row-tile 0,
    // the B parts (bf16 halves, fp32 floats), then the other A row-tiles
    auto read_op = [&](unsigned st, int kk, int par, int o) {
        if (o == 0) {
            a[par][0] = lds_read_b128(st + rdA[kk]);
        } else if (o <= Cf::RDB * FN) {
            const int j = (o - 1) / Cf::RDB, h = (o - 1) % Cf::RDB;
            if constexpr (F32) {
                b[par][j][h] = lds_read_b32(st + rdB[j] + (unsigned)((kk * 16 + h) * RB));
            } else {
                const u32x2_t w = lds_read_tr(st + rdB[j] + (unsigned)((kk * 32 + h * 16) * RB));
                b[par][j][2 * h] = w.x;
                b[par][j][2 * h + 1] = w.y;
            }
        } else {
            const int i = o - Cf::RDB * FN;
            a[par][i] = lds_read_b128(st + rdA[kk] + (unsigned)(i * 16 * Cf::ROWB));
        }
    };
    // The MFMAs of one slice with NOPS other instructions spread among them.
    // Op o goes right after MFMA (o NS) / NOPS.  fp32: MFMA x takes element
    // x / NMF of its fragments, so consecutive MFMAs add into different
    // accumulators wherever the wave has more than one.
    auto slice = [&](int par, auto NOPS, auto&& op) {
        constexpr int nops = decltype(NOPS)::value;
        constexpr int NS = Cf::NMF * Cf::MPS;
#pragma unroll
        for (int x = 0; x < NS; ++x) {
            const int m = x % Cf::NMF, e = x / Cf::NMF;
            const int i = m / FN, j = m % FN;
            // element first, then reinterpret: a bit cast applied to a vector
            // element lvalue reads element 0 whatever the index
            if constexpr (F32)
                acc[e % KA][i][j] = mfma_f32(__uint_as_float((unsigned)a[par][i][e]),
                                             __uint_as_float((unsigned)b[par][j][e]), acc[e % KA][i][j]);
            else
                acc[0][i][j] = mfma_bf16(a[par][i], b[par][j], acc[0][i][j]);
            // the MFMA goes first: a read hoisted above it would make the
            // MFMA's own wait for older fragments wait for this read as well
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int o = (x * nops + NS - 1) / NS; o < ((x + 1) * nops + NS - 1) / NS; ++o)
                op(o);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // One stage: tile t in buffer buf, its first slice in fragment set PAR0.
    auto stage = [&](int t, int buf, auto PAR0) {
        constexpr int par0 = decltype(PAR0)::value;
        const unsigned st = lds_base + (unsigned)(buf * Cf::STAGE_BYTES);
#pragma unroll
        for (int kk = 0; kk < KKW; ++kk) {
            const int par = (par0 + kk) & 1;
            if (kk + 1 < KKW) {
                slice(par, IntC<Cf::NRD>{}, [&](int o) { read_op(st, kk + 1, par ^ 1, o); });
            } else {
                // all reads of this buffer have returned, tile t+1 has landed
                wait_lgkm0();
                wait_vmcnt<Cf::WAIT_N>();
                block_barrier();
                const int nbuf = buf + 1 == ST ? 0 : buf + 1;
                const unsigned nst = lds_base + (unsigned)(nbuf * Cf::STAGE_BYTES);
                const Tile d = tile_desc(t + ST, buf);
                // transfers spaced evenly among the reads: issued in a burst
                // they back up in the address unit (one 1 KiB transfer takes
                // 16 cycles there) and stall the issuing waves' MFMAs
                constexpr int NOPS = Cf::NRD + Cf::LPW_MAX;
                slice(par, IntC<NOPS>{}, [&](int o) {
                    const int before = o * Cf::LPW_MAX / NOPS;          // transfers among ops 0 .. o-1
                    if ((o + 1) * Cf::LPW_MAX / NOPS > before)
                        dma_op(before, d);
                    else
                        read_op(nst, 0, par ^ 1, o - before);
                });
            }
        }
    };

    // ---- prologue: tiles 0 .. ST-1 in flight, slice 0 of tile 0 in registers
#pragma unroll
    for (int t = 0; t < ST; ++t) {
        const Tile d = tile_desc(t, t);
#pragma unroll
        for (int q = 0; q < Cf::LPW_MAX; ++q)
            dma_op(q, d);
    }
    wait_vmcnt<Cf::WAIT_P>();
    block_barrier();
#pragma unroll
    for (int o = 0; o < Cf::NRD; ++o)
        read_op(lds_base, 0, 0, o);

    // ---- main loop; with an odd number of slices per stage (of one wave) the
    // fragment set of a stage's first slice alternates, so stages go in pairs
    if constexpr (KKW % 2 == 0) {
        int buf = 0;
        for (int t = 0; t < nk; ++t) {
            stage(t, buf, IntC<0>{});
            buf = buf + 1 == ST ? 0 : buf + 1;
        }
    } else {
        int buf = 0;
        for (int t = 0; t < nk; t += 2) {
            stage(t, buf, IntC<0>{});
            buf = buf + 1 == ST ? 0 : buf + 1;
            if (t + 1 >= nk)
                break;
            stage(t + 1, buf, IntC<1>{});
            buf = buf + 1 == ST ? 0 : buf + 1;
        }
    }
    // the zero-filling transfers of tiles past the end may still be in flight:
    // they must land before LDS is reused or released
    wait_vm_all();
#pragma unroll
    for (int ka = 0; ka < KA; ++ka)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                __asm__ __volatile__("" : "+a"(acc[ka][i][j]));
    f32x4_t (&res)[FM][FN] = acc[0];
#pragma unroll
    for (int ka = 1; ka < KA; ++ka)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                res[i][j] += acc[ka][i][j];
    if constexpr (WK > 1) {
        // the K groups' sums meet in LDS (every transfer has landed, and the
        // barrier waits for every read): groups 1 .. WK-1 store theirs, group
        // 0 adds them in group order
        __syncthreads();
        f32x4_t* part = reinterpret_cast<f32x4_t*>(lds);
        if (kg > 0) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    part[(((kg - 1) * WO + wo) * Cf::NMF + i * FN + j) * 64 + lane] = res[i][j];
        }
        __syncthreads();
        if (kg == 0) {
#pragma unroll
            for (int kq = 1; kq < WK; ++kq)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        res[i][j] += part[(((kq - 1) * WO + wo) * Cf::NMF + i * FN + j) * 64 + lane];
        }
    }

    // ---- epilogue: bias, activation, convert, store.  The lane coordinates
    // are derived afresh from an opaque copy of the thread index, so that
    // nothing the epilogue needs is computed before the K loop and held in
    // registers across it.
    int tid_e = tid;
    __asm__ __volatile__("" : "+v"(tid_e));
    const int lane_e = tid_e & 63;
    const int l16e = lane_e & 15, ge = lane_e >> 4;
    const int wave_e = W == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid_e >> 6);
    // with K groups only group 0 (waves 0 .. WO-1) holds the finished sums
    const bool owner = WK == 1 || wave_e < WO;
    const int wme = wave_e / WGN % WGM, wne = wave_e % WGN;
    const int row_w = m0 + wme * Cf::WM;          // first output row of the wave tile
    const int col_w = n0 + wne * Cf::WN;          // first output column

    if constexpr (Cf::EPI_LDS) {
        // Each wave turns its accumulators, one 16-row slab at a time, into
        // whole rows through a private LDS slab (row stride WN + 4 floats keeps
        // the four row groups of a write in different banks), then every lane
        // stores 8 consecutive outputs with one 16-byte (bf16) or two (fp32)
        // stores.  A lane always owns the same 8 columns, so it loads their
        // bias once.
        constexpr int RS = Cf::WN + 4;                 // slab row stride, floats
        constexpr int CPR = Cf::WN / 8;                // 8-column chunks per row
        constexpr int PASSES = (16 * CPR + 63) / 64;   // 64-chunk rounds per slab
        float* slab = reinterpret_cast<float*>(lds) + wave_e * 16 * RS;
        const int c8 = lane_e % CPR;                   // the lane's column chunk
        const int col0 = col_w + c8 * 8;
        // N is a multiple of 8 with bf16 operands and of 4 with fp32 ones, so a
        // chunk is whole or (fp32) its first half is
        const bool col_ok = col0 < N;
        const bool hi_ok = col0 + 4 < N;
        float bias8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            bias8[e] = (out.bias && (e < 4 ? col_ok : hi_ok)) ? out.bias[col0 + e] : 0.0f;
        __syncthreads();   // every wave's last transfers and reads are done: LDS is free
        if (!owner)
            return;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    slab[(ge * 4 + r) * RS + j * 16 + l16e] = res[i][j][r];
#pragma unroll
            for (int ps = 0; ps < PASSES; ++ps) {
                const int c = ps * 64 + lane_e;
                const int r = c / CPR;
                const int row = row_w + i * 16 + r;
                if (c < 16 * CPR && row < M && col_ok) {
                    const f32x4_t* src = reinterpret_cast<const f32x4_t*>(slab + r * RS + c8 * 8);
                    const f32x4_t v0 = src[0], v1 = src[1];
                    float o[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        o[e] = apply_act(o[e] + bias8[e], out.act);
                    const int64_t idx = (int64_t)(row - out.row0) * out.ld + (col0 - out.col0);
                    if (out.bf16) {
                        u32x4_t w;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            w[e] = (unsigned)f32_to_bf16_rne(o[2 * e]) | ((unsigned)f32_to_bf16_rne(o[2 * e + 1]) << 16);
                        *reinterpret_cast<u32x4_t*>(static_cast<unsigned short*>(out.dst) + idx) = w;
                    } else {
                        f32x4_t* dst = reinterpret_cast<f32x4_t*>(static_cast<float*>(out.dst) + idx);
                        dst[0] = f32x4_t{o[0], o[1], o[2], o[3]};
                        if (hi_ok)
                            dst[1] = f32x4_t{o[4], o[5], o[6], o[7]};
                    }
                }
            }
        }
    } else {
        if (!owner)
            return;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = col_w + j * 16 + l16e;
            const bool cv = col < N;
            const float bj = (out.bias && cv) ? out.bias[col] : 0.0f;
#pragma unroll
            for (int i = 0; i < FM; ++i) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = row_w + i * 16 + ge * 4 + r;
                    if (cv && row < M) {
                        const float v = apply_act(res[i][j][r] + bj, out.act);
                        const int64_t idx = (int64_t)(row - out.row0) * out.ld + (col - out.col0);
                        if (out.bf16)
                            static_cast<unsigned short*>(out.dst)[idx] = f32_to_bf16_rne(v);
                        else
                            static_cast<float*>(out.dst)[idx] = v;
                    }
                }
            }
        }
    }
}

// NTB: B is streamed -- the launch has a single row of tiles, so every
// element of B is read by exactly one workgroup (the decode regime: a
// matrix-vector-like product reads the weights once and reuses nothing, page
// "Tiling the hierarchy", failure regimes) -- and its transfers carry the
// non-temporal policy.  Measured on the 16 x 28672 x 8192 decode it lifts the
// weight stream by 3-5 %; where tiles of other rows re-read B through L2 the
// same policy costs 6-19 %, so it is never used there.
template <int BM, int BN, int BK, int WGM, int WGN, int ST, bool NTB, bool F32, int WK>
__global__ void __launch_bounds__(64 * WGM * WGN * WK)
gemm_tiled_dma_kernel(GemmParams p)
{
    __shared__ u32x4_t lds[ST * TiledDma<BM, BN, BK, WGM, WGN, ST, F32, WK>::STAGE_BYTES / 16];
    int tile, tm, tn, split;
    map_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tile, tm, tn, split);
    const int kbeg = split * p.kps;
    const int kend = min(p.K, kbeg + p.kps);
    dma_tile<BM, BN, BK, WGM, WGN, ST, NTB, F32, WK>(p, lds, tm, tn, kbeg, kend, out_spec(p, split));
}

// Data-parallel tiles plus a stream-K tail (page "Compilers and Kernel
// Languages", "A different tile for every shape": the order and the way tiles
// are handed to compute units is a choice of its own).  Blocks below sk_dp
// each run one whole tile, the first sk_dp tiles of the scheduling order
// (full rounds of the machine).  The sk_g blocks after them split the
// remaining sk_tail tiles' K steps evenly: each takes a contiguous range of
// (tile, K step) iterations, which covers the end of one tile, possibly whole
// tiles, and the start of another.  A piece that is a whole tile goes through
// the epilogue into C; any other piece writes its raw fp32 sums to its slot,
// and streamk_fixup adds a tile's pieces in K order afterwards (no flags, no
// atomics: the kernel boundary orders the two passes, and the sums do not
// depend on timing).
// One piece: iterations [it, it + n) of tile j (scheduling order), n <= ks.
template <int BM, int BN, int BK, int WGM, int WGN, int ST>
__device__ __forceinline__ void streamk_piece(const GemmParams& p, u32x4_t* lds, int64_t it, int64_t end, int64_t g)
{
    const int64_t G = p.sk_g, ks = p.sk_ks, dp = p.sk_dp;
    const int64_t I = (int64_t)p.sk_tail * ks;
    const int64_t j = it / ks;
    const int64_t kb = it - j * ks;
    const int64_t ke = min(ks, kb + (end - it));
    int tm, tn;
    tile_coords((int)j, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    OutSpec out = out_spec(p, 0);
    if (kb != 0 || ke != ks) {
        // a piece of a tail tile: raw sums to its slot
        const int64_t jt = j - dp;
        const int64_t piece = g - sk_owner(jt * ks, I, G);
        out = OutSpec{p.ws + (jt * p.sk_smax + piece) * (int64_t)(BM * BN), nullptr, 0, 0, tm * BM, tn * BN,
                      (int64_t)BN};
    }
    const int kend = ke * BK < (int64_t)p.K ? (int)(ke * BK) : p.K;
    dma_tile<BM, BN, BK, WGM, WGN, ST, false>(p, lds, tm, tn, (int)(kb * BK), kend, out);
}

template <int BM, int BN, int BK, int WGM, int WGN, int ST>
__global__ void __launch_bounds__(64 * WGM * WGN)
gemm_streamk_kernel(GemmParams p)
{
    __shared__ u32x4_t lds[ST * TiledDma<BM, BN, BK, WGM, WGN, ST>::STAGE_BYTES / 16];
    const int bid = blockIdx.x;
    if (bid < p.sk_dp) {
        int tile, tm, tn, split;
        map_block(bid, p.sk_dp, p.tiles_m, p.tiles_n, p.group_m, tile, tm, tn, split);
        dma_tile<BM, BN, BK, WGM, WGN, ST, false>(p, lds, tm, tn, 0, p.K, out_spec(p, 0));
        return;
    }
    // iterations (tile, K step) in scheduling order; this block's share of the
    // tail is fewer than one tile's K steps (the tail has fewer tiles than a
    // round has blocks), so it touches at most two tiles
    const int64_t G = p.sk_g, ks = p.sk_ks, dp = p.sk_dp;
    const int64_t I = (int64_t)p.sk_tail * ks;
    const int64_t g = bid - dp;
    const int64_t it = dp * ks + sk_start(g, I, G);
    const int64_t end = dp * ks + sk_start(g + 1, I, G);
    if (it >= end)
        return;
    streamk_piece<BM, BN, BK, WGM, WGN, ST>(p, lds, it, end, g);
    const int64_t next = (it / ks + 1) * ks;             // first iteration of the next tile
    if (next < end) {
        __syncthreads();   // the next piece's transfers overwrite the LDS this one's epilogue used
        streamk_piece<BM, BN, BK, WGM, WGN, ST>(p, lds, next, end, g);
    }
}

}  // namespace tg
