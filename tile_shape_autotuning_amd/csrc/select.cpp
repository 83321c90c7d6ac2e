// Tile selection rules (host only).
//
// Candidate space and feasibility filter: page "Tile Selection: Cost Models
// Against Measurement", "The structure of the search space" -- the block
// tile, reduction step and per-thread (here per-wave) tile are the free
// parameters; resource limits that can be checked without generating or
// running any code bound the space: both panels must fit in on-chip memory,
// the accumulators must fit in registers, and the tile must leave the device
// filled.  On MI355X
// these become: LDS per workgroup and per CU (160 KiB), 256 accumulator and
// 512 unified VGPR+AGPR registers per lane, 8 wave slots per SIMD, whole
// 16x16 MFMA tiles per wave, K step a multiple of the MFMA K.
//
// Cost model: same page, "Analytical models and where they break" (per-block
// traffic eb*K*(BM+BN), work 2*BM*BN*K, grid traffic = per-block x blocks,
// time bounded by the busier of compute and memory, with corrections for
// occupancy, pipeline fill and the tail) and page "Compilers and Kernel
// Languages", "Workshop" (HBM traffic divided by g, compute divided by wave
// efficiency and tile efficiency, time = the larger).  The H100 replica mode
// reproduces that page's model; the MI355X mode adds the CU/SIMD occupancy,
// pipeline-fill, output-store and split-K (slabs, second pass) terms.  Every
// expression below is in the same order as the selection rules the tests
// compare against.
#include "select.hpp"

#include <algorithm>
#include <cmath>
#include <mutex>

namespace tg {

tg_device_desc mi355x_desc()
{
    tg_device_desc d{};
    d.mode = 0;
    d.n_cu = 256;
    d.simds = 4;
    d.lds_cu = 163840;
    d.lds_block = 163840;
    d.max_threads = 1024;
    d.waves_max = 8;
    d.blocks_max = 32;
    d.vgpr_max = 512;
    d.acc_max = 256;
    d.r0 = 24;
    d.peak_bf16 = 2516.6e12;
    d.peak_f32 = 157.3e12;
    d.bw = 8.0e12;
    d.a_ref = 16384.0;
    d.c_fill = 2.0;
    d.t0 = 4.0e-6;
    d.unaligned_eff = 0.125;
    d.lat_mem = 2.0e-6;
    d.cu_bw = 50.0e9;
    d.lds_bw_cu = 192.0e9;
    d.lat_step = 1.25e-6;
    d.lat_l2 = 0.3e-6;
    d.l2_bytes = 32.0e6;
    d.w1_eff = 0.35;
    d.skinny_eff = 0.75;
    d.hbm_eff = 0.9125;
    d.sliced_eff = 1.0;
    return d;
}

tg_device_desc h100_replica_desc()
{
    tg_device_desc d{};
    d.mode = 1;
    d.n_cu = 132;
    d.simds = 1;
    d.lds_cu = 233472;
    d.lds_block = 233472;
    d.max_threads = 1024;
    d.waves_max = 8;
    d.blocks_max = 1;
    d.vgpr_max = 1 << 30;
    d.acc_max = 1 << 30;
    d.r0 = 0;
    d.peak_bf16 = 989e12;
    d.peak_f32 = 989e12;
    d.bw = 3.35e12;
    d.a_ref = 16384.0;
    d.c_fill = 0.0;
    d.t0 = 0.0;
    d.unaligned_eff = 1.0;
    d.lat_mem = 0.0;
    d.cu_bw = 0.0;
    d.lds_bw_cu = 0.0;
    d.lat_step = 0.0;
    d.w1_eff = 1.0;
    d.skinny_eff = 1.0;
    d.hbm_eff = 1.0;
    d.sliced_eff = 1.0;
    return d;
}

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool cfg_less(const tg_cfg& a, const tg_cfg& b)
{
    const int32_t x[8] = {a.kind, a.bm, a.bn, a.bk, a.wgm, a.wgn, a.stages, a.split_k};
    const int32_t y[8] = {b.kind, b.bm, b.bn, b.bk, b.wgm, b.wgn, b.stages, b.split_k};
    return std::lexicographical_compare(x, x + 8, y, y + 8);
}

bool cfg_equal(const tg_cfg& a, const tg_cfg& b)
{
    return a.kind == b.kind && a.bm == b.bm && a.bn == b.bn && a.bk == b.bk && a.wgm == b.wgm &&
           a.wgn == b.wgn && a.stages == b.stages && a.split_k == b.split_k;
}

int in_bytes(int dtype) { return dtype == TG_F32 ? 4 : 2; }
int out_bytes(int dtype) { return dtype == TG_BF16 ? 2 : 4; }

bool shape_aligned(int64_t N, int64_t K, int dtype)
{
    const int64_t vec = dtype == TG_F32 ? 4 : 8;
    return K % vec == 0 && N % vec == 0;
}

int64_t pad_extent(int64_t x, int dtype)
{
    const int64_t vec = dtype == TG_F32 ? 4 : 8;
    return (x + vec - 1) / vec * vec;
}

bool padded_path(int64_t N, int64_t K, int dtype, const tg_cfg& c, const tg_device_desc& d)
{
    return d.mode == 0 && c.kind == TG_KIND_TILED && !shape_aligned(N, K, dtype);
}

// the kernels that move panels straight into LDS: the tiled and sliced-K
// kinds (fp32 and bf16) and stream-K (bf16 only)
static bool dma_kind(const tg_cfg& c, int dtype)
{
    return c.kind == TG_KIND_TILED || c.kind == TG_KIND_SLICEDK || (c.kind == TG_KIND_STREAMK && dtype != TG_F32);
}

int64_t cta_splits(const tg_cfg& c) { return c.kind == TG_KIND_SLICEDK ? 1 : c.split_k; }
int64_t k_groups(const tg_cfg& c) { return c.kind == TG_KIND_SLICEDK ? c.split_k : 1; }
int64_t waves_per_block(const tg_cfg& c) { return (int64_t)c.wgm * c.wgn * k_groups(c); }

// ------------------------------------------------------------------ space
static const int kWaveGrids[6][2] = {{1, 1}, {1, 2}, {2, 1}, {2, 2}, {2, 4}, {4, 2}};
static const int kSplits[5] = {1, 2, 4, 8, 16};
static const int kUnaligned[3][4] = {{32, 32, 1, 1}, {64, 64, 2, 2}, {128, 128, 2, 2}};

static std::vector<tg_cfg> build_space(int dtype, int mode)
{
    std::vector<tg_cfg> out;
    if (mode == 1) {
        const int t[4] = {32, 64, 128, 256};
        for (int bm : t)
            for (int bn : t)
                out.push_back(tg_cfg{TG_KIND_TILED, bm, bn, 64, 1, 1, 1, 1});
        return out;
    }
    std::vector<int> ms, ns, bks, sts;
    // 16-row tiles: a 16-row decode wastes no MFMA rows; the reduction step
    // spans 64, 128 or 256 bytes of an A row; the direct-to-LDS kernel keeps
    // 2 to 8 stages in flight
    if (dtype == TG_F32) {
        ms = {16, 32, 64, 128};
        ns = {32, 64, 128};
        bks = {16, 32, 64};
    } else {
        ms = {16, 32, 64, 128, 256};
        ns = {32, 64, 128, 256};
        bks = {32, 64, 128};
    }
    sts = {2, 3, 4, 6, 8};
    for (int bm : ms)
        for (int bn : ns)
            for (int bk : bks)
                for (const auto& w : kWaveGrids)
                    for (int st : sts)
                        for (int s : kSplits)
                            out.push_back(tg_cfg{TG_KIND_TILED, bm, bn, bk, w[0], w[1], st, s});
    if (dtype != TG_F32) {
        const int bms[4] = {16, 32, 48, 64}, ws[4] = {1, 2, 4, 8}, us[3] = {1, 2, 4};
        const int ss[6] = {1, 2, 4, 8, 16, 32};
        for (int bm : bms)
            for (int w : ws)
                for (int u : us)
                    for (int s : ss)
                        out.push_back(tg_cfg{TG_KIND_SKINNY, bm, 128, 32, w, 1, u, s});
    }
    const int ubk = dtype == TG_F32 ? 16 : 32;
    for (const auto& t : kUnaligned)
        for (int s : kSplits)
            out.push_back(tg_cfg{TG_KIND_UNALIGNED, t[0], t[1], ubk, t[2], t[3], 2, s});
    if (dtype != TG_F32) {
        // stream-K: the large tiles whose last partial round is worth spreading
        const int ts[2] = {128, 256}, wg[3][2] = {{2, 2}, {2, 4}, {4, 2}}, sts[3] = {2, 3, 4};
        for (int bm : ts)
            for (int bn : ts)
                for (const auto& w : wg)
                    for (int st : sts)
                        out.push_back(tg_cfg{TG_KIND_STREAMK, bm, bn, 64, w[0], w[1], st, 1});
    }
    {
        // sliced-K: small tiles whose K loop is a chain of short steps; 2 or 4
        // K groups per workgroup, each at least one slice of every stage
        const int sms[3] = {16, 32, 64}, sws[3][2] = {{1, 1}, {1, 2}, {2, 2}}, ssts[3] = {2, 3, 4}, sgs[2] = {2, 4};
        const std::vector<int> sns = dtype == TG_F32 ? std::vector<int>{32, 64} : std::vector<int>{64, 128};
        const std::vector<int> sbks = dtype == TG_F32 ? std::vector<int>{32, 64} : std::vector<int>{64, 128};
        for (int bm : sms)
            for (int bn : sns)
                for (int bk : sbks)
                    for (const auto& w : sws)
                        for (int st : ssts)
                            for (int g : sgs)
                                out.push_back(tg_cfg{TG_KIND_SLICEDK, bm, bn, bk, w[0], w[1], st, g});
    }
    return out;
}

const std::vector<tg_cfg>& space(int dtype, const tg_device_desc& d)
{
    static std::once_flag once;
    static std::vector<tg_cfg> spaces[2][3];
    std::call_once(once, [] {
        for (int m = 0; m < 2; ++m)
            for (int dt = 0; dt < 3; ++dt)
                spaces[m][dt] = build_space(dt, m);
    });
    const int m = d.mode == 1 ? 1 : 0;
    const int dt = (dtype >= 0 && dtype <= 2) ? dtype : 0;
    return spaces[m][dt];
}

bool in_space(int dtype, const tg_device_desc& d, const tg_cfg& c)
{
    const auto& sp = space(dtype, d);
    return std::binary_search(sp.begin(), sp.end(), c, cfg_less);
}

// ------------------------------------------------------------------ resources
int64_t lds_bytes(const tg_cfg& c, int dtype)
{
    const int64_t eb = in_bytes(dtype);
    if (c.kind == TG_KIND_SKINNY)
        return c.wgm > 1 ? (int64_t)c.wgm * c.bm * 128 * 4 : 0;
    // the register-staged fp32 kernel pads B rows by 4 floats
    const int64_t pad_b = dtype == TG_F32 && !dma_kind(c, dtype) ? 4 : 0;
    return (int64_t)c.stages * ((int64_t)c.bm * c.bk + (int64_t)c.bk * (c.bn + pad_b)) * eb;
}

int64_t acc_regs(const tg_cfg& c)
{
    if (c.kind == TG_KIND_SKINNY)
        return (int64_t)(c.bm / 16) * 32;
    return (int64_t)(c.bm / c.wgm) * (c.bn / c.wgn) / 64;
}

int64_t vgpr_estimate(const tg_cfg& c, int dtype, const tg_device_desc& d)
{
    if (c.kind == TG_KIND_SKINNY) {
        const int64_t mt = c.bm / 16;
        return 64 * (int64_t)c.stages + 8 * (int64_t)c.stages * mt + 32 * mt + d.r0;
    }
    const int64_t threads = 64 * (int64_t)c.wgm * c.wgn;
    const int64_t eb = in_bytes(dtype);
    const int64_t frag = 4 * ((c.bm / c.wgm) / 16 + (c.bn / c.wgn) / 16);
    if (dma_kind(c, dtype))
        return acc_regs(c) + frag + d.r0;   // panels go global -> LDS directly: no staging registers
    const int64_t chunks_a = (int64_t)c.bm * c.bk * eb / 16;
    int64_t stage = 4 * cdiv(chunks_a, threads);
    if (dtype == TG_F32)
        stage += 4 * cdiv((int64_t)c.bk * c.bn / 4, threads);
    else
        stage += 32 * cdiv((int64_t)c.bk * c.bn / 64, threads);
    return acc_regs(c) + frag + stage + d.r0;
}

int64_t waves_per_simd(const tg_cfg& c, int dtype, const tg_device_desc& d)
{
    const int64_t v = vgpr_estimate(c, dtype, d);
    const int64_t v8 = cdiv(v, 8) * 8;
    return v8 > 0 ? std::min<int64_t>(d.waves_max, d.vgpr_max / v8) : d.waves_max;
}

int64_t blocks_per_cu(const tg_cfg& c, int dtype, const tg_device_desc& d)
{
    const int64_t w = waves_per_block(c);
    int64_t b = std::min<int64_t>(d.blocks_max, (d.simds * waves_per_simd(c, dtype, d)) / w);
    const int64_t lds = lds_bytes(c, dtype);
    if (lds > 0)
        b = std::min<int64_t>(b, d.lds_cu / lds);
    return b;
}

int64_t waves_per_simd_alloc(int64_t vgpr, int64_t agpr, const tg_device_desc& d)
{
    const int64_t regs = cdiv(cdiv(vgpr, 4) * 4 + agpr, 8) * 8;
    return regs > 0 ? std::min<int64_t>(d.waves_max, d.vgpr_max / regs) : d.waves_max;
}

int64_t resident_blocks(const tg_cfg& c, int dtype, const tg_device_desc& d)
{
    Alloc a;
    if (d.mode != 0 || !compiled_alloc(dtype, c, &a) || a.vgpr < 0 || a.agpr < 0 || a.lds < 0)
        return blocks_per_cu(c, dtype, d);
    const int64_t w = waves_per_block(c);
    int64_t b = std::min<int64_t>(d.blocks_max, (d.simds * waves_per_simd_alloc(a.vgpr, a.agpr, d)) / w);
    if (a.lds > 0)
        b = std::min<int64_t>(b, d.lds_cu / a.lds);
    return b;
}

int64_t transfers_per_wave(const tg_cfg& c, int dtype)
{
    const int64_t inst = ((int64_t)c.bm + c.bn) * c.bk * in_bytes(dtype) / 1024;
    return cdiv(inst, waves_per_block(c));
}

int64_t k_per_split(const tg_cfg& c, int64_t K)
{
    const int64_t unit = c.kind == TG_KIND_SKINNY ? 32 : c.bk;
    return cdiv(cdiv(K, cta_splits(c)), unit) * unit;
}

int check_static(int dtype, const tg_cfg& c, const tg_device_desc& d)
{
    const int64_t w = waves_per_block(c);
    if (64 * w > d.max_threads)
        return R_WAVES;
    if (c.kind != TG_KIND_SKINNY) {
        // each K group takes whole MFMA slices of every stage
        const int64_t kstep = (dtype == TG_F32 ? 16 : 32) * k_groups(c);
        if (c.bm % (16 * c.wgm) || c.bn % (16 * c.wgn) || c.bk % kstep)
            return R_DIV;
    }
    if (lds_bytes(c, dtype) > d.lds_block)
        return R_LDS;
    // the sliced-K kind's groups add their sums through the stage buffers
    if (k_groups(c) > 1 && (k_groups(c) - 1) * c.bm * c.bn * 4 > lds_bytes(c, dtype))
        return R_LDS;
    // the direct-to-LDS kernel keeps ST stages of transfers in flight after its
    // prologue; a wave's memory counter tracks at most 63 (MI355X only)
    if (d.mode == 0 && dma_kind(c, dtype) && c.stages * transfers_per_wave(c, dtype) > 63)
        return R_INFLIGHT;
    if (acc_regs(c) > d.acc_max)
        return R_ACC;
    if (vgpr_estimate(c, dtype, d) > d.vgpr_max)
        return R_VGPR;
    if (blocks_per_cu(c, dtype, d) < 1)
        return R_OCC;
    return OK;
}

int check(int64_t M, int64_t N, int64_t K, int dtype, const tg_cfg& c, const tg_device_desc& d)
{
    if (dtype != TG_F32 && dtype != TG_BF16 && dtype != TG_BF16_F32OUT)
        return R_DTYPE;
    if (M < 1 || N < 1 || K < 0)
        return R_SHAPE;
    if (!in_space(dtype, d, c))
        return R_SPACE;
    if ((c.kind == TG_KIND_SKINNY || c.kind == TG_KIND_STREAMK) && dtype == TG_F32)
        return R_DTYPE;
    // a stream-K workgroup spreads K steps: K = 0 has none to spread
    if (c.kind == TG_KIND_STREAMK && K == 0)
        return R_SHAPE;
    const bool aligned = shape_aligned(N, K, dtype);
    if (d.mode == 0) {
        if (c.kind == TG_KIND_UNALIGNED && aligned)
            return R_ALIGN;
        // the tiled kind takes an unaligned shape through the padded path
        if (c.kind != TG_KIND_UNALIGNED && c.kind != TG_KIND_TILED && !aligned)
            return R_ALIGN;
    }
    const int64_t Ke = padded_path(N, K, dtype, c, d) ? pad_extent(K, dtype) : K;
    if (c.kind == TG_KIND_SKINNY && (M > 64 || c.bm != 16 * cdiv(M, 16)))
        return R_SHAPE;
    const int st = check_static(dtype, c, d);
    if (st != OK)
        return st;
    // the register cliff (page "Autotuning & cost models", the search space:
    // a tile past the register file spills and falls off a cliff): a
    // configuration whose compiled kernel spills is not a candidate
    Alloc a;
    if (d.mode == 0 && compiled_alloc(dtype, c, &a) && a.scratch > 0)
        return R_SPILL;
    if (resident_blocks(c, dtype, d) < 1)
        return R_OCC;
    // without a partial last round the stream-K kind is the data-parallel one
    if (c.kind == TG_KIND_STREAMK && streamk_plan(M, N, K, c, d).tail == 0)
        return R_SHAPE;
    if (cta_splits(c) > 1) {
        if (Ke == 0 || cdiv(Ke, k_per_split(c, Ke)) != c.split_k)
            return R_SPLIT;
    }
    return OK;
}

std::vector<tg_cfg> enumerate_feasible(int64_t M, int64_t N, int64_t K, int dtype, const tg_device_desc& d)
{
    std::vector<tg_cfg> out;
    for (const tg_cfg& c : space(dtype, d))
        if (check(M, N, K, dtype, c, d) == OK)
            out.push_back(c);
    return out;
}

// ------------------------------------------------------------------ geometry
void grid(int64_t M, int64_t N, int64_t K, const tg_cfg& c, int64_t* tiles, int64_t* blocks, const tg_device_desc* d)
{
    const int64_t t = cdiv(M, c.bm) * cdiv(N, c.bn);
    *tiles = t;
    if (c.kind == TG_KIND_STREAMK) {
        *blocks = streamk_plan(M, N, K, c, d ? *d : mi355x_desc()).blocks;
        return;
    }
    *blocks = t * cta_splits(c);
}

int64_t sk_owner_host(int64_t x, int64_t I, int64_t G) { return ((x + 1) * G - 1) / I; }

SkPlan streamk_plan(int64_t M, int64_t N, int64_t K, const tg_cfg& c, const tg_device_desc& d)
{
    SkPlan p{};
    p.tiles = cdiv(M, c.bm) * cdiv(N, c.bn);
    p.G = (int64_t)d.n_cu * std::max<int64_t>(1, resident_blocks(c, TG_BF16, d));
    p.tail = p.tiles % p.G;
    p.dp = p.tiles - p.tail;
    p.ks = cdiv(K, c.bk);
    // never more stream-K workgroups than tail iterations: every one then has
    // at least one, and the pieces of a tile come from consecutive workgroups
    p.wgs = std::min(p.G, p.tail * p.ks);
    p.blocks = p.dp + (p.tail > 0 ? p.wgs : 0);
    if (p.tail > 0 && p.ks > 0) {
        const int64_t I = p.tail * p.ks;
        p.segmax = 1;
        for (int64_t j = 0; j < p.tail; ++j) {
            const int64_t first = sk_owner_host(j * p.ks, I, p.wgs);
            const int64_t n = sk_owner_host((j + 1) * p.ks - 1, I, p.wgs) - first + 1;
            p.smax = std::max(p.smax, n);
            if (n >= 2)
                p.pieces += n;
            // a tile that starts inside a workgroup's range: that workgroup
            // runs the end of the previous tile and the start of this one
            if (j > 0 && first * I / p.wgs != j * p.ks)
                p.segmax = 2;
        }
    }
    return p;
}

// ------------------------------------------------------------------ cost model
static int64_t line_bytes(int64_t x) { return cdiv(x, (int64_t)128) * 128; }

// The roofline model of page "Compilers and Kernel Languages" ("Workshop"):
// the larger of the compute time at the wave, SIMD, tile and fill
// efficiencies and the memory time of the traffic, plus split-K workspace.
static double model_page(int64_t K, int dtype, const tg_cfg& c, const tg_device_desc& d, int64_t eb, double peak,
                         double flops, double compulsory, int64_t tiles, int64_t units, int64_t w, int64_t bcu)
{
    const int64_t par_need = std::max<int64_t>(1, d.simds / w);
    const int64_t par = std::min(bcu, par_need);
    const int64_t slots = (int64_t)d.n_cu * par;
    const int64_t rounds = cdiv(units, slots);
    const double wave_eff = (double)units / (double)(rounds * slots);
    const double simd_eff = std::min(1.0, (double)(par * w) / (double)d.simds);
    const double tile_eff = std::min(1.0, 0.5 + 0.5 * (double)((int64_t)c.bm * c.bn) / d.a_ref);
    const int64_t ktiles = cdiv(k_per_split(c, K), c.bk);
    const double fill_eff = ktiles > 0 ? (double)ktiles / ((double)ktiles + d.c_fill) : 1.0;
    double eff = wave_eff * simd_eff * tile_eff * fill_eff;
    if (c.kind == TG_KIND_UNALIGNED)
        eff = eff * d.unaligned_eff;
    const double t_c = flops / (peak * eff);
    const double raw = (double)tiles * (double)eb * (double)K * (double)(c.bm + c.bn);
    const double g = std::sqrt((double)std::min<int64_t>(units, (int64_t)d.n_cu * bcu));
    const double ws = cta_splits(c) > 1 ? 8.0 * (double)tiles * (double)c.bm * (double)c.bn * (double)c.split_k : 0.0;
    const double t_m = (std::max(compulsory, raw / g) + ws) / d.bw;
    return std::max(t_c, t_m) + d.t0;
}

// Split-K (page "Compilers and Kernel Languages", "A different tile for a
// different shape"): the fp32 partial-sum slabs, one M x N slab per split
// (the padded path writes them with any split) ...
static double splitk_slabs(int64_t M, int64_t N, const tg_cfg& c, bool padded = false)
{
    return (cta_splits(c) > 1 || padded) ? 4.0 * (double)c.split_k * (double)M * (double)N : 0.0;
}

// ... and the second pass: one more launch reading every slab once and
// writing C at the HBM rate.
static double splitk_pass(int64_t M, int64_t N, int64_t ec, const tg_cfg& c, const tg_device_desc& d,
                          bool padded = false)
{
    if (cta_splits(c) <= 1 && !padded)
        return 0.0;
    return (splitk_slabs(M, N, c, padded) + (double)ec * (double)M * (double)N) / (d.bw * d.hbm_eff) + d.t0;
}

// MI355X: the roofline of "Analytical models and where they break" per CU and
// per K step.  One K step of the blocks resident on a CU takes the longest of
// their MFMA work on the SIMDs their waves occupy, their LDS traffic, their
// L2-to-CU traffic (rows narrower than a cache line cost a line) and the
// memory latency over the pipeline depth; a lone wave on a SIMD issues its
// MFMAs and LDS reads in order (w1_eff; the global-to-LDS transfers run
// without it).  Blocks run in rounds of n_cu x resident, the partial
// last round spread out, each round starting with one latency; the HBM time of
// the traffic bounds it from below (with split-K that traffic includes
// writing the partial-sum slabs). The output stores come after each block's
// K loop and add their HBM time to the per-CU time; split-K adds the second
// pass.
static double model_cu(int64_t M, int64_t N, int64_t K, int dtype, const tg_cfg& c, const tg_device_desc& d,
                       int64_t eb, int64_t ec, double peak, double compulsory, int64_t tiles, int64_t units,
                       int64_t w, int64_t bcu, bool padded = false)
{
    const int64_t ktiles = cdiv(k_per_split(c, K), c.bk);
    const int64_t wm = c.bm / c.wgm, wn = c.bn / c.wgn;
    const double simd_peak = peak / (double)((int64_t)d.n_cu * d.simds);
    const double f_step = 2.0 * (double)c.bm * (double)c.bn * (double)c.bk;
    // fragment reads (each K group reads only its own slices, so the reads of a
    // step are those of one group's wgm x wgn waves) plus the transfers' writes
    const int64_t wo = (int64_t)c.wgm * c.wgn;
    const double lds_step = (double)(c.bk * eb * (wo * (wm + wn) + c.bm + c.bn));
    const int64_t qw = dma_kind(c, dtype) ? std::min<int64_t>(c.bn, 64) : c.bn;
    double l2_step = (double)(c.bm * line_bytes(c.bk * eb) + c.bk * (c.bn / qw) * line_bytes(qw * eb));
    if (c.kind == TG_KIND_UNALIGNED)
        l2_step = l2_step / d.unaligned_eff;
    const int64_t depth = dma_kind(c, dtype) ? std::max<int64_t>(1, c.stages - 1) : 1;
    const double lat = compulsory > d.l2_bytes ? d.lat_step : d.lat_l2;

    auto step = [&](int64_t res) {
        const int64_t busy = std::min<int64_t>(d.simds, res * w);
        double issue = (double)res * f_step / (simd_peak * (double)busy);
        issue = std::max(issue, (double)res * lds_step / d.lds_bw_cu);
        if (res * w <= d.simds)
            issue = issue / d.w1_eff;
        if (c.kind == TG_KIND_SLICEDK)
            issue = issue / d.sliced_eff;
        double t = std::max(issue, (double)res * l2_step / d.cu_bw);
        return std::max(t, lat / (double)depth);
    };
    const int64_t slots = (int64_t)d.n_cu * bcu;
    if (c.kind == TG_KIND_STREAMK) {
        // full rounds of whole tiles, then the tail's K steps spread evenly
        // over a round of workgroups; the pieces of split tiles are stored as
        // fp32 and read back once by the second pass.  Every piece is a run
        // of the tile loop of its own, like a whole tile: it starts with one
        // latency and issues the stages of zero-filling transfers past its K
        // range (a stream-K workgroup runs up to segmax pieces)
        const SkPlan sp = streamk_plan(M, N, K, c, d);
        const int64_t dp_rounds = sp.dp / slots;
        const int64_t sk_steps = sp.tail > 0 ? cdiv(sp.tail * sp.ks, sp.wgs) : 0;
        double t_cu = (double)(dp_rounds * ktiles + sk_steps) * step(bcu);
        t_cu = t_cu + (double)(dp_rounds + sp.segmax) * lat;
        const int64_t runs_cu = dp_rounds * bcu + (sp.tail > 0 ? cdiv(sp.wgs, (int64_t)d.n_cu) * sp.segmax : 0);
        t_cu = t_cu + (double)runs_cu * (double)c.stages * l2_step / d.cu_bw;
        const double pieces = 4.0 * (double)c.bm * (double)c.bn * (double)sp.pieces;
        const double raw = (double)tiles * (double)eb * (double)K * (double)(c.bm + c.bn);
        const double g = std::sqrt((double)std::min<int64_t>(tiles, slots));
        const double t_hbm = (std::max(compulsory, raw / g) + pieces) / (d.bw * d.hbm_eff);
        t_cu = t_cu + ((double)ec * (double)M * (double)N + pieces) / (d.bw * d.hbm_eff);
        double fix = 0.0;
        if (sp.pieces > 0)
            fix = (pieces + (double)ec * (double)c.bm * (double)c.bn * (double)sp.tail) / (d.bw * d.hbm_eff) + d.t0;
        return std::max(t_cu, t_hbm) + fix + d.t0;
    }
    const int64_t full = units / slots;
    const int64_t rem = units - full * slots;
    double t_cu = (double)(full * ktiles) * step(bcu);
    if (rem > 0)
        t_cu = t_cu + (double)ktiles * step(cdiv(rem, (int64_t)d.n_cu));
    const int64_t rounds = full + (rem > 0 ? 1 : 0);
    t_cu = t_cu + (double)rounds * lat;
    // blocks a CU runs over all rounds
    const int64_t per_cu = full * bcu + (rem > 0 ? cdiv(rem, (int64_t)d.n_cu) : 0);
    // the direct-to-LDS kernels keep every stage the same: each block also
    // issues the transfers of the ST tiles past the end of its K range, which
    // the range check turns into zeros -- address-unit time at the L2-to-CU
    // rate, no traffic (they matter where the K loop is short)
    if (dma_kind(c, dtype))
        t_cu = t_cu + (double)per_cu * (double)c.stages * l2_step / d.cu_bw;
    // sliced-K: after its K loop a tile's groups 1 .. g-1 write their sums to
    // LDS and group 0 reads them back
    const double red = k_groups(c) > 1 ? 8.0 * (double)(k_groups(c) - 1) * (double)c.bm * (double)c.bn / d.lds_bw_cu
                                       : 0.0;
    t_cu = t_cu + (double)per_cu * red;
    const double raw = (double)tiles * (double)eb * (double)K * (double)(c.bm + c.bn);
    const double g = std::sqrt((double)std::min<int64_t>(units, slots));
    const double t_hbm = (std::max(compulsory, raw / g) + splitk_slabs(M, N, c, padded)) / (d.bw * d.hbm_eff);
    // every block stores its outputs (C, or its split-K slab) after its K
    // loop: those stores do not overlap the loop
    const double stores = (cta_splits(c) > 1 || padded) ? splitk_slabs(M, N, c, padded)
                                                        : (double)ec * (double)M * (double)N;
    t_cu = t_cu + stores / (d.bw * d.hbm_eff);
    return std::max(t_cu, t_hbm) + splitk_pass(M, N, ec, c, d, padded) + d.t0;
}

double model_time(int64_t M, int64_t N, int64_t K, int dtype, const tg_cfg& c, const tg_device_desc& d)
{
    const int64_t eb = in_bytes(dtype);
    const int64_t ec = out_bytes(dtype);
    const double peak = dtype == TG_F32 ? d.peak_f32 : d.peak_bf16;
    const double flops = 2.0 * (double)M * (double)N * (double)K;
    const double compulsory = (double)(eb * (M * K + K * N) + ec * M * N);
    int64_t tiles, units;
    grid(M, N, K, c, &tiles, &units, &d);
    const int64_t w = waves_per_block(c);
    const int64_t bcu = resident_blocks(c, dtype, d);

    if (c.kind == TG_KIND_SKINNY) {
        const double flops_pad = 2.0 * (double)c.bm * (double)N * (double)K;
        const double t_c = flops_pad / peak;
        const double ws = d.mode == 0 ? splitk_slabs(M, N, c)
                          : (c.split_k > 1 ? 8.0 * (double)c.bm * 128.0 * (double)tiles * (double)c.split_k : 0.0);
        const int64_t resident = std::min<int64_t>(units * w, (int64_t)d.n_cu * bcu * w);
        const double inflight = (double)resident * 64.0 * (double)c.stages * 8.0 * 16.0;
        const double bw_eff = std::min(1.0, inflight / (d.bw * d.lat_mem));
        const int64_t active = std::min<int64_t>(units, d.n_cu);
        const double bw = std::min(d.bw * bw_eff, (double)active * d.cu_bw);
        const double t_m = (compulsory + ws) / bw;
        const double t = std::max(t_c, t_m);
        if (d.mode == 0)
            return t / d.skinny_eff + splitk_pass(M, N, ec, c, d) + d.t0;
        return t + d.t0;
    }
    if (d.mode == 1)
        return model_page(K, dtype, c, d, eb, peak, flops, compulsory, tiles, units, w, bcu);
    if (padded_path(N, K, dtype, c, d)) {
        // the padded path: one launch copies the operands whose rows are
        // ragged into their padded forms (A when K is; B when N is, with K
        // rounded up -- a B with only K ragged is read in place, its missing
        // rows as zeros), each read once and written once; then the tiled
        // kind on the padded problem, its sums in slabs and an output pass
        // (priced as the split-K one) when N is ragged, since C's rows then
        // cannot take the kernel's 16-byte stores
        const int64_t Np = pad_extent(N, dtype), Kp = pad_extent(K, dtype);
        const bool pad_a = Kp != K, pad_b = Np != N;
        const double comp_p = (double)(eb * (M * Kp + Kp * Np) + ec * M * Np);
        const int64_t copied = (pad_a ? eb * (M * K + M * Kp) : 0) + (pad_b ? eb * (K * N + Kp * Np) : 0);
        const double copies = (double)copied / (d.bw * d.hbm_eff) + d.t0;
        return model_cu(M, Np, Kp, dtype, c, d, eb, ec, peak, comp_p, tiles, units, w, bcu, pad_b) + copies;
    }
    return model_cu(M, N, K, dtype, c, d, eb, ec, peak, compulsory, tiles, units, w, bcu);
}

bool model_choice(int64_t M, int64_t N, int64_t K, int dtype, const tg_device_desc& d, tg_cfg* out, double* t)
{
    bool found = false;
    double best = 0.0;
    for (const tg_cfg& c : space(dtype, d)) {
        if (check(M, N, K, dtype, c, d) != OK)
            continue;
        const double x = model_time(M, N, K, dtype, c, d);
        if (!found || x < best) {
            found = true;
            best = x;
            *out = c;
        }
    }
    if (found && t)
        *t = best;
    return found;
}

tg_cfg default_cfg(int64_t N, int64_t K, int dtype)
{
    if (!shape_aligned(N, K, dtype))
        return tg_cfg{TG_KIND_UNALIGNED, 64, 64, dtype == TG_F32 ? 16 : 32, 2, 2, 2, 1};
    if (dtype == TG_F32)
        return tg_cfg{TG_KIND_TILED, 128, 128, 32, 2, 2, 2, 1};
    return tg_cfg{TG_KIND_TILED, 128, 128, 64, 2, 2, 2, 1};
}

// Run-time dispatch over shape buckets (page "Tile Selection: Cost Models
// Against Measurement", "Hybrid strategies": a few tuned variants chosen at
// launch from the actual extents; "Selection is per device, and devices
// change": the batch-1 tile is not the batch-32 tile, so the buckets are
// narrow where M is small).  Up to 64 rows, M rounded up to the 16-row MFMA
// tile (the rows a kernel computes are the same across the bucket, and the
// skinny kind's row tile is exactly that); then 128 and 256.  A bucket's
// entry is tuned at its largest M.
int64_t bucket_m(int64_t M)
{
    if (M <= 0 || M > kBucketMaxM)
        return M;
    if (M <= 64)
        return cdiv(M, (int64_t)16) * 16;
    return M <= 128 ? 128 : 256;
}

}  // namespace tg
