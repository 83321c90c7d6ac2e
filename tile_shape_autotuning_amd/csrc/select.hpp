// Host-only tile selection: candidate space, feasibility filter, cost model.
// Pure C++ (no HIP), compiled with -ffp-contract=off so that every float64
// operation happens exactly in the order written.
#pragma once

#include <cstdint>
#include <vector>

#include "../../include/tilegemm.h"

namespace tg {

enum Reason {
    OK = 0, R_DTYPE = 1, R_ALIGN = 2, R_SHAPE = 3, R_WAVES = 4, R_DIV = 5, R_LDS = 6,
    R_ACC = 7, R_VGPR = 8, R_OCC = 9, R_SPLIT = 10, R_SPACE = 11, R_INFLIGHT = 12, R_SPILL = 13
};

tg_device_desc mi355x_desc();
tg_device_desc h100_replica_desc();

bool cfg_less(const tg_cfg& a, const tg_cfg& b);
bool cfg_equal(const tg_cfg& a, const tg_cfg& b);

int in_bytes(int dtype);
int out_bytes(int dtype);
bool shape_aligned(int64_t N, int64_t K, int dtype);
// The padded path: on a shape that is not shape_aligned (MI355X rules), the
// tiled kind runs on zero-padded copies of the operands whose rows are ragged,
// K and N rounded up to whole 16-byte chunks (pad_extent); with N ragged it
// writes fp32 slabs and finishes in an output pass.
bool padded_path(int64_t N, int64_t K, int dtype, const tg_cfg& c, const tg_device_desc& d);
int64_t pad_extent(int64_t x, int dtype);

// canonical-order candidate space for a dtype
const std::vector<tg_cfg>& space(int dtype, const tg_device_desc& d);
bool in_space(int dtype, const tg_device_desc& d, const tg_cfg& c);

// Workgroups that share one tile's K range (split_k, except for the sliced-K
// kind, whose split_k groups live inside one workgroup), the K groups inside
// a workgroup (split_k for the sliced-K kind, else 1), and waves per workgroup.
int64_t cta_splits(const tg_cfg& c);
int64_t k_groups(const tg_cfg& c);
int64_t waves_per_block(const tg_cfg& c);

int64_t lds_bytes(const tg_cfg& c, int dtype);
int64_t acc_regs(const tg_cfg& c);
int64_t vgpr_estimate(const tg_cfg& c, int dtype, const tg_device_desc& d);
int64_t waves_per_simd(const tg_cfg& c, int dtype, const tg_device_desc& d);
int64_t blocks_per_cu(const tg_cfg& c, int dtype, const tg_device_desc& d);
int64_t transfers_per_wave(const tg_cfg& c, int dtype);

// What the compiler allotted to the kernel that serves a configuration (its
// resource remarks at build time).  compiled_alloc is defined by the kernel
// registry of the library (false when no kernel serves c) and returns false
// in programs built without one (the instantiation-set generator, which runs
// before any kernel exists).
struct Alloc {
    int vgpr, agpr, lds, scratch;
};
bool compiled_alloc(int dtype, const tg_cfg& c, Alloc* out);
// Waves of one kernel a SIMD holds with that allocation: the register file
// has vgpr_max registers per lane; a wave's share is its architectural VGPRs
// rounded up to 4, plus its AGPRs, rounded up to 8.
int64_t waves_per_simd_alloc(int64_t vgpr, int64_t agpr, const tg_device_desc& d);
// Workgroups resident on one CU, as the cost model counts them: from the
// compiled kernel's registers and LDS where it exists (MI355X rules), else
// the filter's estimate (blocks_per_cu).
int64_t resident_blocks(const tg_cfg& c, int dtype, const tg_device_desc& d);
int64_t k_per_split(const tg_cfg& c, int64_t K);

// shape-independent rules only (waves, divisibility, LDS, registers, occupancy)
int check_static(int dtype, const tg_cfg& c, const tg_device_desc& d);
int check(int64_t M, int64_t N, int64_t K, int dtype, const tg_cfg& c, const tg_device_desc& d);

// Launch geometry: output tiles and launched workgroups.  The stream-K kind's
// workgroup count depends on the device (d; NULL = MI355X defaults) and on K.
void grid(int64_t M, int64_t N, int64_t K, const tg_cfg& c, int64_t* tiles, int64_t* blocks,
          const tg_device_desc* d = nullptr);

// The stream-K kind's partition (see TG_KIND_STREAMK): G = CUs x resident
// workgroups; the first dp = tiles - tail tiles (tail = tiles mod G) run one
// workgroup each; the tail tiles' ks K steps each are spread over
// wgs = min(G, I) more workgroups, workgroup g taking iterations
// [g I / wgs, (g + 1) I / wgs) of I = tail * ks.  smax: most pieces any tail
// tile is split into; pieces: slots written (pieces of the tiles split in two
// or more).
struct SkPlan {
    // segmax: most pieces one stream-K workgroup runs (1, or 2 when its range
    // crosses a tile boundary)
    int64_t tiles, G, dp, tail, ks, wgs, smax, pieces, blocks, segmax;
};
SkPlan streamk_plan(int64_t M, int64_t N, int64_t K, const tg_cfg& c, const tg_device_desc& d);
// the workgroup that holds iteration x of I over G workgroups
int64_t sk_owner_host(int64_t x, int64_t I, int64_t G);
double model_time(int64_t M, int64_t N, int64_t K, int dtype, const tg_cfg& c, const tg_device_desc& d);
std::vector<tg_cfg> enumerate_feasible(int64_t M, int64_t N, int64_t K, int dtype, const tg_device_desc& d);
bool model_choice(int64_t M, int64_t N, int64_t K, int dtype, const tg_device_desc& d, tg_cfg* out, double* t);
tg_cfg default_cfg(int64_t N, int64_t K, int dtype);

// Shape buckets of the run-time dispatch: row counts up to kBucketMaxM share
// the entry of their bucket's largest M (16, 32, 48, 64, 128, 256); larger M
// keep their own.
constexpr int64_t kBucketMaxM = 256;
int64_t bucket_m(int64_t M);

}  // namespace tg
