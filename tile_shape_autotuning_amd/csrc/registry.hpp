// Kernel registry: one entry per compiled kernel instantiation.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/tilegemm.h"
#include "kernels/common.hpp"

namespace tg {

typedef hipError_t (*LaunchFn)(const GemmParams& p, int blocks, hipStream_t stream);

// What the compiler allotted (from its resource remarks at build time; -1 = unknown).
struct KernelResources {
    int vgpr, agpr, scratch, lds, occupancy;
};

struct KernelEntry {
    int in_bf16;        // 1: bf16 operands, 0: fp32 operands
    tg_cfg cfg;         // split_k: the compiled K-group count of a sliced-K kernel, else 0 (a run-time value)
    LaunchFn launch;
    int threads;
    KernelResources res;
    // the same kernel reading B with the non-temporal policy, for launches
    // with a single row of tiles (B read exactly once); null if not built
    LaunchFn launch_stream_b;
};


// all entries, sorted by (in_bf16, cfg)
const KernelEntry* registry_begin();
const KernelEntry* registry_end();
const KernelEntry* find_kernel(int dtype, const tg_cfg& c);

}  // namespace tg
