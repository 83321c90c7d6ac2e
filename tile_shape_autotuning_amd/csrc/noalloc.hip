// gemm_bias_act_noalloc: the fused GEMM for callers that cannot allocate
// device memory (code under graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  The only device memory the library itself needs
// for a call is the split-K partial-sum slabs; here they live in one
// file-scope device array of fixed size instead of the grown-on-demand
// workspace, so a call makes no hipMalloc, no hipFree and no allocating
// library call, and never tunes (tuning allocates operand copies).
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>
#include <string>

#include "runtime.hpp"
#include "select.hpp"

namespace tg {

// 32 MiB of fp32 partial sums per GPU: split_k x M x N floats (each split's
// slab rounded up to 64 floats) up to 8,388,608 floats -- e.g. four splits of
// a 1000 x 1000 output, or two of a 16 x 28672 one many times over.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

// The array's device address on each GPU (each holds its own copy), looked
// up once per device with that device current.  On the host the name
// `scratch` is only a stand-in and is never passed to a kernel or a copy.
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static float* g_scratch_ptr[kMaxDevices] = {};
// calls on one device take this lock while their kernels are queued, so the
// GEMM and the second pass of one call stay adjacent on a shared stream
static std::mutex g_scratch_call_mu[kMaxDevices];

static int scratch_for_device(float** out, int* dev_out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return set_hip_error(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return set_error(TG_E_UNSUPPORTED, "device index beyond the no-allocation entry point's table");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return set_hip_error(e, "hipGetSymbolAddress(scratch)");
        if (!p)
            return set_error(TG_E_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = static_cast<float*>(p);
    }
    *out = g_scratch_ptr[dev];
    *dev_out = dev;
    return TG_OK;
}

}  // namespace tg

using namespace tg;

extern "C" {

size_t tg_noalloc_scratch_bytes(void) { return kScratchBytes; }

int gemm_bias_act_noalloc(int64_t M, int64_t N, int64_t K, const void* A, const void* B, const float* bias,
                          void* C, int dtype, int act, const tg_cfg* cfg)
{
    int st = validate_call(M, N, K, A, B, C, dtype, act);
    if (st != TG_OK || M == 0 || N == 0)
        return st;
    tg_cfg c;
    if (cfg) {
        c = *cfg;
    } else {
        st = select_for_call(M, N, K, A, B, bias, dtype, act, false, &c);
        if (st != TG_OK)
            return st;
    }
    const size_t need = workspace_bytes_for(M, N, K, dtype, c);
    if (need > kScratchBytes)
        return set_error(TG_E_INVAL, "the workspace of this call (split-K partial sums, padded operands) needs " +
                                         std::to_string(need) + " bytes; the no-allocation entry point has " +
                                         std::to_string(kScratchBytes));
    float* ws = nullptr;
    int dev = 0;
    st = scratch_for_device(&ws, &dev);
    if (st != TG_OK)
        return st;
    const ExternalWorkspace ext{ws, kScratchBytes};
    std::lock_guard<std::mutex> lk(g_scratch_call_mu[dev]);
    return launch_cfg(M, N, K, A, B, bias, C, dtype, act, c, current_stream(), cfg == nullptr, &ext);
}

}  // extern "C"
