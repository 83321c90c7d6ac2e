// Split-K workspaces: library-owned device memory for the fp32 partial sums
// of split-K calls, one buffer per (device, stream), grown on demand.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "runtime.hpp"

namespace tg {

// ------------------------------------------------------------------ workspace
// One split-K workspace per (device, stream): the slabs a GEMM writes are read
// by the second pass queued behind it on the same stream, so calls on
// different streams never touch each other's slabs and may run concurrently.
struct Workspace {
    float* ws = nullptr;
    size_t ws_bytes = 0;
};
static std::mutex g_ws_mu;
static std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

size_t workspace_bytes_for(int64_t M, int64_t N, const tg_cfg& c)
{
    if (c.split_k <= 1)
        return 0;
    return (size_t)c.split_k * (size_t)splitk_slab(M, N) * sizeof(float);
}

int ensure_workspace(size_t ws_bytes, hipStream_t stream, float** ws)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return set_hip_error(e, "hipGetDevice");
    std::lock_guard<std::mutex> lk(g_ws_mu);
    Workspace& w = g_ws[{dev, stream}];
    if (w.ws_bytes < ws_bytes) {
        // the old buffer may still be in use by kernels queued on this stream
        e = hipStreamSynchronize(stream);
        if (e != hipSuccess)
            return set_hip_error(e, "hipStreamSynchronize (workspace growth)");
        if (w.ws)
            (void)hipFree(w.ws);
        w.ws = nullptr;
        w.ws_bytes = 0;
        e = hipMalloc(&w.ws, ws_bytes);
        if (e != hipSuccess)
            return set_error(TG_E_NOMEM, std::string("split-K workspace: ") + hipGetErrorString(e));
        w.ws_bytes = ws_bytes;
    }
    *ws = w.ws;
    return TG_OK;
}

}  // namespace tg
