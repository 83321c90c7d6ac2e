// Split-K workspaces: library-owned device memory for the fp32 partial sums
// of split-K calls, one buffer per (device, stream), grown on demand.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "runtime.hpp"
#include "select.hpp"

namespace tg {

// ------------------------------------------------------------------ workspace
// One split-K workspace per (device, stream): the slabs a GEMM writes are read
// by the second pass queued behind it on the same stream, so calls on
// different streams never touch each other's slabs and may run concurrently.
// Host threads that share a stream (every thread's default is the null
// stream) take the workspace's lock from the size check until both kernels
// of their call are queued: the GEMM and the second pass of one call are
// then adjacent on the stream, and the buffer is never replaced between them.
struct Workspace {
    std::mutex mu;
    float* ws = nullptr;
    size_t ws_bytes = 0;
};
static std::mutex g_ws_mu;   // guards the map itself
static std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

size_t workspace_bytes_for(int64_t M, int64_t N, int64_t K, int dtype, const tg_cfg& c)
{
    const PaddedLayout pl = padded_layout(M, N, K, dtype, c, padded_path(N, K, dtype, c, current_desc()));
    if (pl.on)
        return pl.total;
    if (c.kind == TG_KIND_STREAMK) {
        // one bm x bn slot per piece: tail tiles x most pieces per tile
        const SkPlan sp = streamk_plan(M, N, K, c, current_desc());
        if (sp.smax < 2)
            return 0;
        return (size_t)sp.tail * (size_t)sp.smax * (size_t)c.bm * (size_t)c.bn * sizeof(float);
    }
    if (cta_splits(c) <= 1)
        return 0;
    return (size_t)c.split_k * (size_t)splitk_slab(M, N) * sizeof(float);
}

PaddedLayout padded_layout(int64_t M, int64_t N, int64_t K, int dtype, const tg_cfg& c, bool on)
{
    PaddedLayout l{};
    if (!on)
        return l;
    auto up256 = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t eb = (size_t)in_bytes(dtype);
    l.on = true;
    l.Np = pad_extent(N, dtype);
    l.Kp = pad_extent(K, dtype);
    l.slab = splitk_slab(M, l.Np);
    l.a_off = up256((size_t)c.split_k * (size_t)l.slab * sizeof(float));
    l.b_off = l.a_off + up256((size_t)M * (size_t)l.Kp * eb);
    l.total = l.b_off + up256((size_t)l.Kp * (size_t)l.Np * eb);
    return l;
}

int ensure_workspace(size_t ws_bytes, hipStream_t stream, float** ws, std::unique_lock<std::mutex>* hold)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return set_hip_error(e, "hipGetDevice");
    Workspace* wp;
    {
        std::lock_guard<std::mutex> lk(g_ws_mu);
        wp = &g_ws[{dev, stream}];   // map nodes never move
    }
    Workspace& w = *wp;
    std::unique_lock<std::mutex> lk(w.mu);
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
    if (hold)
        *hold = std::move(lk);
    return TG_OK;
}

}  // namespace tg
