// Host runtime shared by the C ABI and the autotuner.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <string>

#include "../../include/tilegemm.h"
#include "registry.hpp"

namespace tg {

int set_error(int status, const std::string& msg);   // returns status
int set_hip_error(hipError_t e, const char* what);     // returns TG_E_HIP

// identity of the device the selection rules and the cache are keyed on
struct DeviceKey {
    std::string arch;   // e.g. "gfx950", or "h100-replica" under that override
    int n_cu;
};

// description in force: override if set, else the current HIP device's, else MI355X defaults
tg_device_desc current_desc();
DeviceKey current_key();
bool have_device();

hipStream_t current_stream();

// Split-K partial sums in memory the caller provides instead of the
// library-owned workspace: `bytes` of device memory at `ws`, 256-byte aligned.
struct ExternalWorkspace {
    float* ws;
    size_t bytes;
};

// Validates arguments and launches one configuration (no selection).
// `from_selection` = true: the configuration came from selection, which did
// not see the pointers, so misaligned pointers run the element-load kernel
// instead; false (a configuration the caller named): they are refused.
// `ext`: split-K slabs go there (nothing is allocated; a call needing more
// than ext->bytes is refused), else into the (device, stream) workspace.
int launch_cfg(int64_t M, int64_t N, int64_t K, const void* A, const void* B, const float* bias,
               void* C, int dtype, int act, const tg_cfg& cfg, hipStream_t stream, bool from_selection,
               const ExternalWorkspace* ext = nullptr);

// The configuration a call without cfg uses: the cache entry of M's shape
// bucket; on a miss, tuning (allow_tuning, unless TILEGEMM_DISABLE_AUTOTUNE
// is set) or else the cost model's choice.
int select_for_call(int64_t M, int64_t N, int64_t K, const void* A, const void* B, const float* bias, int dtype,
                    int act, bool allow_tuning, tg_cfg* out);
int validate_call(int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* C, int dtype, int act);

// Split-K workspace of the current device and `stream`: grows to at least
// `ws_bytes`.  With `hold`, the workspace's lock is handed to the caller, who
// keeps it until every kernel that uses the buffer is queued.
int ensure_workspace(size_t ws_bytes, hipStream_t stream, float** ws, std::unique_lock<std::mutex>* hold = nullptr);
size_t workspace_bytes_for(int64_t M, int64_t N, int64_t K, int dtype, const tg_cfg& cfg);
// Workspace of the padded path (a ragged shape, padded_path in select.hpp,
// or operands off 16-byte alignment on the tiled kind): room for `split`
// fp32 slabs of [M x Np] (slab floats apart) from offset 0, then A' [M x Kp]
// at a_off and B' [Kp x Np] at b_off (bytes, 256-byte aligned), whichever of
// them a call uses; `on` (the call takes the padded path) false: all zero.
struct PaddedLayout {
    bool on;
    int64_t Np, Kp, slab;
    size_t a_off, b_off, total;
};
PaddedLayout padded_layout(int64_t M, int64_t N, int64_t K, int dtype, const tg_cfg& c, bool on);

// Split-K second pass (splitk_reduce.hip): C = act(sum of the split slabs +
// bias), slabs `splitk_slab(M, N)` floats apart.
int64_t splitk_slab(int64_t M, int64_t N);
hipError_t splitk_reduce(const float* ws, int split, int64_t M, int64_t N, const float* bias, void* C,
                         int out_bf16, int act, hipStream_t stream);

// The padded path (pad.hip): zero-padded copies A' [M x Kp], B' [Kp x Np] of
// A [M x K], B [K x N] (eb bytes per element; each only if its flag is set),
// and the output pass that adds `split` slabs of row stride ldp in split
// order, then bias, activation, conversion into C [M x N].
hipError_t pad_operands(const void* A, const void* B, void* Ap, void* Bp, int64_t M, int64_t N, int64_t K,
                        int64_t Np, int64_t Kp, int eb, bool copy_a, bool copy_b, hipStream_t stream);
hipError_t padded_output(const float* ws, int split, int64_t slab, int64_t ldp, int64_t M, int64_t N,
                         const float* bias, void* C, int out_bf16, int act, hipStream_t stream);

// Stream-K second pass (splitk_reduce.hip): adds the pieces of every tail
// tile split among workgroups, then bias, activation, conversion into C.
hipError_t streamk_fixup(const GemmParams& p, int bm, int bn, hipStream_t stream);

// Argument validation shared by the entry points.
int validate_problem(int64_t M, int64_t N, int64_t K, int dtype);

// tuner.  `data` (optional): the caller's operands of the call being tuned
// (rows of A available: data->rows <= M); the timed runs then use their values
// instead of synthetic ones.
struct TuneData {
    const void* A;
    const void* B;
    const float* bias;
    int64_t rows;
};
// Candidates are timed running the call's epilogue (act, bias or not), and
// the result is cached under that epilogue.
int autotune(int64_t M, int64_t N, int64_t K, int dtype, int act, bool has_bias, tg_cfg* out,
             const TuneData* data = nullptr);
bool cache_find(int64_t M, int64_t N, int64_t K, int dtype, int act, bool bias, tg_cfg* out, double* measured_us);
void count_cache_hit();

// fill kernels for tuning scratch (defined in tune_kernels.hip)
hipError_t fill_uniform(void* p, int64_t n, int is_bf16, uint32_t seed, hipStream_t s);

}  // namespace tg
