// C ABI of the fused GEMM library: argument checking, device description,
// launch geometry, split-K workspace, and the selection queries.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "registry.hpp"
#include "runtime.hpp"
#include "select.hpp"

namespace tg {

// ------------------------------------------------------------------ errors
static thread_local std::string t_err;

int set_error(int status, const std::string& msg)
{
    t_err = msg;
    return status;
}

int set_hip_error(hipError_t e, const char* what)
{
    return set_error(TG_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// ------------------------------------------------------------------ device description
static std::mutex g_desc_mu;
static bool g_override_set = false;
static tg_device_desc g_override;

struct DevInfo {
    bool valid = false;
    tg_device_desc desc{};
    DeviceKey key;
};
static std::vector<DevInfo> g_devs;

static int device_count()
{
    static int n = -1;
    static std::once_flag once;
    std::call_once(once, [] {
        int c = 0;
        if (hipGetDeviceCount(&c) != hipSuccess)
            c = 0;
        n = c;
    });
    return n;
}

bool have_device() { return device_count() > 0; }

// caller holds g_desc_mu
static const DevInfo* real_device_info()
{
    if (!have_device())
        return nullptr;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return nullptr;
    if ((int)g_devs.size() <= dev)
        g_devs.resize(dev + 1);
    DevInfo& di = g_devs[dev];
    if (!di.valid) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess)
            return nullptr;
        di.desc = mi355x_desc();
        di.desc.n_cu = p.multiProcessorCount;
        if (p.maxSharedMemoryPerMultiProcessor > 0)
            di.desc.lds_cu = (int32_t)p.maxSharedMemoryPerMultiProcessor;
        if (p.sharedMemPerBlock > 0)
            di.desc.lds_block = (int32_t)std::min<size_t>(p.sharedMemPerBlock, (size_t)di.desc.lds_cu);
        std::string arch = p.gcnArchName;
        const size_t colon = arch.find(':');
        if (colon != std::string::npos)
            arch = arch.substr(0, colon);
        di.key = DeviceKey{arch, p.multiProcessorCount};
        di.valid = true;
    }
    return &di;
}

tg_device_desc current_desc()
{
    std::lock_guard<std::mutex> lk(g_desc_mu);
    if (g_override_set)
        return g_override;
    if (const DevInfo* di = real_device_info())
        return di->desc;
    return mi355x_desc();
}

DeviceKey current_key()
{
    std::lock_guard<std::mutex> lk(g_desc_mu);
    if (g_override_set)
        return DeviceKey{g_override.mode == 1 ? "h100-replica" : "gfx950-override", g_override.n_cu};
    if (const DevInfo* di = real_device_info())
        return di->key;
    return DeviceKey{"gfx950-nodevice", 256};
}

// ------------------------------------------------------------------ shape buckets
// on unless TILEGEMM_SHAPE_BUCKETS=0; tg_set_shape_buckets switches it
static std::atomic<int> g_buckets{[] {
    const char* s = std::getenv("TILEGEMM_SHAPE_BUCKETS");
    return (s && s[0] && std::strcmp(s, "0") == 0) ? 0 : 1;
}()};

// the M a dispatch without an explicit configuration is keyed (and tuned) on
static int64_t dispatch_m(int64_t M) { return g_buckets.load() ? bucket_m(M) : M; }

// ------------------------------------------------------------------ tile order
// Tile rows per scheduling group (page "Compilers and Kernel Languages", "A
// different tile for every shape": the order in which tiles are scheduled is
// a choice of its own).  The order changes which tiles share an XCD's L2 at a
// time, never what a tile computes.  Default 8 (TILEGEMM_GROUP_M overrides);
// tg_set_tile_order changes it process-wide.
static int default_tile_order()
{
    const char* s = std::getenv("TILEGEMM_GROUP_M");
    const int v = s ? std::atoi(s) : 0;
    return v > 0 ? v : 8;
}
static std::atomic<int> g_group_m{default_tile_order()};
static int tile_order() { return g_group_m.load(); }

// ------------------------------------------------------------------ stream
static thread_local hipStream_t t_stream = nullptr;
hipStream_t current_stream() { return t_stream; }

// ------------------------------------------------------------------ launch
static constexpr int64_t kMaxKN = int64_t(1) << 21;
static constexpr int64_t kMaxM = (int64_t(1) << 31) - 1;

int validate_problem(int64_t M, int64_t N, int64_t K, int dtype)
{
    if (dtype != TG_F32 && dtype != TG_BF16 && dtype != TG_BF16_F32OUT)
        return set_error(TG_E_INVAL, "unknown dtype " + std::to_string(dtype));
    if (M < 0 || N < 0 || K < 0)
        return set_error(TG_E_INVAL, "negative dimension");
    if (K > kMaxKN || N > kMaxKN || M > kMaxM)
        return set_error(TG_E_UNSUPPORTED, "shape beyond the supported limits (K, N <= 2^21, M < 2^31)");
    return TG_OK;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// A launch with a single row of tiles reads every element of B in exactly one
// workgroup: B is then streamed with the non-temporal policy, where such an
// instantiation exists (page "Tiling the hierarchy", failure regimes: a
// matrix-vector-like product moves the weights once and reuses none of them).
static LaunchFn launch_fn(const KernelEntry& ke, const GemmParams& p)
{
    return (p.tiles_m == 1 && ke.launch_stream_b) ? ke.launch_stream_b : ke.launch;
}

int launch_cfg(int64_t M, int64_t N, int64_t K, const void* A, const void* B, const float* bias, void* C,
               int dtype, int act, const tg_cfg& cfg, hipStream_t stream, bool from_selection,
               const ExternalWorkspace* ext)
{
    const tg_device_desc d = current_desc();
    tg_cfg c = cfg;
    // the padded path copies the operands it cannot read in place and writes
    // a C it cannot store into through its output pass: the tiled kind takes
    // it for a ragged shape and for operands off 16-byte alignment
    bool misaligned = !(aligned16(A) && aligned16(B) && aligned16(C));
    bool padded = padded_path(N, K, dtype, c, d) || (d.mode == 0 && c.kind == TG_KIND_TILED && misaligned);
    if (c.kind != TG_KIND_UNALIGNED && misaligned && !padded) {
        if (!from_selection)
            return set_error(TG_E_INVAL, "A, B and C must be 16-byte aligned for the skinny, stream-K and sliced-K kinds");
        // selection ran without knowing the pointers: the same tile as the
        // tiled kind, which takes misaligned operands padded, else the
        // element-load kernel
        const tg_cfg t{TG_KIND_TILED, c.bm, c.bn, c.bk, c.wgm, c.wgn, c.stages, 1};
        if (d.mode == 0 && check(M, N, K, dtype, t, d) == OK && find_kernel(dtype, t)) {
            c = t;
            padded = true;
        } else {
            c = tg_cfg{TG_KIND_UNALIGNED, 64, 64, dtype == TG_F32 ? 16 : 32, 2, 2, 2, 1};
        }
    } else {
        const int r = check(M, N, K, dtype, c, d);
        if (r != OK)
            return set_error(TG_E_INFEASIBLE, "configuration infeasible for this shape (rule " +
                                                  std::to_string(r) + ")");
    }
    if (bias && ((uintptr_t)bias & 3u))
        return set_error(TG_E_INVAL, "bias must be 4-byte aligned");
    if (c.kind == TG_KIND_SKINNY && bias && misaligned)
        return set_error(TG_E_INVAL, "misaligned pointers");
    const KernelEntry* ke = find_kernel(dtype, c);
    if (!ke)
        return set_error(TG_E_INFEASIBLE, "no compiled kernel for this configuration");

    GemmParams p{};
    p.A = A;
    p.B = B;
    p.bias = bias;
    p.C = C;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    p.kps = (int)k_per_split(c, K);
    p.split = (int)cta_splits(c);
    if (c.kind == TG_KIND_SKINNY) {
        p.tiles_m = 1;
        p.tiles_n = (int)((N + 127) / 128);
    } else {
        p.tiles_m = (int)((M + c.bm - 1) / c.bm);
        p.tiles_n = (int)((N + c.bn - 1) / c.bn);
    }
    p.out_bf16 = dtype == TG_BF16 ? 1 : 0;
    p.act = act;
    p.group_m = tile_order();
    // the padded path: the kernel runs on the padded extents.  It copies the
    // operands whose rows are ragged or that are not 16-byte aligned (the
    // kernel moves 16-byte chunks of rows); a B read in place has its rows
    // past K read as zero.  When N is ragged (or C misaligned) the sums go to
    // slabs whatever the split and the output pass writes C.
    const PaddedLayout pl = padded_layout(M, N, K, dtype, c, padded);
    bool copy_a = false, copy_b = false, out_pass = false;
    if (pl.on) {
        copy_a = pl.Kp != K || !aligned16(A);
        copy_b = pl.Np != N || !aligned16(B);
        out_pass = pl.Np != N || !aligned16(C);
        p.N = (int)pl.Np;
        p.K = (int)pl.Kp;
        p.kps = (int)k_per_split(c, pl.Kp);
        if (!copy_b)
            p.kb = (int)K;
        if (out_pass) {
            p.C = nullptr;
            p.slab_out = 1;
        }
    }
    int64_t tiles, blocks;
    grid(M, N, K, c, &tiles, &blocks, &d);
    if (blocks > 0x7FFFFFFF)
        return set_error(TG_E_UNSUPPORTED, "too many workgroups");
    bool fixup = false;
    if (c.kind == TG_KIND_STREAMK) {
        const SkPlan sp = streamk_plan(M, N, K, c, d);
        p.sk_dp = (int)sp.dp;
        p.sk_g = (int)sp.wgs;
        p.sk_tail = (int)sp.tail;
        p.sk_ks = (int)sp.ks;
        p.sk_smax = (int)std::max<int64_t>(1, sp.smax);
        fixup = sp.smax >= 2;
    }
    // held until every kernel of a call that uses the workspace is queued (see
    // ensure_workspace)
    std::unique_lock<std::mutex> ws_hold;
    if (cta_splits(c) > 1 || fixup || pl.on) {
        const size_t need = pl.on ? pl.total : workspace_bytes_for(M, N, K, dtype, c);
        if (ext) {
            if (need > ext->bytes)
                return set_error(TG_E_INVAL, "the workspace of this call needs " + std::to_string(need) +
                                                 " bytes, more than the " + std::to_string(ext->bytes) +
                                                 " bytes of the caller-independent scratch");
            p.ws = ext->ws;
        } else {
            const int st = ensure_workspace(need, stream, &p.ws, &ws_hold);
            if (st != TG_OK)
                return st;
        }
        p.slab = pl.on ? pl.slab : splitk_slab(M, N);
    }
    hipError_t e;
    if (copy_a || copy_b) {
        char* base = reinterpret_cast<char*>(p.ws);
        if (copy_a)
            p.A = base + pl.a_off;
        if (copy_b)
            p.B = base + pl.b_off;
        e = pad_operands(A, B, base + pl.a_off, base + pl.b_off, M, N, K, pl.Np, pl.Kp, in_bytes(dtype), copy_a,
                         copy_b, stream);
        if (e != hipSuccess)
            return set_hip_error(e, "operand padding launch");
    }
    e = launch_fn(*ke, p)(p, (int)blocks, stream);
    if (e != hipSuccess)
        return set_hip_error(e, "kernel launch");
    if (out_pass) {
        e = padded_output(p.ws, c.split_k, pl.slab, pl.Np, M, N, bias, C, p.out_bf16, act, stream);
        if (e != hipSuccess)
            return set_hip_error(e, "padded output pass launch");
    } else if (cta_splits(c) > 1) {
        e = splitk_reduce(p.ws, c.split_k, M, N, bias, C, p.out_bf16, act, stream);
        if (e != hipSuccess)
            return set_hip_error(e, "split-K reduction launch");
    }
    if (fixup) {
        e = streamk_fixup(p, c.bm, c.bn, stream);
        if (e != hipSuccess)
            return set_hip_error(e, "stream-K second pass launch");
    }
    return TG_OK;
}

int validate_call(int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* C, int dtype, int act)
{
    const int st = validate_problem(M, N, K, dtype);
    if (st != TG_OK)
        return st;
    if (act < TG_ACT_NONE || act > TG_ACT_GELU)
        return set_error(TG_E_INVAL, "unknown activation " + std::to_string(act));
    if (M == 0 || N == 0)
        return TG_OK;
    if (!C || (K > 0 && (!A || !B)))
        return set_error(TG_E_INVAL, "NULL pointer for a non-empty operand");
    if (!have_device())
        return set_error(TG_E_UNSUPPORTED, "no HIP device");
    return TG_OK;
}

int select_for_call(int64_t M, int64_t N, int64_t K, const void* A, const void* B, const float* bias, int dtype,
                    int act, bool allow_tuning, tg_cfg* out)
{
    // the cache entry of M's shape bucket: chosen (tuned) at the bucket's
    // largest M, so one tuning serves the whole bucket
    const int64_t Mk = dispatch_m(M);
    tg_cfg c;
    double us;
    if (cache_find(Mk, N, K, dtype, act, bias != nullptr, &c, &us)) {
        count_cache_hit();
    } else {
        const char* dis = std::getenv("TILEGEMM_DISABLE_AUTOTUNE");
        if (!allow_tuning || (dis && std::strcmp(dis, "0") != 0 && dis[0])) {
            if (!model_choice(Mk, N, K, dtype, current_desc(), &c, nullptr))
                return set_error(TG_E_INFEASIBLE, "no feasible configuration");
        } else {
            const TuneData own{A, B, bias, M};
            const int st = autotune(Mk, N, K, dtype, act, bias != nullptr, &c, &own);
            if (st != TG_OK)
                return st;
        }
    }
    // every rule that depends on M holds across a bucket (the skinny kind's
    // row tile is M rounded up to 16, the same for the whole bucket); the
    // check stays as a guard
    if (Mk != M && check(M, N, K, dtype, c, current_desc()) != OK &&
        !model_choice(M, N, K, dtype, current_desc(), &c, nullptr))
        return set_error(TG_E_INFEASIBLE, "no feasible configuration");
    *out = c;
    return TG_OK;
}

}  // namespace tg

using namespace tg;

extern "C" {

const char* tg_last_error(void) { return t_err.c_str(); }

int tg_version(void) { return TG_VERSION; }

int tg_set_stream(void* hip_stream)
{
    t_stream = static_cast<hipStream_t>(hip_stream);
    return TG_OK;
}

int gemm_bias_act(int64_t M, int64_t N, int64_t K, const void* A, const void* B, const float* bias, void* C,
                  int dtype, int act, const tg_cfg* cfg)
{
    const int st = validate_call(M, N, K, A, B, C, dtype, act);
    if (st != TG_OK || M == 0 || N == 0)
        return st;
    tg_cfg c;
    if (cfg) {
        c = *cfg;
    } else {
        const int r = select_for_call(M, N, K, A, B, bias, dtype, act, true, &c);
        if (r != TG_OK)
            return r;
    }
    return launch_cfg(M, N, K, A, B, bias, C, dtype, act, c, current_stream(), cfg == nullptr);
}

int tg_set_tile_order(int group_m)
{
    if (group_m < 0 || group_m > 4096)
        return set_error(TG_E_INVAL, "tile rows per scheduling group must be 0 (default) .. 4096");
    g_group_m.store(group_m == 0 ? default_tile_order() : group_m);
    return TG_OK;
}

int tg_tile_order(void) { return tile_order(); }

int tg_set_shape_buckets(int on)
{
    g_buckets.store(on ? 1 : 0);
    return TG_OK;
}

int tg_dispatch_m(int64_t M, int64_t* key_m)
{
    if (!key_m)
        return set_error(TG_E_INVAL, "key_m is NULL");
    if (M < 0)
        return set_error(TG_E_INVAL, "negative dimension");
    *key_m = dispatch_m(M);
    return TG_OK;
}

int gemm_autotune_ep(int64_t M, int64_t N, int64_t K, int dtype, int act, int has_bias, tg_cfg* out)
{
    if (!out)
        return set_error(TG_E_INVAL, "out is NULL");
    const int st = validate_problem(M, N, K, dtype);
    if (st != TG_OK)
        return st;
    if (act < TG_ACT_NONE || act > TG_ACT_GELU)
        return set_error(TG_E_INVAL, "unknown activation " + std::to_string(act));
    if (M == 0 || N == 0)
        return set_error(TG_E_INVAL, "empty problem has nothing to tune");
    return autotune(M, N, K, dtype, act, has_bias != 0, out);
}

int gemm_autotune(int64_t M, int64_t N, int64_t K, int dtype, tg_cfg* out)
{
    return gemm_autotune_ep(M, N, K, dtype, TG_ACT_NONE, 0, out);
}

int tg_enumerate(int64_t M, int64_t N, int64_t K, int dtype, tg_cfg* out, int cap, int* n_feasible)
{
    const int st = validate_problem(M, N, K, dtype);
    if (st != TG_OK)
        return st;
    if (cap < 0 || (cap > 0 && !out))
        return set_error(TG_E_INVAL, "bad output buffer");
    const std::vector<tg_cfg> v = enumerate_feasible(M, N, K, dtype, current_desc());
    const int n = (int)std::min<size_t>(v.size(), (size_t)cap);
    if (n > 0)
        std::memcpy(out, v.data(), n * sizeof(tg_cfg));
    if (n_feasible)
        *n_feasible = (int)v.size();
    return TG_OK;
}

int tg_space(int dtype, tg_cfg* out, int cap, int* n_total)
{
    if (dtype != TG_F32 && dtype != TG_BF16 && dtype != TG_BF16_F32OUT)
        return set_error(TG_E_INVAL, "unknown dtype");
    if (cap < 0 || (cap > 0 && !out))
        return set_error(TG_E_INVAL, "bad output buffer");
    const auto& sp = space(dtype, current_desc());
    const int n = (int)std::min<size_t>(sp.size(), (size_t)cap);
    if (n > 0)
        std::memcpy(out, sp.data(), n * sizeof(tg_cfg));
    if (n_total)
        *n_total = (int)sp.size();
    return TG_OK;
}

int tg_check_cfg(int64_t M, int64_t N, int64_t K, int dtype, const tg_cfg* cfg, int* reason)
{
    if (!cfg || !reason)
        return set_error(TG_E_INVAL, "NULL argument");
    *reason = check(M, N, K, dtype, *cfg, current_desc());
    return TG_OK;
}

int tg_model_time(int64_t M, int64_t N, int64_t K, int dtype, const tg_cfg* cfg, double* us)
{
    if (!cfg || !us)
        return set_error(TG_E_INVAL, "NULL argument");
    const tg_device_desc d = current_desc();
    const int r = check(M, N, K, dtype, *cfg, d);
    if (r != OK)
        return set_error(TG_E_INFEASIBLE, "configuration infeasible (rule " + std::to_string(r) + ")");
    *us = model_time(M, N, K, dtype, *cfg, d) * 1e6;
    return TG_OK;
}

int tg_model_times(int64_t M, int64_t N, int64_t K, int dtype, const tg_cfg* cfgs, int n, double* us)
{
    if (n < 0 || (n > 0 && (!cfgs || !us)))
        return set_error(TG_E_INVAL, "bad buffers");
    const int st = validate_problem(M, N, K, dtype);
    if (st != TG_OK)
        return st;
    const tg_device_desc d = current_desc();
    for (int i = 0; i < n; ++i)
        us[i] = check(M, N, K, dtype, cfgs[i], d) == OK ? model_time(M, N, K, dtype, cfgs[i], d) * 1e6 : -1.0;
    return TG_OK;
}

int tg_model_choice(int64_t M, int64_t N, int64_t K, int dtype, tg_cfg* out, double* us)
{
    if (!out)
        return set_error(TG_E_INVAL, "NULL argument");
    const int st = validate_problem(M, N, K, dtype);
    if (st != TG_OK)
        return st;
    double t = 0.0;
    if (!model_choice(M, N, K, dtype, current_desc(), out, &t))
        return set_error(TG_E_INFEASIBLE, "no feasible configuration");
    if (us)
        *us = t * 1e6;
    return TG_OK;
}

int tg_grid(int64_t M, int64_t N, int64_t K, const tg_cfg* cfg, int64_t* tiles, int64_t* blocks)
{
    if (!cfg || !tiles || !blocks || cfg->bm <= 0 || cfg->bn <= 0 || cfg->bk <= 0 || cfg->split_k <= 0 || M < 0 ||
        N < 0 || K < 0)
        return set_error(TG_E_INVAL, "bad argument");
    const tg_device_desc d = current_desc();
    grid(M, N, K, *cfg, tiles, blocks, &d);
    return TG_OK;
}

int tg_default_cfg(int64_t M, int64_t N, int64_t K, int dtype, tg_cfg* out)
{
    (void)M;
    if (!out)
        return set_error(TG_E_INVAL, "NULL argument");
    const int st = validate_problem(M, N, K, dtype);
    if (st != TG_OK)
        return st;
    *out = default_cfg(N, K, dtype);
    return TG_OK;
}

int tg_resources(int dtype, const tg_cfg* cfg, int* lds, int* vgprs, int* bpc)
{
    if (!cfg)
        return set_error(TG_E_INVAL, "NULL argument");
    if (cfg->wgm <= 0 || cfg->wgn <= 0 || cfg->bm <= 0 || cfg->bn <= 0)
        return set_error(TG_E_INVAL, "bad configuration");
    const tg_device_desc d = current_desc();
    if (lds)
        *lds = (int)lds_bytes(*cfg, dtype);
    if (vgprs)
        *vgprs = (int)vgpr_estimate(*cfg, dtype, d);
    if (bpc)
        *bpc = (int)blocks_per_cu(*cfg, dtype, d);
    return TG_OK;
}

int tg_set_device_override(const tg_device_desc* desc)
{
    std::lock_guard<std::mutex> lk(g_desc_mu);
    if (desc) {
        if (desc->n_cu <= 0 || desc->simds <= 0 || desc->bw <= 0 || desc->peak_bf16 <= 0 || desc->peak_f32 <= 0)
            return set_error(TG_E_INVAL, "implausible device description");
        g_override = *desc;
        g_override_set = true;
    } else {
        g_override_set = false;
    }
    return TG_OK;
}

int tg_get_device_desc(tg_device_desc* out)
{
    if (!out)
        return set_error(TG_E_INVAL, "NULL argument");
    *out = current_desc();
    return TG_OK;
}

int tg_builtin_device_desc(int which, tg_device_desc* out)
{
    if (!out || (which != 0 && which != 1))
        return set_error(TG_E_INVAL, "bad argument");
    *out = which == 0 ? mi355x_desc() : h100_replica_desc();
    return TG_OK;
}

int tg_kernel_count(void) { return (int)(registry_end() - registry_begin()); }

int tg_has_kernel(int dtype, const tg_cfg* cfg)
{
    if (!cfg)
        return 0;
    return find_kernel(dtype, *cfg) ? 1 : 0;
}

int tg_streams_b(int64_t M, int dtype, const tg_cfg* cfg, int* out)
{
    if (!cfg || !out)
        return set_error(TG_E_INVAL, "NULL argument");
    if (M < 0)
        return set_error(TG_E_INVAL, "negative dimension");
    const KernelEntry* k = find_kernel(dtype, *cfg);
    if (!k)
        return set_error(TG_E_INFEASIBLE, "no compiled kernel for this configuration");
    GemmParams p{};
    p.tiles_m = cfg->kind == TG_KIND_SKINNY ? 1 : (int)((M + cfg->bm - 1) / cfg->bm);
    *out = (cfg->kind == TG_KIND_SKINNY || launch_fn(*k, p) == k->launch_stream_b) ? 1 : 0;
    return TG_OK;
}

int tg_kernel_resources(int dtype, const tg_cfg* cfg, int* out5)
{
    if (!cfg || !out5)
        return set_error(TG_E_INVAL, "NULL argument");
    const KernelEntry* k = find_kernel(dtype, *cfg);
    if (!k)
        return set_error(TG_E_INFEASIBLE, "no compiled kernel for this configuration");
    out5[0] = k->res.vgpr;
    out5[1] = k->res.agpr;
    out5[2] = k->res.scratch;
    out5[3] = k->res.lds;
    out5[4] = k->res.occupancy;
    return TG_OK;
}

}  // extern "C"
