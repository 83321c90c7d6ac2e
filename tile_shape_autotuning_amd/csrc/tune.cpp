// Measuring autotuner and the shape-keyed tuning cache.
//
// Page "Tile Selection: Cost Models Against Measurement":
//   * "Hybrid strategies": the resource filter discards what cannot fit, the
//     cost model ranks the rest, a handful of the best is measured;
//   * "Measurement, and what it must control": candidates are interleaved
//     (round robin over several rounds, so clock drift hits all of them), the
//     inputs have the workload's kind of values, and each sample times many
//     back-to-back launches so launch overhead is divided out;
//   * the result is cached keyed by shape, dtype, device and library version
//     and can be stored in a file that outlives the process.
// Page "CuTile Autotuning" (rules): the fixed default configuration is always
// among the measured candidates, so tuning never picks something slower than
// the default it replaces; at most 30 candidates are measured in hybrid mode.
//
// Short samples rank every candidate; the best eight and the default are then
// timed again with samples five times longer, each after as long again of
// untimed launches of the same candidate, and the choice is made among
// those.  Configurations that burn matrix-core power they do not need run
// fast in short bursts and lose their lead once the clock settles to their
// own power draw (on the 16 x 28672 x 8192 decode, a 64-row, 8-wave tile that
// led the 2 ms ranking by 0.3 % runs 5 % behind a 32-row, 2-wave one
// sustained; with all-zero operands, which draw little matrix-core power,
// the two tie).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <map>
#include <mutex>
#include <sstream>
#include <string>
#include <tuple>
#include <vector>

#include "runtime.hpp"
#include "select.hpp"

namespace tg {

// A call is keyed by what it runs: the device, the shape and dtype, and the
// epilogue (activation, bias or not), since the candidates are timed with it.
struct CacheKey {
    std::string arch;
    int n_cu;
    int64_t M, N, K;
    int dtype;
    int act;
    int bias;
    bool operator<(const CacheKey& o) const
    {
        return std::tie(arch, n_cu, M, N, K, dtype, act, bias) <
               std::tie(o.arch, o.n_cu, o.M, o.N, o.K, o.dtype, o.act, o.bias);
    }
};

struct CacheEntry {
    tg_cfg cfg;
    double measured_us;
    double predicted_us;
    std::vector<tg_tune_row> table;
};

static std::mutex g_cache_mu;
static std::map<CacheKey, CacheEntry> g_cache;
static int64_t g_n_tunes = 0, g_n_timed = 0, g_n_hits = 0;

static CacheKey make_key(int64_t M, int64_t N, int64_t K, int dtype, int act, bool bias)
{
    const DeviceKey dk = current_key();
    return CacheKey{dk.arch, dk.n_cu, M, N, K, dtype, act, bias ? 1 : 0};
}

bool cache_find(int64_t M, int64_t N, int64_t K, int dtype, int act, bool bias, tg_cfg* out, double* measured_us)
{
    const CacheKey k = make_key(M, N, K, dtype, act, bias);
    std::lock_guard<std::mutex> lk(g_cache_mu);
    auto it = g_cache.find(k);
    if (it == g_cache.end())
        return false;
    *out = it->second.cfg;
    if (measured_us)
        *measured_us = it->second.measured_us;
    return true;
}

void count_cache_hit()
{
    std::lock_guard<std::mutex> lk(g_cache_mu);
    ++g_n_hits;
}

static int env_int(const char* name, int def)
{
    const char* s = std::getenv(name);
    if (!s || !*s)
        return def;
    return std::atoi(s);
}

static std::string env_str(const char* name, const char* def)
{
    const char* s = std::getenv(name);
    return (s && *s) ? std::string(s) : std::string(def);
}

namespace {

// Device scratch operands filled with uniform values in [-1, 1).
struct Scratch {
    void* A = nullptr;
    std::vector<void*> B;   // one or more copies of B (see b_copies)
    void* C = nullptr;
    float* bias = nullptr;
    ~Scratch()
    {
        if (A) (void)hipFree(A);
        for (void* b : B)
            if (b) (void)hipFree(b);
        if (C) (void)hipFree(C);
        if (bias) (void)hipFree(bias);
    }
};

// Page "Tile Selection: Cost Models Against Measurement", "Measurement, and
// what it must control": the timed runs must see the cache state the real
// calls see.  A problem with at most 64 rows is a decode step streaming
// weights that no cache holds between calls (each layer has its own), so its
// candidates are timed rotating through copies of B that together exceed the
// 256 MiB last-level cache twice over; larger problems reuse their operands
// call after call and are timed warm.
static int b_copies(int64_t M, int64_t b_bytes)
{
    if (M > 64 || b_bytes <= 0)
        return 1;
    const int64_t need = (int64_t)512 << 20;
    return (int)std::min<int64_t>(8, std::max<int64_t>(2, (need + b_bytes - 1) / b_bytes));
}

struct Timed {
    tg_cfg cfg;
    double predicted_us;
    int reps = 1;
    bool ok = true;
    std::vector<double> samples;   // us per launch, short samples
    std::vector<double> confirm;   // us per launch, long samples (confirmation stage)
    double med = -1.0, med_confirm = -1.0;
};

double median_of(std::vector<double> v)
{
    if (v.empty())
        return -1.0;
    std::sort(v.begin(), v.end());
    return v[v.size() / 2];
}

}  // namespace

int autotune(int64_t M, int64_t N, int64_t K, int dtype, int act, bool has_bias, tg_cfg* out, const TuneData* data)
{
    const CacheKey key = make_key(M, N, K, dtype, act, has_bias);
    {
        std::lock_guard<std::mutex> lk(g_cache_mu);
        auto it = g_cache.find(key);
        if (it != g_cache.end()) {
            *out = it->second.cfg;
            return TG_OK;
        }
    }
    const tg_device_desc d = current_desc();
    const std::string mode = env_str("TILEGEMM_TUNE_MODE", "hybrid");
    int topk = env_int("TILEGEMM_TUNE_TOPK", 16);
    topk = std::max(1, std::min(topk, 30));
    const int rounds = std::max(3, std::min(env_int("TILEGEMM_TUNE_SAMPLES", 7), 51));
    const bool log = env_int("TILEGEMM_LOG", 0) != 0;

    // filter + rank (stable: equal model times keep canonical order)
    std::vector<tg_cfg> feas = enumerate_feasible(M, N, K, dtype, d);
    if (feas.empty())
        return set_error(TG_E_INFEASIBLE, "no feasible configuration");
    std::vector<std::pair<double, size_t>> ranked;
    ranked.reserve(feas.size());
    for (size_t i = 0; i < feas.size(); ++i)
        ranked.emplace_back(model_time(M, N, K, dtype, feas[i], d), i);
    std::stable_sort(ranked.begin(), ranked.end(),
                     [](const auto& a, const auto& b) { return a.first < b.first; });

    CacheEntry entry;
    if (mode == "model") {
        entry.cfg = feas[ranked[0].second];
        entry.predicted_us = ranked[0].first * 1e6;
        entry.measured_us = -1.0;
        entry.table.push_back(tg_tune_row{entry.cfg, entry.predicted_us, -1.0, -1.0});
    } else {
        if (!have_device())
            return set_error(TG_E_UNSUPPORTED, "measured tuning needs a HIP device (TILEGEMM_TUNE_MODE=model does not)");
        // only candidates with a compiled kernel can be measured (kernels the
        // compiler had to spill are already out: the filter's spill rule)
        const int max_split = env_int("TILEGEMM_TUNE_MAX_SPLIT", 1 << 30);
        auto runnable = [&](const tg_cfg& c) { return find_kernel(dtype, c) != nullptr && cta_splits(c) <= max_split; };
        std::vector<Timed> cands;
        const size_t take = mode == "exhaustive" ? ranked.size() : (size_t)topk;
        std::vector<char> picked(ranked.size(), 0);
        for (size_t i = 0; i < ranked.size() && cands.size() < take; ++i)
            if (runnable(feas[ranked[i].second])) {
                cands.push_back(Timed{feas[ranked[i].second], ranked[i].first * 1e6});
                picked[i] = 1;
            }
        // the model cannot rank across kernel kinds reliably (kinds often tie
        // at the memory floor), so the best few of every kind are measured too
        if (mode != "exhaustive") {
            const size_t per_kind = std::max<size_t>(2, (size_t)topk / 4);
            for (int kind = 0; kind <= 2; ++kind) {
                size_t have = 0;
                for (size_t i = 0; i < ranked.size() && have < per_kind; ++i) {
                    const tg_cfg& c = feas[ranked[i].second];
                    if (c.kind != kind || !runnable(c))
                        continue;
                    ++have;
                    if (!picked[i]) {
                        picked[i] = 1;
                        cands.push_back(Timed{c, ranked[i].first * 1e6});
                    }
                }
            }
        }
        const tg_cfg def = default_cfg(N, K, dtype);
        bool have_def = false;
        for (const Timed& t : cands)
            have_def = have_def || cfg_equal(t.cfg, def);
        if (!have_def && check(M, N, K, dtype, def, d) == OK && find_kernel(dtype, def))
            cands.push_back(Timed{def, model_time(M, N, K, dtype, def, d) * 1e6});
        if (cands.empty())
            return set_error(TG_E_INFEASIBLE, "no compiled kernel among the candidates");

        // scratch operands of the problem's shape
        const int eb = in_bytes(dtype), ec = out_bytes(dtype);
        Scratch s;
        hipStream_t st = current_stream();
        hipError_t e = hipSuccess;
        const size_t na = (size_t)std::max<int64_t>(M * K, 1), nb = (size_t)std::max<int64_t>(K * N, 1);
        const int nbc = b_copies(M, (int64_t)(nb * eb));
        s.B.assign(nbc, nullptr);
        if ((e = hipMalloc(&s.A, na * eb)) != hipSuccess || (e = hipMalloc(&s.C, (size_t)M * N * ec)) != hipSuccess ||
            (e = hipMalloc(&s.bias, (size_t)N * sizeof(float))) != hipSuccess)
            return set_error(TG_E_NOMEM, std::string("tuning scratch: ") + hipGetErrorString(e));
        for (int i = 0; i < nbc; ++i)
            if ((e = hipMalloc(&s.B[i], nb * eb)) != hipSuccess)
                return set_error(TG_E_NOMEM, std::string("tuning scratch: ") + hipGetErrorString(e));
        // The matrix cores' power draw, and with it the clock a configuration
        // sustains, depends on the operand values (on the decode weights an
        // 8-wave tile runs 78 us on the workload's values and 74.5 us on
        // zeros).  A call tuned on first use therefore times its candidates on
        // copies of its own operands; explicit tuning, which has none, on
        // uniform values in [-1, 1).
        const bool own = data && data->A && data->B && K > 0;
        const int64_t own_rows = own ? std::min<int64_t>(data->rows, M) : 0;
        if (own_rows > 0 &&
            (e = hipMemcpyAsync(s.A, data->A, (size_t)(own_rows * K) * eb, hipMemcpyDeviceToDevice, st)) != hipSuccess)
            return set_hip_error(e, "tuning scratch copy");
        if (own_rows < M &&
            (e = fill_uniform(static_cast<char*>(s.A) + (size_t)(own_rows * K) * eb, (M - own_rows) * K,
                              dtype != TG_F32, 0x1234u, st)) != hipSuccess)
            return set_hip_error(e, "tuning scratch fill");
        if (own && data->bias)
            e = hipMemcpyAsync(s.bias, data->bias, (size_t)N * sizeof(float), hipMemcpyDeviceToDevice, st);
        else
            e = fill_uniform(s.bias, N, 0, 0x9abcu, st);
        if (e != hipSuccess)
            return set_hip_error(e, "tuning scratch fill");
        for (int i = 0; i < nbc; ++i) {
            e = own ? hipMemcpyAsync(s.B[i], data->B, nb * eb, hipMemcpyDeviceToDevice, st)
                    : fill_uniform(s.B[i], (int64_t)nb, dtype != TG_F32, 0x5678u + (uint32_t)i, st);
            if (e != hipSuccess)
                return set_hip_error(e, "tuning scratch fill");
        }
        if (log)
            std::fprintf(stderr, "[tilegemm] tuning %lldx%lldx%lld dt%d on %s operands\n", (long long)M, (long long)N,
                         (long long)K, dtype, own ? "the caller's" : "uniform synthetic");
        // workspace for the largest split-K candidate, allocated before timing
        size_t wsb = 0;
        for (const Timed& t : cands)
            wsb = std::max(wsb, workspace_bytes_for(M, N, K, dtype, t.cfg));
        if (wsb > 0) {
            float* w;
            const int r = ensure_workspace(wsb, st, &w);
            if (r != TG_OK)
                return r;
        }
        hipEvent_t e0, e1;
        if ((e = hipEventCreate(&e0)) != hipSuccess || (e = hipEventCreate(&e1)) != hipSuccess)
            return set_hip_error(e, "hipEventCreate");
        size_t launches = 0;
        auto run = [&](Timed& t, int reps) -> bool {
            for (int r = 0; r < reps; ++r) {
                const void* b = s.B[launches++ % s.B.size()];
                // the call being tuned: its activation, its bias or none
                if (launch_cfg(M, N, K, s.A, b, has_bias ? s.bias : nullptr, s.C, dtype, act, t.cfg, st, false) !=
                    TG_OK)
                    return false;
            }
            return true;
        };
        const bool progress = env_int("TILEGEMM_PROGRESS", 0) != 0;
        if (progress)
            std::fprintf(stderr, "[tilegemm] tuning %lldx%lldx%lld dt%d: %zu candidates, %d rounds\n",
                         (long long)M, (long long)N, (long long)K, dtype, cands.size(), rounds);
        // warm-up and a single-launch estimate to size each sample: long enough
        // (2 ms by default) for the clock to settle where back-to-back calls run
        // it -- a configuration that burns more matrix-core power than it needs
        // looks fast in short bursts and slows down when sustained
        const double sample_us = (double)std::max(50, env_int("TILEGEMM_TUNE_SAMPLE_US", 2000));
        size_t done = 0;
        for (Timed& t : cands) {
            if (progress && ++done % 100 == 0)
                std::fprintf(stderr, "[tilegemm]   warm-up %zu/%zu\n", done, cands.size());
            if (!run(t, 1)) {
                t.ok = false;
                continue;
            }
            hipEventRecord(e0, st);
            t.ok = run(t, 1);
            hipEventRecord(e1, st);
            hipEventSynchronize(e1);
            float ms = 0.f;
            hipEventElapsedTime(&ms, e0, e1);
            const double us = std::max(1.0, (double)ms * 1e3);
            t.reps = (int)std::max(1.0, std::min(2000.0, std::ceil(sample_us / us)));
        }
        int64_t timed = 0;
        // one stage: `rounds` interleaved samples of every candidate in `set`
        // (the order rotates every round), each sample `scale` times the
        // sized repetition count
        auto measure = [&](const std::vector<size_t>& set, int scale, bool conf) -> int {
            for (int r = 0; r < rounds; ++r) {
                const size_t n = set.size();
                for (size_t j = 0; j < n; ++j) {
                    Timed& t = cands[set[(j + (size_t)r) % n]];
                    if (!t.ok)
                        continue;
                    const int reps = (int)std::min<int64_t>((int64_t)t.reps * scale, 20000);
                    // a long sample starts after as long again of untimed launches of
                    // the same candidate: the clock then reflects this candidate's
                    // own power draw, not that of the one timed before it
                    if (conf && !run(t, reps)) {
                        t.ok = false;
                        continue;
                    }
                    hipEventRecord(e0, st);
                    t.ok = run(t, reps);
                    hipEventRecord(e1, st);
                    e = hipEventSynchronize(e1);
                    if (e != hipSuccess)
                        return set_hip_error(e, "timing");
                    float ms = 0.f;
                    hipEventElapsedTime(&ms, e0, e1);
                    (conf ? t.confirm : t.samples).push_back((double)ms * 1e3 / reps);
                    timed += reps;
                }
                if (progress)
                    std::fprintf(stderr, "[tilegemm]   %s round %d/%d done\n", conf ? "confirmation" : "ranking",
                                 r + 1, rounds);
            }
            return TG_OK;
        };
        std::vector<size_t> all(cands.size());
        for (size_t i = 0; i < all.size(); ++i)
            all[i] = i;
        int rc = measure(all, 1, false);
        if (rc == TG_OK) {
            for (Timed& t : cands)
                t.med = (t.ok && !t.samples.empty()) ? median_of(t.samples) : -1.0;
            // confirmation stage: the best few by the short samples, plus the default
            const int n_conf = std::max(0, std::min(env_int("TILEGEMM_TUNE_CONFIRM", 8), 30));
            const int conf_us = std::max(100, env_int("TILEGEMM_TUNE_CONFIRM_US", 10000));
            std::vector<size_t> order;
            for (size_t i = 0; i < cands.size(); ++i)
                if (cands[i].med > 0)
                    order.push_back(i);
            std::stable_sort(order.begin(), order.end(), [&](size_t a, size_t b) {
                return cands[a].med < cands[b].med;
            });
            std::vector<size_t> conf(order.begin(), order.begin() + std::min<size_t>(order.size(), n_conf));
            if (!conf.empty())
                for (size_t i = 0; i < cands.size(); ++i)
                    if (cfg_equal(cands[i].cfg, def) && cands[i].med > 0 &&
                        std::find(conf.begin(), conf.end(), i) == conf.end())
                        conf.push_back(i);
            if (!conf.empty()) {
                const int scale = std::max(1, (int)std::lround((double)conf_us / sample_us));
                rc = measure(conf, scale, true);
                for (size_t i : conf)
                    cands[i].med_confirm = (cands[i].ok && !cands[i].confirm.empty()) ? median_of(cands[i].confirm)
                                                                                       : -1.0;
            }
        }
        hipEventDestroy(e0);
        hipEventDestroy(e1);
        if (rc != TG_OK)
            return rc;
        // the choice: fastest confirmed candidate, or fastest by the short
        // samples when the confirmation stage is off (ties: canonical order)
        bool any_conf = false;
        for (const Timed& t : cands)
            any_conf = any_conf || t.med_confirm > 0;
        int best = -1;
        double best_us = 0.0;
        for (size_t i = 0; i < cands.size(); ++i) {
            Timed& t = cands[i];
            const double v = any_conf ? t.med_confirm : t.med;
            if (v > 0 && (best < 0 || v < best_us || (v == best_us && cfg_less(t.cfg, cands[best].cfg)))) {
                best = (int)i;
                best_us = v;
            }
            entry.table.push_back(tg_tune_row{t.cfg, t.predicted_us, t.med, t.med_confirm});
            if (log)
                std::fprintf(stderr,
                             "[tilegemm] %lldx%lldx%lld dt%d kind%d %dx%dx%d w%dx%d st%d sk%d: model %.2f us, measured %.2f us"
                             "%s%.2f\n",
                             (long long)M, (long long)N, (long long)K, dtype, t.cfg.kind, t.cfg.bm, t.cfg.bn, t.cfg.bk,
                             t.cfg.wgm, t.cfg.wgn, t.cfg.stages, t.cfg.split_k, t.predicted_us, t.med,
                             t.med_confirm > 0 ? ", confirmed " : "", t.med_confirm > 0 ? t.med_confirm : 0.0);
        }
        if (best < 0)
            return set_error(TG_E_HIP, "every candidate failed to launch: " + std::string(tg_last_error()));
        entry.cfg = cands[best].cfg;
        entry.measured_us = best_us;
        entry.predicted_us = cands[best].predicted_us;
        e = hipStreamSynchronize(st);
        if (e != hipSuccess)
            return set_hip_error(e, "hipStreamSynchronize");
        std::lock_guard<std::mutex> lk(g_cache_mu);
        g_n_timed += timed;
    }
    std::lock_guard<std::mutex> lk(g_cache_mu);
    ++g_n_tunes;
    *out = entry.cfg;
    g_cache[key] = std::move(entry);
    return TG_OK;
}

}  // namespace tg

using namespace tg;

static const char* kHeader = "# tilegemm tuning cache v2";

extern "C" {

int tg_autotune_table(int64_t M, int64_t N, int64_t K, int dtype, int act, int has_bias, tg_tune_row* rows, int cap,
                      int* n)
{
    if (cap < 0 || (cap > 0 && !rows))
        return set_error(TG_E_INVAL, "bad output buffer");
    const CacheKey k = make_key(M, N, K, dtype, act, has_bias != 0);
    std::lock_guard<std::mutex> lk(g_cache_mu);
    auto it = g_cache.find(k);
    if (it == g_cache.end()) {
        if (n)
            *n = 0;
        return TG_OK;
    }
    const auto& t = it->second.table;
    const int m = (int)std::min<size_t>(t.size(), (size_t)cap);
    for (int i = 0; i < m; ++i)
        rows[i] = t[i];
    if (n)
        *n = (int)t.size();
    return TG_OK;
}

int tg_cache_lookup(int64_t M, int64_t N, int64_t K, int dtype, int act, int has_bias, tg_cfg* out,
                    double* measured_us, int* hit)
{
    if (!out || !hit)
        return set_error(TG_E_INVAL, "NULL argument");
    *hit = cache_find(M, N, K, dtype, act, has_bias != 0, out, measured_us) ? 1 : 0;
    return TG_OK;
}

int tg_cache_save(const char* path)
{
    if (!path)
        return set_error(TG_E_INVAL, "NULL path");
    std::ostringstream os;
    os << kHeader << "\n";
    {
        std::lock_guard<std::mutex> lk(g_cache_mu);
        char buf[512];
        for (const auto& kv : g_cache) {
            const CacheKey& k = kv.first;
            const CacheEntry& e = kv.second;
            std::snprintf(buf, sizeof buf, "%s %d %d %lld %lld %lld %d %d %d %d %d %d %d %d %d %d %d %.17g %.17g\n",
                          k.arch.c_str(), k.n_cu, TG_VERSION, (long long)k.M, (long long)k.N, (long long)k.K,
                          k.dtype, k.act, k.bias, e.cfg.kind, e.cfg.bm, e.cfg.bn, e.cfg.bk, e.cfg.wgm, e.cfg.wgn, e.cfg.stages,
                          e.cfg.split_k, e.measured_us, e.predicted_us);
            os << buf;
        }
    }
    std::ofstream f(path, std::ios::out | std::ios::trunc);
    if (!f)
        return set_error(TG_E_CACHE, std::string("cannot write ") + path);
    f << os.str();
    f.close();
    if (!f)
        return set_error(TG_E_CACHE, std::string("write failed: ") + path);
    return TG_OK;
}

int tg_cache_load(const char* path, int* n_loaded, int* n_skipped)
{
    if (!path)
        return set_error(TG_E_INVAL, "NULL path");
    std::ifstream f(path);
    if (!f)
        return set_error(TG_E_CACHE, std::string("cannot read ") + path);
    std::string line;
    if (!std::getline(f, line) || line != kHeader)
        return set_error(TG_E_CACHE, "not a tilegemm tuning cache (bad header)");
    std::vector<std::pair<CacheKey, CacheEntry>> parsed;
    int skipped = 0, lineno = 1;
    while (std::getline(f, line)) {
        ++lineno;
        if (line.empty() || line[0] == '#')
            continue;
        std::istringstream is(line);
        CacheKey k;
        CacheEntry e{};
        int ver;
        long long M, N, K;
        if (!(is >> k.arch >> k.n_cu >> ver >> M >> N >> K >> k.dtype >> k.act >> k.bias >> e.cfg.kind >> e.cfg.bm >> e.cfg.bn >>
              e.cfg.bk >> e.cfg.wgm >> e.cfg.wgn >> e.cfg.stages >> e.cfg.split_k >> e.measured_us >>
              e.predicted_us))
            return set_error(TG_E_CACHE, "malformed cache line " + std::to_string(lineno));
        std::string rest;
        if (is >> rest)
            return set_error(TG_E_CACHE, "trailing fields on cache line " + std::to_string(lineno));
        k.M = M;
        k.N = N;
        k.K = K;
        if (ver != TG_VERSION || validate_problem(M, N, K, k.dtype) != TG_OK || k.act < TG_ACT_NONE ||
            k.act > TG_ACT_GELU || (k.bias != 0 && k.bias != 1)) {
            ++skipped;   // another library version, or not a valid problem
            continue;
        }
        // a configuration that this build cannot run is stale
        const tg_device_desc d = k.arch == "h100-replica" ? h100_replica_desc() : mi355x_desc();
        if (check(M, N, K, k.dtype, e.cfg, d) != OK) {
            ++skipped;
            continue;
        }
        e.table.push_back(tg_tune_row{e.cfg, e.predicted_us, e.measured_us, -1.0});
        parsed.emplace_back(k, e);
    }
    std::lock_guard<std::mutex> lk(g_cache_mu);
    for (auto& kv : parsed)
        g_cache[kv.first] = kv.second;
    if (n_loaded)
        *n_loaded = (int)parsed.size();
    if (n_skipped)
        *n_skipped = skipped;
    return TG_OK;
}

void tg_cache_clear(void)
{
    std::lock_guard<std::mutex> lk(g_cache_mu);
    g_cache.clear();
}

int tg_cache_size(void)
{
    std::lock_guard<std::mutex> lk(g_cache_mu);
    return (int)g_cache.size();
}

int tg_stats(int64_t* n_tunes, int64_t* n_timed_launches, int64_t* n_cache_hits)
{
    std::lock_guard<std::mutex> lk(g_cache_mu);
    if (n_tunes)
        *n_tunes = g_n_tunes;
    if (n_timed_launches)
        *n_timed_launches = g_n_timed;
    if (n_cache_hits)
        *n_cache_hits = g_n_hits;
    return TG_OK;
}

}  // extern "C"
