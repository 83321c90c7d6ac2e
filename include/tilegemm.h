/*
 * tilegemm -- fused GEMM with per-shape tile selection for AMD MI355X (gfx950).
 *
 * Operation (page "Tile Selection: Cost Models Against Measurement", opening
 * section and "The structure of the search space"; epilogue fusion per page
 * "Tiling the hierarchy", fusion section):
 *
 *     C[i][j] = act( sum_k A[i][k] * B[k][j] + bias[j] )
 *
 * Layouts: A is M x K, B is K x N, C is M x N, all row-major with leading
 * dimensions K, N and N; bias is N float32 values or NULL (= 0).
 *
 * Every function is extern "C", never throws and returns a tg_status
 * (0 = success).  On failure a message is available from tg_last_error() on
 * the calling thread.  Device pointers are caller-owned; the library never
 * retains or frees them.  C must not overlap A, B or bias.
 */
#ifndef TILEGEMM_H
#define TILEGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TG_VERSION 3

typedef enum {
    TG_OK = 0,
    TG_E_INVAL = -1,        /* bad argument (size, pointer, code) */
    TG_E_INFEASIBLE = -2,   /* the configuration fails the feasibility filter for this shape */
    TG_E_UNSUPPORTED = -3,  /* shape beyond the supported limits, or no device */
    TG_E_HIP = -4,          /* a HIP runtime call failed */
    TG_E_NOMEM = -5,        /* device or host allocation failed */
    TG_E_CACHE = -6         /* tuning-cache file missing, unreadable or malformed */
} tg_status;

/* input -> output element types; accumulation is always fp32 */
typedef enum {
    TG_F32 = 0,          /* fp32 in, fp32 out */
    TG_BF16 = 1,         /* bf16 in, bf16 out (round to nearest even) */
    TG_BF16_F32OUT = 2   /* bf16 in, fp32 out */
} tg_dtype;

typedef enum {
    TG_ACT_NONE = 0,
    TG_ACT_RELU = 1,     /* max(0, x) */
    TG_ACT_GELU = 2      /* 0.5 x (1 + erf(x / sqrt 2)) */
} tg_act;

typedef enum {
    TG_KIND_TILED = 0,     /* block-tiled MFMA kernel, 16-byte transfers of
                              rows straight into LDS; on a shape whose K or N
                              is not a whole 16-byte vector it runs padded (see
                              gemm_bias_act) */
    TG_KIND_SKINNY = 1,    /* M <= 64 weight-streaming kernel (bf16 only) */
    TG_KIND_UNALIGNED = 2, /* block-tiled kernel with element loads, for K or N
                              not a multiple of the 16-byte vector */
    TG_KIND_STREAMK = 3,   /* bf16 block-tiled kernel: full rounds of tiles one
                              workgroup each, the last partial round's K steps
                              spread evenly over a full round of workgroups
                              (stream-K), pieces of split tiles added in K order
                              by a second pass; split_k = 1; feasible only
                              when the tiles do not fill whole rounds */
    TG_KIND_SLICEDK = 4    /* block-tiled kernel whose workgroup holds split_k
                              groups of wgm x wgn waves, each multiplying its
                              own share of every stage's K slices; the groups'
                              sums meet in LDS before the epilogue (K split
                              inside one workgroup: one launch, no partial-sum
                              slabs; page "Compilers and Kernel Languages", "A
                              different tile for every shape": how the K
                              reduction is shared out is a choice of its own) */
} tg_kind;

/*
 * One point of the tile space ("The structure of the search space": block
 * tile, reduction step, per-thread tile; page "Compilers and Kernel
 * Languages": pipeline depth and split-K are further choices).
 *   tiled / unaligned: bm x bn block tile, bk reduction step, wgm x wgn waves
 *       (64 lanes each) per workgroup, stages = pipeline depth (tiled: 2, 3,
 *       4, 6 or 8 K steps in flight global -> LDS; unaligned: 2 LDS
 *       buffers), split_k = workgroups sharing one tile's K range.
 *   sliced-K: as tiled, with split_k = the K groups inside one workgroup
 *       (2 or 4; the workgroup has wgm x wgn x split_k waves).
 *   skinny: bm = 16 * ceil(M / 16), bn = 128 columns per workgroup, bk = 32,
 *       wgm = waves per workgroup (each takes interleaved 32-row chunks of
 *       K), wgn = 1, stages = chunks per pipelined step, split_k as above.
 * Field order is the canonical order used for ties.
 */
typedef struct {
    int32_t kind, bm, bn, bk, wgm, wgn, stages, split_k;
} tg_cfg;

/* Device description the selection rules use.  mode 0 = MI355X rules,
 * mode 1 = replica of the H100 model on page "Compilers and Kernel Languages"
 * ("Workshop").  Peaks in FLOP/s and bytes/s, times in seconds. */
typedef struct {
    int32_t mode, n_cu, simds, lds_cu, lds_block, max_threads, waves_max, blocks_max,
            vgpr_max, acc_max, r0, reserved;
    double peak_bf16, peak_f32, bw, a_ref, c_fill, t0, unaligned_eff, lat_mem, cu_bw,
           lds_bw_cu,   /* LDS bytes/s per CU */
           lat_step,    /* memory latency a K step waits for, divided by the pipeline depth (s) */
           lat_l2,      /* the same when the problem's compulsory bytes fit in l2_bytes (s) */
           l2_bytes,
           w1_eff,      /* issue efficiency of a lone wave on a SIMD */
           skinny_eff,  /* achievable fraction of the decode kernel's streaming model */
           hbm_eff,     /* achievable fraction of the HBM peak */
           sliced_eff;  /* issue efficiency of the sliced-K kind (its K groups meet a
                           barrier after every short run of MFMAs) */
/* The MI355X mode prices a K step per CU (MFMA, LDS, L2-to-CU, latency /
 * depth) over rounds of resident blocks; the replica mode is the page's
 * formula and ignores lds_bw_cu .. sliced_eff. */
} tg_device_desc;

/* One row of an autotuning table.  Every candidate is first measured with
 * short samples (TILEGEMM_TUNE_SAMPLE_US, default 2 ms of back-to-back
 * launches); the best few of those (TILEGEMM_TUNE_CONFIRM, default 8; 0 turns
 * the stage off) and the fixed default are then measured again with long
 * samples (TILEGEMM_TUNE_CONFIRM_US, default 10 ms), each preceded by as long
 * again of untimed launches of the same candidate so that clocks have settled
 * as in sustained use, and the tuner's choice is the fastest of those. */
typedef struct {
    tg_cfg cfg;
    double predicted_us;   /* cost-model time */
    double measured_us;    /* median of the short samples per launch, or -1 if not measured */
    double confirmed_us;   /* median of the long samples, or -1 if not in the confirmation stage */
} tg_tune_row;

/* ---------------------------------------------------------------- errors */
const char *tg_last_error(void);    /* thread-local; valid until the next call on this thread */
int tg_version(void);

/* ---------------------------------------------------------------- compute */
/*
 * Stream for later launches on this thread (a hipStream_t; NULL = the null
 * stream).
 */
int tg_set_stream(void *hip_stream);

/*
 * C = act(A . B + bias) on the device current for this thread, on the stream
 * set with tg_set_stream.  Asynchronous: returns once the kernel is queued,
 * except that cfg == NULL with a shape not yet in the tuning cache first runs
 * gemm_autotune (blocking; it times the candidates on copies of this call's
 * A, B and bias), or takes the cost model's choice when the
 * environment variable TILEGEMM_DISABLE_AUTOTUNE=1 is set.  With cfg == NULL
 * the cache is keyed on M's shape bucket (tg_dispatch_m): one tuning serves
 * every M of the bucket.
 *   M, N >= 0, K >= 0 (M or N = 0: nothing to do; K = 0: C = act(bias)).
 *   A, B, C: device pointers, 16-byte aligned for the skinny, stream-K and
 *     sliced-K kinds; any element alignment for the unaligned kind and for
 *     the tiled kind, whose padded path copies an A or B off 16-byte
 *     alignment and writes such a C through its output pass (a call without
 *     cfg whose selection picked another kind runs the same tile on the
 *     tiled kind then, or the unaligned kind where that tile does not fit).
 *   bias: device pointer to N floats, or NULL.
 *   dtype: tg_dtype; act: tg_act; cfg: explicit configuration or NULL.
 * Limits: K <= 2^21, N <= 2^21, M <= 2^31 - 1 (TG_E_UNSUPPORTED beyond).
 * Errors: TG_E_INVAL (NULL pointer with a non-empty operand, bad code,
 * negative size, misaligned pointer for the chosen kind), TG_E_INFEASIBLE
 * (cfg fails the filter: nothing is launched), TG_E_HIP, TG_E_NOMEM.
 * Split-K configurations (split_k > 1, except the sliced-K kind, whose
 * groups add their sums inside the workgroup) run two kernels on the
 * stream: the GEMM writes one
 * fp32 slab of partial sums per split (split_k x M x N floats) to a
 * library-owned workspace, then a second kernel adds the slabs in split order
 * and applies bias, activation and conversion.  The tiled kind on a shape
 * whose K or N is not a multiple of 8 bf16 / 4 fp32 elements takes the
 * padded path (page "Compilers and Kernel Languages", "A different tile for
 * every shape": ragged shapes): one kernel copies into the workspace the
 * operands whose rows are ragged or not 16-byte aligned (A with K rounded
 * up to a whole vector, B with N and K rounded up; new rows and columns
 * zero; a B with only K ragged is read in place, its missing rows as
 * zeros), the GEMM runs on the padded extents, and when N is ragged (or C
 * misaligned) it writes fp32 slabs of M x Np with any split_k and an output
 * pass adds them, applies bias, activation and conversion and writes C --
 * two or three kernels, results as on an aligned shape.
 * There is one workspace per (device, stream), grown on demand (growth waits
 * for that stream), so calls on different streams may run concurrently;
 * calls on one stream are ordered by it.
 */
int gemm_bias_act(int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                  const float *bias, void *C, int dtype, int act, const tg_cfg *cfg);

/*
 * gemm_bias_act for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, layouts, stream and results as gemm_bias_act (the same
 * kernels run), but the call allocates nothing: no hipMalloc, no hipFree, no
 * allocating library routine, and it never tunes -- with cfg == NULL it takes
 * the cache entry of M's shape bucket, else the cost model's choice.
 * Split-K partial sums (and the padded path's operand copies) go to one
 * fixed device array of tg_noalloc_scratch_bytes() bytes (32 MiB) that each
 * GPU the library runs on holds until the process ends; a call that needs
 * more (split_k x M x N floats, each slab rounded up to 64, plus the padded
 * copies) is refused with TG_E_INVAL before anything is queued.  Every call on one GPU shares that
 * GPU's array: calls on one stream are ordered by it, but calls that overlap
 * on one GPU through different streams race on the array and may return
 * wrong results.  Other errors as gemm_bias_act.
 */
int gemm_bias_act_noalloc(int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                          const float *bias, void *C, int dtype, int act, const tg_cfg *cfg);
size_t tg_noalloc_scratch_bytes(void);

/*
 * Tile scheduling order (page "Compilers and Kernel Languages", "A different
 * tile for every shape": the order in which tiles are scheduled is one of the
 * choices the analytical model leaves out).  Workgroups are renumbered so
 * that each of the 8 XCDs owns a contiguous range of tiles, enumerated in
 * groups of group_m tile rows, column-major inside a group (tiles that share
 * A rows and B columns then share an L2).  The order never changes results,
 * only which operands an L2 holds at a time.  tg_set_tile_order: group_m
 * tile rows per group, 1 .. 4096, or 0 for the default (8, or the
 * environment variable TILEGEMM_GROUP_M); process-wide; TG_E_INVAL outside
 * that range.  tg_tile_order: the value in force.
 */
int tg_set_tile_order(int group_m);
int tg_tile_order(void);

/*
 * Run-time dispatch over shape buckets (page "Tile Selection: Cost Models
 * Against Measurement", "Hybrid strategies": a few tuned variants selected at
 * launch from the actual extents, so that a varying batch does not make every
 * request a new cache key, a miss and a re-tune).  With buckets on (the
 * default; TILEGEMM_SHAPE_BUCKETS=0 starts the process with them off), a
 * gemm_bias_act call without cfg uses the cache entry of key_m: M rounded up
 * to a multiple of 16 for 1 <= M <= 64, to 128 for 64 < M <= 128, to 256 for
 * 128 < M <= 256, M itself otherwise; that entry is tuned at key_m, the
 * bucket's largest M, whose configuration is feasible for every M of the
 * bucket.  gemm_autotune and explicit cfgs are not affected.
 * tg_set_shape_buckets: on != 0 switches buckets on, 0 off (process-wide).
 * tg_dispatch_m: the M a call without cfg is keyed on now; TG_E_INVAL for
 * M < 0 or a NULL key_m.
 */
int tg_set_shape_buckets(int on);
int tg_dispatch_m(int64_t M, int64_t *key_m);

/*
 * Choose a configuration for (M, N, K, dtype) on the current device and store
 * it in the tuning cache (page "Tile Selection: Cost Models Against
 * Measurement", "Measurement, and what it must control" and "Hybrid
 * strategies"): the feasibility filter, then the cost model ranks the
 * survivors, then the best top_k plus the fixed default configuration are
 * timed on scratch inputs (uniform values in [-1, 1); a gemm_bias_act call
 * tuned on first use times copies of its own operands instead), running the
 * epilogue of the call being tuned (the measured runs must be the runs that
 * are served: same page, "Measurement, and what it must control"), interleaved
 * over several rounds; the best few by those medians and the default are
 * re-timed with long samples (see tg_tune_row) and the fastest of those
 * wins.  A cache hit returns at once
 * without measuring.  Blocking.  Mode and top_k come from
 * TILEGEMM_TUNE_MODE = hybrid (default) | model | exhaustive and
 * TILEGEMM_TUNE_TOPK (default 16, at most 30).  Each sample is about
 * TILEGEMM_TUNE_SAMPLE_US (default 2000) of back-to-back launches; problems
 * with at most 64 rows rotate through copies of B that exceed the last-level
 * cache (weights streamed from HBM, as in a decode step).  Scratch memory:
 * A, C, bias and one to eight copies of B, freed before returning.
 */
int gemm_autotune(int64_t M, int64_t N, int64_t K, int dtype, tg_cfg *out);
/*
 * The tuning cache is keyed by (device, M, N, K, dtype, act, bias present):
 * gemm_autotune tunes and caches the call without activation and bias;
 * gemm_autotune_ep the call with activation act (tg_act) and, if has_bias is
 * nonzero, a bias vector -- the entry a gemm_bias_act call of that epilogue
 * without cfg uses.  Errors as gemm_autotune, plus TG_E_INVAL for an unknown
 * act.
 */
int gemm_autotune_ep(int64_t M, int64_t N, int64_t K, int dtype, int act, int has_bias, tg_cfg *out);

/* ---------------------------------------------------------------- selection queries (host only)
 * None of these touches the GPU; all use the device description in force
 * (tg_set_device_override, else the current device's, else MI355X). */
/* Candidate enumeration (page "Tile Selection: Cost Models Against
 * Measurement", "The structure of the search space": the cross product of
 * block tile, reduction step and per-wave tile, cut down by resource limits
 * checkable before anything runs): the feasible configurations for the shape
 * in canonical order; writes at most cap into out (may be NULL when cap is
 * 0), reports the total in *n_feasible.  TG_E_INVAL for a bad dtype, negative
 * sizes or a NULL out with cap > 0. */
int tg_enumerate(int64_t M, int64_t N, int64_t K, int dtype, tg_cfg *out, int cap, int *n_feasible);
/* The whole candidate space before filtering (same section), canonical order;
 * buffer convention as tg_enumerate. */
int tg_space(int dtype, tg_cfg *out, int cap, int *n_total);
/* Feasibility filter for one configuration (same section: LDS for both panels,
 * accumulator registers, the register file, whole MFMA tiles, occupancy):
 * *reason = 0 if feasible, else the first failing rule:
 * 1 dtype, 2 alignment, 3 shape, 4 waves, 5 divisibility, 6 LDS, 7 accumulators,
 * 8 VGPR estimate, 9 occupancy, 10 split-K, 11 not in the space, 12 more transfers in flight per
 * wave than the memory counter tracks (63; bf16 tiled kind, ST x transfers per wave and stage),
 * 13 the compiled kernel spills registers (page "Autotuning & cost models", the search space:
 * the register cliff).  TG_E_INVAL for NULL pointers. */
int tg_check_cfg(int64_t M, int64_t N, int64_t K, int dtype, const tg_cfg *cfg, int *reason);
/* Cost-model time of a feasible configuration, in microseconds (page "Tile
 * Selection: Cost Models Against Measurement", "Analytical models and where
 * they break"; page "Compilers and Kernel Languages", "Workshop": the larger
 * of compute time at the wave and tile efficiencies and memory time).
 * TG_E_INFEASIBLE if cfg fails the filter for the shape. */
int tg_model_time(int64_t M, int64_t N, int64_t K, int dtype, const tg_cfg *cfg, double *us);
/* The cost-model times of n configurations at once (same passages), in
 * microseconds; -1 for a configuration that fails the filter for the shape.
 * For fitting the model's constants to measured tables.  TG_E_INVAL for
 * n < 0 or NULL buffers with n > 0. */
int tg_model_times(int64_t M, int64_t N, int64_t K, int dtype, const tg_cfg *cfgs, int n, double *us);
/* The model's choice (same passages; ties keep the first in canonical order):
 * the feasible configuration with the smallest model time and that time (us
 * may be NULL).  TG_E_INFEASIBLE if nothing is feasible. */
int tg_model_choice(int64_t M, int64_t N, int64_t K, int dtype, tg_cfg *out, double *us);
/* Launch geometry (page "Tile Selection: Cost Models Against Measurement",
 * "The structure of the search space": ceil(M/bm) * ceil(N/bn) blocks): output
 * tiles and launched workgroups (tiles * split_k; tiles for the sliced-K
 * kind; for the stream-K kind the data-parallel tiles plus min(CUs x
 * resident workgroups, tail tiles x K steps) workgroups for the tail, on the
 * device description in force).
 * TG_E_INVAL for NULL pointers, non-positive tile sizes, K step or split, and
 * negative M, N or K. */
int tg_grid(int64_t M, int64_t N, int64_t K, const tg_cfg *cfg, int64_t *tiles, int64_t *blocks);
/* The fixed configuration autotuning is always compared against (page "CuTile
 * Autotuning", key rules: the default is among the measured candidates):
 * 128 x 128 tiles where the shape allows vector loads. */
int tg_default_cfg(int64_t M, int64_t N, int64_t K, int dtype, tg_cfg *out);
/* The filter's pre-build estimates (page "Tile Selection: Cost Models Against
 * Measurement", "The structure of the search space": shared memory for both
 * panels, registers per thread): LDS bytes, VGPR+AGPR per lane, workgroups per
 * CU.  They decide which kernels are compiled; once a kernel exists the cost
 * model counts resident workgroups from what the compiler allotted
 * (tg_kernel_resources) instead.  Outputs may be NULL. */
int tg_resources(int dtype, const tg_cfg *cfg, int *lds_bytes, int *vgprs, int *blocks_per_cu);
/* Use desc for every selection rule (NULL = the real device / MI355X defaults);
 * mode 1 replays the H100 model of page "Compilers and Kernel Languages",
 * "Workshop".  TG_E_INVAL for an implausible description. */
int tg_set_device_override(const tg_device_desc *desc);
/* The description in force (override, else the current device's, else MI355X defaults). */
int tg_get_device_desc(tg_device_desc *out);
/* Built-in descriptions: which = 0 MI355X, 1 H100 replica (page "Compilers and
 * Kernel Languages", "Workshop": 132 SMs, 989 TFLOP/s, 3.35 TB/s). */
int tg_builtin_device_desc(int which, tg_device_desc *out);

/* ---------------------------------------------------------------- kernel registry (host only) */
/* Number of compiled kernel instantiations. */
int tg_kernel_count(void);
/* 1 if a compiled kernel serves cfg for dtype, else 0. */
int tg_has_kernel(int dtype, const tg_cfg *cfg);
/* What the compiler allotted to the kernel serving cfg (from its resource
 * report at build time): out[0..4] = VGPRs, AGPRs, scratch bytes per lane
 * (register spills), LDS bytes, waves per SIMD; -1 where unknown.
 * TG_E_INFEASIBLE if no kernel serves cfg.  A kernel that spills fails the
 * filter (rule 13); the cost model counts resident workgroups from these
 * registers and LDS bytes. */
int tg_kernel_resources(int dtype, const tg_cfg *cfg, int *out5);
/* Whether a call of M rows with cfg reads B with the non-temporal cache
 * policy (*out = 1) or the default one (*out = 0).  B is streamed that way
 * when every element of it is read by exactly one workgroup: the skinny kind
 * always, and bf16 tiled kinds of at most 64 rows when M fits in one tile row
 * (page "Tiling the hierarchy", failure regimes: matrix-vector-like products
 * move the weights once and reuse none of them).  Host-only: no GPU work.
 * TG_E_INFEASIBLE if no kernel serves cfg, TG_E_INVAL for NULL pointers or
 * M < 0. */
int tg_streams_b(int64_t M, int dtype, const tg_cfg *cfg, int *out);

/* ---------------------------------------------------------------- tuning cache
 * Page "Tile Selection: Cost Models Against Measurement", "Measurement, and
 * what it must control": the results are cached keyed by device, shape, dtype
 * and library version, and may be stored in a file.  Keys here are
 * (device, M, N, K, dtype, act, has_bias != 0). */
/* Table of the last tuning run for this key: every measured candidate with the
 * model's time, the short-sample median and the confirmation median; rows in
 * measurement order; writes at most cap, reports the count in *n (0 if the
 * key has no table). */
int tg_autotune_table(int64_t M, int64_t N, int64_t K, int dtype, int act, int has_bias, tg_tune_row *rows,
                      int cap, int *n);
/* Cached entry for the key on the current device: *hit = 1 and *out filled
 * (and *measured_us, if not NULL), or *hit = 0. */
int tg_cache_lookup(int64_t M, int64_t N, int64_t K, int dtype, int act, int has_bias, tg_cfg *out,
                    double *measured_us, int *hit);
/* Persist / restore the cache as text, one line per key (arch, CU count,
 * library version, M, N, K, dtype, act, bias -> cfg, measured and predicted
 * us).  Loading skips lines for another library version and configurations
 * this build cannot run; a malformed file is TG_E_CACHE and leaves the cache
 * unchanged. */
int tg_cache_save(const char *path);
int tg_cache_load(const char *path, int *n_loaded, int *n_skipped);
void tg_cache_clear(void);
int tg_cache_size(void);
/* Counters: tuning runs, timed launches, cache hits served by gemm_bias_act. */
int tg_stats(int64_t *n_tunes, int64_t *n_timed_launches, int64_t *n_cache_hits);

/* ---------------------------------------------------------------- RMS normalisation (occupancy-only tuning) */
/*
 * A memory-bound second kernel whose only tuned parameter is occupancy
 * (page "CuTile Autotuning", "Quick Reference -- Occupancy-Only Autotune":
 * normalisation kernels tune the resident workgroups per compute unit only;
 * grid = CUs x occupancy; tune once per shape, cache, launch directly).
 *   y[r, :] = x[r, :] / sqrt(mean(x[r, :]^2) + eps) * w
 * x, y: device pointers to rows x n bf16 (row-major), w: n bf16; all three
 * 16-byte aligned; fp32 arithmetic, each row reduced in a fixed order (the
 * result does not depend on the occupancy).  Constraints: n a multiple of 8,
 * 8 <= n <= 32768, 0 <= rows < 2^31 (TG_E_UNSUPPORTED otherwise), eps finite
 * and >= 0 (TG_E_INVAL).
 * tg_rmsnorm: occupancy 1, 2, 4 or 8 launches min(rows, CUs x occupancy)
 *   workgroups that stride over the rows; 0 takes the cached choice for
 *   (device, rows, n), tuning first on a miss (blocking).  Asynchronous on the
 *   stream set with tg_set_stream otherwise.  rows = 0: nothing to do.
 * tg_rmsnorm_autotune: times occupancies 1, 2, 4, 8 on scratch rows of the
 *   shape (interleaved rounds of about 1 ms of back-to-back launches, median)
 *   and caches the fastest; a cached shape returns at once.  Blocking;
 *   allocates and frees its scratch.  Outputs may be NULL.
 * tg_rmsnorm_cache_lookup: *hit = 1 with the cached occupancy and its
 *   measured microseconds, else *hit = 0.  In-memory cache, per device.
 * tg_rmsnorm_tunes: number of tuning runs so far (this process).
 */
int tg_rmsnorm(int64_t rows, int64_t n, const void *x, const void *w, void *y, float eps, int occupancy);
int tg_rmsnorm_autotune(int64_t rows, int64_t n, int *occupancy, double *us);
int tg_rmsnorm_cache_lookup(int64_t rows, int64_t n, int *occupancy, double *us, int *hit);
int tg_rmsnorm_tunes(int64_t *n_tunes);

#ifdef __cplusplus
}
#endif

#endif /* TILEGEMM_H */
