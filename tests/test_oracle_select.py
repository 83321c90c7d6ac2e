"""Pins for the tile-selection oracle (CPU only).

* The H100 replica of the model on page "Compilers and Kernel Languages"
  ("Workshop"; results in "A different tile for every shape") must reproduce
  every number the page prints (tests/golden/h100_model_page_results.json).
* Counting invariants: blocks = ceil(M/BM) * ceil(N/BN) (page "Tile Selection:
  Cost Models Against Measurement", search-space section, checked by brute
  force), the shared-memory cap of 12,288 float32 elements at 48 KB (same
  section), the size of the space that section describes (hundreds to
  thousands of points; 398 here), and loop-nest traffic 2 N^3 / T (page "Tiling the hierarchy",
  derivation, checked by simulating the loop nest).
* Invariants of the MI355X model whose constants the pages do not give
  ("parity unpinned" against the pages): wave efficiency is 1 exactly when
  the work divides the slots, the memory time never undercuts the compulsory
  floor, and time never rises when a peak rises.
"""
import dataclasses
import json
import math
import os

import pytest

from oracle import select_ref as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "h100_model_page_results.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _tile_times(M, N, K):
    return {(c.bm, c.bn): t for c, t in S.rank(M, N, K, S.BF16, S.H100_REPLICA)}


def test_replica_constants_match_page():
    g = _golden()["device"]
    d = S.H100_REPLICA
    assert d.n_cu == g["sms"]
    assert d.lds_cu == g["shared_memory_kb"] * 1024
    assert d.peak_bf16 == g["bf16_tflops"] * 1e12
    assert d.bw == g["hbm_tbps"] * 1e12
    assert {c.bk for c in S.space(S.BF16, d)} == {g["bk"]}
    assert len(S.space(S.BF16, d)) == 16


def test_replica_large_square():
    case = _golden()["cases"][0]
    M, N, K = case["M"], case["N"], case["K"]
    best, best_t = S.model_choice(M, N, K, S.BF16, S.H100_REPLICA)
    assert [best.bm, best.bn] == case["best_tile"]
    assert round(best_t * 1e6) == case["best_us_rounded"]
    times = _tile_times(M, N, K)
    assert round(max(times.values()) / best_t, 2) == case["worst_over_best_2dp"]
    assert round(times[(128, 128)] / best_t, 2) == case["fixed_128x128_over_best_2dp"]


def test_replica_small_problem_wave_quantisation():
    case = _golden()["cases"][1]
    M, N, K = case["M"], case["N"], case["K"]
    fixed = S.Cfg(S.KIND_TILED, 128, 128, 64, 1, 1, 1, 1)
    assert S.grid(M, N, fixed)[0] == case["tiles_at_128x128"]
    best, best_t = S.model_choice(M, N, K, S.BF16, S.H100_REPLICA)
    assert [best.bm, best.bn] == case["best_tile"]
    tiles = S.grid(M, N, best)[0]
    slots = S.H100_REPLICA.n_cu
    wave_eff = tiles / (math.ceil(tiles / slots) * slots)
    assert round(100 * wave_eff) == case["best_wave_efficiency_pct"]
    assert round(_tile_times(M, N, K)[(128, 128)] / best_t, 2) == case["fixed_128x128_over_best_2dp"]


def test_replica_decode_all_tie_at_weight_floor():
    case = _golden()["cases"][2]
    M, N, K = case["M"], case["N"], case["K"]
    times = set(_tile_times(M, N, K).values())
    assert len(times) == 1
    assert round(times.pop() * 1e6, 1) == case["floor_us_1dp"]


def test_replica_catches_model_mistakes():
    # dropping the g divisor, the tile efficiency, or the compulsory floor each
    # breaks one printed number
    d = S.H100_REPLICA
    M = N = K = 8192
    no_tile_eff = dataclasses.replace(d, a_ref=1.0)
    best, _ = S.model_choice(M, N, K, S.BF16, no_tile_eff)
    t = {(c.bm, c.bn): x for c, x in S.rank(M, N, K, S.BF16, no_tile_eff)}
    assert round(max(t.values()) / t[(best.bm, best.bn)], 2) != 1.83


@pytest.mark.parametrize("M,N,bm,bn", [(1, 1, 32, 32), (1000, 1000, 128, 128), (4100, 3000, 128, 128),
                                       (4100, 3000, 256, 64), (16, 28672, 16, 128), (8192, 8192, 256, 256)])
def test_block_count_formula_vs_brute_force(M, N, bm, bn):
    c = S.Cfg(S.KIND_TILED, bm, bn, 32, 1, 1, 1, 1)
    assert S.grid(M, N, c)[0] == S.block_count_brute(M, N, bm, bn)
    c4 = dataclasses.replace(c, split_k=4)
    assert S.grid(M, N, c4)[1] == 4 * S.block_count_brute(M, N, bm, bn)


def test_page1_space_size_and_caps():
    n, triples, widest = S.page1_space_count()
    # the section puts such spaces at hundreds to thousands of points
    assert 200 <= n <= 5000
    assert (n, triples) == (398, 55)
    # 48 KB of float32 panels caps BM*KS + KS*BN at 12,288 elements
    assert widest == 12288
    # the count against brute force over the whole cross product (a planted
    # mistake in either constraint would move it)
    brute = 0
    for bm in (32, 64, 128, 256):
        for bn in (32, 64, 128, 256):
            for ks in (8, 16, 32, 64):
                for tm in (2, 4, 8):
                    for tn in (2, 4, 8):
                        thr = (bm // tm) * (bn // tn)
                        brute += 4 * ks * (bm + bn) <= 48 * 1024 and thr % 32 == 0 and 32 <= thr <= 1024 \
                            and tm * tn <= 128
    assert brute == n
    # a larger shared memory admits strictly more tuples; a smaller thread cap fewer
    assert S.page1_space_count(smem_bytes=96 * 1024)[0] > n
    assert S.page1_space_count(max_threads=256)[0] < n


@pytest.mark.parametrize("n,t", [(8, 8), (16, 4), (32, 8), (64, 8), (64, 16), (48, 12)])
def test_loop_nest_traffic_is_2n3_over_t(n, t):
    assert S.loop_nest_traffic(n, t) * t == 2 * n ** 3


def test_square_root_law_halving_tile_doubles_traffic():
    # traffic ~ 1/T: a 4x smaller capacity (T halves) doubles the traffic
    assert S.loop_nest_traffic(64, 8) == 2 * S.loop_nest_traffic(64, 16)


# ---------------------------------------------------------------- MI355X rules
SHAPES = [(256, 256, 256, S.F32), (1000, 1000, 8192, S.BF16_F32OUT), (8192, 8192, 8192, S.BF16),
          (16, 28672, 8192, S.BF16), (4100, 3000, 1000, S.BF16), (17, 65, 15, S.BF16), (1, 1, 1, S.F32)]


def test_lds_examples():
    d = S.MI355X
    two = S.Cfg(S.KIND_TILED, 256, 256, 64, 2, 2, 2, 1)
    assert S.lds_bytes(two, S.BF16) == 2 * 64 * 1024
    assert S.check(8192, 8192, 8192, S.BF16, two, d) == S.OK
    big = S.Cfg(S.KIND_TILED, 256, 256, 128, 2, 2, 2, 1)
    assert S.lds_bytes(big, S.BF16) == 256 * 1024 > d.lds_block
    assert S.check(8192, 8192, 8192, S.BF16, big, d) == S.R_LDS     # 2 x 128 KiB stages
    one = S.Cfg(S.KIND_TILED, 128, 128, 128, 2, 4, 2, 1)              # 2 x 64 KiB stages fit
    assert S.lds_bytes(one, S.BF16) == 2 * 64 * 1024 and S.check(8192, 8192, 8192, S.BF16, one, d) == S.OK
    odd = S.Cfg(S.KIND_TILED, 128, 128, 96, 2, 4, 2, 1)
    assert S.check(8192, 8192, 8192, S.BF16, odd, d) == S.R_SPACE     # bf16 BK is 32, 64 or 128
    # the largest bf16 tiles at two stages fit; fp32 128x128x32 two stages fit
    assert S.check(8192, 8192, 8192, S.BF16, S.Cfg(0, 256, 256, 64, 2, 4, 2, 1), d) == S.OK
    assert S.check(8192, 8192, 8192, S.BF16, S.Cfg(0, 256, 256, 64, 2, 4, 3, 1), d) == S.R_LDS
    assert S.check(8192, 8192, 8192, S.BF16, S.Cfg(0, 256, 256, 64, 2, 4, 1, 1), d) == S.R_SPACE
    # fp32 tiles travel straight into LDS unpadded; the register-staged
    # kernel of the unaligned kind pads each B row by 4 floats
    assert S.lds_bytes(S.Cfg(0, 128, 128, 32, 2, 2, 2, 1), S.F32) == 2 * (128 * 32 + 32 * 128) * 4
    assert S.lds_bytes(S.Cfg(S.KIND_UNALIGNED, 128, 128, 16, 2, 2, 2, 1), S.F32) == 2 * (128 * 16 + 16 * 132) * 4
    # all 36 fp32 tile triples fit LDS at two stages
    for bm in (16, 32, 64, 128):
        for bn in (32, 64, 128):
            for bk in (16, 32, 64):
                assert S.lds_bytes(S.Cfg(0, bm, bn, bk, 1, 1, 2, 1), S.F32) <= d.lds_block


def test_rejections_have_reasons():
    d = S.MI355X
    assert S.check(256, 256, 256, S.F32, S.Cfg(0, 16, 64, 16, 2, 1, 2, 1), d) == S.R_DIV      # 16 rows, 2 waves
    assert S.check(256, 256, 256, S.F32, S.Cfg(0, 64, 64, 8, 1, 1, 2, 1), d) == S.R_SPACE     # fp32 BK is 16, 32, 64
    assert S.check(256, 256, 256, S.BF16, S.Cfg(0, 32, 32, 32, 1, 4, 1, 1), d) == S.R_SPACE
    assert S.check(256, 256, 256, S.BF16, S.Cfg(0, 32, 32, 32, 2, 4, 2, 1), d) == S.R_DIV
    assert S.check(256, 256, 256, S.BF16, S.Cfg(0, 256, 128, 32, 1, 1, 2, 1), d) == S.R_ACC
    # 64x256x64 panels are 40 one-KiB transfers per stage; one wave, 4 stages
    # in flight = 160 outstanding > 63 (the 160 KiB of LDS would fit)
    assert S.lds_bytes(S.Cfg(0, 64, 256, 64, 1, 1, 4, 1), S.BF16) == 4 * 40 * 1024
    assert S.check(256, 256, 256, S.BF16, S.Cfg(0, 64, 256, 64, 1, 1, 4, 1), d) == S.R_INFLIGHT
    assert S.check(256, 256, 256, S.BF16, S.Cfg(0, 64, 256, 64, 2, 4, 4, 1), d) == S.OK    # 5 per wave
    assert S.check(256, 256, 256, S.BF16, S.Cfg(0, 256, 256, 32, 1, 1, 2, 1), d) == S.R_INFLIGHT
    # a 16-row decode tile: 9 transfers per wave and stage; 6 stages fit, 8 do not
    assert S.transfers_per_wave(S.Cfg(0, 16, 128, 64, 1, 2, 8, 1), S.BF16) == 9
    assert S.check(16, 28672, 8192, S.BF16, S.Cfg(0, 16, 128, 64, 1, 2, 6, 1), d) == S.OK
    assert S.check(16, 28672, 8192, S.BF16, S.Cfg(0, 16, 128, 64, 1, 2, 8, 1), d) == S.R_INFLIGHT
    # an unaligned shape: the tiled kind takes it padded (K 15 -> 16), the
    # kinds without a padded path do not
    assert S.check(256, 256, 15, S.BF16, S.Cfg(0, 64, 64, 32, 2, 2, 2, 1), d) == S.OK
    assert S.check(256, 256, 15, S.BF16, S.Cfg(4, 32, 64, 64, 1, 2, 2, 2), d) == S.R_ALIGN
    assert S.check(256, 257, 4096, S.BF16, S.Cfg(3, 128, 128, 64, 2, 4, 3, 1), d) == S.R_ALIGN
    assert S.check(16, 257, 4096, S.BF16, S.Cfg(1, 16, 128, 32, 1, 1, 1, 1), d) == S.R_ALIGN
    # split-K on the padded K: 1025 -> 1032 = 2 x 516, so 2 splits of 544 (whole 32-k steps)
    assert S.check(256, 256, 1025, S.BF16, S.Cfg(0, 64, 64, 32, 2, 2, 2, 2), d) == S.OK
    assert S.check(256, 256, 15, S.BF16, S.Cfg(0, 64, 64, 32, 2, 2, 2, 2), d) == S.R_SPLIT
    assert S.check(256, 256, 256, S.BF16, S.Cfg(2, 64, 64, 32, 2, 2, 2, 1), d) == S.R_ALIGN
    assert S.check(256, 256, 64, S.BF16, S.Cfg(0, 64, 64, 32, 2, 2, 2, 4), d) == S.R_SPLIT
    assert S.check(100, 256, 256, S.BF16, S.Cfg(1, 112, 128, 32, 1, 1, 1, 1), d) == S.R_SPACE
    assert S.check(100, 256, 256, S.BF16, S.Cfg(1, 64, 128, 32, 1, 1, 1, 1), d) == S.R_SHAPE
    assert S.check(20, 256, 256, S.BF16, S.Cfg(1, 16, 128, 32, 1, 1, 1, 1), d) == S.R_SHAPE
    assert S.check(20, 256, 256, S.F32, S.Cfg(1, 32, 128, 32, 1, 1, 1, 1), d) in (S.R_SPACE, S.R_DTYPE)
    assert S.check(0, 256, 256, S.BF16, S.Cfg(0, 64, 64, 32, 2, 2, 2, 1), d) == S.R_SHAPE


@pytest.mark.parametrize("M,N,K,dt", SHAPES)
def test_model_invariants(M, N, K, dt):
    d = S.MI355X
    floor = (S.in_bytes(dt) * (M * K + K * N) + S.out_bytes(dt) * M * N) / d.bw
    faster = dataclasses.replace(d, peak_bf16=2 * d.peak_bf16, peak_f32=2 * d.peak_f32, bw=2 * d.bw)
    feas = S.enumerate_feasible(M, N, K, dt, d)
    assert feas, "every shape has at least one feasible candidate"
    for c in feas[:: max(1, len(feas) // 150)]:
        t = S.model_time(M, N, K, dt, c, d)
        assert t >= floor + d.t0 - 1e-18
        assert S.model_time(M, N, K, dt, c, faster) <= t
    best, bt = S.model_choice(M, N, K, dt, d)
    assert all(S.model_time(M, N, K, dt, c, d) >= bt for c in feas)
    # the default is always feasible (so it can always be measured)
    assert S.check(M, N, K, dt, S.default_cfg(N, K, dt), d) == S.OK


def test_wave_quantisation_in_the_per_cu_model():
    # compute alone: LDS, L2, latency and output-store terms made negligible, no lone-wave penalty
    d = dataclasses.replace(S.MI355X, lds_bw_cu=1e30, cu_bw=1e30, lat_step=0.0, lat_l2=0.0, w1_eff=1.0, bw=1e30)
    # 128x128 tiles, W = 4, two blocks fit a CU (64 KiB of LDS each): 256 tiles are one
    # partial round with one block per CU
    c = S.Cfg(S.KIND_TILED, 128, 128, 64, 2, 2, 2, 1)
    assert S.blocks_per_cu(c, S.BF16, d) == 2
    t256 = S.model_time(2048, 2048, 4096, S.BF16, c, d) - d.t0
    flops = 2.0 * 2048 * 2048 * 4096
    assert t256 == pytest.approx(flops / d.peak_bf16)            # every SIMD busy: the roofline
    # 272 tiles: the round holds two blocks on some CUs, which then take twice as long
    t272 = S.model_time(2048 + 128, 2048, 4096, S.BF16, c, d) - d.t0
    assert t272 == pytest.approx(2 * t256)
    # 512 tiles: exactly one full round of two blocks per CU, no waste
    t512 = S.model_time(4096, 2048, 4096, S.BF16, c, d) - d.t0
    assert t512 == pytest.approx(2 * flops / d.peak_bf16)
    # one-wave blocks occupy as many SIMDs as there are blocks on the CU
    c1 = S.Cfg(S.KIND_TILED, 128, 128, 64, 1, 2, 2, 1)
    b1 = S.blocks_per_cu(c1, S.BF16, d)
    busy = min(4, 2 * b1)
    t1 = S.model_time(4096, 4096, 4096, S.BF16, c1, d) - d.t0
    assert t1 >= (2.0 * 4096 ** 3 / d.peak_bf16) * 4 / busy * (1 - 1e-12)
    if busy < 4:
        assert t1 > 1.5 * (2.0 * 4096 ** 3 / d.peak_bf16)


def test_output_stores_follow_the_k_loop():
    # compute-bound 2048x2048x4096 on 128x128 tiles: the C stores (bf16) add their HBM time
    fast = dataclasses.replace(S.MI355X, lds_bw_cu=1e30, cu_bw=1e30, lat_step=0.0, lat_l2=0.0, w1_eff=1.0, bw=1e30)
    real_bw = dataclasses.replace(fast, bw=S.MI355X.bw)
    c = S.Cfg(S.KIND_TILED, 128, 128, 64, 2, 2, 2, 1)
    t_inf = S.model_time(2048, 2048, 4096, S.BF16, c, fast)
    t_bw = S.model_time(2048, 2048, 4096, S.BF16, c, real_bw)
    assert t_bw - t_inf == pytest.approx(2 * 2048 * 2048 / (S.MI355X.bw * S.MI355X.hbm_eff))
    # with split-K the stores are the fp32 slabs, and the second pass reads them and writes C
    c2 = dataclasses.replace(c, split_k=2)
    t2_inf = S.model_time(2048, 2048, 4096, S.BF16, c2, fast)
    t2_bw = S.model_time(2048, 2048, 4096, S.BF16, c2, real_bw)
    bw = S.MI355X.bw * S.MI355X.hbm_eff
    assert t2_bw - t2_inf == pytest.approx((2 * 4 * 2048 * 2048 + (2 * 4 + 2) * 2048 * 2048) / bw)


def test_per_cu_model_terms():
    d = S.MI355X
    c = S.Cfg(S.KIND_TILED, 256, 256, 64, 2, 4, 2, 1)
    # a half-line A row (BK = 32 bf16) costs a whole line: more L2 time per byte than BK = 64
    assert S._line(32 * 2) == 128 and S._line(64 * 2) == 128 and S._line(16 * 4) == 128
    # a deeper pipeline never makes the latency-bound step slower
    base = S.Cfg(S.KIND_TILED, 64, 64, 32, 2, 2, 2, 1)
    deeper = S.Cfg(S.KIND_TILED, 64, 64, 32, 2, 2, 4, 1)
    assert S.model_time(1000, 1000, 8192, S.BF16, deeper, d) <= S.model_time(1000, 1000, 8192, S.BF16, base, d)
    # split-K costs the slab writes and the second pass
    s1 = S.Cfg(S.KIND_TILED, 128, 128, 64, 2, 2, 2, 1)
    s2 = S.Cfg(S.KIND_TILED, 128, 128, 64, 2, 2, 2, 2)
    t_no = S.model_time(8192, 8192, 8192, S.BF16, s1, d)
    t_sk = S.model_time(8192, 8192, 8192, S.BF16, s2, d)
    assert t_sk > t_no          # 4096 tiles already fill the chip: splitting only adds work
    # the second split-K pass is a launch of its own that reads every fp32 slab once and writes C
    M, Nn, K = 1000, 1000, 8192
    c4 = S.Cfg(S.KIND_TILED, 128, 128, 64, 2, 4, 3, 4)
    assert S.model_time(M, Nn, K, S.BF16_F32OUT, c4, d) >= (4 * 4 * M * Nn + 4 * M * Nn) / d.bw + 2 * d.t0
    sk = S.Cfg(S.KIND_SKINNY, 16, 128, 32, 4, 1, 2, 2)
    assert S.model_time(16, 28672, 8192, S.BF16, sk, d) >= (4 * 2 * 16 * 28672 + 2 * 16 * 28672) / d.bw + 2 * d.t0
    # the HBM floor binds the 16-row decode
    dec = S.model_time(16, 28672, 8192, S.BF16, S.Cfg(S.KIND_TILED, 32, 128, 64, 1, 2, 4, 1), d)
    floor = (2 * (16 * 8192 + 8192 * 28672) + 2 * 16 * 28672) / (d.bw * d.hbm_eff)
    assert dec >= floor + d.t0


def test_skinny_only_for_small_m_and_bf16():
    for M, N, K, dt in SHAPES:
        kinds = {c.kind for c in S.enumerate_feasible(M, N, K, dt)}
        if M <= 64 and dt != S.F32 and S.shape_aligned(N, K, dt):
            assert S.KIND_SKINNY in kinds
        else:
            assert S.KIND_SKINNY not in kinds
        assert (S.KIND_UNALIGNED in kinds) == (not S.shape_aligned(N, K, dt))


def test_choice_tie_break_is_first_in_canonical_order():
    feas = S.enumerate_feasible(4100, 3000, 1000, S.BF16)
    assert feas == sorted(feas)
    best, bt = S.model_choice(4100, 3000, 1000, S.BF16)
    ties = [c for c in feas if S.model_time(4100, 3000, 1000, S.BF16, c) == bt]
    assert best == ties[0]


def test_shape_buckets():
    # a handful of keys for every batch size a decode step can have
    keys = [S.bucket_m(M) for M in range(1, 257)]
    assert sorted(set(keys)) == [16, 32, 48, 64, 128, 256]
    assert all(k >= M for M, k in zip(range(1, 257), keys))           # tuned at the bucket's largest M
    assert all(S.bucket_m(k) == k for k in set(keys))                  # a key is its own bucket
    assert [S.bucket_m(M) for M in (1, 16, 17, 33, 48, 49, 64, 65, 128, 129, 256)] == \
        [16, 16, 32, 48, 48, 64, 64, 128, 128, 256, 256]
    assert [S.bucket_m(M) for M in (0, 257, 1000, 4100)] == [0, 257, 1000, 4100]   # exact keys


@pytest.mark.parametrize("N,K,dt", [(28672, 8192, S.BF16), (1032, 1064, S.BF16_F32OUT), (1000, 8192, S.F32),
                                    (33, 630, S.BF16)])
def test_bucket_configuration_fits_every_m_of_the_bucket(N, K, dt):
    # what is feasible at a bucket's key is feasible for every M the bucket serves
    for key in (16, 32, 48, 64, 128, 256):
        members = [M for M in range(1, 257) if S.bucket_m(M) == key]
        feas = S.enumerate_feasible(key, N, K, dt)
        assert feas
        for c in feas:
            for M in (members[0], members[len(members) // 2], members[-1]):
                assert S.check(M, N, K, dt, c) == S.OK, (key, M, c)


# ---------------------------------------------------------------- register file and occupancy
# The oracle counts resident workgroups from the compiler's allocation
# (oracle/kernel_allocation.json, a fixed input).  Its register-file rule is
# pinned against the compiler's own occupancy figure for every compiled
# kernel; the compiler also bounds the waves by LDS, rounding the waves a CU's
# worth of workgroups gives each SIMD up.

def _compiler_occupancy(vgpr, agpr, lds, w, dev=S.MI355X):
    occ = S.waves_per_simd_alloc(vgpr, agpr, dev)
    if lds > 0:
        occ = min(occ, S.cdiv((dev.lds_cu // lds) * w, dev.simds))
    return occ


def _cfg_of(key):
    """The configuration an allocation-table key names (split_k = 1, or the
    compiled K groups of a sliced-K kernel)."""
    return key[1:8] + (key[8] if key[1] == S.KIND_SLICEDK else 1,)


def _waves(key):
    """Waves per workgroup of an allocation-table key: wgm for the skinny
    kind, wgm x wgn x the compiled K groups for sliced-K, wgm x wgn else."""
    kind, wgm, wgn, kg = key[1], key[5], key[6], key[8]
    return wgm * (1 if kind == S.KIND_SKINNY else wgn) * (kg if kind == S.KIND_SLICEDK else 1)


def test_register_file_rule_reproduces_the_compilers_occupancy():
    table = S.allocation_table()
    assert len(table) > 1000
    for key, (vgpr, agpr, lds, scratch, occ) in table.items():
        w = _waves(key)
        assert _compiler_occupancy(vgpr, agpr, lds, w) == occ, (key, vgpr, agpr, lds, occ)


def test_register_file_rule_closed_forms():
    d = S.MI355X
    # 512 registers per lane: a wave of 128 registers leaves room for four
    assert S.waves_per_simd_alloc(64, 64, d) == 4
    # VGPRs round up to 4, the sum to 8: 61 + 3 -> 64 + 3 -> 72 -> 7 waves
    assert S.waves_per_simd_alloc(61, 3, d) == 7
    assert S.waves_per_simd_alloc(256, 256, d) == 1
    # at most 8 waves per SIMD however few registers
    assert S.waves_per_simd_alloc(8, 0, d) == 8
    # a planted mistake (AGPRs not counted) fails the pin above
    bad = 0
    for key, (vgpr, agpr, lds, scratch, occ) in S.allocation_table().items():
        w = _waves(key)
        o = S.waves_per_simd_alloc(vgpr, 0, d)
        if lds > 0:
            o = min(o, S.cdiv((d.lds_cu // lds) * w, d.simds))
        bad += o != occ
    assert bad > 50


def test_bf16_accumulators_are_exactly_the_agprs():
    # the bf16 tiled kernel keeps its BM x BN / (64 W) fp32 accumulators in AGPRs
    n = 0
    for key, (vgpr, agpr, lds, scratch, occ) in S.allocation_table().items():
        in_bf16, kind = key[0], key[1]
        if in_bf16 == 1 and kind == S.KIND_TILED:
            c = S.Cfg(*key[1:8], 1)
            assert agpr == S.acc_regs(c), key
            assert lds == S.lds_bytes(c, S.BF16), key
            n += 1
    assert n > 500


def test_resident_blocks_from_the_allocation():
    d = S.MI355X
    # 256 x 256 x 64 tile, 2 x 4 waves: 128 AGPRs of accumulators per lane,
    # 128 KiB of LDS -- one workgroup per CU whatever the registers allow
    c = S.Cfg(S.KIND_TILED, 256, 256, 64, 2, 4, 2, 1)
    vgpr, agpr, lds, scratch = S.compiled_alloc(S.BF16, c)
    assert lds == 2 * (256 * 64 + 64 * 256) * 2 and scratch == 0
    assert S.resident_blocks(c, S.BF16, d) == 1
    # a configuration without a compiled kernel falls back to the estimate
    assert S.compiled_alloc(S.BF16, S.Cfg(S.KIND_TILED, 256, 256, 128, 2, 4, 2, 1)) is None
    # the H100 replica never looks at the allocation
    assert S.resident_blocks(c, S.BF16, S.H100_REPLICA) == S.blocks_per_cu(c, S.BF16, S.H100_REPLICA)
    # wherever the two counts differ, the model prices the compiler's
    diff = 0
    for key in S.allocation_table():
        c = S.Cfg(*_cfg_of(key))
        dt = S.BF16 if key[0] else S.F32
        if S.check_static(dt, c) == S.OK and S.resident_blocks(c, dt, d) != S.blocks_per_cu(c, dt, d):
            diff += 1
    assert diff > 0


def test_spilling_kernels_are_rejected():
    spilling = [k for k, v in S.allocation_table().items() if v[3] > 0]
    assert spilling
    for key in spilling:
        c = S.Cfg(*_cfg_of(key))
        dt = S.BF16 if key[0] else S.F32
        M = c.bm if c.kind == S.KIND_SKINNY else 1024
        Nn, K = 1024, 1024
        assert S.check(M, Nn, K, dt, c) == S.R_SPILL, key
    # the estimate is only the pre-build filter: it lets through every kernel
    # that was compiled, and those that spill are caught by the rule above
    for key in S.allocation_table():
        c = S.Cfg(*_cfg_of(key))
        dt = S.BF16 if key[0] else S.F32
        assert S.check_static(dt, c) == S.OK


# ---------------------------------------------------------------- skinny branch of the model
def _neutral_skinny(**kw):
    # no latency limit on the stream (a vanishing latency), no per-CU limit,
    # no efficiency factors, no launch overhead
    base = dict(lat_mem=1e-30, cu_bw=1e30, skinny_eff=1.0, hbm_eff=1.0, t0=0.0)
    base.update(kw)
    return dataclasses.replace(S.MI355X, **base)


def test_skinny_model_closed_forms():
    M, Nn, K = 16, 28672, 8192
    comp = 2 * (M * K + K * Nn) + 2 * M * Nn
    c = S.Cfg(S.KIND_SKINNY, 16, 128, 32, 4, 1, 2, 1)
    d = _neutral_skinny()
    # memory-bound: the compulsory bytes at the HBM rate, nothing else
    assert S.model_time(M, Nn, K, S.BF16, c, d) == pytest.approx(comp / d.bw, rel=1e-12)
    # the achievable fraction divides the stream time
    d2 = _neutral_skinny(skinny_eff=0.5)
    assert S.model_time(M, Nn, K, S.BF16, c, d2) == pytest.approx(2 * comp / d.bw, rel=1e-12)
    # too few loads in flight: bytes in flight = resident waves x 64 lanes x
    # stages x 8 x 16 bytes; with a latency that makes them half of bw x latency,
    # the stream runs at half the rate
    tiles = S.cdiv(Nn, 128)
    w = c.wgm
    resident = min(tiles * w, d.n_cu * S.resident_blocks(c, S.BF16, d) * w)
    inflight = resident * 64.0 * c.stages * 8 * 16
    d3 = _neutral_skinny(lat_mem=2 * inflight / d.bw)
    assert S.model_time(M, Nn, K, S.BF16, c, d3) == pytest.approx(2 * comp / d.bw, rel=1e-12)
    # per-CU limit: 224 active workgroups each at a quarter of the share the
    # HBM rate would give them
    d4 = _neutral_skinny(cu_bw=d.bw / (4 * min(tiles, d.n_cu)))
    assert S.model_time(M, Nn, K, S.BF16, c, d4) == pytest.approx(4 * comp / d.bw, rel=1e-12)
    # compute-bound: padded rows count (17 rows run as 32)
    d5 = _neutral_skinny(peak_bf16=1e9)
    c32 = S.Cfg(S.KIND_SKINNY, 32, 128, 32, 4, 1, 2, 1)
    assert S.model_time(17, Nn, K, S.BF16, c32, d5) == pytest.approx(2.0 * 32 * Nn * K / 1e9, rel=1e-12)
    # split-K adds the fp32 slabs to the stream and the second pass after it
    cs = S.Cfg(S.KIND_SKINNY, 16, 128, 32, 4, 1, 2, 2)
    slabs = 4.0 * 2 * M * Nn
    want = (comp + slabs) / d.bw + (slabs + 2 * M * Nn) / d.bw
    assert S.model_time(M, Nn, K, S.BF16, cs, d) == pytest.approx(want, rel=1e-12)


# ---------------------------------------------------------------- stream-K partition
def _simulate_streamk(tail, ks, G):
    """Brute force: cut the tail's iterations into min(G, I) contiguous ranges
    the plain way, list every workgroup's pieces (tile, first K step, end)."""
    I = tail * ks
    G = min(G, I)
    bounds = [g * I // G for g in range(G + 1)]
    pieces = {}
    for g in range(G):
        it = bounds[g]
        while it < bounds[g + 1]:
            j, kb = divmod(it, ks)
            ke = min(ks, kb + bounds[g + 1] - it)
            pieces.setdefault(j, []).append((g, kb, ke))
            it += ke - kb
    return pieces


@pytest.mark.parametrize("tail,ks,G", [(33, 128, 256), (16, 128, 256), (204, 16, 256), (1, 5, 8), (7, 3, 8),
                                       (255, 1, 256), (81, 256, 256), (3, 1, 8)])
def test_streamk_partition_against_brute_force(tail, ks, G):
    pieces = _simulate_streamk(tail, ks, G)
    I = tail * ks
    wgs = min(G, I)
    smax = 0
    total = 0
    for j in range(tail):
        ps = pieces[j]
        # the pieces of a tile cover its K steps once, in order, from consecutive workgroups
        assert ps[0][1] == 0 and ps[-1][2] == ks
        assert all(a[2] == b[1] for a, b in zip(ps, ps[1:]))
        assert [p[0] for p in ps] == list(range(ps[0][0], ps[0][0] + len(ps)))
        # the owner formula names the workgroup of a tile's first and last step
        assert S.sk_owner(j * ks, I, wgs) == ps[0][0] and S.sk_owner((j + 1) * ks - 1, I, wgs) == ps[-1][0]
        smax = max(smax, len(ps))
        total += len(ps) if len(ps) >= 2 else 0
    # no workgroup holds more than two pieces, nor more than ceil(I / G) steps
    per_g = {}
    for j, ps in pieces.items():
        for g, kb, ke in ps:
            per_g.setdefault(g, []).append(ke - kb)
    assert len(per_g) == wgs
    assert all(len(v) <= 2 and 1 <= sum(v) <= S.cdiv(I, wgs) for v in per_g.values())
    # the plan's counts agree (a configuration with G = CUs x resident blocks)
    dev = dataclasses.replace(S.MI355X, n_cu=G)
    c = S.Cfg(S.KIND_STREAMK, 256, 256, 64, 2, 4, 2, 1)
    assert S.resident_blocks(c, S.BF16, dev) == 1
    M, Nn = 256 * (G + tail), 256
    plan = S.streamk_plan(M, Nn, 64 * ks, c, dev)
    assert (plan["G"], plan["dp"], plan["tail"], plan["ks"]) == (G, G, tail, ks)
    assert plan["wgs"] == wgs and plan["smax"] == smax and plan["pieces"] == total
    assert plan["segmax"] == max(len(v) for v in per_g.values())
    assert plan["blocks"] == G + wgs and S.grid(M, Nn, c, dev, 64 * ks) == (G + tail, G + wgs)


def test_streamk_model_closed_form():
    # compute only (no LDS, L2, latency, store or fixup costs): a full round
    # plus the tail's K steps spread over a round, against two rounds
    d = dataclasses.replace(S.MI355X, lds_bw_cu=1e30, cu_bw=1e30, lat_step=0.0, lat_l2=0.0, w1_eff=1.0, bw=1e30, t0=0.0)
    sk = S.Cfg(S.KIND_STREAMK, 256, 256, 64, 2, 4, 2, 1)
    dp = S.Cfg(S.KIND_TILED, 256, 256, 64, 2, 4, 2, 1)
    M, Nn, K = 256 * 17, 256 * 17, 8192            # 289 tiles: one round of 256 and a tail of 33
    step = 2.0 * 256 * 256 * 64 / (d.peak_bf16 / (d.n_cu * d.simds) * d.simds)
    assert S.model_time(M, Nn, K, S.BF16, dp, d) == pytest.approx(2 * 128 * step, rel=1e-12)
    assert S.model_time(M, Nn, K, S.BF16, sk, d) == pytest.approx((128 + S.cdiv(33 * 128, 256)) * step, rel=1e-12)
    # no tail: the stream-K kind would be the data-parallel one, so it is not a candidate
    assert S.check(4096, 4096, K, S.BF16, sk) == S.R_SHAPE
    # K = 0 has nothing to spread; fp32 has no stream-K kernel
    assert S.check(4096, 4096, 0, S.BF16, sk) == S.R_SHAPE
    assert S.check(4096, 4096, 64, S.F32, sk) != S.OK


def test_streamk_pieces_restart_the_tile_loop():
    # Every piece a stream-K workgroup runs is a run of the tile loop of its
    # own: it starts with one latency and issues the stages of zero-filling
    # transfers past its K range, as a whole tile does.  289 tiles of 256 x 256
    # (one round of 256 and a tail of 33; 33 x 128 steps over 256 workgroups
    # cross tile boundaries, so some run two pieces) against 288 (a tail of 32:
    # 16 steps each, 8 to a tile, one piece per workgroup).
    sk = S.Cfg(S.KIND_STREAMK, 256, 256, 64, 2, 4, 2, 1)
    K = 8192
    two, one = (256 * 289, 256), (256 * 288, 256)
    assert S.streamk_plan(*two, K, sk)["segmax"] == 2 and S.streamk_plan(*one, K, sk)["segmax"] == 1
    # the L2-to-CU rate alone: a step moves 256 A rows of one 128-byte line and
    # four 64-column B blocks of 64 rows; the data-parallel round pays 2 stages
    # past its range, the stream-K one 2 per piece
    d = dataclasses.replace(S.MI355X, peak_bf16=1e30, lds_bw_cu=1e30, lat_step=0.0, lat_l2=0.0, w1_eff=1.0,
                            bw=1e30, t0=0.0)
    l2 = (256 * 128 + 64 * 4 * 128) / d.cu_bw
    assert S.model_time(*two, K, S.BF16, sk, d) == pytest.approx((128 + 17 + 2 + 2 * 2) * l2, rel=1e-12)
    assert S.model_time(*one, K, S.BF16, sk, d) == pytest.approx((128 + 16 + 2 + 2 * 1) * l2, rel=1e-12)
    # latency alone: every step waits latency / (stages - 1), every run of the
    # loop one latency more (the round of whole tiles, then each piece)
    lat = 1e-6
    d = dataclasses.replace(S.MI355X, peak_bf16=1e30, lds_bw_cu=1e30, cu_bw=1e30, lat_step=lat, lat_l2=lat,
                            w1_eff=1.0, bw=1e30, t0=0.0)
    assert S.model_time(*two, K, S.BF16, sk, d) == pytest.approx((128 + 17) * lat + (1 + 2) * lat, rel=1e-12)
    assert S.model_time(*one, K, S.BF16, sk, d) == pytest.approx((128 + 16) * lat + (1 + 1) * lat, rel=1e-12)


def test_padded_path_closed_form():
    # an unaligned shape on the tiled kind: memory terms only (everything else
    # made free).  Both K and N ragged: the copies read A [256 x 777] and
    # B [777 x 1001] and write
    # A' [256 x 784] and B' [784 x 1008]; the kernel on the padded problem
    # moves its compulsory bytes and writes one fp32 slab [256 x 1008] (split
    # 1); the output pass reads that slab and writes 256 x 1008 outputs
    d = dataclasses.replace(S.MI355X, peak_bf16=1e30, lds_bw_cu=1e30, cu_bw=1e30, lat_step=0.0, lat_l2=0.0,
                            w1_eff=1.0, t0=0.0)
    c = S.Cfg(S.KIND_TILED, 128, 128, 64, 2, 4, 2, 1)
    M, Nn, K = 256, 1001, 777
    assert S.padded_path(Nn, K, S.BF16, c, d) and (S.pad_extent(Nn, S.BF16), S.pad_extent(K, S.BF16)) == (1008, 784)
    assert S.check(M, Nn, K, S.BF16, c, d) == S.OK
    rate = d.bw * d.hbm_eff
    copies = 2 * (256 * 777 + 777 * 1001 + 256 * 784 + 784 * 1008)
    compulsory = 2 * (256 * 784 + 784 * 1008) + 2 * 256 * 1008
    slab = 4 * 256 * 1008
    want = (compulsory + slab) / rate + (slab + 2 * 256 * 1008) / rate + copies / rate
    assert S.model_time(M, Nn, K, S.BF16, c, d) == pytest.approx(want, rel=1e-12)
    # the same tiles on the aligned shape 256 x 1008 x 784 skip the copies,
    # store C directly and need no output pass
    aligned = S.model_time(M, 1008, 784, S.BF16, c, d)
    assert aligned == pytest.approx(compulsory / rate, rel=1e-12)
    # only K ragged (N = 1008): A alone is copied, B is read in place and the
    # kernel stores C itself -- no slab, no output pass
    copies_a = 2 * (256 * 777 + 256 * 784)
    want_k = compulsory / rate + copies_a / rate
    assert S.model_time(M, 1008, K, S.BF16, c, d) == pytest.approx(want_k, rel=1e-12)
    # ... and with split 2 the usual split-K slabs and second pass
    c2 = S.Cfg(S.KIND_TILED, 128, 128, 64, 2, 4, 2, 2)
    slabs2 = 2 * slab
    want_k2 = (compulsory + slabs2) / rate + (slabs2 + 2 * 256 * 1008) / rate + copies_a / rate
    assert S.model_time(M, 1008, K, S.BF16, c2, d) == pytest.approx(want_k2, rel=1e-12)
    # only N ragged (K = 784): B alone is copied, then slab and output pass
    copies_b = 2 * (784 * 1001 + 784 * 1008)
    want_n = (compulsory + slab) / rate + (slab + 2 * 256 * 1008) / rate + copies_b / rate
    assert S.model_time(M, Nn, 784, S.BF16, c, d) == pytest.approx(want_n, rel=1e-12)
    # the H100 replica keeps the page's rules: no alignment rule, no padding
    assert not S.padded_path(Nn, K, S.BF16, c, S.H100_REPLICA)


def test_sliced_k_rules_closed_forms():
    d = S.MI355X
    SK = S.KIND_SLICEDK
    # the workgroup holds wgm x wgn x split_k waves; each K group takes whole
    # MFMA slices (bf16 32 k, fp32 16 k) of every stage
    c = S.Cfg(SK, 32, 64, 128, 1, 2, 2, 4)
    assert S.waves_per_block(c) == 8 and S.k_groups(c) == 4 and S.cta_splits(c) == 1
    assert S.check(256, 256, 1024, S.BF16, c, d) == S.OK
    assert S.check(256, 256, 1024, S.BF16, S.Cfg(SK, 32, 64, 64, 1, 2, 2, 4), d) == S.R_DIV     # 64 k: two slices
    assert S.check(256, 256, 1024, S.F32, S.Cfg(SK, 32, 32, 32, 1, 1, 2, 4), d) == S.R_DIV      # 32 k: two slices
    assert S.check(256, 256, 1024, S.F32, S.Cfg(SK, 32, 32, 64, 1, 1, 2, 4), d) == S.OK
    # the other groups' fp32 sums (3 x 64 x 64 x 4 = 48 KiB) must fit in the
    # stage buffers (2 x (64 x 32 + 32 x 64) x 4 = 32 KiB)
    big = S.Cfg(SK, 64, 64, 32, 1, 1, 2, 2)
    assert S.lds_bytes(big, S.F32) == 32 * 1024 and (2 - 1) * 64 * 64 * 4 <= 32 * 1024
    assert S.check(256, 256, 1024, S.F32, big, d) == S.OK
    assert S.check_static(S.F32, S.Cfg(SK, 64, 64, 64, 1, 1, 2, 4)) == S.OK          # 64 KiB >= 48 KiB
    # 64 x 256 bf16 tiles, 4 groups: the stages (160 KiB) fit the LDS, the
    # other groups' sums (3 x 64 x 256 x 4 = 192 KiB) do not
    wide = S.Cfg(SK, 64, 256, 128, 1, 1, 2, 4)
    assert S.lds_bytes(wide, S.BF16) == 160 * 1024 <= d.lds_block
    assert S.check_static(S.BF16, wide) == S.R_LDS
    # one launch of one workgroup per tile, the whole K range in each
    assert S.grid(1000, 1000, c, d, 8192) == (32 * 16, 32 * 16)
    assert S.k_per_split(c, 8192) == 8192 and S.k_per_split(c, 1000) == 1024
    # no split-K rule, no partial-sum slabs, no second pass
    assert S._splitk_slabs(1000, 1000, c) == 0.0
    assert S._splitk_pass(1000, 1000, 2, c, d) == 0.0
    # transfers are spread over every wave of the workgroup: (32 + 64) x 128 x 2 / 1 KiB = 24 over 8
    assert S.transfers_per_wave(c, S.BF16) == 3


def test_sliced_k_in_the_per_cu_model():
    # MFMA work alone (LDS, L2, latency and stores negligible, no lone-wave
    # penalty): a block's step is its flops over the SIMDs its waves occupy, so
    # four K groups of one wave run a one-wave tile's step four times as fast
    d = dataclasses.replace(S.MI355X, lds_bw_cu=1e30, cu_bw=1e30, lat_step=0.0, lat_l2=0.0, w1_eff=1.0, bw=1e30)
    one = S.Cfg(S.KIND_TILED, 32, 32, 64, 1, 1, 2, 1)
    four = S.Cfg(S.KIND_SLICEDK, 32, 32, 64, 1, 1, 2, 4)
    M = Nn = 256
    K = 1024
    t1 = S.model_time(M, Nn, K, S.F32, one, d) - d.t0
    t4 = S.model_time(M, Nn, K, S.F32, four, d) - d.t0
    # 64 tiles, one per CU (64 CUs busy): the K loop is 16 steps of 2 x 32 x 32 x 64 flops
    step_flops = 2.0 * 32 * 32 * 64
    simd = d.peak_f32 / (d.n_cu * d.simds)
    assert t1 == pytest.approx(16 * step_flops / simd)
    assert t4 == pytest.approx(16 * step_flops / (4 * simd))
    # the cross-group sum: (g - 1) bm bn fp32 values written and read once in LDS, per tile
    dl = dataclasses.replace(d, lds_bw_cu=1e12)
    red = 8.0 * 3 * 32 * 32 / 1e12
    lds_steps = 16 * (64 * 4 * (1 * (32 + 32) + 32 + 32)) / 1e12   # fragment reads of one group + transfer writes
    t4l = S.model_time(M, Nn, K, S.F32, four, dl) - d.t0
    assert t4l == pytest.approx(max(16 * step_flops / (4 * simd), lds_steps) + red)


def test_transfers_past_the_k_range_are_priced():
    # everything but the L2-to-CU rate made negligible: a K step costs its
    # L2-to-CU bytes, and a direct-to-LDS block also pays for the ST stages of
    # zero-filling transfers it issues past its K range
    d = dataclasses.replace(S.MI355X, peak_bf16=1e30, lds_bw_cu=1e30, lat_step=0.0, lat_l2=0.0, w1_eff=1.0,
                            bw=1e30, t0=0.0)
    two = S.Cfg(S.KIND_TILED, 128, 128, 64, 2, 2, 2, 1)
    four = S.Cfg(S.KIND_TILED, 128, 128, 64, 2, 2, 4, 1)
    # 64 tiles: one block on each of 64 CUs; a step is 128 A rows and two
    # 64-column B blocks of 64 rows, each row one 128-byte line
    l2_step = 128 * 128 + 64 * 2 * 128
    M, Nn, K = 1024, 1024, 256
    for c in (two, four):
        assert S.check(M, Nn, K, S.BF16, c, d) == S.OK
        t = S.model_time(M, Nn, K, S.BF16, c, d)
        assert t == pytest.approx((K // 64 + c.stages) * l2_step / d.cu_bw)
    # the register-staged kernel of the unaligned kind issues none: eight
    # 32-k steps of 128 A rows (one line each) and 32 B rows of 256 bytes, at
    # the element-load efficiency
    u = S.Cfg(S.KIND_UNALIGNED, 128, 128, 32, 2, 2, 2, 1)
    assert S.check(M, Nn - 4, K - 4, S.BF16, u, d) == S.OK
    u_step = (128 * 128 + 32 * 256) / d.unaligned_eff
    assert S.model_time(M, Nn - 4, K - 4, S.BF16, u, d) == pytest.approx(8 * u_step / d.cu_bw)
