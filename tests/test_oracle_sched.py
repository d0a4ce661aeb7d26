"""Pins of the oracle's host-side algorithms: bubble formula vs a brute-force
simulator, greedy partitioner vs exhaustive search, LPT vs the brute-force
optimum (Graham's bound), and the activation-memory model vs the paper's
printed footprint. CPU only."""
import json
import os
import random
from fractions import Fraction

import pytest

from oracle import sched as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "paper_numbers.json")


def test_bubble_formula_exact_on_its_domain():
    """Section 3.3: total GPU time (M S + N (N-1)) t. The brute-force simulator
    reproduces it exactly whenever S >= N and (M_R = N or R S = 0 mod N)."""
    n_exact = 0
    for N in range(1, 6):
        for MR in range(N, 2 * N + 2):
            for R in range(1, 4):
                for St in range(1, 9):
                    M = MR * R
                    ms, busy, bub = S.simulate_roundpipe(N, M, MR, St)
                    assert busy == M * St
                    if St >= N and (MR == N or (R * St) % N == 0):
                        assert bub == S.bubble_formula(N, M, St), (N, MR, R, St)
                        assert ms * N == M * St + N * (N - 1)
                        n_exact += 1
    assert n_exact > 200


def test_bubble_formula_outside_domain_is_approximate():
    # S < N: a round never fills the GPUs and consecutive rounds land on other
    # GPUs, so the simulated ratio departs from the formula (here it is lower)
    ms, busy, bub = S.simulate_roundpipe(4, 8, 4, 2)
    assert bub != S.bubble_formula(4, 8, 2)
    # M_R > N with R S not a multiple of N: also off the formula
    ms, busy, bub = S.simulate_roundpipe(2, 3, 3, 3)
    assert bub == Fraction(1, 4) and S.bubble_formula(2, 3, 3) == Fraction(2, 11)
    # single GPU: no bubble at all
    assert S.simulate_roundpipe(1, 6, 3, 5)[2] == 0 == S.bubble_formula(1, 6, 5)


def test_bubble_paper_setting_is_small():
    # section 5.8.1 simulates 16 micro-batches on 8 GPUs; with S = 24 stages in one round
    b = S.bubble_formula(8, 16, 24)
    assert b == Fraction(56, 16 * 24 + 56)
    ms, busy, bub = S.simulate_roundpipe(8, 16, 16, 24)
    assert bub <= b + Fraction(1, 100)


def test_simulator_non_uniform_stage_times_bottleneck():
    # the slowest stage bounds throughput: makespan >= M * t_max
    times = [1, 1, 3, 1]
    ms, busy, bub = S.simulate_roundpipe(2, 4, 4, 4, times)
    assert ms >= 4 * 3
    assert busy == 4 * sum(times)


def test_partitioner_greedy_equals_exhaustive():
    rng = random.Random(1234)
    n = 0
    for _ in range(400):
        L = rng.randint(1, 7)
        f = [rng.randint(1, 9) for _ in range(L)]
        b = [max(1, 3 * x + rng.randint(-2, 2)) for x in f]
        h = rng.randint(1, 25)
        mf = [rng.randint(1, 5) for _ in range(L)]
        mb = [rng.randint(1, 8) for _ in range(L)]
        mh = rng.randint(1, 8)
        cap = rng.randint(8, 30)
        M, N = rng.randint(1, 16), rng.randint(1, 8)
        e = S.partition_exhaustive(f, b, h, mf, mb, mh, cap, M, N)
        g = S.partition_greedy(f, b, h, mf, mb, mh, cap, M, N)
        assert (e is None) == (g is None)
        if e is not None:
            n += 1
            assert e[0] == g[0]
            fwd, b1, bwd = g[1], g[2], g[3]
            assert sum(fwd) + b1 == L and b1 + sum(bwd) == L  # section 3.2 constraints
    assert n > 300


def test_partitioner_greedy_equals_exhaustive_real_times():
    # measured stage times are real numbers: a backward group summed back to
    # front may differ from the same candidate summed front to back by a few
    # ulps, which must not turn an exactly fitting stage into two
    rng = random.Random(99)
    n = 0
    for _ in range(300):
        L = rng.randint(1, 7)
        f = [rng.uniform(0.5, 9.0) for _ in range(L)]
        b = [3.0 * x + rng.uniform(-1.0, 1.0) for x in f]
        h = rng.uniform(1.0, 25.0)
        mf = [rng.randint(1, 5) for _ in range(L)]
        mb = [rng.randint(1, 8) for _ in range(L)]
        mh, cap = rng.randint(1, 8), rng.randint(8, 30)
        M, N = rng.randint(1, 16), rng.randint(1, 8)
        e = S.partition_exhaustive(f, b, h, mf, mb, mh, cap, M, N)
        g = S.partition_greedy(f, b, h, mf, mb, mh, cap, M, N)
        assert (e is None) == (g is None)
        if e is not None:
            n += 1
            assert abs(e[0] - g[0]) <= 1e-9 * e[0]
    assert n > 200


def test_partitioner_fills_fused_stage_first():
    # section 4.4.2: the greedy fills the first backward stage to capacity, so
    # one more layer in B_1 would exceed the partition's bottleneck time
    f = [1] * 8
    b = [3] * 8
    val, fwd, b1, bwd = S.partition_greedy(f, b, 3, [1] * 8, [1] * 8, 1, 100, 16, 4)
    times = S._stage_times(f, b, 3, fwd, b1, bwd)
    assert (fwd, b1, bwd) == ((6,), 2, (3, 3)) and times == [6, 9, 9, 9]
    assert 3 + 3 * (b1 + 1) > max(times)
    assert val == S.partition_exhaustive(f, b, 3, [1] * 8, [1] * 8, 1, 100, 16, 4)[0]


def test_split_items_cover_exactly():
    sizes = [1000, 10, 4096 * 3 + 5, 7]
    for nw in (1, 2, 3, 5):
        for cap in (0, 777):
            chunks = S.split_items(sizes, nw, align=256, max_chunk=cap)
            total = sum(sizes)
            thr = -(-total // nw)
            if cap:
                thr = min(thr, cap)
            for i, s in enumerate(sizes):
                parts = [(o, n) for (j, o, n) in chunks if j == i]
                assert sum(n for _, n in parts) == s
                off = 0
                for o, n in parts:
                    assert o == off
                    off += n
                if len(parts) > 1:
                    assert all(o % 256 == 0 for o, _ in parts)
                    assert len(parts) == -(-s // thr) or parts[0][1] % 256 == 0


def test_lpt_within_graham_bound_of_bruteforce():
    rng = random.Random(7)
    for _ in range(150):
        m = rng.randint(1, 4)
        sizes = [rng.randint(1, 100) for _ in range(rng.randint(1, 8))]
        win = S.lpt_assign(sizes, m)
        got = S.makespan(sizes, win, m)
        opt = S.optimal_makespan(sizes, m)
        assert opt <= got
        assert got * 3 * m <= (4 * m - 1) * opt  # (4/3 - 1/(3m)) OPT
    # Graham's tight instance for m = 2: 3,3,2,2,2 -> LPT 7, OPT 6
    assert S.makespan([3, 3, 2, 2, 2], S.lpt_assign([3, 3, 2, 2, 2], 2), 2) == 7
    assert S.optimal_makespan([3, 3, 2, 2, 2], 2) == 6


def test_lpt_tie_breaks():
    assert S.lpt_assign([5, 5, 5], 3) == [0, 1, 2]
    assert S.lpt_assign([1, 4, 4, 2], 2) == [1, 0, 1, 0]


def test_activation_footprint_matches_paper():
    g = json.load(open(GOLDEN))["activation_footprint"]
    per = S.activation_bytes_per_layer(g["seq"], g["batch"], g["hidden"], g["kv_hidden"],
                                       g["ffn"], g["e_act"])
    total = per * g["layers"]
    assert total == 73_014_444_032
    assert round(total / 2 ** 30, 3) == g["stated_gb"]  # 68.000 GiB
    ck = S.checkpoint_bytes_per_layer(g["seq"], g["batch"], g["hidden"])
    assert ck == g["seq"] * g["hidden"] * 2
    assert per == 17 * ck  # recomputation keeps 1/17 of the layer's activations here


def test_model_state_bytes_match_paper():
    g = json.load(open(GOLDEN))["model_states"]
    for c in g["cases"]:
        assert c["params_b"] * g["bytes_per_param"] == c["stated_gb"]
