"""Pins of the oracle's allocator over every candidate width (allocator 1).

The pages define the top-p% rule between two widths only (TAH-Quant §3.2);
the greedy allocator is this library's reading of it for three or more widths:
each tile's upgrade c_j -> c_(j+1) is ranked by the base-2 logarithm of its
gain per bit, kappa = 2 H + lambda_j, lambda_j = log2((Delta(c_j) -
Delta(c_(j+1))) / (c_(j+1) - c_j)), Delta(b) = (2^b - 1)^-2, and upgrades are
taken in that order while the sample's bits last. What pins it:
  - the two-width case equals the pages' top-k rule (itself pinned by brute
    force in test_oracle_pins.py);
  - brute force over every allocation of tiny samples: none that spends at most
    the bits the greedy spent has a lower objective sum w_u Delta(b_u),
    w_u = 2^(2 H_u) (the greedy stops at a threshold gain per bit, so it
    minimizes the Lagrangian and is optimal for the bits it spends);
  - the walk stops only when the next upgrade in order no longer fits;
  - lambda_j from exact rational arithmetic;
  - payload invariants: fixed size, budget, level map, block table, and with
    two candidates the same decoded tensor as the top-p% payload.
"""

import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

import synth


def delta(b):
    return Fraction(1, (2**b - 1) ** 2)


def test_lambda_from_exact_fractions(ref):
    for cands in [(2, 3, 4, 8), (1, 2, 3, 4), (3, 4), (4, 8), (1, 8), (5, 6, 7)]:
        lam = ref.greedy_lambda(cands)
        for j in range(len(cands) - 1):
            gain = (delta(cands[j]) - delta(cands[j + 1])) / (cands[j + 1] - cands[j])
            want = math.log2(gain.numerator) - math.log2(gain.denominator)
            assert abs(float(lam[j]) - want) <= 2.0**-20 * max(1.0, abs(want)), (cands, j)
        # Delta is convex: gains per bit fall with j, so a tile's upgrades come in order
        assert np.all(np.diff(lam) < 0)


@pytest.mark.parametrize("cands", [(3, 4), (2, 3), (4, 8), (1, 8)])
def test_two_widths_is_the_pages_top_k(ref, cands):
    g = np.random.default_rng(3)
    c1, c2 = cands
    for trial in range(200):
        N = int(g.integers(1, 40))
        H = (g.choice([0.5, 1.0, 2.5, 4.0], N) if trial % 2 else g.random(N) * 6).astype(np.float32)
        k = int(g.integers(0, N + 1))
        extra = int(g.integers(0, c2 - c1))  # bits that cannot buy one more upgrade
        lv = ref.allocate_greedy(H, cands, k * (c2 - c1) + extra)
        assert np.array_equal(lv, ref.allocate(H, k)), (H, k)


def objective(H, cands, levels):
    return sum(2.0 ** (2.0 * float(h)) * float(delta(cands[l])) for h, l in zip(H, levels))


def test_brute_force_optimal_for_the_bits_spent(ref):
    g = np.random.default_rng(11)
    for trial in range(300):
        n = int(g.integers(3, 5))
        cands = tuple(sorted(g.choice(np.arange(1, 9), n, replace=False).tolist()))
        N = int(g.integers(1, 6))
        H = (g.random(N) * 6).astype(np.float32)
        R = int(g.integers(0, (cands[-1] - cands[0]) * N + 1))
        lv = ref.allocate_greedy(H, cands, R)
        spent = sum(cands[l] - cands[0] for l in lv)
        assert spent <= R
        got = objective(H, cands, lv)
        best = min(objective(H, cands, alt) for alt in itertools.product(range(n), repeat=N)
                   if sum(cands[l] - cands[0] for l in alt) <= spent)
        assert got <= best * (1 + 1e-5), (cands, H, R, lv)


def test_walk_stops_only_when_the_next_upgrade_does_not_fit(ref):
    """Brute force on the order itself: list every (tile, upgrade) pair with its
    gain per bit in exact arithmetic, sort, and check that the greedy takes
    exactly the longest prefix that fits."""
    g = np.random.default_rng(5)
    for trial in range(300):
        cands = (2, 3, 4, 8) if trial % 3 else (1, 2, 5)
        N = int(g.integers(1, 30))
        H = np.round(g.random(N) * 48).astype(np.float32) / np.float32(8)  # exact, with ties
        R = int(g.integers(0, (cands[-1] - cands[0]) * N + 1))
        lv = ref.allocate_greedy(H, cands, R)
        ups = []
        for u in range(N):
            for j in range(len(cands) - 1):
                ups.append((u, j, cands[j + 1] - cands[j]))
        # the order: kappa = 2H + lambda_j, H on a grid of 1/8 (exact in fp32),
        # so equal entropies give equal keys and the tile index decides; sort
        # by (2H + lambda_j) in float64, then u, then j
        lam = [float(v) for v in ref.greedy_lambda(cands)]
        ups.sort(key=lambda e: (-(2.0 * float(H[e[0]]) + lam[e[1]]), e[0], e[1]))
        want = np.zeros(N, np.uint8)
        spent = 0
        for u, j, cost in ups:
            if spent + cost > R:
                break
            spent += cost
            assert want[u] == j
            want[u] += 1
        assert np.array_equal(lv, want), (cands, H, R)


def test_monotone_in_entropy(ref):
    g = np.random.default_rng(9)
    for trial in range(100):
        cands = (2, 3, 4, 8)
        N = int(g.integers(2, 200))
        H = (g.random(N) * 6).astype(np.float32)
        R = int(g.integers(0, 6 * N + 1))
        lv = ref.allocate_greedy(H, cands, R)
        o = np.argsort(-H.astype(np.float64), kind="stable")
        assert np.all(np.diff(lv[o].astype(int)) <= 0)


def test_all_or_nothing_budgets(ref):
    H = np.linspace(0, 5, 37).astype(np.float32)
    assert np.all(ref.allocate_greedy(H, (2, 3, 4, 8), 0) == 0)
    assert np.all(ref.allocate_greedy(H, (2, 3, 4, 8), 6 * 37) == 3)
    assert np.all(ref.allocate_greedy(H, (4,), 100) == 0)


# ---------------------------------------------------------------- plan and payload ----
def gp(**kw):
    base = dict(tile=32, tokens_per_sample=0, bit_budget=3.5, candidates=(2, 3, 4, 8), tau=2.0, allocator=1)
    return synth.Params(**{**base, **kw})


def test_plan_numbers(ref):
    # 64 x 256 at G = 32: 512 tiles, one sample; R = floor((3.5 - 2) * 512) = 768
    pl = ref.plan(64, 256, gp())
    assert (pl["allocator"], pl["R"], pl["b_lo"], pl["b_hi"], pl["k"]) == (1, 768, 2, 8, 0)
    assert pl["code_bytes"] == (32 // 8) * (2 * 512 + 768)
    assert pl["off_side"] - pl["off_bitmap"] >= 16 * pl["nblocks"]
    # budget above the widest candidate: capped at every tile at 8 bits
    pl = ref.plan(64, 256, gp(bit_budget=9.0))
    assert pl["R"] == 6 * 512 and pl["code_bytes"] == 4 * 8 * 512
    # samples of 16 tokens, A = 64: 64 allocation tiles per sample, R = floor(1.5 * 64)
    pl = ref.plan(64, 256, gp(tokens_per_sample=16, alloc_tile=64))
    assert pl["R"] == 96 and pl["code_bytes"] == 4 * (64 // 8) * (2 * 64 + 96)
    with pytest.raises(ref.OracleError) as e:
        ref.plan(64, 256, gp(allocator=2))
    assert e.value.code == 1


def unpack_levels(P, pl):
    words = P[pl["off_bitmap"]:pl["off_bitmap"] + 16 * pl["nblocks"]].view(np.uint32)
    t = np.arange(pl["tiles"])
    return ((words[t // 16] >> (2 * (t % 16)).astype(np.uint32)) & 3).astype(np.uint8)


@pytest.mark.parametrize("A,S", [(0, 0), (0, 16), (64, 8), (256, 0)])
def test_payload_levels_table_and_budget(ref, A, S):
    p = gp(alloc_tile=A, tokens_per_sample=S)
    x = synth.random_tensor(64, 256, synth.F32, 21, n_out=4, mult=30)
    P = ref.encode(x, p)
    pl = ref.plan(64, 256, p)
    assert P.size == pl["total"] and P[124] == 1
    lv = unpack_levels(P, pl)
    st = ref.tile_stats(x, p)
    assert np.array_equal(lv, st["hi"])
    w = np.array(p.candidates)[lv]
    # per sample: the widths above c_1, counted once per allocation tile, fit R
    kA = pl["kA"]
    per = ((w - p.candidates[0]).reshape(pl["nsamples"], -1)).sum(1) // kA
    assert np.all(per <= pl["R"])
    assert np.all(lv.reshape(-1, kA) == lv.reshape(-1, kA)[:, :1])
    # the block table is the running width sum at each run of 64 tiles
    tab = P[pl["off_table"]:pl["off_table"] + 4 * pl["nblocks"]].view(np.uint32)
    cs = np.concatenate([[0], np.cumsum(w)])
    assert np.array_equal(tab, cs[np.arange(pl["nblocks"]) * 64].astype(np.uint32))
    # the unused tail of the code section is zero
    used = pl["off_codes"] + int(cs[-1]) * pl["G"] // 8
    assert not P[used:].any()
    # more than two widths really occur (per-tile allocation; token-level
    # allocation tiles of similar rows use two)
    assert len(np.unique(lv)) >= (3 if A == 0 else 2)
    # and the decoder reads it back, with the reconstruction error of each tile's width
    y = ref.decode(P, 64, 256, p)
    assert np.isfinite(y).all()
    xt, yt = x.reshape(-1, 32).astype(np.float64), y.reshape(-1, 32).astype(np.float64)
    for i in range(xt.shape[0]):
        s = float(st["scale"][i])
        e = np.linalg.norm(xt[i] - yt[i]) if st["flag"][i] else np.abs(xt[i] - yt[i]).max()
        assert e <= s / 2 * 1.001 + 1e-6 * (1 + np.abs(xt[i]).max()) * 32


def test_two_candidates_decode_like_top_p(ref):
    x = synth.random_tensor(96, 512, synth.BF16, 5, n_out=3, mult=50)
    for cands, budget in [((3, 4), 3.8), ((4, 8), 5.0), ((2, 3), 2.25)]:
        p0 = synth.Params(tile=64, tokens_per_sample=32, bit_budget=budget, candidates=cands, tau=2.0)
        p1 = synth.Params(**{**p0.__dict__, "allocator": 1})
        y0 = ref.decode(ref.encode(x, p0), 96, 512, p0)
        y1 = ref.decode(ref.encode(x, p1), 96, 512, p1)
        assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32)), cands


def test_decode_rejects_mismatches(ref):
    p = gp()
    x = synth.random_tensor(64, 256, synth.F32, 2, n_out=4, mult=30)
    P = ref.encode(x, p)
    pl = ref.plan(64, 256, p)
    with pytest.raises(ref.OracleError) as e:  # read as a top-p% payload
        ref.decode(P, 64, 256, gp(allocator=0))
    assert e.value.code == 5
    # a level out of range (index 3 with three candidates)
    p3 = gp(candidates=(2, 3, 8), bit_budget=3.0)
    Q = ref.encode(x, p3)
    pl3 = ref.plan(64, 256, p3)
    Q[pl3["off_bitmap"]] |= 3
    with pytest.raises(ref.OracleError) as e:
        ref.decode(Q, 64, 256, p3)
    assert e.value.code == 5
    Q = P.copy()  # a block-table entry off by one
    Q[pl["off_table"] + 4] ^= 1
    with pytest.raises(ref.OracleError) as e:
        ref.decode(Q, 64, 256, p)
    assert e.value.code == 5
