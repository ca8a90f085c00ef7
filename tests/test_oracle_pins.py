"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks an oracle routine against something other than itself: a
closed form, a library routine (numpy, scipy), brute force on tiny inputs, or a
tile worked out by hand (tests/golden/worked_tiles.json). Sources:
TAH-Quant (arXiv 2506.01352v2) Sec. 3.1-3.4 and Appendix F; the Sylvester
Hadamard construction and low-nibble-first packing from arXiv 2306.11987.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg
import scipy.stats

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_tiles.json")
# log2 of the entropy: exact 7-bit mantissa nodes, linear in between. Linear
# interpolation of log2(1 + f) on steps of h = 1/128 is off by at most
# h^2/8 * max|d2/df2 log2(1 + f)| = 2^-14 / 8 / ln 2 < 1.11e-5.
INTERP_BOUND = 1.11e-5
LOG2_BOUND = 1.2e-5  # INTERP_BOUND plus the roundings of the tables and the result (|log2 u| <= 64)


def entropy_tol(a, n_interp=2):
    """Error bound of the oracle entropy of tile a against exact Shannon entropy:
    n_interp interpolated logs (per element and of L; bf16 elements sit on the
    exact nodes), plus G roundings of the fp32 accumulation relative to the
    largest |log2 a_k|, plus the final subtraction."""
    a = np.abs(np.asarray(a, np.float64))
    nz = a[a > 0]
    big = np.abs(np.log2(nz)).max() if nz.size else 0.0
    lgL = abs(math.log2(a.sum())) if a.sum() > 0 else 0.0
    return n_interp * LOG2_BOUND + a.size * 2.0**-23 * (1 + big) + 2.0**-21 * (1 + lgL)


def sylvester(G):
    H = np.array([[1]], dtype=np.int64)
    while H.shape[0] < G:
        H = np.block([[H, H], [H, -H]])
    return H


# ---------------------------------------------------------------- log2 ----
def test_log2s_exact_at_powers_of_two(ref):
    for e in range(-60, 20):
        assert ref.log2s([2.0**e])[0] == np.float32(e)


def test_log2s_bf16_values_are_rounded_log2(ref):
    # every (1 + j/128) 2^e is a node: only the table entry and the sum round
    j = np.arange(128, dtype=np.float64)
    for e in (-40, -7, -1, 0, 1, 5, 30):
        u = ((1.0 + j / 128.0) * 2.0**e).astype(np.float32)
        got = ref.log2s(u).astype(np.float64)
        exact = np.log2(u.astype(np.float64))
        assert np.all(np.abs(got - exact) <= 2.0**-25 + np.spacing(np.abs(got).astype(np.float32)) / 2 * 1.0001)


def test_log2s_error_bound(ref):
    g = np.random.default_rng(1)
    u = np.concatenate([g.uniform(2.0**-40, 1.0, 4000), np.exp2(g.uniform(-40, 1, 4000)),
                        1.0 - np.exp2(-g.uniform(1, 24, 500)), g.uniform(1.0, 2.0, 2000)]).astype(np.float32)
    got = ref.log2s(u)
    err = np.abs(got.astype(np.float64) - np.log2(u.astype(np.float64)))
    assert np.all(err <= INTERP_BOUND + np.spacing(np.abs(got)) + 2.0**-24)
    assert err.max() <= LOG2_BOUND
    # the interpolation error is one-signed (log2 is concave): never above the exact value
    m = (u >= 1.0) & (u < 2.0)
    assert np.all(got[m].astype(np.float64) <= np.log2(u[m].astype(np.float64)) + 2.0**-23)
    assert err[m].max() > 1e-5  # and it is there: the linear segments are not exact


# ---------------------------------------------------------------- Hadamard --
@pytest.mark.parametrize("G", [2, 8, 16, 32, 64, 128])
def test_sylvester_orthogonal_and_matches_scipy(G):
    H = sylvester(G)
    assert np.array_equal(H @ H.T, G * np.eye(G, dtype=np.int64))
    assert np.array_equal(H, scipy.linalg.hadamard(G))
    i, j = np.meshgrid(np.arange(G), np.arange(G), indexing="ij")
    pop = np.vectorize(lambda v: bin(v).count("1"))(i & j)
    assert np.array_equal(H, np.where(pop % 2 == 0, 1, -1))


@pytest.mark.parametrize("G", [8, 16, 32, 64, 128])
def test_fwht_equals_dense_product_on_integers(ref, G):
    g = np.random.default_rng(G)
    H = scipy.linalg.hadamard(G)
    for _ in range(20):
        x = g.integers(-1000, 1000, G)
        y = ref.fwht(x.astype(np.float32))
        assert np.array_equal(y.astype(np.int64), H @ x)
        # H is symmetric and H^2 = G I: the transform twice scales by G
        assert np.array_equal(ref.fwht(y).astype(np.int64), G * x)


@pytest.mark.parametrize("G", [32, 64, 128])
def test_fwht_fp32_error_vs_fp64_dense(ref, G):
    g = np.random.default_rng(7)
    H = scipy.linalg.hadamard(G).astype(np.float64)
    for _ in range(50):
        x = g.standard_normal(G).astype(np.float32) * 10
        y = ref.fwht(x).astype(np.float64)
        exact = H @ x.astype(np.float64)
        bound = math.log2(G) * np.abs(x).sum() * 2.0**-24 * 1.01
        assert np.abs(y - exact).max() <= bound


# ---------------------------------------------------------------- entropy ----
@pytest.mark.parametrize("G", [8, 32, 64, 128])
def test_entropy_closed_forms(ref, G):
    u = np.full(G, 0.37, np.float32)
    assert abs(ref.entropy(u) - math.log2(G)) <= entropy_tol(u)
    u = -np.full(G, 3.0, np.float32)
    assert abs(ref.entropy(u) - math.log2(G)) <= entropy_tol(u)
    one_hot = np.zeros(G, np.float32)
    one_hot[G // 3] = -7.5
    assert abs(ref.entropy(one_hot)) <= 4 * 2.0**-24 * math.log2(7.5)
    for m in (2, 4, 5):
        spikes = np.zeros(G, np.float32)
        spikes[np.arange(m) * (G // m)] = 2.0
        assert abs(ref.entropy(spikes) - math.log2(m)) <= entropy_tol(spikes)
    half = np.zeros(G, np.float32)
    half[:3] = [2.0, 1.0, 1.0]
    assert abs(ref.entropy(half) - 1.5) <= entropy_tol(half)
    assert ref.entropy(np.zeros(G, np.float32)) == 0.0


def test_entropy_matches_scipy_shannon(ref):
    g = np.random.default_rng(3)
    for G in (32, 64, 128):
        for _ in range(100):
            a = (g.standard_normal(G) * np.exp(g.standard_normal())).astype(np.float32)
            a[g.integers(0, G)] *= 50
            p = np.abs(a.astype(np.float64))
            want = scipy.stats.entropy(p / p.sum(), base=2)
            assert abs(ref.entropy(a) - want) <= entropy_tol(a)
            # sign and order of a tile do not matter beyond rounding
            assert abs(ref.entropy(-a[::-1]) - want) <= entropy_tol(a)


def test_entropy_of_bf16_tiles_has_only_rounding_error(ref):
    # bf16 inputs hit the exact log2 nodes: what is left is accumulation rounding
    g = np.random.default_rng(11)
    for G in (32, 64, 128):
        for _ in range(50):
            a = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(
                (g.standard_normal(G) * np.exp(g.standard_normal())).astype(np.float32)))
            p = np.abs(a.astype(np.float64))
            want = scipy.stats.entropy(p / p.sum(), base=2)
            assert abs(ref.entropy(a) - want) <= entropy_tol(a, n_interp=1)


def test_entropy_high_for_spread_low_for_spike(ref):
    # Sec. 3.2: high when energy is spread evenly, low for a sharp outlier
    g = np.random.default_rng(5)
    flat = g.uniform(0.9, 1.1, 64).astype(np.float32)
    spiky = flat.copy()
    spiky[10] = 500
    assert ref.entropy(flat) > 5.9
    p = np.abs(spiky.astype(np.float64))
    assert abs(ref.entropy(spiky) - scipy.stats.entropy(p / p.sum(), base=2)) <= entropy_tol(spiky)
    assert ref.entropy(spiky) < ref.entropy(flat) / 4


# ---------------------------------------------------------------- outlier ----
def test_outlier_against_numpy_sort(ref):
    g = np.random.default_rng(11)
    for _ in range(400):
        G = int(g.choice([8, 32, 64]))
        a = g.standard_normal(G).astype(np.float32)
        if g.random() < 0.5:
            a[g.integers(0, G)] *= 10
        if g.random() < 0.2:  # tied maxima
            a[g.integers(0, G)] = a[np.argmax(np.abs(a))]
        mag = np.abs(a)
        d_np = int(np.argmax(mag))  # first occurrence of the max
        m2_np = np.sort(np.delete(mag, d_np))[-1]
        for tau in (0.0, 2.0, 4.0, math.inf):
            f, d, m1, m2 = ref.outlier(a, tau)
            assert d == d_np and m1 == mag.max() and m2 == m2_np
            want = bool(mag.max() > np.float32(np.float32(tau) * np.float32(m2_np + np.float32(2.0**-40))))
            assert f == want


def test_outlier_tau_semantics(ref):
    a = np.array([0.1, 0.1, 0.1, 3.0, 0.1, 0.1, 0.1, 0.1], np.float32)
    assert ref.outlier(a, 0.0)[0] and ref.outlier(a, 2.0)[0]
    assert not ref.outlier(a, math.inf)[0]
    z = np.zeros(8, np.float32)
    assert not ref.outlier(z, 0.0)[0]  # tau = 0 flags every tile that is not all zero
    flat = np.ones(8, np.float32)
    assert ref.outlier(flat, 0.0)[0] and not ref.outlier(flat, 2.0)[0]
    # ratio exactly tau is not "exceeding" tau
    edge = np.array([4.0, 2.0, 0, 0, 0, 0, 0, 0], np.float32)
    assert not ref.outlier(edge, 2.0)[0]
    edge[0] = np.nextafter(np.float32(4.0), np.float32(5.0))
    assert ref.outlier(edge, 2.0)[0]


# ---------------------------------------------------------------- quantizer ----
@pytest.mark.parametrize("b", [1, 2, 3, 4, 5, 6, 7, 8])
def test_quantizer_bounds(ref, b):
    g = np.random.default_rng(b)
    L = 2**b - 1
    for _ in range(200):
        y = (g.standard_normal(64) * np.exp(g.standard_normal()) + g.standard_normal() * 5).astype(np.float32)
        lo, s, q = ref.quantize(y, b)
        assert lo == y.min()
        assert q.max() <= L and q.min() == 0
        assert np.float32(s).view(np.uint32) & 0xFFFF == 0  # a bf16 value
        assert s >= (np.float64(y.max()) - np.float64(y.min())) / L * (1 - 2**-23)
        yhat = ref.dequantize(q, s, lo, False, 0)
        err = np.abs(yhat.astype(np.float64) - y.astype(np.float64))
        assert err.max() <= s / 2 * (1 + 2**-20) + 4 * np.spacing(np.abs(y).max())


def test_quantizer_error_shrinks_with_bits(ref):
    g = np.random.default_rng(9)
    y = (g.standard_normal((300, 64))).astype(np.float32)
    prev = None
    for b in (1, 2, 3, 4, 5, 6, 7, 8):
        worst = 0.0
        for row in y:
            lo, s, q = ref.quantize(row, b)
            worst = max(worst, float(np.abs(ref.dequantize(q, s, lo, False, 0) - row).max()))
        if prev is not None:
            assert worst < prev * 0.75
        prev = worst


def test_constant_tile_is_exact(ref):
    y = np.full(64, -3.25, np.float32)
    lo, s, q = ref.quantize(y, 3)
    assert s == 0 and lo == -3.25 and not q.any()
    assert np.array_equal(ref.dequantize(q, s, lo, False, 0), y)


def test_one_hot_tile_transforms_to_constant_and_decodes_exactly(ref):
    # swap moves the pivot to index 0; column 0 of H is all ones (Sylvester order),
    # so c e_0 maps to the constant vector c 1: zero range, exact reconstruction
    for G in (8, 32, 64, 128):
        for d in (0, 1, G // 2 + 1, G - 1):
            a = np.zeros(G, np.float32)
            a[d] = -13.0
            f, dd, _, _ = ref.outlier(a, 2.0)
            assert f and dd == d
            x = a.copy()
            x[0], x[d] = x[d], x[0]
            y = ref.fwht(x)
            assert np.all(y == -13.0)
            lo, s, q = ref.quantize(y, 3)
            assert s == 0
            assert np.array_equal(ref.dequantize(q, s, lo, True, d), a)


def test_swap_is_an_involution_and_transform_inverts(ref):
    g = np.random.default_rng(13)
    for G in (32, 64, 128):
        for _ in range(50):
            a = g.standard_normal(G).astype(np.float32)
            d = int(g.integers(0, G))
            x = a.copy()
            x[0], x[d] = x[d], x[0]
            x[0], x[d] = x[d], x[0]
            assert np.array_equal(x, a)
            # 8-bit codec through the transform: ||x - xhat||_2 <= s/2 (orthogonality)
            x = a.copy()
            x[0], x[d] = x[d], x[0]
            y = ref.fwht(x)
            lo, s, q = ref.quantize(y, 8)
            xh = ref.dequantize(q, s, lo, True, d)
            assert np.linalg.norm(xh.astype(np.float64) - a) <= s / 2 * 1.001 + G * 1e-6 * np.abs(y).max()


# ---------------------------------------------------------------- worked tiles ----
def test_worked_tiles_by_hand(ref):
    data = json.load(open(GOLDEN))
    for t in data["tiles"]:
        x = np.array(t["x"], np.float32)
        f, d, m1, m2 = ref.outlier(x, t["tau"])
        assert (f, d, float(m1), float(m2)) == (t["flag"], t["pivot"], t["m1"], t["m2"])
        y = x.copy()
        if f:
            y[0], y[d] = y[d], y[0]
            y = ref.fwht(y)
            assert y.tolist() == t["y_transformed"]
        lo, s, q = ref.quantize(y, t["bits"])
        assert float(lo) == t["lo"] and float(s) == t["scale"]
        assert int(np.float32(s).view(np.uint32) >> 16) == t["scale_bf16_bits"]
        assert q.tolist() == t["codes"]
        assert ref.dequantize(q, s, lo, f, d).tolist() == t["decoded"]
        assert abs(ref.entropy(x) - t["entropy_exact"]) <= entropy_tol(x)


def test_worked_tile_payload_bytes(ref):
    # the flagged worked tile as a 1 x 8 tensor with tile 8 at 3 bits
    t = json.load(open(GOLDEN))["tiles"][0]
    x = np.array([t["x"]], np.float32)
    p = synth.Params(tile=8, tokens_per_sample=0, bit_budget=3.0, candidates=(3,), tau=2.0)
    P = ref.encode(x, p)
    pl = ref.plan(1, 8, p)
    assert P[pl["off_side"]] == 0x80 | 1
    assert int(P[pl["off_scale"]]) | (int(P[pl["off_scale"] + 1]) << 8) == t["scale_bf16_bits"]
    assert P[pl["off_zero"]:pl["off_zero"] + 4].view(np.float32)[0] == 3.0
    # codes 7,0,0,7,0,7,7,0 at 3 bits each, least significant bit first:
    # bits 0-2 = 111, 9-11 = 111, 15-17 = 111, 18-20 = 111 -> 0x1F8E07 little-endian
    assert P[pl["off_codes"]:pl["off_codes"] + 3].tolist() == [0x07, 0x8E, 0x1F]
    y = ref.decode(P, 1, 8, p)
    assert y[0].tolist() == t["decoded"]


def test_nibble_order_low_first(ref):
    # 4-bit codes: the first element sits in the low nibble (INT4 packing order of arXiv 2306.11987)
    x = np.array([[0, 15, 0, 15, 0, 15, 0, 15, 1, 2, 3, 4, 5, 6, 7, 8]], np.float32)
    p = synth.Params(tile=8, tokens_per_sample=0, bit_budget=4.0, candidates=(4,), tau=math.inf)
    P = ref.encode(x, p)
    pl = ref.plan(1, 16, p)
    # tile 0: lo = 0, s = 1 -> codes = values -> bytes 0xF0 x4
    assert P[pl["off_codes"]:pl["off_codes"] + 4].tolist() == [0xF0] * 4
    # tile 1: lo = 1, range 7 -> s = 7/15 rounded up; codes of 1 and 8 are 0 and 15
    c = P[pl["off_codes"] + 4:pl["off_codes"] + 8]
    assert c[0] & 0xF == 0 and c[3] >> 4 == 15


# ---------------------------------------------------------------- allocation ----
def test_allocation_brute_force(ref):
    g = np.random.default_rng(17)
    for trial in range(300):
        N = int(g.integers(1, 11))
        H = g.choice([0.5, 1.0, 1.5, 2.0, 2.5], N).astype(np.float32) if trial % 2 else g.random(N).astype(np.float32)
        for k in range(N + 1):
            hi = ref.allocate(H, k)
            best = None
            for sub in itertools.combinations(range(N), k):  # lexicographic order
                v = float(sum(np.float64(H[i]) for i in sub))
                if best is None or v > best[0] + 1e-12:
                    best = (v, sub)
            want = np.zeros(N, np.uint8)
            want[list(best[1])] = 1
            assert np.array_equal(hi, want), (H, k)


@pytest.mark.parametrize("N,budget,cands,blo,bhi,k", [
    (32768, 3.5, (2, 3, 4, 8), 3, 4, 16384),
    (1048576, 3.8, (3, 4, 8), 3, 4, 838860),  # the pages' default 80% INT4 + 20% INT3
    (32768, 5.0, (3, 4, 8), 4, 8, 8192),
    (32768, 2.5, (2, 3, 4, 8), 2, 3, 16384),
    (4096, 4.0, (3, 4, 8), 4, 8, 0),
    (1048576, 3.0, (3, 4, 8), 3, 4, 0),
    (100, 9.0, (2, 4), 4, 4, 0),
])
def test_width_pair_and_k(ref, N, budget, cands, blo, bhi, k):
    p = synth.Params(tile=64, tokens_per_sample=0, bit_budget=budget, candidates=cands, tau=2.0)
    pl = ref.plan(N // 32 if N % 32 == 0 else N, 2048 if N % 32 == 0 else 64, p)
    assert pl["tiles_per_sample"] == N
    assert (pl["b_lo"], pl["b_hi"], pl["k"]) == (blo, bhi, k)
    # budget conservation: the average code width never exceeds the budget, and
    # one more upgraded tile would exceed it
    total = (N - k) * blo + k * bhi
    assert total <= budget * N + 1e-9
    if bhi > blo:
        assert total + (bhi - blo) > budget * N


@pytest.mark.parametrize("N", [5, 10, 80, 10240, 1048575])
def test_k_of_decimal_budgets(ref, N):
    # The pages' default is 80% INT4 / 20% INT3 (Sec. 3.2, Sec. 5.1): k = 0.8 N
    # exactly when 0.8 N is an integer, although 3.8 in fp32 is 3.79999995.
    # The budget is the shortest decimal that rounds to the fp32 value.
    for budget, cands, frac in [(3.8, (3, 4), (4, 5)), (3.3, (3, 4), (3, 10)), (3.7, (3, 4, 8), (7, 10)),
                                (2.6, (2, 3), (3, 5)), (4.2, (2, 4, 8), (1, 20)), (3.5, (3, 4), (1, 2))]:
        assert float(np.float32(budget)) != budget or budget == 3.5
        p = synth.Params(tile=64, tokens_per_sample=0, bit_budget=budget, candidates=cands, tau=2.0)
        pl = ref.plan(N, 64, p)
        assert pl["k"] == N * frac[0] // frac[1], (budget, N)
        # the greedy allocator's bits above c_1: R = floor((B - c_1) N) with the same decimal B
        g = synth.Params(**{**p.__dict__, "allocator": 1})
        c1, cn = cands[0], cands[-1]
        want = min((N * round((budget - c1) * 10)) // 10, (cn - c1) * N)
        assert ref.plan(N, 64, g)["R"] == want, (budget, N)
    # a budget with more digits: 3.1415927 (fp32 of pi - 0.0000001) keeps all its digits
    p = synth.Params(tile=64, tokens_per_sample=0, bit_budget=float(np.float32(3.1415927)), candidates=(3, 4))
    assert ref.plan(N, 64, p)["k"] == (N * 1415927) // 10000000


def test_budget_errors(ref):
    with pytest.raises(ref.OracleError) as e:
        ref.plan(4, 64, synth.Params(tile=64, bit_budget=2.5, candidates=(3, 4)))
    assert e.value.code == 4
    for bad in (dict(tile=48), dict(tile=4), dict(candidates=(4, 3)), dict(candidates=(0, 3)), dict(candidates=(3, 9)),
                dict(candidates=()), dict(tau=float("nan")), dict(bit_budget=float("nan")), dict(tokens_per_sample=3)):
        with pytest.raises(ref.OracleError) as e:
            ref.plan(4, 128, synth.Params(**{**dict(tile=64, bit_budget=3.5, candidates=(3, 4)), **bad}))
        assert e.value.code == 1


# ---------------------------------------------------------------- payload ----
def test_plan_layout_numbers(ref):
    # hand-computed: 4096 tiles of 32 at 4 bits; sections on 256-byte boundaries
    w = synth.workload("c1_256x512_f32_g32")
    pl = ref.plan(w.tokens, w.hidden, w.params)
    assert (pl["off_table"], pl["off_bitmap"], pl["off_side"], pl["off_scale"], pl["off_zero"], pl["off_codes"], pl["total"]) == (
        256, 512, 1024, 5120, 13312, 29696, 95232)
    # 8192 x 8192 at G = 64, all 3-bit: 1,048,576 tiles x 24 bytes of codes
    w = synth.workload("c5_8192x8192_bf16_g64")
    pl = ref.plan(w.tokens, w.hidden, w.params)
    assert pl["code_bytes"] == 25165824 and pl["k"] == 0
    # paper default 80/20 split at the same shape: 838,860 tiles get 4 bits
    w = synth.workload("x2_c5_budget3p8")
    pl = ref.plan(w.tokens, w.hidden, w.params)
    assert pl["code_bytes"] == 1048576 * 24 + 838860 * 8


def test_payload_fixed_shape(ref):
    p = synth.Params(tile=32, tokens_per_sample=16, bit_budget=3.5, candidates=(3, 4, 8), tau=2.0)
    a = synth.random_tensor(64, 256, synth.F32, 1)
    b = synth.random_tensor(64, 256, synth.F32, 2, scale=100, n_out=3, mult=40)
    Pa, Pb = ref.encode(a, p), ref.encode(b, p)
    assert Pa.size == Pb.size
    assert np.array_equal(Pa[:256], Pb[:256])
    pl = ref.plan(64, 256, p)
    # every sample upgrades exactly k tiles
    bm = np.unpackbits(Pa[pl["off_bitmap"]:pl["off_bitmap"] + 4 * ((pl["tiles"] + 31) // 32)], bitorder="little")
    per = bm[:pl["tiles"]].reshape(pl["nsamples"], -1).sum(1)
    assert np.all(per == pl["k"]) and pl["k"] == 64


def test_scale_invariance(ref):
    p = synth.Params(tile=64, tokens_per_sample=8, bit_budget=3.5, candidates=(3, 4), tau=2.0)
    x = synth.random_tensor(32, 512, synth.F32, 4, n_out=6, mult=30)
    P1 = ref.encode(x, p)
    P2 = ref.encode((x * np.float32(8.0)).astype(np.float32), p)
    pl = ref.plan(32, 512, p)
    n = pl["tiles"]
    assert np.array_equal(P1[pl["off_bitmap"]:pl["off_side"]], P2[pl["off_bitmap"]:pl["off_side"]])
    assert np.array_equal(P1[pl["off_side"]:pl["off_side"] + n], P2[pl["off_side"]:pl["off_side"] + n])
    assert np.array_equal(P1[pl["off_codes"]:], P2[pl["off_codes"]:])
    s1 = (P1[pl["off_scale"]:pl["off_scale"] + 2 * n].view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    s2 = (P2[pl["off_scale"]:pl["off_scale"] + 2 * n].view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(s1 * 8, s2)
    z1 = P1[pl["off_zero"]:pl["off_zero"] + 4 * n].view(np.float32)
    z2 = P2[pl["off_zero"]:pl["off_zero"] + 4 * n].view(np.float32)
    assert np.array_equal(z1 * 8, z2)


def test_codec_roundtrip_error_bound(ref):
    # whole tensor: per element |x - xhat| <= s/2 on plain tiles; ||.||_2 <= s/2 on transformed tiles
    p = synth.Params(tile=32, tokens_per_sample=0, bit_budget=3.5, candidates=(3, 4), tau=2.0)
    x = synth.random_tensor(48, 256, synth.F32, 6, n_out=5, mult=60)
    P = ref.encode(x, p)
    y = ref.decode(P, 48, 256, p)
    st = ref.tile_stats(x, p)
    xt = x.reshape(-1, 32).astype(np.float64)
    yt = y.reshape(-1, 32).astype(np.float64)
    for i in range(xt.shape[0]):
        s = float(st["scale"][i])
        slack = 1e-6 * (1 + np.abs(xt[i]).max()) * 32
        if st["flag"][i]:
            assert np.linalg.norm(xt[i] - yt[i]) <= s / 2 * 1.001 + slack
        else:
            assert np.abs(xt[i] - yt[i]).max() <= s / 2 * 1.001 + slack
    assert st["flag"].any() and not st["flag"].all()


def test_decode_rejects_bad_header(ref):
    p = synth.Params(tile=32, tokens_per_sample=0, bit_budget=3.0, candidates=(3,), tau=2.0)
    x = synth.random_tensor(4, 64, synth.F32, 8)
    P = ref.encode(x, p)
    for off in (0, 8, 16, 45, 112):
        Q = P.copy()
        Q[off] ^= 1
        with pytest.raises(ref.OracleError) as e:
            ref.decode(Q, 4, 64, p)
        assert e.value.code == 5
    with pytest.raises(ref.OracleError):
        ref.decode(P, 4, 64, synth.Params(tile=32, bit_budget=3.0, candidates=(3,), tau=4.0))


def test_bf16_input_widens_exactly(ref):
    p = synth.Params(tile=32, tokens_per_sample=0, bit_budget=3.0, candidates=(3,), tau=2.0)
    xb = synth.random_tensor(8, 128, synth.BF16, 9, n_out=2, mult=20)
    xf = synth.bf16_bits_to_f32(xb).reshape(8, 128)
    Pb, Pf = ref.encode(xb, p), ref.encode(xf, p)
    assert Pb[6] == 1 and Pf[6] == 0
    Pb[6] = 0
    assert np.array_equal(Pb, Pf)


# ------------------------------------------------ backward compressor (Q_Naive) ----
# Algorithm 1, backward pass (fixed-point compressor of the activation gradients) and
# Appendix H Eq. (24) g_hat = Q(c g) / c; Q read as b-bit signed fixed point with
# b-1 fractional bits, round half to even, saturating.

def test_naive_quantize_worked_values(ref):
    # b = 8, c = 1: step 2^-7; range [-1, 1 - 2^-7]
    got = ref.naive_quantize([0.5, -1.0, 0.999, 3.0, -3.0, 2.0**-8, 1.5 * 2.0**-7, -2.5 * 2.0**-7, 0.0, -0.0], 8, 1.0)
    # 0.5*128 = 64; -128; 127.87 -> 128 saturates to 127; +-3 saturate; 0.5 -> 0 (tie to even);
    # 1.5 -> 2 (tie to even); -2.5 -> -2 (tie to even); zeros
    assert got.tolist() == [64, -128, 127, 127, -128, 0, 2, -2, 0, 0]


def test_naive_grid_points_round_trip_exactly(ref):
    # every representable k / (c 2^(b-1)) comes back bit for bit
    for bits, c in ((4, 1.0), (6, 1e4), (8, 3.5), (10, 2.0**-3)):
        cq = np.float32(c) * np.float32(2.0 ** (bits - 1))
        k = np.arange(-(2 ** (bits - 1)), 2 ** (bits - 1), dtype=np.int64)
        g = (k.astype(np.float64) / np.float64(cq)).astype(np.float32)
        q = ref.naive_quantize(g, bits, c)
        assert np.array_equal(q, k)
        assert np.array_equal(ref.naive_dequantize(q, bits, c), g)


def test_naive_error_bound_and_saturation(ref):
    g = np.random.default_rng(4).standard_normal(4000).astype(np.float32) * 0.3
    for bits, c in ((4, 1.0), (8, 1.0), (8, 2.0), (10, 0.5)):
        cq = c * 2.0 ** (bits - 1)
        lo, hi = -(2 ** (bits - 1)) / cq, (2 ** (bits - 1) - 1) / cq
        gh = ref.naive_dequantize(ref.naive_quantize(g, bits, c), bits, c).astype(np.float64)
        inside = (g >= lo) & (g <= hi)
        # half a step plus the fp32 roundings of the product and of the division
        tol = 0.5 / cq + 2.0 ** -23 * np.abs(g[inside]) * 2
        assert np.all(np.abs(gh[inside] - g[inside]) <= tol)
        assert np.all(gh[g > hi] == np.float32(hi)) and np.all(gh[g < lo] == np.float32(lo))


def test_naive_scaling_keeps_small_gradients(ref):
    # App. H: gradients of order 1e-5 vanish in 8-bit fixed point; Eq. (24) with c = 1e4 keeps them
    g = np.random.default_rng(6).uniform(-3e-5, 3e-5, 1000).astype(np.float32)
    assert np.all(ref.naive_quantize(g, 8, 1.0) == 0)
    gh = ref.naive_dequantize(ref.naive_quantize(g, 8, 1e4), 8, 1e4)
    assert np.count_nonzero(gh) > 900
    assert np.abs(gh - g).max() <= 0.5 / (1e4 * 128) * 1.001


def test_naive_payload_bytes_worked_by_hand(ref):
    # b = 4, c = 1 (step 1/8): 0.5 -> 4 = 0100b, -0.25 -> -2 = 1110b, 0.125 -> 1 = 0001b, -1 -> -8 = 1000b.
    # Stream, LSB first: byte 0 = code1 << 4 | code0 = 0xE4, byte 1 = code3 << 4 | code2 = 0x81.
    P = ref.naive_encode(np.array([0.5, -0.25, 0.125, -1.0], np.float32), 4, 1.0)
    assert P.size == 512  # 256-byte header region + one 32-code group of 16 bytes, padded to 256
    assert bytes(P[0:4]) == b"TAHN" and P[4] == 1 and P[5] == 0 and P[6] == 0 and P[7] == 4
    assert int.from_bytes(bytes(P[8:16]), "little") == 4
    assert bytes(P[16:20]) == np.float32(1.0).tobytes()
    assert int.from_bytes(bytes(P[24:32]), "little") == 512
    assert P[256] == 0xE4 and P[257] == 0x81 and not P[258:].any()
    assert ref.naive_decode(P, 4, 4, 1.0).tolist() == [0.5, -0.25, 0.125, -1.0]


def test_naive_payload_size_and_padding(ref):
    for n, bits in ((0, 8), (1, 8), (31, 6), (32, 6), (33, 10), (1000, 16)):
        groups = (n + 31) // 32
        want = ((256 + groups * 4 * bits) + 255) // 256 * 256
        assert ref.naive_payload_bytes(n, bits) == want
        g = np.linspace(-1, 1, n, dtype=np.float32)
        P = ref.naive_encode(g, bits, 1.0)
        used = 256 + (n * bits + 7) // 8
        assert not P[used:].any()


# ---------------------------------------------------------------- allocation tiles (A = kA * G) ----
def shannon64(a):
    p = np.abs(np.asarray(a, np.float64))
    return float(scipy.stats.entropy(p / p.sum(), base=2)) if p.sum() > 0 else 0.0


def test_alloc_entropy_grouping_identity(ref):
    # Sec. 3.2 forms Eq. (1) over all A channels. Grouping property of Shannon
    # entropy: kA copies of one tile spread the mass evenly over kA blocks, so
    # H(A-tile) = H(G-tile) + log2(kA); a zero block adds nothing.
    g = np.random.default_rng(23)
    for G in (32, 64):
        for kA in (2, 3, 4, 5, 16):
            t = (g.standard_normal(G) * np.exp(g.standard_normal())).astype(np.float32)
            rep = np.tile(t, kA)
            want = shannon64(t) + math.log2(kA)
            assert abs(ref.alloc_entropy(rep, G) - want) <= entropy_tol(rep), (G, kA)
            z = np.concatenate([t, np.zeros(G * (kA - 1), np.float32)])
            assert abs(ref.alloc_entropy(z, G) - shannon64(t)) <= entropy_tol(z), (G, kA)


def test_alloc_entropy_matches_scipy_and_reduces_to_tile_entropy(ref):
    g = np.random.default_rng(29)
    for G in (32, 64, 128):
        for kA in (1, 2, 3, 8, 64):
            a = (g.standard_normal(G * kA) * np.exp(g.standard_normal())).astype(np.float32)
            a[g.integers(0, a.size)] *= 80
            assert abs(ref.alloc_entropy(a, G) - shannon64(a)) <= entropy_tol(a), (G, kA)
            # block order does not matter beyond rounding; signs not at all
            blocks = a.reshape(kA, G)[::-1].ravel()
            assert abs(ref.alloc_entropy(-blocks, G) - shannon64(a)) <= entropy_tol(a)
        # A = G is the quantization-tile entropy itself
        a = g.standard_normal(G).astype(np.float32)
        assert ref.alloc_entropy(a, G) == ref.entropy(a)
    # uniform magnitudes over A channels: log2 A; one spike in A channels: 0
    u = np.full(64 * 48, -0.25, np.float32)
    assert abs(ref.alloc_entropy(u, 64) - math.log2(u.size)) <= entropy_tol(u)
    s = np.zeros(64 * 48, np.float32)
    s[1000] = 3.0
    assert abs(ref.alloc_entropy(s, 64)) <= 4 * 2.0**-24 * math.log2(3.0)
    assert ref.alloc_entropy(np.zeros(256, np.float32), 64) == 0.0


@pytest.mark.parametrize("A,S", [(128, 0), (256, 4), (512, 0), (1536, 2), (3072, 0)])
def test_alloc_tile_selection_brute_force(ref, A, S):
    # widths against an fp64 ranking of the allocation tiles of each sample; A =
    # hidden is the token-level allocation of Sec. 3.2. The random entropies are
    # far apart compared with the fp32 error, so the fp64 top-k is the oracle's.
    G, tokens, hidden = 64, 16, 3072
    p = synth.Params(tile=G, tokens_per_sample=S, bit_budget=3.3, candidates=(3, 4), tau=2.0, alloc_tile=A)
    x = synth.random_tensor(tokens, hidden, synth.F32, 31, n_out=40, mult=50)
    pl = ref.plan(tokens, hidden, p)
    kA, NA = A // G, pl["atiles_per_sample"]
    assert (pl["A"], pl["kA"], pl["MA"], pl["atiles"]) == (A, kA, hidden // A, tokens * hidden // A)
    assert pl["k"] == math.floor(0.3 * NA + 1e-9)
    st = ref.tile_stats(x, p)
    assert st["H"].size == pl["atiles"]
    Hx = np.array([shannon64(r) for r in x.reshape(-1, A)])
    for u in range(pl["atiles"]):
        assert abs(st["H"][u] - Hx[u]) <= entropy_tol(x.reshape(-1, A)[u])
    hi = st["hi"].reshape(-1, kA)
    assert np.all(hi == hi[:, :1])  # one width per allocation tile
    for s in range(pl["nsamples"]):
        Hs = Hx[s * NA:(s + 1) * NA]
        order = np.argsort(-Hs, kind="stable")
        k = pl["k"]
        if 0 < k < NA:
            assert Hs[order[k - 1]] - Hs[order[k]] > 1e-4  # no near-ties at the cut
        want = np.zeros(NA, np.uint8)
        want[order[:k]] = 1
        assert np.array_equal(hi[s * NA:(s + 1) * NA, 0], want), s


def test_token_level_allocation_plan_and_payload(ref):
    # 8192 x 8192 at G = 64, A = C (token level), the pages' 80/20 split over the
    # 8192 tokens: 6553 tokens of 128 tiles each get 4 bits.
    p = synth.Params(tile=64, tokens_per_sample=0, bit_budget=3.8, candidates=(3, 4), alloc_tile=8192)
    pl = ref.plan(8192, 8192, p)
    assert (pl["kA"], pl["MA"], pl["atiles_per_sample"], pl["k"]) == (128, 1, 8192, 6553)
    assert pl["code_bytes"] == 1048576 * 24 + 6553 * 128 * 8
    # small tensor: header records A; the bitmap holds one run per upgraded token
    p = synth.Params(tile=32, tokens_per_sample=8, bit_budget=3.5, candidates=(3, 4), alloc_tile=256)
    x = synth.random_tensor(32, 256, synth.F32, 37, n_out=6, mult=30)
    P = ref.encode(x, p)
    pl = ref.plan(32, 256, p)
    assert P[4] == 2 and P[5] == 0 and int(P[120:124].view(np.uint32)[0]) == 256
    bm = np.unpackbits(P[pl["off_bitmap"]:pl["off_bitmap"] + 4 * ((pl["tiles"] + 31) // 32)], bitorder="little")
    rows = bm[:pl["tiles"]].reshape(32, 8)
    assert np.all(rows == rows[:, :1])
    assert np.all(rows[:, 0].reshape(4, 8).sum(1) == pl["k"]) and pl["k"] == 4
    # A = G spelled out is the same codec as the default
    q = synth.Params(tile=32, tokens_per_sample=8, bit_budget=3.5, candidates=(3, 4))
    x2 = synth.random_tensor(32, 256, synth.F32, 38, n_out=6, mult=30)
    assert np.array_equal(ref.encode(x2, q), ref.encode(x2, synth.Params(**{**q.__dict__, "alloc_tile": 32})))
    y = ref.decode(P, 32, 256, p)
    assert np.abs(y - x).max() < np.abs(x).max() / 2  # decodes


def test_alloc_tile_errors(ref):
    base = dict(tile=64, bit_budget=3.5, candidates=(3, 4))
    for A in (32, 96, 200, 640, -64):  # below G, not a multiple of G, not dividing hidden = 512
        with pytest.raises(ref.OracleError) as e:
            ref.plan(4, 512, synth.Params(**base, alloc_tile=A))
        assert e.value.code == 1, A
    for A in (0, 64, 128, 256, 512):
        ref.plan(4, 512, synth.Params(**base, alloc_tile=A))
    # a payload made for one A does not decode as another
    x = synth.random_tensor(4, 512, synth.F32, 41)
    P = ref.encode(x, synth.Params(**base, alloc_tile=128))
    with pytest.raises(ref.OracleError) as e:
        ref.decode(P, 4, 512, synth.Params(**base, alloc_tile=256))
    assert e.value.code == 5
