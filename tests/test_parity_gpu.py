"""GPU-vs-oracle parity of the TAH-Quant HIP path, through the C ABI.

Bar: width bits, side bytes, scale bits, zero-points and
packed codes bit-exact; decoded fp32 within 1e-5 * tile scale. The fp32
operation order is shared by specification, so every payload byte and every
decoded value is expected to be identical; the tests require exactly that,
and on a mismatch report which payload section and how many elements differ.

The workloads run at their full sizes (4096 x 2048 ... 16384 x 5120), element
by element, with the launch configuration the benchmark times.
"""

import functools
import math

import numpy as np
import pytest
import torch

import activation_quantization_pipeline_amd as tah
import oracle
import synth

pytestmark = pytest.mark.gpu

SECTIONS = ("table", "bitmap", "side", "scale", "zero", "codes")


def say(*a):
    print(*a, flush=True)


def to_dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def section_report(P, R, pl):
    bounds = [("header", 0, 256), ("table", pl["off_table"], pl["off_bitmap"]), ("bitmap", pl["off_bitmap"], pl["off_side"]),
              ("side", pl["off_side"], pl["off_scale"]), ("scale", pl["off_scale"], pl["off_zero"]),
              ("zero", pl["off_zero"], pl["off_codes"]), ("codes", pl["off_codes"], pl["total"])]
    out = []
    for name, a, b in bounds:
        d = int(np.count_nonzero(P[a:b] != R[a:b]))
        if d:
            first = a + int(np.flatnonzero(P[a:b] != R[a:b])[0])
            out.append(f"{name}: {d} bytes differ (first at {first})")
    return "; ".join(out)


def assert_payload_equal(P, R, pl, what):
    assert P.shape == R.shape, f"{what}: size {P.shape} vs {R.shape}"
    if not np.array_equal(P, R):
        pytest.fail(f"{what}: payload differs from the oracle: {section_report(P, R, pl)}")


def assert_decoded_equal(y, y_ref, R, pl, what):
    if np.array_equal(y.view(np.uint32) if y.dtype == np.float32 else y,
                      y_ref.view(np.uint32) if y_ref.dtype == np.float32 else y_ref):
        return
    # report against the bar: |diff| <= 1e-5 * tile scale
    G = pl["G"]
    s = (R[pl["off_scale"]:pl["off_scale"] + 2 * pl["tiles"]].view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    yf = y.astype(np.float32) if y.dtype == np.float32 else synth.bf16_bits_to_f32(y)
    rf = y_ref.astype(np.float32) if y_ref.dtype == np.float32 else synth.bf16_bits_to_f32(y_ref)
    diff = np.abs(yf.reshape(-1, G).astype(np.float64) - rf.reshape(-1, G))
    bad = int(np.count_nonzero(diff > 1e-5 * s[:, None]))
    pytest.fail(f"{what}: decoded values differ from the oracle in {int(np.count_nonzero(diff))} elements, "
                f"{bad} beyond 1e-5 * scale")


@functools.lru_cache(maxsize=1)
def workload_case(name, seed):
    w = synth.workload(name)
    x = synth.generate(name, seed)
    R = oracle.encode(x, w.params)
    pl = oracle.plan(w.tokens, w.hidden, w.params)
    return w, x, R, pl


WORKLOADS = list(synth.WORKLOADS) + list(synth.COVERAGE)


@pytest.mark.parametrize("name", WORKLOADS)
def test_workload_parity(name):
    w, x, R, pl = workload_case(name, 0)
    p = w.params
    say(f"[parity] {name}: {w.tokens}x{w.hidden} tile {p.tile} budget {p.bit_budget} cands {p.candidates} "
        f"tau {p.tau} k={pl['k']}")
    xt = to_dev(x)
    ws = tah.alloc_workspace(w.tokens, w.hidden, p)

    say(f"[parity] {name}: encode")
    P = to_host(tah.encode(xt, p, ws=ws))
    torch.cuda.synchronize()
    assert_payload_equal(P, R, pl, f"{name} encode")

    say(f"[parity] {name}: allocation-tile entropy in workspace vs oracle (A = {pl['A']})")
    off = tah.workspace_entropy_offset(w.tokens, w.hidden, p)
    H = ws[off:off + 4 * pl["atiles"]].cpu().numpy().view(np.float32)
    rng = np.random.default_rng(1)
    idx = rng.choice(pl["atiles"], size=min(4000, pl["atiles"]), replace=False)
    xf = x.astype(np.float32) if x.dtype == np.float32 else synth.bf16_bits_to_f32(x)
    atiles = xf.reshape(-1, pl["A"])
    H_ref = np.array([oracle.alloc_entropy(atiles[i], p.tile) for i in idx], np.float32)
    assert np.array_equal(H[idx].view(np.uint32), H_ref.view(np.uint32))

    say(f"[parity] {name}: oracle decode")
    y_ref = oracle.decode(R, w.tokens, w.hidden, p, oracle.F32)

    say(f"[parity] {name}: decode of the oracle payload (fp32)")
    y = to_host(tah.decode(to_dev(R), w.tokens, w.hidden, p, torch.float32, ws=ws))
    torch.cuda.synchronize()
    assert tah.read_device_status(ws) == 0
    assert_decoded_equal(y, y_ref, R, pl, f"{name} decode")

    say(f"[parity] {name}: fused round trip (fp32 out)")
    y2, P2 = tah.roundtrip(xt, p, torch.float32, ws=ws)
    assert_payload_equal(to_host(P2), R, pl, f"{name} roundtrip payload")
    assert_decoded_equal(to_host(y2), y_ref, R, pl, f"{name} roundtrip")
    del y2, P2

    if w.dtype == synth.BF16:
        say(f"[parity] {name}: fused round trip (bf16 out, the benchmarked launch)")
        y_ref16 = oracle.decode(R, w.tokens, w.hidden, p, oracle.BF16)
        y3, _ = tah.roundtrip(xt, p, torch.bfloat16, ws=ws)
        assert_decoded_equal(to_host(y3), y_ref16, R, pl, f"{name} roundtrip bf16")
        say(f"[parity] {name}: decode (bf16 out)")
        y4 = to_host(tah.decode(to_dev(R), w.tokens, w.hidden, p, torch.bfloat16, ws=ws))
        assert_decoded_equal(y4, y_ref16, R, pl, f"{name} decode bf16")


@pytest.mark.parametrize("name", ["c2_4096x2048_bf16_g64", "c1_256x512_f32_g32"])
@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_seed_sweep(name, seed):
    w = synth.workload(name)
    x = synth.generate(name, seed)
    say(f"[seeds] {name} seed {seed}")
    R = oracle.encode(x, w.params)
    pl = oracle.plan(w.tokens, w.hidden, w.params)
    y_ref = oracle.decode(R, w.tokens, w.hidden, w.params)
    y, P = tah.roundtrip(to_dev(x), w.params, torch.float32)
    assert_payload_equal(to_host(P), R, pl, f"{name} seed {seed}")
    assert_decoded_equal(to_host(y), y_ref, R, pl, f"{name} seed {seed}")


def run_case(x, p, what):
    """encode, decode and round trip of one small tensor against the oracle."""
    tokens, hidden = x.shape
    say(f"[edge] {what}: {tokens}x{hidden} {x.dtype} tile {p.tile} S {p.tokens_per_sample} budget {p.bit_budget} "
        f"cands {p.candidates} tau {p.tau} A {p.alloc_tile}")
    R = oracle.encode(x, p)
    pl = oracle.plan(tokens, hidden, p)
    xt = to_dev(x)
    P = to_host(tah.encode(xt, p))
    torch.cuda.synchronize()
    assert_payload_equal(P, R, pl, what)
    y_ref = oracle.decode(R, tokens, hidden, p)
    y = to_host(tah.decode(to_dev(R), tokens, hidden, p, torch.float32))
    assert_decoded_equal(y, y_ref, R, pl, what + " decode")
    y2, P2 = tah.roundtrip(xt, p, torch.float32)
    assert_payload_equal(to_host(P2), R, pl, what + " roundtrip")
    assert_decoded_equal(to_host(y2), y_ref, R, pl, what + " roundtrip")
    y3, P3 = tah.roundtrip(xt, p, torch.float32, write_payload=False)
    assert P3 is None
    assert_decoded_equal(to_host(y3), y_ref, R, pl, what + " roundtrip without payload")
    return R, y_ref


P = tah.TahParams


@pytest.mark.parametrize("tile", [32, 64, 128])
@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_ragged_shapes(tile, dtype):
    # tile counts that are not multiples of the 64-tile wave or the workgroup
    for tokens, mult in ((1, 5), (3, 5), (7, 9), (65, 3), (300, 7)):
        x = synth.random_tensor(tokens, tile * mult, dtype, tokens + mult, n_out=2, mult=25)
        run_case(x, P(tile=tile, tokens_per_sample=0, bit_budget=3.5, candidates=(3, 4), tau=2.0),
                 f"ragged t{tokens} m{mult} mixed")
        run_case(x, P(tile=tile, tokens_per_sample=0, bit_budget=4.0, candidates=(4, 8), tau=2.0),
                 f"ragged t{tokens} m{mult} uniform")


@pytest.mark.parametrize("S", [1, 3, 16])
def test_many_small_samples(S):
    # samples whose tile count is not a multiple of 64 (ranking scope crosses waves)
    x = synth.random_tensor(48, 320, synth.BF16, S, n_out=3, mult=30)
    run_case(x, P(tile=64, tokens_per_sample=S, bit_budget=3.5, candidates=(2, 3, 4, 8), tau=2.0), f"S={S}")
    run_case(x, P(tile=32, tokens_per_sample=S, bit_budget=2.2, candidates=(2, 3), tau=2.0), f"S={S} tile32")


@pytest.mark.parametrize("lo,hi", [(1, 2), (2, 3), (3, 4), (4, 8), (5, 6), (6, 7), (7, 8), (1, 8)])
@pytest.mark.parametrize("tile", [32, 64, 128])
def test_every_width(lo, hi, tile):
    x = synth.random_tensor(40, 4 * tile, synth.F32, lo * 10 + hi, n_out=2, mult=20)
    run_case(x, P(tile=tile, tokens_per_sample=8, bit_budget=lo + 0.3, candidates=(lo, hi), tau=2.0),
             f"widths {lo}/{hi}")


@pytest.mark.parametrize("tau", [0.0, 2.0, 4.0, math.inf])
def test_tau_semantics(tau):
    x = synth.random_tensor(64, 512, synth.BF16, 7, n_out=5, mult=40)
    R, _ = run_case(x, P(tile=64, tokens_per_sample=0, bit_budget=3.8, candidates=(3, 4), tau=tau), f"tau={tau}")
    pl = oracle.plan(64, 512, P(tile=64, bit_budget=3.8, candidates=(3, 4), tau=tau))
    side = R[pl["off_side"]:pl["off_side"] + pl["tiles"]]
    if tau == 0.0:
        assert np.all(side >> 7 == 1)
    if tau == math.inf:
        assert not np.any(side >> 7)


@pytest.mark.parametrize("tile", [32, 64, 128])
@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_allocation_tiles(tile, dtype):
    # allocation tiles of kA quantization tiles (Sec. 3.2), kA a power of two or
    # not, up to whole tokens; ragged tile counts, one or several samples
    M = 12
    for tokens, S in ((37, 0), (40, 8), (130, 13)):
        x = synth.random_tensor(tokens, tile * M, dtype, tokens + tile, n_out=4, mult=40)
        for kA in (2, 3, 4, 6, M):
            run_case(x, P(tile=tile, tokens_per_sample=S, bit_budget=3.6, candidates=(3, 4), tau=2.0, alloc_tile=kA * tile),
                     f"alloc kA={kA} t{tokens} S{S}")
    # several widths, and a budget on a candidate (no selection, k = 0)
    x = synth.random_tensor(64, tile * 8, dtype, 99, n_out=3, mult=30)
    run_case(x, P(tile=tile, tokens_per_sample=16, bit_budget=5.5, candidates=(2, 4, 8), tau=2.0, alloc_tile=4 * tile),
             "alloc kA=4 widths 4/8")
    run_case(x, P(tile=tile, tokens_per_sample=16, bit_budget=4.0, candidates=(2, 4, 8), tau=2.0, alloc_tile=4 * tile),
             "alloc kA=4 k=0")


def test_allocation_tile_ties_and_entropy_api():
    # equal allocation-tile entropies: the lower index wins
    z = np.zeros((16, 512), np.float32)
    run_case(z, P(tile=64, tokens_per_sample=4, bit_budget=3.5, candidates=(3, 4), tau=2.0, alloc_tile=128), "alloc zero")
    row = synth.random_tensor(1, 128, synth.F32, 3)
    x = np.tile(row, (32, 4))
    run_case(x, P(tile=64, tokens_per_sample=8, bit_budget=3.3, candidates=(3, 4), tau=2.0, alloc_tile=128),
             "alloc repeated")
    run_case(x, P(tile=64, tokens_per_sample=8, bit_budget=3.3, candidates=(3, 4), tau=2.0, alloc_tile=512),
             "token level repeated rows")
    # tah_tile_entropy returns one entropy per allocation tile
    x = synth.random_tensor(300, 640, synth.BF16, 12, n_out=3, mult=30)
    for A in (64, 128, 320, 640):
        p = P(tile=64, tokens_per_sample=0, bit_budget=3.5, candidates=(3, 4), tau=2.0, alloc_tile=A)
        say(f"[edge] tile_entropy A={A}")
        h = tah.tile_entropy(to_dev(x), p).cpu().numpy()
        st = oracle.tile_stats(x, p)
        assert h.size == 300 * 640 // A
        assert np.array_equal(h.view(np.uint32), st["H"].view(np.uint32)), A


@pytest.mark.parametrize("tile", [32, 64, 128])
@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
@pytest.mark.parametrize("tau", [0.0, 0.5])
def test_small_tau_every_tile_transformed(tile, dtype, tau):
    # tau < 1 takes the encoder variant that transforms each tile in its own lane
    for tokens, mult in ((3, 5), (65, 3), (130, 4)):
        x = synth.random_tensor(tokens, tile * mult, dtype, tokens + mult + 7, n_out=3, mult=20)
        run_case(x, P(tile=tile, tokens_per_sample=0, bit_budget=3.5, candidates=(3, 4), tau=tau),
                 f"tau {tau} t{tokens} m{mult} mixed")
        run_case(x, P(tile=tile, tokens_per_sample=0, bit_budget=4.0, candidates=(4, 8), tau=tau),
                 f"tau {tau} t{tokens} m{mult} uniform")
    # tied maxima are not transformed even at tau = 0.5; all-zero tiles never are
    z = np.zeros((8, tile * 2), np.float32)
    z[:, 3] = 2.0
    z[:, 5] = -2.0
    run_case(z, P(tile=tile, tokens_per_sample=0, bit_budget=3.0, candidates=(3,), tau=tau), f"tau {tau} ties")


def test_ties_all_zero_and_repeated_tiles():
    # every tile has entropy 0: the selection keeps the lowest indices
    z = np.zeros((16, 256), np.float32)
    run_case(z, P(tile=64, tokens_per_sample=4, bit_budget=3.5, candidates=(3, 4), tau=2.0), "all zero")
    # the same tile everywhere: equal entropies, ties broken by index
    row = synth.random_tensor(1, 64, synth.F32, 3)
    x = np.tile(row, (32, 8))
    run_case(x, P(tile=64, tokens_per_sample=8, bit_budget=3.3, candidates=(3, 4), tau=2.0), "repeated tile")
    # half the tiles tied at the threshold
    x2 = np.concatenate([x[:16], synth.random_tensor(16, 512, synth.F32, 4, scale=3)], 0)
    run_case(x2, P(tile=64, tokens_per_sample=32, bit_budget=3.6, candidates=(3, 4), tau=2.0), "half tied")


def test_value_extremes():
    g = np.random.default_rng(5)
    cases = {
        "subnormal": (g.standard_normal((8, 256)) * 1e-39).astype(np.float32),
        "tiny_range": (1e-38 + g.standard_normal((8, 256)) * 1e-45).astype(np.float32),
        "huge": (g.standard_normal((8, 256)) * 1e35).astype(np.float32),
        "one_hot": np.where(g.random((8, 256)) < 1 / 64, -7.0, 0.0).astype(np.float32),
        "neg_zero": np.full((8, 256), -0.0, np.float32),
        "constant": np.full((8, 256), 3.25, np.float32),
    }
    for name, x in cases.items():
        run_case(x, P(tile=64, tokens_per_sample=0, bit_budget=3.5, candidates=(3, 4), tau=2.0), name)
        run_case(x, P(tile=32, tokens_per_sample=0, bit_budget=8.0, candidates=(8,), tau=0.0), name + " 8-bit tau0")


def test_empty_tensor():
    p = P(tile=64, tokens_per_sample=0, bit_budget=3.0, candidates=(3,), tau=2.0)
    x = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    say("[edge] empty tensor")
    Pg = to_host(tah.encode(x, p))
    R = oracle.encode(np.zeros((0, 128), np.uint16), p)
    assert np.array_equal(Pg, R)
    y = tah.decode(to_dev(R), 0, 128, p, torch.float32)
    assert y.shape == (0, 128)


def test_bad_header_sets_status_and_leaves_output():
    p = P(tile=64, tokens_per_sample=0, bit_budget=3.5, candidates=(3, 4), tau=2.0)
    x = synth.random_tensor(32, 256, synth.BF16, 9)
    xt = to_dev(x)
    ws = tah.alloc_workspace(32, 256, p)
    say("[edge] corrupted header")
    Pg = tah.encode(xt, p, ws=ws)
    y = tah.decode(Pg, 32, 256, p, torch.float32, ws=ws)
    assert tah.read_device_status(ws) == 0
    for off in (0, 8, 16, 45, 64):
        bad = Pg.clone()
        bad[off] ^= 1
        sentinel = torch.full((32, 256), 123.0, device="cuda")
        tah.decode(bad, 32, 256, p, torch.float32, y=sentinel, ws=ws)
        assert tah.read_device_status(ws) == 5
        assert torch.all(sentinel == 123.0)
    # params that disagree with the header
    sentinel = torch.full((32, 256), 123.0, device="cuda")
    tah.decode(Pg, 32, 256, P(tile=64, bit_budget=3.5, candidates=(3, 4), tau=4.0), torch.float32, y=sentinel, ws=ws)
    assert tah.read_device_status(ws) == 5 and torch.all(sentinel == 123.0)
    tah.decode(Pg, 32, 256, p, torch.float32, y=sentinel, ws=ws)
    assert tah.read_device_status(ws) == 0 and torch.equal(sentinel, y)


def test_determinism_and_tile_entropy_api():
    w = synth.workload("c2_4096x2048_bf16_g64")
    x = synth.generate(w.name, 5)
    xt = to_dev(x)
    say("[edge] determinism")
    a = tah.encode(xt, w.params)
    b = tah.encode(xt, w.params)
    assert torch.equal(a, b)
    h = tah.tile_entropy(xt, w.params).cpu().numpy()
    st = oracle.tile_stats(x[:256], synth.Params(tile=64, tokens_per_sample=0, bit_budget=3.5, candidates=(2, 3, 4, 8)))
    assert np.array_equal(h[:st["H"].size].view(np.uint32), st["H"].view(np.uint32))


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_flagged_tiles_per_group(dtype):
    """Groups of 64 tile-64 tiles (one wavefront's work) with 0, 1, ..., 12
    flagged tiles each, pivots at the first, the last and other elements,
    spikes of both signs, and a ragged last group."""
    rng = np.random.default_rng(17)
    G, n_tiles, hidden = 64, 64 * 26 + 40, 512
    x = rng.standard_normal((n_tiles, G)) * 0.5
    for g in range((n_tiles + 63) // 64):
        tiles = np.arange(64 * g, min(64 * g + 64, n_tiles))
        for i, t in enumerate(rng.permutation(tiles)[:(g + 5) % 13]):
            pos = (0, G - 1, int(rng.integers(1, G - 1)))[i % 3]
            x[t, pos] = (40.0 + 10 * rng.random()) * (1 if i % 2 else -1)
    x = x.reshape(-1, hidden)
    x = x.astype(np.float32) if dtype == synth.F32 else synth.f32_to_bf16_bits(x)
    for p in (P(tile=G, tokens_per_sample=0, bit_budget=3.0, candidates=(3, 4, 8), tau=2.0),
              P(tile=G, tokens_per_sample=0, bit_budget=3.6, candidates=(3, 4), tau=2.0)):
        R, _ = run_case(x, p, f"flagged per group {dtype} budget {p.bit_budget}")
        y_ref16 = oracle.decode(R, x.shape[0], hidden, p, oracle.BF16)
        y16, _ = tah.roundtrip(to_dev(x), p, torch.bfloat16)
        assert_decoded_equal(to_host(y16), y_ref16, R, oracle.plan(x.shape[0], hidden, p), "bf16 out")


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_threshold_inside_a_large_tie(dtype):
    """One sample of 8192 tiles (two digits of tile index): 30% flat tiles
    (highest entropy), 60% copies of one tile (all the same entropy), 10% spiky
    tiles (lowest). At budget 3.5 over {3, 4} the 4096 selected tiles end inside
    the tied class, so the lowest-index tied tiles must be the ones selected."""
    rng = np.random.default_rng(23)
    T, H, G = 512, 1024, 64
    tiles = np.empty((T * H // G, G))
    n = tiles.shape[0]
    kind = rng.permutation(np.repeat([0, 1, 2], [int(0.3 * n), int(0.6 * n), n - int(0.3 * n) - int(0.6 * n)]))
    tied = np.where(np.arange(G) % 2 == 0, 1.0, 0.0) * np.linspace(0.5, 1.5, G)
    for t in range(n):
        if kind[t] == 0:
            tiles[t] = rng.uniform(0.9, 1.1, G) * rng.choice([-1, 1], G)
        elif kind[t] == 1:
            tiles[t] = tied
        else:
            tiles[t] = rng.standard_normal(G) * 0.01
            tiles[t, rng.integers(G)] = 5.0
    x = tiles.reshape(T, H)
    x = x.astype(np.float32) if dtype == synth.F32 else synth.f32_to_bf16_bits(x)
    p = P(tile=G, tokens_per_sample=0, bit_budget=3.5, candidates=(3, 4), tau=2.0)
    pl = oracle.plan(T, H, p)
    assert pl["atiles_per_sample"] == n and pl["k"] == n // 2
    run_case(x, p, f"large tie {dtype}")


def test_threshold_inside_a_tie_across_workgroups():
    """One sample of 40960 tiles (three histogram workgroups of the select):
    20400 flat tiles above, 200 copies of one tile spread over the sample, the
    rest spiky below; k = 20480, so 80 of the 200 tied tiles (the lowest
    indices) are selected, from candidate lists that three workgroups append
    to the same sample's list."""
    rng = np.random.default_rng(29)
    T, H, G = 640, 4096, 64
    n = T * H // G
    kind = np.full(n, 2)
    idx = rng.permutation(n)
    kind[idx[:20400]] = 0
    kind[idx[20400:20600]] = 1
    tiles = np.empty((n, G))
    tied = np.where(np.arange(G) % 2 == 0, 1.0, 0.0) * np.linspace(0.5, 1.5, G)
    for t in range(n):
        if kind[t] == 0:
            tiles[t] = rng.uniform(0.9, 1.1, G) * rng.choice([-1, 1], G)
        elif kind[t] == 1:
            tiles[t] = tied
        else:
            tiles[t] = rng.standard_normal(G) * 0.01
            tiles[t, rng.integers(G)] = 5.0
    x = tiles.reshape(T, H).astype(np.float32)
    p = P(tile=G, tokens_per_sample=0, bit_budget=3.5, candidates=(3, 4), tau=2.0)
    assert oracle.plan(T, H, p)["k"] == 20480
    R, _ = run_case(x, p, "tie across workgroups")
    # the width map: every flat tile and the 80 lowest-index tied tiles are at 4 bits
    pl = oracle.plan(T, H, p)
    bm = R[pl["off_bitmap"]:pl["off_bitmap"] + 8 * pl["nblocks"]].view(np.uint64)
    hi = np.unpackbits(bm.view(np.uint8), bitorder="little")[:n].astype(bool)
    tied_idx = np.flatnonzero(kind == 1)
    assert hi[kind == 0].all() and not hi[kind == 2].any()
    assert hi[tied_idx[:80]].all() and not hi[tied_idx[80:]].any()


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
@pytest.mark.parametrize("tile", [32, 64, 128])
def test_transformed_tiles_at_extreme_magnitudes(dtype, tile):
    """Transformed tiles whose dequantized values are subnormal, tiny, huge or
    ordinary, mixed within every wavefront: the round trip may take the
    receiver's 1/G into the dequantization only where that is exact, and
    must match the oracle's H then 1/G bit for bit everywhere."""
    rng = np.random.default_rng(41 + tile)
    T, M = 96, 12
    x = rng.standard_normal((T, tile * M))
    x[:, ::tile] *= 40.0  # a spike in every tile: flagged at tau = 2
    # the transformed values of a tile reach about 200 times its scale: the
    # largest scales straddle 2^120 there while no sum of the inverse overflows
    scales = np.array([1e-38, 2.0 ** -120, 1e-30, 2.0 ** -97, 2.0 ** -96, 2.0 ** -90, 1e-3, 1.0,
                       2.0 ** 100, 2.0 ** 110, 2.0 ** 112.5, 2.0 ** 113])
    idx = (np.arange(T)[:, None] + np.arange(M)[None, :]) % len(scales)
    x = (x.reshape(T, M, tile) * scales[idx][:, :, None]).reshape(T, tile * M)
    x = x.astype(np.float32) if dtype == synth.F32 else synth.f32_to_bf16_bits(x)
    for tau in (2.0, 0.0):
        run_case(x, P(tile=tile, tokens_per_sample=0, bit_budget=3.5, candidates=(3, 4), tau=tau),
                 f"extreme magnitudes tile {tile} tau {tau}")


def random_config(seed):
    """A seeded random shape and parameter set within the library's limits."""
    r = np.random.default_rng(1000 + seed)
    G = int(r.choice([32, 64, 128]))
    M = int(r.integers(1, 17))
    hidden = G * M
    tokens = int(r.integers(1, 200))
    divisors = [d for d in range(1, tokens + 1) if tokens % d == 0]
    S = int(r.choice([0] + divisors))
    kAs = [k for k in range(1, M + 1) if M % k == 0]
    A = G * int(r.choice(kAs))
    n_c = int(r.integers(1, 5))
    cands = tuple(sorted(int(c) for c in r.choice(np.arange(1, 9), size=n_c, replace=False)))
    budget = float(np.float32(r.uniform(cands[0], cands[-1] + 0.5)))
    tau = float(r.choice([0.0, 0.5, 1.0, 2.0, 4.0, math.inf]))
    dtype = synth.F32 if r.random() < 0.5 else synth.BF16
    x = synth.random_tensor(tokens, hidden, dtype, 2000 + seed, scale=float(r.choice([1e-3, 1.0, 50.0])),
                            n_out=int(r.integers(0, 4)), mult=float(r.choice([5.0, 40.0, 300.0])))
    p = P(tile=G, tokens_per_sample=S, bit_budget=budget, candidates=cands, tau=tau, alloc_tile=A)
    return x, p


@pytest.mark.parametrize("seed", range(120))
def test_random_configurations(seed):
    x, p = random_config(seed)
    R, y_ref = run_case(x, p, f"random config {seed}")
    if x.dtype == np.uint16:
        tokens, hidden = x.shape
        y16, _ = tah.roundtrip(to_dev(x), p, torch.bfloat16)
        assert_decoded_equal(to_host(y16), oracle.decode(R, tokens, hidden, p, oracle.BF16), R,
                             oracle.plan(tokens, hidden, p), f"random config {seed} bf16 out")


FULL_SIZE_SEEDS = [(n, sd) for n in ("c3_16384x4096_bf16_g64", "c4_16384x5120_f32_g128", "c5_8192x8192_bf16_g64")
                   for sd in (1, 2, 3, 4)] + [("x2_c5_budget3p8", 1), ("x5b_c5_greedy", 1)]


@pytest.mark.parametrize("name,seed", FULL_SIZE_SEEDS)
def test_full_size_other_seed(name, seed):
    """The large workloads at full size with other seeds: payload and fused
    round trip (the benchmarked launch for c5) against the oracle."""
    w = synth.workload(name)
    x = synth.generate(name, seed)
    say(f"[seed{seed}] {name}: oracle")
    R = oracle.encode(x, w.params)
    pl = oracle.plan(w.tokens, w.hidden, w.params)
    y_dt, o_dt = (torch.bfloat16, oracle.BF16) if w.dtype == synth.BF16 else (torch.float32, oracle.F32)
    y_ref = oracle.decode(R, w.tokens, w.hidden, w.params, o_dt)
    say(f"[seed{seed}] {name}: GPU round trip")
    y, P = tah.roundtrip(to_dev(x), w.params, y_dt)
    assert_payload_equal(to_host(P), R, pl, f"{name} seed {seed}")
    assert_decoded_equal(to_host(y), y_ref, R, pl, f"{name} seed {seed}")


@pytest.mark.parametrize("n_tied", [3, 40, 64, 65, 200, 6000])
def test_threshold_inside_a_tie_in_a_large_sample(n_tied):
    """One sample of 163840 tiles, above the size that one workgroup selects
    alone, so the select runs grid-wide (40 histogram workgroups, then the tie
    step): half the tiles flat (above), n_tied copies of one tile spread over
    the sample, the rest spiky (below); k = 81920 lands inside the tied class.
    Up to 64 tied tiles are ranked by one wavefront; with 65 and 200 the tie
    is broken by digit passes over the listed candidates; with 6000 the list
    overflows and the whole sample is scanned."""
    rng = np.random.default_rng(31 + n_tied)
    T, H, G = 2560, 4096, 64
    n = T * H // G
    n_flat = 81920 - n_tied // 2
    kind = np.full(n, 2)
    idx = rng.permutation(n)
    kind[idx[:n_flat]] = 0
    kind[idx[n_flat:n_flat + n_tied]] = 1
    flat = rng.uniform(0.9, 1.1, (n, G)) * rng.choice([-1, 1], (n, G))
    spiky = rng.standard_normal((n, G)) * 0.01
    spiky[np.arange(n), rng.integers(G, size=n)] = 5.0
    tied = np.where(np.arange(G) % 2 == 0, 1.0, 0.0) * np.linspace(0.5, 1.5, G)
    tiles = np.where((kind == 0)[:, None], flat, np.where((kind == 1)[:, None], tied[None, :], spiky))
    x = tiles.reshape(T, H).astype(np.float32)
    p = P(tile=G, tokens_per_sample=0, bit_budget=3.5, candidates=(3, 4), tau=2.0)
    pl = oracle.plan(T, H, p)
    assert pl["k"] == 81920 and pl["tiles_per_sample"] > 131072
    R, _ = run_case(x, p, f"tie in a large sample, {n_tied} tied")
    bm = R[pl["off_bitmap"]:pl["off_bitmap"] + 8 * pl["nblocks"]].view(np.uint64)
    hi = np.unpackbits(bm.view(np.uint8), bitorder="little")[:n].astype(bool)
    tied_idx = np.flatnonzero(kind == 1)
    n_sel = 81920 - n_flat
    assert hi[kind == 0].all() and not hi[kind == 2].any()
    assert hi[tied_idx[:n_sel]].all() and not hi[tied_idx[n_sel:]].any()


@pytest.mark.parametrize("A,T,n_tied", [(256, 2560, 3), (256, 2560, 65), (256, 2560, 6000), (4096, 5120, 3),
                                         (4096, 5120, 200)])
def test_threshold_inside_a_tie_with_allocation_tiles(A, T, n_tied):
    """The same construction over allocation tiles of A channels (4 or 64
    quantization tiles of 64): one sample of 40960 or 5120 allocation tiles,
    whose width-map bits and block table come from the last select pass and
    the tie step (one bit per quantization tile), with the threshold inside a
    class of n_tied equal allocation tiles (one wavefront, digit passes over
    the list, and the list overflowing)."""
    rng = np.random.default_rng(57 + n_tied + A)
    H, G = 4096, 64
    na = T * H // A
    n_flat = na // 2 - n_tied // 2
    kind = np.full(na, 2)
    idx = rng.permutation(na)
    kind[idx[:n_flat]] = 0
    kind[idx[n_flat:n_flat + n_tied]] = 1
    flat = rng.uniform(0.9, 1.1, (na, A)) * rng.choice([-1, 1], (na, A))
    spiky = rng.standard_normal((na, A)) * 0.01
    spiky[np.arange(na), rng.integers(A, size=na)] = 5.0
    tied = np.where(np.arange(A) % 2 == 0, 1.0, 0.0) * np.linspace(0.5, 1.5, A)
    tiles = np.where((kind == 0)[:, None], flat, np.where((kind == 1)[:, None], tied[None, :], spiky))
    x = tiles.reshape(T, H).astype(np.float32)
    p = P(tile=G, tokens_per_sample=0, bit_budget=3.5, candidates=(3, 4), tau=2.0, alloc_tile=A)
    pl = oracle.plan(T, H, p)
    assert pl["k"] == na // 2 and pl["atiles_per_sample"] == na
    R, _ = run_case(x, p, f"tie over allocation tiles, {n_tied} tied")
    bm = R[pl["off_bitmap"]:pl["off_bitmap"] + 8 * pl["nblocks"]].view(np.uint64)
    hi = np.unpackbits(bm.view(np.uint8), bitorder="little")[:T * H // G].astype(bool).reshape(na, A // G)
    tied_idx = np.flatnonzero(kind == 1)
    n_sel = na // 2 - n_flat
    assert hi[kind == 0].all() and not hi[kind == 2].any()
    assert hi[tied_idx[:n_sel]].all() and not hi[tied_idx[n_sel:]].any()


@pytest.mark.parametrize("S,ns", [(65, 5), (193, 3), (1024, 2)])
def test_counts_in_place_of_the_block_table(S, ns):
    """Samples of whole runs of 64 tiles above the one-workgroup select: the
    last select pass writes the width map's sure bits and the counts per run
    and per chunk of 64 runs, the resolve step adds the tiles at the
    threshold, and the encoder sums the counts into the block table. Chunks
    that end inside a sample (65 and 193 runs), several samples, and a
    threshold inside a class of equal tiles spread over every sample."""
    G, M = 64, 64
    T = S * ns
    x = synth.random_tensor(T, G * M, synth.BF16, 70 + S, n_out=3, mult=40)
    p = P(tile=G, tokens_per_sample=S, bit_budget=3.4, candidates=(3, 4), tau=2.0)
    assert oracle.plan(T, G * M, p)["atiles_per_sample"] == S * M
    run_case(x, p, f"counts S={S} samples={ns}")
    # a third of the tiles one repeated tile whose entropy sits in the middle
    rng = np.random.default_rng(S)
    tiles = rng.standard_normal((T * M, G)) * rng.choice([0.01, 1.0], (T * M, 1))
    tied = np.where(np.arange(G) % 2 == 0, 1.0, 0.0) * np.linspace(0.5, 1.5, G)
    tiles[rng.random(T * M) < 0.33] = tied
    xt = tiles.reshape(T, G * M).astype(np.float32)
    for budget in (3.2, 3.5, 3.8):
        run_case(xt, P(tile=G, tokens_per_sample=S, bit_budget=budget, candidates=(3, 4), tau=2.0),
                 f"counts ties S={S} samples={ns} budget {budget}")


def test_one_sample_past_the_in_place_table_limit():
    """One sample of 1,064,960 tiles (16,640 runs of 64, more than the resolve
    workgroup scans in LDS): the select marks and scans in separate launches;
    payload and round trip against the oracle, checked at sampled tiles of
    the whole width map and every block-table entry."""
    T, H = 8320, 8192
    x = synth.random_tensor(T, H, synth.BF16, 77, n_out=8, mult=60)
    p = P(tile=64, tokens_per_sample=0, bit_budget=3.8, candidates=(3, 4), tau=2.0)
    pl = oracle.plan(T, H, p)
    assert pl["tiles_per_sample"] // 64 > 16384
    say("[edge] one sample past the in-place table limit: oracle")
    R = oracle.encode(x, p)
    say("[edge] one sample past the in-place table limit: GPU")
    y, P_ = tah.roundtrip(to_dev(x), p, torch.bfloat16)
    assert_payload_equal(to_host(P_), R, pl, "one sample past the in-place table limit")
    y_ref = oracle.decode(R, T, H, p, oracle.BF16)
    assert_decoded_equal(to_host(y), y_ref, R, pl, "one sample past the in-place table limit")


def random_config_large(seed):
    """A seeded random configuration of up to 3000 tokens and 64 tiles per
    token: samples above the one-workgroup select's 4096 keys, several groups
    per encoder workgroup; both allocators."""
    r = np.random.default_rng(90000 + seed)
    G = int(r.choice([32, 64, 128]))
    M = int(r.integers(1, 65))
    tokens = int(r.integers(1, 3001))
    divisors = [d for d in range(1, tokens + 1) if tokens % d == 0]
    S = int(r.choice([0] + divisors))
    kA = int(r.choice([k for k in range(1, M + 1) if M % k == 0]))
    n_c = int(r.integers(1, 5))
    cands = tuple(sorted(int(c) for c in r.choice(np.arange(1, 9), size=n_c, replace=False)))
    budget = float(np.float32(r.uniform(cands[0], cands[-1] + 0.5)))
    tau = float(r.choice([0.0, 1.0, 2.0, 4.0, math.inf]))
    dtype = synth.F32 if r.random() < 0.5 else synth.BF16
    x = synth.random_tensor(tokens, G * M, dtype, 95000 + seed, scale=float(r.choice([1e-3, 1.0, 50.0])),
                            n_out=int(r.integers(0, 4)), mult=float(r.choice([5.0, 40.0, 300.0])))
    p = P(tile=G, tokens_per_sample=S, bit_budget=budget, candidates=cands, tau=tau, alloc_tile=G * kA,
          allocator=seed % 2)
    return x, p


@pytest.mark.parametrize("seed", range(30))
def test_random_larger_configurations(seed):
    x, p = random_config_large(seed)
    R, _ = run_case(x, p, f"larger random config {seed}")
    if x.dtype == np.uint16:
        tokens, hidden = x.shape
        y16, _ = tah.roundtrip(to_dev(x), p, torch.bfloat16)
        assert_decoded_equal(to_host(y16), oracle.decode(R, tokens, hidden, p, oracle.BF16), R,
                             oracle.plan(tokens, hidden, p), f"larger random config {seed} bf16 out")


@pytest.mark.parametrize("tile,dtype", [(64, synth.BF16), (32, synth.F32), (32, synth.BF16)])
def test_ragged_tail_with_several_groups_per_workgroup(tile, dtype):
    # 9001 tokens of 37 tiles: 333,037 tiles, more 64-tile groups than the
    # encoder has resident workgroups, so workgroups prefetch further groups
    # and one of them ends on a group of 45 tiles; uniform, top-p and greedy
    x = synth.random_tensor(9001, tile * 37, dtype, 4242 + tile, n_out=3, mult=40)
    run_case(x, P(tile=tile, tokens_per_sample=0, bit_budget=3.0, candidates=(3, 4, 8), tau=2.0),
             f"ragged tail t{tile} uniform")
    run_case(x, P(tile=tile, tokens_per_sample=0, bit_budget=3.5, candidates=(3, 4), tau=2.0),
             f"ragged tail t{tile} top-p")
    run_case(x, P(tile=tile, tokens_per_sample=0, bit_budget=3.3, candidates=(2, 3, 4, 8), tau=2.0, allocator=1),
             f"ragged tail t{tile} greedy")


@pytest.mark.parametrize("budget", [3.0, 3.8])
def test_beyond_2_31_elements(budget):
    # 513 samples of one 64 x 65536 bf16 block: 2,151,677,952 elements (past 2^31;
    # input and output offsets past 2^32 bytes). Every sample is the same
    # block, so each sample's allocation, payload sections and rebuilt rows are the
    # oracle's encoding of that block, shifted by the sample's position; sampled
    # samples (first, middle, last) are compared byte for byte. Uniform 3-bit and
    # the 80/20 split (the grid-wide select with the width map written in place).
    reps, T, C = 513, 64, 65536
    B = synth.random_tensor(T, C, synth.BF16, 31, n_out=3, mult=40)
    p = P(tile=64, tokens_per_sample=T, bit_budget=budget, candidates=(3, 4, 8), tau=2.0)
    say(f"[large] {reps * T}x{C} bf16, budget {budget}")
    R = oracle.encode(B, p)
    plb = oracle.plan(T, C, p)
    y_ref = oracle.decode(R, T, C, p, oracle.BF16)
    pl = oracle.plan(reps * T, C, p)
    assert pl["tiles"] * 64 > 2 ** 31 and pl["total"] < 2 ** 32
    xt = to_dev(B).repeat(reps, 1)
    y, Pg = tah.roundtrip(xt, p, torch.bfloat16)
    y2 = tah.decode(Pg, reps * T, C, p, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "decode of the payload differs from the round trip"
    del xt, y2
    n = plb["tiles"]  # tiles per sample
    k = plb["k"]
    sz_lo, sz_hi = 8 * plb["b_lo"], 8 * plb["b_hi"]
    code_b = n * sz_lo + k * (sz_hi - sz_lo)  # code bytes of one sample
    assert code_b == plb["code_bytes"]

    def sec(t, off, width, count):
        return to_host(Pg[off + width * t: off + width * (t + count)])

    for s in (0, reps // 2, reps - 1):
        t0 = s * n
        what = f"sample {s} of {reps}, budget {budget}"
        for name, w in (("side", 1), ("scale", 2), ("zero", 4)):
            got = sec(t0, pl[f"off_{name}"], w, n)
            want = R[plb[f"off_{name}"]: plb[f"off_{name}"] + w * n]
            assert np.array_equal(got, want), f"{what}: {name} differs"
        got = to_host(Pg[pl["off_bitmap"] + t0 // 8: pl["off_bitmap"] + (t0 + n) // 8])
        assert np.array_equal(got, R[plb["off_bitmap"]: plb["off_bitmap"] + n // 8]), f"{what}: width map differs"
        tab = to_host(Pg[pl["off_table"] + 4 * (t0 // 64): pl["off_table"] + 4 * ((t0 + n) // 64)]).view(np.uint32)
        tab_b = R[plb["off_table"]: plb["off_table"] + 4 * (n // 64)].view(np.uint32)
        assert np.array_equal(tab, tab_b + np.uint32(s * k)), f"{what}: block table differs"
        c0 = pl["off_codes"] + s * code_b
        got = to_host(Pg[c0: c0 + code_b])
        assert np.array_equal(got, R[plb["off_codes"]: plb["off_codes"] + code_b]), f"{what}: codes differ"
        assert np.array_equal(to_host(y[s * T:(s + 1) * T]), y_ref), f"{what}: rebuilt rows differ"
