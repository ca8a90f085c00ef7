"""GPU-vs-oracle parity of the greedy allocator over every candidate width
(allocator 1), through the C ABI: payload bytes bit for bit (level map,
width-sum table, codes, the zeroed tail of the code section) and decoded
values bit for bit, for encode, decode and both round trips.

The full-size workloads with this allocator (4096 x 2048 over {2,3,4,8},
8192 x 8192 over {3,4,8}, 16384 x 5120 fp32 with A = 640) run in
test_parity_gpu.py's workload test; here: the degenerate budgets (nothing
fits, everything fits, one candidate), ties of every key, ragged shapes,
small samples, and seeded random configurations.
"""

import dataclasses

import numpy as np
import pytest
import torch

import activation_quantization_pipeline_amd as tah
import oracle
import synth
from test_parity_gpu import assert_decoded_equal, random_config, run_case, say, to_dev, to_host

pytestmark = pytest.mark.gpu

P = tah.TahParams
GREEDY = tah.ALLOC_GREEDY


def levels_used(R, pl):
    words = R[pl["off_bitmap"]:pl["off_bitmap"] + 16 * pl["nblocks"]].view(np.uint32)
    t = np.arange(pl["tiles"])
    return np.unique((words[t // 16] >> (2 * (t % 16)).astype(np.uint32)) & 3)


@pytest.mark.parametrize("budget,cands,want", [
    (2.0, (2, 3, 4, 8), {0}),          # R = 0: every tile at c_1, no select
    (8.0, (2, 3, 4, 8), {3}),          # R covers every upgrade
    (9.5, (3, 4, 8), {2}),             # budget above the widest candidate
    (4.0, (4,), {0}),                  # one candidate
    (2.01, (2, 8), {0, 1}),            # R below one upgrade's cost in most samples
    (3.3, (2, 3, 4, 8), {0, 1, 2, 3}),
])
def test_degenerate_budgets(budget, cands, want):
    x = synth.random_tensor(96, 512, synth.BF16, 3, n_out=3, mult=40)
    p = P(tile=64, tokens_per_sample=32, bit_budget=budget, candidates=cands, tau=2.0, allocator=GREEDY)
    R, _ = run_case(x, p, f"greedy budget {budget} cands {cands}")
    pl = oracle.plan(96, 512, p)
    assert set(levels_used(R, pl).tolist()) <= want | {0}
    if len(want) == 1:
        assert set(levels_used(R, pl).tolist()) == want


@pytest.mark.parametrize("tokens,mult", [(97, 64), (130, 33), (257, 40)])
def test_one_sample_levels_in_place(tokens, mult):
    """One sample above the one-workgroup select (more than 4096 upgrades):
    the last key digit writes the levels of the upgrades above the threshold's
    prefix and each run's width sum, the resolve step adds the selected ones
    that match the prefix and scans the sums into the table and the total;
    tile counts that end inside a run, and a tensor of equal tiles (the list
    of candidates overflows and the resolve step goes through every upgrade)."""
    x = synth.random_tensor(tokens, 64 * mult, synth.BF16, tokens + mult, n_out=3, mult=40)
    for budget, cands in ((3.37, (2, 3, 4, 8)), (4.6, (3, 4, 8)), (2.2, (2, 5))):
        run_case(x, P(tile=64, tokens_per_sample=0, bit_budget=budget, candidates=cands, tau=2.0, allocator=GREEDY),
                 f"greedy one sample t{tokens} m{mult} {budget} {cands}")
    row = synth.random_tensor(1, 64, synth.F32, 7, n_out=1, mult=10)
    z = np.tile(row, (tokens, mult)).astype(np.float32)
    run_case(z, P(tile=64, tokens_per_sample=0, bit_budget=3.37, candidates=(2, 3, 4, 8), tau=2.0, allocator=GREEDY),
             f"greedy one sample of equal tiles t{tokens} m{mult}")


@pytest.mark.parametrize("budget", [2.86875, 3.84375, 7.475])
def test_threshold_inside_a_small_tie(budget):
    """One sample of 6144 tiles over {2, 3, 4, 8} with 40 copies of one tile:
    at these budgets e*, the first upgrade that does not fit, is one of the
    copies' equal upgrades, so the copies split between two levels by tile
    index (a class of at most 64 upgrades, ranked by one wavefront)."""
    rng = np.random.default_rng(5)
    T, M, G = 96, 64, 64
    tiles = rng.standard_normal((T * M, G)) * rng.choice([0.05, 1.0], (T * M, 1))
    tiles[rng.integers(0, T * M, size=T * M // 8), rng.integers(0, G, size=T * M // 8)] *= 30
    copy = rng.standard_normal(G)
    copy[3] *= 5
    idx = rng.choice(T * M, size=40, replace=False)
    tiles[idx] = copy
    x = tiles.reshape(T, M * G).astype(np.float32)
    p = P(tile=G, tokens_per_sample=0, bit_budget=budget, candidates=(2, 3, 4, 8), tau=2.0, allocator=GREEDY)
    R, _ = run_case(x, p, f"greedy small tie budget {budget}")
    pl = oracle.plan(T, M * G, p)
    words = R[pl["off_bitmap"]:pl["off_bitmap"] + 16 * pl["nblocks"]].view(np.uint32)
    t = np.arange(pl["tiles"])
    lv = (words[t // 16] >> (2 * (t % 16)).astype(np.uint32)) & 3
    assert len(set(lv[idx].tolist())) == 2  # the threshold lies inside the copies' class


@pytest.mark.parametrize("tile", [32, 64, 128])
@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_one_level_ragged(tile, dtype):
    """Every tile at one level (nothing fits, everything fits, one candidate)
    on tile counts that end inside a 64-tile run: the level map's entries past
    the last tile stay zero, the width-sum table is 64 widths a run."""
    for tokens, mult in ((1, 5), (7, 9), (65, 3)):
        x = synth.random_tensor(tokens, tile * mult, dtype, 11 + tokens, n_out=2, mult=25)
        for budget, cands in ((2.0, (2, 3, 4, 8)), (8.0, (2, 3, 4, 8)), (4.0, (4,)), (9.0, (1, 5))):
            run_case(x, P(tile=tile, tokens_per_sample=0, bit_budget=budget, candidates=cands, tau=2.0,
                          allocator=GREEDY), f"greedy one level t{tokens} m{mult} {budget} {cands}")


@pytest.mark.parametrize("tile", [32, 64, 128])
def test_every_key_ties(tile):
    """A tensor of identical tiles: every entropy is equal, so every upgrade of
    a level ties and the upgrade index alone orders them (the lower tile first)."""
    row = synth.random_tensor(1, tile, synth.F32, 5, n_out=1, mult=10)
    x = np.tile(row, (40, 7)).astype(np.float32)
    for budget, cands in ((3.37, (2, 3, 4, 8)), (4.5, (3, 8)), (2.9, (1, 2, 3, 4))):
        run_case(x, P(tile=tile, tokens_per_sample=0, bit_budget=budget, candidates=cands, tau=2.0, allocator=GREEDY),
                 f"ties tile {tile} {cands} {budget}")
    z = np.zeros((40, tile * 7), np.float32)  # all-zero tiles: H = 0 everywhere
    run_case(z, P(tile=tile, tokens_per_sample=8, bit_budget=3.5, candidates=(2, 3, 4, 8), tau=2.0, allocator=GREEDY),
             f"zeros tile {tile}")
    # a sample of 4096 tiles (12288 upgrades): the select runs grid-wide, every
    # upgrade of a level shares one key, the tie list overflows and the tie
    # step goes through the whole sample
    zb = np.zeros((64, tile * 64), np.float32)
    run_case(zb, P(tile=tile, tokens_per_sample=0, bit_budget=3.37, candidates=(2, 3, 4, 8), tau=2.0,
                   allocator=GREEDY), f"zeros tile {tile}, one large sample")


@pytest.mark.parametrize("tile", [32, 64, 128])
@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_ragged_shapes(tile, dtype):
    for tokens, mult in ((1, 5), (3, 5), (7, 9), (65, 3), (300, 7)):
        x = synth.random_tensor(tokens, tile * mult, dtype, tokens + mult, n_out=2, mult=25)
        run_case(x, P(tile=tile, tokens_per_sample=0, bit_budget=3.4, candidates=(2, 3, 4, 8), tau=2.0,
                      allocator=GREEDY), f"greedy ragged t{tokens} m{mult}")


@pytest.mark.parametrize("S,A", [(1, 0), (3, 0), (16, 0), (16, 320), (4, 64)])
def test_small_samples_and_allocation_tiles(S, A):
    x = synth.random_tensor(48, 320, synth.BF16, S, n_out=3, mult=30)
    run_case(x, P(tile=64, tokens_per_sample=S, bit_budget=3.5, candidates=(2, 3, 4, 8), tau=2.0, alloc_tile=A,
                  allocator=GREEDY), f"greedy S={S} A={A}")
    run_case(x, P(tile=32, tokens_per_sample=S, bit_budget=2.6, candidates=(1, 2, 5), tau=2.0, alloc_tile=A // 2,
                  allocator=GREEDY), f"greedy S={S} A={A // 2} tile32")


def test_empty_tensor():
    p = P(tile=64, tokens_per_sample=0, bit_budget=3.5, candidates=(2, 3, 4, 8), tau=2.0, allocator=GREEDY)
    x = np.zeros((0, 256), np.float32)
    R = oracle.encode(x, p)
    P_ = to_host(tah.encode(to_dev(x), p))
    torch.cuda.synchronize()
    assert np.array_equal(P_, R)


@pytest.mark.parametrize("seed", range(60))
def test_random_configurations(seed):
    x, p = random_config(500 + seed)
    p = dataclasses.replace(p, allocator=GREEDY)
    R, y_ref = run_case(x, p, f"greedy random config {500 + seed}")
    if x.dtype == np.uint16:
        tokens, hidden = x.shape
        y16, _ = tah.roundtrip(to_dev(x), p, torch.bfloat16)
        assert_decoded_equal(to_host(y16), oracle.decode(R, tokens, hidden, p, oracle.BF16), R,
                             oracle.plan(tokens, hidden, p), f"greedy random config {500 + seed} bf16 out")


def test_header_mismatch_sets_status():
    """A top-p% payload decoded as greedy (and the reverse) is rejected on the device."""
    x = synth.random_tensor(64, 512, synth.BF16, 9, n_out=3, mult=40)
    p0 = P(tile=64, tokens_per_sample=0, bit_budget=3.5, candidates=(3, 4), tau=2.0)
    p1 = dataclasses.replace(p0, allocator=GREEDY)
    for a, b in ((p0, p1), (p1, p0)):
        Pa = tah.encode(to_dev(x), a)
        buf = torch.zeros(max(Pa.numel(), tah.payload_bytes(64, 512, b)), dtype=torch.uint8, device="cuda")
        buf[:Pa.numel()] = Pa
        ws = tah.alloc_workspace(64, 512, b)
        tah.decode(buf, 64, 512, b, torch.float32, ws=ws)
        assert tah.read_device_status(ws) == 5


@pytest.mark.parametrize("tokens", [200, 2000])
@pytest.mark.parametrize("tile,budget,cands", [(64, 3.3, (2, 3, 4, 8)), (32, 2.7, (1, 2, 4)), (128, 4.6, (3, 4, 8))])
def test_ties_resolved_from_the_list(tile, budget, cands, tokens):
    """Eight distinct rows repeated: 8 distinct entropies, each shared by many
    tiles, so e*'s key is tied across tiles but few keys match its prefix. With
    200 tokens the sample is small enough for the one-workgroup select; with
    2000 the select runs grid-wide and the tie is broken from the listed
    (key, index) pairs, not by the whole-sample scan."""
    rows = synth.random_tensor(8, tile * 3, synth.F32, tile, n_out=1, mult=20)
    order = np.random.default_rng(tile).integers(0, 8, size=tokens)
    x = np.ascontiguousarray(rows[order]).astype(np.float32)
    p = P(tile=tile, tokens_per_sample=0, bit_budget=budget, candidates=cands, tau=2.0, allocator=GREEDY)
    R, _ = run_case(x, p, f"listed ties tile {tile}, {tokens} tokens")
    pl = oracle.plan(tokens, tile * 3, p)
    assert len(levels_used(R, pl)) >= 2
