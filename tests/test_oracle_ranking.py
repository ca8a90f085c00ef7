"""The oracle's whole-sample allocation against the pages' definition, at the
workloads' full sizes.

TAH-Quant (arXiv 2506.01352v2) Sec. 3.2 ranks a sample's tiles by the Shannon
entropy of their normalised magnitudes (Eq. 1-2) and gives the top p% the
higher width. The oracle evaluates that entropy in fp32 through a tabulated
log2, so near the cut its ranking may differ from the exact one. These pins
rank every tile by its exact entropy (fp64, scipy's own routine, no shared
formula with the oracle) and require the oracle's width wherever the exact
entropy is farther from the cut than the oracle's error bound allows, and
count the tiles left in that band.

Error bound per tile: |H_oracle - H_exact| <= e_t, derived term by term in
exact_entropy_and_bound and checked on every tile. A tile that fewer than k
others could outrank within those bounds is selected by the oracle, and one
that fewer than N - k others could rank below is not (sure_widths).

The block table of a top-p% payload is checked against a running count of
the width map's bits, computed here with numpy.
"""

import math

import numpy as np
import pytest
import scipy.stats

import synth

INTERP_BOUND = 1.11e-5  # linear interpolation of log2(1 + f) on steps of 1/128 (see test_oracle_pins)
U = 2.0**-24  # unit roundoff of fp32


def exact_entropy_and_bound(x, G, chunk=1 << 16):
    """Exact Shannon entropy (bits) of every tile's normalised magnitudes, in
    fp64 by scipy, and a bound e_t on the error of the oracle's fp32 value.

    The oracle evaluates H = log2 L - S / L with L = sum a_k (fp32, left to
    right) and S = sum a_k log2s(a_k) (fma chain), log2s the tabulated log2.
    With u = 2^-24, m = S / L and M = sum a_k |log2 a_k| / L (exact):
      L's relative error        dL <= (G - 1) u                (positive terms)
      log2s(L~) - log2 L       <= I + spacing + dL / ln 2      (I: interpolation)
      S~ / L - S / L           <= (G + 1) u M + 2^-25 [+ I for fp32 elements]
                                  (fma chain over partial sums bounded by M L;
                                  each element's log2 on a table node is off by
                                  its T rounding 2^-25 and one rounding of the sum)
      dividing by L~ not L     <= |m| dL, plus one rounding u |m|
      the final subtraction    <= u |H|."""
    xf = x.astype(np.float32) if x.dtype == np.float32 else synth.bf16_bits_to_f32(x)
    node = x.dtype != np.float32  # widened bf16 values sit on the log2 table's nodes
    tiles = xf.reshape(-1, G)
    n = tiles.shape[0]
    H = np.empty(n)
    tol = np.empty(n)
    dL = (G - 1) * U * 1.001
    for a0 in range(0, n, chunk):
        a = np.abs(tiles[a0:a0 + chunk].astype(np.float64))
        L = a.sum(1)
        pos = L > 0
        Ls = np.where(pos, L, 1.0)
        with np.errstate(invalid="ignore", divide="ignore"):
            h = np.where(pos, scipy.stats.entropy(a, base=2, axis=1), 0.0)
            lg = np.where(a > 0, np.log2(np.where(a > 0, a, 1.0)), 0.0)
        m = (a * lg).sum(1) / Ls
        M = (a * np.abs(lg)).sum(1) / Ls
        lgL = np.abs(np.log2(Ls))
        e = (INTERP_BOUND + np.spacing(lgL.astype(np.float32)).astype(np.float64) + U + dL / math.log(2)
             + (G + 1) * U * M + 2.0**-25 + (0.0 if node else INTERP_BOUND)
             + np.abs(m) * (dL + U) + U * np.abs(h))
        H[a0:a0 + chunk] = h
        tol[a0:a0 + chunk] = np.where(pos, e * 1.01, 0.0)
    return H, tol


def sure_widths(H_exact, tol, k):
    """Tiles that the oracle must select (sure_hi) and must not (sure_lo) in a
    sample whose oracle entropies lie within tol of the exact ones.

    If t is not selected, at least k other tiles rank above it, so at least k
    others have H_exact + tol >= H_exact(t) - tol(t): a tile with fewer such
    rivals is selected. If t is selected, the N - k unselected tiles rank
    below it, so at least N - k others have H_exact - tol <= H_exact(t) +
    tol(t): a tile with fewer is not."""
    up = np.sort(H_exact + tol)
    dn = np.sort(H_exact - tol)
    N = H_exact.size
    lo_t, hi_t = H_exact - tol, H_exact + tol
    rivals_above = N - np.searchsorted(up, lo_t, side="left") - 1  # others with up >= lo_t (t itself counts once)
    rivals_below = np.searchsorted(dn, hi_t, side="right") - 1  # others with dn <= hi_t
    return rivals_above < k, rivals_below < N - k


@pytest.mark.parametrize("name,band_max", [("c2_4096x2048_bf16_g64", 32), ("x2_c5_budget3p8", 256)])
def test_allocation_is_the_exact_entropy_ranking(ref, name, band_max):
    w = synth.workload(name)
    p = w.params
    x = synth.generate(name, 0)
    pl = ref.plan(w.tokens, w.hidden, p)
    st = ref.tile_stats(x, p)
    H_exact, tol = exact_entropy_and_bound(x, p.tile)
    # the oracle's entropy of every tile within its bound of the exact one
    err = np.abs(st["H"].astype(np.float64) - H_exact)
    assert np.all(err <= tol), f"{int((err > tol).sum())} tiles beyond the bound, worst {err.max():.3g}"
    N, k = pl["tiles_per_sample"], pl["k"]
    assert 0 < k < N
    band_total = 0
    differ_total = 0
    for s in range(pl["nsamples"]):
        sl = slice(s * N, (s + 1) * N)
        He, hi = H_exact[sl], st["hi"][sl].astype(bool)
        assert int(hi.sum()) == k
        sure_hi, sure_lo = sure_widths(He, tol[sl], k)
        assert not (sure_hi & sure_lo).any()
        assert hi[sure_hi].all()
        assert not hi[sure_lo].any()
        band = ~(sure_hi | sure_lo)
        band_total += int(band.sum())
        # the exact top k (lower index first among exact ties) differs only inside the band
        order = np.lexsort((np.arange(N), -He))
        want = np.zeros(N, bool)
        want[order[:k]] = True
        differ = want != hi
        assert not (differ & ~band).any()
        differ_total += int(differ.sum())
    print(f"{name}: per-tile bound up to {tol.max():.3g} bits (median {np.median(tol):.3g}); {band_total} tiles "
          f"in the band around the cut, {differ_total} of {pl['tiles']} tiles with a width other than the exact "
          f"ranking's")
    assert band_total <= band_max


def test_top_p_block_table_is_the_bitmap_running_count(ref):
    # Sec. 3.4 packs the 1-bit width map with the codes; the block table holds,
    # for every run of 64 tiles, how many tiles before it have the higher width.
    cases = [("c2_4096x2048_bf16_g64", synth.generate("c2_4096x2048_bf16_g64", 0), None)]
    for A, S, seed in [(64, 8, 3), (256, 4, 5), (1024, 0, 7)]:
        x = synth.random_tensor(64, 1024, synth.F32, seed, n_out=5, mult=40)
        cases.append((f"A={A} S={S}", x, synth.Params(tile=64, tokens_per_sample=S, bit_budget=3.3,
                                                       candidates=(3, 4, 8), alloc_tile=A)))
    for what, x, p in cases:
        if p is None:
            p = synth.workload(what).params
        tokens, hidden = x.shape
        P = ref.encode(x, p)
        pl = ref.plan(tokens, hidden, p)
        n, nb = pl["tiles"], pl["nblocks"]
        bits = np.unpackbits(P[pl["off_bitmap"]:pl["off_bitmap"] + 8 * nb], bitorder="little")[:n]
        st = ref.tile_stats(x, p)
        assert np.array_equal(bits, st["hi"]), what
        run = np.concatenate([[0], np.cumsum(bits.astype(np.int64))])
        tab = P[pl["off_table"]:pl["off_table"] + 4 * nb].view(np.uint32)
        assert np.array_equal(tab, run[np.arange(nb) * 64].astype(np.uint32)), what
        # every sample holds k allocation tiles, kA quantization tiles each, at the higher width
        per = bits.reshape(pl["nsamples"], -1).sum(1)
        assert np.all(per == pl["k"] * pl["kA"]), what
        # and the code blocks follow: tile t starts after the widths of the tiles before it
        w = np.where(bits == 1, pl["b_hi"], pl["b_lo"]).astype(np.int64)
        assert pl["code_bytes"] == int(w.sum()) * p.tile // 8
