"""GPU checks of the standalone tile-local Hadamard transform (TAH-Quant §3.3,
Eq. 4), through the C ABI.

The butterfly is the codec's transform and must equal the oracle's bit for bit.
The matrix-core product adds the same G exact terms in the hardware's own
order, so it is held to the error bound of any fp32 summation of G terms
against the exact product (computed in float64, where a sum of 64 bf16 or fp32
values times +-1 is exact up to one final rounding); on inputs whose sums are
exact in fp32 (small integers) it must equal the butterfly bit for bit.
"""

import numpy as np
import pytest
import torch

import activation_quantization_pipeline_amd as tah
import oracle
import synth

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24  # unit roundoff of fp32


def say(*a):
    print(*a, flush=True)


def to_dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def as_f32(x: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_to_f32(x) if x.dtype == np.uint16 else np.asarray(x, np.float32)


def sylvester(G: int) -> np.ndarray:
    """H[i][j] = (-1)^popcount(i & j), the Sylvester construction."""
    i = np.arange(G)
    return np.where(np.bitwise_count(i[:, None] & i[None, :]) & 1, -1.0, 1.0)


def run(x: np.ndarray, G: int, method: int) -> np.ndarray:
    y = tah.hadamard(to_dev(x.ravel()), G, method)
    torch.cuda.synchronize()
    return y.cpu().numpy().reshape(-1, G)


def oracle_rows(X: np.ndarray, idx) -> np.ndarray:
    return np.stack([oracle.fwht(X[i]) for i in idx]) if len(idx) else np.zeros((0, X.shape[1]), np.float32)


def check_butterfly(x: np.ndarray, G: int, idx, what: str):
    X = as_f32(x).reshape(-1, G)
    Y = run(x, G, tah.HADAMARD_BUTTERFLY)
    R = oracle_rows(X, idx)
    got = Y[idx]
    if not np.array_equal(got.view(np.uint32), R.view(np.uint32)):
        bad = np.argwhere(got.view(np.uint32) != R.view(np.uint32))
        raise AssertionError(f"{what}: {len(bad)} values differ from the oracle, first at tile {idx[bad[0][0]]}")
    return X, Y


def check_mfma_bound(X: np.ndarray, Ym: np.ndarray, idx, what: str):
    """|y - exact| <= G u sum|x| per tile (recursive summation bound, any order)."""
    G = X.shape[1]
    H = sylvester(G)
    X64 = X[idx].astype(np.float64)
    exact = X64 @ H
    bound = G * U32 * np.abs(X64).sum(axis=1, keepdims=True)
    err = np.abs(Ym[idx].astype(np.float64) - exact)
    worst = float((err / np.maximum(bound, 1e-300)).max()) if len(idx) else 0.0
    assert np.all(err <= bound), f"{what}: error {worst:.3g} x the bound"
    return worst


@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
@pytest.mark.parametrize("n_tiles", [1, 63, 64, 65, 64 * 9 + 13])
def test_butterfly_is_the_oracle_transform(G, dtype, n_tiles):
    say(f"[hadamard] butterfly G={G} dtype={dtype} tiles={n_tiles}")
    x = synth.random_tensor(n_tiles, G, dtype, seed=G + n_tiles, n_out=2, mult=300.0)
    check_butterfly(x, G, np.arange(n_tiles), f"G={G} dtype={dtype} tiles={n_tiles}")


@pytest.mark.parametrize("n_tiles", [1, 63, 64, 65, 64 * 300 + 5])
def test_mfma_within_summation_bound(n_tiles):
    say(f"[hadamard] mfma tiles={n_tiles}")
    x = synth.random_tensor(n_tiles, 64, synth.BF16, seed=7 + n_tiles, n_out=3, mult=200.0)
    X = as_f32(x).reshape(-1, 64)
    Ym = run(x, 64, tah.HADAMARD_MFMA)
    check_mfma_bound(X, Ym, np.arange(n_tiles), f"tiles={n_tiles}")


def test_mfma_exact_on_integer_tiles():
    """Integers in [-128, 127]: every partial sum is an integer below 2^14, exact
    in fp32, so any order of addition gives the exact product; the two methods
    and the dense definition agree bit for bit. A wrong operand layout (a
    transposed or shifted row or column) cannot pass this."""
    rng = np.random.default_rng(11)
    n = 64 * 40 + 17
    xi = rng.integers(-128, 128, size=(n, 64)).astype(np.float32)
    x = synth.f32_to_bf16_bits(xi)
    assert np.array_equal(synth.bf16_bits_to_f32(x), xi)
    Ym = run(x, 64, tah.HADAMARD_MFMA)
    Yb = run(x, 64, tah.HADAMARD_BUTTERFLY)
    exact = (xi.astype(np.float64) @ sylvester(64)).astype(np.float32)
    assert np.array_equal(Ym, exact)
    assert np.array_equal(Yb, exact)


def test_full_size_sampled_and_code_changes():
    """The 8192 x 8192 bf16 GeLU activations with outlier channels, tile 64: the
    butterfly equals the oracle on sampled tiles; the matrix-core product stays
    within its bound, and the count of tiles whose 3- and 4-bit codes (the
    oracle's quantizer on each transformed tile) would change if it replaced
    the butterfly is reported."""
    name = "c5_8192x8192_bf16_g64"
    x = synth.generate(name, 0)
    G = 64
    rng = np.random.default_rng(5)
    n_tiles = x.size // G
    idx = np.sort(rng.choice(n_tiles, size=3000, replace=False))
    X, Yb = check_butterfly(x, G, idx, name)
    Ym = run(x, G, tah.HADAMARD_MFMA)
    worst = check_mfma_bound(X, Ym, idx, name)
    diff_vals = int(np.count_nonzero(Ym.view(np.uint32) != Yb.view(np.uint32)))
    # the codec transforms only flagged tiles, after the pivot swap P_d: build
    # those swapped tiles (bf16 bits, so the swap is exact), transform them both
    # ways and quantize each with the oracle's quantizer
    xb = x.reshape(-1, G)
    rows = []
    for i in idx:
        f, d, _, _ = oracle.outlier(X[i], 2.0)
        if f:
            t = xb[i].copy()
            t[0], t[d] = t[d], t[0]
            rows.append(t)
    assert rows, "no sampled tile is flagged at tau = 2"
    S = np.stack(rows)
    Sb = run(S, G, tah.HADAMARD_BUTTERFLY)
    Sm = run(S, G, tah.HADAMARD_MFMA)
    tiles_changed, codes_changed = {3: 0, 4: 0}, {3: 0, 4: 0}
    for r in range(len(rows)):
        for b in tiles_changed:
            lb, sb, qb = oracle.quantize(Sb[r], b)
            lm, sm, qm = oracle.quantize(Sm[r], b)
            n = int(np.count_nonzero(qb != qm))
            codes_changed[b] += n
            tiles_changed[b] += int(n > 0 or lb != lm or sb != sm)
    say(f"[hadamard] {name}: {diff_vals} of {Ym.size} values of the whole tensor differ bitwise between methods; "
        f"worst error {worst:.3g} x bound; {len(rows)} of {len(idx)} sampled tiles flagged; "
        f"flagged tiles whose codes or scale change with the matrix-core product: {tiles_changed}, "
        f"codes changed: {codes_changed}")
