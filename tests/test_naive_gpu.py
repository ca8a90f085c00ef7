"""GPU-vs-oracle parity of the backward compressor Q_Naive (Algorithm 1,
backward pass; Appendix H Eq. 24), through the C ABI.

Codes are integers decided in fp32 by the same operations on both sides, so
the payload must be byte-identical and the decoded values bit-identical.
"""

import numpy as np
import pytest
import torch

import activation_quantization_pipeline_amd as tah
import oracle
import synth

pytestmark = pytest.mark.gpu


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


def check(g: np.ndarray, bits: int, c: float, what: str):
    """Encode on both sides, compare payload bytes; decode the oracle's payload
    on the GPU to fp32 and bf16 and compare with the oracle's decode."""
    n = g.size
    say(f"[naive] {what}: n={n} bits={bits} c={c} dtype={g.dtype}")
    R = oracle.naive_encode(g, bits, c)
    P = to_host(tah.naive_encode(to_dev(g.ravel()), bits, c))
    assert P.shape == R.shape
    if not np.array_equal(P, R):
        d = np.flatnonzero(P != R)
        raise AssertionError(f"{what}: {d.size} payload bytes differ, first at {d[0]}")
    Pd = to_dev(R)
    for ydt, odt in ((torch.float32, oracle.F32), (torch.bfloat16, oracle.BF16)):
        y = to_host(tah.naive_decode(Pd, n, bits, c, ydt))
        want = oracle.naive_decode(R, n, bits, c, odt)
        if not np.array_equal(y.view(np.uint32 if ydt == torch.float32 else np.uint16),
                              want.view(np.uint32 if ydt == torch.float32 else np.uint16)):
            bad = np.flatnonzero(y != want)
            raise AssertionError(f"{what}: decode {ydt}: {bad.size} values differ, first at {bad[:1]}")


@pytest.mark.parametrize("name", list(synth.NAIVE))
def test_gradient_workloads_full_size(name):
    w = synth.workload(name)
    g = synth.generate(name, 0)
    check(g, synth.NAIVE[name]["bits"], synth.NAIVE[name]["c"], name)


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16])
def test_every_width(bits):
    rng = np.random.default_rng(bits)
    g = (rng.standard_normal(8192 + 5) * 0.4).astype(np.float32)  # some values saturate
    check(g, bits, 1.0, f"width {bits}")
    check(synth.f32_to_bf16_bits(g), bits, 3.5, f"width {bits} bf16")


@pytest.mark.parametrize("n", [0, 1, 7, 31, 32, 33, 255, 256 * 32 - 1, 256 * 32, 256 * 32 + 1, 100003])
def test_ragged_lengths(n):
    g = synth.gen_gradients(1, n, synth.F32, 3, 60).ravel() if n else np.zeros(0, np.float32)
    check(g, 8, 4096.0, f"length {n}")
    check(synth.f32_to_bf16_bits(g), 6, 4096.0, f"length {n} bf16")


def test_ties_saturation_and_zeros():
    # exact ties k + 1/2 (round to even), saturation at both ends, signed zeros
    bits, c = 8, 1.0
    k = np.arange(-140, 140, dtype=np.float64)
    g = np.concatenate([(k + 0.5) / 128.0, k / 128.0, [0.0, -0.0, 5.0, -5.0, 1e30, -1e30]]).astype(np.float32)
    check(g, bits, c, "ties and saturation")


def test_bad_header_sets_status_and_leaves_output():
    g = np.linspace(-1, 1, 1000, dtype=np.float32)
    R = oracle.naive_encode(g, 8, 1.0)
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    sentinel = torch.full((1000,), 7.0, dtype=torch.float32, device="cuda")
    for byte, val in ((0, 0), (7, 9), (8, 1), (16, 0), (24, 0)):  # magic, bits, n, c, total
        Rb = R.copy()
        Rb[byte] ^= 0x40 if val == 0 else val
        say(f"[naive] corrupt header byte {byte}")
        y = sentinel.clone()
        tah.naive_decode(to_dev(Rb), 1000, 8, 1.0, torch.float32, y=y, ws=ws)
        assert tah.read_device_status(ws) == 5
        assert torch.equal(y, sentinel)
    # a good header resets the status; the input-dtype byte is not checked
    Rb = R.copy()
    Rb[6] = 1
    y = tah.naive_decode(to_dev(Rb), 1000, 8, 1.0, torch.float32, ws=ws)
    assert tah.read_device_status(ws) == 0
    assert np.array_equal(to_host(y), oracle.naive_decode(R, 1000, 8, 1.0))
