"""tah_roundtrip_noalloc (the round trip without a workspace, for callers that
cannot allocate) against tah_roundtrip with a workspace of its own: payload
and rebuilt tensor byte for byte, two calls in a row on one GPU, the second on
a smaller input, for a uniform, a two-width and a greedy allocation (the
select kernels use most of the scratch) and without a payload."""

import numpy as np
import pytest
import torch

import activation_quantization_pipeline_amd as tah
import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def to_dev(x):
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def same(a, b):
    return torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                       b.view(torch.uint8) if b.dtype != torch.uint8 else b)


def check(x, p, what, write_payload=True):
    tokens, hidden = x.shape
    say(f"[noalloc] {what}: {tokens}x{hidden} tile {p.tile} S {p.tokens_per_sample} budget {p.bit_budget} "
        f"cands {p.candidates} A {p.alloc_tile} allocator {p.allocator}")
    assert tah.workspace_bytes(tokens, hidden, p) <= tah.NOALLOC_SCRATCH_BYTES
    xt = to_dev(x)
    y_ref, P_ref = tah.roundtrip(xt, p, write_payload=write_payload)
    y = torch.full_like(y_ref, 7.0)
    P = torch.full_like(P_ref, 0xA5) if write_payload else None
    tah.roundtrip_noalloc(xt, p, P, y)
    torch.cuda.synchronize()
    if write_payload:
        assert same(P, P_ref), f"{what}: payload differs from tah_roundtrip"
    assert same(y, y_ref), f"{what}: rebuilt tensor differs from tah_roundtrip"


P = tah.TahParams


@pytest.mark.parametrize("kind", ["uniform", "top_p", "greedy"])
def test_noalloc_matches_roundtrip_twice_second_smaller(kind):
    if kind == "uniform":
        big = (synth.generate("c5_8192x8192_bf16_g64", 0), synth.workload("c5_8192x8192_bf16_g64").params)
        small = (synth.generate("c5_8192x8192_bf16_g64", 1, tokens=512)[:, :2048].copy(),
                 P(tile=64, tokens_per_sample=0, bit_budget=3.0, candidates=(3, 4, 8), tau=2.0))
    elif kind == "top_p":
        big = (synth.generate("x2_c5_budget3p8", 0), synth.workload("x2_c5_budget3p8").params)
        small = (synth.generate("c2_4096x2048_bf16_g64", 2, tokens=1024),
                 P(tile=64, tokens_per_sample=256, bit_budget=3.5, candidates=(2, 3, 4, 8), tau=2.0))
    else:
        big = (synth.generate("x5b_c5_greedy", 0), synth.workload("x5b_c5_greedy").params)
        small = (synth.random_tensor(300, 1024, synth.F32, 5, n_out=3, mult=40),
                 P(tile=32, tokens_per_sample=100, bit_budget=3.4, candidates=(2, 3, 4, 8), tau=2.0, allocator=1))
    check(*big, f"{kind}, first call")
    check(*small, f"{kind}, second call, smaller")


def test_noalloc_without_payload_and_fp32_out():
    x = synth.generate("c2_4096x2048_bf16_g64", 0)
    p = synth.workload("c2_4096x2048_bf16_g64").params
    xt = to_dev(x)
    y_ref, _ = tah.roundtrip(xt, p, torch.float32, write_payload=False)
    y = torch.empty_like(y_ref)
    tah.roundtrip_noalloc(xt, p, None, y)
    torch.cuda.synchronize()
    assert same(y, y_ref)
    check(synth.random_tensor(64, 512, synth.BF16, 3, n_out=2, mult=30),
          P(tile=64, tokens_per_sample=16, bit_budget=3.5, candidates=(3, 4), tau=2.0, alloc_tile=256), "A = 256")


def test_noalloc_rejects_a_shape_beyond_its_scratch():
    p = P(tile=64, bit_budget=3.8, candidates=(3, 4))
    x = torch.empty((65536, 8192), dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    with pytest.raises(tah.TahError) as e:
        tah.roundtrip_noalloc(x, p, tah.alloc_payload(65536, 8192, p), y)
    assert e.value.code == 7
