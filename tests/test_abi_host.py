"""Host-only checks of the C-ABI library: it loads, exports every symbol that
include/tah.h declares, and rejects bad arguments before touching a device.
No compute call is made here (no GPU in this environment)."""

import ctypes
import math
import os
import re

import numpy as np
import pytest

import activation_quantization_pipeline_amd as tah
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tah.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tah_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = tah.lib()
    names = declared_functions()
    assert len(names) >= 11
    assert set(names) == set(tah.EXPORTS)
    for n in names:
        assert hasattr(L, n), n
    assert tah.abi_version() == 4


def test_params_default_is_paper_default():
    p = tah.params_default()
    assert (p.tile, p.candidates, p.tau) == (64, (3, 4), 2.0)
    assert abs(p.bit_budget - 3.8) < 1e-6


def test_sizes_match_oracle_layout(ref):
    for name in list(synth.WORKLOADS) + list(synth.COVERAGE):
        w = synth.workload(name)
        pl = ref.plan(w.tokens, w.hidden, w.params)
        assert tah.payload_bytes(w.tokens, w.hidden, w.params) == pl["total"], name
        assert tah.workspace_bytes(w.tokens, w.hidden, w.params) >= 4 * pl["atiles"]
    for A in (128, 384, 768, 1536):  # kA = 2, 6, 12, 24 over hidden 1536
        p = synth.Params(tile=64, tokens_per_sample=10, bit_budget=3.7, candidates=(3, 4, 8), alloc_tile=A)
        assert tah.payload_bytes(50, 1536, p) == ref.plan(50, 1536, p)["total"], A


def test_decimal_budget_sizes_match_oracle(ref):
    # k (top-p) and R (greedy) follow the budget read as a decimal: 3.8 bits over
    # N = 5 tiles is 4 tiles at 4 bits, which the code section's size shows
    for N in (5, 80, 10240):
        for budget, cands in [(3.8, (3, 4)), (3.3, (3, 4, 8)), (2.6, (2, 3)), (3.1415927, (3, 4))]:
            for alloc in (0, 1):
                p = synth.Params(tile=64, tokens_per_sample=0, bit_budget=budget, candidates=cands, allocator=alloc)
                assert tah.payload_bytes(N, 64, p) == ref.plan(N, 64, p)["total"], (N, budget, alloc)
    p = synth.Params(tile=64, tokens_per_sample=0, bit_budget=3.8, candidates=(3, 4))
    pl = ref.plan(80, 64, p)
    assert pl["code_bytes"] == 80 * 24 + 64 * 8
    assert tah.payload_bytes(80, 64, p) == pl["off_codes"] + ((80 * 24 + 64 * 8 + 255) // 256) * 256


def test_budget_reading_agrees_with_oracle_on_random_budgets(ref):
    # 32 samples of 64-bit-wide tiles: one more upgraded tile per sample adds
    # 32 x 8 bytes, so any difference in k between the library's planner and the
    # oracle's moves the payload size by a whole 256-byte step
    r = np.random.default_rng(77)
    for _ in range(1500):
        S, M = int(r.integers(1, 40)), int(r.integers(1, 9))
        lo = int(r.integers(1, 8))
        digits = int(r.integers(1, 9))
        budget = float(np.float32(round(lo + r.random(), digits)))
        if budget >= lo + 1:
            continue
        p = synth.Params(tile=64, tokens_per_sample=S, bit_budget=budget, candidates=(lo, lo + 1))
        assert tah.payload_bytes(32 * S, 64 * M, p) == ref.plan(32 * S, 64 * M, p)["total"], (budget, S, M)
        g = synth.Params(**{**p.__dict__, "candidates": (lo, lo + 1, 8) if lo + 1 < 8 else (lo, 8), "allocator": 1})
        assert tah.payload_bytes(32 * S, 64 * M, g) == ref.plan(32 * S, 64 * M, g)["total"], (budget, S, M)


def test_noalloc_round_trip_rejects_shapes_beyond_its_scratch():
    # checked on the host before any device call: no GPU is needed to see it
    L = tah.lib()
    v = ctypes.c_void_p
    p = tah.TahParams(tile=64, bit_budget=3.8, candidates=(3, 4))
    cp = tah._cparams(p)
    big = (65536, 8192)
    assert tah.workspace_bytes(*big, p) > tah.NOALLOC_SCRATCH_BYTES
    need = tah.payload_bytes(*big, p)
    assert L.tah_roundtrip_noalloc(v(16), 1, *big, ctypes.byref(cp), v(16), need, v(16), 1, v(0)) == 7
    assert "scratch" in tah.status_string(7)
    # the other argument errors come first, as in tah_roundtrip
    assert L.tah_roundtrip_noalloc(v(0), 1, *big, ctypes.byref(cp), v(16), need, v(16), 1, v(0)) == 1
    assert L.tah_roundtrip_noalloc(v(16), 1, *big, ctypes.byref(cp), v(16), need - 1, v(16), 1, v(0)) == 3
    assert L.tah_roundtrip_noalloc(v(16), 1, 4, 100, ctypes.byref(cp), v(16), 1 << 20, v(16), 1, v(0)) == 1
    # the workloads all fit
    for name in list(synth.WORKLOADS) + list(synth.COVERAGE):
        w = synth.workload(name)
        assert tah.workspace_bytes(w.tokens, w.hidden, w.params) <= tah.NOALLOC_SCRATCH_BYTES, name


def test_status_strings():
    for c in range(8):
        assert tah.status_string(c)


def _call_encode(p, tokens=4, hidden=128, x=16, payload=16, ws=16, pcap=1 << 20, wcap=1 << 20, dtype=1):
    cp = tah._cparams(p)
    return tah.lib().tah_encode(ctypes.c_void_p(x), dtype, tokens, hidden, ctypes.byref(cp), ctypes.c_void_p(payload),
                                pcap, ctypes.c_void_p(ws), wcap, ctypes.c_void_p(0))


def test_argument_errors_without_device():
    good = tah.TahParams(tile=64, bit_budget=3.5, candidates=(3, 4))
    bad = [
        (dict(tile=48), 1), (dict(tile=256), 1), (dict(candidates=(4, 3)), 1), (dict(candidates=(0, 3)), 1),
        (dict(candidates=(3, 9)), 1), (dict(tau=math.nan), 1), (dict(tau=-1.0), 1), (dict(bit_budget=math.nan), 1),
        (dict(bit_budget=math.inf), 1), (dict(tokens_per_sample=3), 1), (dict(bit_budget=2.0), 4),
        (dict(tile=16), 2), (dict(tile=8), 2),
        (dict(alloc_tile=32), 1), (dict(alloc_tile=96), 1), (dict(alloc_tile=256), 1), (dict(alloc_tile=-64), 1),
    ]
    for over, code in bad:
        fields = {**good.__dict__, **over}
        assert _call_encode(tah.TahParams(**fields)) == code, over
    for A in (0, 64, 128):  # allocation tiles that fit hidden = 128 pass validation (then fail on the pointers)
        assert _call_encode(tah.TahParams(**{**good.__dict__, "alloc_tile": A}), x=0) == 1
        assert _call_encode(tah.TahParams(**{**good.__dict__, "alloc_tile": A}), pcap=10) == 3
    # shape and pointer errors
    assert _call_encode(good, hidden=100) == 1
    assert _call_encode(good, tokens=-1) == 1
    assert _call_encode(good, x=0) == 1
    assert _call_encode(good, x=8) == 1  # not 16-byte aligned
    assert _call_encode(good, payload=0) == 1
    assert _call_encode(good, ws=0) == 1
    assert _call_encode(good, dtype=7) == 1
    assert _call_encode(good, pcap=10) == 3
    assert _call_encode(good, wcap=10) == 3


def test_decode_argument_errors_without_device():
    p = tah.TahParams(tile=64, bit_budget=3.0, candidates=(3,))
    cp = tah._cparams(p)
    L = tah.lib()
    need = tah.payload_bytes(4, 128, p)
    v = ctypes.c_void_p
    assert L.tah_decode(v(16), need - 1, 4, 128, ctypes.byref(cp), v(16), 0, v(16), 1 << 20, v(0)) == 3
    assert L.tah_decode(v(0), need, 4, 128, ctypes.byref(cp), v(16), 0, v(16), 1 << 20, v(0)) == 1
    assert L.tah_decode(v(16), need, 4, 128, ctypes.byref(cp), v(16), 5, v(16), 1 << 20, v(0)) == 1
    assert L.tah_decode(v(16), need, 4, 128, ctypes.byref(cp), v(0), 0, v(16), 1 << 20, v(0)) == 1


def test_payload_size_is_shape_only(ref):
    p = tah.TahParams(tile=64, tokens_per_sample=1024, bit_budget=3.5, candidates=(2, 3, 4, 8))
    n1 = tah.payload_bytes(4096, 2048, p)
    assert n1 == tah.payload_bytes(4096, 2048, p)
    # no tokens: every section is empty, only the 256-byte header section is left
    assert tah.payload_bytes(0, 2048, p) == ref.plan(0, 2048, p)["total"] == 256


def test_device_log2_tables_match_their_definition():
    """The GPU library's log2 tables of the entropy (literal constants in its
    device header) against their definition, recomputed here in double
    precision: T[j] = fp32(log2(1 + j/128) - 1), D[j] = fp32((log2(1 + (j+1)/128)
    - log2(1 + j/128)) / 2^16)."""
    import numpy as np

    src = open(os.path.join(ROOT, "activation_quantization_pipeline_amd", "csrc", "tah_device.hpp")).read()
    body = src[src.index("kLog2Tab[256] = {"):]
    body = body[body.index("{") + 1:body.index("};")]
    vals = [float.fromhex(x[:-1]) for x in re.findall(r"-?0x1[0-9a-f.]*p[+-]\d+f", body)]
    assert len(vals) == 256
    for j in range(128):
        a, b = math.log2(1 + j / 128), math.log2(1 + (j + 1) / 128)
        assert np.float32(vals[j]) == np.float32(a - 1.0), j
        assert np.float32(vals[128 + j]) == np.float32((b - a) / 65536.0), j


def test_naive_sizes_match_oracle(ref):
    for n, bits in ((0, 8), (1, 2), (31, 6), (32, 6), (33, 10), (4096 * 2048, 8), (1000, 16)):
        assert tah.naive_payload_bytes(n, bits) == ref.naive_payload_bytes(n, bits)


def test_naive_argument_errors_without_device():
    L = tah.lib()
    v = ctypes.c_void_p
    need = tah.naive_payload_bytes(1000, 8)
    enc = lambda g=16, dt=1, n=1000, bits=8, c=1.0, P=16, cap=need: L.tah_naive_encode(v(g), dt, n, bits, c, v(P), cap, v(0))
    assert enc(bits=1) == 1 and enc(bits=17) == 1 and enc(c=0.0) == 1 and enc(c=-1.0) == 1
    assert enc(c=math.inf) == 1 and enc(c=math.nan) == 1 and enc(c=3e38, bits=16) == 1  # c 2^15 overflows
    assert enc(n=-1) == 1 and enc(g=0) == 1 and enc(g=8) == 1 and enc(P=0) == 1 and enc(dt=3) == 1
    assert enc(cap=need - 1) == 3
    dec = lambda P=16, ln=need, n=1000, bits=8, c=1.0, y=16, dt=0, ws=16, wcap=256: L.tah_naive_decode(
        v(P), ln, n, bits, c, v(y), dt, v(ws), wcap, v(0))
    assert dec(ln=need - 1) == 3 and dec(wcap=255) == 3
    assert dec(P=0) == 1 and dec(y=0) == 1 and dec(ws=0) == 1 and dec(dt=2) == 1 and dec(bits=0) == 1
    with pytest.raises(tah.TahError):
        tah.naive_payload_bytes(10, 20)


def test_hadamard_argument_errors_without_device():
    L = tah.lib()
    v = ctypes.c_void_p
    had = lambda x=16, dt=1, n=10, G=64, m=0, y=16: L.tah_hadamard(v(x), dt, n, G, m, v(y), v(0))
    assert had(G=16) == 1 and had(G=256) == 1 and had(G=48) == 1
    assert had(m=2) == 1 and had(m=-1) == 1 and had(dt=3) == 1 and had(n=-1) == 1
    assert had(x=0) == 1 and had(y=0) == 1 and had(x=8) == 1 and had(y=4) == 1
    # the matrix-core form exists only for bf16 tiles of 64
    assert had(m=1, G=32) == 2 and had(m=1, G=128) == 2 and had(m=1, dt=0) == 2
    # nothing to do: no pointer is needed and no device is touched
    assert had(n=0, x=0, y=0) == 0 and had(n=0, x=0, y=0, m=1) == 0


def test_binding_refuses_host_tensors_before_any_device_call():
    """A host pointer handed to a kernel would be a device memory fault: every
    entry point of the binding refuses CPU tensors up front."""
    import torch

    p = tah.TahParams(tile=64, bit_budget=3.5, candidates=(3, 4))
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    u8 = torch.zeros(1 << 16, dtype=torch.uint8)
    calls = [
        lambda: tah.encode(x, p),
        lambda: tah.roundtrip(x, p),
        lambda: tah.tile_entropy(x, p),
        lambda: tah.decode(u8, 4, 64, p),
        lambda: tah.naive_encode(x, 8, 1.0),
        lambda: tah.naive_decode(u8, 10, 8, 1.0),
        lambda: tah.hadamard(x, 64),
        lambda: tah.read_device_status(u8),
        lambda: tah.Codec(4, 64, p, torch.bfloat16).roundtrip(x, u8, x, u8, 0),
    ]
    for i, call in enumerate(calls):
        with pytest.raises(tah.TahError):
            call()


def test_greedy_allocator_sizes_and_errors(ref):
    """The greedy allocator's payload and header layout agree with the oracle's
    plan (sizes of every section, R), and its argument errors come back before
    any device call."""
    g = np.random.default_rng(4)
    for trial in range(200):
        G = int(g.choice([32, 64, 128]))
        M = int(g.integers(1, 20))
        tokens = int(g.integers(0, 300))
        S = int(g.choice([0] + [d for d in range(1, max(tokens, 1) + 1) if tokens % d == 0][:6]))
        kA = int(g.choice([k for k in range(1, M + 1) if M % k == 0]))
        n = int(g.integers(1, 5))
        cands = tuple(sorted(int(c) for c in g.choice(np.arange(1, 9), n, replace=False)))
        budget = float(np.float32(g.uniform(cands[0], cands[-1] + 1)))
        p = synth.Params(tile=G, tokens_per_sample=S, bit_budget=budget, candidates=cands, alloc_tile=G * kA,
                         allocator=1)
        pl = ref.plan(tokens, G * M, p)
        assert tah.payload_bytes(tokens, G * M, p) == pl["total"], p
        assert tah.workspace_bytes(tokens, G * M, p) >= 4 * pl["atiles"]
    good = tah.TahParams(tile=64, bit_budget=3.5, candidates=(2, 3, 4, 8), allocator=tah.ALLOC_GREEDY)
    assert _call_encode(tah.TahParams(**{**good.__dict__, "allocator": 2})) == 1
    assert _call_encode(tah.TahParams(**{**good.__dict__, "allocator": -1})) == 1
    assert _call_encode(tah.TahParams(**{**good.__dict__, "bit_budget": 1.5})) == 4
    assert _call_encode(good, x=0) == 1  # valid parameters, then the null input pointer
    # the block table's running width sums are 32-bit: 2^32 / 8 tiles at 8 bits do not fit
    big = tah.TahParams(tile=64, bit_budget=8.0, candidates=(8,), allocator=tah.ALLOC_GREEDY)
    assert _call_encode(big, tokens=1 << 23, hidden=64 * 64) == 1
