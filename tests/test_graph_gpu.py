"""HIP graph capture of the codec calls (no host synchronisation, no memset,
no allocation inside the library: every call is a sequence of kernel
launches on the caller's stream), through the C ABI.

A captured mixed-allocation round trip (entropy pass, three select passes,
tie resolution, width map, block table, encoder: ten kernels; with the greedy
allocator, five cost-weighted select passes, the final digit, the level map,
the block table and the encoder) and a captured decode are replayed several
times, with eager work on the same buffers
between the replays, and every replay must reproduce the eager results bit for
bit.
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


@pytest.mark.parametrize("name", [
    "c2_4096x2048_bf16_g64",  # top-p mixed allocation at budget 3.5 over {2,3,4,8}
    "x5a_c2_greedy",          # the greedy allocator: cost-weighted select passes, level map, width sums
])
def test_captured_round_trip_and_decode_replay_like_eager(name):
    w = synth.workload(name)
    p = w.params
    T, C = w.tokens, w.hidden
    x = synth.generate(name, 0)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    ws = tah.alloc_workspace(T, C, p)
    P = tah.alloc_payload(T, C, p)
    y = torch.empty((T, C), dtype=torch.bfloat16, device="cuda")
    yd = torch.empty((T, C), dtype=torch.float32, device="cuda")
    ws_d = tah.alloc_workspace(T, C, p)

    say(f"[graph] {name}: eager reference")
    y_ref, P_ref = tah.roundtrip(xt, p, torch.bfloat16)
    yd_ref = tah.decode(P_ref, T, C, p, torch.float32)
    torch.cuda.synchronize()
    R = oracle.encode(x, p)
    assert np.array_equal(P_ref.cpu().numpy(), R)  # the reference itself is the oracle's payload

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the capture stream
        tah.roundtrip(xt, p, payload=P, y=y, ws=ws)
        tah.decode(P, T, C, p, y=yd, ws=ws_d)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    say(f"[graph] {name}: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        tah.roundtrip(xt, p, payload=P, y=y, ws=ws)
        tah.decode(P, T, C, p, y=yd, ws=ws_d)
    torch.cuda.synchronize()

    for rep in range(4):
        # eager work on the same buffers between replays
        P.fill_(0xA5)
        y.fill_(7.0)
        yd.fill_(-3.0)
        ws.fill_(0x5A)
        torch.cuda.synchronize()
        say(f"[graph] {name}: replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(P, P_ref), f"replay {rep}: payload"
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), f"replay {rep}: round trip"
        assert torch.equal(yd.view(torch.int32), yd_ref.view(torch.int32)), f"replay {rep}: decode"
        assert tah.read_device_status(ws_d) == 0
