"""Benchmark of the TAH-Quant codec on one MI355X.

One step = one fused encode + decode (tah_roundtrip: entropy, allocation,
outlier test, pivot swap + Hadamard, quantization, packing of the payload,
and the rebuilt bf16 tensor) of the 8192 x 8192 bf16 stage-boundary tensor
(GeLU(N(0, 2)) activations with 0.1% outlier channels x200; tile 64; budget
3 bits over {3, 4, 8}). Inputs are resident in HBM before the timed region;
three buffer sets rotate so no step reads what the previous step left in the
256 MB Infinity Cache.

value = algorithmic bytes per step (activations read + payload written +
activations written) / wall time per step, in GB/s; the activation rate
|X| / t is reported beside it (extras.activation_gbps_roundtrip).

Prints one JSON line. Extra legs: the fused round trip of every workload
shape (c1-c4 beside the headline c5, each with its fraction of the HBM peak),
the headline shape on the general path (entropy pass, per-sample select,
width map and block table, then the encoder: a budget of 3.000001 bits makes
k = 1, so every kernel of the mixed path runs), encode-only and decode-only
rates, the same shape with a mixed 80% INT4 / 20% INT3 allocation (the
paper's default), the backward path on activation gradients of the same
shape (the 8-bit fixed-point compressor with the scaling of Eq. 24, encode and
decode, and the TAH-Quant codec at 4 bits), the tile-local Hadamard alone
(the butterfly against the dense product on the matrix cores), a 512 MB device
copy for the achievable bandwidth, and the CPU oracle on the host (single
thread).
"""

import argparse
import dataclasses
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD published figure
WORKLOAD = "c5_8192x8192_bf16_g64"
MIXED = "x2_c5_budget3p8"
GREEDY = "x5b_c5_greedy"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_encode_c5_roundtrip_traffic.json")
CSRC = os.path.join(ROOT, "activation_quantization_pipeline_amd", "csrc")


# The sources the headline kernel (the fused encode + decode) is built and
# launched from: a change to any of them makes the stored counters stale. (The
# headline allocation is uniform, so no selection kernel runs.)
HEADLINE_SOURCES = ("tah_abi.hip", "tah_encode.hip", "tah_device.hpp", "tah_internal.hpp")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in HEADLINE_SOURCES:
        h.update(f.encode())
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def _profiled():
    """The committed counter file, or None when it is missing or the kernel
    sources changed since its counters were taken."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    return t if t.get("kernel_source_hash") == kernel_source_hash() else None


def measured_traffic(bytes_alg):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    runs (scaled by the same counters on a plain copy), or None when stale."""
    t = _profiled()
    return t.get("traffic_bytes_per_launch") if t else None


def measured_valu():
    """VALU lane-ops per element and VALU busy fraction of the same kernel from
    the committed SQ counter runs, or None when stale."""
    t = _profiled()
    sq = t.get("sq") if t else None
    return {"lane_ops_per_element": sq["valu_lane_ops_per_element"], "busy_frac": sq["valu_busy_frac"]} if sq else None


def host_cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def environment(torch) -> dict:
    """GPU, ROCm and host figures recorded with the line."""
    props = torch.cuda.get_device_properties(0)
    rocm = None
    try:
        rocm = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        pass
    return {
        "gpu": props.name,
        "gpu_arch": getattr(props, "gcnArchName", None),
        "compute_units": props.multi_processor_count,
        "gpu_memory_gib": round(props.total_memory / 2**30, 1),
        "rocm": rocm,
        "torch_hip": torch.version.hip,
        "host_cpu": host_cpu_model(),
        "host_nproc": os.cpu_count(),
        "host_cpus_usable": len(os.sched_getaffinity(0)),
    }


def allocation_label(p) -> str:
    """The width pair of the budget (the two candidates around it) as a label."""
    lo = max(c for c in p.candidates if c <= p.bit_budget)
    hi = [c for c in p.candidates if c > p.bit_budget]
    return f"uniform {lo}-bit" if not hi or p.bit_budget == lo else f"top-p {lo}/{hi[0]}-bit"


def to_dev(x, torch):
    import numpy as np

    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


# Extra legs (not the headline step): at least this much untimed back-to-back
# work before each timed window. The round trip's duration follows the part's
# power management: after an idle spell it runs slower for the first
# milliseconds of sustained load (about 65 us, then 75-83 us, before settling
# at 61-63 us on the headline kernel), so short warm-ups would time each leg in
# a different state.
EXTRA_WARM_MS = 40.0


def time_launches(torch, launch, n_sets, steps, warmup, warm_ms=0.0):
    """Times `steps` back-to-back launches after `warmup` untimed ones (and,
    with warm_ms, more untimed launches until that much wall time has passed).

    The timed region is bracketed by synchronize on both sides (wall clock) and
    by one pair of HIP events recorded on the launch stream: their interval / steps
    is the average launch duration (gaps between launches included, so it never
    flatters the kernel). Events between the launches would add their own packets
    to every step, so per-launch events are taken in a second, untimed pass that
    only supplies the median and minimum.
    Returns (wall ms per step, mean ms per launch, median ms, min ms)."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        launch(i % n_sets)
    if warm_ms > 0:
        torch.cuda.synchronize()
        t_w = time.perf_counter()
        i = warmup
        while (time.perf_counter() - t_w) * 1e3 < warm_ms:
            for _ in range(10):
                launch(i % n_sets)
                i += 1
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        launch(i % n_sets)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean = e0.elapsed_time(e1) / steps
    n_ev = min(steps, 50)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_ev)]
    for i in range(n_ev):
        ev[i][0].record(stream)
        launch(i % n_sets)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in ev]
    return wall / steps * 1e3, mean, statistics.median(per), min(per)


def time_extra(torch, launch, n_sets, args):
    """An extra leg: at least 50 warm-up launches and EXTRA_WARM_MS of warm-up
    work, then at least 100 timed launches."""
    return time_launches(torch, launch, n_sets, max(args.steps, 100), max(args.warmup, 50), warm_ms=EXTRA_WARM_MS)


def roundtrip_leg_fn(torch, tah, synth, dev, stream_h, n_sets, args):
    """A timer of the fused round trip of one workload shape."""

    def roundtrip_leg(name, params=None, seed=0, x_sets=None):
        """Fused round trip of one workload shape (payload written, output in the
        input's dtype, three rotating buffer sets): time per launch from the
        events around all launches, GB/s of algorithmic bytes and their fraction
        of the HBM peak."""
        wl = synth.workload(name)
        prm = params or wl.params
        tdt = torch.bfloat16 if wl.dtype == synth.BF16 else torch.float32
        if x_sets is None:
            xh = synth.generate(name, seed)
            x_sets = [to_dev(xh, torch) for _ in range(n_sets)]
        cl = tah.Codec(wl.tokens, wl.hidden, prm, tdt, tdt)
        yl = [torch.empty((wl.tokens, wl.hidden), dtype=tdt, device=dev) for _ in range(n_sets)]
        pl_ = [torch.empty(cl.payload_bytes, dtype=torch.uint8, device=dev) for _ in range(n_sets)]
        wsl = torch.empty(cl.workspace_bytes, dtype=torch.uint8, device=dev)
        xb = x_sets[0].numel() * x_sets[0].element_size()
        nbytes = 2 * xb + cl.payload_bytes
        # extra legs: at least 50 untimed launches and EXTRA_WARM_MS of untimed
        # work, then at least 100 timed launches
        l_ms, l_mean, _, _ = time_extra(torch, lambda i: cl.roundtrip(x_sets[i], pl_[i], yl[i], wsl, stream_h), n_sets, args)
        del yl, pl_, wsl
        gbps = nbytes / (l_mean * 1e-3) / 1e9
        return {"shape": f"{wl.tokens}x{wl.hidden} {'bf16' if wl.dtype == synth.BF16 else 'fp32'} tile {prm.tile}",
                "budget": prm.bit_budget, "candidates": list(prm.candidates), "allocation": allocation_label(prm),
                "us_per_launch": round(l_mean * 1e3, 2), "us_wall_per_step": round(l_ms * 1e3, 2),
                "algorithmic_bytes": nbytes, "gbps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4),
                "activation_gbps": round(xb / (l_mean * 1e-3) / 1e9, 1)}

    return roundtrip_leg


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-extras", action="store_true", help="time only the headline round trip")
    ap.add_argument("--copy-only", action="store_true", help="only a 512 MB device copy (counter calibration)")
    ap.add_argument("--workload", default=None,
                    help="only the fused round trip of this workload (a name from synth), for kernel traces")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the TAH-Quant codec is a per-stage, single-GPU kernel; it measures one GPU only "
              "and does not run with --gpus > 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import activation_quantization_pipeline_amd as tah
    import synth

    dev = torch.device("cuda:0")
    stream_h = torch.cuda.current_stream().cuda_stream

    if args.copy_only:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        ms, mean, med, mn = time_launches(torch, lambda i: dst.copy_(src), 1, args.steps, args.warmup)
        print(json.dumps({"copy_bytes": 512 << 20, "copy_ms": med, "copy_gbps": 2 * (512 << 20) / (med * 1e-3) / 1e9}))
        return

    n_sets = 3
    if args.workload:
        leg = roundtrip_leg_fn(torch, tah, synth, dev, stream_h, n_sets, args)(args.workload)
        print(json.dumps({"workload": args.workload, **leg}))
        return

    w = synth.workload(WORKLOAD)
    p = w.params
    T, C = w.tokens, w.hidden
    x_host = synth.generate(WORKLOAD, 0)
    codec = tah.Codec(T, C, p, torch.bfloat16, torch.bfloat16)
    xs = [to_dev(x_host, torch) for _ in range(n_sets)]
    ys = [torch.empty((T, C), dtype=torch.bfloat16, device=dev) for _ in range(n_sets)]
    ps = [torch.empty(codec.payload_bytes, dtype=torch.uint8, device=dev) for _ in range(n_sets)]
    ws = torch.empty(codec.workspace_bytes, dtype=torch.uint8, device=dev)
    x_bytes = T * C * 2
    bytes_step = x_bytes + codec.payload_bytes + x_bytes  # X read, payload written, Y written

    ms, k_mean, k_med, k_min = time_launches(
        torch, lambda i: codec.roundtrip(xs[i], ps[i], ys[i], ws, stream_h), n_sets, args.steps, args.warmup)
    value = bytes_step / (ms * 1e-3) / 1e9
    achieved = bytes_step / (k_mean * 1e-3) / 1e9

    out = {
        "metric": "encode+decode GB/s of activations on 1 MI355X; % of HBM peak",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "io_dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "8192x8192 bf16 stage-boundary activations, GeLU(N(0,2)) + 0.1% outlier channels x200; "
                        "tile 64, budget 3 bits over {3,4,8}, tau 2; fused encode+decode (tah_roundtrip)",
            "tokens": T,
            "hidden": C,
            "tile": p.tile,
            "bit_budget": p.bit_budget,
            "candidates": list(p.candidates),
            "tau": p.tau,
            "payload_bytes": codec.payload_bytes,
            "bytes_per_step": bytes_step,
            "value_is": "algorithmic bytes per second: activations read + payload written + activations written",
            "hbm_fraction": round(value / HBM_PEAK_GBPS, 4),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "k_encode<64, bf16, bf16 out, uniform allocation>",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(bytes_step),
            "valu": measured_valu(),  # from the SQ counters: the kernel's practical limiter
            "kernel_ms_mean": round(k_mean, 5),
            "kernel_ms_median_separate_pass": round(k_med, 5),
            "kernel_ms_min_separate_pass": round(k_min, 5),
            "algorithmic_bytes_per_launch": bytes_step,
        },
    }

    out["environment"] = environment(torch)

    roundtrip_leg = roundtrip_leg_fn(torch, tah, synth, dev, stream_h, n_sets, args)

    if not args.no_extras:
        extras = {"timing": f"each extra leg: >= 50 warm-up launches and >= {EXTRA_WARM_MS:.0f} ms of warm-up "
                            "work, then >= 100 timed launches (the headline: exactly --warmup and --steps)"}
        # the fused round trip of every workload shape (c5 is the headline, timed above)
        legs = {}
        for name in ("c1_256x512_f32_g32", "c2_4096x2048_bf16_g64", "c3_16384x4096_bf16_g64",
                     "c4_16384x5120_f32_g128"):
            legs[name] = roundtrip_leg(name)
        legs[WORKLOAD] = roundtrip_leg(WORKLOAD, x_sets=xs)
        extras["workloads_roundtrip"] = legs
        # the headline shape on the general path: entropy pass, select, width map
        # and block table, encoder; a budget of 3.000001 bits gives k = 1 of the
        # 1,048,576 tiles, the smallest allocation that runs every kernel of it
        extras["general_path_c5_k1"] = roundtrip_leg(
            WORKLOAD, params=dataclasses.replace(p, bit_budget=3.000001), x_sets=xs)
        # encode only and decode only on the same tensor
        _, e_mean, _, _ = time_extra(torch, lambda i: codec.encode(xs[i], ps[i], ws, stream_h), n_sets, args)
        extras["encode_gbps"] = round((x_bytes + codec.payload_bytes) / (e_mean * 1e-3) / 1e9, 1)
        _, d_mean, _, _ = time_extra(torch, lambda i: codec.decode(ps[i], ys[i], ws, stream_h), n_sets, args)
        extras["decode_gbps"] = round((x_bytes + codec.payload_bytes) / (d_mean * 1e-3) / 1e9, 1)
        extras["activation_gbps_roundtrip"] = round(x_bytes / (ms * 1e-3) / 1e9, 1)
        # general path with a mixed allocation (80% INT4 / 20% INT3) at the same shape
        wm = synth.workload(MIXED)
        cm = tah.Codec(T, C, wm.params, torch.bfloat16, torch.bfloat16)
        pm = [torch.empty(cm.payload_bytes, dtype=torch.uint8, device=dev) for _ in range(n_sets)]
        wsm = torch.empty(cm.workspace_bytes, dtype=torch.uint8, device=dev)
        m_ms, _, _, _ = time_extra(torch, lambda i: cm.roundtrip(xs[i], pm[i], ys[i], wsm, stream_h), n_sets, args)
        extras["mixed_80_20_roundtrip_gbps"] = round((2 * x_bytes + cm.payload_bytes) / (m_ms * 1e-3) / 1e9, 1)
        extras["mixed_80_20_ms_per_step"] = round(m_ms, 5)
        # the sender's and the receiver's side of that allocation apart (one stage
        # encodes, the next decodes): the encode runs the statistics pass, the
        # select and the encoder; the decode reads the payload it wrote
        _, me_mean, _, _ = time_extra(torch, lambda i: cm.encode(xs[i], pm[i], wsm, stream_h), n_sets, args)
        extras["mixed_80_20_encode_gbps"] = round((x_bytes + cm.payload_bytes) / (me_mean * 1e-3) / 1e9, 1)
        extras["mixed_80_20_encode_ms"] = round(me_mean, 5)
        _, md_mean, _, _ = time_extra(torch, lambda i: cm.decode(pm[i], ys[i], wsm, stream_h), n_sets, args)
        extras["mixed_80_20_decode_gbps"] = round((x_bytes + cm.payload_bytes) / (md_mean * 1e-3) / 1e9, 1)
        extras["mixed_80_20_decode_ms"] = round(md_mean, 5)
        del pm, wsm
        # allocation tiles of several quantization tiles (Sec. 3.2), up to token-level
        # allocation (A = hidden), at the same 80/20 split
        for label, A in (("alloc256", 256), ("alloc_token", C)):
            ca = tah.Codec(T, C, dataclasses.replace(wm.params, alloc_tile=A), torch.bfloat16, torch.bfloat16)
            pa = [torch.empty(ca.payload_bytes, dtype=torch.uint8, device=dev) for _ in range(n_sets)]
            wsa = torch.empty(ca.workspace_bytes, dtype=torch.uint8, device=dev)
            a_ms, _, _, _ = time_extra(torch, lambda i: ca.roundtrip(xs[i], pa[i], ys[i], wsa, stream_h), n_sets, args)
            extras[f"mixed_80_20_{label}_roundtrip_gbps"] = round((2 * x_bytes + ca.payload_bytes) / (a_ms * 1e-3) / 1e9,
                                                                 1)
            del pa, wsa
        # the greedy allocator over every candidate width ({3, 4, 8} at 3.8 bits: some tiles
        # take 8 bits where the 80/20 rule gives 4)
        wg = synth.workload(GREEDY)
        cgd = tah.Codec(T, C, wg.params, torch.bfloat16, torch.bfloat16)
        pgd = [torch.empty(cgd.payload_bytes, dtype=torch.uint8, device=dev) for _ in range(n_sets)]
        wsgd = torch.empty(cgd.workspace_bytes, dtype=torch.uint8, device=dev)
        gd_ms, _, _, _ = time_extra(torch, lambda i: cgd.roundtrip(xs[i], pgd[i], ys[i], wsgd, stream_h), n_sets, args)
        extras["greedy_3_4_8_roundtrip_gbps"] = round((2 * x_bytes + cgd.payload_bytes) / (gd_ms * 1e-3) / 1e9, 1)
        extras["greedy_3_4_8_ms_per_step"] = round(gd_ms, 5)
        del pgd, wsgd
        # the outlier thresholds of App. F on the headline configuration (tau = 2 is the headline)
        taus = {"2.0": round(value, 1)}
        for tau in (0.0, 4.0, math.inf):
            ct = tah.Codec(T, C, dataclasses.replace(p, tau=tau), torch.bfloat16, torch.bfloat16)
            pt = [torch.empty(ct.payload_bytes, dtype=torch.uint8, device=dev) for _ in range(n_sets)]
            t_ms, _, _, _ = time_extra(torch, lambda i: ct.roundtrip(xs[i], pt[i], ys[i], ws, stream_h), n_sets, args)
            taus[str(tau)] = round(bytes_step / (t_ms * 1e-3) / 1e9, 1)
            del pt
        extras["tau_sweep_roundtrip_gbps"] = taus
        # the tile-local Hadamard of Eq. (4) alone on the same tensor, fp32 out: the
        # codec's butterfly against the dense product on the matrix cores
        Lb = tah.lib()
        yh = torch.empty(T * C, dtype=torch.float32, device=dev)
        n_t = T * C // p.tile
        had = {}
        for label, meth in (("butterfly", tah.HADAMARD_BUTTERFLY), ("mfma", tah.HADAMARD_MFMA)):
            h_args = [(xs[i].data_ptr(), 1, n_t, p.tile, meth, yh.data_ptr(), stream_h) for i in range(n_sets)]
            rc = Lb.tah_hadamard(*h_args[0])
            if rc != 0:
                raise RuntimeError(f"tah_hadamard({label}): {tah.status_string(rc)}")
            _, h_mean, _, _ = time_extra(torch, lambda i: Lb.tah_hadamard(*h_args[i]), n_sets, args)
            had[label] = round((x_bytes + 4 * T * C) / (h_mean * 1e-3) / 1e9, 1)
        extras["hadamard_alone_gbps"] = had
        del yh
        # the backward path (Algorithm 1, backward pass): activation gradients of the same shape,
        # fixed-point compressor at 8 bits with the scaling of Eq. (24), and TAH-Quant at 4 bits
        gname = "g1_8192x8192_bf16_grad"
        gw = synth.workload(gname)
        g_host = synth.generate(gname, 0)
        gs = [to_dev(g_host, torch) for _ in range(n_sets)]
        nb, nc = synth.NAIVE[gname]["bits"], synth.NAIVE[gname]["c"]
        n_el = gw.tokens * gw.hidden
        npb = tah.naive_payload_bytes(n_el, nb)
        nps = [torch.empty(npb, dtype=torch.uint8, device=dev) for _ in range(n_sets)]
        wsn = torch.zeros(256, dtype=torch.uint8, device=dev)
        ne_args = [(gs[i].data_ptr(), 1, n_el, nb, nc, nps[i].data_ptr(), npb, stream_h) for i in range(n_sets)]
        nd_args = [(nps[i].data_ptr(), npb, n_el, nb, nc, ys[i].data_ptr(), 1, wsn.data_ptr(), 256, stream_h)
                   for i in range(n_sets)]
        _, ne_mean, _, _ = time_extra(torch, lambda i: Lb.tah_naive_encode(*ne_args[i]), n_sets, args)
        _, nd_mean, _, _ = time_extra(torch, lambda i: Lb.tah_naive_decode(*nd_args[i]), n_sets, args)
        extras["bw_naive8_encode_gbps"] = round((2 * n_el + npb) / (ne_mean * 1e-3) / 1e9, 1)
        extras["bw_naive8_decode_gbps"] = round((npb + 2 * n_el) / (nd_mean * 1e-3) / 1e9, 1)
        cg = tah.Codec(gw.tokens, gw.hidden, gw.params, torch.bfloat16, torch.bfloat16)
        pg = [torch.empty(cg.payload_bytes, dtype=torch.uint8, device=dev) for _ in range(n_sets)]
        wsg = torch.empty(cg.workspace_bytes, dtype=torch.uint8, device=dev)
        g_ms, _, _, _ = time_extra(torch, lambda i: cg.roundtrip(gs[i], pg[i], ys[i], wsg, stream_h), n_sets, args)
        extras["bw_tah4_roundtrip_gbps"] = round((2 * 2 * n_el + cg.payload_bytes) / (g_ms * 1e-3) / 1e9, 1)
        del gs, nps, pg, wsg
        # achievable bandwidth of a plain 512 MB device copy
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        _, c_mean, _, _ = time_extra(torch, lambda i: dst.copy_(src), 1, args)
        extras["copy_512MB_gbps"] = round(2 * (512 << 20) / (c_mean * 1e-3) / 1e9, 1)
        del src, dst
        out["extras"] = extras

    if not args.no_cpu_baseline:
        import oracle

        # repeat the whole-tensor encode + decode until about 10 s of CPU work
        runs = []
        while sum(runs) < 10.0 and len(runs) < 20:
            t0 = time.perf_counter()
            R = oracle.encode(x_host, p)
            oracle.decode(R, T, C, p, oracle.BF16)
            runs.append(time.perf_counter() - t0)
        t_cpu = statistics.median(runs)
        out["cpu_baseline"] = {
            "value": round(bytes_step / t_cpu / 1e9, 4),
            "unit": "GB/s",
            "cores": 1,
            "kind": "oracle",
            "host_cpu": host_cpu_model(),
            "host_nproc": os.cpu_count(),
            "sample": f"the full 8192x8192 tensor of this workload, oracle encode then decode to bf16, "
                      f"single thread, median of {len(runs)} runs ({t_cpu:.2f} s each, {sum(runs):.1f} s in all)",
        }

    print(json.dumps(out))


if __name__ == "__main__":
    main()
