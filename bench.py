"""Benchmark one routed-MoE step (route -> bucket -> expert FFN) on one MI355X.

A step is one pass of the whole path over one batch: routing (top-k and
bucketing) and the expert FFN with the weighted unroute.  By default it is
one moe_step_packed call (at decode size two launches: the selection with
the gate/up projection, then the down projection with the weighted unroute;
larger batches route, bucket and run the expert kernels), the weights also
packed once in MFMA tile order at load
time, outside every timed region (only the MFMA tiles of large batches read
that copy); --path step runs moe_step on the standard layout alone, --path
calls_unfused the three separate calls.  Steps are captured in HIP graphs.
The default workload is the decode verify step: T=4 tokens, H=2048, I=512,
E=512 experts, top-10, NVFP4 experts, bf16 activations.

Cache control: NB weight banks (expert e of bank b is expert e-67b of bank 0,
at distinct addresses) with NB activation/routing sets; one HIP graph holds
the NB steps back to back, so no expert's bytes are re-read within NB steps
of traffic (the 256 MB MALL would otherwise hold a step's ~69 MB).

Output: one JSON line.  `value` is the effective HBM bandwidth on unique
expert bytes (unique experts of the step x 1,769,484 B) divided by the
measured step time; `us_per_step` is the step time.  `roofline` covers the
dominant kernel, the selection + gate/up launch at decode size (the gate/up
projection at larger batches): HIP events on its stream around a
graph of back-to-back launches of that kernel alone.
`cpu_baseline` is the fp64 CPU oracle timed on this host on a bounded sample.
`router` times the router projection that produces the logits
(moe_router_logits, outside the step) on the workload's tokens, over
rotating copies of the router weights so they are read from HBM, against
its own roofline (HBM for small batches, fp64 arithmetic for large ones),
with the oracle's projection timed on the host beside it.  `layers` chains
L layers (router projection + step per layer, each on its own weight bank
and router weights) in one graph, each layer's input the previous input
plus the previous output (a residual stream).  `protocol` adds seven timed
rounds (median, min, max), the same step on one bank (cache-resident), the
expert FFN alone, a device-to-device copy as the practical bandwidth ceiling
and the bytes a per-route kernel would stream; `cpu_baseline.one_core` is the
oracle with its BLAS on one thread.  `clocks` samples the GPU's clocks and
socket power (amdsmi) while the headline steps replay back to back for a few
seconds after the timed region.  `configs` times every workload (the five
configurations and the Flash-Next expert shape H=2560, I=640 at decode) the
same way, with the no-reuse per-route variant beside the step at decode_t4
and verify_t32, the bf16 MFMA rate on the method's own flops at the prefill
chunk, and the oracle's host time per step on a labelled token sample.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
EXPERT_BYTES_EXTRA = 12         # three fp32 global scales per expert
METRIC = "routed-MoE µs/step + effective HBM TB/s, T=4 E=512 top-10 NVFP4"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--config", default="decode_t4")
    ap.add_argument("--path", default="packed", choices=["packed", "step", "calls", "calls_unfused"],
                    help="step: moe_step (one call); calls: moe_route_bucket + moe_expert_ffn; "
                         "calls_unfused: the three separate calls")
    ap.add_argument("--banks", type=int, default=8)
    ap.add_argument("--ffn-launches", type=int, default=400,
                    help="launches of the dominant kernel timed with events for the roofline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU oracle sample budget (0 disables the cpu_baseline leg)")
    ap.add_argument("--router-copies", type=int, default=80,
                    help="router weight copies rotated in the router leg (80 x 4 MB: beyond the 256 MB "
                         "Infinity Cache, so each call reads its weights from HBM); 0 skips the leg")
    ap.add_argument("--layers", type=int, default=8,
                    help="layers of the chained leg: router projection + routed step per layer, layer l+1's "
                         "input = layer l's input + its output, layer l on weight bank l (0 skips the leg)")
    ap.add_argument("--shared", type=int, default=1,
                    help="1: the chained layers again with a dense bf16 shared expert per layer, after and beside "
                         "the routed step (0 skips the leg)")
    ap.add_argument("--protocol", type=int, default=1,
                    help="1: add the protocol figures (timed rounds, cache-resident step, FFN alone, copy ceiling); "
                         "0: skip them (counter runs)")
    ap.add_argument("--configs", type=int, default=1,
                    help="1: time every workload (the five configs and the Flash-Next expert shape) after the "
                         "headline and report them under `configs`; 0: skip")
    ap.add_argument("--config-steps", type=int, default=96,
                    help="steps timed per workload in the configs leg")
    ap.add_argument("--clock-seconds", type=float, default=3.0,
                    help="seconds of back-to-back headline steps during which amdsmi samples the GPU's "
                         "clocks and power (0 skips the `clocks` record)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="after the bench, run a plain device-to-device copy of this many MiB three times "
                         "(the known-size kernel that calibrates FETCH_SIZE / WRITE_SIZE counter runs)")
    return ap.parse_args()


def traffic_file(kernel: str, workload: str) -> str:
    """The committed counter record of this kernel at this workload."""
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
KERNEL_SOURCES = ["sparse_moe_expert_amd/csrc/expert_ffn.hip", "sparse_moe_expert_amd/csrc/row_dot.h",
                  "sparse_moe_expert_amd/csrc/moe_common.h", "sparse_moe_expert_amd/csrc/shared_rows.h",
                  "sparse_moe_expert_amd/csrc/work_list.h", "sparse_moe_expert_amd/csrc/select.h",
                  "sparse_moe_expert_amd/csrc/bucket_block.h"]


def kernel_sources_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of the dominant kernel from the committed counter
    runs (FETCH_SIZE + WRITE_SIZE, calibrated against a copy of known size),
    or None when there are none for this workload and kernel or the kernel
    sources changed since."""
    try:
        with open(traffic_file(kernel, workload)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if (rec.get("workload") != workload or rec.get("kernel", "gate_up_kernel") != kernel
            or rec.get("sources_sha256") != kernel_sources_digest()):
        return None
    return int(rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"])


FP64_PEAK_TFLOPS = 78.6


def router_leg(args, cfg, wl, dev):
    """The router projection (moe_router_logits) on the workload's tokens:
    graph-replayed calls over rotating copies of the router weights, HIP
    events on the library's stream; the bound is HBM for small batches (the
    weights, E*H*4 bytes, dominate) and fp64 arithmetic for large ones
    (2*T*H*E flop).  The oracle's router projection is timed on the host
    beside it."""
    import numpy as np
    import torch
    import oracle
    import sparse_moe_expert_amd as sme
    T, H, E = cfg.T, cfg.H, cfg.E
    n = args.router_copies
    x = torch.from_numpy(wl.x.view(np.int16)).to(dev)
    w0 = torch.from_numpy(wl.w_router).to(dev)
    ws = [w0] + [torch.roll(w0, shifts=131 * i, dims=0).contiguous() for i in range(1, n)]
    outs = [torch.empty((T, E), dtype=torch.float32, device=dev) for _ in range(2)]
    for i in range(n):
        sme.moe_router_logits(x, ws[i], outs[i % 2])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            sme.moe_router_logits(x, ws[i], outs[i % 2])
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, 200 // n) if T <= 64 else 1
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * n)
    wbytes = E * H * 4 + T * H * 2 + T * E * 4
    flop = 2.0 * T * H * E
    gbps = wbytes / us / 1e3
    tflops = flop / us / 1e6
    kernel = "router_rows_kernel" if T <= 64 else "router_logits_kernel"
    bound = "hbm" if T <= 64 else "fp64"
    # the oracle's projection on the same tokens (a few calls, host cores)
    t0 = time.perf_counter()
    calls = 0
    while calls == 0 or time.perf_counter() - t0 < 0.5:
        oracle.router_logits(wl.x, wl.w_router)
        calls += 1
    cpu_us = (time.perf_counter() - t0) / calls * 1e6
    return {"kernel": kernel, "us_per_call": round(us, 3), "bound": bound,
            "achieved": round(gbps, 1) if bound == "hbm" else round(tflops, 3),
            "peak": HBM_PEAK_GBPS if bound == "hbm" else FP64_PEAK_TFLOPS,
            "unit": "GB/s" if bound == "hbm" else "TFLOP/s",
            "frac": round(gbps / HBM_PEAK_GBPS, 4) if bound == "hbm" else round(tflops / FP64_PEAK_TFLOPS, 4),
            "bytes_per_call": int(wbytes), "flop_per_call": int(flop), "calls": reps * n,
            "weight_copies": n, "cpu_oracle_us_per_call": round(cpu_us, 1)}


def layers_leg(args, cfg, x0, banks, pks, bias, dev, expert_bytes: int):
    """L routed-MoE layers chained in one graph: per layer the router
    projection (its own router weights) and one step on weight bank l; the
    input of layer l+1 is layer l's input plus its bf16 output.
    Timed per pass with HIP events; bytes are the unique expert bytes of
    every layer plus its router weights."""
    import numpy as np
    import torch
    import sparse_moe_expert_amd as sme
    from moe_inputs import make_workload
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    L = min(args.layers, len(banks))
    w_rs = [torch.from_numpy(make_workload(cfg.name, seed=cfg.seed + 100 + l, with_bank=False).w_router).to(dev)
            for l in range(L)]
    steps = [sme.MoeStep(T, H, I, E, k, dev, path=args.path) for _ in range(L)]
    logits = [torch.empty((T, E), dtype=torch.float32, device=dev) for _ in range(L)]

    # the residual stream: layer l's input is the sum of the first input and
    # the outputs of layers 0..l-1 (a bf16 add by torch, outside the library);
    # without it the outputs shrink layer by layer until the routing degenerates
    xs_l = [x0.view(torch.bfloat16)] + [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in range(L - 1)]

    def one_pass():
        for l in range(L):
            sme.moe_router_logits(xs_l[l], w_rs[l], logits[l])
            steps[l].run(xs_l[l], logits[l], bias, banks[l], packed=pks[l])
            if l + 1 < L:
                torch.add(xs_l[l], steps[l].y, out=xs_l[l + 1])

    one_pass()
    torch.cuda.synchronize()
    n_unique = [int(st.buckets.n_active.item()) for st in steps]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        one_pass()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    reps = max(1, args.steps // (4 * L))
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    nbytes = float(np.sum(n_unique)) * expert_bytes + L * E * H * 4
    out = {"layers": L, "us_per_pass": round(us, 2), "us_per_layer": round(us / L, 3),
           "effective_TBps": round(nbytes / us / 1e6, 4), "unique_experts_per_layer": n_unique,
           "bytes_per_pass": int(nbytes), "passes": reps,
           "per_layer": "router projection + route/bucket + expert FFN (library) + residual add (torch, bf16); "
                        "the input of layer l+1 is the input of layer l plus its output"}

    # the same chain with the router projection, selection and buckets in one
    # call (moe_router_route_bucket: one launch up to 16 tokens) followed by
    # the expert FFN (moe_expert_ffn on the standard layout: below 64 tokens
    # the packed copy is not read)
    if T <= 16:
        counters = [torch.zeros(1, dtype=torch.int32, device=dev) for _ in range(L)]

        def one_pass_fused():
            for l in range(L):
                st = steps[l]
                sme.moe_router_route_bucket(xs_l[l], w_rs[l], bias, k, logits[l], st.topk_idx, st.topk_w,
                                            st.buckets, counters[l])
                st.ffn(xs_l[l], banks[l])
                if l + 1 < L:
                    torch.add(xs_l[l], st.y, out=xs_l[l + 1])

        one_pass_fused()
        torch.cuda.synchronize()
        gf = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gf):
            one_pass_fused()
        for _ in range(3):
            gf.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            gf.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        usf = e0.elapsed_time(e1) * 1e3 / reps
        out["fused_router"] = {
            "us_per_pass": round(usf, 2), "us_per_layer": round(usf / L, 3),
            "effective_TBps": round(nbytes / usf / 1e6, 4),
            "per_layer": "moe_router_route_bucket (projection, top-k and buckets in one launch) + moe_expert_ffn "
                         "+ residual add (torch)"}
    return out


def shared_expert_weights(L, H, Is, dev, seed=500):
    """Per layer a dense bf16 SwiGLU shared expert: W_g, W_u [Is, H] and W_d
    [H, Is], drawn N(0, 1/fan_in) and rounded to bf16."""
    import numpy as np
    import torch
    out = []
    for l in range(L):
        rng = np.random.default_rng([seed, l])
        wg = rng.standard_normal((Is, H)) / np.sqrt(H)
        wu = rng.standard_normal((Is, H)) / np.sqrt(H)
        wd = rng.standard_normal((H, Is)) / np.sqrt(Is)
        out.append(tuple(torch.from_numpy(w.astype(np.float32)).to(dev).to(torch.bfloat16) for w in (wg, wu, wd)))
    return out


def shared_leg(args, cfg, x0, banks, pks, bias, dev, expert_bytes: int):
    """The chained layers with a dense shared expert per layer (bf16 weights,
    Is = I), its output added to the routed one.  Timed three ways, one graph
    each: moe_shared_expert on the routed step's stream after it; on a second
    stream beside it (forked after the router projection, joined before the
    residual add); and moe_step_shared, whose launches carry the shared
    expert's rows.  Then moe_shared_expert alone, cycling over enough weight
    copies that each call reads its weights from HBM."""
    import numpy as np
    import torch
    import sparse_moe_expert_amd as sme
    from moe_inputs import make_workload
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    L = min(args.layers, len(banks))
    w_rs = [torch.from_numpy(make_workload(cfg.name, seed=cfg.seed + 100 + l, with_bank=False).w_router).to(dev)
            for l in range(L)]
    w_sh = shared_expert_weights(L, H, I, dev)
    steps = [sme.MoeStep(T, H, I, E, k, dev, path=args.path) for _ in range(L)]
    logits = [torch.empty((T, E), dtype=torch.float32, device=dev) for _ in range(L)]
    xs_l = [x0.view(torch.bfloat16)] + [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    ys = [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    ws = [torch.empty(max(16, sme.load_library().moe_shared_expert_workspace_size(T, H, I)), dtype=torch.uint8,
                      device=dev) for _ in range(L)]
    side = torch.cuda.Stream(dev)      # default priority

    def one_pass(mode):
        main = torch.cuda.current_stream(dev)
        for l in range(L):
            sme.moe_router_logits(xs_l[l], w_rs[l], logits[l])
            if mode == "fused":
                s = steps[l]
                sme.moe_step_shared(xs_l[l], logits[l], bias, banks[l], k, s.topk_idx, s.topk_w, s.buckets,
                                    s.workspace, s.y, w_sh[l], ys[l], ws[l], packed=pks[l])
            elif mode == "overlapped":
                side.wait_stream(main)
                with torch.cuda.stream(side):
                    sme.moe_shared_expert(xs_l[l], *w_sh[l], y=ys[l], workspace=ws[l])
                steps[l].run(xs_l[l], logits[l], bias, banks[l], packed=pks[l])
                main.wait_stream(side)
            else:
                steps[l].run(xs_l[l], logits[l], bias, banks[l], packed=pks[l])
                sme.moe_shared_expert(xs_l[l], *w_sh[l], y=ys[l], workspace=ws[l])
            torch.add(torch.add(xs_l[l], steps[l].y), ys[l], out=xs_l[l + 1])

    res = {}
    for mode in ("sequential", "overlapped", "fused"):
        one_pass(mode)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            one_pass(mode)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        reps = max(1, args.steps // (4 * L))
        stream = torch.cuda.current_stream(dev)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        res[mode] = round(e0.elapsed_time(e1) * 1e3 / reps / L, 3)
    # alone: 3 * H * Is * 2 weight bytes per call, 96 copies (> the 256 MB Infinity Cache)
    n_cp = 96
    cps = [tuple((torch.randn(shp, device=dev) / shp[1] ** 0.5).to(torch.bfloat16)
                 for shp in ((I, H), (I, H), (H, I))) for _ in range(n_cp)]
    y1, w1 = ys[0], ws[0]
    for c in cps[:4]:
        sme.moe_shared_expert(xs_l[0], *c, y=y1, workspace=w1)
    torch.cuda.synchronize()
    ga = torch.cuda.CUDAGraph()
    with torch.cuda.graph(ga):
        for c in cps:
            sme.moe_shared_expert(xs_l[0], *c, y=y1, workspace=w1)
    ga.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record(stream)
    for _ in range(reps):
        ga.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us_alone = e0.elapsed_time(e1) * 1e3 / reps / n_cp
    wbytes = 3 * H * I * 2
    del cps
    return {"layers": L, "us_per_layer_sequential": res["sequential"], "us_per_layer_overlapped": res["overlapped"],
            "us_per_layer_fused": res["fused"],
            "alone": {"us_per_call": round(us_alone, 3), "weight_bytes": wbytes,
                      "achieved_GBps": round(wbytes / us_alone / 1e3, 1),
                      "frac_of_8TBps": round(wbytes / us_alone / 1e3 / 8000.0, 4),
                      "note": "moe_shared_expert alone (two kernels), 96 weight copies in turn, HIP events"},
            "shared_expert": f"dense SwiGLU, bf16 weights, H={H}, Is={I} ({3 * H * I * 2} bytes per layer), "
                             "moe_shared_expert",
            "per_layer": "router projection + routed step + shared expert (library) + residual add (torch); "
                         "fused: moe_step_shared in place of the step and the shared-expert call"}


def _smi_handle(dev):
    """amdsmi handle of the GPU torch uses (matched by PCI bus), or an error string."""
    import amdsmi
    import torch
    amdsmi.amdsmi_init()
    handles = amdsmi.amdsmi_get_processor_handles()
    if not handles:
        return None, "amdsmi lists no GPU"
    props = torch.cuda.get_device_properties(dev)
    bus = getattr(props, "pci_bus_id", None)
    if bus is not None:
        for h in handles:
            try:
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)
                if int(bdf.split(":")[1], 16) == int(bus):
                    return h, None
            except Exception:
                continue
    if len(handles) == 1:
        return handles[0], None
    return None, f"{len(handles)} GPUs listed and none matched PCI bus {bus}"


def _smi_sample(amdsmi, h):
    """One reading: gfx and memory clocks (MHz), socket power (W), busy (%), hotspot temperature (C)."""
    m = amdsmi.amdsmi_get_gpu_metrics_info(h)

    def num(key):
        v = m.get(key)
        if isinstance(v, (list, tuple)):
            v = [x for x in v if isinstance(x, (int, float)) and x not in (0xFFFF, 0xFFFFFFFF)]
            return float(sum(v) / len(v)) if v else None
        return float(v) if isinstance(v, (int, float)) and v not in (0xFFFF, 0xFFFFFFFF) else None

    return {"gfx_MHz": num("current_gfxclk") or num("current_gfxclks"),
            "mem_MHz": num("current_uclk"),
            "power_W": num("current_socket_power") or num("average_socket_power"),
            "busy_pct": num("average_gfx_activity"),
            "hotspot_C": num("temperature_hotspot")}


def clocks_leg(full, NB: int, dev, seconds: float):
    """Clocks and power while the headline graph replays back to back.

    A thread samples amdsmi's GPU metrics every ~10 ms while the main thread
    keeps the graph queued (a synchronisation every 32 replays) for `seconds`;
    one idle reading is taken before.  Reported: median, min and max of each
    quantity over the samples.  Any amdsmi failure is reported instead of the
    figures (no effect on the timed results, which were taken before)."""
    import threading

    import torch
    try:
        import amdsmi
        h, err = _smi_handle(dev)
        if h is None:
            return {"error": err}
        torch.cuda.synchronize()
        idle = _smi_sample(amdsmi, h)
    except Exception as e:           # no driver access for this user, older metrics table, ...
        return {"error": f"{type(e).__name__}: {e}"}
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                samples.append(_smi_sample(amdsmi, h))
            except Exception:
                pass
            stop.wait(0.01)

    th = threading.Thread(target=sampler, daemon=True)
    full.replay()
    torch.cuda.synchronize()
    th.start()
    t_end = time.perf_counter() + seconds
    n = 0
    while time.perf_counter() < t_end:
        full.replay()
        n += 1
        if n % 32 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    stop.set()
    th.join()
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:
        pass

    # the firmware refreshes the metrics table far less often than we read
    # it: keep the readings taken under load (busy >= 50%); the first ones
    # still show the idle state that preceded the replays
    loaded = [x for x in samples if (x.get("busy_pct") or 0) >= 50]
    use = loaded if loaded else samples

    def stats(key):
        v = sorted(x[key] for x in use if x.get(key) is not None)
        if not v:
            return None
        return {"median": round(v[len(v) // 2], 1), "min": round(v[0], 1), "max": round(v[-1], 1)}

    return {"samples": len(samples), "samples_under_load": len(loaded), "steps": n * NB, "seconds": seconds,
            "gfx_clock_MHz": stats("gfx_MHz"), "mem_clock_MHz": stats("mem_MHz"),
            "socket_power_W": stats("power_W"), "gfx_busy_pct": stats("busy_pct"),
            "hotspot_C": stats("hotspot_C"), "idle": idle,
            "note": "amdsmi GPU metrics read every ~10 ms while the headline graph replays back to back "
                    "(after the timed region); figures over the readings that show the GPU busy"}


def cpu_baseline(cfg, budget_s: float, expert_bytes: int):
    """Time the fp64 oracle (as it stands) on whole steps of the same workload."""
    import numpy as np
    import oracle
    from moe_inputs import make_workload
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = 1
    def sample(budget, seed):
        steps, total, nbytes = 0, 0.0, 0
        while steps == 0 or total < budget:
            wl = make_workload(cfg.name, x_seed=seed + steps)
            t0 = time.perf_counter()
            idx, w = oracle.route_topk(wl.logits, wl.bias, wl.k)
            oracle.bucket_routes(idx, wl.E)
            oracle.moe_output(wl.x, wl.bank, idx, w)
            total += time.perf_counter() - t0
            nbytes += len(np.unique(idx)) * expert_bytes
            steps += 1
        return steps, total, nbytes

    seed = 1000
    steps, total, nbytes = sample(budget_s, seed)
    s_per_step = total / steps
    out = {
        "value": round(nbytes / steps / s_per_step / 1e12, 9),
        "unit": "TB/s",
        "us_per_step": round(s_per_step * 1e6, 1),
        "cores": int(cores),
        "host_cpus": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
        "kind": "oracle",
        "sample": f"{steps} whole steps of {cfg.name} (x seeds {seed}..{seed + steps - 1}), "
                  f"route + buckets + FFN in fp64, {total:.1f} s",
    }
    # the same oracle with its BLAS pinned to one thread, on a smaller sample
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            s1, t1, _ = sample(budget_s / 3, seed)
        out["one_core"] = {"us_per_step": round(t1 / s1 * 1e6, 1), "cores": 1,
                           "sample": f"{s1} whole steps (x seeds {seed}..{seed + s1 - 1}), {t1:.1f} s"}
    except Exception:  # pragma: no cover
        pass
    return out


def protocol_leg(step, full, gu_steps, xs, ls, bias, banks, pks, stream, dev, NB, eff_tbps, route_bytes,
                 bytes_per_step):
    """Measurement protocol figures beside the contract's single timed region:
    seven timed rounds of about 100 steps each (median, min, max), the same
    step replayed on one bank and routing set (cache-resident: the MALL holds
    its experts), the expert FFN alone (moe_expert_ffn over the NB pairs, HIP
    events), a plain device-to-device copy as the device's practical
    bandwidth ceiling, and the bytes a per-route kernel would stream."""
    import numpy as np
    import torch
    log("[bench] protocol figures")
    rounds = []
    per_round = max(1, 100 // NB)
    for _ in range(7):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(per_round):
            full.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        rounds.append(e0.elapsed_time(e1) * 1e3 / (per_round * NB))
    g_hot = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_hot):
        for _ in range(NB):
            step.run(xs[0], ls[0], bias, banks[0], packed=pks[0])
    g_hot.replay()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(per_round):
        g_hot.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    hot_us = e0.elapsed_time(e1) * 1e3 / (per_round * NB)
    g_ffn = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_ffn):
        for b in range(NB):
            gu_steps[b].ffn(xs[b], banks[b], stage=3)
    g_ffn.replay()
    e0.record(stream)
    for _ in range(per_round):
        g_ffn.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ffn_us = e0.elapsed_time(e1) * 1e3 / (per_round * NB)
    cbytes = 1 << 30
    csrc = torch.ones(cbytes, dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(csrc)
    cdst.copy_(csrc)
    e0.record(stream)
    for _ in range(5):
        cdst.copy_(csrc)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_tbps = 2 * cbytes * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del csrc, cdst
    protocol = {
        "rounds_us_per_step": {"median": round(float(np.median(rounds)), 3), "min": round(min(rounds), 3),
                               "max": round(max(rounds), 3), "rounds": 7, "steps_per_round": per_round * NB},
        "hot_us_per_step": round(hot_us, 3),
        "hot_note": "one bank and routing set replayed: its experts stay in the 256 MB Infinity Cache",
        "ffn_only_us": round(ffn_us, 3),
        "ffn_only_note": "moe_expert_ffn alone on the standard weight layout (routing prepared), HIP events over "
                         "the NB pairs; only moe_step_packed's MFMA tiles read the packed copy, so at decode sizes "
                         "the kernels are the step's",
        "copy_ceiling_TBps": round(copy_tbps, 3),
        "value_frac_of_copy": round(eff_tbps / copy_tbps, 4),
        "route_issued_bytes_per_step": int(route_bytes),
        "reuse_factor": round(route_bytes / bytes_per_step, 3),
    }
    log(f"[bench] rounds median {protocol['rounds_us_per_step']['median']} us, hot {hot_us:.2f} us, "
        f"ffn {ffn_us:.2f} us, copy {copy_tbps:.2f} TB/s")

    return protocol

MFMA_PEAK_TFLOPS = 2500.0       # MI355X dense bf16, published


def oracle_step_seconds(wl, budget_s: float):
    """The oracle (as it stands) on one step of `wl`: routing and buckets on
    the whole batch, the FFN on the first n tokens (n grows until the budget
    is spent or every token is done), scaled by T / n.  Returns (seconds per
    step, sample description)."""
    import oracle
    t0 = time.perf_counter()
    idx, w = oracle.route_topk(wl.logits, wl.bias, wl.k)
    oracle.bucket_routes(idx, wl.E)
    t_route = time.perf_counter() - t0
    n, t_ffn = 0, 0.0
    while n < wl.T and (n == 0 or t_ffn < budget_s):
        m = min(wl.T - n, max(1, n))                  # double the sample each round
        t0 = time.perf_counter()
        oracle.moe_output(wl.x, wl.bank, idx, w, tokens=range(n, n + m))
        t_ffn += time.perf_counter() - t0
        n += m
    return t_route + t_ffn * wl.T / n, (f"routing and buckets on all {wl.T} tokens, FFN on tokens 0..{n - 1} "
                                        f"({t_ffn:.1f} s) scaled by {wl.T}/{n}")


def configs_leg(args, dev, NB: int):
    """Every workload at its full size, one after another on the same box:
    the step (path `packed`) graph-replayed over NB weight banks (8 banks of
    ~0.9 GB at the Flash-Next shape, distinct addresses, so no expert is
    re-read from the 256 MB Infinity Cache within NB steps): us/step,
    tokens/s, unique expert bytes per step, effective TB/s on them and the
    fraction of 8 TB/s; at the prefill chunk also the bf16 MFMA rate on the
    method's own 6*H*I flops per route against 2.5 PFLOP/s; at decode_t4 and
    verify_t32 the no-reuse variant (moe_route_topk + moe_expert_ffn_per_route,
    every route streaming its own expert) beside the step; and the oracle's
    host time per step.  The Flash-Next expert shape (H = 2560, I = 640) is
    reported beside the five workloads."""
    import numpy as np
    import torch
    import sparse_moe_expert_amd as sme
    from moe_inputs import get_config, make_workload
    from moe_inputs.configs import CONFIG_ORDER
    names = CONFIG_ORDER + ["flashnext_t4"]
    dev_banks = {}
    out = {}
    stream = torch.cuda.current_stream(dev)
    for name in names:
        cfg = get_config(name)
        T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
        log(f"[bench] configs: {name}")
        wls = [make_workload(name, x_seed=b) for b in range(NB)]
        key = (E, H, I)
        if key not in dev_banks:
            dev_banks.clear()                                    # one shape's banks resident at a time
            torch.cuda.empty_cache()
            W0 = sme.expert_weights_from_numpy(wls[0].bank, dev)
            banks = [W0] + [sme.ExpertWeights(*(torch.roll(t, shifts=67 * b, dims=0).contiguous() for t in W0))
                            for b in range(1, NB)]
            pks = [sme.pack_weights(W) for W in banks] if H % 64 == 0 and I % 64 == 0 else [None] * NB
            dev_banks[key] = (banks, pks)
        banks, pks = dev_banks[key]
        path = "packed" if pks[0] is not None else "step"
        xs = [torch.from_numpy(w.x.view(np.int16)).to(dev) for w in wls]
        ls = [torch.from_numpy(w.logits).to(dev) for w in wls]
        bias = None if wls[0].bias is None else torch.from_numpy(wls[0].bias).to(dev)
        step = sme.MoeStep(T, H, I, E, k, dev, path=path)
        n_unique = []
        for b in range(NB):
            step.run(xs[b], ls[b], bias, banks[b], packed=pks[b])
            torch.cuda.synchronize()
            n_unique.append(int(step.buckets.n_active.item()))
        ebytes = cfg.expert_bytes() + EXPERT_BYTES_EXTRA
        ubytes = float(np.mean(n_unique)) * ebytes

        def timed(fn_graph, nsteps_per_replay):
            fn_graph.replay()
            torch.cuda.synchronize()
            reps = max(2, args.config_steps // nsteps_per_replay)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn_graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e-3 / (reps * nsteps_per_replay), reps * nsteps_per_replay

        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for b in range(NB):
                step.run(xs[b], ls[b], bias, banks[b], packed=pks[b])
        s_step, n_timed = timed(g, NB)
        rec = {"T": T, "H": H, "I": I, "E": E, "k": k, "path": path, "steps_timed": n_timed,
               "us_per_step": round(s_step * 1e6, 3), "tokens_per_s": round(T / s_step, 1),
               "unique_experts_per_step": round(float(np.mean(n_unique)), 2),
               "unique_expert_bytes_per_step": int(ubytes),
               "eff_TBps": round(ubytes / s_step / 1e12, 4),
               "frac_of_8TBps": round(ubytes / s_step / 1e12 / (HBM_PEAK_GBPS / 1e3), 4)}
        if T >= 1024:
            flops = 6.0 * H * I * T * k
            rec["mfma_TFLOPs_algorithmic"] = round(flops / s_step / 1e12, 1)
            rec["mfma_frac_of_2.5PFLOPs"] = round(flops / s_step / 1e12 / MFMA_PEAK_TFLOPS, 4)
        if name in ("decode_t4", "verify_t32"):
            idxs = [torch.empty((T, k), dtype=torch.int32, device=dev) for _ in range(NB)]
            wts = [torch.empty((T, k), dtype=torch.float32, device=dev) for _ in range(NB)]
            ws = sme.make_workspace(T, H, I, E, k, dev)
            y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
            for b in range(NB):
                sme.moe_route_topk(ls[b], bias, k, idxs[b], wts[b])
            gpr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gpr):
                for b in range(NB):
                    sme.moe_route_topk(ls[b], bias, k, idxs[b], wts[b])
                    sme.moe_expert_ffn_per_route(xs[b], banks[b], idxs[b], wts[b], ws, y)
            s_pr, _ = timed(gpr, NB)
            issued = T * k * ebytes
            rec["per_route_variant"] = {
                "us_per_step": round(s_pr * 1e6, 3),
                "route_issued_bytes_per_step": int(issued),
                "issued_TBps": round(issued / s_pr / 1e12, 4),
                "step_speedup_from_reuse": round(s_pr / s_step, 3),
                "note": "moe_route_topk + moe_expert_ffn_per_route (every route streams its own expert), graph "
                        "over the same banks and routing sets"}
        if args.cpu_seconds > 0:
            s_or, sample = oracle_step_seconds(wls[0], min(5.0, args.cpu_seconds / 2))
            rec["oracle"] = {"s_per_step": round(s_or, 4), "gpu_speedup": round(s_or / s_step, 1),
                             "sample": sample}
        log(f"[bench] {name}: {rec['us_per_step']} us/step, {rec['eff_TBps']} TB/s"
            + (f", per-route {rec['per_route_variant']['us_per_step']} us" if "per_route_variant" in rec else ""))
        out[name] = rec
        del g, step
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_moe_expert_amd as sme
    from moe_inputs import get_config, make_workload

    cfg = get_config(args.config)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    expert_bytes = cfg.expert_bytes() + EXPERT_BYTES_EXTRA
    # gate + up codes and scales plus their two fp32 global scales
    GATE_UP_BYTES_PER_EXPERT = 2 * (I * H // 2 + I * H // 16) + 8
    n_routes = T * k
    NB = args.banks

    log(f"[bench] generating {cfg.name} inputs and weights")
    wls = [make_workload(cfg.name, x_seed=b) for b in range(NB)]
    W0 = sme.expert_weights_from_numpy(wls[0].bank, dev)
    banks = [W0] + [sme.ExpertWeights(*(torch.roll(t, shifts=67 * b, dims=0).contiguous() for t in W0))
                    for b in range(1, NB)]
    xs = [torch.from_numpy(w.x.view(np.int16)).to(dev) for w in wls]
    ls = [torch.from_numpy(w.logits).to(dev) for w in wls]
    bias = None if wls[0].bias is None else torch.from_numpy(wls[0].bias).to(dev)
    # path "packed": each bank's weights are also packed in MFMA tile order
    # once, at load time (outside every timed region, like loading a model)
    pks = [sme.pack_weights(W) if args.path == "packed" else None for W in banks]
    torch.cuda.synchronize()
    step = sme.MoeStep(T, H, I, E, k, dev, path=args.path)

    # unique experts per routing set, and warm-up outside capture
    n_unique = []
    for b in range(NB):
        step.run(xs[b], ls[b], bias, banks[b], packed=pks[b])
        torch.cuda.synchronize()
        n_unique.append(int(step.buckets.n_active.item()))
    bytes_per_step = float(np.mean(n_unique)) * expert_bytes

    # One graph holds NB consecutive steps (bank b, routing set b), so the
    # host-side graph launch cost is paid once per NB steps; a second graph
    # holds the remainder so that exactly K steps are timed.
    def capture(nsteps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for b in range(nsteps):
                step.run(xs[b], ls[b], bias, banks[b], packed=pks[b])
        return g

    full = capture(NB)
    rem = args.steps % NB
    tail = capture(rem) if rem else None
    torch.cuda.synchronize()

    log(f"[bench] warm-up {args.warmup} steps")
    for _ in range((args.warmup + NB - 1) // NB):
        full.replay()
    torch.cuda.synchronize()

    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps // NB):
        full.replay()
    if tail is not None:
        tail.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    s_per_step = wall / args.steps
    eff_tbps = bytes_per_step / s_per_step / 1e12
    log(f"[bench] {s_per_step * 1e6:.2f} us/step, {eff_tbps:.3f} TB/s effective")

    # Roofline leg: the dominant kernel is the gate/up projection (two thirds
    # of the weight bytes, the longest kernel of the step).  HIP events on the
    # stream the library launches on (torch's current stream) bracket the
    # replay of a graph that holds only launches of that kernel
    # (moe_expert_ffn_stage 1), back to back over the NB (bank, routing set)
    # pairs, so the average launch duration includes no host launch gaps.
    # Each pair keeps its own step object, so the routing stays that pair's.
    stream = torch.cuda.current_stream(dev)
    reps = max(1, args.ffn_launches // NB)
    # Small batches (at most 40 routes at H = 2048, the rows of one 16-byte
    # chunk per lane) run the small step, whose first launch selects and
    # computes gate/up per route: that launch is the dominant kernel and
    # streams each route's expert tile (route-issued bytes).  Otherwise the
    # gate/up row-dot kernel of moe_expert_ffn on the bucketed routes.
    C_i = I // 32
    small = (T * k <= 40 and H == 2048 and C_i <= 64 and C_i & (C_i - 1) == 0 and args.path in ("packed", "step"))
    gu_steps = []
    for b in range(NB):
        sb = sme.MoeStep(T, H, I, E, k, dev, path=args.path)
        sb.routing(ls[b], bias)
        gu_steps.append(sb)
    if small:
        kname = "select_gate_up_kernel"
        dom_bytes = n_routes * GATE_UP_BYTES_PER_EXPERT + T * H * 2 + n_routes * I * 2 + T * E * 4
        dom_bytes_unique = float(np.mean(n_unique)) * GATE_UP_BYTES_PER_EXPERT + T * H * 2 + n_routes * I * 2
    else:
        kname = "gate_up_kernel"
        dom_bytes = float(np.mean(n_unique)) * GATE_UP_BYTES_PER_EXPERT + T * H * 2 + n_routes * I * 2
        dom_bytes_unique = dom_bytes
    g_dom = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_dom):
        for _ in range(reps):
            for b in range(NB):
                if small:
                    gu_steps[b].run(xs[b], ls[b], bias, banks[b], packed=pks[b], stage=1)
                else:
                    gu_steps[b].ffn(xs[b], banks[b], stage=1)
    g_dom.replay()                      # warm-up
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    g_dom.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    n_dom = reps * NB
    avg = ev0.elapsed_time(ev1) * 1e-3 / n_dom          # seconds per launch
    achieved = dom_bytes / avg / 1e9
    log(f"[bench] {kname} avg {avg * 1e6:.2f} us over {n_dom} launches -> {achieved:.1f} GB/s")

    protocol = None
    if args.protocol:
        protocol = protocol_leg(step, full, gu_steps, xs, ls, bias, banks, pks, stream, dev, NB, eff_tbps,
                                n_routes * expert_bytes, bytes_per_step)

    out = {
        "metric": METRIC,
        "value": round(eff_tbps, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(s_per_step * 1e3, 6),
        "us_per_step": round(s_per_step * 1e6, 3),
        "tokens_per_s": round(T / s_per_step, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": T, "H": H, "I": I, "E": E, "k": k,
                   "weights": "nvfp4", "banks": NB, "path": args.path,
                   "unique_experts_per_step": round(float(np.mean(n_unique)), 2),
                   "unique_expert_bytes_per_step": int(bytes_per_step)},
        "roofline": {"bound": "hbm", "kernel": kname,
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(cfg.name, kname),
                     "avg_launch_us": round(avg * 1e6, 3),
                     "bytes_per_launch": int(dom_bytes), "launches": n_dom,
                     "bytes_basis": ("route-issued: each route's expert gate/up tile, x, logits, h"
                                     if small else "unique experts' gate/up weights, x, h"),
                     "achieved_on_unique_expert_bytes": round(dom_bytes_unique / avg / 1e9, 1)},
    }
    if protocol is not None:
        out["protocol"] = protocol
    if args.clock_seconds > 0:
        log(f"[bench] clocks and power ({args.clock_seconds:.1f} s of steps)")
        out["clocks"] = clocks_leg(full, NB, dev, args.clock_seconds)
    if args.router_copies > 0:
        log(f"[bench] router projection leg ({args.router_copies} weight copies)")
        out["router"] = router_leg(args, cfg, wls[0], dev)
    if args.layers > 0:
        log(f"[bench] chained layers leg ({min(args.layers, NB)} layers)")
        out["layers"] = layers_leg(args, cfg, xs[0], banks, pks, bias, dev, expert_bytes)
    if args.layers > 0 and args.shared:
        log("[bench] shared-expert leg")
        out["shared"] = shared_leg(args, cfg, xs[0], banks, pks, bias, dev, expert_bytes)
    if args.copy_mb > 0:
        nbytes = args.copy_mb << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copies: 3 x {nbytes} bytes device to device")
        del src, dst
    if args.cpu_seconds > 0:
        log(f"[bench] cpu baseline ({args.cpu_seconds:.0f} s budget)")
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds, expert_bytes)
    if args.configs:
        del banks, pks, full, tail, g_dom, gu_steps, step
        torch.cuda.empty_cache()
        out["configs"] = configs_leg(args, dev, NB)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
