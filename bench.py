"""Benchmark of the Engram gate on one MI355X.

One step = one pass of the whole path over one batch of tokens:
tk_engram_gate_fwd, then tk_engram_gate_bwd, then tk_engram_grad_w_reduce,
all on the same stream, inputs already resident in HBM.

Prints one JSON line: fwd+bwd tokens/s on the main workload, the roofline of
the dominant kernel (HBM-bound; algorithmic bytes / average launch time from
HIP events on the launch stream against 8 TB/s), the same figures for the
other tuned width and the stress workload, the 1024-token forward hot and
after a cache scrub, a 128-bit tiled copy and the read/write-mix probes as
practical HBM ceilings, the N-gram hash and the table gather (uniform and
Zipf(1) token ids), the autograd module's step, the fused weight, a short
step eager and replayed from a HIP graph, and the fp64 oracle's throughput
on the host as a reported CPU baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4]

With --widths it instead times the forward and backward kernels at every
planned width (one JSON line per width).

With --traffic-from FETCH_CSV WRITE_CSV it runs no GPU work: it reads the
counter_collection.csv files of two rocprofv3 --pmc runs of this script
(FETCH_SIZE, then WRITE_SIZE), scales each counter by what it reads for the
copy probe of known size in the same run, and writes the measured HBM bytes
per launch of every kernel to profiles/traffic_<workload>.json.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBPS = 8000.0          # MI355X published HBM3E bandwidth
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SRC = os.path.join(ROOT, "engram_conditional_memory_amd", "csrc", "engram_gate.hip")
HASH_SRC = os.path.join(ROOT, "engram_conditional_memory_amd", "csrc", "engram_hash.hip")
# VALU issue: MI355X has 256 CUs of 4 SIMDs at 2.4 GHz; a SIMD issues one
# VALU instruction of a 64-wide wave every 4 cycles (16 lanes per cycle)
VALU_WAVE_INSTS_PER_S = 256 * 4 * 2.4e9 / 4
HASH_WORKLOAD = "hash_b1024s4096"
# GPU time of untimed warm-up before a timed line that follows host-side work
WARM_MS = 50.0
GATHER_SRC = os.path.join(ROOT, "engram_conditional_memory_amd", "csrc", "engram_gather.hip")
MEMORY_READ_TRAFFIC = "traffic_memory_read.json"


def kernel_source_hash(path: str = KERNEL_SRC) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def algorithmic_bytes(T: int, H: int) -> dict:
    """Bytes the method itself must move per launch (bf16 tensors, fp32 [H]
    weights and the fp32 gate); partial sums are implementation overhead."""
    return {
        "fwd": 8 * T * H + 4 * T + 8 * H,        # read x, k, v; write out, gate
        "bwd": 14 * T * H + 8 * H,               # read g, x, k, v; write dx, dk, dv
    }


def to_dev(bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


class Workload:
    def __init__(self, cfg: int, dev, eg):
        import synth
        import torch
        c = synth.CONFIGS[cfg]
        self.cfg, self.c, self.T, self.H = cfg, c, c.T, c.H
        d = synth.make_inputs(cfg)
        self.host = d
        self.x, self.k, self.v = to_dev(d["x"], dev), to_dev(d["k"], dev), to_dev(d["v"], dev)
        self.g = to_dev(d["grad_out"], dev)
        self.wh = torch.from_numpy(d["wh"]).to(dev)
        self.we = torch.from_numpy(d["we"]).to(dev)
        T, H = self.T, self.H
        bf = torch.bfloat16
        self.out = torch.empty((T, H), dtype=bf, device=dev)
        self.gate = torch.empty((T,), dtype=torch.float32, device=dev)
        self.dx = torch.empty((T, H), dtype=bf, device=dev)
        self.dk = torch.empty((T, H), dtype=bf, device=dev)
        self.dv = torch.empty((T, H), dtype=bf, device=dev)
        self.P = eg.tk_engram_num_partials(T, H)
        self.ws = torch.empty((max(1, self.P), H), dtype=torch.float32, device=dev)
        self.dwh = torch.empty((H,), dtype=torch.float32, device=dev)
        self.dwe = torch.empty((H,), dtype=torch.float32, device=dev)
        # the three C-ABI calls of one step, arguments marshalled once
        self.fwd = eg.bind_gate_fwd(self.x, self.k, self.v, self.wh, self.we, self.out,
                                    self.gate)
        self.bwd = eg.bind_gate_bwd(self.g, self.x, self.k, self.v, self.wh, self.we,
                                    self.dx, self.dk, self.dv, self.ws)
        self.red = eg.bind_grad_w_reduce(self.ws, self.P, self.H, self.wh, self.we,
                                         self.dwh, self.dwe)

    def step(self):
        self.fwd()
        self.bwd()
        self.red()

    def free(self):
        for n in ("x", "k", "v", "g", "out", "gate", "dx", "dk", "dv", "ws", "dwh", "dwe",
                  "fwd", "bwd", "red"):
            setattr(self, n, None)


def avg_launch_us(fn, reps: int, min_warmup_ms: float = 0.0) -> float:
    """Average duration of one call of `fn`, from HIP events on the launch
    stream around `reps` back-to-back calls (the queue stays ahead of the
    host, so the figure is the kernels' own time). One untimed call comes
    first; with min_warmup_ms, untimed calls continue until that much GPU
    time has passed, for calls that follow host-side work during which the
    GPU idled (its first ~10 ms of work afterwards run slow)."""
    import torch
    fn()
    torch.cuda.synchronize()
    if min_warmup_ms > 0:
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        n = 1
        while True:
            for _ in range(n):
                fn()
            b.record()
            torch.cuda.synchronize()
            if a.elapsed_time(b) >= min_warmup_ms:
                break
            n *= 2
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return 1e3 * a.elapsed_time(b) / reps


def time_workload(w: Workload, steps: int, warmup: int, min_warmup_ms: float = 0.0) -> dict:
    """`warmup` untimed steps, then `steps` timed ones. With min_warmup_ms,
    warm-up continues until that much GPU time has passed: after the GPU has
    idled (while the host generates a workload) its first ~10 ms of work run
    up to 25% slow, which is tens of steps at the shorter workloads."""
    import torch
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    done, elapsed = 0, 0.0
    while done < warmup or elapsed < min_warmup_ms:
        batch = warmup - done if done < warmup else max(warmup, 1)
        for _ in range(batch):
            w.step()
        done += batch
        b.record()
        torch.cuda.synchronize()
        elapsed = a.elapsed_time(b)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        w.step()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(stop) / steps
    # per-kernel averages: each call alone, back to back, same stream
    f_us = avg_launch_us(w.fwd, steps)
    b_us = avg_launch_us(w.bwd, steps)
    r_us = avg_launch_us(w.red, steps)
    T, H = w.T, w.H
    ab = algorithmic_bytes(T, H)
    return {
        "workload": w.c.name, "T": T, "H": H, "P": w.P,
        "warmup_steps": done, "ms_per_step": ms_step, "wall_s": wall,
        "tokens_per_s": T / (ms_step / 1e3),
        "fwd": {"us": f_us, "tokens_per_s": T / (f_us / 1e6), "bytes": ab["fwd"],
                "GBps": ab["fwd"] / (f_us * 1e3), "frac": ab["fwd"] / (f_us * 1e3) / HBM_PEAK_GBPS},
        "bwd_kernel": {"us": b_us, "bytes": ab["bwd"], "GBps": ab["bwd"] / (b_us * 1e3),
                       "frac": ab["bwd"] / (b_us * 1e3) / HBM_PEAK_GBPS},
        "reduce_us": r_us,
        "bwd": {"us": b_us + r_us, "tokens_per_s": T / ((b_us + r_us) / 1e6),
                "GBps": ab["bwd"] / ((b_us + r_us) * 1e3),
                "frac": ab["bwd"] / ((b_us + r_us) * 1e3) / HBM_PEAK_GBPS},
    }


def time_autograd(w: Workload, eg, steps: int, warmup: int, raw_ms: float,
                  min_warmup_ms: float = 50.0) -> dict:
    """The autograd wrapper (EngramGate) on a workload's tensors: forward, then
    backward with fresh .grad tensors each step (set to None first, as
    zero_grad(set_to_none=True) does); HIP events on torch's current stream.
    The outputs and gradients come from torch's caching allocator. Warm-up
    runs `warmup` steps and at least min_warmup_ms of GPU time, as the
    secondary workloads' does: the first ~10 ms of a phase run slow."""
    import torch
    layer = eg.EngramGate(w.H, device=w.x.device)
    with torch.no_grad():
        layer.wh.copy_(w.wh)
        layer.we.copy_(w.we)
    x, k, v = (t.detach().requires_grad_() for t in (w.x, w.k, w.v))
    leaves = (x, k, v, layer.wh, layer.we)

    def step():
        for t in leaves:
            t.grad = None
        layer(x, k, v).backward(w.g)

    # the first step allocates the outputs; the warm-up clock starts after it
    step()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    done, elapsed = 1, 0.0
    while done < warmup or elapsed < min_warmup_ms:
        step()
        done += 1
        if done >= warmup:
            b.record()
            torch.cuda.synchronize()
            elapsed = a.elapsed_time(b)
    a.record()
    for _ in range(steps):
        step()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    for t in leaves:
        t.grad = None
    del layer, x, k, v, leaves
    return {"workload": w.c.name, "warmup_steps": done, "steps": steps, "ms_per_step": ms,
            "tokens_per_s": w.T / (ms / 1e3), "vs_c_abi_step": raw_ms / ms}


def time_fused_weight(eg, dev, H: int, reps: int = 50) -> dict:
    """tk_engram_fused_weight at width H: 8 bytes read and 8 written per
    element; at these widths one launch is a few microseconds of latency."""
    import torch
    g = torch.Generator().manual_seed(0)
    wh = (1 + 0.1 * torch.randn(H, generator=g)).to(dev)
    we = (1 + 0.1 * torch.randn(H, generator=g)).to(dev)
    w = torch.empty((H,), dtype=torch.float64, device=dev)
    us = avg_launch_us(eg.bind_fused_weight(wh, we, w), reps)
    gbps = 16 * H / (us * 1e3)
    return {"H": H, "us": us, "bytes": 16 * H,
            "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": gbps / HBM_PEAK_GBPS, "traffic": None,
                         "note": f"one launch moves {16 * H} bytes; its time is launch latency"}}


WIDTHS = (2048, 3072, 4096, 5120, 6144, 7168, 8192)


def time_widths(eg, dev, reps: int = 30) -> list:
    """Forward and backward kernels at every width with a launch plan of its
    own, and at 6144 and 8192 (generic plans), each on about 470 MB per bf16
    tensor (T = 235 Mi / H), past the 256 MB Infinity Cache. Inputs are
    seeded normals; HIP events over back-to-back bound calls."""
    import torch
    res = []
    for H in WIDTHS:
        T = (235 * 1024 * 1024) // H
        print(f"[bench] width H={H} T={T}", file=sys.stderr, flush=True)
        g = torch.Generator(device=dev).manual_seed(H)

        def mk():
            return torch.randn((T, H), device=dev, generator=g).to(torch.bfloat16)

        x, k, v, go = mk(), mk(), mk(), mk()
        wh = 1 + 0.1 * torch.randn(H, device=dev, generator=g)
        we = 1 + 0.1 * torch.randn(H, device=dev, generator=g)
        out, gate = torch.empty_like(x), torch.empty(T, device=dev)
        dx, dk, dv = torch.empty_like(x), torch.empty_like(x), torch.empty_like(x)
        P = eg.tk_engram_num_partials(T, H)
        ws = torch.empty((P, H), device=dev)
        f_us = avg_launch_us(eg.bind_gate_fwd(x, k, v, wh, we, out, gate), reps)
        b_us = avg_launch_us(eg.bind_gate_bwd(go, x, k, v, wh, we, dx, dk, dv, ws), reps)
        ab = algorithmic_bytes(T, H)
        res.append({"H": H, "T": T, "P": P,
                    "fwd_us": f_us, "fwd_frac": ab["fwd"] / (f_us * 1e3) / HBM_PEAK_GBPS,
                    "bwd_us": b_us, "bwd_frac": ab["bwd"] / (b_us * 1e3) / HBM_PEAK_GBPS})
        del x, k, v, go, out, gate, dx, dk, dv, ws
        torch.cuda.empty_cache()
    return res


PLACEMENT_GAPS = (0, 16, 256, 4096, 65536, 1 << 21)
FOOTPRINT_TOKENS = (8192, 16384, 32768, 49152, 65536, 65537, 131072)


def _best_us(fn, reps: int, tries: int = 3) -> float:
    return min(avg_launch_us(fn, reps) for _ in range(tries))


def placement_layouts(S: int) -> list:
    """Placements of the backward's seven [T, H] streams (grad_out, x, k, v,
    dx, dk, dv; S bytes each): a label and, per stream, (buffer, byte offset),
    each buffer one allocation."""
    four = 4096
    lay = [("separate allocations", [(i, 0) for i in range(7)])]
    for gap in PLACEMENT_GAPS:
        lay.append((f"one buffer, gap {gap} B", [(0, i * (S + gap)) for i in range(7)]))
    lay.append(("inputs separate, outputs one buffer gap 4096 B",
                [(i, 0) for i in range(4)] + [(4, i * (S + four)) for i in range(3)]))
    lay.append(("inputs one buffer gap 4096 B, outputs separate",
                [(0, i * (S + four)) for i in range(4)] + [(i, 0) for i in range(1, 4)]))
    lay.append(("one buffer, inputs gap 0, outputs gap 0, outputs shifted 4096 B",
                [(0, i * S + (four if i >= 4 else 0)) for i in range(7)]))
    return lay


def time_placement(eg, dev, T: int = 32768, H: int = 7168, reps: int = 20,
                   rounds: int = 2) -> list:
    """Where a kernel's streams lie in HBM, against its time. The seven
    [T, H] bf16 tensors of the backward (grad_out, x, k, v in; dx, dk, dv
    out) are placed as placement_layouts lists: in separate allocations (2 MiB
    aligned, the caching allocator's default), or as views into shared
    buffers at staggered offsets. Each placement times the backward and the
    forward (x, k, v in, out) kernels, and the stream probe with the same
    mixes (4 reads + 3 writes, 3 + 1) on the same views. Inputs are seeded
    normals. The sweep runs `rounds` times, the second in reverse order; one
    record per placement and round; every figure is the best of three
    averages over `reps` back-to-back launches."""
    import torch
    S = 2 * T * H
    bf = torch.bfloat16
    g = torch.Generator(device=dev).manual_seed(7)
    wh = 1 + 0.1 * torch.randn(H, device=dev, generator=g)
    we = 1 + 0.1 * torch.randn(H, device=dev, generator=g)
    gate = torch.empty((T,), device=dev)
    P = eg.tk_engram_num_partials(T, H)
    ws = torch.empty((P, H), device=dev)
    ab = algorithmic_bytes(T, H)

    def measure(views, label, rnd):
        go, x, k, v, dx, dk, dv = views
        for t in (go, x, k, v):
            t.normal_(generator=g)
        fwd = eg.bind_gate_fwd(x, k, v, wh, we, dx, gate)
        bwd = eg.bind_gate_bwd(go, x, k, v, wh, we, dx, dk, dv, ws)
        as_i32 = [t.view(-1).view(torch.int32) for t in views]
        p43 = (lambda: eg.tk_engram_stream_probe(as_i32[:4], as_i32[4:]))
        p31 = (lambda: eg.tk_engram_stream_probe(as_i32[1:4], as_i32[4:5]))
        b_us, f_us = _best_us(bwd, reps), _best_us(fwd, reps)
        p43_us, p31_us = _best_us(p43, reps), _best_us(p31, reps)
        rec = {"placement": label, "round": rnd, "T": T, "H": H,
               "bwd_us": b_us, "bwd_frac": ab["bwd"] / (b_us * 1e3) / HBM_PEAK_GBPS,
               "fwd_us": f_us, "fwd_frac": ab["fwd"] / (f_us * 1e3) / HBM_PEAK_GBPS,
               "probe_4r3w_frac": 7 * S / (p43_us * 1e3) / HBM_PEAK_GBPS,
               "probe_3r1w_frac": 4 * S / (p31_us * 1e3) / HBM_PEAK_GBPS}
        print(f"[bench] placement {label} (round {rnd}): bwd {rec['bwd_frac']:.3f} "
              f"fwd {rec['fwd_frac']:.3f} probe 4r3w {rec['probe_4r3w_frac']:.3f} "
              f"3r1w {rec['probe_3r1w_frac']:.3f}", file=sys.stderr, flush=True)
        return rec

    # the GPU's first ~10 ms after idling run slow
    warm = torch.empty(2 * T * H, dtype=bf, device=dev)
    t_end = time.perf_counter() + 0.2
    while time.perf_counter() < t_end:
        eg.tk_engram_copy_probe(warm[: T * H], warm[T * H:])
        torch.cuda.synchronize()
    del warm
    res = []
    layouts = placement_layouts(S)
    for rnd in range(rounds):
        for label, spec in (layouts if rnd % 2 == 0 else layouts[::-1]):
            size = {}
            for b, off in spec:
                size[b] = max(size.get(b, 0), off + S)
            bufs = {b: torch.empty(n // 2, dtype=bf, device=dev) for b, n in size.items()}
            views = [bufs[b][off // 2:(off + S) // 2].view(T, H) for b, off in spec]
            res.append(measure(views, label, rnd))
            del views, bufs
            torch.cuda.empty_cache()
    return res


FOOTPRINT_SPLITS = (8192, 16384, 32768)


def time_footprint(eg, dev, H: int = 7168, reps: int = 10) -> list:
    """The backward kernel and its 4-read, 3-write probe against the token
    count (the footprint of the seven tensors), on seeded normals in separate
    allocations, at H = 7168; and the same rows as back-to-back launches of
    at most `split` rows each (views of the same tensors, each launch with a
    workspace of its own), for each split of FOOTPRINT_SPLITS below T."""
    import torch
    res = []
    g = torch.Generator(device=dev).manual_seed(11)
    wh = 1 + 0.1 * torch.randn(H, device=dev, generator=g)
    we = 1 + 0.1 * torch.randn(H, device=dev, generator=g)
    for T in FOOTPRINT_TOKENS:
        ts = [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in range(7)]
        for t in ts[:4]:
            t.normal_(generator=g)
        P = eg.tk_engram_num_partials(T, H)
        ws = torch.empty((P, H), device=dev)
        bwd = eg.bind_gate_bwd(*ts[:4], wh, we, *ts[4:], ws)
        as_i32 = [t.view(-1).view(torch.int32) for t in ts]
        t_end = time.perf_counter() + 0.1
        while time.perf_counter() < t_end:
            bwd()
            torch.cuda.synchronize()
        b_us = _best_us(bwd, reps)
        p_us = _best_us(lambda: eg.tk_engram_stream_probe(as_i32[:4], as_i32[4:]), reps)
        ab = algorithmic_bytes(T, H)["bwd"]
        rec = {"T": T, "H": H, "footprint_GB": 14 * T * H / 1e9, "bwd_us": b_us,
               "bwd_frac": ab / (b_us * 1e3) / HBM_PEAK_GBPS,
               "probe_4r3w_frac": 14 * T * H / (p_us * 1e3) / HBM_PEAK_GBPS, "split": {}}
        for split in FOOTPRINT_SPLITS:
            if split >= T:
                continue
            calls = []
            for a in range(0, T, split):
                n = min(split, T - a)
                wsn = torch.empty((eg.tk_engram_num_partials(n, H), H), device=dev)
                calls.append(eg.bind_gate_bwd(*[t[a:a + n] for t in ts[:4]], wh, we,
                                              *[t[a:a + n] for t in ts[4:]], wsn))

            def run_all():
                for c in calls:
                    c()

            s_us = _best_us(run_all, reps)
            rec["split"][str(split)] = {"launches": len(calls), "us": s_us,
                                        "frac": ab / (s_us * 1e3) / HBM_PEAK_GBPS}
            del calls
        print(f"[bench] footprint T={T}: bwd {rec['bwd_frac']:.3f} probe "
              f"{rec['probe_4r3w_frac']:.3f} split "
              + " ".join(f"{k}:{v['frac']:.3f}" for k, v in rec["split"].items()),
              file=sys.stderr, flush=True)
        res.append(rec)
        del ts, ws, bwd, as_i32
        torch.cuda.empty_cache()
    return res


FOOTPRINT_COUNTER_TOKENS = (32768, 65536, 131072)
FOOTPRINT_COUNTER_LAUNCHES = 3


def footprint_counter_run(eg, dev, H: int = 7168) -> dict:
    """A fixed sequence of launches for rocprofv3 --pmc runs: one copy probe
    of 2 x 32768 x H bf16 (the byte counters' calibration), then for each
    token count of FOOTPRINT_COUNTER_TOKENS, FOOTPRINT_COUNTER_LAUNCHES
    backward kernels followed by as many 4-read, 3-write stream probes on the
    same seven tensors. footprint_from_counters attributes the dispatches by
    this order."""
    import torch
    g = torch.Generator(device=dev).manual_seed(11)
    wh = 1 + 0.1 * torch.randn(H, device=dev, generator=g)
    we = 1 + 0.1 * torch.randn(H, device=dev, generator=g)
    src = torch.empty(32768 * H, dtype=torch.bfloat16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    eg.tk_engram_copy_probe(src, dst)
    torch.cuda.synchronize()
    del src, dst
    out = {"H": H, "tokens": list(FOOTPRINT_COUNTER_TOKENS), "launches": FOOTPRINT_COUNTER_LAUNCHES}
    for T in FOOTPRINT_COUNTER_TOKENS:
        ts = [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in range(7)]
        for t in ts[:4]:
            t.normal_(generator=g)
        ws = torch.empty((eg.tk_engram_num_partials(T, H), H), device=dev)
        bwd = eg.bind_gate_bwd(*ts[:4], wh, we, *ts[4:], ws)
        as_i32 = [t.view(-1).view(torch.int32) for t in ts]
        for _ in range(FOOTPRINT_COUNTER_LAUNCHES):
            bwd()
        for _ in range(FOOTPRINT_COUNTER_LAUNCHES):
            eg.tk_engram_stream_probe(as_i32[:4], as_i32[4:])
        torch.cuda.synchronize()
        print(f"[bench] footprint counters T={T} done", file=sys.stderr, flush=True)
        del ts, ws, bwd, as_i32
        torch.cuda.empty_cache()
    return out


def footprint_from_counters(csvs: list, H: int = 7168, name: str = "") -> dict:
    """Per token count, the mean per call of every counter in the given
    rocprofv3 --pmc runs of --footprint-counters (summed over a backward
    call's epoch launches), for the backward kernel and the stream probe;
    FETCH_SIZE and WRITE_SIZE also as bytes (scaled by their reading for the
    copy probe) over the algorithmic bytes. Written to
    profiles/footprint_counters_h<H><name>.json."""
    import csv
    n = FOOTPRINT_COUNTER_LAUNCHES
    per_call = [gate_launches(T, H)["gate_bwd_kernel"] for T in FOOTPRINT_COUNTER_TOKENS]
    rec = {"H": H, "tokens": list(FOOTPRINT_COUNTER_TOKENS), "calls_each": n, "runs": [],
           "bwd_launches_per_call": per_call, "kernel_source_sha256_16": kernel_source_hash()}
    table = {}
    for path in csvs:
        names = sorted({r["Counter_Name"] for r in csv.DictReader(open(path))})
        rec["runs"].append({"file": os.path.basename(os.path.dirname(path)) or path,
                            "counters": names})
        for counter in names:
            rows = _per_dispatch(path, counter)
            cp = [v for _, k, _, v in rows if k == "copy_probe_kernel"]
            bw = [v for _, k, _, v in rows if k == "gate_bwd_kernel"]
            pr = [v for _, k, _, v in rows if k == "stream_probe_kernel"]
            if (len(bw) != n * sum(per_call) or len(pr) != n * len(FOOTPRINT_COUNTER_TOKENS)
                    or len(cp) != 1):
                raise SystemExit(f"{path}: unexpected dispatch counts {len(cp)}, {len(bw)}, "
                                 f"{len(pr)} for {counter}")
            scale = None
            if counter in ("FETCH_SIZE", "WRITE_SIZE"):
                scale = 2 * 32768 * H / (1024.0 * cp[0])
                rec[f"{counter.lower()}_scale"] = scale
            starts = np.concatenate([[0], np.cumsum([n * L for L in per_call])])
            for i, T in enumerate(FOOTPRINT_COUNTER_TOKENS):
                # per call: the backward's epoch launches summed, one probe launch
                for kern, vals in (("gate_bwd_kernel", bw[starts[i]:starts[i + 1]]),
                                   ("stream_probe_kernel", pr[i * n:(i + 1) * n])):
                    m = float(np.sum(vals)) / n
                    d = table.setdefault(str(T), {}).setdefault(kern, {})
                    d[counter] = m
                    if scale is not None:
                        d[counter.lower() + "_bytes"] = m * 1024.0 * scale
    for T, kk in table.items():
        for kern, d in kk.items():
            if "fetch_size_bytes" in d and "write_size_bytes" in d:
                algo = 14 * int(T) * H
                d["measured_over_algorithmic"] = (d["fetch_size_bytes"] + d["write_size_bytes"]) / algo
            if "TCP_UTCL1_TRANSLATION_MISS_sum" in d and "TCP_UTCL1_REQUEST_sum" in d:
                d["utcl1_miss_per_request"] = (d["TCP_UTCL1_TRANSLATION_MISS_sum"]
                                               / max(1.0, d["TCP_UTCL1_REQUEST_sum"]))
                d["utcl1_miss_per_MiB"] = (d["TCP_UTCL1_TRANSLATION_MISS_sum"]
                                           / (14 * int(T) * H / 2 ** 20))
    rec["per_tokens"] = table
    path = os.path.join(PROFILES, f"footprint_counters_h{H}{name}.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    return rec


def _kernel_label(name: str) -> str:
    """`gate_bwd_kernel<7, 2, true, 3, true, false>` from a demangled name."""
    name = name.replace("(anonymous namespace)::", "")
    if name.startswith("void "):
        name = name[len("void "):]
    return name.split("(")[0].strip()


TRACE_DOC = """bench.py defaults: 50 timed steps after 20 warm-up steps, then each call alone
50 times back to back (plus one untimed call), on T=32768 H=7168; then 20
steps of the autograd module on the same tensors after at least 20 steps and
50 ms of warm-up (it runs the fused-weight forms of the gate kernels, the
last template argument `true`); the same calls on T=16384 H=4096 after at
least 50 ms of warm-up steps; 20 steps and 20 single calls on the stress
workload (T=65537, H=7168) after at least 50 ms of warm-up; the 1024-token
forward 51 times hot and 50 times after a 1 GiB write; the copy probe; the
stream probe for the 3-in/1-out and 4-in/3-out mixes; PyTorch's bf16 copy
and addcmul on the same bytes; the N-gram hash; the table gather on uniform,
then Zipf(1) token ids; the fused weight at H=7168; a 1024-token step at
H=4096 eagerly, on the capture stream and replayed from a HIP graph."""


def trace_summary(trace_csv: str, stats_csv: str, cmd: str) -> str:
    """Markdown summary of a rocprofv3 kernel trace of the default bench run:
    rocprofv3's per-dispatch statistics of the library's kernels, then the
    gate kernels per call on each H = 7168 workload (a call on a long batch
    is several epoch launches, summed here; `span` also counts the gaps
    between them, as HIP events around the call do)."""
    import csv
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))
    out = ["# Engram kernels, bench.py default run: rocprofv3 kernel trace", "",
           "Command (from the repository root, on one MI355X):", "", "    " + cmd, "",
           f"Summarised by `python3 bench.py --trace-from {os.path.basename(trace_csv)} "
           f"{os.path.basename(stats_csv)}` (paths of the run's output directory).", "",
           TRACE_DOC, "",
           f"Kernel source sha256 prefixes: gate {kernel_source_hash()}, "
           f"hash {kernel_source_hash(HASH_SRC)}, gather {kernel_source_hash(GATHER_SRC)}.", "",
           "Per dispatch, from the stats file (durations in microseconds):", "",
           "| kernel | dispatches | average | min | max | % of GPU time |",
           "|---|---|---|---|---|---|"]
    for r in csv.DictReader(open(stats_csv)):
        lab = _kernel_label(r["Name"])
        if not lab.split("<")[0].endswith(("_kernel", "_kernel_vec", "_kernel_any")):
            continue
        if lab.startswith(("at::", "void at::")):
            continue
        out.append(f"| `{lab}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{float(r['Percentage']):.2f} |")
    # the H = 7168 gate kernels in time order: the main workload's unfused
    # kernels come before the autograd module's fused ones, the stress
    # workload's after them
    fused = [int(r["Start_Timestamp"]) for r in rows
             if _kernel_label(r["Kernel_Name"]).startswith("gate_")
             and _kernel_label(r["Kernel_Name"]).endswith(", true>")
             and "<7, 2" in r["Kernel_Name"]]
    t_fused = min(fused) if fused else None
    out += ["", "Per call of the gate kernels at H = 7168 (microseconds; `kernel` sums a "
            "call's epoch launches, `span` runs from the first launch's start to the last "
            "one's end):", "",
            "| workload | kernel | launches per call | calls | kernel average | span average |",
            "|---|---|---|---|---|---|"]
    for wl, T, when in (("T=32768, H=7168 (main)", 32768, "before"),
                        ("T=32768, H=7168 (autograd module)", 32768, "fused"),
                        ("T=65537, H=7168 (stress)", 65537, "after")):
        L = gate_launches(T, 7168)
        for kern in ("gate_fwd_kernel", "gate_bwd_kernel"):
            sel = []
            for r in rows:
                lab = _kernel_label(r["Kernel_Name"])
                if not lab.startswith(kern + "<7, 2"):
                    continue
                st = int(r["Start_Timestamp"])
                is_fused = lab.endswith(", true>")
                if when == "fused" and not is_fused:
                    continue
                if when != "fused" and (is_fused or t_fused is None
                                        or (st > t_fused) != (when == "after")):
                    continue
                sel.append((st, int(r["End_Timestamp"]), lab))
            n = L[kern]
            if not sel or len(sel) % n:
                out.append(f"| {wl} | `{kern}` | {n} | (dispatch count {len(sel)} "
                           "not a multiple) | | |")
                continue
            calls = [sel[i:i + n] for i in range(0, len(sel), n)]
            k_us = np.mean([sum(e - b for b, e, _ in c) for c in calls]) / 1e3
            s_us = np.mean([c[-1][1] - c[0][0] for c in calls]) / 1e3
            out.append(f"| {wl} | `{sel[0][2]}` | {n} | {len(calls)} | {k_us:.2f} | "
                       f"{s_us:.2f} |")
    return "\n".join(out) + "\n"


def widths_trace_summary(trace_csv: str, widths_jsonl: str, cmd: str) -> str:
    """Markdown summary of a rocprofv3 kernel trace of `bench.py --widths`:
    per width, the forward's and the backward's average per call (the sum of
    a call's epoch launches), its fraction of 8 TB/s, and the HIP-event
    figure the same run printed. Each width's plan is its own kernel
    instantiation, in WIDTHS order."""
    import csv
    widths = [json.loads(line) for line in open(widths_jsonl) if line.startswith("{")]
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))
    per = {}
    for r in rows:
        lab = _kernel_label(r["Kernel_Name"])
        if lab.startswith(("gate_fwd_kernel", "gate_bwd_kernel")):
            per.setdefault(lab, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    fwd_labels = [k for k in per if k.startswith("gate_fwd")]
    bwd_labels = [k for k in per if k.startswith("gate_bwd")]
    out = ["# Gate kernels at every planned width: rocprofv3 kernel trace", "",
           "Command (from the repository root, on one MI355X):", "", "    " + cmd, "",
           f"Summarised by `python3 bench.py --widths-trace-from {os.path.basename(trace_csv)} "
           "<the run's stdout>` (paths of the run's output).", "",
           "`bench.py --widths` runs the forward and then the backward 31 times each (one "
           "untimed call, then 30 back to back) at each width, on about 470 MB per bf16 "
           "tensor (T = 235 Mi / H), past the 256 MB Infinity Cache. A call is one or more "
           "launches (epochs of about 240 MB per tensor); the averages are per call. "
           "Fractions are algorithmic bytes (forward 8·T·H + 4·T + 8·H, backward "
           "14·T·H + 8·H) over the trace's average per call, against 8 TB/s.", "",
           f"Kernel source sha256 prefix: {kernel_source_hash()}.", "",
           "| H | T | kernel | launches per call | calls | trace average per call (us) | "
           "fraction of 8 TB/s | events in the same run (us) |",
           "|---|---|---|---|---|---|---|---|"]
    for w in widths:
        T, H = w["T"], w["H"]
        L = gate_launches(T, H)
        ab = algorithmic_bytes(T, H)
        for key, labels, ev in (("gate_fwd_kernel", fwd_labels, w["fwd_us"]),
                                ("gate_bwd_kernel", bwd_labels, w["bwd_us"])):
            n = L[key]
            # the width's instantiation: the one whose dispatch count is 31 calls
            cand = [k for k in labels if len(per[k]) == 31 * n and not k.endswith(", true>")]
            lab = None
            for k in cand:
                avg = sum(per[k]) / (len(per[k]) / n) / 1e3
                if abs(avg - ev) / ev < 0.1:
                    lab = k
                    break
            if lab is None:
                out.append(f"| {H} | {T} | `{key}` | {n} | (not found) | | | {ev:.1f} |")
                continue
            labels.remove(lab)
            calls = len(per[lab]) // n
            avg = sum(per[lab]) / calls / 1e3
            b = ab["fwd" if key == "gate_fwd_kernel" else "bwd"]
            out.append(f"| {H} | {T} | `{lab}` | {n} | {calls} | {avg:.1f} | "
                       f"{b / (avg * 1e3) / HBM_PEAK_GBPS:.3f} | {ev:.1f} |")
    out += ["", "Template arguments are <waves per row, chunks per thread, full rows, rows in "
            "flight[, fp64 weights in LDS], fused weight>. H = 8192 runs the generic plan "
            "(8 waves x 2 chunks, compiled with the tail mask, which is never taken at this "
            "width)."]
    return "\n".join(out) + "\n"


def time_graph_step(eg, dev, T: int = 1024, H: int = 4096, reps: int = 50) -> dict:
    """One step (forward, backward, reduction) on a short batch, called eagerly
    through the Python binding and replayed from a captured HIP graph; the
    three calls allocate nothing and write no memset, so they capture as
    they are. HIP events over back-to-back steps on the launch stream."""
    import torch
    g = torch.Generator(device=dev).manual_seed(T + H)

    def mk():
        return torch.randn((T, H), device=dev, generator=g).to(torch.bfloat16)

    x, k, v, go = mk(), mk(), mk(), mk()
    wh = 1 + 0.1 * torch.randn(H, device=dev, generator=g)
    we = 1 + 0.1 * torch.randn(H, device=dev, generator=g)
    out, dx, dk, dv = (torch.empty_like(x) for _ in range(4))
    gate = torch.empty((T,), device=dev)
    P = eg.tk_engram_num_partials(T, H)
    ws = torch.empty((P, H), device=dev)
    dwh, dwe = torch.empty(H, device=dev), torch.empty(H, device=dev)

    def step():
        eg.tk_engram_gate_fwd(x, k, v, wh, we, out, gate)
        eg.tk_engram_gate_bwd(go, x, k, v, wh, we, dx, dk, dv, ws)
        eg.tk_engram_grad_w_reduce(ws, P, H, wh, we, dwh, dwe)

    eager = avg_launch_us(step, reps)
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    replay = avg_launch_us(graph.replay, reps)
    del graph, x, k, v, go, out, dx, dk, dv, ws
    torch.cuda.empty_cache()
    return {"T": T, "H": H, "eager_us": eager, "graph_us": replay,
            "eager_over_graph": eager / replay,
            "graph_tokens_per_s": T / (replay / 1e6)}


def time_hash(eg, dev, name: str = "b1024s4096", reps: int = 20) -> dict:
    """tk_engram_hash throughput on a large batch: average launch time from HIP
    events over back-to-back launches; algorithmic bytes = 4 per token read
    plus 4 per index written."""
    import synth
    import torch
    c = synth.HASH_CONFIGS[name]
    p = synth.hash_params(c)
    tokens = torch.from_numpy(synth.hash_tokens(c)).to(dev)
    out = torch.empty((c.B, c.S, len(c.ngram), c.tables), dtype=torch.int32, device=dev)

    def call():
        eg.tk_engram_hash(tokens, p["ngram"], p["mult"], p["table_size"], p["pad"], out)

    us = avg_launch_us(call, reps, min_warmup_ms=WARM_MS)
    n = c.B * c.S
    nbytes = n * (4 + 4 * len(c.ngram) * c.tables)
    del tokens, out
    torch.cuda.empty_cache()
    res = {"workload": c.name, "tokens": n, "us": us, "tokens_per_s": n / (us / 1e6),
           "bytes": nbytes, "GBps": nbytes / (us * 1e3),
           "frac": nbytes / (us * 1e3) / HBM_PEAK_GBPS}
    if name == HASH_WORKLOAD[len("hash_"):]:
        res["roofline"] = {"bound": "hbm", "achieved": res["GBps"], "peak": HBM_PEAK_GBPS,
                           "unit": "GB/s", "frac": res["frac"],
                           "traffic": memory_read_bytes("hash")}
        res["valu_issue_note"] = hash_valu_note(res["tokens_per_s"])
    return res


def time_gather(eg, dev, reps: int = 20) -> tuple:
    """tk_engram_gather on the H=7168 workload's memory read: 32768 tokens, 16
    tables (2 layers x 8) of 2^19 rows x 448 bf16, indices from
    tk_engram_hash, for uniform token ids and for Zipf(1) token frequencies.
    Algorithmic bytes per (token, table): 4 (index) + 2d (row read) + 2d (row
    written); with Zipf tokens some rows repeat and may be served from cache,
    so that line also states the fraction of distinct rows."""
    import synth
    import torch
    gc = synth.GATHER_CONFIGS["t32768_d448"]
    stride = 1 << 19
    data = torch.empty((gc.tables * stride, gc.d), dtype=torch.bfloat16, device=dev)
    for q in range(gc.tables):
        synth.fill_table_bits_torch(data, q, q * stride, stride, gc.d)
    off = np.arange(gc.tables, dtype=np.int64) * stride
    out = torch.empty((gc.T, gc.tables, gc.d), dtype=torch.bfloat16, device=dev)
    res = []
    for recipe in ("b8s4096", "b8s4096_zipf"):
        hc = synth.HASH_CONFIGS[recipe]
        p = synth.hash_params(hc)
        sizes = p["table_size"].reshape(-1)
        tokens = torch.from_numpy(synth.hash_tokens(hc)).to(dev)
        idx = eg.tk_engram_hash(tokens, p["ngram"], p["mult"], p["table_size"], p["pad"])
        idx2 = idx.view(gc.T, gc.tables)

        def call():
            eg.tk_engram_gather(idx2, data, off, sizes, out)

        us = avg_launch_us(call, reps, min_warmup_ms=WARM_MS)
        ih = idx2.cpu().numpy()
        distinct = sum(len(np.unique(ih[:, q])) for q in range(gc.tables))
        n = gc.T * gc.tables
        nbytes = n * (4 + 4 * gc.d)
        gbps = nbytes / (us * 1e3)
        res.append({"workload": gc.name + ("_zipf" if hc.zipf else ""), "tokens": gc.T,
                    "token_ids": "Zipf(1)" if hc.zipf else "uniform",
                    "rows_gathered": n, "distinct_rows_frac": distinct / n, "us": us,
                    "tokens_per_s": gc.T / (us / 1e6), "bytes": nbytes,
                    "GBps": gbps, "frac": gbps / HBM_PEAK_GBPS,
                    "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS,
                                 "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS,
                                 "traffic": memory_read_bytes(
                                     "gather_zipf" if hc.zipf else "gather")}})
        del tokens, idx, idx2
    del data, out
    torch.cuda.empty_cache()
    return res[0], res[1]


def copy_ceiling(nbytes: int, eg, dev, reps: int = 20) -> dict:
    import torch
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    us = avg_launch_us(lambda: eg.tk_engram_copy_probe(src, dst), reps,
                       min_warmup_ms=WARM_MS)
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_moved": 2 * nbytes, "us": us, "GBps": 2 * nbytes / (us * 1e3),
            "frac": 2 * nbytes / (us * 1e3) / HBM_PEAK_GBPS}


def mix_ceiling(nsrc: int, ndst: int, nbytes: int, eg, dev, reps: int = 20) -> dict:
    """Practical HBM ceiling of a read/write mix: the library's stream probe
    with nsrc input and ndst output streams of nbytes each, random data."""
    import torch
    n = nbytes // 4
    srcs = [torch.randint(-(1 << 31), (1 << 31) - 1, (n,), dtype=torch.int32, device=dev)
            for _ in range(nsrc)]
    dsts = [torch.empty_like(srcs[0]) for _ in range(ndst)]
    us = avg_launch_us(lambda: eg.tk_engram_stream_probe(srcs, dsts), reps,
                       min_warmup_ms=WARM_MS)
    moved = (nsrc + ndst) * nbytes
    del srcs, dsts
    torch.cuda.empty_cache()
    return {"reads": nsrc, "writes": ndst, "bytes_each": nbytes, "us": us,
            "GBps": moved / (us * 1e3), "frac": moved / (us * 1e3) / HBM_PEAK_GBPS}


def vendor_reference(nbytes: int, dev, reps: int = 20) -> dict:
    """PyTorch's own ROCm kernels on tensors of the same size, for reference
    beside the library's probes: a bf16 copy (one read, one write) and
    addcmul, out = x + k * v (three reads and one write, the forward's mix).
    Random data, as for the probes."""
    import torch
    n = nbytes // 2
    g = torch.Generator(device=dev).manual_seed(7)
    x, k, v = (torch.randn(n, device=dev, generator=g).to(torch.bfloat16) for _ in range(3))
    o = torch.empty_like(x)
    res = {}
    for name, fn, moved in (("torch_copy", lambda: o.copy_(x), 2 * nbytes),
                            ("torch_addcmul_3r1w", lambda: torch.addcmul(x, k, v, out=o),
                             4 * nbytes)):
        us = avg_launch_us(fn, reps, min_warmup_ms=WARM_MS)
        res[name] = {"us": us, "bytes": moved, "GBps": moved / (us * 1e3),
                     "frac": moved / (us * 1e3) / HBM_PEAK_GBPS}
    del x, k, v, o
    torch.cuda.empty_cache()
    return res


def time_fwd_small(eg, dev, reps: int = 50) -> dict:
    """The forward-only workload (batch 2 x seq 512 = 1024 tokens, H=4096,
    33.6 MB): it fits the 256 MB Infinity Cache, so it is timed two ways:
    hot (back-to-back launches) and flushed (a 1 GiB write between launches,
    each launch timed alone with its own events)."""
    import synth
    import torch
    c = synth.CONFIGS[2]
    d = synth.make_inputs(2, with_grad=False)
    x, k, v = to_dev(d["x"], dev), to_dev(d["k"], dev), to_dev(d["v"], dev)
    wh = torch.from_numpy(d["wh"]).to(dev)
    we = torch.from_numpy(d["we"]).to(dev)
    out = torch.empty_like(x)
    gate = torch.empty((c.T,), dtype=torch.float32, device=dev)
    fwd = eg.bind_gate_fwd(x, k, v, wh, we, out, gate)
    hot = avg_launch_us(fwd, reps, min_warmup_ms=WARM_MS)
    scrub = torch.empty(1 << 29, dtype=torch.int16, device=dev)
    times = []
    for i in range(reps):
        scrub.fill_(i)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fwd()
        b.record()
        torch.cuda.synchronize()
        times.append(1e3 * a.elapsed_time(b))
    flushed = float(np.median(times))
    nbytes = algorithmic_bytes(c.T, c.H)["fwd"]
    del x, k, v, out, gate, scrub, fwd
    torch.cuda.empty_cache()
    return {"workload": c.name, "T": c.T, "H": c.H, "bytes": nbytes,
            "hot_us": hot, "hot_GBps": nbytes / (hot * 1e3),
            "flushed_us": flushed, "flushed_GBps": nbytes / (flushed * 1e3),
            "flushed_frac": nbytes / (flushed * 1e3) / HBM_PEAK_GBPS}


def _oracle_rate(host: dict, threads: int, budget_s: float, backward: bool):
    """Tokens per second of the fp64 oracle over the workload's tokens in
    chunks of 4096, repeating passes until `budget_s` of wall time is spent:
    forward alone, or forward + backward (incl. dwh/dwe)."""
    import oracle
    T = host["x"].shape[0]
    chunk = 4096
    done = 0
    t0 = time.perf_counter()
    while True:
        a = done % T
        sl = slice(a, min(T, a + chunk))
        oracle.fwd_bf16(host["x"][sl], host["k"][sl], host["v"][sl], host["wh"],
                        host["we"], want_out=True, threads=threads)
        if backward:
            oracle.bwd_bf16(host["grad_out"][sl], host["x"][sl], host["k"][sl],
                            host["v"][sl], host["wh"], host["we"], threads=threads)
        done += sl.stop - sl.start
        if time.perf_counter() - t0 >= budget_s:
            break
    return done, time.perf_counter() - t0


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cpu_share() -> dict:
    """The host CPUs this process may use: the machine's count, the CPUs in
    its affinity mask, and the cgroup CPU quota (cgroup v2 cpu.max) if one is
    set. `threads` is the smaller of the last two: every CPU the process can
    actually run on."""
    total = os.cpu_count() or 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = total
    quota = None
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            q, period = f.read().split()[:2]
            if q != "max":
                quota = int(q) / int(period)
    except (OSError, ValueError):
        pass
    threads = affinity if quota is None else max(1, min(affinity, int(quota)))
    return {"host_cpus": total, "affinity_cpus": affinity, "cgroup_cpu_quota": quota,
            "threads": threads}


def cpu_baseline(host: dict, budget_s: float = 10.0, side_s: float = 3.0) -> dict:
    """The fp64 oracle, as it stands, on the host cores. `value` is forward +
    backward on every CPU this process may use (host_cpu_share); beside it,
    the same on one thread and the forward alone on every CPU, each over a
    shorter sample, with their algorithmic bytes per second."""
    share = host_cpu_share()
    th = share["threads"]
    T, H = host["x"].shape
    ab = {key: b / T for key, b in algorithmic_bytes(T, H).items()}   # per token
    done, dt = _oracle_rate(host, th, budget_s, True)
    done1, dt1 = _oracle_rate(host, 1, side_s, True)
    donef, dtf = _oracle_rate(host, th, side_s, False)
    rate, rate1, ratef = done / dt, done1 / dt1, donef / dtf
    return {"value": rate, "unit": "tokens/s", "cores": th, "kind": "oracle",
            "sample": f"{done} tokens ({done / T:.2f} passes over the {T}-token workload, "
                      f"chunks of 4096), fp64 forward + backward incl. dwh/dwe, "
                      f"{dt:.1f} s wall on {th} threads",
            "threads": th, "host_cpus": share["host_cpus"],
            "affinity_cpus": share["affinity_cpus"],
            "cgroup_cpu_quota": share["cgroup_cpu_quota"],
            "GBps_equiv": rate * (ab["fwd"] + ab["bwd"]) / 1e9,
            "single_thread": {"value": rate1, "sample": f"{done1} tokens, {dt1:.1f} s",
                              "GBps_equiv": rate1 * (ab["fwd"] + ab["bwd"]) / 1e9},
            "fwd_only": {"value": ratef, "cores": th, "sample": f"{donef} tokens, {dtf:.1f} s",
                         "GBps_equiv": ratef * ab["fwd"] / 1e9},
            "cpu_model": cpu_model()}


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_call")


def read_counter_csv(path: str, counter: str) -> dict:
    """Mean value per dispatch of `counter`, by kernel base name."""
    import csv
    per = {}
    for r in csv.DictReader(open(path)):
        if r.get("Counter_Name") != counter:
            continue
        name = r["Kernel_Name"].replace("(anonymous namespace)::", "")
        if name.startswith("void "):
            name = name[len("void "):]
        base = name.split("(")[0].split("<")[0].split("::")[-1].strip()
        per.setdefault(base, []).append(float(r["Counter_Value"]))
    return {k: float(np.mean(v)) for k, v in per.items()}


def gate_launches(T: int, H: int) -> dict:
    """Kernel launches per call of the forward and the backward at (T, H):
    both walk their rows in epochs (tk_engram_gate_launches)."""
    import engram_conditional_memory_amd as eg
    return {"gate_fwd_kernel": eg.tk_engram_gate_launches(T, H, False),
            "gate_bwd_kernel": eg.tk_engram_gate_launches(T, H, True)}


def traffic_from_counters(fetch_csv: str, write_csv: str, workload: int) -> dict:
    """HBM bytes per call of each kernel: the mean per dispatch times the
    kernel's launches per call (several for the gate kernels on long
    batches, one for the rest)."""
    import synth
    c = synth.CONFIGS[workload]
    fetch = read_counter_csv(fetch_csv, "FETCH_SIZE")
    write = read_counter_csv(write_csv, "WRITE_SIZE")
    per_call = gate_launches(c.T, c.H)
    for counts in (fetch, write):
        for k, n in per_call.items():
            if k in counts:
                counts[k] *= n
    copy_bytes = 2 * c.T * c.H              # the copy probe reads and writes this
    f_scale = copy_bytes / (1024.0 * fetch["copy_probe_kernel"])
    w_scale = copy_bytes / (1024.0 * write["copy_probe_kernel"])
    ab = algorithmic_bytes(c.T, c.H)
    algo = {"gate_fwd_kernel": ab["fwd"], "gate_bwd_kernel": ab["bwd"]}
    kernels = {}
    for k in sorted(set(fetch) & set(write)):
        rd = fetch[k] * 1024.0 * f_scale
        wr = write[k] * 1024.0 * w_scale
        kernels[k] = {"fetch_kib_per_call": fetch[k], "write_kib_per_call": write[k],
                      "read_bytes": rd, "write_bytes": wr, "bytes_per_call": rd + wr,
                      "algorithmic_bytes": algo.get(k),
                      "measured_over_algorithmic": (rd + wr) / algo[k] if k in algo else None}
    rec = {"workload": c.name, "T": c.T, "H": c.H, "launches_per_call": per_call,
           "kernel_source_sha256_16": kernel_source_hash(),
           "calibration": {"copy_bytes_each_way": copy_bytes,
                           "fetch_scale": f_scale, "write_scale": w_scale},
           "kernels": kernels}
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, f"traffic_{c.name}.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    return rec


def valu_from_counters(sq_csv: str) -> dict:
    """Executed instructions per wave of the N-gram hash on the hash_b1024s4096
    workload (the 4,194,304-thread dispatches) from one rocprofv3 --pmc run
    with SQ_WAVES, SQ_INSTS_VALU and SQ_INSTS_SALU; written beside the
    profiles with the hash source's sha256 prefix."""
    import csv
    import synth
    c = synth.HASH_CONFIGS[HASH_WORKLOAD[len("hash_"):]]
    threads = str(c.B * c.S)
    per = {}
    for r in csv.DictReader(open(sq_csv)):
        if "hash_kernel" not in r["Kernel_Name"] or r["Grid_Size"] != threads:
            continue
        d = per.setdefault(r["Dispatch_Id"], {})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no hash dispatch of {threads} threads in {sq_csv}")
    valu = float(np.mean([d["SQ_INSTS_VALU"] / d["SQ_WAVES"] for d in per.values()]))
    salu = float(np.mean([d["SQ_INSTS_SALU"] / d["SQ_WAVES"] for d in per.values()]))
    waves = float(np.mean([d["SQ_WAVES"] for d in per.values()]))
    rec = {"workload": HASH_WORKLOAD, "tokens": c.B * c.S, "dispatches": len(per),
           "waves": waves, "tokens_per_wave": c.B * c.S / waves,
           "valu_insts_per_wave": valu, "salu_insts_per_wave": salu,
           "hash_source_sha256_16": kernel_source_hash(HASH_SRC)}
    path = os.path.join(PROFILES, f"valu_{HASH_WORKLOAD}.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    return rec


def _per_dispatch(path: str, counter: str) -> list:
    """(dispatch id, kernel base name, grid size, value) of `counter`, in
    dispatch order."""
    import csv
    rows = []
    for r in csv.DictReader(open(path)):
        if r.get("Counter_Name") != counter:
            continue
        name = r["Kernel_Name"].replace("(anonymous namespace)::", "")
        if name.startswith("void "):
            name = name[len("void "):]
        base = name.split("(")[0].split("<")[0].split("::")[-1].strip()
        rows.append((int(r["Dispatch_Id"]), base, int(r["Grid_Size"]), float(r["Counter_Value"])))
    rows.sort()
    return rows


def memory_read_traffic(fetch_csv: str, write_csv: str) -> dict:
    """HBM bytes per launch of the hash (its 4,194,304-token launches) and of
    the gather (the launches after the hash of the uniform token ids, then
    those after the hash of the Zipf(1) ids; each group's warm-up and timed
    launches alike) from two rocprofv3 --pmc runs over --memory-read, each
    counter scaled by its reading for the copy probe of known size; written
    beside the profiles with the two kernel sources' sha256 prefixes."""
    import synth
    c4 = synth.CONFIGS[4]
    copy_bytes = 2 * c4.T * c4.H
    hc = synth.HASH_CONFIGS[HASH_WORKLOAD[len("hash_"):]]
    gc = synth.GATHER_CONFIGS["t32768_d448"]
    rec = {"calibration": {"copy_bytes_each_way": copy_bytes},
           "hash_source_sha256_16": kernel_source_hash(HASH_SRC),
           "gather_source_sha256_16": kernel_source_hash(GATHER_SRC)}
    per = {}
    for key, path, counter in (("read", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        rows = _per_dispatch(path, counter)
        cp = [v for _, k, _, v in rows if k == "copy_probe_kernel"]
        scale = copy_bytes / (1024.0 * float(np.mean(cp)))
        rec["calibration"][f"{counter.lower()}_scale"] = scale
        hash_v = [v for _, k, g, v in rows if k == "hash_kernel_vec" and g == hc.B * hc.S]
        # the gather's index hashes (32768 tokens each) split its launches
        groups = []
        for _, k, g, v in rows:
            if k == "hash_kernel_vec" and g == gc.T:
                groups.append([])
            elif k == "gather_kernel" and groups:
                groups[-1].append(v)
        if len(groups) != 2 or not all(groups) or not hash_v:
            raise SystemExit(f"{path}: expected the hash's launches and two groups of gather "
                             f"launches, found {len(hash_v)} and {[len(g) for g in groups]}")
        for name, vals in (("hash", hash_v), ("gather", groups[0]), ("gather_zipf", groups[1])):
            per.setdefault(name, {})[key] = float(np.mean(vals)) * 1024.0 * scale
    algo = {"hash": hc.B * hc.S * (4 + 4 * len(hc.ngram) * hc.tables),
            "gather": gc.T * gc.tables * (4 + 4 * gc.d)}
    algo["gather_zipf"] = algo["gather"]
    for name, d in per.items():
        total = d["read"] + d["write"]
        rec[name] = {"read_bytes": d["read"], "write_bytes": d["write"], "bytes_per_launch": total,
                     "algorithmic_bytes": algo[name], "measured_over_algorithmic": total / algo[name]}
    with open(os.path.join(PROFILES, MEMORY_READ_TRAFFIC), "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    return rec


def memory_read_bytes(name: str):
    """Counter bytes per launch of `name` ("hash", "gather", "gather_zipf") from
    the committed record, if it was taken on the current kernel source."""
    try:
        rec = json.load(open(os.path.join(PROFILES, MEMORY_READ_TRAFFIC)))
    except (OSError, ValueError):
        return None
    src = HASH_SRC if name == "hash" else GATHER_SRC
    key = "hash_source_sha256_16" if name == "hash" else "gather_source_sha256_16"
    if rec.get(key) != kernel_source_hash(src) or name not in rec:
        return None
    return rec[name]["bytes_per_launch"]


def hash_valu_note(tokens_per_s: float):
    """Not a roofline: tokens per second if every SIMD issued one VALU
    instruction every 4 cycles, at the hash's own executed instruction count
    from the committed counter record of the current hash source; None if
    that record is missing or stale."""
    path = os.path.join(PROFILES, f"valu_{HASH_WORKLOAD}.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("hash_source_sha256_16") != kernel_source_hash(HASH_SRC):
        return None
    issue = VALU_WAVE_INSTS_PER_S * rec["tokens_per_wave"] / rec["valu_insts_per_wave"]
    return {"tokens_per_s_at_valu_issue_rate": issue, "frac": tokens_per_s / issue,
            "basis": f"{rec['valu_insts_per_wave']:.0f} VALU instructions per wave of "
                     f"{rec['tokens_per_wave']:.0f} tokens as executed (rocprofv3 "
                     "SQ_INSTS_VALU / SQ_WAVES), one per SIMD every 4 cycles, 1024 SIMDs "
                     "at 2.4 GHz; the kernel's own count, so not a bound on the method"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=4, choices=[3, 4, 5],
                    help="main workload (3: T=16384 H=4096, 4: T=32768 H=7168, 5: stress)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the other workloads (second width, stress, small forward, "
                         "memory read)")
    ap.add_argument("--widths", action="store_true",
                    help="instead of the default run, time the forward and backward kernels "
                         "at H = " + ", ".join(map(str, WIDTHS)) + " (one JSON line each)")
    ap.add_argument("--memory-read", action="store_true",
                    help="instead of the default run, time only the copy probe (470 MB each "
                         "way, the counters' calibration), the N-gram hash and the table "
                         "gather on uniform and Zipf(1) token ids (one JSON line); for "
                         "rocprofv3 counter runs")
    ap.add_argument("--placement", action="store_true",
                    help="instead of the default run, time the gate kernels and the stream "
                         "probe with their tensors at staggered offsets in one buffer and in "
                         "separate allocations, then the backward against its footprint "
                         "(one JSON line per measurement)")
    ap.add_argument("--footprint-only", action="store_true",
                    help="with --placement, run only its footprint sweep")
    ap.add_argument("--footprint-counters", action="store_true",
                    help="instead of the default run, launch the backward and its stream "
                         "probe a fixed number of times at T = "
                         + ", ".join(map(str, FOOTPRINT_COUNTER_TOKENS))
                         + " (H = 7168), for rocprofv3 --pmc runs")
    ap.add_argument("--footprint-from", nargs="+", metavar="CSV",
                    help="summarise rocprofv3 --pmc runs of --footprint-counters")
    ap.add_argument("--footprint-name", default="",
                    help="suffix of the --footprint-from record's file name")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc runs instead of benchmarking")
    ap.add_argument("--widths-trace-from", nargs=2, metavar=("TRACE_CSV", "WIDTHS_JSONL"),
                    help="summarise a rocprofv3 --kernel-trace run of --widths (and its "
                         "stdout) into profiles/gate_kernels_widths_h2048_to_h8192_kernel_trace.md")
    ap.add_argument("--trace-from", nargs=2, metavar=("TRACE_CSV", "STATS_CSV"),
                    help="summarise a rocprofv3 --kernel-trace --stats run of the default "
                         "bench into profiles/engram_kernels_bench_default_kernel_trace.md")
    ap.add_argument("--memory-read-traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc runs over --memory-read (the hash's "
                         "and the gather's HBM bytes per launch)")
    ap.add_argument("--valu-from", metavar="SQ_CSV",
                    help="summarise a rocprofv3 --pmc run of SQ_WAVES, SQ_INSTS_VALU and "
                         "SQ_INSTS_SALU over --memory-read (the hash's instruction counts)")
    args = ap.parse_args()
    if args.memory_read_traffic_from:
        rec = memory_read_traffic(*args.memory_read_traffic_from)
        print(json.dumps(rec, indent=1, sort_keys=True))
        return
    if args.widths_trace_from:
        cmd = ("rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_widths "
               "-o widths -- python3 bench.py --widths > gpurun_out/widths.jsonl")
        text = widths_trace_summary(args.widths_trace_from[0], args.widths_trace_from[1], cmd)
        with open(os.path.join(PROFILES, "gate_kernels_widths_h2048_to_h8192_kernel_trace.md"),
                  "w") as f:
            f.write(text)
        print(text)
        return
    if args.trace_from:
        cmd = ("rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof -o bench "
               "-- python3 bench.py --no-cpu-baseline")
        text = trace_summary(args.trace_from[0], args.trace_from[1], cmd)
        with open(os.path.join(PROFILES, "engram_kernels_bench_default_kernel_trace.md"), "w") as f:
            f.write(text)
        print(text)
        return
    if args.footprint_from:
        print(json.dumps(footprint_from_counters(args.footprint_from, name=args.footprint_name),
                         indent=1, sort_keys=True))
        return
    if args.valu_from:
        print(json.dumps(valu_from_counters(args.valu_from), indent=1, sort_keys=True))
        return
    if args.traffic_from:
        rec = traffic_from_counters(args.traffic_from[0], args.traffic_from[1], args.workload)
        print(json.dumps(rec, indent=1, sort_keys=True))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported. The gate "
              "shards by tokens: each GPU runs these kernels on its share of the rows, and "
              "the only exchange is one all-reduce of the H-wide weight-gradient vector.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import engram_conditional_memory_amd as eg
    eg.load_library()
    dev = torch.device("cuda:0")

    if args.widths:
        for r in time_widths(eg, dev):
            print(json.dumps(r))
        return
    if args.placement:
        if not args.footprint_only:
            for r in time_placement(eg, dev):
                print(json.dumps(r), flush=True)
        for r in time_footprint(eg, dev):
            print(json.dumps(r), flush=True)
        return
    if args.footprint_counters:
        print(json.dumps(footprint_counter_run(eg, dev)), flush=True)
        return
    if args.memory_read:
        import synth
        c = synth.CONFIGS[4]
        copy = copy_ceiling(2 * c.T * c.H, eg, dev)
        hash_res = time_hash(eg, dev)
        gather_res, gather_zipf_res = time_gather(eg, dev)
        print(json.dumps({"copy_probe": copy, "hash": hash_res, "gather": gather_res,
                          "gather_zipf": gather_zipf_res}))
        return

    print(f"[bench] generating workload {args.workload}", file=sys.stderr, flush=True)
    w = Workload(args.workload, dev, eg)
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    main_res = time_workload(w, args.steps, args.warmup)
    autograd_res = None
    if not args.no_secondary:
        print("[bench] timing the autograd wrapper", file=sys.stderr, flush=True)
        autograd_res = time_autograd(w, eg, min(args.steps, 20), args.warmup,
                                     main_res["ms_per_step"])
    host = w.host
    w.free()
    torch.cuda.empty_cache()

    secondary = None
    if not args.no_secondary:
        other = 3 if args.workload != 3 else 4
        print(f"[bench] generating workload {other}", file=sys.stderr, flush=True)
        w2 = Workload(other, dev, eg)
        secondary = time_workload(w2, args.steps, args.warmup, min_warmup_ms=50.0)
        w2.free()
        del w2
        torch.cuda.empty_cache()

    stress = small = None
    if not args.no_secondary:
        if args.workload != 5:
            print("[bench] generating workload 5 (stress, T=65537)", file=sys.stderr, flush=True)
            w5 = Workload(5, dev, eg)
            stress = time_workload(w5, min(args.steps, 20), args.warmup, min_warmup_ms=50.0)
            w5.free()
            del w5
            torch.cuda.empty_cache()
        print("[bench] timing the small forward", file=sys.stderr, flush=True)
        small = time_fwd_small(eg, dev)

    copy = copy_ceiling(2 * main_res["T"] * main_res["H"], eg, dev)
    print("[bench] measuring the read/write-mix ceilings", file=sys.stderr, flush=True)
    tensor_bytes = 2 * main_res["T"] * main_res["H"]
    ceilings = {"fwd_3r1w": mix_ceiling(3, 1, tensor_bytes, eg, dev),
                "bwd_4r3w": mix_ceiling(4, 3, tensor_bytes, eg, dev)}
    main_res["fwd"]["frac_of_mix_ceiling"] = main_res["fwd"]["GBps"] / ceilings["fwd_3r1w"]["GBps"]
    main_res["bwd_kernel"]["frac_of_mix_ceiling"] = (main_res["bwd_kernel"]["GBps"]
                                                     / ceilings["bwd_4r3w"]["GBps"])
    vendor = vendor_reference(tensor_bytes, dev)
    hash_res = gather_res = gather_zipf_res = fused_res = graph_res = None
    if not args.no_secondary:
        print("[bench] timing the N-gram hash", file=sys.stderr, flush=True)
        hash_res = time_hash(eg, dev)
        print("[bench] timing the hashed gather", file=sys.stderr, flush=True)
        gather_res, gather_zipf_res = time_gather(eg, dev)
        fused_res = time_fused_weight(eg, dev, main_res["H"])
        print("[bench] timing a short step eagerly and from a HIP graph", file=sys.stderr,
              flush=True)
        graph_res = time_graph_step(eg, dev)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        cpu = cpu_baseline(host)

    bk = main_res["bwd_kernel"]
    traffic = measured_traffic("gate_bwd_kernel", main_res["workload"])
    line = {
        "metric": "Engram gate fwd+bwd tokens/s and achieved HBM GB/s, bf16 H=4096/7168",
        "value": main_res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Philox-4x32-10 inputs of the stated recipe)",
        "config": {"workload": main_res["workload"], "tokens": main_res["T"],
                   "hidden": main_res["H"], "tensor_dtype": "bf16", "elementwise": "f32",
                   "row_sums": "f64",
                   "step": "gate_fwd + gate_bwd + grad_w_reduce", "partials": main_res["P"]},
        "roofline": {"bound": "hbm", "kernel": "gate_bwd_kernel",
                     "achieved": bk["GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": bk["frac"], "traffic": traffic},
        "fwd": main_res["fwd"],
        "bwd": main_res["bwd"],
        "bwd_kernel": bk,
        "reduce_us": main_res["reduce_us"],
        "secondary": secondary,
        "stress": stress,
        "fwd_small": small,
        "copy_probe": copy,
        "mix_ceilings": ceilings,
        "vendor_reference": vendor,
        "hash": hash_res,
        "gather": gather_res,
        "autograd": autograd_res,
        "fused_weight": fused_res,
        "graph_step_small": graph_res,
        "gather_zipf": gather_zipf_res,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
