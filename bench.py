"""Throughput of the frame-block-causal attention hot path on one MI355X.

A step is one pass of the streaming hot path at steady state: the chunk's
queries attend to the anchored reference frame, the full rolling window and the
chunk's own frames (rtr_attn_stream_step), then the chunk's K/V are committed to
the ring (rtr_kv_append_evict).  Default workload: the Wan-1.3B-shaped layer
(12 heads, head_dim 128, 1560 tokens per latent frame, chunk of 3 frames,
1 reference frame + 6-frame window), bf16 inputs, fp32 accumulation.

Prints one JSON line.  `value` is algorithmic TFLOP/s of the whole step
(4 * d * H * visible query-key pairs, masked pairs not counted) with all inputs
resident in HBM.  `roofline` reports the attention kernel alone, timed with HIP
events around each launch on the stream it runs on.  `cpu_baseline` times the
float64 oracle on a bounded sample of the same workload on the host cores.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 4096 dense bf16 flop/clk x 2.4 GHz
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
METRIC = "block-causal attn TFLOP/s + latent frames/s per layer (frac of MFMA peak)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_{workload}.txt")
CSRC = os.path.join(ROOT, "causal_attention_frame_amd", "csrc")
# Sources whose code the counter runs of a workload depend on.
KERNEL_SRCS = {
    "forward": [os.path.join(CSRC, "attn_fwd.hip"), os.path.join(CSRC, "device_util.h")],
    "backward": [os.path.join(CSRC, "attn_bwd.hip"), os.path.join(CSRC, "device_util.h")],
}


def stream_pairs_per_head(kpf, C, prefix_frames, block_frames=1):
    """Visible (query, key) pairs of one head in a streaming step: chunk frame c
    sees the prefix frames and the chunk frames of its mask block and earlier
    blocks (blocks of block_frames frames; 1 = the per-frame mask)."""
    B = max(1, min(block_frames, C))
    return sum(kpf * (prefix_frames * kpf + min((c // B + 1) * B, C) * kpf) for c in range(C))


def full_pairs_per_head(T, kpf):
    pairs = 0
    for f0 in range(0, T, kpf):
        rows = min(kpf, T - f0)
        pairs += rows * min(f0 + kpf, T)
    return pairs


def kernel_hash(which="forward"):
    """Hash of the kernel sources' code: // comments, trailing blanks and
    blank lines are dropped, so editing a comment does not orphan the
    committed counter runs (the sources have no block comments)."""
    lines = []
    for path in KERNEL_SRCS[which]:
        with open(path) as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


def read_traffic(workload):
    """HBM bytes per attention launch from committed rocprofv3 counter runs;
    None when absent or taken on a different kernel source."""
    path = TRAFFIC_FILE.format(workload=workload)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    which = "backward" if workload.endswith("_bwd") else "forward"
    if vals.get("kernel_source_sha256_16") != kernel_hash(which):
        return None
    try:
        return float(vals["attn_hbm_bytes_per_launch_calibrated"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(workload, x, w, heads):
    """The float64 oracle (as it stands) on `heads` heads of the same inputs."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count()
    kpf, H, d = w["k"], w["H"], w["d"]
    sl = slice(0, heads)
    if workload.endswith("stream_step"):
        pk = np.concatenate([x["ref_k"].values.reshape(-1, H, d),
                             x["ring_k"].values.reshape(-1, H, d)])[:, sl]
        pv = np.concatenate([x["ref_v"].values.reshape(-1, H, d),
                             x["ring_v"].values.reshape(-1, H, d)])[:, sl]
        args = (pk, pv, x["q"].values[:, sl], x["k"].values[:, sl], x["v"].values[:, sl], kpf)
        t0 = time.perf_counter()
        oracle.attn_stream_step(*args)
        dt = time.perf_counter() - t0
        C = x["q"].shape[0] // kpf
        flops = 4 * d * heads * stream_pairs_per_head(kpf, C, x["ref_k"].shape[0] + w["W"])
        sample = (f"oracle.attn_stream_step (dense float64) on heads 0..{heads - 1} of {H}, "
                  f"all {C * kpf} query rows")
    else:
        T = x["q"].shape[0]
        rows = list(range(0, T, max(1, T // 256)))
        t0 = time.perf_counter()
        oracle.attn_rows(x["q"].values, x["k"].values, x["v"].values, kpf, rows, list(range(heads)))
        dt = time.perf_counter() - t0
        pairs = sum(min((r // kpf + 1) * kpf, T) for r in rows)
        flops = 4 * d * heads * pairs
        sample = f"oracle.attn_rows on {len(rows)} query rows x {heads} heads"
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": sample, "seconds": round(dt, 3)}


def prewarm(step, dev, seconds):
    """Untimed back-to-back steps for `seconds` of wall time, so that the GPU
    has left its idle clock before the counted warm-up steps (an idle MI355X
    sits at a few hundred MHz and takes tens of milliseconds to ramp up, longer
    than a short timed region).  Returns the number of steps run."""
    import torch
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            step()
        n += 10
        torch.cuda.synchronize(dev)
    return n


def device_info(dev):
    import torch
    p = torch.cuda.get_device_properties(dev)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
            "hbm_gib": round(p.total_memory / 2 ** 30, 1)}


def clock_mhz(dev):
    """Shader clock right now (library clock probe, ~50 us), in MHz."""
    from causal_attention_frame_amd import rtr
    return round(rtr.rtr_clock_sample(dev), 1)


class ClockSampler:
    """Shader-clock samples taken while the timed steps run: every `every`-th
    step, once that step's first launch has started, a 100-us clock probe runs
    on a side stream (one lane of one compute unit, next to the step's
    kernels; nothing on the timed stream waits for it).  begin() marks the
    step start with an event of its own on steps i % every == phase, which the
    event-timed steps (i % EV_EVERY == 0) avoid when phase is not 0; maybe()
    uses a start event the caller already recorded."""

    def __init__(self, dev, steps, every=4, phase=0):
        import torch
        from causal_attention_frame_amd import rtr
        import ctypes
        self.every, self.phase = every, phase
        self.side = torch.cuda.Stream(dev)
        self.marks = [torch.cuda.Event() for _ in range(steps // every + 1)]
        self.buf = torch.zeros((steps // every + 1, 2), dtype=torch.int64, device=dev)
        self.ptrs = [ctypes.c_void_p(self.buf[i].data_ptr()) for i in range(self.buf.shape[0])]
        self.sp = ctypes.c_void_p(self.side.cuda_stream)
        self.n = 0
        self.fn = rtr.lib().rtr_clock_sample
        # first use of the side stream and of the probe outside the timed region
        self.fn(self.ptrs[0], 100, self.sp)
        torch.cuda.synchronize(dev)

    def maybe(self, i, start_event):
        if i % self.every != self.phase or self.n >= self.buf.shape[0]:
            return
        self.side.wait_event(start_event)
        self.fn(self.ptrs[self.n], 10000, self.sp)
        self.n += 1

    def begin(self, i, stream):
        if i % self.every != self.phase or self.n >= self.buf.shape[0]:
            return
        self.marks[self.n].record(stream)
        self.maybe(i, self.marks[self.n])

    def summary(self):
        if self.n == 0:
            return None
        t = self.buf[:self.n].cpu().numpy().astype(np.float64)
        mhz = 100.0 * t[:, 0] / np.maximum(t[:, 1], 1.0)
        return {"median": round(float(np.median(mhz)), 1), "min": round(float(mhz.min()), 1),
                "max": round(float(mhz.max()), 1), "samples": int(self.n)}


# HIP events bracket every EV_EVERY-th timed step only: each record is a marker
# on the stream that costs a few microseconds of its own, which a step of a
# few hundred microseconds would otherwise carry on every step (measured on the
# Wan-1.3B step: 0.418 ms per step with four records per step, 0.401 ms with
# three records per four steps, the kernel's own time unchanged).
EV_EVERY = 4


class SampledEvents:
    """Events for the timed loop: on steps i with i % EV_EVERY == 0, one
    record before the step's first part and one after each part, so that each
    part's device time is sampled there.  Created before the pre-warm (event
    creation idles the GPU)."""

    def __init__(self, steps, nparts):
        import torch
        n = (steps + EV_EVERY - 1) // EV_EVERY
        self.ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nparts + 1)] for _ in range(n)]

    def run(self, stream, steps, parts, clk):
        """The timed steps; returns the wall time in seconds (synchronised)."""
        import torch
        torch.cuda.synchronize(stream.device)
        t0 = time.perf_counter()
        for i in range(steps):
            if i % EV_EVERY == 0:
                e = self.ev[i // EV_EVERY]
                e[0].record(stream)
                for j, part in enumerate(parts):
                    part()
                    e[j + 1].record(stream)
            else:
                clk.begin(i, stream)
                for part in parts:
                    part()
        torch.cuda.synchronize(stream.device)
        return time.perf_counter() - t0

    def ms(self, j):
        """Device milliseconds of part j on the sampled steps."""
        return np.array([e[j].elapsed_time(e[j + 1]) for e in self.ev])


def timing_stats(ms):
    return {"kernel_avg_us": round(float(np.mean(ms)) * 1e3, 2),
            "kernel_median_us": round(float(np.median(ms)) * 1e3, 2),
            "kernel_min_us": round(float(np.min(ms)) * 1e3, 2)}


def cpu_single_thread(workload_x, w):
    """The float64 oracle on one host thread (BLAS limited to 1 thread): the
    tiny float32 workload (full form, 144 tokens) and one head of the
    Wan-1.3B streaming step, as TFLOP/s."""
    import oracle
    from causal_attention_frame_amd import inputs as gen
    try:
        from threadpoolctl import threadpool_limits
    except Exception:
        return None
    out = {}
    with threadpool_limits(limits=1):
        tw = gen.WORKLOADS["tiny_fp32"]
        T = tw["k"] * tw["frames"]
        q, k, v = gen.full_sequence_inputs(T, tw["H"], tw["d"], "f32", base_seed=0, wid=tw["wid"])
        t0 = time.perf_counter()
        reps = 20
        for _ in range(reps):
            oracle.attn_block_causal(q.values, k.values, v.values, tw["k"])
        dt = (time.perf_counter() - t0) / reps
        f = 4 * tw["d"] * tw["H"] * full_pairs_per_head(T, tw["k"])
        out["tiny_fp32_full"] = {"value": f / dt / 1e12, "unit": "TFLOP/s", "seconds_per_call": round(dt, 5),
                                 "sample": f"oracle.attn_block_causal, {T} tokens x {tw['H']} heads"}
        if workload_x is not None:
            x, H, d, kpf = workload_x["x"], w["H"], w["d"], w["k"]
            sl = slice(0, 1)
            pk = np.concatenate([x["ref_k"].values.reshape(-1, H, d), x["ring_k"].values.reshape(-1, H, d)])[:, sl]
            pv = np.concatenate([x["ref_v"].values.reshape(-1, H, d), x["ring_v"].values.reshape(-1, H, d)])[:, sl]
            t0 = time.perf_counter()
            oracle.attn_stream_step(pk, pv, x["q"].values[:, sl], x["k"].values[:, sl], x["v"].values[:, sl], kpf)
            dt = time.perf_counter() - t0
            C = x["q"].shape[0] // kpf
            f = 4 * d * stream_pairs_per_head(kpf, C, x["ref_k"].shape[0] + w["W"])
            out["stream_step_one_head"] = {"value": f / dt / 1e12, "unit": "TFLOP/s", "seconds": round(dt, 3),
                                           "sample": f"oracle.attn_stream_step, head 0 of {H}, all {C * kpf} rows"}
    out["cores"] = 1
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="wan13b_stream_step",
                    choices=["wan13b_stream_step", "wan14b_stream_step", "full_block_causal",
                             "full_block_causal_bwd", "wan13b_stream_step_bwd", "wan13b_cross_step",
                             "wan13b_cross_step_bwd", "rollout"],
                    help="rollout: one step is a whole 240-chunk rollout (stream step, commit, "
                         "and a reference swap every 60 chunks)")
    ap.add_argument("--cpu-heads", type=int, default=12,
                    help="heads of the workload the CPU oracle baseline runs on")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prewarm-s", type=float, default=0.5,
                    help="untimed wall-clock seconds of steps before the warm-up steps (GPU clock ramp)")
    ap.add_argument("--chunk-frames", type=int, default=0,
                    help="streaming forward workloads: frames per chunk (default: the workload's; "
                         "1 is the lowest-latency streaming step)")
    ap.add_argument("--ref-frames", type=int, default=0,
                    help="streaming workloads: anchored reference frames (default: the workload's)")
    ap.add_argument("--block-frames", type=int, default=1,
                    help="streaming workloads: frames per in-chunk mask block (chunk-level causality "
                         "with the chunk length; default 1, the per-frame mask)")
    ap.add_argument("--ref-rope", action="store_true",
                    help="streaming workloads: position-aware reference (re-encoded in front of the "
                         "window every step; 22 temporal rotary pairs, as Wan's 44 temporal dims)")
    ap.add_argument("--no-cache-grads", action="store_true",
                    help="wan13b_stream_step_bwd: treat the cache as constant (no gradients of the "
                         "cached keys and values)")
    ap.add_argument("--cold", type=int, default=0,
                    help="after the timed steps, time the attention kernel of this many more steps, each "
                         "after overwriting a 512 MiB buffer (L2 and the last-level cache start cold); "
                         "reported as cold_cache, outside value")
    ap.add_argument("--head-dim", type=int, default=0, choices=[0, 64, 128],
                    help="streaming forward workloads: head dim, with the heads rescaled to keep the "
                         "model width (64: twice the heads; the head_dim-64 kernel)")
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "f32"],
                    help="streaming forward workloads: input and arithmetic type (f32: the float32 "
                         "kernel, bound by the fp32 vector ALUs)")
    ap.add_argument("--overlap-append", action="store_true",
                    help="streaming forward workloads: a ring of W + C slots and each chunk's commit "
                         "on a second stream beside the step that reads the window (default: the "
                         "commit after the step on the same stream, over a ring of W slots; faster "
                         "here, since the chip runs the step at its power limit)")
    ap.add_argument("--tokens-per-frame", type=int, default=0,
                    help="streaming forward workloads: tokens per latent frame instead of the workload's "
                         "(e.g. 2080 = 40x52 patches of an 832x640 frame, a sensitivity run)")
    ap.add_argument("--split", action="store_true",
                    help="split-K schedule with a workspace (default: one workgroup per "
                         "(head, query block), the faster schedule on these shapes)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(the attention would shard by head, with no exchange between GPUs).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from causal_attention_frame_amd import inputs as gen
    from causal_attention_frame_amd import rtr

    rtr.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = gen.WORKLOADS[args.workload]
    if args.workload == "rollout":
        return rollout(args, w, dev)
    if args.workload == "full_block_causal_bwd":
        return backward(args, w, dev)
    if args.workload == "wan13b_stream_step_bwd":
        return stream_backward(args, w, dev)
    if args.workload in ("wan13b_cross_step", "wan13b_cross_step_bwd"):
        return cross(args, w, dev)

    if args.tokens_per_frame:
        w = dict(w, k=args.tokens_per_frame)
    f32 = args.dtype == "f32"
    if (f32 or args.head_dim or args.tokens_per_frame) and not args.workload.endswith("stream_step"):
        sys.exit("--dtype f32, --head-dim and --tokens-per-frame apply to the streaming forward workloads")

    def to_dev(t):
        if f32:
            return torch.from_numpy(np.ascontiguousarray(t.values, dtype=np.float32)).to(dev)
        return torch.from_numpy(t.bits.view(np.int16)).to(dev).view(torch.bfloat16)

    kpf, H, d = w["k"], w["H"], w["d"]
    if args.head_dim:
        H, d = H * d // args.head_dim, args.head_dim
    tdt = torch.float32 if f32 else torch.bfloat16
    stream = torch.cuda.current_stream(dev)
    ws = rtr.new_workspace(d, rtr.RTR_F32 if f32 else rtr.RTR_BF16, dev) if args.split else None
    if args.workload.endswith("stream_step"):
        C, W, R = (args.chunk_frames or w["C"]), w["W"], (args.ref_frames or w["R"])
        x = gen.stream_inputs(kpf, H, d, C, W, R, args.dtype, base_seed=0, wid=w["wid"],
                              outlier_frac=w.get("outlier_frac", 0.0),
                              outlier_scale=w.get("outlier_scale", 1.0))
        overlap = args.overlap_append
        N = W + C if overlap else W       # spare slots: the commit writes none the step reads
        kr = torch.empty((N, kpf, H, d), dtype=tdt, device=dev)
        vr = torch.empty_like(kr)
        kf = torch.empty((R, kpf, H, d), dtype=tdt, device=dev)
        vf = torch.empty_like(kf)
        kv = rtr.rtr_kv_create_slots(kr, vr, kf, vf, W, N, R, kpf, H, d,
                                     rtr.RTR_F32 if f32 else rtr.RTR_BF16)
        if args.ref_rope:
            rtr.rtr_kv_set_ref_rope(kv, torch.empty_like(kf), 22, 10000.0, R)
        rtr.rtr_kv_reset_ref(kv, rtr.RTR_REF_REPLACE, to_dev(x["ref_k"]), to_dev(x["ref_v"]), R, -1)
        rtr.rtr_kv_append_evict(kv, to_dev(x["ring_k"]), to_dev(x["ring_v"]), W)
        q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
        o = torch.empty_like(q)
        frames = C
        flops = 4 * d * H * stream_pairs_per_head(kpf, C, R + W, args.block_frames)
        append_bytes = 2 * 2 * C * kpf * H * d * (4 if f32 else 2)     # K and V, read + write
        config = {"workload": args.workload, "heads": H, "head_dim": d, "tokens_per_frame": kpf,
                  "chunk_frames": C, "window_frames": W, "ref_frames": R,
                  "query_tokens": C * kpf, "key_tokens": (R + W + C) * kpf,
                  "append": ("overlapped: a second stream, ring of W + C slots" if overlap
                             else "serial: same stream, ring of W slots")}
        if args.block_frames != 1:
            config["mask_block_frames"] = args.block_frames
        if args.ref_rope:
            config["position_aware_reference"] = True

        # Overlapped commit: step t's commit writes the slots that step t-1
        # read, so it waits for step t-1's attention; step t+1 waits for it.
        # Events come from a small pool (a re-recorded event is only waited
        # on after its new record is enqueued).
        side = torch.cuda.Stream(dev) if overlap else None   # default priority
        pool = [torch.cuda.Event() for _ in range(8)]
        # timing events of the commit on the side stream, on the sampled steps
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range((args.steps + EV_EVERY - 1) // EV_EVERY)] if overlap else []
        ov = {"n": 0, "a_prev": None, "a_cur": None, "c": None, "step": -1}
        torch.cuda.synchronize(dev)   # inputs and the initial ring resident before the side stream runs

        def attention():
            if ov["c"] is not None:
                stream.wait_event(ov["c"])
            if args.block_frames == 1:
                rtr.rtr_attn_stream_step(kv, q, k, v, C, o=o, workspace=ws)
            else:
                rtr.rtr_attn_stream_step_blocked(kv, q, k, v, C, args.block_frames, o=o, workspace=ws)
            if overlap:
                ev = pool[ov["n"] % 8]
                ov["n"] += 1
                ev.record(stream)
                ov["a_cur"] = ev

        def commit():
            if not overlap:
                rtr.rtr_kv_append_evict(kv, k, v, C)
                return
            if ov["a_prev"] is not None:
                side.wait_event(ov["a_prev"])
            st = ov["step"]
            sample = cev[st // EV_EVERY] if 0 <= st < args.steps and st % EV_EVERY == 0 else None
            if st >= 0:
                ov["step"] += 1
            if sample is not None:
                sample[0].record(side)
            rtr.rtr_kv_append_evict(kv, k, v, C, stream=side)
            if sample is not None:
                sample[1].record(side)
            ev = pool[ov["n"] % 8]
            ov["n"] += 1
            ev.record(side)
            ov["c"] = ev
            ov["a_prev"] = ov["a_cur"]
    else:
        F = w["frames"]
        T = kpf * F
        x = dict(zip("qkv", gen.full_sequence_inputs(T, H, d, "bf16", base_seed=0, wid=w["wid"])))
        q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
        o = torch.empty_like(q)
        frames = F - 1   # latent frames, the reference frame excluded
        flops = 4 * d * H * full_pairs_per_head(T, kpf)
        append_bytes = 0
        config = {"workload": args.workload, "heads": H, "head_dim": d, "tokens_per_frame": kpf,
                  "frames": F, "tokens": T}

        def attention():
            rtr.rtr_attn_block_causal(q, k, v, kpf, o=o, workspace=ws)

        def commit():
            pass

    def whole_step():
        attention()
        commit()

    # everything that idles the GPU (event creation, the clock probes) comes
    # before the pre-warm, so that the load runs on into the timed steps
    sev = SampledEvents(args.steps, 2)
    mhz_before = clock_mhz(dev)
    clk = ClockSampler(dev, args.steps, every=EV_EVERY, phase=EV_EVERY // 2)
    nwarm = prewarm(whole_step, dev, args.prewarm_s)
    for _ in range(args.warmup):
        whole_step()
    if append_bytes and overlap:
        ov["step"] = 0     # the timed steps: sample the side-stream commits
    elapsed = sev.run(stream, args.steps, [attention, commit], clk)
    mhz_after = clock_mhz(dev)

    attn_ms = sev.ms(0)
    commit_ms = sev.ms(1)
    if append_bytes and overlap:
        ov["step"] = -1
        commit_ms = np.array([a.elapsed_time(b) for a, b in cev])
    cold = None
    if args.cold > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        evk = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.cold)]
        for i in range(args.cold):
            flush.fill_(i & 0xFF)
            evk[i][0].record(stream)
            attention()
            evk[i][1].record(stream)
            commit()
        torch.cuda.synchronize(dev)
        cms = np.array([a.elapsed_time(b) for a, b in evk])
        cold = dict(timing_stats(cms), steps=args.cold, flush_bytes=512 << 20)
        del flush
    ms_per_step = elapsed * 1e3 / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    attn_avg_s = float(attn_ms.mean()) * 1e-3
    achieved = flops / attn_avg_s / 1e12
    # the committed counter records cover each workload's own configuration only
    default_cfg = (not args.split and not args.ref_rope and args.block_frames == 1
                   and args.chunk_frames in (0, w.get("C", 0)) and args.ref_frames in (0, w.get("R", 0)))
    default_cfg = default_cfg and not f32 and args.head_dim in (0, w["d"])
    traffic = read_traffic(args.workload) if default_cfg else None
    peak = PEAK_F32_TFLOPS if f32 else PEAK_BF16_TFLOPS
    if f32:
        kname = "attn_fwd_f32"
    else:
        kname = ("attn_fwd_bf16_d128" if d == 128 else "attn_fwd_bf16") \
            + ("" if ws is None else " (+ attn_combine_d128 when the library splits)")

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": config,
        "latent_frames_per_s_per_layer": round(frames / (ms_per_step * 1e-3), 1),
        "frac_of_mfma_peak": round(value / peak, 4),
        "roofline": {
            "bound": "alu" if f32 else "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "kernel": kname,
            "schedule": "plain" if ws is None else "workspace given: split-K where the planner predicts a gain",
            **timing_stats(attn_ms),
            "algorithmic_flop_per_launch": flops,
        },
        "gpu": dict(device_info(dev), sclk_mhz_before_timed=mhz_before, sclk_mhz_after_timed=mhz_after,
                    sclk_mhz_during_timed=clk.summary(), prewarm_steps=nwarm, prewarm_s=args.prewarm_s),
    }
    if cold is not None:
        out["cold_cache"] = cold
    if append_bytes:
        cs = float(np.median(commit_ms)) * 1e-3
        out["kv_append"] = {"bound": "hbm", "median_us": round(cs * 1e6, 2),
                            "stream": "second stream, beside the step" if overlap else "the step's stream",
                            "achieved": round(append_bytes / cs / 1e9, 1), "unit": "GB/s",
                            "peak": PEAK_HBM_GBS,
                            "frac": round(append_bytes / cs / 1e9 / PEAK_HBM_GBS, 4),
                            "algorithmic_bytes": append_bytes}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.workload, x, w, args.cpu_heads)
        if args.workload == "wan13b_stream_step":
            st = cpu_single_thread({"x": x}, w)
            if st is not None:
                out["cpu_baseline_single_thread"] = st
    print(json.dumps(out), flush=True)


def backward(args, w, dev):
    """Gradients of the full-sequence form (the training step's attention
    backward): one step is one rtr_attn_block_causal_bwd call -- the prep, dK/dV
    and dQ kernels -- on resident q, k, v, o, lse and dO (o and lse from the
    library's forward).  Algorithmic work: the five products of the standard
    count (S recomputed, dP, dV, dK, dQ), 2.5x the forward's."""
    import torch
    from causal_attention_frame_amd import inputs as gen
    from causal_attention_frame_amd import rtr

    kpf, H, d, F = w["k"], w["H"], w["d"], w["frames"]
    T = kpf * F
    x = gen.bwd_inputs(T, H, d, "bf16", base_seed=0, wid=w["wid"])
    q, k, v, do = (torch.from_numpy(t.bits.view(np.int16)).to(dev).view(torch.bfloat16) for t in x)
    o, lse = rtr.rtr_attn_block_causal(q, k, v, kpf, want_lse=True)
    ws = torch.empty(rtr.rtr_attn_bwd_workspace_size(T, H, d), dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stream = torch.cuda.current_stream(dev)
    pairs = full_pairs_per_head(T, kpf)
    flops = 10 * d * H * pairs

    def step():
        rtr.rtr_attn_block_causal_bwd(q, k, v, o, lse, do, kpf, dq, dk, dv, workspace=ws)

    sev = SampledEvents(args.steps, 1)
    mhz_before = clock_mhz(dev)
    clk = ClockSampler(dev, args.steps, every=EV_EVERY, phase=EV_EVERY // 2)
    nwarm = prewarm(step, dev, args.prewarm_s)
    for _ in range(args.warmup):
        step()
    elapsed = sev.run(stream, args.steps, [step], clk)
    mhz_after = clock_mhz(dev)
    call_ms = sev.ms(0)
    ms_per_step = elapsed * 1e3 / args.steps
    call_s = float(call_ms.mean()) * 1e-3
    out = {
        "metric": METRIC,
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "full_block_causal_bwd", "heads": H, "head_dim": d,
                   "tokens_per_frame": kpf, "frames": F, "tokens": T},
        "roofline": {
            "bound": "mfma",
            "achieved": round(flops / call_s / 1e12, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(flops / call_s / 1e12 / PEAK_BF16_TFLOPS, 4),
            "traffic": read_traffic("full_block_causal_bwd"),
            "kernel": "attn_bwd_prep + attn_bwd_dkdv_d128 + attn_bwd_dq_d128 (one call)",
            **timing_stats(call_ms),
            "algorithmic_flop_per_launch": flops,
        },
        "gpu": dict(device_info(dev), sclk_mhz_before_timed=mhz_before, sclk_mhz_after_timed=mhz_after,
                    sclk_mhz_during_timed=clk.summary(), prewarm_steps=nwarm, prewarm_s=args.prewarm_s),
    }
    if not args.no_cpu_baseline:
        import oracle
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            cores = os.cpu_count()
        heads = list(range(min(H, args.cpu_heads)))
        rows = list(range(0, T, max(1, T // 64)))
        t1 = time.perf_counter()
        oracle.attn_bwd_rows(x[0].values, x[1].values, x[2].values, x[3].values, kpf, rows, heads)
        dt = time.perf_counter() - t1
        seen = sum(min((r // kpf + 1) * kpf, T) for r in rows)
        # per (row, key) pair the row variant forms S, dP and dQ: 6 d flops
        out["cpu_baseline"] = {"value": 6 * d * len(heads) * seen / dt / 1e12, "unit": "TFLOP/s",
                               "cores": int(cores), "kind": "oracle",
                               "sample": f"oracle.attn_bwd_rows (dQ) on {len(rows)} rows x "
                                         f"{len(heads)} heads", "seconds": round(dt, 3)}
    print(json.dumps(out), flush=True)


def stream_backward(args, w, dev):
    """Gradients of one streaming step (the Self-Forcing-style rollout's
    attention backward): one step is one rtr_attn_stream_step_bwd call --
    prep, dK/dV of the chunk keys and of the cached keys in one launch, and dQ
    over the segmented keys -- on resident inputs, o and lse from the library's
    own streaming step.  Algorithmic work per visible (row, key) pair: 10 d
    (S recomputed, dP, dV, dK, dQ); without cache gradients the cached keys'
    pairs count 6 d (S, dP, dQ)."""
    import torch
    from causal_attention_frame_amd import inputs as gen
    from causal_attention_frame_amd import rtr

    kpf, H, d, C, W = w["k"], w["H"], w["d"], w["C"], w["W"]
    R = args.ref_frames or w["R"]
    x = gen.stream_inputs(kpf, H, d, C, W, R, "bf16", base_seed=0, wid=w["wid"])
    do_h = gen.normal((C * kpf, H, d), "bf16", 0, w["wid"], 0, gen.TAG_DO)

    def to_dev(t):
        return torch.from_numpy(t.bits.view(np.int16)).to(dev).view(torch.bfloat16)

    kr = torch.empty((W, kpf, H, d), dtype=torch.bfloat16, device=dev)
    vr = torch.empty_like(kr)
    kf = torch.empty((R, kpf, H, d), dtype=torch.bfloat16, device=dev)
    vf = torch.empty_like(kf)
    kv = rtr.rtr_kv_create(kr, vr, kf, vf, W, R, kpf, H, d)
    rtr.rtr_kv_reset_ref(kv, rtr.RTR_REF_REPLACE, to_dev(x["ref_k"]), to_dev(x["ref_v"]), R, -1)
    rtr.rtr_kv_append_evict(kv, to_dev(x["ring_k"]), to_dev(x["ring_v"]), W)
    q, k, v, do = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(do_h)
    o, lse = rtr.rtr_attn_stream_step(kv, q, k, v, C, want_lse=True)
    Tq, P = C * kpf, (R + W) * kpf
    ws = torch.empty(rtr.rtr_attn_bwd_workspace_size(Tq, H, d), dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    cache_grads = not args.no_cache_grads
    dkc = torch.empty((P, H, d), dtype=torch.bfloat16, device=dev) if cache_grads else None
    dvc = torch.empty_like(dkc) if cache_grads else None
    stream = torch.cuda.current_stream(dev)
    chunk_pairs = stream_pairs_per_head(kpf, C, 0)
    prefix_pairs = Tq * P
    flops = 10 * d * H * chunk_pairs + (10 if cache_grads else 6) * d * H * prefix_pairs

    def step():
        rtr.rtr_attn_stream_step_bwd(kv, q, k, v, o, lse, do, C, 1, dq, dk, dv, dkc, dvc, workspace=ws)

    sev = SampledEvents(args.steps, 1)
    mhz_before = clock_mhz(dev)
    clk = ClockSampler(dev, args.steps, every=EV_EVERY, phase=EV_EVERY // 2)
    nwarm = prewarm(step, dev, args.prewarm_s)
    for _ in range(args.warmup):
        step()
    elapsed = sev.run(stream, args.steps, [step], clk)
    mhz_after = clock_mhz(dev)
    call_ms = sev.ms(0)
    ms_per_step = elapsed * 1e3 / args.steps
    call_s = float(call_ms.mean()) * 1e-3
    config = {"workload": args.workload, "heads": H, "head_dim": d, "tokens_per_frame": kpf,
              "chunk_frames": C, "window_frames": W, "ref_frames": R, "query_tokens": Tq,
              "key_tokens": P + Tq, "cache_grads": cache_grads}
    out = {
        "metric": METRIC,
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": config,
        "roofline": {
            "bound": "mfma",
            "achieved": round(flops / call_s / 1e12, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(flops / call_s / 1e12 / PEAK_BF16_TFLOPS, 4),
            "traffic": read_traffic(args.workload) if cache_grads and R == w["R"] else None,
            "kernel": "attn_bwd_prep + attn_bwd_dkdv_d128 + attn_bwd_dq_d128<SEG> (one call)",
            **timing_stats(call_ms),
            "algorithmic_flop_per_launch": flops,
        },
        "gpu": dict(device_info(dev), sclk_mhz_before_timed=mhz_before, sclk_mhz_after_timed=mhz_after,
                    sclk_mhz_during_timed=clk.summary(), prewarm_steps=nwarm, prewarm_s=args.prewarm_s),
    }
    if not args.no_cpu_baseline:
        import oracle
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            cores = os.cpu_count()
        h = list(range(min(H, args.cpu_heads)))   # dense float64 oracle, one head at a time
        pk = np.concatenate([x["ref_k"].values.reshape(-1, H, d), x["ring_k"].values.reshape(-1, H, d)])
        pv = np.concatenate([x["ref_v"].values.reshape(-1, H, d), x["ring_v"].values.reshape(-1, H, d)])
        args1 = (pk[:, h], pv[:, h], x["q"].values[:, h], x["k"].values[:, h], x["v"].values[:, h],
                 do_h.values[:, h], kpf)
        t1 = time.perf_counter()
        for j in range(len(h)):
            oracle.attn_stream_step_bwd(*(a[:, j:j + 1] for a in args1[:6]), kpf)
        dt = time.perf_counter() - t1
        f1 = 10 * d * len(h) * (chunk_pairs + prefix_pairs)
        out["cpu_baseline"] = {"value": f1 / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores),
                               "kind": "oracle",
                               "sample": f"oracle.attn_stream_step_bwd (dense float64, every "
                                         f"gradient) on heads 0..{len(h) - 1} of {H}",
                               "seconds": round(dt, 3)}
    print(json.dumps(out), flush=True)


def cross(args, w, dev):
    """Text cross-attention of one chunk: one step is one rtr_attn_cross call of
    the chunk's C*k query rows against the text cache's tokens (no mask).  The
    cache reset of a text switch (copy of the new condition's K and V) is timed
    separately and reported as `text_reset`.  The _bwd workload times
    rtr_attn_cross_bwd instead (dq and the text keys' and values' gradients;
    10 d flops per (row, text token) pair: S recomputed, dP, dV, dK, dQ)."""
    import torch
    from causal_attention_frame_amd import inputs as gen
    from causal_attention_frame_amd import rtr

    H, d, Lt = w["H"], w["d"], w["text_tokens"]
    Tq = w["C"] * w["k"]
    x = gen.cross_inputs(Tq, Lt, H, d, "bf16", base_seed=0, wid=w["wid"])
    q, kt, vt = (torch.from_numpy(t.bits.view(np.int16)).to(dev).view(torch.bfloat16) for t in x)
    kb, vb = torch.empty_like(kt), torch.empty_like(vt)
    tc = rtr.rtr_text_cache_create(kb, vb, Lt, H, d)
    rtr.rtr_text_cache_reset(tc, kt, vt, Lt)
    o = torch.empty_like(q)
    ws = rtr.new_workspace(d, rtr.RTR_BF16, dev) if args.split else None
    stream = torch.cuda.current_stream(dev)
    bwd = args.workload.endswith("_bwd")
    flops = (10 if bwd else 4) * d * H * Tq * Lt
    if bwd:
        o, lse = rtr.rtr_attn_cross(tc, q, want_lse=True)
        do_h = gen.normal((Tq, H, d), "bf16", 0, w["wid"], 0, gen.TAG_DO)
        do = torch.from_numpy(do_h.bits.view(np.int16)).to(dev).view(torch.bfloat16)
        dq, dkt, dvt = torch.empty_like(q), torch.empty_like(kt), torch.empty_like(vt)
        wsb = torch.empty(rtr.rtr_attn_cross_bwd_workspace_size(Tq, Lt, H, d), dtype=torch.uint8, device=dev)

    def step():
        if bwd:
            rtr.rtr_attn_cross_bwd(tc, q, o, lse, do, dq, dkt, dvt, workspace=wsb)
        else:
            rtr.rtr_attn_cross(tc, q, o=o, workspace=ws)

    sev = SampledEvents(args.steps, 1)
    mhz_before = clock_mhz(dev)
    clk = ClockSampler(dev, args.steps, every=EV_EVERY, phase=EV_EVERY // 2)
    nwarm = prewarm(step, dev, args.prewarm_s)
    for _ in range(args.warmup):
        step()
    elapsed = sev.run(stream, args.steps, [step], clk)
    mhz_after = clock_mhz(dev)
    call_ms = sev.ms(0)
    # text switch: re-initialise the cache with a condition of the same length
    er = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
    for a, b in er:
        a.record(stream)
        rtr.rtr_text_cache_reset(tc, vt, kt, Lt)
        b.record(stream)
    torch.cuda.synchronize(dev)
    reset_s = float(np.median([a.elapsed_time(b) for a, b in er])) * 1e-3
    reset_bytes = 2 * 2 * Lt * H * d * 2
    ms_per_step = elapsed * 1e3 / args.steps
    call_s = float(call_ms.mean()) * 1e-3
    out = {
        "metric": METRIC,
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "heads": H, "head_dim": d, "query_tokens": Tq,
                   "text_tokens": Lt},
        "roofline": {
            "bound": "mfma",
            "achieved": round(flops / call_s / 1e12, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(flops / call_s / 1e12 / PEAK_BF16_TFLOPS, 4),
            "traffic": None,
            "kernel": ("attn_bwd_prep + attn_bwd_dkdv_d128 + attn_bwd_dq_d128<SEG> (one call)" if bwd else
                       "attn_fwd_bf16_d128" + ("" if ws is None else " (+ split-K when planned)")),
            **timing_stats(call_ms),
            "algorithmic_flop_per_launch": flops,
        },
        "gpu": dict(device_info(dev), sclk_mhz_before_timed=mhz_before, sclk_mhz_after_timed=mhz_after,
                    sclk_mhz_during_timed=clk.summary(), prewarm_steps=nwarm, prewarm_s=args.prewarm_s),
        "text_reset": {"bound": "hbm", "median_us": round(reset_s * 1e6, 2),
                       "achieved": round(reset_bytes / reset_s / 1e9, 1), "unit": "GB/s",
                       "peak": PEAK_HBM_GBS, "algorithmic_bytes": reset_bytes},
    }
    tc.close()
    if not args.no_cpu_baseline:
        import oracle
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            cores = os.cpu_count()
        heads = min(H, args.cpu_heads)
        t1 = time.perf_counter()
        if bwd:
            oracle.attn_cross_bwd(x[0].values[:, :heads], x[1].values[:, :heads], x[2].values[:, :heads],
                                  do_h.values[:, :heads])
        else:
            oracle.attn_cross(x[0].values[:, :heads], x[1].values[:, :heads], x[2].values[:, :heads])
        dt = time.perf_counter() - t1
        name = "oracle.attn_cross_bwd" if bwd else "oracle.attn_cross"
        out["cpu_baseline"] = {"value": (10 if bwd else 4) * d * heads * Tq * Lt / dt / 1e12,
                               "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
                               "sample": f"{name} (dense float64) on heads 0..{heads - 1} of {H}",
                               "seconds": round(dt, 3)}
    print(json.dumps(out), flush=True)


def rollout(args, w, dev):
    """A long streaming rollout: `chunks` successive C-frame chunks through the
    W-frame window with an anchored reference that is replaced before chunks
    0, swap_every, 2*swap_every, ... (RTR-DiT notes, Key Designs 4).  At each
    swap the window keeps its newest frame (at chunk 0 it starts empty), so the
    prefix refills from 1 frame.  One timed step is one whole rollout: every
    reset, stream step and commit, all on device-resident inputs drawn from a
    pool of P seeded chunk inputs and P reference frames."""
    import torch
    from causal_attention_frame_amd import inputs as gen
    from causal_attention_frame_amd import rtr

    kpf, H, d, C, W, R = w["k"], w["H"], w["d"], w["C"], w["W"], w["R"]
    chunks, every, P = w["chunks"], w["swap_every"], 4

    def dev_bf16(shape, step, tag):
        t = gen.normal(shape, "bf16", 0, w["wid"], step, tag)
        return torch.from_numpy(t.bits.view(np.int16)).to(dev).view(torch.bfloat16)

    pool = [tuple(dev_bf16((C * kpf, H, d), s, t) for t in (gen.TAG_Q, gen.TAG_K, gen.TAG_V))
            for s in range(P)]
    refs = [tuple(dev_bf16((R, kpf, H, d), s, t) for t in (gen.TAG_REFK, gen.TAG_REFV))
            for s in range(P)]
    kr = torch.empty((W, kpf, H, d), dtype=torch.bfloat16, device=dev)
    vr = torch.empty_like(kr)
    kf = torch.empty((R, kpf, H, d), dtype=torch.bfloat16, device=dev)
    vf = torch.empty_like(kf)
    kv = rtr.rtr_kv_create(kr, vr, kf, vf, W, R, kpf, H, d)
    o = torch.empty_like(pool[0][0])
    stream = torch.cuda.current_stream(dev)
    ws = rtr.new_workspace(d, rtr.RTR_BF16, dev) if args.split else None

    # window occupancy before each chunk, known on the host from the schedule
    flops, count = [], 0
    for i in range(chunks):
        if i % every == 0:
            count = 0 if i == 0 else min(count, 1)
        flops.append(4 * d * H * stream_pairs_per_head(kpf, C, R + count))
        count = min(W, count + C)
    flops_total = sum(flops)

    def one_rollout(ev=None):
        for i in range(chunks):
            if i % every == 0:
                rk, rv = refs[(i // every) % P]
                rtr.rtr_kv_reset_ref(kv, rtr.RTR_REF_REPLACE, rk, rv, R, 0 if i == 0 else 1)
            q, k, v = pool[i % P]
            if ev is not None:
                ev[i][0].record(stream)
            rtr.rtr_attn_stream_step(kv, q, k, v, C, o=o, workspace=ws)
            if ev is not None:
                ev[i][1].record(stream)
            rtr.rtr_kv_append_evict(kv, k, v, C)

    mhz_before = clock_mhz(dev)
    clk = ClockSampler(dev, args.steps, every=1)
    nwarm = prewarm(one_rollout, dev, args.prewarm_s)
    for _ in range(args.warmup):
        one_rollout()
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for i in range(args.steps):
        e0 = torch.cuda.Event()
        e0.record(stream)
        one_rollout()
        clk.maybe(i, e0)
    torch.cuda.synchronize(dev)
    elapsed = time.perf_counter() - t0
    mhz_after = clock_mhz(dev)
    # one more rollout with events around each stream step, for the kernel time
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(chunks)]
    one_rollout(ev)
    torch.cuda.synchronize(dev)
    attn_s = sum(a.elapsed_time(b) for a, b in ev) * 1e-3

    ms_per_step = elapsed * 1e3 / args.steps
    frames = C * chunks
    achieved = flops_total / attn_s / 1e12
    out = {
        "metric": METRIC,
        "value": round(flops_total / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "rollout", "heads": H, "head_dim": d, "tokens_per_frame": kpf,
                   "chunk_frames": C, "window_frames": W, "ref_frames": R, "chunks": chunks,
                   "ref_swap_every": every, "keep_recent": 1},
        "latent_frames_per_s_per_layer": round(frames / (ms_per_step * 1e-3), 1),
        "ms_per_chunk": round(ms_per_step / chunks, 5),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": None,
            "kernel": "attn_fwd_bf16_d128" + ("" if ws is None else " (+ split-K when planned)"),
            "kernel_avg_us": round(attn_s / chunks * 1e6, 2),
            "algorithmic_flop_per_launch": round(flops_total / chunks),
        },
        "gpu": dict(device_info(dev), sclk_mhz_before_timed=mhz_before, sclk_mhz_after_timed=mhz_after,
                    sclk_mhz_during_timed=clk.summary(), prewarm_steps=nwarm, prewarm_s=args.prewarm_s),
    }
    rtr.rtr_kv_destroy(kv)
    if not args.no_cpu_baseline:
        x = gen.stream_inputs(kpf, H, d, C, W, R, "bf16", base_seed=0, wid=w["wid"])
        out["cpu_baseline"] = cpu_baseline("rollout_stream_step", x, w, args.cpu_heads)
        out["cpu_baseline"]["sample"] += " (one steady-state chunk of the rollout)"
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
