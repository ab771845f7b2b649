"""Benchmark of the 4-bit grouped-expert MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode|decode64|prefill512|prefill4096|stack40]

With no --workload, one process times every workload: the decode step (T=1)
is the headline line, and decode64, prefill512, prefill4096 and stack40 are
extra keys of the same JSON line, each with its own roofline and CPU baseline.

A step is one pass of the whole layer (routing, permute, gate/up + SwiGLU,
down + weighted combine + shared expert) over one batch of synthetic tokens,
through the C ABI entry point ``moe_layer``.  Inputs are resident in HBM before
timing starts.  Successive steps cycle through distinct weight sets drawn in
device memory, so a step does not find the previous steps' weights in the
256 MB last-level cache, and use fresh activations.  The headline workload is
one decode step (T=1) of the Qwen3.6-35B-A3B layer shape (H=2048, 256 experts,
top-8, shared expert, I=512).  After the timed region the decode path's
control words are read back: a device-side wait that timed out (workspace word
255) or a call counter that did not advance once per call ends the run with an
error.

Launch: the K timed steps are captured once into a HIP graph and replayed
(how an engine issues a fixed-shape layer step; ``--mode eager`` launches
them one by one instead).  The timed region carries no instrumentation.  Per-kernel durations
for the roofline come from an eager, instrumented run of the same K steps
through ``moe_layer_events`` (HIP events recorded on the launch stream around
every kernel; events inside a captured graph do not time kernels).

``roofline.traffic`` is the dominant kernel's HBM bytes per launch measured by
rocprofv3 counters (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter
reads for a plain copy of known size; ``--copy-calibration`` runs that copy).
The figures live in ``profiles/<kernel>_<workload>_pmc.txt`` together with the
SHA-256 of the kernel's source file; when the source has changed since, the
field is null.

Prints one JSON line.  ``cpu_baseline`` times the CPU oracle (single-threaded
C, pinned to one core) on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s (prefill T=512/4096), decode µs/layer; % HBM / MFMA peak"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense f16/bf16 MFMA, TFLOP/s

WORKLOADS = {
    # name: (config name, layers per step, bound of the dominant kernel, default weight sets)
    "decode": ("decode", 1, "hbm", 40),
    "decode64": ("decode64", 1, "hbm", 8),
    "prefill512": ("prefill512", 1, "hbm", 4),
    "prefill4096": ("prefill4096", 1, "mfma", 4),
    "stack40": ("stack40", 40, "mfma", 40),
    # one decode step (one token) through 40 layers in one launch of moe_decode_stack
    "decode_stack40": ("decode", 40, "hbm", 40),
    # decode attention of one token at 32K context (16 query / 2 KV heads, D = 128)
    "gqa32k": ("gqa32k", 1, "hbm", 12),
}


def expert_bytes(H, I, sb_bytes, group=64):
    """Packed codes + scales + biases of one expert's gate, up and down matrices."""
    mat = lambda N, K: N * K // 2 + 2 * N * (K // group) * sb_bytes  # noqa: E731
    return {"gate_up": 2 * mat(I, H), "down": mat(H, I)}


def stage_work(name, sh, T, touched, shared):
    """Algorithmic bytes and flops of one launch of a stage.

    touched: number of routed experts with at least one token; the shared expert
    is added when present.  Bytes count what the step must move: the touched
    experts' packed weights, scales and biases, the router, the activations read
    and the results written; no padding, no re-reads."""
    H, I, E, k = sh.H, sh.I, sh.E, sh.top_k
    sb = 2 if sh.sb_bf16 else 4
    eb = expert_bytes(H, I, sb)
    rows = T * k + (T if shared else 0)
    n_exp = touched + (1 if shared else 0)
    router = (E * H * 2 + T * H * 2, 2.0 * T * H * E)
    gate_up = (n_exp * eb["gate_up"] + T * H * 2 + rows * I * 2, 2.0 * rows * H * 2 * I)
    down = (n_exp * eb["down"] + rows * I * 2 + T * H * 4, 2.0 * rows * I * H)
    if name == "router":  # logits to the workspace
        return router[0] + T * E * 4, router[1]
    if name == "topk":  # logits in, routing out, float16 copy of x
        return T * E * 4 + T * k * 8 + T * H * 2 + T * H * 2, 0.0
    if name == "permute":
        return T * k * 4 * 2 + E * 8, 0.0
    if name == "gate_up":
        return gate_up
    if name == "down":  # rows written as float16 slot rows
        return (n_exp * eb["down"] + rows * I * 2 + rows * H * 2, 2.0 * rows * I * H)
    if name == "combine":
        return (rows * H * 2 + T * k * 4 + T * H * 4, 2.0 * T * k * H)
    if name == "decode_layer":  # the whole layer in one kernel: router + all touched experts + output
        return (router[0] + n_exp * (eb["gate_up"] + eb["down"]) + T * H * 4,
                router[1] + gate_up[1] + down[1])
    return 0, 0.0


# kernel name -> source file that holds it (for the counter figures' freshness)
KERNEL_SOURCES = {
    "decode_layer": "bit_expert_grouped_amd/csrc/decode.hip",
    "decode_stack": "bit_expert_grouped_amd/csrc/decode_stack.hip",
    "gqa_partial": "bit_expert_grouped_amd/csrc/gqa_decode.hip",
    "router": "bit_expert_grouped_amd/csrc/router.hip",
    "topk": "bit_expert_grouped_amd/csrc/router.hip",
    "permute": "bit_expert_grouped_amd/csrc/permute.hip",
    "gate_up": "bit_expert_grouped_amd/csrc/expert_gemm.hip",
    "down": "bit_expert_grouped_amd/csrc/expert_gemm.hip",
    "combine": "bit_expert_grouped_amd/csrc/misc.hip",
}


def source_sha(kernel):
    path = os.path.join(ROOT, KERNEL_SOURCES.get(kernel, ""))
    if not os.path.isfile(path):
        return None
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, if it is for the
    current source of the kernel; else None."""
    path = os.path.join(ROOT, "profiles", "%s_%s_pmc.txt" % (kernel, workload))
    if not os.path.isfile(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith((" ", "#", "$")):
            key, v = line.split(":", 1)
            vals[key.strip()] = v.strip()
    if vals.get("source_sha256") != source_sha(kernel):
        return None
    try:
        return int(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration():
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch

    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": 3}))


def cpu_baseline(cfg, T, seconds, layers=1):
    """Time the CPU oracle (single-threaded C, pinned to one core) on a bounded
    sample of the workload; tokens/s.

    Decode (T <= 4): whole oracle calls of T tokens.  Larger batches: oracle
    calls on 64-token sub-batches of the workload's tokens; each call routes its
    tokens and restores every expert they touch, so the per-token cost sits
    above that of one call over the whole batch.  For a layer stack the rate is
    per layer (every layer costs the same)."""
    import oracle

    import moe_synth

    pinned = _pin_one_core()
    try:
        w = moe_synth.layer_weights(cfg)
        n = T if T <= 4 else 64  # tokens per oracle call
        pool = 64 if T <= 4 else 256
        x_all = moe_synth.token_rows(cfg, pool)
        done_tokens, calls = 0, 0
        t0 = time.perf_counter()
        while True:
            lo = (calls * n) % pool
            oracle.moe_layer(w, x_all[lo:lo + n], cfg.shape.top_k)
            done_tokens += n
            calls += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    finally:
        _unpin(pinned)
    what = ("%d oracle calls of %d token(s) each" % (calls, n) if T <= 4 else
            "%d oracle calls on 64-token sub-batches of the T=%d batch (each call routes its tokens and restores "
            "every expert they touch)" % (calls, T))
    if layers > 1:
        what += "; one layer of the %d-layer stack, rate per layer" % layers
    return {"value": round(done_tokens / el, 4), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": "%s on one %s layer (H=%d, E=%d, top-%d, I=%d), %.1f s single-threaded, pinned to core %s"
                      % (what, cfg.name, cfg.shape.H, cfg.shape.E, cfg.shape.top_k, cfg.shape.I, el,
                         pinned[1] if pinned else "none"),
            "seconds": round(el, 2), "cpu": _cpu_model(), "nproc": os.cpu_count()}


def _pin_one_core():
    """Pin this process to one core of its allowed set; returns (old set, core) or None."""
    try:
        old = os.sched_getaffinity(0)
        core = max(old)
        os.sched_setaffinity(0, {core})
        return old, core
    except (AttributeError, OSError):
        return None


def _unpin(pinned):
    if pinned:
        try:
            os.sched_setaffinity(0, pinned[0])
        except OSError:
            pass


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def check_decode_words(ws, decode_calls_expected=None):
    """The decode path's control words after a run: the timeout flag (word 255)
    must be clear; the call counter (the high halves of the 32 64-bit words the
    decode workgroups count themselves in on, uint32 words 513 + 32 g) must
    agree and have advanced by the number of decode calls made, when that is
    known, and no call may be left half counted (words 512 + 32 g).  Raises on
    a violation."""
    import torch

    words = ws[:8192].view(torch.int32).cpu()
    counts = {int(words[513 + 32 * g]) for g in range(32)}
    flag = int(words[255])
    if len(counts) != 1 or any(int(words[512 + 32 * g]) != 0 for g in range(32)):
        raise RuntimeError("decode arrival words disagree after the run: %s" % sorted(counts))
    calls = counts.pop()
    if flag != 0:
        raise RuntimeError("a device-side wait of the decode kernel timed out (workspace word 255 = %d): "
                           "the timed outputs are invalid" % flag)
    if decode_calls_expected is not None and calls != decode_calls_expected:
        raise RuntimeError("decode call counter reads %d after %d decode calls" % (calls, decode_calls_expected))
    return calls


def run_workload(name, steps_arg, warmup_arg, args, with_cpu=True, cpu_seconds=None):
    """Time one workload; returns its record (the fields of the JSON line)."""
    import torch

    import bit_expert_grouped_amd as bem
    import moe_synth

    cfg_name, layers_per_step, bound, default_sets = WORKLOADS[name]
    cfg = moe_synth.CONFIGS[cfg_name]
    sh = cfg.shape
    T = sh.T
    big = T >= 512
    steps = steps_arg if steps_arg is not None else (20 if big else 200)
    warmup = warmup_arg if warmup_arg is not None else (3 if big else 20)
    n_sets = args.weight_sets or default_sets
    if layers_per_step > 1:
        n_sets = layers_per_step

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    alpha = moe_synth.zipf_alpha() if cfg.zipf else None
    tensors = [moe_synth.device_layer(sh, cfg.seed, l, dev, alpha) for l in range(n_sets)]
    if args.shared_gate:
        for l, t in enumerate(tensors):
            gbits = moe_synth.shared_expert_gate(cfg, l)
            t["shared_expert_gate"] = torch.from_numpy(gbits.view("int16")).to(dev).view(torch.bfloat16)
    if args.router_q8:
        for l, t in enumerate(tensors):
            r = moe_synth.router_q8(cfg, l)
            t["router"] = None
            t["router_q8"] = torch.from_numpy(r["router_q8"].view("int32")).to(dev)
            for key in ("router_scale", "router_bias"):
                v = r[key]
                t[key] = (torch.from_numpy(v.view("int16")).to(dev).view(torch.bfloat16) if v.dtype.itemsize == 2
                          else torch.from_numpy(v).to(dev))
    sets = [bem.LayerWeights(t) for t in tensors]
    n_x = min(steps + warmup, 64) if not big else 4
    xs = [moe_synth.device_tokens(sh, T, cfg.seed, i, dev) for i in range(n_x)]
    d = sets[0].dims(T, sh.top_k)
    ws = bem.workspace(d, dev)
    out = torch.empty(T, sh.H, dtype=torch.float32, device=dev)
    stages = bem.moe_layer_stages(d)
    is_decode = stages == ["decode_layer"]
    n_calls = steps * layers_per_step
    counts = torch.zeros(n_calls, sh.E, dtype=torch.int32, device=dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(n_calls)]
    mode = args.mode or "graph"
    torch.cuda.synchronize()

    # Pre-built argument tuples of the C entry points: the timed loop is one
    # foreign call per layer call.
    stream = torch.cuda.current_stream()
    lib = bem.lib()
    dref = ctypes.byref(d)
    for e in evs:
        for ev in e:
            ev.record()
    torch.cuda.synchronize()
    decode_calls = 0

    def call_args(i, li, s_handle, with_events, set_offset=0):
        w = sets[li % n_sets] if layers_per_step > 1 else sets[(i + set_offset) % n_sets]
        x = xs[i % n_x]
        c = i * layers_per_step + li
        base = (dref, ctypes.byref(w.struct), x.data_ptr(), out.data_ptr(), None, None, None, ws.data_ptr(),
                ws.numel(), s_handle)
        if not with_events:
            return base
        arr = (ctypes.c_void_p * len(evs[c]))(*[ev.cuda_event for ev in evs[c]])
        return base + (ctypes.cast(arr, ctypes.c_void_p), len(evs[c])), arr

    def run_eager(record):
        keep = []
        for i in range(steps):
            for li in range(layers_per_step):
                if record:
                    a, arr = call_args(i, li, stream.cuda_stream, True)
                    keep.append(arr)
                    st = lib.moe_layer_events(*a)
                else:
                    st = lib.moe_layer(*call_args(i, li, stream.cuda_stream, False))
                if st != 0:
                    raise bem.MoeError(st, "moe_layer")
        return keep

    # warm-up (eager)
    for i in range(warmup):
        for li in range(layers_per_step):
            st = lib.moe_layer(*call_args(i + 1000, li, stream.cuda_stream, False))
            if st != 0:
                raise bem.MoeError(st, "moe_layer")
    decode_calls += warmup * layers_per_step
    torch.cuda.synchronize()

    def capture(set_offset):
        """One HIP graph holding all K steps (weight sets shifted by set_offset)."""
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            prepared = [call_args(i, li, side.cuda_stream, False, set_offset)
                        for i in range(steps) for li in range(layers_per_step)]
            with torch.cuda.graph(g, stream=side):
                for a in prepared:
                    st = lib.moe_layer(*a)
                    if st != 0:
                        raise bem.MoeError(st, "moe_layer (capture)")
        torch.cuda.synchronize()
        return g

    plain = None
    if mode == "graph":
        # the timed graph runs weight sets 0..K-1; an untimed replay of it, then
        # one of a graph over the other sets, so that the timed replay finds its
        # weights evicted from the last-level cache (when there are 2K sets)
        plain = capture(0)
        plain.replay()
        torch.cuda.synchronize()
        if layers_per_step == 1 and n_sets > steps:
            other = capture(steps)
            other.replay()
            torch.cuda.synchronize()
            decode_calls += n_calls
        decode_calls += n_calls

    # ---- timed region: exactly K steps, no instrumentation ----
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_host0 = time.perf_counter()
    start.record()
    if plain is not None:
        plain.replay()
    else:
        for i in range(steps):
            for li in range(layers_per_step):
                st = lib.moe_layer(*call_args(i, li, stream.cuda_stream, False))
                if st != 0:
                    raise bem.MoeError(st, "moe_layer")
    stop.record()
    torch.cuda.synchronize()
    host_s = time.perf_counter() - t_host0
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / steps
    decode_calls += n_calls
    if is_decode:
        check_decode_words(ws, decode_calls)

    # ---- instrumented eager run of the same K steps: HIP events around every kernel ----
    _keep = run_eager(True)
    torch.cuda.synchronize()
    decode_calls += n_calls

    # per-stage durations
    stage_us = {st_name: 0.0 for st_name in stages}
    for e in evs:
        for j, st_name in enumerate(stages):
            stage_us[st_name] += e[j].elapsed_time(e[j + 1]) * 1000.0
    for st_name in stages:
        stage_us[st_name] /= n_calls
    # experts touched per call (outside the timed region: the same calls again,
    # with the per-expert counts requested)
    n_count = 0
    for i in range(min(steps, 16)):
        for li in range(layers_per_step if layers_per_step <= 4 else 4):
            a = call_args(i, li, stream.cuda_stream, False)
            st = lib.moe_layer(*(a[:6] + (counts[i * layers_per_step + li].data_ptr(),) + a[7:]))
            if st != 0:
                raise bem.MoeError(st, "moe_layer")
            n_count += 1
    torch.cuda.synchronize()
    decode_calls += n_count
    if is_decode:
        check_decode_words(ws, decode_calls)
    c = counts.cpu()
    c = c[(c.sum(dim=1) > 0)]
    touched = float((c > 0).sum(dim=1).double().mean())
    shared = sh.I_shared > 0
    dominant = max(stages, key=lambda st_name: stage_us[st_name])
    nbytes, flops = stage_work(dominant, sh, T, touched, shared)
    us_layer = total_ms * 1000.0 / n_calls
    # A layer that is one kernel: its duration is the timed region's per-call
    # time (back-to-back launches); else the instrumented per-kernel events.
    kernel_us = us_layer if len(stages) == 1 else stage_us[dominant]
    dur_s = kernel_us * 1e-6
    if bound == "hbm":
        achieved = nbytes / dur_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        achieved = flops / dur_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None}
    roof["traffic"] = measured_traffic(dominant, name)
    roof.update({"kernel": dominant, "kernel_us": round(kernel_us, 2),
                 "kernel_us_source": "timed region per call" if len(stages) == 1 else "instrumented events",
                 "algorithmic_bytes_per_launch": int(nbytes), "algorithmic_flops_per_launch": flops})

    tokens = T * steps * layers_per_step
    value = tokens / (total_ms / 1000.0)
    layer_bytes = sum(stage_work(st_name, sh, T, touched, shared)[0] for st_name in stages)
    layer_flops = sum(stage_work(st_name, sh, T, touched, shared)[1] for st_name in stages)
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": name, "T": T, "H": sh.H, "E": sh.E, "top_k": sh.top_k, "I": sh.I,
                   "I_shared": sh.I_shared, "layers_per_step": layers_per_step, "weight_sets": n_sets,
                   "weights": "affine 4-bit g64, bf16 scales/biases", "activations": "bf16",
                   "routing": "Zipf(1.1)-skewed logit offsets" if cfg.zipf else "random router weights",
                   "shared_expert_gate": bool(args.shared_gate), "router_q8": bool(args.router_q8),
                   "products": "f16 MFMA, fp32 accumulation; router bf16 MFMA; fp32 output"},
        "us_per_layer": round(us_layer, 3),
        "layer_hbm_frac": round(layer_bytes / (us_layer * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "layer_mfma_frac": round(layer_flops / (us_layer * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
        "touched_experts": round(touched, 2),
        "stages_us": {k_: round(v, 2) for k_, v in stage_us.items()},
        "stages_note": "per-kernel durations from HIP events around each kernel in an eager instrumented run of "
                       "the same K steps (the timed region itself carries no per-kernel events)",
        "host_wall_s": round(host_s, 4),
        "launch": mode,
        "timed_weight_sets": "0..%d of %d (the untimed replay just before ran sets %s)" % (
            min(steps, n_sets) - 1, n_sets,
            "%d..%d" % (steps, min(2 * steps, n_sets) - 1) if (mode == "graph" and layers_per_step == 1
                                                                and n_sets > steps) else "0..%d" % (n_sets - 1)),
        "roofline": roof,
    }
    if is_decode:
        rec["decode_timeout_flag"] = 0  # checked: a set flag raises before this point
    del sets, tensors, xs, ws, out, counts
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if with_cpu and not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(cfg, T, cpu_seconds or args.cpu_seconds, layers_per_step)
    return rec


def run_decode_stack(name, steps_arg, warmup_arg, args, with_cpu=True, cpu_seconds=None):
    """One decode step of one token through a stack of 40 layers per launch
    (moe_decode_stack: each layer reads the RMS-normalised residual stream and
    adds its output to it).  40 distinct layers (centred biases, the stack's
    weight recipe) are resident: a step streams every layer's touched experts
    (about 680 MB), far beyond the 256 MB last-level cache."""
    import torch

    import bit_expert_grouped_amd as bem
    import moe_synth

    cfg_name, n_layers, bound, _ = WORKLOADS[name]
    cfg = moe_synth.CONFIGS[cfg_name]
    sh = cfg.shape
    steps = steps_arg if steps_arg is not None else 20
    warmup = warmup_arg if warmup_arg is not None else 5
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stack = bem.StackWeights(moe_synth.device_stack(sh, cfg.seed, n_layers, dev))
    lib = bem.lib()
    d = stack.dims(sh.top_k)
    ws = bem.workspace(d, dev)
    n_x = min(steps + warmup, 32)
    xs = [moe_synth.device_tokens(sh, 1, cfg.seed, 5000 + i, dev) for i in range(n_x)]
    outs = [torch.empty(1, sh.H, dtype=torch.bfloat16, device=dev) for _ in range(n_x)]
    stream = torch.cuda.current_stream()

    def args_for(i, s_handle):
        return (ctypes.byref(d), ctypes.byref(stack.layer0.struct), None, ctypes.byref(stack.strides), n_layers,
                xs[i % n_x].data_ptr(), outs[i % n_x].data_ptr(), None, None, None, None, None, ws.data_ptr(),
                ws.numel(), s_handle)

    calls = 0
    for i in range(warmup):
        st = lib.moe_decode_stack(*args_for(i, stream.cuda_stream))
        if st != 0:
            raise bem.MoeError(st, "moe_decode_stack")
        calls += 1
    torch.cuda.synchronize()
    mode = args.mode or "graph"
    g = None
    if mode == "graph":
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            prepared = [args_for(i, side.cuda_stream) for i in range(steps)]
            with torch.cuda.graph(g, stream=side):
                for a in prepared:
                    st = lib.moe_decode_stack(*a)
                    if st != 0:
                        raise bem.MoeError(st, "moe_decode_stack (capture)")
        torch.cuda.synchronize()
        g.replay()  # one untimed replay
        torch.cuda.synchronize()
        calls += steps
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    if g is not None:
        g.replay()
    else:
        for i in range(steps):
            st = lib.moe_decode_stack(*args_for(i, stream.cuda_stream))
            if st != 0:
                raise bem.MoeError(st, "moe_decode_stack")
    stop.record()
    torch.cuda.synchronize()
    calls += steps
    total_ms = start.elapsed_time(stop)
    words = ws[:16384].view(torch.int32).cpu()
    if int(words[255]) != 0:
        raise RuntimeError("a device-side wait of the stack kernel timed out (workspace word 255)")
    if int(words[2048]) != calls * n_layers:
        raise RuntimeError("stack epoch reads %d after %d calls of %d layers" % (int(words[2048]), calls, n_layers))
    us_step = total_ms * 1000.0 / steps
    us_layer = us_step / n_layers
    nbytes, flops = stage_work("decode_layer", sh, 1, float(sh.top_k), sh.I_shared > 0)
    launch_bytes, launch_flops = nbytes * n_layers, flops * n_layers
    achieved = launch_bytes / (us_step * 1e-6) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic("decode_stack", name),
            "kernel": "decode_stack", "kernel_us": round(us_step, 2),
            "kernel_us_source": "timed region per launch (one launch per step)",
            "algorithmic_bytes_per_launch": int(launch_bytes), "algorithmic_flops_per_launch": launch_flops}
    rec = {
        "metric": METRIC, "value": round(n_layers * steps / (total_ms / 1000.0), 2), "unit": "token-layers/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(total_ms / steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": name, "T": 1, "H": sh.H, "E": sh.E, "top_k": sh.top_k, "I": sh.I,
                   "I_shared": sh.I_shared, "layers_per_step": n_layers, "weight_sets": n_layers,
                   "weights": "affine 4-bit g64, bf16 scales/biases, biases centred on the code midpoint",
                   "activations": "bf16 residual stream, RMS-normalised before each layer",
                   "products": "f16 dot products, fp32 accumulation; output sums in a fixed order"},
        "us_per_layer": round(us_layer, 3),
        "layer_hbm_frac": roof["frac"],
        "touched_experts": float(sh.top_k),
        "launch": mode,
        "roofline": roof,
    }
    del stack, xs, outs, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if with_cpu and not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(cfg, 1, cpu_seconds or args.cpu_seconds, n_layers)
    return rec


def gqa_bytes(shape, n):
    """Algorithmic bytes of one decode-attention call: every valid K and V row
    once (the packing reads each for all query heads of its KV head), q in, out."""
    return shape.B * shape.Hkv * n * shape.D * 2 * 2 + shape.B * shape.Hq * shape.D * (2 + 4) + shape.B * 4


def cpu_baseline_gqa(shape, seconds):
    """The oracle (single-threaded C, fp64, pinned to one core) on whole calls of
    the same attention workload; tokens/s."""
    import numpy as np

    import oracle

    import moe_synth

    q, k, v = moe_synth.attn_inputs(shape, 5)
    lens = np.full(shape.B, shape.S, dtype=np.int32)
    pinned = _pin_one_core()
    try:
        calls = 0
        t0 = time.perf_counter()
        while True:
            oracle.gqa_decode(q, k, v, lens)
            calls += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    finally:
        _unpin(pinned)
    return {"value": round(calls * shape.B / el, 4), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": "%d whole oracle calls (B=%d, %d query / %d KV heads, D=%d, %d cached rows), %.1f s "
                      "single-threaded, pinned to core %s" % (calls, shape.B, shape.Hq, shape.Hkv, shape.D, shape.S,
                                                              el, pinned[1] if pinned else "none"),
            "seconds": round(el, 2), "cpu": _cpu_model(), "nproc": os.cpu_count()}


def run_gqa(name, steps_arg, warmup_arg, args, with_cpu=True, cpu_seconds=None):
    """Decode attention of one token per sequence over a 32K-row KV cache
    (moe_gqa_decode).  Distinct caches are rotated (12 x 33.5 MB, past the
    256 MB last-level cache), so every step streams its K and V from HBM."""
    import torch

    import bit_expert_grouped_amd as bem
    import moe_synth

    shape = moe_synth.GQA32K
    n_sets = args.weight_sets or WORKLOADS[name][3]
    steps = steps_arg if steps_arg is not None else 20
    warmup = warmup_arg if warmup_arg is not None else 5
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sets = [moe_synth.device_attn(shape, 100 + i, dev) for i in range(n_sets)]
    lens = torch.full((shape.B,), shape.S, dtype=torch.int32, device=dev)
    d = bem.gqa_dims(shape.B, shape.Hq, shape.Hkv, shape.D, shape.S)
    ws = bem.gqa_workspace(d, dev)
    out = torch.empty(shape.B, shape.Hq, shape.D, dtype=torch.float32, device=dev)

    def call(i, events=None):
        q, k, v = sets[i % n_sets]
        bem.gqa_decode(q, k, v, lens, out=out, ws=ws, events=events)

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    mode = args.mode or "graph"
    g = None
    if mode == "graph":
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for i in range(steps):
                    call(i)
        torch.cuda.synchronize()
        g.replay()  # one untimed replay
        torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    if g is not None:
        g.replay()
    else:
        for i in range(steps):
            call(i)
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    # the two kernels, timed with events on the launch stream in an eager run of the same steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        call(i, evs[i])
    torch.cuda.synchronize()
    part_us = sum(e[0].elapsed_time(e[1]) for e in evs) * 1000.0 / steps
    merge_us = sum(e[1].elapsed_time(e[2]) for e in evs) * 1000.0 / steps
    us_call = total_ms * 1000.0 / steps
    nbytes = gqa_bytes(shape, shape.S)
    # with the merge in the same launch a call is one kernel, timed by the
    # graph's timed region per call; otherwise the partial pass alone, by its events
    fused = bem.gqa_decode_kernels(d) == 1
    kern_us = us_call if fused else part_us
    achieved = nbytes / (kern_us * 1e-6) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic("gqa_partial", name),
            "kernel": "gqa_partial", "kernel_us": round(kern_us, 2),
            "kernel_us_source": ("timed region per call (one kernel per call: partials and their merge)" if fused
                                 else "HIP events around the kernel on its stream, eager run of the same steps"),
            "algorithmic_bytes_per_launch": int(nbytes)}
    rec = {
        "metric": METRIC, "value": round(shape.B * steps / (total_ms / 1000.0), 2), "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(total_ms / steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": name, "B": shape.B, "n_q_heads": shape.Hq, "n_kv_heads": shape.Hkv,
                   "head_dim": shape.D, "context": shape.S, "kv_sets": n_sets,
                   "inputs": "q, K, V ~ N(0, 1) in bf16, scale 1/sqrt(D)",
                   "products": "bf16 MFMA, fp32 accumulation; probabilities rounded to bf16"},
        "us_per_call": round(us_call, 3),
        "us_per_layer": round(us_call, 3),
        "stages_us": ({"gqa_partial_and_merge_eager": round(part_us, 2)} if fused else
                      {"gqa_partial": round(part_us, 2), "gqa_merge": round(merge_us, 2)}),
        "call_hbm_frac": round(nbytes / (us_call * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "launch": mode,
        "roofline": roof,
    }
    del sets, ws, out
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if with_cpu and not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_gqa(shape, cpu_seconds or args.cpu_seconds)
    return rec


# workloads the default run times beside the headline decode line
EXTRA_WORKLOADS = ("decode_stack40", "gqa32k", "decode64", "prefill512", "prefill4096", "stack40")
EXTRA_KEYS = ("value", "unit", "ms_per_step", "us_per_layer", "us_per_call", "call_hbm_frac", "steps", "warmup", "config", "layer_hbm_frac",
              "layer_mfma_frac", "touched_experts", "stages_us", "launch", "timed_weight_sets", "roofline",
              "cpu_baseline")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default=None, choices=sorted(WORKLOADS),
                    help="time one workload only (default: the decode headline line plus every other "
                         "workload as extra keys)")
    ap.add_argument("--weight-sets", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--extra-cpu-seconds", type=float, default=8.0,
                    help="oracle seconds for each extra workload of the default run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 256 MiB device copy (three times) for counter calibration")
    ap.add_argument("--shared-gate", action="store_true",
                    help="give the shared expert a sigmoid gate vector (an optional checkpoint detail; the "
                         "configs have none)")
    ap.add_argument("--router-q8", action="store_true",
                    help="store the router as 8-bit codes in the MLX affine layout (an optional checkpoint "
                         "detail; the configs use a bf16 router)")
    ap.add_argument("--mode", choices=("eager", "graph"), default=None,
                    help="graph: replay one HIP graph holding the K timed steps (default); "
                         "eager: one foreign call per layer call")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the layer would shard by tokens or by experts; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import bit_expert_grouped_amd as bem

    bem.lib()
    def run(name, **kw):
        fn = (run_decode_stack if name.startswith("decode_stack") else run_gqa if name.startswith("gqa")
              else run_workload)
        return fn(name, args.steps, args.warmup, args, **kw)

    if args.workload is not None:
        print(json.dumps(run(args.workload)))
        return
    # default: the decode headline line, every other workload as an extra key
    rec = run("decode")
    for name in EXTRA_WORKLOADS:
        sub = run(name, cpu_seconds=args.extra_cpu_seconds)
        rec[name] = {k_: sub[k_] for k_ in EXTRA_KEYS if k_ in sub}
        print("bench: %s %.3f us/layer" % (name, sub["us_per_layer"]), file=sys.stderr, flush=True)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
