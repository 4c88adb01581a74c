"""Benchmark: MoE-layer tokens/s on one MI355X, with the dominant kernel's roofline
fraction and the fp64 oracle timed on the host cores beside it.

A step is one moe_layer_forward (gate, dispatch, expert FFN, combine) over one
batch of seeded synthetic tokens, inputs and weights resident in HBM. The
default workload is the 350M+MoE-128 decode step (8 tokens, hidden 1024, FFN
4096, 128 experts, top-1, capacity factor 1.0, fp16). Steps rotate over 64 token
batches and over several independent weight sets (layers of a deeper stack),
so a step does not find the previous step's experts in the 256 MB Infinity
Cache: every active expert's weights come from HBM, as in a real decode pass.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from mixture_experts_transformer_moe_amd import binding as B  # noqa: E402
from mixture_experts_transformer_moe_amd import workloads as W  # noqa: E402

METRIC = "MoE-layer tokens/sec at 1 GPU + % of HBM BW (decode) / % MFMA peak (prefill)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix peak, TFLOP/s


# ---------------------------------------------------------------- HIP events via the runtime torch already loaded
class _Hip:
    def __init__(self):
        self.L = ctypes.CDLL("libamdhip64.so")
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        if self.L.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        if self.L.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, e):
        self.L.hipEventDestroy(e)


def expert_unit_bytes(shape) -> int:
    """Algorithmic bytes of one active expert: its W1, b1, W2, b2, read once."""
    s = 4 if shape.dtype == "f32" else 2
    return (2 * shape.H * shape.F + shape.F + shape.H) * s


def layer_bytes(shape, n_active: int) -> int:
    """Algorithmic bytes of the whole layer: active experts once, the gate, x and y."""
    s = 4 if shape.dtype == "f32" else 2
    b = n_active * expert_unit_bytes(shape) + shape.E * shape.H * s + 2 * shape.T * shape.H * s
    if shape.zipf_s is not None:
        b += 4 * shape.E
    if shape.residual:
        b += expert_unit_bytes(shape)
    return b


def layer_flops(shape, rows: int) -> int:
    f = 2 * shape.T * shape.H * shape.E + 4 * shape.H * shape.F * rows
    if shape.residual:
        f += 4 * shape.H * shape.F * shape.T
    return f


# the grouped-GEMM workloads measured beside the decode headline, in one process
PREFILL_CONFIGS = ["prefill_1p3b_moe128", "prmoe_residual", "share_24b_moe128"]
RIDGE = MFMA_F16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)   # flop per byte where the two roofs meet


def graded_bound(shape, n_active: float, rows: float) -> str:
    """The roof a layer is graded against: the matrix cores once its arithmetic
    intensity (algorithmic flops per algorithmic byte) reaches half the ridge,
    else HBM bandwidth."""
    return "mfma" if layer_flops(shape, rows) / layer_bytes(shape, n_active) >= RIDGE / 2 else "hbm"


class ClockSampler:
    """Samples the GPU's graphics clock (amdsmi, by the device's PCI address)
    from a background thread, keeping the samples taken while `active` is set
    (the timed passes)."""

    def __init__(self, period_s: float = 0.01):
        import threading
        self.mhz, self.err, self.period = [], None, period_s
        self.source = "amdsmi"
        self._stop = threading.Event()
        self.active = threading.Event()
        self._handle = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            pr = torch.cuda.get_device_properties(0)
            bdf = f"{pr.pci_domain_id:04x}:{pr.pci_bus_id:02x}:{pr.pci_device_id:02x}.0"
            self._smi = amdsmi
            self._handle = amdsmi.amdsmi_get_processor_handle_from_bdf(bdf)
            self._read()
        except Exception as e:          # monitoring only: report why it is missing
            self.err = f"{type(e).__name__}: {e}"[:160]
            self._handle = None
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self) -> float:
        """The graphics clock in MHz from the firmware's metrics table (the
        highest per-XCD value when it lists them), else the clock info."""
        try:
            m = self._smi.amdsmi_get_gpu_metrics_info(self._handle)
            for key in ("current_gfxclks", "current_gfxclk", "average_gfxclk_frequency"):
                v = m.get(key)
                if isinstance(v, (list, tuple)):
                    v = max([float(c) for c in v if isinstance(c, (int, float)) and 0 < c < 65535] or [0])
                if isinstance(v, (int, float)) and 0 < v < 65535:
                    self.source = f"amdsmi gpu metrics {key}"
                    return float(v)
        except Exception:
            pass
        info = self._smi.amdsmi_get_clock_info(self._handle, self._smi.AmdSmiClkType.GFX)
        self.source = "amdsmi clock info gfx clk"
        return float(info["clk"])

    def _run(self):
        while not self._stop.is_set():
            if self.active.wait(0.05):
                self.sample_now()
                self._stop.wait(self.period)

    def sample_now(self):
        """One reading (also called from the timing loop itself, for passes
        shorter than the thread's period)."""
        if self._handle is None:
            return
        try:
            self.mhz.append(self._read())
        except Exception as e:
            self.err = f"{type(e).__name__}: {e}"[:160]

    def __enter__(self):
        if self._handle is not None:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._handle is not None:
            self._thread.join(timeout=2)

    def summary(self) -> dict:
        if not self.mhz:
            return {"mhz_median": None, "samples": 0, "source": "amdsmi gfx clock", "error": self.err}
        v = np.array(self.mhz)
        if np.median(v) < 500:   # below the part's lowest clock level: not a live reading of this device
            return {"mhz_median": None, "samples": int(v.size), "source": self.source,
                    "error": f"reads {float(np.median(v)):.0f} MHz while the passes run, below the part's "
                             "500 MHz minimum: not a live clock (the clock under load is in the counter "
                             "summaries, from GRBM_GUI_ACTIVE)"}
        return {"mhz_median": float(np.median(v)), "mhz_min": float(v.min()), "mhz_max": float(v.max()),
                "samples": int(v.size), "source": self.source + ", sampled during the timed, graph and per-step "
                                                                "passes"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="decode_350m_moe128", choices=sorted(W.WORKLOADS))
    ap.add_argument("--store-slots", type=int, default=None,
                    help="keep the experts in pinned host memory with this many device slots (expert store)")
    ap.add_argument("--stack", default=None, choices=sorted(W.STACKS),
                    help="time a stack of MoE layers chained through their outputs instead of one layer")
    ap.add_argument("--layers", type=int, default=None, help="independent weight sets rotated per step")
    ap.add_argument("--batches", type=int, default=64, help="token batches rotated per step")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle CPU baseline")
    ap.add_argument("--config-cpu-seconds", type=float, default=6.0,
                    help="budget of the oracle CPU baseline of each extra grouped-GEMM workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="time only --workload (no extra grouped-GEMM workloads in the same run)")
    ap.add_argument("--one-launch", action="store_true",
                    help="decode path: both expert products in one launch (MOE_FLAG_DECODE_ONE_LAUNCH)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the eager launches only (no graph replay of the K steps)")
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="skip the pass that times the expert kernels with launch-recorded events")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="after timing, copy a buffer of this size 3 times (reference kernel for HBM counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library runs the layer on one GPU's expert share "
              "(no collectives); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.stack:
        return run_stack(args)
    torch.cuda.set_device(0)
    shape = W.WORKLOADS[args.workload]
    if args.one_launch:
        shape = shape.with_(one_launch=True)
    clock = ClockSampler()
    with clock:
        head = run_layer(shape, args, cpu_budget=0.0 if args.no_cpu_baseline else args.cpu_seconds,
                         store_slots=args.store_slots, clock=clock)
    torch.cuda.empty_cache()

    configs = {}
    if not args.no_configs and args.workload == "decode_350m_moe128" and args.store_slots is None \
            and not args.one_launch:
        # the same decode workload with both expert products in one launch
        with ClockSampler() as ck:
            r = run_layer(shape.with_(one_launch=True), args, cpu_budget=0.0, clock=ck)
        configs["decode_350m_moe128_one_launch"] = config_entry(r, ck.summary())
        torch.cuda.empty_cache()
        print(f"[bench] decode, one launch: {r['ms_per_step'] * 1e3:.2f} us/step", file=sys.stderr, flush=True)
        for name in PREFILL_CONFIGS:
            with ClockSampler() as ck:
                r = run_layer(W.WORKLOADS[name], args, cpu_budget=0.0 if args.no_cpu_baseline
                              else args.config_cpu_seconds, clock=ck)
            configs[name] = config_entry(r, ck.summary())
            torch.cuda.empty_cache()
            print(f"[bench] {name}: {r['ms_per_step'] * 1e3:.1f} us/step, graded {configs[name]['graded']}",
                  file=sys.stderr, flush=True)

    out = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "timing": head["timing"],
        "eager_ms_per_step": head["eager_ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": shape.dtype,
        "data": "synthetic",
        "plan": head["plan"],
        "config": head["config"],
        "roofline": head["roofline"],
        **({"store": head["store"]} if head.get("store") else {}),
        "layer": head["layer"],
        "step_us": head["step_us"],
        "clock": clock.summary(),
    }
    if "cpu_baseline" in head:
        out["cpu_baseline"] = head["cpu_baseline"]
    if configs:
        out["configs"] = configs
    if args.copy_probe_mb:
        n = args.copy_probe_mb * (1 << 20) // 2
        src = torch.empty(n, dtype=torch.float16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    print(json.dumps(out), flush=True)


def config_entry(r: dict, clock: dict) -> dict:
    """The compact record of one extra workload in the headline line."""
    lay = r["layer"]
    bound = lay["graded_bound"]
    frac = lay["mfma_frac"] if bound == "mfma" else lay["hbm_frac"]
    e = {"tokens_per_s": r["tokens_per_s"], "ms_per_step": r["ms_per_step"], "timing": r["timing"],
         "eager_ms_per_step": r["eager_ms_per_step"], "step_us": r["step_us"],
         "f_hbm": lay["hbm_frac"], "f_mfma": lay["mfma_frac"],
         "graded": {"bound": bound, "frac": float(frac),
                    "target": 0.5 if bound == "mfma" else 0.7},
         "config": r["config"], "plan": r["plan"], "roofline": r["roofline"],
         "layer": {k: lay[k] for k in ("algorithmic_bytes", "algorithmic_flops", "mean_active_experts",
                                       "mean_rows", "phase_us")},
         "clock": clock}
    if "cpu_baseline" in r:
        e["cpu_baseline"] = r["cpu_baseline"]
    return e


def run_layer(shape, args, *, cpu_budget: float, store_slots=None, clock=None) -> dict:
    """Times moe_layer_forward on one workload: the K timed steps (value), the
    same steps with an event pair around each (p10 / p50 / p90), the same
    steps each after a 1 GiB write that evicts the caches (cold), then the
    phase-event and kernel-event passes that time the dominant kernel."""
    n_layers = args.layers if args.layers else (4 if shape.T <= 64 else 1)
    n_batches = args.batches if shape.T <= 64 else min(args.batches, 2)
    dev = "cuda"
    stream = torch.cuda.current_stream()

    # ---- inputs, resident in HBM before any timing
    weights = [W.make_weights(shape, seed=s, device=dev) for s in range(n_layers)]
    xs = [W.make_x(shape, seed=1000 + b, device=dev) for b in range(n_batches)]
    stores = []
    if store_slots is not None:
        # experts in pinned host memory, a device cache of store_slots experts per layer
        for w in weights:
            st_ = B.ExpertStore(shape, store_slots)
            st_.fill({k: w[k].cpu() for k in ("w1", "b1", "w2", "b2")})
            stores.append(st_)
    layers = [B.MoELayer(shape, w, store=stores[i] if stores else None) for i, w in enumerate(weights)]
    ws = layers[0].ws
    for L in layers[1:]:
        L.ws = ws
    y = torch.empty_like(xs[0])
    torch.cuda.synchronize()

    # routing statistics per (layer, batch), from the gate and dispatch entry points,
    # read back once outside the timed regions (they size the algorithmic bytes)
    desc = layers[0].desc
    R_max = B.moe_max_rows(desc)
    n_active = np.zeros((n_layers, n_batches), dtype=np.int64)
    rows = np.zeros((n_layers, n_batches), dtype=np.int64)
    idx = torch.empty((shape.T, shape.k), dtype=torch.int32, device=dev)
    tw = torch.empty((shape.T, shape.k), dtype=torch.float32, device=dev)
    demand = torch.empty(shape.E, dtype=torch.int32, device=dev)
    offsets = torch.empty(shape.E_loc + 1, dtype=torch.int32, device=dev)
    slot_token = torch.empty(max(R_max, 1), dtype=torch.int32, device=dev)
    token_slot = torch.empty((shape.T, shape.k), dtype=torch.int32, device=dev)
    active_sets = {}
    demand_sum = np.zeros((n_layers, shape.E), dtype=np.int64)
    for li in range(n_layers):
        for bi in range(n_batches):
            B.moe_gate(desc, xs[bi], weights[li]["gate_w"], weights[li]["gate_b"], idx, tw, None, ws)
            B.moe_dispatch(desc, idx, xs[bi], demand, offsets, slot_token, token_slot, None, ws)
            off = offsets.cpu().numpy()
            n_active[li, bi] = int((np.diff(off) > 0).sum())
            rows[li, bi] = int(off[-1])
            active_sets[li, bi] = np.nonzero(np.diff(off) > 0)[0]
            demand_sum[li] += demand.cpu().numpy()
    store_info = None
    if stores:
        # residency from the demand of all batches, fixed during the timed steps
        copied = [st_.update(np.minimum(demand_sum[li], 2**31 - 1).astype(np.int32), stream)
                  for li, st_ in enumerate(stores)]
        res = [st_.residency() for st_ in stores]
        hits = [np.mean(res[li][active_sets[li, bi]] >= 0) if len(active_sets[li, bi]) else 1.0
                for li in range(n_layers) for bi in range(n_batches)]
        host_experts = np.mean([np.sum(res[li][active_sets[li, bi]] < 0)
                                for li in range(n_layers) for bi in range(n_batches)])
        store_info = {"slots": store_slots, "experts_copied": int(sum(copied)),
                      "resident_hit_rate": round(float(np.mean(hits)), 4),
                      "host_read_experts_per_step": round(float(host_experts), 3),
                      "host_read_bytes_per_step": int(host_experts * expert_unit_bytes(shape))}
    del idx, tw, demand, offsets, slot_token, token_slot
    torch.cuda.synchronize()

    def lb(i):
        return i % n_layers, (i // n_layers) % n_batches

    def step(i, events=None):
        li, bi = lb(i)
        layers[li].forward(xs[bi], y, stream, events=events)

    print(f"[bench] {shape.name}: inputs ready, routing stats taken ({n_layers} weight sets x {n_batches} batches)",
          file=sys.stderr, flush=True)
    # ---- warmup, then exactly K timed steps
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    if clock:
        clock.active.set()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
        if clock and i % 8 == 7:
            clock.sample_now()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / args.steps
    tokens_per_s = shape.T * args.steps / (ms_total / 1e3)
    print(f"[bench] {shape.name}: timed pass done: {ms_per_step * 1e3:.2f} us/step", file=sys.stderr, flush=True)

    # ---- the same K steps captured once in a HIP graph and replayed: the GPU's
    # time for them without the host's launch cost (a decode step is ~30 us of
    # GPU work, the same order as the Python + runtime cost of enqueuing it)
    graph_ms = None
    if not args.no_graph and not stores:
        side = torch.cuda.Stream()      # default priority, like every stream here
        side.wait_stream(stream)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            for i in range(args.steps):
                li, bi = lb(i)
                layers[li].forward(xs[bi], y)     # the capture stream is current here
        graph.replay()                            # warm replay
        torch.cuda.synchronize()
        if clock:
            clock.active.set()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        if clock:
            clock.active.clear()
        graph_ms = g0.elapsed_time(g1) / args.steps
        del graph
        print(f"[bench] {shape.name}: graph replay {graph_ms * 1e3:.2f} us/step", file=sys.stderr, flush=True)

    hip = _Hip()
    # ---- per-step distribution: an event pair around each step (same steps, same stream)
    pe0 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    pe1 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for i in range(args.warmup):
        step(i)
    for i in range(args.steps):
        pe0[i].record(stream)
        step(i)
        pe1[i].record(stream)
    torch.cuda.synchronize()
    if clock:
        clock.active.clear()
    per_step = np.array([a.elapsed_time(b) for a, b in zip(pe0, pe1)]) * 1e3
    # ---- cold: before each step write 1 GiB (evicts the L2s and the 256 MB Infinity Cache)
    flush = torch.empty(1 << 29, dtype=torch.float16, device=dev)
    for i in range(args.steps):
        flush.fill_(float(i & 7))
        pe0[i].record(stream)
        step(i)
        pe1[i].record(stream)
    torch.cuda.synchronize()
    cold = np.array([a.elapsed_time(b) for a, b in zip(pe0, pe1)]) * 1e3
    del flush
    step_us = {"p10": round(float(np.percentile(per_step, 10)), 2), "p50": round(float(np.median(per_step)), 2),
               "p90": round(float(np.percentile(per_step, 90)), 2),
               "cold_p50": round(float(np.median(cold)), 2),
               "note": "event pair around each of the K steps (warm: the steps rotate weight sets and batches as in "
                       "the timed pass); cold: each step after a 1 GiB write that evicts the L2s and the "
                       "Infinity Cache"}

    # ---- phase events (same stream): gate, dispatch, the two expert kernels
    # (W1 kernel "up", W2 kernel "down"), combine
    names = ["gate", "dispatch", "up", "down", "combine"]
    pairs = [("gate_begin", "gate_end"), ("dispatch_begin", "dispatch_end"), ("ffn_begin", "ffn_split"),
             ("ffn_split", "ffn_end"), ("combine_begin", "combine_end")]
    fields = [f for f, _ in B.PhaseEvents._fields_]
    evs = [{f: hip.event() for f in fields} for _ in range(args.steps)]
    for i in range(args.warmup):
        step(i)
    for i in range(args.steps):
        step(i, B.PhaseEvents(**{f: e.value for f, e in evs[i].items()}))
    torch.cuda.synchronize()
    phase_ms = {n: 0.0 for n in names}
    s_w = 4 if shape.dtype == "f32" else 2
    HF = shape.H * shape.F
    win_bytes = {"up": 0, "down": 0}
    win_flops = {"up": 0, "down": 0}
    units = 0
    for i in range(args.steps):
        for n, (a, b) in zip(names, pairs):
            phase_ms[n] += hip.elapsed_ms(evs[i][a], evs[i][b])
        li, bi = lb(i)
        na, nr = int(n_active[li, bi]), int(rows[li, bi])
        units += na
        win_bytes["up"] += na * (HF + shape.F) * s_w
        win_bytes["down"] += na * (HF + shape.H) * s_w + ((2 * HF + shape.F + shape.H) * s_w if shape.residual else 0)
        win_flops["up"] += 2 * HF * nr + (2 * HF * shape.T if shape.residual else 0)
        win_flops["down"] += 2 * HF * nr + (2 * HF * shape.T if shape.residual else 0)
    for d in evs:
        for e in d.values():
            hip.destroy(e)
    # ---- the expert kernels timed by their own dispatch (start / end timestamps
    # of the launch itself, no queue packets between kernels)
    plan = B.moe_layer_plan(desc)
    one_launch = bool(plan["experts_one_launch"])
    if one_launch:   # both products in the W1 window's one launch
        win_bytes = {"up": win_bytes["up"] + win_bytes["down"], "down": 0}
        win_flops = {"up": win_flops["up"] + win_flops["down"], "down": 0}
    kern_ms = {"up": phase_ms["up"], "down": phase_ms["down"]}
    kernel_events = not args.no_kernel_events
    if kernel_events:
        kf = ("up_start", "up_stop") if one_launch else ("up_start", "up_stop", "down_start", "down_stop")
        kev = [{f: hip.event() for f in kf} for _ in range(args.steps)]
        for i in range(args.warmup):
            step(i)
        for i in range(args.steps):
            step(i, B.PhaseEvents(**{f: e.value for f, e in kev[i].items()}))
        torch.cuda.synchronize()
        kern_ms = {"up": 0.0, "down": 0.0}
        for i in range(args.steps):
            kern_ms["up"] += hip.elapsed_ms(kev[i]["up_start"], kev[i]["up_stop"])
            if not one_launch:
                kern_ms["down"] += hip.elapsed_ms(kev[i]["down_start"], kev[i]["down_stop"])
        for d in kev:
            for e in d.values():
                hip.destroy(e)
    dense_inside = bool(plan["dense_in_expert_kernels"])
    if shape.residual:
        if dense_inside:
            # the MLP's first product runs in the W1 launch, its second in the W2 launch
            win_bytes["up"] += (HF + shape.F) * s_w * args.steps
            win_bytes["down"] -= (HF + shape.F) * s_w * args.steps
        else:
            # the MLP's two launches follow the W2 kernel: the phase window is the unit
            kern_ms["down"] = phase_ms["down"]
            win_flops["up"] -= 2 * HF * shape.T * args.steps
            win_flops["down"] += 2 * HF * shape.T * args.steps
    kern = max(("up", "down"), key=lambda n: kern_ms[n])
    k_s = kern_ms[kern] / 1e3
    achieved_gbs = win_bytes[kern] / k_s / 1e9
    achieved_tflops = win_flops[kern] / k_s / 1e12
    mean_active = float(n_active.mean())
    mean_rows = float(rows.mean())
    # the layer's algorithmic work over the timed steps (the pairs they visit)
    steps_active = np.mean([n_active[lb(i)] for i in range(args.steps)])
    steps_rows = np.mean([rows[lb(i)] for i in range(args.steps)])
    lay_b = layer_bytes(shape, steps_active)
    lay_f = layer_flops(shape, steps_rows)
    bound = graded_bound(shape, steps_active, steps_rows)
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved_gbs / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        roof = {"bound": "mfma", "achieved": round(achieved_tflops, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved_tflops / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None}
    if kern == "up" and one_launch:
        unit_b = (2 * HF + shape.F + shape.H) * s_w
        unit_f = 4 * HF
        kname = ("expert FFN kernel (routing, h = GeLU(x W1^T + b1), y = h W2^T + b2"
                 + (" and the top-1 combine" if plan["combine_in_expert_kernel"] else "") + " in one launch)")
    elif kern == "up":
        unit_b = (HF + shape.F) * s_w
        unit_f = 2 * HF
        kname = "expert W1 kernel (h = GeLU(x W1^T + b1))"
    else:
        unit_b = (HF + shape.H) * s_w
        unit_f = 2 * HF
        kname = "expert W2 kernel (y = h W2^T + b2)"
    if shape.residual:
        kname += " + dense MLP " + ("tiles in the same launch" if dense_inside else "launches after it")
    roof.update(kernel=kname,
                avg_launch_us=round(kern_ms[kern] * 1e3 / args.steps, 2),
                timing=("kernel dispatch start/end events" if kernel_events and (dense_inside or not shape.residual
                                                                               or kern == "up")
                        else "phase events around the kernel window"),
                bytes_per_launch=int(win_bytes[kern] / args.steps),
                flops_per_launch=int(win_flops[kern] / args.steps),
                unit_bytes=unit_b, unit_flops_per_row=unit_f,
                units_per_launch=round(units / args.steps, 3),
                rows_per_launch=round(float(steps_rows), 2),
                frac_hbm=round(achieved_gbs / HBM_PEAK_GBS, 4),
                frac_mfma=round(achieved_tflops / MFMA_F16_PEAK_TFLOPS, 4),
                kernels_us={n: round(v * 1e3 / args.steps, 2) for n, v in kern_ms.items()},
                ffn_phase={"us": round((kern_ms["up"] + kern_ms["down"]) * 1e3 / args.steps, 2),
                           "GB/s": round((win_bytes["up"] + win_bytes["down"]) /
                                         ((kern_ms["up"] + kern_ms["down"]) / 1e3) / 1e9, 1)})
    roof["traffic"] = measured_traffic(shape.name + ("_one_launch" if shape.one_launch else ""), kern)

    # value: the graph replay of the K steps when taken (the eager rate is
    # reported beside it and depends on the host's launch speed)
    eager_ms = ms_per_step
    if graph_ms is not None:
        ms_per_step = graph_ms
        tokens_per_s = shape.T / (graph_ms / 1e3)
    res = {
        "tokens_per_s": round(tokens_per_s, 1),
        "ms_per_step": round(ms_per_step, 5),
        "timing": ("K steps replayed from one captured HIP graph" if graph_ms is not None
                   else "K steps launched eagerly"),
        "eager_ms_per_step": round(eager_ms, 5),
        "step_us": step_us,
        "plan": plan,
        "config": {"workload": shape.name + ("_one_launch" if shape.one_launch else ""), "tokens": shape.T,
                   "hidden": shape.H, "ffn": shape.F,
                   "experts": shape.E, "local_experts": shape.E_loc, "first_local_expert": shape.e_lo,
                   "top_k": shape.k, "capacity_factor": shape.cf, "mlp_type": shape.mlp_type,
                   "zipf_s": shape.zipf_s, "weight_sets": n_layers, "token_batches": n_batches,
                   "parallelism": "one GPU"},
        "roofline": roof,
        "layer": {"hbm_frac": round(lay_b / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                  "mfma_frac": round(lay_f / (ms_per_step / 1e3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                  "graded_bound": bound,
                  "algorithmic_bytes": int(lay_b), "algorithmic_flops": int(lay_f),
                  "mean_active_experts": round(float(steps_active), 3), "mean_rows": round(float(steps_rows), 2),
                  "all_pairs_mean_active_experts": round(mean_active, 3),
                  "phase_us": {n: round(v * 1e3 / args.steps, 2) for n, v in phase_ms.items()},
                  "wall_s": round(wall, 3)},
    }
    if store_info:
        res["store"] = store_info
    print(f"[bench] {shape.name}: event passes done", file=sys.stderr, flush=True)
    if cpu_budget > 0:
        res["cpu_baseline"] = cpu_baseline(shape, weights[0], xs, cpu_budget)
    for st_ in stores:
        st_.close()
    del layers, weights, xs, y, ws
    return res


def run_stack(args):
    """A stack of MoE layers, each layer's output feeding the next; a step pushes
    one token batch through every layer. Token batches rotate as in the
    single-layer run; the algorithmic bytes of a step sum each layer's (active
    experts, dense MLP, gate, x and y) with the active-expert counts read once,
    outside the timed region, from the gate and dispatch entry points on the
    chained inputs."""
    shapes = W.STACKS[args.stack]
    T = shapes[0].T
    n_batches = args.batches if T <= 64 else min(args.batches, 2)
    dev = "cuda"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    layers = [B.MoELayer(sh, W.make_weights(sh, seed=i, device=dev)) for i, sh in enumerate(shapes)]
    xs = [W.make_x(shapes[0], seed=1000 + b, device=dev) for b in range(n_batches)]
    bufs = [torch.empty_like(xs[0]) for _ in range(2)]
    torch.cuda.synchronize()

    n_active = np.zeros((len(layers), n_batches), dtype=np.int64)
    for bi in range(n_batches):
        x = xs[bi]
        for li, L in enumerate(layers):
            sh = L.shape
            R = max(B.moe_max_rows(L.desc), 1)
            idx = torch.empty((T, sh.k), dtype=torch.int32, device=dev)
            tw = torch.empty((T, sh.k), dtype=torch.float32, device=dev)
            demand = torch.empty(sh.E, dtype=torch.int32, device=dev)
            offsets = torch.empty(sh.E_loc + 1, dtype=torch.int32, device=dev)
            st = torch.empty(R, dtype=torch.int32, device=dev)
            ts = torch.empty((T, sh.k), dtype=torch.int32, device=dev)
            B.moe_gate(L.desc, x, L.weights["gate_w"], L.weights["gate_b"], idx, tw, None, L.ws)
            B.moe_dispatch(L.desc, idx, x, demand, offsets, st, ts, None, L.ws)
            n_active[li, bi] = int((np.diff(offsets.cpu().numpy()) > 0).sum())
            y = bufs[li % 2]
            L.forward(x, y, stream)
            x = y
    torch.cuda.synchronize()

    def step(i):
        x = xs[i % n_batches]
        for li, L in enumerate(layers):
            L.forward(x, bufs[li % 2], stream)
            x = bufs[li % 2]

    print(f"[bench] stack {args.stack}: {len(layers)} layers ready, routing stats taken", file=sys.stderr,
          flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    step_bytes = sum(layer_bytes(L.shape, float(n_active[li].mean())) for li, L in enumerate(layers))
    gbs = step_bytes / (ms_per_step / 1e3) / 1e9
    out = {
        "metric": "MoE-stack tokens/sec at 1 GPU (every layer of the stack per token)",
        "value": round(T / (ms_per_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": shapes[0].dtype,
        "data": "synthetic",
        "config": {"workload": args.stack, "layers": len(layers), "tokens": T, "hidden": shapes[0].H,
                   "ffn": shapes[0].F, "experts": [sh.E for sh in shapes], "top_k": shapes[0].k,
                   "capacity_factor": shapes[0].cf, "mlp_type": shapes[0].mlp_type, "token_batches": n_batches,
                   "parallelism": "one GPU"},
        "stack": {"us_per_layer": round(ms_per_step * 1e3 / len(layers), 2),
                  "algorithmic_bytes_per_step": int(step_bytes),
                  "mean_active_experts": [round(float(v), 2) for v in n_active.mean(axis=1)],
                  "hbm": {"achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(gbs / HBM_PEAK_GBS, 4)}},
    }
    print(json.dumps(out), flush=True)


CSRC = os.path.join(ROOT, "mixture_experts_transformer_moe_amd", "csrc")
# translation units of the measured kernels and what they include
KERNEL_SOURCES = {
    "decode": ["decode_ffn.hip", "common.h", "dispatch_common.h", "kernels.h", "topk.h"],
    "gemm": ["gemm.hip", "common.h", "kernels.h"],
}


def strip_comments(text: str) -> str:
    """C/C++ source without its comments, blank lines and runs of blanks (line
    breaks kept for the preprocessor), so that a change to comments or layout
    does not count as a kernel change."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":                     # string or character literal, escapes kept
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = (" ".join(line.split()) for line in "".join(out).splitlines())
    return "\n".join(line for line in lines if line)


def kernel_source_digest(files) -> str:
    """sha256 over the code of the named HIP sources (comments and whitespace
    left out): stored counter readings hold only while it matches."""
    import hashlib
    h = hashlib.sha256()
    for f in sorted(files):
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(f.encode() + b"\0" + strip_comments(fh.read()).encode())
    return h.hexdigest()


def measured_traffic(workload: str, kern: str):
    """HBM bytes per launch of the kernel from the committed rocprofv3 counter
    passes (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel reference), or None
    when none were taken or the kernel's sources changed since."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    files = t.get("sources")
    if not files or t.get("source_sha256") != kernel_source_digest(files) or kern not in t.get("kernels", {}):
        return None
    k = t["kernels"][kern]
    return {"read_bytes": k["read_bytes"], "write_bytes": k["write_bytes"],
            "total_bytes": k["read_bytes"] + k["write_bytes"], "unit": "bytes per launch"}


def _threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))
    except Exception:
        return 1


def cpu_baseline(shape, w, xs, budget_s: float) -> dict:
    """The fp64 oracle on host copies of the same inputs, timed on the host cores.

    Decode-sized batches: whole oracle layer forwards over the rotating token
    batches until the budget is spent. Larger batches (one forward can take
    tens of seconds): one batch, with the oracle's own steps timed one by one:
    gate, softmax, top-k and dispatch of every token, then the expert FFNs in
    local-expert order until the budget is spent (the remaining experts'
    time scaled by their dispatched rows: an expert's FFN cost is linear in its
    rows), the dense MLP in residual mode, and the combine."""
    import oracle
    threads = _threads()
    if shape.T <= 64:
        hw = {k: W.to_host_f64_ready(v) for k, v in w.items()}
        hxs = [W.to_host_f64_ready(x) for x in xs]
        n = 0
        t0 = time.perf_counter()
        while True:
            oracle.layer_forward(hxs[n % len(hxs)], hw, E=shape.E, k=shape.k, cf=shape.cf, e_lo=shape.e_lo,
                                 E_loc=shape.E_loc, residual=shape.residual, renorm=shape.renorm)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s or n >= 10000:
                break
        return {"value": round(shape.T * n / el, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
                "sample": f"{n} layer forwards of {shape.T} tokens (weight set 0, rotating token batches), "
                          f"{el:.1f} s, numpy float64",
                "cpu_model": _cpu_model()}
    hx = W.to_host_f64_ready(xs[0])
    gw = W.to_host_f64_ready(w["gate_w"])
    gb = W.to_host_f64_ready(w["gate_b"])
    t0 = time.perf_counter()
    r = oracle.route(hx, gw, gb, shape.k, shape.renorm)
    C = oracle.capacity(shape.T, shape.E, shape.k, shape.cf)
    d = oracle.dispatch(r["idx"], shape.E, C, shape.e_lo, shape.E_loc)
    t_route = time.perf_counter() - t0
    off = d["offsets"]
    active = [e for e in range(shape.E_loc) if off[e + 1] > off[e]]
    t_ffn, rows_done, n_done = 0.0, 0, 0
    y_disp = np.zeros((d["R"], shape.H))
    for e in active:
        a, b = int(off[e]), int(off[e + 1])
        ew = [W.to_host_f64_ready(w[n][e]) for n in ("w1", "b1", "w2", "b2")]   # host copy, not timed
        t1 = time.perf_counter()
        y_disp[a:b] = oracle.ffn(hx[d["slot_token"][a:b]], *ew)
        t_ffn += time.perf_counter() - t1
        rows_done += b - a
        n_done += 1
        del ew
        if t_route + t_ffn >= budget_s:
            break
    t_ffn_all = t_ffn * (d["R"] / max(rows_done, 1))
    t_dense = 0.0
    dense = None
    if shape.residual:
        mw = [W.to_host_f64_ready(w[n]) for n in ("mlp_w1", "mlp_b1", "mlp_w2", "mlp_b2")]
        t1 = time.perf_counter()
        dense = oracle.ffn(hx, *mw)
        t_dense = time.perf_counter() - t1
    t1 = time.perf_counter()
    oracle.combine(y_disp, d["token_slot"], r["w"], shape.T, shape.H, dense)
    t_comb = time.perf_counter() - t1
    total = t_route + t_ffn_all + t_dense + t_comb
    return {"value": round(shape.T / total, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"one batch of {shape.T} tokens: gate, softmax, top-k and dispatch of all tokens "
                      f"({t_route:.1f} s); FFNs of {n_done} of {len(active)} active experts timed "
                      f"({rows_done} of {d['R']} rows, {t_ffn:.1f} s) and scaled by rows to {t_ffn_all:.1f} s"
                      + (f"; dense MLP over all tokens {t_dense:.1f} s" if shape.residual else "")
                      + f"; combine {t_comb:.1f} s; numpy float64",
            "cpu_model": _cpu_model()}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
